"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: routing indices, permutation maps, split_sizes/offsets and MXFP8 codes
and scales bit-exact; routing weights within 1 float32 ulp; bf16 outputs and
gradients within normwise relative error 2e-2 (and 4e-2 per token row /
per expert slice); MXFP8 layer outputs within 6e-2 of the oracle running the
same MXFP8 algorithm.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import CONFIGS, bf16_bits, bf16_to_f32, bf16_to_f64, generate

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_MX = 6e-2


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_grouped_router_amd as mod
    mod.load_library()   # raises if the HIP library is missing
    return mod


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def host_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host_f64(t):
    return bf16_to_f64(host_bits(t))


def _ulp_diff_f32(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


def assert_rows_close(got, ref, tol, name):
    err = O.rel_err(got, ref)
    assert err <= tol, f"{name}: normwise {err:.3e} > {tol}"
    n = np.linalg.norm(ref, axis=-1)
    d = np.linalg.norm(got - ref, axis=-1)
    ok = n > 0
    worst = (d[ok] / n[ok]).max() if ok.any() else 0.0
    assert worst <= 2 * tol, f"{name}: worst row {worst:.3e}"
    assert np.all(d[~ok] == 0), f"{name}: non-zero where reference is zero"


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("T,E,k,renorm,seed", [
    (256, 8, 2, True, 0), (1000, 128, 8, True, 1), (333, 100, 5, False, 2),
    (64, 8, 8, True, 3), (1, 3, 1, True, 4), (513, 1024, 32, True, 5),
    (200, 64, 6, False, 6),
    # 16 lanes per token up to k = 16 and E = 256, one wave beyond
    (300, 256, 16, False, 8), (300, 256, 17, True, 9), (77, 40, 16, True, 10),
    (129, 257, 4, False, 11)])
def test_route_topk_matches_oracle(m, T, E, k, renorm, seed):
    lg = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    idx, w = m.moe_route_topk(torch.from_numpy(lg).cuda(), k, renorm)
    ridx, rw = O.route_topk(lg, k, renorm)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert _ulp_diff_f32(w.cpu().numpy(), rw).max() <= 1


@pytest.mark.parametrize("E,k", [(16, 4), (128, 8), (300, 8)])
def test_route_topk_ties_and_signed_zero(m, E, k):
    rng = np.random.default_rng(7)
    lg = rng.integers(-2, 3, size=(4096, E)).astype(np.float32)
    lg[rng.random(lg.shape) < 0.2] = -0.0
    idx, w = m.moe_route_topk(torch.from_numpy(lg).cuda(), k)
    ridx, rw = O.route_topk(lg, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert _ulp_diff_f32(w.cpu().numpy(), rw).max() <= 1


@pytest.mark.parametrize("name", ["tiny", "qwen3"])
def test_route_topk_config_logits(m, name):
    c = CONFIGS[name]
    d = generate(c.T, c.H, c.F, c.E, c.k, zipf=c.zipf, want=("logits",))
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), c.k)
    ridx, rw = O.route_topk(d["logits"], c.k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert _ulp_diff_f32(w.cpu().numpy(), rw).max() <= 1


# ------------------------------------------------------------ permutation
def _perm_case(m, T, H, E, k, zipf=0.0, seed=0, logits=None):
    d = generate(T, H, 64, E, k, zipf=zipf, seed=seed, want=("x", "logits"))
    lg = d["logits"] if logits is None else logits
    ridx, rw = O.route_topk(lg, k)
    x = dev_bf16(d["x"])
    out = m.moe_permute(x, torch.from_numpy(ridx).cuda(), E,
                        topk_w=torch.from_numpy(rw).cuda())
    ref = O.permute_index(ridx, E)
    for key in ("split_sizes", "offsets", "row_map", "src_row"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key], key)
    np.testing.assert_array_equal(host_bits(out["x_perm"]),
                                  O.permute_rows(d["x"], ref["src_row"], k))
    np.testing.assert_array_equal(out["w_perm"].cpu().numpy(),
                                  O.permute_weights(rw, ref["src_row"]))
    return d, ridx, rw, out, ref


@pytest.mark.parametrize("T,H,E,k,zipf", [
    (256, 128, 8, 2, 0.0), (2000, 264, 128, 8, 1.2), (1025, 64, 16, 4, 0.0),
    (1, 8, 4, 2, 0.0), (3000, 2048, 128, 8, 1.2),
    # row-copy kernel variants: four tokens per block (H <= 2048), two
    # (H <= 4096), one with a loop over the row (larger H); odd T tails
    (1023, 4096, 8, 2, 0.0), (3, 4096, 8, 2, 0.0), (301, 8192, 8, 3, 0.0),
    (5, 2040, 4, 4, 0.0)])
def test_permute_bit_exact(m, T, H, E, k, zipf):
    _perm_case(m, T, H, E, k, zipf)


def test_permute_degenerate_routings(m):
    T, H, E, k = 700, 96, 32, 1
    lg = np.full((T, E), -5.0, np.float32)
    lg[:, 17] = 3.0                      # every token to expert 17
    _, _, _, out, _ = _perm_case(m, T, H, E, k, logits=lg)
    sp = out["split_sizes"].cpu().numpy()
    assert sp[17] == T and sp.sum() == T
    # E = 1, k = 1: the identity permutation
    _, _, _, out, _ = _perm_case(m, 100, 16, 1, 1)
    assert np.array_equal(out["row_map"].cpu().numpy(), np.arange(100))


@pytest.mark.parametrize("k", [1, 2, 8])
def test_permute_unpermute_identity_bitwise(m, k):
    T, H, E = 500, 256, 8
    d, ridx, rw, out, ref = _perm_case(m, T, H, E, k)
    y = m.moe_unpermute(out["x_perm"], out["row_map"], k)
    x = bf16_to_f64(d["x"])
    np.testing.assert_array_equal(host_bits(y),
                                  bf16_bits((k * x).astype(np.float32)))
    w = torch.full((T, k), 1.0 / k, dtype=torch.float32, device="cuda")
    y2 = m.moe_unpermute(out["x_perm"], out["row_map"], k, topk_w=w)
    np.testing.assert_array_equal(host_bits(y2), d["x"])


def test_unpermute_weighted_matches_oracle(m):
    T, H, E, k = 300, 128, 16, 4
    rng = np.random.default_rng(3)
    d, ridx, rw, out, ref = _perm_case(m, T, H, E, k)
    z = bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    y = m.moe_unpermute(dev_bf16(z), out["row_map"], k,
                        topk_w=torch.from_numpy(rw).cuda())
    yr = O.unpermute(bf16_to_f64(z), ref["row_map"], k, topk_w=rw)
    # float32 sum of k terms, then one bf16 rounding
    np.testing.assert_allclose(host_f64(y), yr, rtol=2 ** -8, atol=1e-6)


def test_unpermute_k1_rounds_to_nearest_even(m):
    """k = 1: y = bf16(w * z) with one float32 product, so every output
    checks the float32 -> bf16 rounding bit for bit, ties included."""
    T, H, E, k = 256, 128, 4, 1
    rng = np.random.default_rng(11)
    d, ridx, rw, out, ref = _perm_case(m, T, H, E, k)
    zf = (rng.standard_normal((T, H)) *
          np.exp2(rng.integers(-20, 20, (T, H)))).astype(np.float32)
    zf[:, :4] = 1.0                        # products that are exact ties
    z = bf16_bits(zf)
    w = rng.uniform(0.01, 1.0, (T, 1)).astype(np.float32)
    w[:64] = np.float32(1 + 2 ** -8)       # tie, rounds down to even
    w[64:128] = np.float32(1 + 3 * 2 ** -8)  # tie, rounds up to even
    y = m.moe_unpermute(dev_bf16(z), out["row_map"], k,
                        topk_w=torch.from_numpy(w).cuda())
    # y[t] = w[t] * z[row_map[t]]: one float32 product, one bf16 rounding
    zt = bf16_to_f64(z).astype(np.float32)[ref["row_map"]]
    want = bf16_bits((w * zt).astype(np.float32))
    np.testing.assert_array_equal(host_bits(y), want)


def test_gather_rows_and_probs_grad(m):
    T, H, E, k = 400, 64, 8, 2
    d, ridx, rw, out, ref = _perm_case(m, T, H, E, k)
    dy = bf16_bits(np.random.default_rng(1).standard_normal(
        (T, H)).astype(np.float32))
    dz = m.moe_gather_rows(dev_bf16(dy), out["row_map"], k)
    np.testing.assert_array_equal(host_bits(dz),
                                  O.gather_rows(dy, ref["src_row"], k))
    dwp = np.random.default_rng(2).standard_normal(T * k).astype(np.float32)
    dp = m.moe_unpermute_probs_grad(torch.from_numpy(dwp).cuda(),
                                    out["row_map"], k)
    np.testing.assert_array_equal(dp.cpu().numpy(),
                                  O.probs_grad(dwp, ref["row_map"], k)
                                  .astype(np.float32))


def test_device_check_flags_bad_expert_id(m):
    T, H, E, k = 64, 32, 8, 2
    idx = np.random.default_rng(0).integers(0, E, size=(T, k)).astype(np.int32)
    idx[5, 1] = E + 3                    # written on the host, then uploaded
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    assert m.check_device_status() == 0
    out = m.moe_permute(x, torch.from_numpy(idx).cuda(), E)
    assert m.check_device_status() == 1
    assert out["row_map"][5 * k + 1].item() == -1
    assert int(out["split_sizes"].sum().item()) == T * k - 1
    assert m.check_device_status() == 0  # cleared by the previous check


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_device_check_flags_nonfinite_logits(m, bad):
    """A NaN or infinite router logit (written on the host) records the
    logits device check; the finite tokens are routed as the oracle routes
    them, and the kernel completes normally."""
    T, E, k = 96, 128, 8
    logits = np.random.default_rng(3).standard_normal((T, E)).astype(
        np.float32)
    logits[17, 40] = bad
    assert m.check_device_status() == 0
    idx, w = m.moe_route_topk(torch.from_numpy(logits).cuda(), k)
    assert m.check_device_status() == 3
    ok = np.ones(T, bool)
    ok[17] = False
    ri, rw = O.route_topk(logits[ok], k)
    np.testing.assert_array_equal(idx.cpu().numpy()[ok], ri)
    assert _ulp_diff_f32(w.cpu().numpy()[ok], rw).max() <= 1
    idx, w = m.moe_route_topk(torch.from_numpy(logits[ok]).cuda(), k)
    assert m.check_device_status() == 0


def test_device_check_flags_bad_offsets(m):
    """Per-expert offsets written on the host that end below the row count
    (non-decreasing, so every access stays in bounds even unchecked) are
    caught on the device by every call that reads them: the grouped MLP
    forward (bf16, MXFP8, FP8 tensor-scaled) and backward (bf16, MXFP8) and
    the token-segment MXFP8 quantiser record the offsets error, run no tile
    and return normally; a following call with valid offsets is unaffected.
    (Decreasing arrays and arrays ending past the rows are rejected by the
    same guard; tests/native/offsets_check.cpp covers them on the host.)"""
    E, H, F, rows = 4, 128, 128, 64
    rng = np.random.default_rng(9)
    x = dev_bf16(bf16_bits(rng.standard_normal((rows, H)).astype(np.float32)))
    dz = dev_bf16(bf16_bits(rng.standard_normal((rows, H)).astype(np.float32)))
    wgu_h = bf16_bits((0.05 * rng.standard_normal((E, 2 * F, H))).astype(
        np.float32))
    wdn_h = bf16_bits((0.05 * rng.standard_normal((E, H, F))).astype(
        np.float32))
    wgu, wdn = dev_bf16(wgu_h), dev_bf16(wdn_h)
    good = torch.tensor([0, 10, 20, 40, 64], dtype=torch.int32, device="cuda")
    bad = torch.tensor([0, 10, 20, 40, 60], dtype=torch.int32, device="cuda")
    assert m.check_device_status() == 0
    for prec in (m.PREC_BF16, m.PREC_MXFP8, m.PREC_FP8_TENSOR):
        m.moe_grouped_mlp_fwd(x, wgu, wdn, bad, precision=prec)
        assert m.check_device_status() == 2, prec
    f = m.moe_grouped_mlp_fwd(x, wgu, wdn, good, save=True)
    assert m.check_device_status() == 0
    for prec in (m.PREC_BF16, m.PREC_MXFP8):
        m.moe_grouped_mlp_bwd(dz, x, wgu, wdn, bad, f["h1"], f["a"],
                              precision=prec)
        assert m.check_device_status() == 2, prec
    m.mxfp8_quantize(x, m.COLWISE, seg_offsets=bad)
    assert m.check_device_status() == 2
    # the valid call after them matches the oracle
    r = m.moe_grouped_mlp_fwd(x, wgu, wdn, good)
    assert m.check_device_status() == 0
    ref = O.grouped_mlp_fwd(host_bits(x), wgu_h, wdn_h, None,
                            good.cpu().numpy())
    assert_rows_close(host_f64(r["z"]), ref["z"], TOL_BF16, "z")


# ------------------------------------------------------------ MXFP8 quant
def _f32_encoder_cases(rng):
    """float32 rows of 32-value blocks that exercise the E4M3 encoder:
    random magnitudes over the whole float32 range (subnormals included),
    exact ties between neighbouring codes, values rounding past 448, small
    values under a large block maximum, zeros and negative zeros."""
    blocks = []
    # random blocks at every block exponent reachable from float32
    for e in range(-149, 121, 2):
        v = rng.standard_normal((4, 32)) * 2.0 ** e
        blocks.append(v.astype(np.float32))
    # exact midpoints between consecutive E4M3 values, times 2^t, in blocks
    # whose lead value pins the scale to 2^t (448 * 2^t as the block max)
    mags = O.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2.0
    for t in (-130, -20, 0, 3, 100):
        v = np.resize(mids, (4, 31)) * rng.choice([-1.0, 1.0], (4, 31))
        lead = np.full((4, 1), 448.0)
        blk = np.concatenate([lead, v], axis=1) * 2.0 ** t
        blocks.append(blk.astype(np.float32))
    # leads whose scaled value falls in (448, 512): saturate to 448;
    # 464 is the tie between 448 and the (NaN) next code
    for lead in (449.0, 463.9, 464.0, 480.0, 500.0, 511.75):
        v = rng.standard_normal((2, 32)) * 100.0
        v[:, 0] = lead
        v[1, 0] = -lead
        blocks.append((v * 2.0 ** -3).astype(np.float32))
    # tiny values under a large maximum: subnormal codes and flushes
    v = rng.standard_normal((8, 32)) * 2.0 ** rng.integers(-14, -4, (8, 32))
    v[:, 0] = 300.0
    blocks.append(v.astype(np.float32))
    z = np.zeros((2, 32), np.float32)
    z[1] = -0.0
    z[1, 5] = -1e-3
    blocks.append(z)
    return np.concatenate(blocks, axis=0).reshape(-1, 64)


def test_mxfp8_quantize_f32_epilogue_encoder(m):
    """The float32 -> MXFP8 encoder of the MXFP8 gate/up epilogue (block
    exponent from the float32 amax, gfx950 scaled conversion, 448 fix-up)
    against the oracle's R7 rule, bit for bit."""
    v = _f32_encoder_cases(np.random.default_rng(21))
    assert np.all(np.isfinite(v))
    codes, scales = m.mxfp8_quantize_f32(torch.from_numpy(v).cuda())
    want_c, want_s = O.mxfp8_quantize_rows(v.astype(np.float64))
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.argwhere(gc != want_c)
    assert bad.size == 0, (bad[:4], v[tuple(bad[0])], gc[tuple(bad[0])],
                           want_c[tuple(bad[0])])
    np.testing.assert_array_equal(gs, want_s)
    assert (want_c & 0x7F).max() == 0x7E and np.any(want_c == 0x80)


def test_mxfp8_a_codes_match_fraction(m):
    """A's on-the-fly MXFP8 codes (quantised from float32 in the gate/up
    epilogue) against the oracle's codes of its float64 A: not bit-gated,
    since the two A values differ by accumulation order, but nearly all
    equal (the share is printed)."""
    T, H, F, E, k = 512, 256, 512, 8, 2
    d = _mlp_case(T, H, F, E, k, 0.0, seed=8)
    ref = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    rq = O.grouped_mlp_fwd_mxfp8(ref["x_perm"], d["w_gu"], d["w_dn"],
                                 ref["w_perm"], ref["offsets"], keep=True)
    want_c, want_s = O.mxfp8_quantize_rows(rq["a"])
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w,
                      precision=m.PREC_MXFP8)
    r = m.moe_grouped_mlp_fwd(p["x_perm"], dev_bf16(d["w_gu"]),
                              dev_bf16(d["w_dn"]), p["offsets"],
                              w_perm=p["w_perm"], precision=m.PREC_MXFP8,
                              x_perm_scale=p["x_perm_scale"],
                              save_a_codes=True)
    fc = float((r["a_q"].cpu().numpy() == want_c).mean())
    fs = float((r["a_s"].cpu().numpy() == want_s).mean())
    print(f"A codes equal to the oracle's: {fc:.6f}; scales: {fs:.6f}")
    assert fc >= 0.99 and fs >= 0.99, (fc, fs)


def test_mxfp8_rowwise_all_bf16_patterns(m):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite values
    rng = np.random.default_rng(0)
    n = (bits.size // 32) * 32
    a = rng.permutation(bits)[:n].reshape(-1, 64) if n % 64 == 0 else \
        rng.permutation(bits)[:(n // 64) * 64].reshape(-1, 64)
    codes, scales = m.mxfp8_quantize(dev_bf16(a), m.ROWWISE)
    rc, rs = O.mxfp8_quantize_rows(a)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


def _every_scale_blocks(seed):
    """One block per (block exponent, magnitude) pair: element 0 is 2^e
    (e = -133 .. 127, so the scale exponent runs over its whole range and
    clamps at -127 for tiny blocks), the other 31 are every finite bf16
    magnitude not above 2^e, with random signs."""
    rng = np.random.default_rng(seed)
    mags = np.arange(0x7f80, dtype=np.uint32)      # finite, non-negative
    rows = []
    for e in range(-133, 128):
        top = (e + 127) << 7 if e >= -126 else 1 << (e + 133)
        cand = mags[mags <= top]
        cand = np.concatenate([cand, np.zeros(-len(cand) % 31, np.uint32)])
        cand |= rng.integers(0, 2, size=cand.size).astype(np.uint32) << 15
        blk = cand.reshape(-1, 31)
        rows.append(np.concatenate(
            [np.full((blk.shape[0], 1), top, np.uint32), blk], axis=1))
    return np.concatenate(rows).astype(np.uint16)


def test_mxfp8_every_scale_and_pattern(m):
    a = _every_scale_blocks(4)                      # [blocks, 32]
    codes, scales = m.mxfp8_quantize(dev_bf16(a), m.ROWWISE)
    rc, rs = O.mxfp8_quantize_rows(a)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    # the same blocks down the columns (transposed output): 32 rows, and
    # 128 rows (four blocks per column, the 128-row tile kernel)
    at = np.ascontiguousarray(a[:4096].T)           # [32, 4096]
    codes, scales = m.mxfp8_quantize(dev_bf16(at), m.COLWISE)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc[:4096])
    np.testing.assert_array_equal(scales.cpu().numpy(), rs[:4096])
    n = 4000
    at4 = np.ascontiguousarray(
        a[:4 * n].reshape(4, n, 32).transpose(0, 2, 1).reshape(128, n))
    codes, scales = m.mxfp8_quantize(dev_bf16(at4), m.COLWISE)
    want_c = rc[:4 * n].reshape(4, n, 32).transpose(1, 0, 2).reshape(n, 128)
    want_s = rs[:4 * n].reshape(4, n).T
    np.testing.assert_array_equal(codes.cpu().numpy(), want_c)
    np.testing.assert_array_equal(scales.cpu().numpy(), want_s)


def test_mxfp8_rowwise_scale_spread(m):
    # blocks whose amax spans the whole exponent range, including subnormals
    rng = np.random.default_rng(1)
    v = rng.standard_normal((512, 256)).astype(np.float32)
    v *= np.ldexp(1.0, rng.integers(-140, 120, size=(512, 8))).repeat(
        32, axis=1).astype(np.float32)
    a = bf16_bits(v)
    codes, scales = m.mxfp8_quantize(dev_bf16(a), m.ROWWISE)
    rc, rs = O.mxfp8_quantize_rows(a)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("rows", [96, 256])   # 32-row and 128-row tiles
def test_mxfp8_colwise_and_batched(m, rows):
    rng = np.random.default_rng(2)
    a = bf16_bits(rng.standard_normal((3, rows, 200)).astype(np.float32))
    codes, scales = m.mxfp8_quantize(dev_bf16(a), m.COLWISE)
    for b in range(3):
        rc, rs = O.mxfp8_quantize_cols(a[b])
        np.testing.assert_array_equal(codes[b].cpu().numpy(), rc)
        np.testing.assert_array_equal(scales[b].cpu().numpy(), rs)


def test_mxfp8_segments(m):
    rng = np.random.default_rng(3)
    off = np.array([0, 0, 45, 45, 77, 200, 200], dtype=np.int32)
    a = bf16_bits(rng.standard_normal((200, 72)).astype(np.float32))
    codes, scales = m.mxfp8_quantize(dev_bf16(a), m.COLWISE,
                                     seg_offsets=torch.from_numpy(off).cuda())
    rc, rs = O.mxfp8_quantize_segments(a, off)
    w = rc.shape[1]
    np.testing.assert_array_equal(codes[:, :w].cpu().numpy(), rc)
    np.testing.assert_array_equal(scales[:, :w // 32].cpu().numpy(), rs)


@pytest.mark.parametrize("T,H,E,k", [
    (300, 256, 8, 2),      # four tokens per block, word scale stores
    (301, 96, 8, 2),       # H % 128 != 0: byte scale stores
    (257, 4096, 8, 2),     # two tokens per block
    (33, 8192, 4, 3),      # one token per block, loop over the row
    (130, 2048, 16, 8), (7, 160, 4, 1)])
def test_permute_fused_mxfp8_bit_exact(m, T, H, E, k):
    d = generate(T, H, 64, E, k, want=("x", "logits"))
    ridx, rw = O.route_topk(d["logits"], k)
    out = m.moe_permute(dev_bf16(d["x"]), torch.from_numpy(ridx).cuda(), E,
                        topk_w=torch.from_numpy(rw).cuda(),
                        precision=m.PREC_MXFP8)
    ref = O.permute_index(ridx, E)
    rc, rs = O.mxfp8_quantize_rows(O.permute_rows(d["x"], ref["src_row"], k))
    np.testing.assert_array_equal(out["x_perm"].cpu().numpy(), rc)
    np.testing.assert_array_equal(out["x_perm_scale"].cpu().numpy(), rs)


# ------------------------------------------------------- grouped MLP, bf16
def _mlp_case(T, H, F, E, k, zipf, seed, logits_shift=None):
    d = generate(T, H, F, E, k, zipf=zipf, seed=seed,
                 want=("x", "logits", "w_gu", "w_dn", "dy"))
    if logits_shift is not None:
        d["logits"] = (d["logits"] + logits_shift).astype(np.float32)
    return d


MLP_CASES = [
    # T, H, F, E, k, zipf
    (256, 128, 256, 8, 2, 0.0),     # the tiny config
    (700, 192, 320, 5, 2, 1.2),     # ragged M, F tail (320 = 2.5 x 128)
    (900, 256, 128, 16, 4, 1.2),    # many experts, some empty
    (64, 64, 64, 4, 1, 0.0),        # tiles larger than the problem
    (300, 2112, 192, 4, 2, 1.2),    # eight-wave gate/up, 33 K steps
    (400, 640, 320, 6, 2, 1.2),     # whole trips of the five-buffer rotation
    (300, 4160, 192, 4, 2, 1.2),    # H > 4096: the four-wave gate/up GEMM
    (512, 256, 8192, 4, 2, 0.0),    # down GEMM's tiles split 4 ways along K
    (700, 256, 8192, 8, 2, 1.2),    # the same with empty and one-row experts
]


def split_plan(offsets, tn, nk, cus):
    """Work-groups sharing each tile of the last, partly filled round of a
    RAGGED_M launch of the eight-wave GEMM, per XCD (1: not split).  Mirrors
    the tile dealing of the library (8 XCDs, contiguous runs of tiles, one
    tile per CU per round); used to check that a case covers the split."""
    cnt_e = np.diff(np.asarray(offsets, dtype=np.int64))
    total = int(sum((c + 255) // 256 for c in cnt_e)) * tn
    per = (total + 7) // 8
    slots_x = 0 if nk < 4 else min(32, per * 8)
    C = cus // 8
    out = []
    for x in range(8):
        cnt = min(per, total - x * per)
        if cnt <= 0:
            continue
        rem = cnt % C
        S = 1
        if slots_x and rem and 2 * rem <= C:
            S = min(C // rem, 8, slots_x // rem, nk // 32)
            S = S if S >= 2 else 1
        out.append(S)
    return out


@pytest.mark.parametrize("T,H,F,E,k,zipf", MLP_CASES)
def test_grouped_mlp_fwd_bf16(m, T, H, F, E, k, zipf):
    d = _mlp_case(T, H, F, E, k, zipf, seed=1)
    ref = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k, keep=True)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    r = m.moe_grouped_mlp_fwd(p["x_perm"], dev_bf16(d["w_gu"]),
                              dev_bf16(d["w_dn"]), p["offsets"],
                              w_perm=p["w_perm"], save=True)
    y = m.moe_unpermute(r["z"], p["row_map"], k)
    assert_rows_close(host_f64(r["z"]), ref["z"], TOL_BF16, "z")
    assert_rows_close(host_f64(r["a"]), ref["a"], TOL_BF16, "a")
    assert_rows_close(host_f64(r["h1"]), ref["h1"], TOL_BF16, "h1")
    assert_rows_close(host_f64(y), ref["y"], TOL_BF16, "y")


@pytest.mark.parametrize("T,H,F,E,k,zipf", MLP_CASES)
def test_expert_loop_mlp_fwd_bf16(m, T, H, F, E, k, zipf):
    """The per-expert loop baseline computes the same layer (its h1 is
    rounded to bf16 before the SwiGLU, within the bf16 tolerance)."""
    d = _mlp_case(T, H, F, E, k, zipf, seed=1)
    ref = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k, keep=True)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    r = m.moe_expert_loop_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                                  w_perm=p["w_perm"], save=True)
    assert_rows_close(host_f64(r["h1"]), ref["h1"], TOL_BF16, "h1")
    assert_rows_close(host_f64(r["a"]), ref["a"], TOL_BF16, "a")
    assert_rows_close(host_f64(r["z"]), ref["z"], TOL_BF16, "z")
    # the same gate/up GEMM as the grouped path, which may split the K range
    # of its last round of tiles (float32 sums in another order): h1 within
    # one bf16 rounding
    g = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], save=True)
    gh, rh = g["h1"].float(), r["h1"].float()
    assert torch.all((gh - rh).abs() <= 2.0 ** -7 * rh.abs()
                     + 1e-4 * rh.abs().max())
    # without saves (h1 and a in the workspace) the output is the same
    r2 = m.moe_expert_loop_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                                   w_perm=p["w_perm"])
    assert torch.equal(r2["z"], r["z"])


def test_expert_loop_rejects_bad_offsets(m):
    T, H, F, E, k = 64, 64, 64, 4, 1
    d = _mlp_case(T, H, F, E, k, 0.0, seed=3)
    x = dev_bf16(d["x"])
    off = torch.tensor([0, 10, 5, 40, 64], dtype=torch.int32, device="cuda")
    with pytest.raises(m.MoEError):
        m.moe_expert_loop_mlp_fwd(x, dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"]),
                                  off)
    off = torch.tensor([0, 10, 20, 40, 60], dtype=torch.int32, device="cuda")
    with pytest.raises(m.MoEError):
        m.moe_expert_loop_mlp_fwd(x, dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"]),
                                  off)


def test_grouped_mlp_one_expert_takes_all(m):
    T, H, F, E, k = 600, 128, 256, 8, 1
    shift = np.zeros(E, np.float32)
    shift[3] = 100.0
    d = _mlp_case(T, H, F, E, k, 0.0, 2, logits_shift=shift)
    ref = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    assert p["split_sizes"].cpu().numpy()[3] == T
    r = m.moe_grouped_mlp_fwd(p["x_perm"], dev_bf16(d["w_gu"]),
                              dev_bf16(d["w_dn"]), p["offsets"],
                              w_perm=p["w_perm"])
    y = m.moe_unpermute(r["z"], p["row_map"], k)
    assert_rows_close(host_f64(y), ref["y"], TOL_BF16, "y")


def test_scaled_swiglu_equals_weighted_combine(m):
    T, H, F, E, k = 300, 128, 128, 8, 2
    d = _mlp_case(T, H, F, E, k, 0.0, 3)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    ya = m.moe_unpermute(m.moe_grouped_mlp_fwd(
        p["x_perm"], wgu, wdn, p["offsets"], w_perm=p["w_perm"])["z"],
        p["row_map"], k)
    yb = m.moe_unpermute(m.moe_grouped_mlp_fwd(
        p["x_perm"], wgu, wdn, p["offsets"])["z"], p["row_map"], k, topk_w=w)
    assert O.rel_err(host_f64(ya), host_f64(yb)) < 1e-2


def test_grouped_mlp_deterministic(m):
    T, H, F, E, k = 500, 256, 256, 16, 4
    d = _mlp_case(T, H, F, E, k, 1.2, 4)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    z1 = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                               w_perm=p["w_perm"])["z"]
    z2 = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                               w_perm=p["w_perm"])["z"]
    assert torch.equal(z1.view(torch.int16), z2.view(torch.int16))


def test_grouped_mlp_split_tail(m):
    """Whole rounds of tiles plus a last round whose tiles are split along K
    over several work-groups (partials added in a fixed order), in the down
    GEMM (K = F = 4096): matches the oracle and the per-expert loop (which
    never splits), bit for bit the same over repeated calls."""
    T, H, F, E, k = 4096, 2048, 4096, 8, 2
    d = _mlp_case(T, H, F, E, k, 0.0, 5)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    offs = p["offsets"].cpu().numpy()
    # the down GEMM (256-column tiles, 64-wide K steps) splits its tail
    assert max(split_plan(offs, H // 256, F // 64, cus)) > 1
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    runs = [m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                                  w_perm=p["w_perm"], save=True)
            for _ in range(3)]
    for r in runs[1:]:
        for key in ("z", "h1", "a"):
            assert torch.equal(r[key].view(torch.int16),
                               runs[0][key].view(torch.int16)), key
    ref = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k, keep=True)
    assert_rows_close(host_f64(runs[0]["z"]), ref["z"], TOL_BF16, "z")
    assert_rows_close(host_f64(runs[0]["h1"]), ref["h1"], TOL_BF16, "h1")
    loop = m.moe_expert_loop_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                                     w_perm=p["w_perm"], save=True)
    # the loop rounds h1 and A to bf16 on the way: close, not bit-equal
    assert O.rel_err(host_f64(runs[0]["z"]), host_f64(loop["z"])) < 1e-2


def test_grouped_mlp_zero_rows(m):
    E, H, F = 4, 64, 64
    x = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    off = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    wgu = torch.zeros((E, 2 * F, H), dtype=torch.bfloat16, device="cuda")
    wdn = torch.zeros((E, H, F), dtype=torch.bfloat16, device="cuda")
    r = m.moe_grouped_mlp_fwd(x, wgu, wdn, off)
    assert r["z"].shape == (0, H)


# ------------------------------------------------------ backward, bf16
BWD_CASES = [
    (256, 128, 256, 8, 2, 0.0),
    (700, 192, 320, 5, 2, 1.2),
    (900, 256, 128, 16, 4, 1.2),
    # weight gradients over longer token segments (the operand rotation's
    # whole trips and tails along the tokens)
    (1200, 128, 256, 2, 2, 0.0),
    (1000, 192, 192, 3, 1, 1.2),
]


@pytest.mark.parametrize("T,H,F,E,k,zipf", BWD_CASES)
def test_grouped_mlp_bwd_bf16(m, T, H, F, E, k, zipf):
    d = _mlp_case(T, H, F, E, k, zipf, seed=5)
    ref = O.layer_bwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], d["dy"], k)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    f = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], save=True)
    dz = m.moe_gather_rows(dev_bf16(d["dy"]), p["row_map"], k)
    g = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                              f["h1"], f["a"], w_perm=p["w_perm"])
    dx = m.moe_unpermute(g["dx_perm"], p["row_map"], k)
    dprobs = m.moe_unpermute_probs_grad(g["dw_perm"], p["row_map"], k)
    assert_rows_close(host_f64(dx), ref["dx"], TOL_BF16, "dx")
    assert_rows_close(dprobs.cpu().numpy().astype(np.float64).reshape(1, -1),
                      ref["dprobs"].reshape(1, -1), TOL_BF16, "dprobs")
    split = ref["split_sizes"]
    gw_gu, gw_dn = host_f64(g["dw_gu"]), host_f64(g["dw_dn"])
    for e in range(E):
        if split[e] == 0:
            assert np.all(gw_gu[e] == 0) and np.all(gw_dn[e] == 0)
    assert O.rel_err(gw_gu, ref["dw_gu"]) <= TOL_BF16
    assert O.rel_err(gw_dn, ref["dw_dn"]) <= TOL_BF16
    for e in range(E):
        if split[e] > 0:
            assert O.rel_err(gw_gu[e], ref["dw_gu"][e]) <= TOL_BF16, e
            assert O.rel_err(gw_dn[e], ref["dw_dn"][e]) <= TOL_BF16, e


# ------------------------------------------------------- grouped MLP, MXFP8
MX_CASES = [
    # T, H, F, E, k, zipf   (H and F multiples of 128)
    (256, 128, 256, 8, 2, 0.0),
    (700, 256, 384, 5, 2, 1.2),     # ragged M tails, odd K-step count (3)
    (900, 384, 128, 16, 4, 1.2),    # many experts, some empty
    (512, 256, 8192, 4, 2, 0.0),    # down GEMM's last tiles split along K
    (700, 256, 8192, 8, 2, 1.2),    # the same with empty and one-row experts
    # operand rotations in whole trips of five K steps plus nk % 5
    (300, 640, 1152, 4, 2, 1.2),    # gate/up nk = 5, down nk = 9
    (200, 1152, 640, 3, 1, 0.0),    # gate/up nk = 9, down nk = 5
]


@pytest.mark.parametrize("T,H,F,E,k,zipf", MX_CASES)
def test_grouped_mlp_fwd_mxfp8(m, T, H, F, E, k, zipf):
    d = _mlp_case(T, H, F, E, k, zipf, seed=7)
    ref = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    rq = O.grouped_mlp_fwd_mxfp8(ref["x_perm"], d["w_gu"], d["w_dn"],
                                 ref["w_perm"], ref["offsets"], keep=True)
    yq = O.unpermute(rq["z"], ref["row_map"], k)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w,
                      precision=m.PREC_MXFP8)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    r = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], precision=m.PREC_MXFP8,
                              x_perm_scale=p["x_perm_scale"], save=True)
    y = m.moe_unpermute(r["z"], p["row_map"], k)
    assert_rows_close(host_f64(r["z"]), rq["z"], TOL_MX, "z")
    assert_rows_close(host_f64(y), yq, TOL_MX, "y")
    # the bf16 A save is the pre-quantisation SwiGLU output
    assert_rows_close(host_f64(r["a"]), rq["a"], TOL_BF16, "a")
    # far below the bar in practice: only A's block codes can differ
    assert O.rel_err(host_f64(y), yq) < 1e-2


def test_mxfp8_fwd_prequantised_equals_on_the_fly(m):
    T, H, F, E, k = 500, 256, 256, 8, 2
    d = _mlp_case(T, H, F, E, k, 1.2, seed=8)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    pb = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    pq = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w,
                       precision=m.PREC_MXFP8)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    # x quantised inside the call, weights quantised inside the call
    z1 = m.moe_grouped_mlp_fwd(pb["x_perm"], wgu, wdn, pb["offsets"],
                               w_perm=pb["w_perm"],
                               precision=m.PREC_MXFP8)["z"]
    # x codes from the permute, weights quantised by mxfp8_quantize
    gq = m.mxfp8_quantize(wgu.reshape(E * 2 * F, H), m.ROWWISE)
    dq = m.mxfp8_quantize(wdn.reshape(E * H, F), m.ROWWISE)
    z2 = m.moe_grouped_mlp_fwd(
        pq["x_perm"], wgu, wdn, pq["offsets"], w_perm=pq["w_perm"],
        precision=m.PREC_MXFP8, x_perm_scale=pq["x_perm_scale"],
        w_gu_q=(gq[0].reshape(E, 2 * F, H), gq[1].reshape(E, 2 * F, H // 32)),
        w_dn_q=(dq[0].reshape(E, H, F), dq[1].reshape(E, H, F // 32)))["z"]
    assert torch.equal(z1.view(torch.int16), z2.view(torch.int16))


def test_mxfp8_fwd_exact_on_representable_operands(m):
    """Operands that MXFP8 represents exactly (block max in the top binade,
    as built here) pass through the quantisation unchanged, so the gate/up
    GEMM equals the float64 product of the same values up to float32
    accumulation order and the bf16 rounding of the saved (g, u)."""
    rng = np.random.default_rng(9)
    T, H, F, E, k = 300, 256, 128, 4, 1

    def rep(shape):
        nb = int(np.prod(shape)) // 32
        mags = rng.integers(0, 0x78, size=(nb, 32))
        mags[:, 0] = rng.integers(0x78, 0x7F, size=nb)
        codes = mags | (rng.integers(0, 2, size=mags.shape) << 7)
        s = rng.integers(-14, -6, size=nb)
        v = np.ldexp(O.e4m3_decode(codes), s[:, None]).reshape(shape)
        return v.astype(np.float32)

    x = rep((T, H))
    wgu = rep((E, 2 * F, H))
    wdn = rep((E, H, F))
    xb, gb, db = bf16_bits(x), bf16_bits(wgu), bf16_bits(wdn)
    # representable in E4M3 with these scales -> exactly representable in bf16
    assert np.array_equal(bf16_to_f32(xb), x)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = m.moe_route_topk(torch.from_numpy(lg).cuda(), k)
    p = m.moe_permute(dev_bf16(xb), idx, E)
    r = m.moe_grouped_mlp_fwd(p["x_perm"], dev_bf16(gb), dev_bf16(db),
                              p["offsets"], precision=m.PREC_MXFP8, save=True)
    ref = O.permute_index(idx.cpu().numpy(), E)
    xp = x.astype(np.float64)[ref["src_row"] // k]
    h1 = np.zeros((T * k, 2 * F))
    for e in range(E):
        lo, hi = ref["offsets"][e], ref["offsets"][e + 1]
        h1[lo:hi] = xp[lo:hi] @ wgu[e].astype(np.float64).T
    got = host_f64(r["h1"])
    # products are exact; what is left is float32 accumulation order and the
    # bf16 rounding of the saved value (relative 2^-9): a wrong scale byte or
    # K block would be off by powers of two
    assert O.rel_err(got, h1) < 3e-3
    assert_rows_close(got, h1, 3e-3, "h1")


# ---------------------------------------------- grouped MLP backward, MXFP8
MX_BWD_CASES = [
    # T, H, F, E, k, zipf   (H and F multiples of 128)
    (256, 128, 256, 8, 2, 0.0),
    (700, 256, 384, 5, 2, 1.2),     # ragged token segments, odd K steps
    (900, 384, 128, 16, 4, 1.2),    # many experts, some empty
    (130, 128, 128, 3, 1, 0.0),     # k = 1, segments shorter than a K step
    # weight gradients with longer token segments: whole trips of the
    # operand rotation (1200 tokens per expert, 10 K steps) and a tail
    (1200, 256, 256, 2, 2, 0.0),
    (1500, 128, 256, 3, 2, 1.2),
]


def _mx_bwd_run(m, d, T, H, F, E, k):
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    f = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], precision=m.PREC_MXFP8,
                              save=True)
    dz = m.moe_gather_rows(dev_bf16(d["dy"]), p["row_map"], k)
    g = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                              f["h1"], f["a"], w_perm=p["w_perm"],
                              precision=m.PREC_MXFP8)
    return p, g


@pytest.mark.parametrize("T,H,F,E,k,zipf", MX_BWD_CASES)
def test_grouped_mlp_bwd_mxfp8(m, T, H, F, E, k, zipf):
    d = _mlp_case(T, H, F, E, k, zipf, seed=11)
    ref = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    dz_ref = O.gather_rows(O._as_f64(d["dy"]), ref["src_row"], k)
    rq = O.grouped_mlp_bwd_mxfp8(dz_ref, ref["x_perm"], d["w_gu"],
                                 d["w_dn"], ref["w_perm"], ref["offsets"])
    p, g = _mx_bwd_run(m, d, T, H, F, E, k)
    assert np.array_equal(p["offsets"].cpu().numpy(), ref["offsets"])
    assert_rows_close(host_f64(g["dx_perm"]), rq["dx_perm"], TOL_MX,
                      "dx_perm")
    dx = m.moe_unpermute(g["dx_perm"], p["row_map"], k)
    assert_rows_close(host_f64(dx), O.unpermute(rq["dx_perm"], ref["row_map"],
                                                k), TOL_MX, "dx")
    dwp = g["dw_perm"].cpu().numpy().astype(np.float64)
    assert O.rel_err(dwp, rq["dw_perm"]) <= TOL_MX
    split = np.diff(ref["offsets"])
    gw_gu, gw_dn = host_f64(g["dw_gu"]), host_f64(g["dw_dn"])
    for e in range(E):
        if split[e] == 0:   # no tokens: exactly zero
            assert np.all(gw_gu[e] == 0) and np.all(gw_dn[e] == 0), e
        else:
            assert O.rel_err(gw_gu[e], rq["dw_gu"][e]) <= TOL_MX, e
            assert O.rel_err(gw_dn[e], rq["dw_dn"][e]) <= TOL_MX, e
    assert O.rel_err(gw_gu, rq["dw_gu"]) <= TOL_MX
    assert O.rel_err(gw_dn, rq["dw_dn"]) <= TOL_MX


def test_mxfp8_bwd_prequantised_weights_equal_on_the_fly(m):
    """The MXFP8 backward with the weights quantised once beforehand
    (mxfp8_quantize COLWISE, the reuse contract) gives the bits of the call
    that quantises them itself."""
    T, H, F, E, k = 500, 256, 384, 8, 2
    d = _mlp_case(T, H, F, E, k, 1.2, seed=13)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    f = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], precision=m.PREC_MXFP8,
                              save=True)
    dz = m.moe_gather_rows(dev_bf16(d["dy"]), p["row_map"], k)
    g1 = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                               f["h1"], f["a"], w_perm=p["w_perm"],
                               precision=m.PREC_MXFP8)
    gqt = m.mxfp8_quantize(wgu, m.COLWISE)      # [E, H, 2F] along 2F
    dqt = m.mxfp8_quantize(wdn, m.COLWISE)      # [E, F, H] along H
    g2 = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                               f["h1"], f["a"], w_perm=p["w_perm"],
                               precision=m.PREC_MXFP8, w_gu_qt=gqt,
                               w_dn_qt=dqt)
    for key in ("dx_perm", "dw_gu", "dw_dn"):
        assert torch.equal(g1[key].view(torch.int16),
                           g2[key].view(torch.int16)), key
    assert torch.equal(g1["dw_perm"], g2["dw_perm"])


def test_grouped_mlp_bwd_mxfp8_close_to_bf16(m):
    """The MXFP8 backward approximates the bf16 backward of the same forward
    saves to within the E4M3 quantisation noise (about 2^-4 per operand)."""
    T, H, F, E, k = 512, 256, 256, 4, 2
    d = _mlp_case(T, H, F, E, k, 0.0, seed=12)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    f = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], save=True)
    dz = m.moe_gather_rows(dev_bf16(d["dy"]), p["row_map"], k)
    gb = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                               f["h1"], f["a"], w_perm=p["w_perm"])
    gq = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                               f["h1"], f["a"], w_perm=p["w_perm"],
                               precision=m.PREC_MXFP8)
    for key in ("dx_perm", "dw_gu", "dw_dn"):
        err = O.rel_err(host_f64(gq[key]), host_f64(gb[key]))
        assert 1e-3 < err < 0.12, (key, err)
