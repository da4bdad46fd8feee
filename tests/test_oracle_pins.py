"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against brute force, a closed form, an
independent library routine, or an exact invariant, chosen so that a plausible
slip in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a wrong tie-break, an off-by-one exponent) fails at least one of
them.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import bf16_bits, bf16_to_f64, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- routing
def _brute_route(lrow, k):
    """argmin over every ordered k-tuple of distinct experts of the key list
    [(-l[e0], e0), (-l[e1], e1), ...]: an exhaustive formulation of
    'descending logit, ties to the lower id'."""
    E = len(lrow)
    best, best_key = None, None
    for tup in itertools.permutations(range(E), k):
        key = [(-float(lrow[e]) + 0.0, e) for e in tup]
        if best_key is None or key < best_key:
            best, best_key = tup, key
    return list(best)


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (5, 3), (8, 2), (8, 3),
                                  (6, 6)])
def test_route_brute_force_with_ties(E, k):
    rng = _rng(E * 10 + k)
    # small integer-valued logits force many exact ties; include -0.0
    lg = rng.integers(-2, 3, size=(200, E)).astype(np.float32)
    lg[rng.random(lg.shape) < 0.1] = -0.0
    idx, w = O.route_topk(lg, k)
    for t in range(lg.shape[0]):
        assert list(idx[t]) == _brute_route(lg[t], k)
        # the chosen set maximises the sum of logits over all k-subsets
        best = max(sum(float(lg[t, e]) for e in s)
                   for s in itertools.combinations(range(E), k))
        assert sum(float(lg[t, e]) for e in idx[t]) == best


def test_route_k_equals_E_is_softmax():
    lg = _rng(1).standard_normal((64, 8)).astype(np.float32)
    idx, w = O.route_topk(lg, 8, renormalize=True)
    ref = torch.softmax(torch.from_numpy(lg.astype(np.float64)), dim=1)
    ref = torch.gather(ref, 1, torch.from_numpy(idx.astype(np.int64)))
    np.testing.assert_array_equal(w, ref.numpy().astype(np.float32))
    # sorted descending
    assert np.all(np.diff(np.take_along_axis(lg, idx, 1), axis=1) <= 0)


def test_route_unrenormalised_is_plain_softmax_entries():
    lg = _rng(2).standard_normal((64, 16)).astype(np.float32)
    idx, w = O.route_topk(lg, 4, renormalize=False)
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)), dim=1).numpy()
    ref = np.take_along_axis(p, idx.astype(np.int64), 1).astype(np.float32)
    np.testing.assert_array_equal(w, ref)
    assert np.all(w.sum(1) < 1.0)


def test_route_weights_sum_to_one_and_k1():
    lg = _rng(3).standard_normal((500, 32)).astype(np.float32) * 3
    for k in (2, 4, 8):
        _, w = O.route_topk(lg, k)
        ulp = np.spacing(np.float32(1.0))
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * ulp)
    _, w1 = O.route_topk(lg, 1)
    assert np.all(w1 == np.float32(1.0))


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_route_rejects_nonfinite_logits(bad):
    lg = np.zeros((3, 4), np.float32)
    lg[1, 2] = bad
    with pytest.raises(ValueError):
        O.route_topk(lg, 2)


def test_route_hand_worked_golden():
    """tests/golden/route_hand.json: a routing example worked by hand."""
    with open(os.path.join(GOLDEN, "route_hand.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        lg = np.array(case["logits"], dtype=np.float32)
        idx, w = O.route_topk(lg, case["k"], bool(case["renormalize"]))
        assert idx.tolist() == case["topk_idx"]
        exp = np.array([[eval(s, {"math": math}) for s in row]
                        for row in case["topk_w_expr"]], dtype=np.float64)
        np.testing.assert_array_equal(w, exp.astype(np.float32))


# ------------------------------------------------------------ permutation
def _brute_permute(idx, E):
    """Counting sort written as the definition: walk the pairs in order and
    hand out the next free row of each expert's segment."""
    flat = idx.reshape(-1)
    counts = [0] * E
    for e in flat:
        counts[int(e)] += 1
    starts = [0] * (E + 1)
    for e in range(E):
        starts[e + 1] = starts[e] + counts[e]
    nxt = list(starts[:E])
    row_map = []
    for e in flat:
        row_map.append(nxt[int(e)])
        nxt[int(e)] += 1
    return counts, starts, row_map


@pytest.mark.parametrize("T,E,k,seed", [(37, 5, 2, 0), (100, 16, 4, 1),
                                        (64, 8, 8, 2), (1, 3, 2, 3)])
def test_permute_matches_counting_sort(T, E, k, seed):
    rng = _rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, 0] += 2.0                      # skew: expert 0 popular
    idx, _ = O.route_topk(lg, k)
    m = O.permute_index(idx, E)
    counts, starts, row_map = _brute_permute(idx, E)
    assert m["split_sizes"].tolist() == counts
    assert m["offsets"].tolist() == starts
    assert m["row_map"].tolist() == row_map
    assert int(m["split_sizes"].sum()) == T * k
    assert np.all(np.diff(m["offsets"]) >= 0)
    # bijection, inverse, ascending tokens inside each segment
    assert sorted(m["row_map"].tolist()) == list(range(T * k))
    assert np.array_equal(m["src_row"][m["row_map"]], np.arange(T * k))
    for e in range(E):
        seg = m["src_row"][m["offsets"][e]:m["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(idx.reshape(-1)[seg] == e)


def test_permute_rows_bitwise_and_weights():
    d = generate(50, 64, 32, 6, 3, want=("x", "logits"))
    idx, w = O.route_topk(d["logits"], 3)
    m = O.permute_index(idx, 6)
    xp = O.permute_rows(d["x"], m["src_row"], 3)
    wp = O.permute_weights(w, m["src_row"])
    for p in range(50 * 3):
        assert np.array_equal(xp[m["row_map"][p]], d["x"][p // 3])
        assert wp[m["row_map"][p]] == w.reshape(-1)[p]


@pytest.mark.parametrize("k", [1, 2, 8])
def test_permute_unpermute_identity(k):
    """Unweighted combine of permuted rows == k * x bitwise (k a power of
    two, so the sum and the bf16 rounding are exact); with weights 1/k it is
    x itself."""
    E = 8
    d = generate(40, 48, 32, E, k, want=("x", "logits"))
    idx, _ = O.route_topk(d["logits"], k)
    m = O.permute_index(idx, E)
    xp = O.permute_rows(bf16_to_f64(d["x"]), m["src_row"], k)
    y = O.unpermute(xp, m["row_map"], k)
    x = bf16_to_f64(d["x"])
    assert np.array_equal(y, k * x)
    assert np.array_equal(bf16_bits(y.astype(np.float32)),
                          bf16_bits((k * x).astype(np.float32)))
    y2 = O.unpermute(xp, m["row_map"], k,
                     topk_w=np.full((40, k), 1.0 / k, np.float32))
    assert np.array_equal(y2, x)


def test_permute_rejects_bad_ids():
    with pytest.raises(ValueError):
        O.permute_index(np.array([[0, 5]]), 4)


# --------------------------------------------------------- grouped MLP fwd
def _ffn(x, wgu, wdn, w):
    F = wgu.shape[0] // 2
    h = wgu @ x
    return wdn @ (w * (h[:F] / (1 + np.exp(-h[:F]))) * h[F:])


def _small_layer(T=24, H=32, F=16, E=5, k=2, seed=0, zipf=0.0):
    d = generate(T, H, F, E, k, zipf=zipf, seed=seed,
                 want=("x", "logits", "w_gu", "w_dn", "dy"))
    return d


def test_grouped_equals_per_token_loop():
    """grouped (sorted-token) == per-token eager loop."""
    T, H, F, E, k = 30, 32, 24, 6, 3
    d = _small_layer(T, H, F, E, k, zipf=1.2)
    out = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    x = bf16_to_f64(d["x"])
    wgu = bf16_to_f64(d["w_gu"])
    wdn = bf16_to_f64(d["w_dn"])
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = out["topk_idx"][t, j]
            y[t] += _ffn(x[t], wgu[e], wdn[e], float(out["topk_w"][t, j]))
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-13)


def test_grouped_equals_dense_masked():
    """grouped == the batched form that runs every expert on every token and
    gates the result by a dense [T, E] weight matrix (0 off-route)."""
    T, H, F, E, k = 20, 16, 8, 4, 2
    d = _small_layer(T, H, F, E, k, seed=4)
    out = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    x = torch.from_numpy(bf16_to_f64(d["x"]))
    wgu = torch.from_numpy(bf16_to_f64(d["w_gu"]))
    wdn = torch.from_numpy(bf16_to_f64(d["w_dn"]))
    gate = torch.zeros(T, E, dtype=torch.float64)
    gate.scatter_(1, torch.from_numpy(out["topk_idx"].astype(np.int64)),
                  torch.from_numpy(out["topk_w"].astype(np.float64)))
    h = torch.einsum("th,eoh->eto", x, wgu)                 # [E, T, 2F]
    a = torch.nn.functional.silu(h[..., :F]) * h[..., F:]
    z = torch.einsum("etf,ehf->eth", a, wdn)                # [E, T, H]
    y = (gate.T[..., None] * z).sum(0)
    np.testing.assert_allclose(out["y"], y.numpy(), rtol=1e-10, atol=1e-12)


def test_single_expert_is_dense_swiglu_mlp():
    """E = 1, k = 1: the layer is the textbook SwiGLU MLP (weight 1)."""
    d = _small_layer(T=10, H=16, F=12, E=1, k=1)
    out = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], 1)
    x = torch.from_numpy(bf16_to_f64(d["x"]))
    wg = torch.from_numpy(bf16_to_f64(d["w_gu"][0, :12]))
    wu = torch.from_numpy(bf16_to_f64(d["w_gu"][0, 12:]))
    wd = torch.from_numpy(bf16_to_f64(d["w_dn"][0]))
    F_ = torch.nn.functional
    ref = F_.linear(F_.silu(F_.linear(x, wg)) * F_.linear(x, wu), wd)
    assert np.all(out["topk_w"] == 1.0)
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-14)


def test_linear_in_routing_weight():
    """Scaling w_perm by 2^n scales z by exactly 2^n."""
    d = _small_layer(T=16, H=16, F=8, E=3, k=2)
    idx, w = O.route_topk(d["logits"], 2)
    m = O.permute_index(idx, 3)
    xp = O.permute_rows(d["x"], m["src_row"], 2)
    wp = O.permute_weights(w, m["src_row"]).astype(np.float64)
    z1 = O.grouped_mlp_fwd(xp, d["w_gu"], d["w_dn"], wp, m["offsets"])["z"]
    z2 = O.grouped_mlp_fwd(xp, d["w_gu"], d["w_dn"], wp * 8.0,
                           m["offsets"])["z"]
    assert np.array_equal(z2, 8.0 * z1)


def test_scaled_swiglu_equals_weighted_combine():
    """Weight applied before the down projection == weight at the combine."""
    d = _small_layer(T=16, H=16, F=8, E=4, k=2)
    idx, w = O.route_topk(d["logits"], 2)
    m = O.permute_index(idx, 4)
    xp = O.permute_rows(d["x"], m["src_row"], 2)
    wp = O.permute_weights(w, m["src_row"])
    za = O.grouped_mlp_fwd(xp, d["w_gu"], d["w_dn"], wp, m["offsets"])["z"]
    zb = O.grouped_mlp_fwd(xp, d["w_gu"], d["w_dn"], None, m["offsets"])["z"]
    ya = O.unpermute(za, m["row_map"], 2)
    yb = O.unpermute(zb, m["row_map"], 2, topk_w=w)
    np.testing.assert_allclose(ya, yb, rtol=1e-12, atol=1e-14)


def test_silu_closed_forms():
    z = np.linspace(-30, 30, 1001)
    s = O.silu(z)
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - O.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert abs(O.silu(np.array([-800.0]))[0]) == 0.0
    assert O.silu(np.array([800.0]))[0] == 800.0
    np.testing.assert_allclose(O.sigmoid(z) + O.sigmoid(-z), 1.0, rtol=1e-15)


# -------------------------------------------------------------- backward
def _fwd_fixed_routing(x, w_gu, w_dn, topk_w, idx, k):
    E = w_gu.shape[0]
    m = O.permute_index(idx, E)
    xp = O.permute_rows(x, m["src_row"], k)
    wp = np.asarray(topk_w, np.float64).reshape(-1)[m["src_row"]]
    z = O.grouped_mlp_fwd(xp, w_gu, w_dn, wp, m["offsets"])["z"]
    return O.unpermute(z, m["row_map"], k)


def test_backward_finite_differences():
    T, H, F, E, k = 3, 8, 16, 3, 2
    d = _small_layer(T, H, F, E, k, seed=7)
    x = bf16_to_f64(d["x"])
    wgu = bf16_to_f64(d["w_gu"]) * 10  # larger weights: non-trivial SwiGLU
    wdn = bf16_to_f64(d["w_dn"]) * 10
    dy = bf16_to_f64(d["dy"])
    idx, w = O.route_topk(d["logits"], k)
    w = w.astype(np.float64)
    g = O.layer_bwd(x, d["logits"], wgu, wdn, dy, k)
    eps = 1e-6

    def L(x_, wgu_, wdn_, w_):
        return float((dy * _fwd_fixed_routing(x_, wgu_, wdn_, w_, idx, k)
                      ).sum())

    def fd(arr, setter):
        out = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            p = arr.copy(); p[i] += eps
            m_ = arr.copy(); m_[i] -= eps
            out[i] = (setter(p) - setter(m_)) / (2 * eps)
        return out

    gx = fd(x, lambda v: L(v, wgu, wdn, w))
    np.testing.assert_allclose(g["dx"], gx, rtol=1e-6, atol=1e-8)
    gdn = fd(wdn, lambda v: L(x, wgu, v, w))
    np.testing.assert_allclose(g["dw_dn"], gdn, rtol=1e-6, atol=1e-8)
    ggu = fd(wgu, lambda v: L(x, v, wdn, w))
    np.testing.assert_allclose(g["dw_gu"], ggu, rtol=1e-6, atol=1e-8)
    gw = fd(w, lambda v: L(x, wgu, wdn, v))
    np.testing.assert_allclose(g["dprobs"], gw, rtol=1e-6, atol=1e-8)


def test_backward_adjoint_and_dprobs_closed_form():
    T, H, F, E, k = 12, 16, 8, 4, 2
    d = _small_layer(T, H, F, E, k, seed=9)
    x = bf16_to_f64(d["x"])
    wgu = bf16_to_f64(d["w_gu"]) * 5
    wdn = bf16_to_f64(d["w_dn"]) * 5
    dy = bf16_to_f64(d["dy"])
    g = O.layer_bwd(x, d["logits"], wgu, wdn, dy, k)
    # adjoint: <dY, J v> == <J^T dY, v> along a random direction in x
    idx, w = O.route_topk(d["logits"], k)
    v = _rng(5).standard_normal(x.shape)
    h = 1e-6
    jv = (_fwd_fixed_routing(x + h * v, wgu, wdn, w, idx, k)
          - _fwd_fixed_routing(x - h * v, wgu, wdn, w, idx, k)) / (2 * h)
    assert abs((dy * jv).sum() - (g["dx"] * v).sum()) <= 1e-6 * abs(
        (dy * jv).sum())
    # dprobs[t, j] = <dY_t, FFN_e(x_t; weight 1)>
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            ref = float(dy[t] @ _ffn(x[t], wgu[e], wdn[e], 1.0))
            assert abs(g["dprobs"][t, j] - ref) <= 1e-10 * max(1.0, abs(ref))


def test_backward_zero_token_experts_get_zero_grads():
    T, H, F, E, k = 16, 8, 8, 6, 1
    d = _small_layer(T, H, F, E, k)
    lg = d["logits"].copy()
    lg[:, 2:] -= 100.0          # experts 2..5 never chosen
    g = O.layer_bwd(d["x"], lg, d["w_gu"], d["w_dn"], d["dy"], k)
    assert np.all(g["split_sizes"][2:] == 0)
    assert np.all(g["dw_gu"][2:] == 0) and np.all(g["dw_dn"][2:] == 0)
    assert np.any(g["dw_gu"][:2] != 0)


# ------------------------------------------------------------------ MXFP8
def _e4m3_grid():
    """All finite non-negative E4M3 values from the bit-field definition
    (sign | 4-bit exponent, bias 7 | 3-bit mantissa; exponent 0 subnormal;
    0x7F NaN), computed with Python fractions-free integer arithmetic."""
    vals = []
    for c in range(0x7F):
        ef, m = c >> 3, c & 7
        if ef == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1 + m / 8.0) * 2.0 ** (ef - 7))
    return np.array(vals)


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    np.testing.assert_array_equal(ours[:0x7F], _e4m3_grid())


def test_e4m3_encode_hand_points():
    """tests/golden/e4m3_points.json: codes worked out by hand from the
    format definition (bias 7, 3 mantissa bits, max 448)."""
    with open(os.path.join(GOLDEN, "e4m3_points.json")) as f:
        pts = json.load(f)["points"]
    v = np.array([eval(p[0]) for p in pts], dtype=np.float64)
    want = np.array([int(p[1], 16) for p in pts], dtype=np.uint8)
    np.testing.assert_array_equal(O.e4m3_encode(v), want)


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_e4m3_encode_exhaustive_bf16_times_all_scales():
    """Every finite bf16 value times every 2^-s, s in [-127, 127], encoded
    and compared with a nearest-of-grid search (ties to the even code,
    saturation at 448, sign kept)."""
    grid = _e4m3_grid()                       # 127 ascending values
    mids = (grid[:-1] + grid[1:]) / 2
    v0 = bf16_to_f64(_all_finite_bf16())
    for s in range(-127, 128):
        v = np.ldexp(v0, -s)
        a = np.abs(v)
        j = np.searchsorted(mids, a, side="left")   # a <= mids[j]
        j = np.minimum(j, len(grid) - 1)
        # exact midpoint: searchsorted picked the lower code j where
        # a == mids[j-?]; resolve ties toward the even code
        at_mid = (j < len(mids)) & (a == mids[np.minimum(j, len(mids) - 1)])
        j = np.where(at_mid & (j % 2 == 1), j + 1, j)
        j = np.where(a >= 448.0, 0x7E, j)
        want = (j.astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 7))
        got = O.e4m3_encode(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (s, v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_encode_matches_torch_in_range():
    v0 = bf16_to_f64(_all_finite_bf16())
    for s in (-3, 0, 5, -10, 2):
        v = np.ldexp(v0, -s)
        v = v[np.abs(v) <= 448.0]
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
        np.testing.assert_array_equal(O.e4m3_encode(v), ref)


def test_e8m0_exponent_exhaustive_positive_bf16():
    a = bf16_to_f64(_all_finite_bf16())
    a = np.unique(np.abs(a))
    s = O.e8m0_exponent(a)
    pos = a > 0
    unclamped = pos & (s > -127)
    r = a[unclamped] / np.ldexp(1.0, s[unclamped])
    assert np.all((r >= 256.0) & (r < 512.0))
    assert s[~pos][0] == -127
    # clamped ones really are below the un-clamped threshold 2^-119
    assert np.all(a[pos & (s == -127)] < 2.0 ** -118)
    assert s.max() <= 127


def test_mx_round_trip_exact_on_representable_values():
    rng = _rng(11)
    nb = 4000
    mags = rng.integers(0, 0x7F, size=(nb, 32))           # finite codes
    # force each block's max magnitude into [256, 448] (binade 2^8)
    top = rng.integers(0x78, 0x7F, size=nb)                 # 256 .. 448
    mags[np.arange(nb), rng.integers(0, 32, size=nb)] = top
    mags = np.minimum(mags, np.maximum(top, 0)[:, None])
    codes = (mags | (rng.integers(0, 2, size=mags.shape) << 7)).astype(
        np.uint8)
    s = rng.integers(-100, 100, size=nb)
    V = np.ldexp(O.e4m3_decode(codes), s[:, None])
    c2, sc2 = O.mx_quantize_blocks(V)
    # zero codes with the sign bit come back as signed zeros: same bits
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(sc2.astype(np.int64) - 127, s)
    np.testing.assert_array_equal(O.mx_dequantize_blocks(c2, sc2), V)


def test_mx_quantize_rows_cols_segments_layout():
    rng = _rng(12)
    a = rng.standard_normal((64, 96))
    c, s = O.mxfp8_quantize_rows(a)
    assert c.shape == (64, 96) and s.shape == (64, 3)
    cb, sb = O.mx_quantize_blocks(a[5, 32:64][None, None, :])
    np.testing.assert_array_equal(c[5, 32:64], cb[0, 0])
    assert s[5, 1] == sb[0, 0]
    ct, st = O.mxfp8_quantize_cols(a)
    assert ct.shape == (96, 64) and st.shape == (96, 2)
    cb, sb = O.mx_quantize_blocks(a[32:64, 7][None, None, :])
    np.testing.assert_array_equal(ct[7, 32:64], cb[0, 0])
    off = np.array([0, 10, 10, 64])
    cs, ss = O.mxfp8_quantize_segments(a, off)
    po = O.padded_offsets(off)
    assert po.tolist() == [0, 32, 32, 96]
    assert cs.shape == (96, 96) and ss.shape == (96, 3)
    blk = np.zeros(32)
    blk[:10] = a[0:10, 3]
    cb, sb = O.mx_quantize_blocks(blk[None, None, :])
    np.testing.assert_array_equal(cs[3, 0:32], cb[0, 0])
    assert ss[3, 0] == sb[0, 0]
    assert np.all(cs[3, 10:32] == 0)


def test_mx_gemm_equals_exact_gemm_on_representable_operands():
    """MXFP8 layer GEMM on operands that are exactly representable equals the
    plain float64 GEMM on those values."""
    rng = _rng(13)
    M, K, N = 16, 64, 8

    def rep(shape):
        nb = shape[0] * shape[1] // 32
        mags = rng.integers(0, 0x78, size=(nb, 32))
        mags[:, 0] = rng.integers(0x78, 0x7F, size=nb)
        codes = (mags | (rng.integers(0, 2, size=mags.shape) << 7))
        s = rng.integers(-10, 0, size=nb)
        return np.ldexp(O.e4m3_decode(codes), s[:, None]).reshape(shape)

    X = rep((M, K))
    W = rep((N, K))
    Xq = O._mx_rows(X)
    Wq = O._mx_rows(W)
    assert np.array_equal(Xq, X) and np.array_equal(Wq, W)
    np.testing.assert_allclose(Xq @ Wq.T, X @ W.T, rtol=0, atol=0)


# ------------------------------------------- MXFP8 layer: exact, by direction
# Operands built block by block from E4M3 codes times a power of two, so that
# quantising along the intended axis returns them unchanged (the round trip
# pinned above), while quantising along the other axis does not (blocks of
# that axis mix scales 2^0 .. 2^-4, so small values lose bits).  Values are
# multiples of 2^-13 below 448, products multiples of 2^-26 below 2^18: every
# float64 sum of up to 2^8 products is exact in any order.

def _rep_blocks(rng, n_blocks, valid=32, smin=-4, smax=0):
    """[n_blocks, 32] float64: each block decode(code) * 2^s with one element
    of magnitude in [256, 448] * 2^s among its first ``valid`` entries and
    zeros past them."""
    mags = rng.integers(0, 0x7F, size=(n_blocks, 32))
    top = rng.integers(0x78, 0x7F, size=n_blocks)
    mags = np.minimum(mags, top[:, None])
    mags[np.arange(n_blocks), rng.integers(0, valid, size=n_blocks)] = top
    codes = mags | (rng.integers(0, 2, size=mags.shape) << 7)
    s = rng.integers(smin, smax + 1, size=n_blocks)
    v = np.ldexp(O.e4m3_decode(codes), s[:, None])
    v[:, valid:] = 0.0
    return v


def _rep_rows(rng, R, C):
    """[R, C] exactly representable with blocks of 32 along each row."""
    return _rep_blocks(rng, R * (C // 32)).reshape(R, C)


def _rep_token_segments(rng, offsets, C):
    """[rows, C], exactly representable along tokens with blocks restarting
    at every offsets[e] (last block of a segment zero-padded)."""
    rows = int(offsets[-1])
    out = np.zeros((rows, C))
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for b0 in range(lo, hi, 32):
            n = min(32, hi - b0)
            out[b0:b0 + n] = _rep_blocks(rng, C, valid=n)[:, :n].T
    return out


def _q_rows(a):
    c, s = O.mxfp8_quantize_rows(a)
    R, C = c.shape
    return O.mx_dequantize_blocks(c.reshape(R, C // 32, 32), s).reshape(R, C)


def test_rep_operands_are_direction_sensitive():
    """The constructions above are exact along their axis only."""
    rng = _rng(60)
    a = _rep_rows(rng, 64, 128)
    assert np.array_equal(_q_rows(a), a)
    assert not np.array_equal(_q_rows(a.T).T, a)
    off = np.array([0, 20, 20, 75])
    t = _rep_token_segments(rng, off, 64)
    for e in range(3):
        lo, hi = off[e], off[e + 1]
        n = hi - lo
        pad = np.zeros((-(-n // 32) * 32, 64))
        pad[:n] = t[lo:hi]
        assert np.array_equal(_q_rows(pad.T).T[:n], t[lo:hi])
    glob = np.zeros((96, 64))
    glob[:75] = t
    assert not np.array_equal(_q_rows(glob.T).T[:75], t)


def test_mx_gemm_rows_exact_along_k_only():
    rng = _rng(61)
    a = _rep_rows(rng, 64, 256)
    b = _rep_rows(rng, 32, 256)
    c = O.mx_gemm_rows(a, b)
    np.testing.assert_array_equal(c, a @ b.T)
    # the same operands blocked along M / N would not give the product
    wrong = _q_rows(a.T).T @ _q_rows(b.T).T.T
    assert O.rel_err(wrong, a @ b.T) > 1e-4


def test_mx_dgrad_quantises_weights_along_n():
    """dX = Q_N(dY) Q_N(W), W [N, K]: W representable along N (its columns)
    but not along K gives the exact product; the row-wise reading of W
    (blocks along K) does not."""
    rng = _rng(62)
    N, K, M = 128, 96, 64
    dy = _rep_rows(rng, M, N)
    w = _rep_rows(rng, K, N).T.copy()          # [N, K], exact along N
    np.testing.assert_array_equal(O.mx_dgrad(dy, w), dy @ w)
    assert not np.array_equal(_q_rows(w), w)
    assert O.rel_err(_q_rows(dy) @ _q_rows(w), dy @ w) > 1e-4


@pytest.mark.parametrize("offsets", [[0, 20, 20, 75], [0, 0, 45, 77, 160]])
def test_mx_wgrad_segment_blocks_restart_at_segment(offsets):
    """Token-direction blocks start at each expert's first row (here rows 20
    and 45 and 77: inside a 32-row block of the whole tensor) and the last
    block is zero-padded; operands representable in those blocks give the
    exact dW, and blocks aligned to the whole tensor would not."""
    rng = _rng(63)
    off = np.array(offsets)
    M, N = 64, 96
    a = _rep_token_segments(rng, off, M)
    b = _rep_token_segments(rng, off, N)
    rows = int(off[-1])
    ga = np.zeros((-(-rows // 32) * 32, M))
    gb = np.zeros((ga.shape[0], N))
    ga[:rows], gb[:rows] = a, b
    qa, qb = _q_rows(ga.T).T[:rows], _q_rows(gb.T).T[:rows]
    moved = False
    for e in range(len(off) - 1):
        lo, hi = off[e], off[e + 1]
        dw = O.mx_wgrad_segment(a, b, off, e)
        np.testing.assert_array_equal(dw, a[lo:hi].T @ b[lo:hi])
        if hi > lo and lo % 32:
            moved |= O.rel_err(qa[lo:hi].T @ qb[lo:hi],
                               a[lo:hi].T @ b[lo:hi]) > 1e-4
        if hi == lo:
            assert dw.shape == (M, N) and not dw.any()
    assert moved


def test_mxfp8_forward_exact_h1_and_quantised_a():
    """grouped_mlp_fwd_mxfp8 with x_perm and W_gu representable along H and
    W_dn representable along F (none of them along the other axis):
      h1 equals the float64 product exactly;
      a equals w * silu(g) * u on that h1;
      z equals Q_F(a) W_dn^T (a quantised row-wise, W_dn unchanged).
    Quantising W_dn along H, skipping A's quantisation or quantising x_perm
    along tokens fails by far more than rounding."""
    rng = _rng(64)
    E, H, F = 3, 128, 64
    off = np.array([0, 37, 37, 90])
    rows = int(off[-1])
    x = _rep_rows(rng, rows, H)
    w_gu = np.stack([_rep_rows(rng, 2 * F, H) for _ in range(E)])
    w_dn = np.stack([_rep_rows(rng, H, F) for _ in range(E)])
    for e in range(E):
        assert not np.array_equal(_q_rows(w_dn[e].T).T, w_dn[e])
    wp = np.ldexp(1.0, -rng.integers(0, 3, size=rows))  # 1, 1/2, 1/4
    out = O.grouped_mlp_fwd_mxfp8(x, w_gu, w_dn, wp, off, keep=True)
    z_unq = np.zeros_like(out["z"])
    z_dn_h = np.zeros_like(out["z"])
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        h1 = x[lo:hi] @ w_gu[e].T
        np.testing.assert_array_equal(out["h1"][lo:hi], h1)
        g, u = h1[:, :F], h1[:, F:]
        np.testing.assert_array_equal(out["a"][lo:hi],
                                      wp[lo:hi, None] * O.silu(g) * u)
        aq = _q_rows(out["a"][lo:hi])
        np.testing.assert_allclose(out["z"][lo:hi], aq @ w_dn[e].T,
                                   rtol=1e-12, atol=0)
        z_unq[lo:hi] = out["a"][lo:hi] @ w_dn[e].T
        z_dn_h[lo:hi] = aq @ _q_rows(w_dn[e].T).T.T
    assert O.rel_err(z_unq, out["z"]) > 1e-3
    assert O.rel_err(z_dn_h, out["z"]) > 1e-3
    assert not out["z"][0:0].size and not out["z"][37:37].size


def test_mxfp8_backward_is_its_pinned_gemms():
    """grouped_mlp_bwd_mxfp8 composes the pinned pieces expert by expert:
    dA = mx_dgrad(dZ, W_dn), (dH1, dw) = swiglu_bwd (pinned through the
    float64 backward's finite differences), dX = mx_dgrad(dH1, W_gu),
    dW_dn = mx_wgrad_segment(dZ, A), dW_gu = mx_wgrad_segment(dH1, X), with
    (g, u) and A from the MXFP8 forward.  An expert boundary at row 21 falls
    inside a 32-row block; an expert without tokens gets dW = 0."""
    rng = _rng(65)
    E, H, F = 4, 64, 32
    off = np.array([0, 21, 21, 58, 70])
    rows = int(off[-1])
    x = rng.standard_normal((rows, H))
    w_gu = 0.1 * rng.standard_normal((E, 2 * F, H))
    w_dn = 0.1 * rng.standard_normal((E, H, F))
    wp = rng.random(rows)
    dz = rng.standard_normal((rows, H))
    got = O.grouped_mlp_bwd_mxfp8(dz, x, w_gu, w_dn, wp, off)
    fwd = O.grouped_mlp_fwd_mxfp8(x, w_gu, w_dn, wp, off, keep=True)
    dh1 = np.zeros((rows, 2 * F))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            assert not got["dw_dn"][e].any() and not got["dw_gu"][e].any()
            continue
        g, u = fwd["h1"][lo:hi, :F], fwd["h1"][lo:hi, F:]
        da = O.mx_dgrad(dz[lo:hi], w_dn[e])
        dh1[lo:hi], dwp = O.swiglu_bwd(da, g, u, wp[lo:hi, None])
        np.testing.assert_array_equal(got["dw_perm"][lo:hi], dwp)
        np.testing.assert_array_equal(got["dx_perm"][lo:hi],
                                      O.mx_dgrad(dh1[lo:hi], w_gu[e]))
    for e in range(E):
        np.testing.assert_array_equal(
            got["dw_dn"][e], O.mx_wgrad_segment(dz, fwd["a"], off, e))
        np.testing.assert_array_equal(
            got["dw_gu"][e], O.mx_wgrad_segment(dh1, x, off, e))


def test_swiglu_bwd_matches_finite_differences():
    """d/d(g, u, w) of sum(dA * w * silu(g) * u), central differences."""
    rng = _rng(66)
    g, u = rng.standard_normal((5, 7)), rng.standard_normal((5, 7))
    w = rng.random((5, 1)) + 0.5
    da = rng.standard_normal((5, 7))
    dh1, dw = O.swiglu_bwd(da, g, u, w)

    def f(g_, u_, w_):
        return float((da * w_ * O.silu(g_) * u_).sum())

    h = 1e-6
    for (i, j) in [(0, 0), (2, 3), (4, 6)]:
        for which, col in ((0, j), (1, 7 + j)):
            gp, up, gm, um = g.copy(), u.copy(), g.copy(), u.copy()
            if which == 0:
                gp[i, j] += h
                gm[i, j] -= h
            else:
                up[i, j] += h
                um[i, j] -= h
            fd = (f(gp, up, w) - f(gm, um, w)) / (2 * h)
            assert abs(fd - dh1[i, col]) < 1e-7 * max(1.0, abs(fd))
        wp_, wm_ = w.copy(), w.copy()
        wp_[i] += h
        wm_[i] -= h
    for i in range(5):
        wp_, wm_ = w.copy(), w.copy()
        wp_[i] += h
        wm_[i] -= h
        fd = (f(g, u, wp_) - f(g, u, wm_)) / (2 * h)
        assert abs(fd - dw[i]) < 1e-7 * max(1.0, abs(fd))


def test_mx_fast_equals_numpy_oracle_every_bf16_and_scale():
    """The C restatement of R7 (oracle/mx_fast.c) gives the numpy oracle's
    codes and scales bit for bit: every finite bf16 pattern, in blocks whose
    amax sets each reachable scale exponent, plus all-zero and tiny
    blocks."""
    from oracle import mx_fast
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(68)
    rows = []
    for be in range(0, 255, 3):          # block amax exponent field
        perm = rng.permutation(bits)[: 31 * 64]
        blk = perm.reshape(64, 31)
        lead = np.full((64, 1), (be << 7) | 0x7F, dtype=np.uint16)
        # keep the other values at or below the lead's magnitude
        mag = blk & 0x7FFF
        blk = np.where(mag > (lead & 0x7FFF), blk & 0x8000, blk)
        rows.append(np.concatenate([lead, blk.astype(np.uint16)], axis=1))
    rows.append(np.zeros((2, 32), dtype=np.uint16))
    rows.append(np.full((2, 32), 0x8001, dtype=np.uint16))
    a = np.concatenate(rows, axis=0).reshape(-1, 64)
    c, s = mx_fast.quantize_rows(a)
    cw, sw = O.mxfp8_quantize_rows(a)
    np.testing.assert_array_equal(c, cw)
    np.testing.assert_array_equal(s, sw)
    np.testing.assert_array_equal(mx_fast.dequantized_rows(a), O._mx_rows_np(a))
    np.testing.assert_array_equal(O._mx_rows(a), O._mx_rows_np(a))
    assert len(np.unique(sw)) > 80


def test_mxfp8_layer_close_to_unquantised():
    """Sanity: the MXFP8 layer tracks the unquantised one (normwise error of
    a few percent, the format's resolution), and equals it exactly when every
    operand is representable is covered above."""
    T, H, F, E, k = 64, 128, 64, 4, 2
    d = _small_layer(T, H, F, E, k, seed=3)
    fwd = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    zq = O.grouped_mlp_fwd_mxfp8(fwd["x_perm"], d["w_gu"], d["w_dn"],
                                 fwd["w_perm"], fwd["offsets"])["z"]
    err = O.rel_err(zq, fwd["z"])
    assert 0.005 < err < 0.15


def test_mxfp8_backward_tracks_bf16_backward():
    T, H, F, E, k = 48, 64, 64, 3, 2
    d = _small_layer(T, H, F, E, k, seed=5)
    fwd = O.layer_fwd(d["x"], d["logits"], d["w_gu"], d["w_dn"], k)
    dz = O.gather_rows(bf16_to_f64(d["dy"]), fwd["src_row"], k)
    a = O.grouped_mlp_bwd(dz, fwd["x_perm"], d["w_gu"], d["w_dn"],
                          fwd["w_perm"], fwd["offsets"])
    b = O.grouped_mlp_bwd_mxfp8(dz, fwd["x_perm"], d["w_gu"], d["w_dn"],
                                fwd["w_perm"], fwd["offsets"])
    for key in ("dx_perm", "dw_gu", "dw_dn", "dw_perm"):
        assert O.rel_err(b[key], a[key]) < 0.2, key


def test_accounting_flops_and_rows():
    from synthetic import CONFIGS
    c = CONFIGS["mixtral"]
    assert c.rows == 16384
    assert abs(c.fwd_flop() - 5.772e12) / 5.772e12 < 1e-3
    q = CONFIGS["qwen3_long"]
    assert abs(q.bwd_flop() - 4.948e12) / 4.948e12 < 1e-3


# ---------------------------------------------------------------- router
def _small_int_bf16(rng, shape, lo=-8, hi=8):
    """bf16 bit patterns of small integers (exact in bf16)."""
    return bf16_bits(rng.integers(lo, hi + 1, shape).astype(np.float32))


def test_router_logits_exact_on_integer_operands():
    """Small-integer operands keep every partial sum exact, so the logits
    are the integer matrix product (plus a dyadic bias), whatever the
    summation order: catches a dropped term or a transposed operand."""
    rng = np.random.default_rng(40)
    T, H, E = 37, 96, 11
    x = _small_int_bf16(rng, (T, H))
    w = _small_int_bf16(rng, (E, H))
    bias = rng.integers(-4, 5, E).astype(np.float64) * 0.25
    got = O.router_logits(x, w, bias)
    xi = bf16_to_f64(x).astype(np.int64)
    wi = bf16_to_f64(w).astype(np.int64)
    want = (xi @ wi.T).astype(np.float64) + bias[None, :]
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got.astype(np.float64), want)


def test_router_logits_single_rounding_to_float32():
    """The float64 sum is rounded to float32 once: 1 + 2^-30 summed from
    exact bf16 terms stays 1 in float32, and 2^24 + 1 rounds to even."""
    one = bf16_bits(np.array([[1.0, 2.0 ** -30]], np.float32))
    w = bf16_bits(np.array([[1.0, 1.0]], np.float32))
    assert O.router_logits(one, w)[0, 0] == np.float32(1.0)
    big = bf16_bits(np.array([[2.0 ** 24, 1.0]], np.float32))
    assert O.router_logits(big, w)[0, 0] == np.float32(2.0 ** 24)
    big3 = bf16_bits(np.array([[2.0 ** 24, 1.0, 2.0]], np.float32))
    w3 = bf16_bits(np.array([[1.0, 1.0, 1.0]], np.float32))
    assert O.router_logits(big3, w3)[0, 0] == np.float32(2.0 ** 24 + 4)


@pytest.mark.parametrize("renorm", [True, False])
def test_router_bwd_finite_differences(renorm):
    """dlogits is the derivative of L = sum_j dw_j * w_j(logits) with the
    selected set held fixed (central differences in float64)."""
    rng = np.random.default_rng(41)
    T, E, k = 5, 9, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    dw = rng.standard_normal((T, k))
    idx, _ = O.route_topk(lg, k, renorm)
    dl = O.router_bwd(lg, idx, dw, renorm)
    lv = lg.astype(np.float64)

    def loss(l):
        tot = 0.0
        for t in range(T):
            ex = np.exp(l[t] - l[t].max())
            S = idx[t]
            den = ex[S].sum() if renorm else ex.sum()
            tot += float((dw[t] * ex[S] / den).sum())
        return tot

    eps = 1e-6
    for t in range(T):
        for e in range(E):
            lp, lm = lv.copy(), lv.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            num = (loss(lp) - loss(lm)) / (2 * eps)
            assert abs(num - dl[t, e]) < 1e-7, (t, e, num, dl[t, e])


@pytest.mark.parametrize("renorm", [True, False])
def test_router_bwd_rows_sum_to_zero_and_support(renorm):
    """Softmax Jacobian rows sum to zero; with renormalisation the gradient
    lives on the chosen set only; k = E without renormalisation is the
    plain softmax backward."""
    rng = np.random.default_rng(42)
    T, E, k = 40, 16, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    dw = rng.standard_normal((T, k))
    idx, w = O.route_topk(lg, k, renorm)
    dl = O.router_bwd(lg, idx, dw, renorm)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-14)
    if renorm:
        mask = np.zeros((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
        assert np.all(dl[~mask] == 0.0)
    else:
        idx_all, p = O.route_topk(lg, E, False)
        g = np.zeros((T, E))
        np.put_along_axis(g, idx_all.astype(np.int64),
                          rng.standard_normal((T, E)), axis=1)
        ga = np.take_along_axis(g, idx_all.astype(np.int64), axis=1)
        dla = O.router_bwd(lg, idx_all, ga, False)
        pe = np.exp(lg - lg.max(axis=1, keepdims=True).astype(np.float64))
        pe = pe / pe.sum(axis=1, keepdims=True)
        want = pe * (g - (pe * g).sum(axis=1, keepdims=True))
        np.testing.assert_allclose(dla, want, rtol=1e-12, atol=1e-15)


def test_router_weight_grads_adjoint():
    """<dl, x W^T> is bilinear: its derivatives w.r.t. W and x are
    dl^T x and dl W (checked entry by entry with exact perturbations)."""
    rng = np.random.default_rng(43)
    T, H, E = 6, 10, 4
    x = rng.standard_normal((T, H))
    w = rng.standard_normal((E, H))
    dl = rng.standard_normal((T, E))
    dW, dx = O.router_weight_grads(dl, x, w)
    base = float((dl * (x @ w.T)).sum())
    for e in range(E):
        for h in range(H):
            w2 = w.copy()
            w2[e, h] += 1.0
            assert abs(float((dl * (x @ w2.T)).sum()) - base - dW[e, h]) < 1e-9
    for t in range(T):
        for h in range(H):
            x2 = x.copy()
            x2[t, h] += 1.0
            assert abs(float((dl * (x2 @ w.T)).sum()) - base - dx[t, h]) < 1e-9


# ------------------------------------------------------ tensor-scaled FP8
def test_fp8_tensor_round_trip_exact_with_power_of_two_scale():
    """Values decode(c) * 2^k with one of them at 448 * 2^k: the scale is
    2^k exactly and every code comes back."""
    rng = np.random.default_rng(50)
    codes = rng.integers(0, 256, 4000).astype(np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]          # no NaN codes
    codes[0] = 0x7E                                 # +448
    for k in (-20, -3, 0, 5):
        v = O.e4m3_decode(codes) * 2.0 ** k
        c2, s = O.fp8_tensor_quantize(v.astype(np.float32))
        assert s == np.float32(2.0 ** k)
        # equal codes, except that -0 and +0 both decode to zero
        d = O.e4m3_decode(c2) * 2.0 ** k
        np.testing.assert_array_equal(d, v)


def test_fp8_tensor_scale_and_error_bound():
    rng = np.random.default_rng(51)
    v = (rng.standard_normal(5000) * 3.7).astype(np.float32)
    c, s = O.fp8_tensor_quantize(v)
    amax = np.abs(v).max()
    assert s == np.float32(np.float32(amax) / np.float32(448.0))
    assert (c & 0x7F).max() == 0x7E               # the amax lands on 448
    d = O.fp8_tensor_dequantize(c, s)
    a = np.abs(v.astype(np.float64))
    normal = a / s >= 2.0 ** -6
    # 3 mantissa bits: half an ulp is 2^-4 relative on the normal grid,
    # 2^-10 * s absolute on the subnormal one
    assert np.all(np.abs(d - v)[normal] <= 2.0 ** -4 * a[normal] * (1 + 1e-6))
    assert np.all(np.abs(d - v)[~normal] <= 2.0 ** -10 * s * (1 + 1e-6))
    # an all-zero tensor has scale 1 and zero codes
    c0, s0 = O.fp8_tensor_quantize(np.zeros(64, np.float32))
    assert s0 == 1.0 and not np.any(c0 & 0x7F)


def test_bf16_round_bits_matches_torch():
    rng = np.random.default_rng(52)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))
    np.testing.assert_array_equal(O._bf16_round_bits(v),
                                  bf16_bits(v.astype(np.float32)))


def _fp8_rep(rng, shape, k):
    """decode(code) * 2^k with one element at +448 * 2^k (so the tensor's
    scale amax / 448 is exactly 2^k) and many small codes, subnormals
    included."""
    c = rng.integers(0, 0x7E, size=shape)
    c = np.where(rng.random(shape) < 0.3, rng.integers(1, 0x10, size=shape),
                 c)
    c = c | (rng.integers(0, 2, size=shape) << 7)
    v = np.ldexp(O.e4m3_decode(c), k)
    v.reshape(-1)[rng.integers(0, v.size)] = 448.0 * 2.0 ** k
    return v


def test_fp8_tensor_layer_scales_per_expert_weight_and_whole_a():
    """R11 on operands whose per-tensor scales are powers of two: x_perm at
    2^-8, expert 0's weights at 2^-8 and expert 1's at 2^-16 (amax 2^8 apart,
    small codes in both).  Each expert's own scale leaves its weights exact,
    so h1 is the exact float64 product; one scale shared by both experts
    would flush expert 1's small values.  A is the bf16 SwiGLU output and z
    its quantisation with ONE scale over all rows (amax of the whole bf16
    A) times W_dn[e]."""
    rng = _rng(67)
    E, H, F = 2, 64, 32
    off = np.array([0, 23, 50])
    rows = int(off[-1])
    x = _fp8_rep(rng, (rows, H), -8)
    w_gu = np.stack([_fp8_rep(rng, (2 * F, H), -8),
                     _fp8_rep(rng, (2 * F, H), -16)])
    w_dn = np.stack([_fp8_rep(rng, (H, F), -8), _fp8_rep(rng, (H, F), -16)])
    wp = rng.random(rows).astype(np.float32).astype(np.float64)
    out = O.grouped_mlp_fwd_fp8_tensor(x.astype(np.float32), w_gu, w_dn, wp,
                                       off)
    shared = np.ldexp(O.e4m3_decode(O.e4m3_encode(w_gu[1] / 2.0 ** -8)), -8)
    assert not np.array_equal(shared, w_gu[1])     # flushes under 2^-8
    a16 = np.zeros((rows, F))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        h1 = x[lo:hi] @ w_gu[e].T
        np.testing.assert_array_equal(out["h1"][lo:hi], h1)
        a16[lo:hi] = bf16_to_f64(O._bf16_round_bits(
            wp[lo:hi, None] * O.silu(h1[:, :F]) * h1[:, F:]))
    np.testing.assert_array_equal(out["a"], a16)
    ac, as_ = O.fp8_tensor_quantize(a16)
    assert as_ == np.float32(np.abs(a16).max() / 448.0)
    aq = O.fp8_tensor_dequantize(ac, as_)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        np.testing.assert_allclose(out["z"][lo:hi], aq[lo:hi] @ w_dn[e].T,
                                   rtol=1e-12, atol=0)
        # a per-expert A scale would change expert 1's rows
        pc, ps = O.fp8_tensor_quantize(a16[lo:hi])
        if e == 1:
            assert O.rel_err(O.fp8_tensor_dequantize(pc, ps) @ w_dn[e].T,
                             out["z"][lo:hi]) > 1e-3


def test_fp8_tensor_layer_close_to_unquantised():
    T, H, F, E, k = 256, 128, 256, 8, 2
    d = generate(T, H, F, E, k, seed=4, want=("x", "logits", "w_gu", "w_dn"))
    idx, w = O.route_topk(d["logits"], k)
    maps = O.permute_index(idx, E)
    xp = O.permute_rows(d["x"], maps["src_row"], k)
    wp = O.permute_weights(w, maps["src_row"])
    ref = O.grouped_mlp_fwd(xp, d["w_gu"], d["w_dn"], wp, maps["offsets"])
    q = O.grouped_mlp_fwd_fp8_tensor(xp, d["w_gu"], d["w_dn"], wp,
                                     maps["offsets"])
    err = O.rel_err(q["z"], ref["z"])
    assert 1e-3 < err < 0.12, err
