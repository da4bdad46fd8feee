"""GPU parity of the tensor-scaled FP8 mode (one float32 scale per tensor,
E4M3 codes) against the oracle.

Bars: codes and scales of the quantiser bit-exact; the layer output within
6e-2 normwise of the oracle running the same algorithm (its A, and so A's
scale, comes from GEMMs summed in a different order); at full size, the
layer stays within quantisation noise of the bf16 layer.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import CONFIGS, bf16_bits, bf16_to_f64, generate, \
    generate_config

pytestmark = pytest.mark.gpu

TOL_8BIT = 6e-2


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


def host_f64(t):
    return bf16_to_f64(t.detach().cpu().view(torch.int16).numpy().view(
        np.uint16))


@pytest.mark.parametrize("n_seg,seg", [(1, 4096), (8, 1024), (3, 8),
                                       (5, 65536)])
def test_fp8_tensor_quantize_bit_exact(m, n_seg, seg):
    rng = np.random.default_rng(n_seg * 7 + seg)
    v = (rng.standard_normal((n_seg, seg)) *
         np.exp2(rng.integers(-12, 12, (n_seg, 1)))).astype(np.float32)
    v[:, :3] = v[:, :3] * 1e-30           # values on the subnormal grid
    if n_seg > 2:
        v[1] = 0.0                          # an all-zero tensor: scale 1
    bits = bf16_bits(v)
    codes, scales = m.fp8_tensor_quantize(dev_bf16(bits), n_seg)
    codes = codes.cpu().numpy().reshape(n_seg, seg)
    scales = scales.cpu().numpy()
    for i in range(n_seg):
        rc, rs = O.fp8_tensor_quantize(bits[i])
        assert scales[i] == rs, (i, scales[i], rs)
        np.testing.assert_array_equal(codes[i], rc)


FP8T_CASES = [
    # T, H, F, E, k, zipf
    (256, 128, 256, 8, 2, 0.0),
    (700, 256, 384, 5, 2, 1.2),     # ragged M, F not a multiple of 256
    (900, 128, 128, 16, 4, 1.2),    # many experts, some empty
    (512, 256, 8192, 4, 2, 0.0),    # down GEMM's last tiles split along K
    # the gate/up GEMM's five-buffer rotation: K steps of 128 (nk = H / 128)
    # in whole trips of five plus a tail of nk % 5 steps
    (300, 640, 256, 4, 2, 1.2),     # nk = 5: one trip, no tail
    (200, 768, 256, 3, 1, 0.0),     # nk = 6: one trip, tail of one
    (300, 1152, 128, 4, 2, 0.0),    # nk = 9: one trip, tail of four
    (260, 1920, 128, 5, 2, 1.2),    # nk = 15: three trips, no tail
    # the down GEMM's rotation (nk = F / 128)
    (300, 256, 640, 4, 2, 1.2),     # nk = 5
    (300, 256, 1152, 4, 2, 0.0),    # nk = 9
]


@pytest.mark.parametrize("T,H,F,E,k,zipf", FP8T_CASES)
def test_fp8_tensor_layer_fwd(m, T, H, F, E, k, zipf):
    d = generate(T, H, F, E, k, zipf=zipf, seed=5,
                 want=("x", "logits", "w_gu", "w_dn"))
    idx, w = O.route_topk(d["logits"], k)
    maps = O.permute_index(idx, E)
    xp = O.permute_rows(d["x"], maps["src_row"], k)
    wp = O.permute_weights(w, maps["src_row"])
    ref = O.grouped_mlp_fwd_fp8_tensor(xp, d["w_gu"], d["w_dn"], wp,
                                       maps["offsets"])
    r = m.moe_grouped_mlp_fwd(dev_bf16(xp), dev_bf16(d["w_gu"]),
                              dev_bf16(d["w_dn"]),
                              torch.from_numpy(maps["offsets"]).cuda(),
                              w_perm=torch.from_numpy(wp).cuda(),
                              precision=m.PREC_FP8_TENSOR, save=True)
    assert O.rel_err(host_f64(r["z"]), ref["z"]) <= TOL_8BIT
    assert O.rel_err(host_f64(r["a"]), ref["a"]) <= TOL_8BIT
    # and close to the unquantised layer
    bf = O.grouped_mlp_fwd(xp, d["w_gu"], d["w_dn"], wp, maps["offsets"])
    err = O.rel_err(host_f64(r["z"]), bf["z"])
    assert 1e-3 < err < 0.12, err


def test_fp8_tensor_full_size_close_to_bf16(m):
    cfg = CONFIGS["mixtral"]
    d = generate_config(cfg, seed=0)
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), cfg.k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, cfg.E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    q = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"],
                              precision=m.PREC_FP8_TENSOR)
    b = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"])
    err = O.rel_err(host_f64(q["z"]), host_f64(b["z"]))
    assert 1e-3 < err < 0.12, err


def test_fp8_tensor_backward_is_rejected(m):
    T, H, F, E, k = 64, 128, 128, 4, 1
    d = generate(T, H, F, E, k, seed=6, want=("x", "w_gu", "w_dn", "dy"))
    x = dev_bf16(d["x"])
    off = torch.tensor([0, 16, 32, 48, 64], dtype=torch.int32, device="cuda")
    h1 = torch.zeros((T, 2 * F), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((T, F), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MoEError):
        m.moe_grouped_mlp_bwd(dev_bf16(d["dy"]), x, dev_bf16(d["w_gu"]),
                              dev_bf16(d["w_dn"]), off, h1, a,
                              precision=m.PREC_FP8_TENSOR)


@pytest.mark.parametrize("T,H,F,E,k,zipf", [(700, 256, 384, 5, 2, 1.2),
                                           (512, 256, 8192, 4, 2, 0.0)])
def test_fp8_tensor_prequantised_weights_equal_on_the_fly(m, T, H, F, E, k,
                                                          zipf):
    """The forward with the weights quantised once beforehand
    (fp8_tensor_quantize with one tensor per expert, the reuse contract)
    gives the bits of the call that quantises them itself; the weights'
    codes and scales equal the oracle's."""
    d = generate(T, H, F, E, k, zipf=zipf, seed=9,
                 want=("x", "logits", "w_gu", "w_dn"))
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    r1 = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                               w_perm=p["w_perm"],
                               precision=m.PREC_FP8_TENSOR, save=True)
    gq = m.fp8_tensor_quantize(wgu, E)
    dq = m.fp8_tensor_quantize(wdn, E)
    rc, rs = O.fp8_tensor_quantize(d["w_gu"][1])
    np.testing.assert_array_equal(gq[0][1].cpu().numpy().ravel(),
                                  np.asarray(rc).ravel())
    assert gq[1][1].item() == rs
    r2 = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                               w_perm=p["w_perm"],
                               precision=m.PREC_FP8_TENSOR, save=True,
                               w_gu_q=gq, w_dn_q=dq)
    for key in ("z", "h1", "a"):
        assert torch.equal(r1[key].view(torch.int16),
                           r2[key].view(torch.int16)), key


def test_fp8_tensor_prequantised_weights_need_both(m):
    T, H, F, E, k = 64, 128, 128, 4, 1
    d = generate(T, H, F, E, k, seed=6, want=("x", "w_gu", "w_dn"))
    off = torch.tensor([0, 16, 32, 48, 64], dtype=torch.int32, device="cuda")
    wgu = dev_bf16(d["w_gu"])
    with pytest.raises(m.MoEError):
        m.moe_grouped_mlp_fwd(dev_bf16(d["x"]), wgu, dev_bf16(d["w_dn"]),
                              off, precision=m.PREC_FP8_TENSOR,
                              w_gu_q=m.fp8_tensor_quantize(wgu, E))
