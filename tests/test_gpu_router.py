"""GPU parity of the router projection and router backward against the
oracle.

Bars: logits bit for bit (float64 accumulation in ascending h, one float32
rounding, on both sides), so the routing decided on them is bit-exact too;
dlogits (float64 inside, stored float32) elementwise within 1e-5 relative
(+1e-12 absolute); dW_r and the router's dx (float32 accumulation) within
1e-4 normwise.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import CONFIGS, bf16_bits, generate, generate_config

pytestmark = pytest.mark.gpu


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


def _inputs(T, H, E, seed):
    d = generate(T, H, 64, E, 1, seed=seed, want=("x", "w_r"))
    return d["x"], d["w_r"]


LOGIT_CASES = [
    # T, H, E, bias
    (300, 256, 16, False),
    (1025, 200, 128, True),     # H not a multiple of the 32-wide chunk
    (5, 64, 8, True),
    (257, 4096, 8, False),
    (64, 96, 1000, True),       # E not a multiple of the 64-wide tile
    (1, 8, 1, False),
]


@pytest.mark.parametrize("T,H,E,use_bias", LOGIT_CASES)
def test_router_logits_bit_exact(m, T, H, E, use_bias):
    x, w = _inputs(T, H, E, seed=T + E)
    bias = (np.random.default_rng(5).standard_normal(E).astype(np.float32)
            if use_bias else None)
    got = m.moe_router_logits(dev_bf16(x), dev_bf16(w),
                              torch.from_numpy(bias).cuda() if use_bias
                              else None).cpu().numpy()
    want = O.router_logits(x, w, bias)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_router_logits_exact_ties_and_zero_signs(m):
    """Integer operands with many equal logits, and rows whose products are
    all signed zeros (the sum keeps the sign of its first term)."""
    rng = np.random.default_rng(7)
    T, H, E = 130, 64, 12
    x = bf16_bits(rng.integers(-2, 3, (T, H)).astype(np.float32))
    w = bf16_bits(rng.integers(-1, 2, (E, H)).astype(np.float32))
    x[0] = bf16_bits(np.full(H, -0.0, np.float32))
    x[1] = bf16_bits(np.zeros(H, np.float32))
    got = m.moe_router_logits(dev_bf16(x), dev_bf16(w)).cpu().numpy()
    want = O.router_logits(x, w)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    # and the routing on them
    idx, wt = m.moe_route_topk(torch.from_numpy(got).cuda(), 4)
    ridx, rw = O.route_topk(want, 4)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)


@pytest.mark.parametrize("name", ["mixtral", "qwen3_long"])
def test_router_logits_full_size_sampled(m, name):
    """Full workload sizes through the launch shape the layer uses; the
    oracle recomputes a sample of tokens (each token's logits depend on its
    own row only)."""
    cfg = CONFIGS[name]
    d = generate_config(cfg, seed=0, want=("x", "w_r"))
    got = m.moe_router_logits(dev_bf16(d["x"]), dev_bf16(d["w_r"]))
    rng = np.random.default_rng(9)
    toks = np.unique(np.concatenate([[0, cfg.T - 1],
                                     rng.integers(0, cfg.T, 30)]))
    want = O.router_logits(d["x"][toks], d["w_r"])
    g = got[torch.from_numpy(toks).cuda()].cpu().numpy()
    np.testing.assert_array_equal(g.view(np.uint32), want.view(np.uint32))


BWD_CASES = [
    # T, H, E, k
    (300, 256, 16, 4),
    (700, 192, 128, 8),
    (33, 64, 5, 5),        # k = E
    (1, 64, 1, 1),         # one expert: renormalised weight 1, zero grad
    (2000, 128, 8, 2),     # several token splits of dW_r
]


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("T,H,E,k", BWD_CASES)
def test_router_bwd_parity(m, T, H, E, k, renorm):
    x, w = _inputs(T, H, E, seed=3 * T + E)
    lg = O.router_logits(x, w)
    idx, _ = O.route_topk(lg, k, renorm)
    dw = np.random.default_rng(T).standard_normal((T, k)).astype(np.float32)
    r = m.moe_router_bwd(torch.from_numpy(lg).cuda(),
                         torch.from_numpy(idx).cuda(),
                         torch.from_numpy(dw).cuda(), dev_bf16(x),
                         dev_bf16(w), renormalize=renorm)
    dl_ref = O.router_bwd(lg, idx, dw, renorm)
    dl = r["dlogits"].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(dl, dl_ref, rtol=1e-5, atol=1e-12)
    if renorm:   # exactly zero off the chosen set
        mask = np.zeros((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
        assert np.all(dl[~mask] == 0.0)
    # weight gradients from the GPU's dlogits (float32 values)
    dW_ref, dx_ref = O.router_weight_grads(dl, x, w)
    dW = r["dw_r"].cpu().numpy().astype(np.float64)
    dx = r["dx"].cpu().numpy().astype(np.float64)
    if np.linalg.norm(dW_ref) == 0:
        assert np.all(dW == 0) and np.all(dx == 0)
    else:
        assert O.rel_err(dW, dW_ref) <= 1e-4
        assert O.rel_err(dx, dx_ref) <= 1e-4


def test_router_bwd_deterministic_and_optional_outputs(m):
    T, H, E, k = 1500, 256, 64, 6
    x, w = _inputs(T, H, E, seed=11)
    lg = torch.from_numpy(O.router_logits(x, w)).cuda()
    idx, _ = m.moe_route_topk(lg, k)
    dw = torch.randn((T, k), dtype=torch.float32, device="cuda")
    a = m.moe_router_bwd(lg, idx, dw, dev_bf16(x), dev_bf16(w))
    b = m.moe_router_bwd(lg, idx, dw, dev_bf16(x), dev_bf16(w))
    for key in ("dlogits", "dw_r", "dx"):
        assert torch.equal(a[key], b[key]), key
    c = m.moe_router_bwd(lg, idx, dw, dev_bf16(x), dev_bf16(w),
                         want_dw=False, want_dx=False)
    assert torch.equal(c["dlogits"], a["dlogits"])
