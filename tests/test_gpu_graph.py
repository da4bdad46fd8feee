"""The layer's library calls enqueue only kernels on the caller's stream (no
allocation, no host synchronisation, no memset inside a call), so a whole
step -- router top-k, permute, grouped MLP forward, combine, and the
backward (gather dY, grouped MLP backward, combine dX, routing-weight
gradients) -- can be captured in a HIP graph and replayed.  Every replay is
compared bit for bit with the eager result (every kernel of the path is
deterministic), with eager library work and synchronisations between the
replays.
"""
import numpy as np
import pytest
import torch

from synthetic import generate

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


def _step(m, inp, E, k, precision, backward):
    idx, w = m.moe_route_topk(inp["logits"], k)
    p = m.moe_permute(inp["x"], idx, E, topk_w=w)
    r = m.moe_grouped_mlp_fwd(p["x_perm"], inp["w_gu"], inp["w_dn"],
                              p["offsets"], w_perm=p["w_perm"],
                              precision=precision, save=backward)
    out = {"idx": idx, "w": w, "x_perm": p["x_perm"], "z": r["z"],
           "y": m.moe_unpermute(r["z"], p["row_map"], k)}
    if backward:
        dz = m.moe_gather_rows(inp["dy"], p["row_map"], k)
        g = m.moe_grouped_mlp_bwd(dz, p["x_perm"], inp["w_gu"], inp["w_dn"],
                                  p["offsets"], r["h1"], r["a"],
                                  w_perm=p["w_perm"], precision=precision)
        out.update(dw_gu=g["dw_gu"], dw_dn=g["dw_dn"],
                   dx=m.moe_unpermute(g["dx_perm"], p["row_map"], k),
                   dprobs=m.moe_unpermute_probs_grad(g["dw_perm"],
                                                     p["row_map"], k))
    return out


@pytest.mark.parametrize("prec_name,backward,F", [
    ("PREC_BF16", True, 384), ("PREC_MXFP8", True, 384),
    ("PREC_FP8_TENSOR", False, 384),
    # long K for the down GEMM: its last tiles are split along K (arrival
    # counters cleared inside every call, so every replay starts clean)
    ("PREC_BF16", False, 8192), ("PREC_MXFP8", False, 8192)])
def test_layer_step_graph_replay(m, prec_name, backward, F):
    T, H, E, k = 700, 256, 8, 2     # ragged experts; F = 384: F tail tile
    d = generate(T, H, F, E, k, zipf=1.2, seed=21,
                 want=("x", "logits", "w_gu", "w_dn", "dy"))
    inp = {"x": dev_bf16(d["x"]), "logits": torch.from_numpy(d["logits"]).cuda(),
           "w_gu": dev_bf16(d["w_gu"]), "w_dn": dev_bf16(d["w_dn"]),
           "dy": dev_bf16(d["dy"])}
    prec = getattr(m, prec_name)
    eager = _step(m, inp, E, k, prec, backward)
    torch.cuda.synchronize()
    ref = {key: v.clone() for key, v in eager.items()}

    # warm-up on a side stream, then capture (allocations come from the
    # graph's private pool)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(m, inp, E, k, prec, backward)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = _step(m, inp, E, k, prec, backward)
    torch.cuda.synchronize()

    for rep in range(3):
        for v in out.values():     # stale results must not survive a replay
            v.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, v in ref.items():
            assert torch.equal(out[key].view(torch.uint8),
                               v.view(torch.uint8)), (rep, key)
        # eager library work between the replays
        _step(m, inp, E, k, prec, backward)
        torch.cuda.synchronize()
