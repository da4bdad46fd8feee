"""GPU parity at the full workload sizes, through the same entry points and
launch shapes the benchmark times.

Routing, split sizes, offsets, maps and the permuted rows are compared in
full (bit-exact).  Layer outputs and gradients are compared on sampled
tokens: the oracle's grouped MLP is evaluated for just those routed rows,
one expert at a time (its rows are independent of the other rows).  Weight
gradients are compared in full for a few experts: two of moderate size, an
empty one and the one with the most rows.  MXFP8 at full size: the same
against the oracle running the MXFP8 rule, the whole expert weights
quantised by its C statement (oracle/mx_fast.c).
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synthetic import CONFIGS, bf16_to_f64, generate_config

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
N_SAMPLE = 12


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_grouped_router_amd as mod
    mod.load_library()
    return mod


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).cuda()


def host_f64(t):
    return bf16_to_f64(t.detach().cpu().view(torch.int16).numpy().view(
        np.uint16))


def sample_tokens(T, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1],
                                     rng.integers(0, T, N_SAMPLE - 2)]))


def row_close(got, ref, tol, what):
    for i in range(ref.shape[0]):
        n = np.linalg.norm(ref[i])
        d = np.linalg.norm(got[i] - ref[i])
        assert d <= tol * max(n, 1e-30), f"{what} row {i}: {d / n:.3e}"


def forward(m, d, cfg, precision):
    T, E, k = cfg.T, cfg.E, cfg.k
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    f = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], precision=precision,
                              save=True)
    y = m.moe_unpermute(f["z"], p["row_map"], k)
    return idx, w, p, wgu, wdn, f, y


def check_maps(d, cfg, idx, w, p):
    ridx, rw = O.route_topk(d["logits"], cfg.k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    wd = np.abs(w.cpu().numpy().view(np.int32).astype(np.int64) -
                rw.astype(np.float32).view(np.int32).astype(np.int64))
    assert wd.max() <= 1
    ref = O.permute_index(ridx, cfg.E)
    for key in ("split_sizes", "offsets", "row_map", "src_row"):
        np.testing.assert_array_equal(p[key].cpu().numpy(), ref[key], key)
    xp = p["x_perm"].cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(xp, O.permute_rows(d["x"], ref["src_row"],
                                                     cfg.k))
    return ridx, rw, ref


def oracle_rows_fwd(d, ridx, rw, toks):
    """z rows of the sampled tokens' routed pairs and y rows (float64)."""
    k = ridx.shape[1]
    y = np.zeros((len(toks), d["x"].shape[1]))
    pairs = [(i, t, j, int(ridx[t, j])) for i, t in enumerate(toks)
             for j in range(k)]
    for e in sorted({p[3] for p in pairs}):
        sel = [p for p in pairs if p[3] == e]
        xr = d["x"][[p[1] for p in sel]]
        wr = np.array([rw[p[1], p[2]] for p in sel], dtype=np.float32)
        z = O.grouped_mlp_fwd(xr, d["w_gu"][e:e + 1], d["w_dn"][e:e + 1], wr,
                              np.array([0, len(sel)]))["z"]
        for (i, t, j, _), zr in zip(sel, z):
            y[i] += zr
    return y


@pytest.mark.parametrize("name", ["mixtral", "qwen3"])
def test_forward_full_size_bf16(m, name):
    cfg = CONFIGS[name]
    d = generate_config(cfg, seed=0)
    idx, w, p, wgu, wdn, f, y = forward(m, d, cfg, m.PREC_BF16)
    ridx, rw, ref = check_maps(d, cfg, idx, w, p)
    toks = sample_tokens(cfg.T, 1)
    yref = oracle_rows_fwd(d, ridx, rw, toks)
    row_close(host_f64(y[torch.from_numpy(toks).cuda()]), yref, TOL_BF16,
              f"{name} y")


def _pairs_by_expert(ridx, rw, toks):
    """The sampled tokens' routed pairs grouped by expert:
    {e: [(i, t, j, w_tj), ...]} (i = position of t in toks)."""
    k = ridx.shape[1]
    out = {}
    for i, t in enumerate(toks):
        for j in range(k):
            out.setdefault(int(ridx[t, j]), []).append(
                (i, int(t), j, np.float32(rw[t, j])))
    return dict(sorted(out.items()))


def test_forward_full_size_mxfp8(m):
    """Mixtral-shaped MXFP8 layer at full size against the MXFP8 oracle on
    sampled tokens: per expert, the oracle quantises the whole W_gu[e] and
    W_dn[e] (the C statement of its rule) and the sampled rows (row-wise
    blocks keep rows independent).  y within 6e-2 per token and 1e-2 over
    the sample; A's codes nearly all equal to the oracle's (printed)."""
    cfg = CONFIGS["mixtral_mxfp8"]
    d = generate_config(cfg, seed=0)
    T, E, k, F = cfg.T, cfg.E, cfg.k, cfg.F
    idx, w = m.moe_route_topk(torch.from_numpy(d["logits"]).cuda(), k)
    p = m.moe_permute(dev_bf16(d["x"]), idx, E, topk_w=w,
                      precision=m.PREC_MXFP8)
    wgu, wdn = dev_bf16(d["w_gu"]), dev_bf16(d["w_dn"])
    f = m.moe_grouped_mlp_fwd(p["x_perm"], wgu, wdn, p["offsets"],
                              w_perm=p["w_perm"], precision=m.PREC_MXFP8,
                              x_perm_scale=p["x_perm_scale"],
                              save_a_codes=True)
    y = m.moe_unpermute(f["z"], p["row_map"], k)
    ridx, rw = O.route_topk(d["logits"], k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    ref = O.permute_index(ridx, E)
    for key in ("split_sizes", "offsets", "row_map", "src_row"):
        np.testing.assert_array_equal(p[key].cpu().numpy(), ref[key], key)
    # the fused MXFP8 permute: codes and scales of every routed row
    xc, xs = O.mxfp8_quantize_rows(d["x"])
    src_tok = ref["src_row"] // k
    np.testing.assert_array_equal(p["x_perm"].cpu().numpy(), xc[src_tok])
    np.testing.assert_array_equal(p["x_perm_scale"].cpu().numpy(),
                                  xs[src_tok])
    toks = sample_tokens(T, 1)
    yref = np.zeros((len(toks), cfg.H))
    rows_gpu, a_ref = [], []
    for e, sel in _pairs_by_expert(ridx, rw, toks).items():
        rows = [t for (_, t, _, _) in sel]
        wr = np.array([q[3] for q in sel], dtype=np.float32)
        o = O.grouped_mlp_fwd_mxfp8(d["x"][rows], d["w_gu"][e:e + 1],
                                    d["w_dn"][e:e + 1], wr,
                                    np.array([0, len(sel)]), keep=True)
        for (i, t, j, _), zr in zip(sel, o["z"]):
            yref[i] += zr
            rows_gpu.append(int(ref["row_map"][t * k + j]))
        a_ref.append(o["a"])
    got = host_f64(y[torch.from_numpy(toks).cuda()])
    row_close(got, yref, 6e-2, "mxfp8 y")
    assert O.rel_err(got, yref) <= 1e-2, O.rel_err(got, yref)
    want_c, want_s = O.mxfp8_quantize_rows(np.concatenate(a_ref, axis=0))
    rsel = torch.tensor(rows_gpu, device="cuda")
    fc = float((f["a_q"][rsel].cpu().numpy() == want_c).mean())
    fs = float((f["a_s"][rsel].cpu().numpy() == want_s).mean())
    print(f"full-size A codes equal to the oracle's: {fc:.6f}; "
          f"scales: {fs:.6f}")
    assert fc >= 0.99 and fs >= 0.99, (fc, fs)
    # extra: the layer output is the bf16 layer's up to E4M3 noise
    _, _, _, _, _, fb, yb = forward(m, d, cfg, m.PREC_BF16)
    err = O.rel_err(host_f64(y), host_f64(yb))
    assert 1e-3 < err < 0.12, err


@pytest.mark.parametrize("name", ["qwen3_long"])
def test_backward_full_size_bf16(m, name):
    cfg = CONFIGS[name]
    d = generate_config(cfg, seed=0)
    idx, w, p, wgu, wdn, f, y = forward(m, d, cfg, m.PREC_BF16)
    ridx, rw, ref = check_maps(d, cfg, idx, w, p)
    dz = m.moe_gather_rows(dev_bf16(d["dy"]), p["row_map"], cfg.k)
    g = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                              f["h1"], f["a"], w_perm=p["w_perm"])
    dx = m.moe_unpermute(g["dx_perm"], p["row_map"], cfg.k)
    dprobs = m.moe_unpermute_probs_grad(g["dw_perm"], p["row_map"], cfg.k)
    # sampled tokens: dx rows and dprobs
    toks = sample_tokens(cfg.T, 3)
    k = cfg.k
    dxref = np.zeros((len(toks), cfg.H))
    dpref = np.zeros((len(toks), k))
    pairs = [(i, t, j, int(ridx[t, j])) for i, t in enumerate(toks)
             for j in range(k)]
    for e in sorted({q[3] for q in pairs}):
        sel = [q for q in pairs if q[3] == e]
        rows = [q[1] for q in sel]
        wr = np.array([rw[q[1], q[2]] for q in sel], dtype=np.float32)
        gr = O.grouped_mlp_bwd(O._as_f64(d["dy"][rows]), d["x"][rows],
                               d["w_gu"][e:e + 1], d["w_dn"][e:e + 1], wr,
                               np.array([0, len(sel)]))
        for (i, t, j, _), dxr, dwr in zip(sel, gr["dx_perm"], gr["dw_perm"]):
            dxref[i] += dxr
            dpref[i, j] = dwr
    tsel = torch.from_numpy(toks).cuda()
    row_close(host_f64(dx[tsel]), dxref, TOL_BF16, "dx")
    row_close(dprobs[tsel].cpu().numpy().astype(np.float64), dpref,
              TOL_BF16, "dprobs")
    # full weight gradients of three experts of moderate size (one empty)
    split = ref["split_sizes"]
    off = ref["offsets"]
    order = np.argsort(split)
    mid = [int(e) for e in order if 200 <= split[e] <= 3000][:2]
    empty = [int(e) for e in order if split[e] == 0][:1]
    hottest = [int(order[-1])]      # the longest K loop of the wgrad GEMMs
    dzh = O._as_f64(d["dy"])
    gw_gu, gw_dn = g["dw_gu"], g["dw_dn"]
    for e in mid + empty + hottest:
        lo, hi = int(off[e]), int(off[e + 1])
        src = ref["src_row"][lo:hi]
        if hi == lo:
            assert torch.count_nonzero(gw_gu[e]).item() == 0
            assert torch.count_nonzero(gw_dn[e]).item() == 0
            continue
        tok = src // k
        wr = rw.reshape(-1)[src].astype(np.float32)
        gr = O.grouped_mlp_bwd(dzh[tok], d["x"][tok], d["w_gu"][e:e + 1],
                               d["w_dn"][e:e + 1], wr, np.array([0, hi - lo]))
        assert O.rel_err(host_f64(gw_gu[e]), gr["dw_gu"][0]) <= TOL_BF16, e
        assert O.rel_err(host_f64(gw_dn[e]), gr["dw_dn"][0]) <= TOL_BF16, e


def test_backward_full_size_mxfp8(m):
    """MXFP8 forward + backward at the Mixtral shapes against the MXFP8
    oracle backward: dx and dprobs on sampled tokens (every quantisation
    feeding a token's dx is row-wise or a whole weight, so rows are
    independent), and the full dW_gu, dW_dn of a mid-size expert (its
    token-direction blocks start at the expert's first row, as in the
    oracle called on that expert's rows).  Within 6e-2; the bf16-backward
    comparison is kept as an extra."""
    cfg = CONFIGS["mixtral_mxfp8_bwd"]
    d = generate_config(cfg, seed=0)
    T, E, k, H, F = cfg.T, cfg.E, cfg.k, cfg.H, cfg.F
    idx, w, p, wgu, wdn, f, y = forward(m, d, cfg, m.PREC_MXFP8)
    ridx, rw, ref = check_maps(d, cfg, idx, w, p)
    dz = m.moe_gather_rows(dev_bf16(d["dy"]), p["row_map"], k)
    gq = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                               f["h1"], f["a"], w_perm=p["w_perm"],
                               precision=m.PREC_MXFP8)
    dx = m.moe_unpermute(gq["dx_perm"], p["row_map"], k)
    dprobs = m.moe_unpermute_probs_grad(gq["dw_perm"], p["row_map"], k)
    toks = sample_tokens(T, 3)
    dxref = np.zeros((len(toks), H))
    dpref = np.zeros((len(toks), k))
    for e, sel in _pairs_by_expert(ridx, rw, toks).items():
        rows = [t for (_, t, _, _) in sel]
        wr = np.array([q[3] for q in sel], dtype=np.float32)
        gr = O.grouped_mlp_bwd_mxfp8(d["dy"][rows], d["x"][rows],
                                     d["w_gu"][e:e + 1], d["w_dn"][e:e + 1],
                                     wr, np.array([0, len(sel)]))
        for (i, t, j, _), dxr, dwr in zip(sel, gr["dx_perm"], gr["dw_perm"]):
            dxref[i] += dxr
            dpref[i, j] = dwr
    tsel = torch.from_numpy(toks).cuda()
    row_close(host_f64(dx[tsel]), dxref, 6e-2, "mxfp8 dx")
    row_close(dprobs[tsel].cpu().numpy().astype(np.float64), dpref, 6e-2,
              "mxfp8 dprobs")
    # whole weight gradients of the median expert
    split = ref["split_sizes"]
    off = ref["offsets"]
    e = int(np.argsort(split)[E // 2])
    lo, hi = int(off[e]), int(off[e + 1])
    src = ref["src_row"][lo:hi]
    tok = src // k
    wr = rw.reshape(-1)[src].astype(np.float32)
    gr = O.grouped_mlp_bwd_mxfp8(d["dy"][tok], d["x"][tok],
                                 d["w_gu"][e:e + 1], d["w_dn"][e:e + 1], wr,
                                 np.array([0, hi - lo]))
    for key in ("dw_gu", "dw_dn"):
        err = O.rel_err(host_f64(gq[key][e]), gr[key][0])
        print(f"expert {e} ({hi - lo} rows) {key}: {err:.3e}")
        assert err <= 6e-2, (key, err)
    # extra: within E4M3 noise of the bf16 backward
    gb = m.moe_grouped_mlp_bwd(dz, p["x_perm"], wgu, wdn, p["offsets"],
                               f["h1"], f["a"], w_perm=p["w_perm"])
    for key in ("dx_perm", "dw_gu", "dw_dn"):
        err = O.rel_err(host_f64(gq[key]), host_f64(gb[key]))
        assert 1e-3 < err < 0.12, (key, err)
