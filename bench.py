#!/usr/bin/env python3
"""Throughput of the MoE expert-MLP hot path on one MI355X.

One step = the whole path over one batch of synthetic tokens, every stage in
libmoe's HIP kernels through the C ABI:
  router top-k -> permute (+split_sizes) -> grouped gate/up GEMM with
  ScaledSwiGLU x routing weight -> grouped down GEMM -> unpermute/combine
(+ for workloads with a backward pass: gather dY -> grouped MLP backward ->
combine dX -> routing-weight grads; MXFP8 workloads quantise on the fly).

Inputs are seeded synthetic tensors already resident in HBM; all buffers are
allocated before the timed region.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload mixtral]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE grouped-MLP TFLOP/s + tokens/s (Mixtral layer, 1 GPU); "
          "% MFMA peak")
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_FP64_TFLOPS = 78.6       # MI355X fp64 (vector and matrix)
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense (MX)fp8 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral",
                    help="mixtral | qwen3 | mixtral_mxfp8 | "
                         "mixtral_mxfp8_bwd | qwen3_long | tiny")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the passes after the timed region (flushed "
                         "HBM timing, per-expert loop, router, pre-quantised "
                         "weights): profiler counter runs see the timed "
                         "step's launches only")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads after the headline "
                         "one (the 'configs' entry of the line)")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle's timed sample (0 = auto)")
    ap.add_argument("--write-traffic", nargs=4, metavar="DB",
                    help="FETCH_SIZE db, WRITE_SIZE db, copy FETCH_SIZE db, "
                         "copy WRITE_SIZE db (rocprofv3 --pmc outputs of "
                         "this workload and of --copy-calibration): record "
                         "the dominant GEMMs' HBM traffic per launch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (the "
                         "reference kernel that scales HBM byte counters)")
    return ap.parse_args()


# library kernel name -> template instantiations in profiler kernel names
# (the forward GEMMs run the eight-wave kernels: bf16 grouped_gemm_w8_kernel
# <EPI> for the down GEMM and for gate/up up to H = 4096,
# 8-bit grouped_gemm_w8q_kernel<P, EPI, G>)
KERNEL_SYMBOL = {
    "gemm_gate_up_swiglu_bf16": ("grouped_gemm_kernel<0, 0, 0, 0, 1>",
                                 "grouped_gemm_w8_kernel<1>"),
    "gemm_down_bf16": ("grouped_gemm_w8_kernel<0>",),
    "gemm_gate_up_swiglu_mxfp8": ("grouped_gemm_w8q_kernel<1, 3, 0>",),
    "gemm_down_mxfp8": ("grouped_gemm_w8q_kernel<1, 0, 0>",),
    "gemm_gate_up_swiglu_fp8t": ("grouped_gemm_w8q_kernel<2, 1, 0>",),
    "gemm_down_fp8t": ("grouped_gemm_w8q_kernel<2, 0, 0>",),
}


def _pmc_means(db, counter):
    """kernel name -> mean counter value (KiB) per dispatch."""
    import sqlite3
    con = sqlite3.connect(db)
    acc = {}
    for name, v in con.execute(
            "select kernel_name, value from counters_collection where "
            "counter_name = ?", (counter,)):
        acc.setdefault(name, []).append(float(v))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(workload, dbs, cmd):
    fetch_db, write_db, cfetch_db, cwrite_db = dbs
    fetch = _pmc_means(fetch_db, "FETCH_SIZE")
    write = _pmc_means(write_db, "WRITE_SIZE")
    cf = [v for k, v in _pmc_means(cfetch_db, "FETCH_SIZE").items()
          if "copyBuffer" in k]
    cw = [v for k, v in _pmc_means(cwrite_db, "WRITE_SIZE").items()
          if "copyBuffer" in k]
    if not cf or not cw:
        raise SystemExit("no copy kernel in the calibration runs")
    f_fac = (1 << 30) / (cf[0] * 1024.0)
    w_fac = (1 << 30) / (cw[0] * 1024.0)
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {"records": []}
    recs = [r for r in data.get("records", [])
            if r.get("workload") != workload]
    for kname, syms in KERNEL_SYMBOL.items():
        fk = [v for k, v in fetch.items() if any(s in k for s in syms)]
        wk = [v for k, v in write.items() if any(s in k for s in syms)]
        if not fk or not wk:
            continue
        recs.append({
            "kernel": kname, "workload": workload,
            "source_digest": sources_digest(kname),
            "fetch_kib_per_launch": round(fk[0], 1),
            "write_kib_per_launch": round(wk[0], 1),
            "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
            "bytes_per_launch": round(fk[0] * 1024 * f_fac +
                                      wk[0] * 1024 * w_fac),
            "command": cmd})
    data["records"] = recs
    data["about"] = ("HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE "
                     "and WRITE_SIZE (separate runs), scaled by the readings "
                     "of a plain 1 GiB copy (bench.py --copy-calibration); "
                     "source_digest identifies the kernel sources measured")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1)
    print(json.dumps(recs[-4:], indent=1))


def copy_calibration():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per
    launch, three launches.  Profiling counters of this run give the
    factor between the FETCH_SIZE / WRITE_SIZE readings and real bytes."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), \
        torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(3):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / 3
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n,
                      "launches": 3, "ms_per_copy": round(ms, 4),
                      "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


class Layer:
    """All device buffers of one layer step, allocated once."""

    def __init__(self, m, cfg, d, dev):
        import torch
        self.m, self.cfg, self.dev = m, cfg, dev
        lib = m.load_library()
        self.lib = lib
        T, H, F, E, k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
        rows = T * k
        self.rows = rows

        def bf(bits):
            return torch.from_numpy(bits.view(np.int16)).view(
                torch.bfloat16).to(dev)

        self.x = bf(d["x"])
        self.logits = torch.from_numpy(d["logits"]).to(dev)
        self.w_gu = bf(d["w_gu"])
        self.w_dn = bf(d["w_dn"])
        self.dy = bf(d["dy"]) if "dy" in d and d["dy"] is not None else None
        i32, f32, b16, u8 = torch.int32, torch.float32, torch.bfloat16, \
            torch.uint8
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.idx = e((T, k), i32)
        self.w = e((T, k), f32)
        self.mx = cfg.mode == "mxfp8"
        self.f8t = cfg.mode == "fp8t"
        # MXFP8 forward only: the permute writes E4M3 codes + E8M0 scales of
        # x (fused quantisation).  With a backward pass the bf16 x_perm is
        # kept for the weight gradient (quantised along tokens there) and
        # the forward call quantises it row-wise.  The weights are quantised
        # from the bf16 masters inside every grouped-MLP call.
        self.mx_codes = self.mx and not cfg.backward
        self.x_perm = e((rows, H), u8 if self.mx_codes else b16)
        self.x_perm_scale = e((rows, H // 32), u8) if self.mx_codes else None
        self.w_perm = e(rows, f32)
        self.row_map = e(rows, i32)
        self.src_row = e(rows, i32)
        self.split = e(E, i32)
        self.offsets = e(E + 1, i32)
        n = ctypes.c_size_t()
        m._check(lib.moe_permute_workspace_size(T, E, k, ctypes.byref(n)))
        self.pws = e(max(n.value, 256), u8)
        self.z = e((rows, H), b16)
        self.y = e((T, H), b16)
        self.bwd = cfg.backward
        save = self.bwd
        self.h1 = e((rows, 2 * F), b16) if save else None
        self.a = e((rows, F), b16) if save else None
        fa = m._FwdArgs()
        fa.E, fa.H, fa.F, fa.rows = E, H, F, rows
        fa.precision = m.PREC_MXFP8 if self.mx else (
            m.PREC_FP8_TENSOR if self.f8t else m.PREC_BF16)
        fa.x_perm = self.x_perm.data_ptr()
        fa.x_perm_scale = self.x_perm_scale.data_ptr() if self.mx_codes \
            else None
        fa.w_gu, fa.w_dn = self.w_gu.data_ptr(), self.w_dn.data_ptr()
        fa.w_perm = self.w_perm.data_ptr()
        fa.offsets = self.offsets.data_ptr()
        fa.z_perm = self.z.data_ptr()
        fa.h1_save = self.h1.data_ptr() if save else None
        fa.a_save = self.a.data_ptr() if save else None
        m._check(lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(fa),
                                                        ctypes.byref(n)))
        self.fws = e(max(n.value, 256), u8)
        fa.ws, fa.ws_bytes = self.fws.data_ptr(), self.fws.numel()
        self.fa = fa
        if self.bwd:
            self.dz = e((rows, H), b16)
            self.dx_perm = e((rows, H), b16)
            self.dw_gu = e((E, 2 * F, H), b16)
            self.dw_dn = e((E, H, F), b16)
            self.dw_perm = e(rows, f32)
            self.dx = e((T, H), b16)
            self.dprobs = e((T, k), f32)
            ba = m._BwdArgs()
            ba.E, ba.H, ba.F, ba.rows = E, H, F, rows
            ba.precision = fa.precision
            ba.x_perm, ba.w_gu, ba.w_dn = fa.x_perm, fa.w_gu, fa.w_dn
            ba.w_perm, ba.offsets = fa.w_perm, fa.offsets
            ba.h1_save, ba.a_save = fa.h1_save, fa.a_save
            ba.dz_perm, ba.dx_perm = self.dz.data_ptr(), \
                self.dx_perm.data_ptr()
            ba.dw_gu, ba.dw_dn = self.dw_gu.data_ptr(), self.dw_dn.data_ptr()
            ba.dw_perm = self.dw_perm.data_ptr()
            m._check(lib.moe_grouped_mlp_bwd_workspace_size(ctypes.byref(ba),
                                                            ctypes.byref(n)))
            self.bws = e(max(n.value, 256), u8)
            ba.ws, ba.ws_bytes = self.bws.data_ptr(), self.bws.numel()
            self.ba = ba
        self.ctx = m._context(torch.device(dev))

    # the stages of one step, in order
    def stages(self):
        c, L, m = self.cfg, self.lib, self.m
        T, H, E, k = c.T, c.H, c.E, c.k
        P = lambda t: t.data_ptr()

        def route(st):
            m._check(L.moe_route_topk(self.ctx, P(self.logits), T, E, k, 1,
                                      P(self.idx), P(self.w), st))

        def permute(st):
            m._check(L.moe_permute(
                self.ctx, P(self.x), P(self.idx), P(self.w), T, H, E, k,
                m.PREC_MXFP8 if self.mx_codes else m.PREC_BF16, P(self.x_perm),
                P(self.x_perm_scale) if self.mx_codes else None,
                P(self.w_perm),
                P(self.row_map), P(self.src_row), P(self.split),
                P(self.offsets), P(self.pws), self.pws.numel(), st))

        def mlp(st):
            m._check(L.moe_grouped_mlp_fwd(self.ctx, ctypes.byref(self.fa),
                                           st))

        def unpermute(st):
            m._check(L.moe_unpermute(self.ctx, P(self.z), P(self.row_map),
                                     None, T, H, k, P(self.y), st))

        out = [("route_topk", route), ("permute", permute),
               ("grouped_mlp_fwd", mlp), ("unpermute", unpermute)]
        if self.bwd:
            def gather(st):
                m._check(L.moe_gather_rows(self.ctx, P(self.dy),
                                           P(self.row_map), T, H, k,
                                           P(self.dz), st))

            def mlp_bwd(st):
                m._check(L.moe_grouped_mlp_bwd(self.ctx, ctypes.byref(self.ba),
                                               st))

            def combine_dx(st):
                m._check(L.moe_unpermute(self.ctx, P(self.dx_perm),
                                         P(self.row_map), None, T, H, k,
                                         P(self.dx), st))

            def probs(st):
                m._check(L.moe_unpermute_probs_grad(
                    self.ctx, P(self.dw_perm), P(self.row_map), T, k,
                    P(self.dprobs), st))

            out += [("gather_dy", gather), ("grouped_mlp_bwd", mlp_bwd),
                    ("unpermute_dx", combine_dx), ("probs_grad", probs)]
        return out


# library kernels timed in the timed region (names as launched)
KERNELS = [
    "route_topk", "permute_index", "permute_gather", "permute_gather_mxfp8",
    "gemm_gate_up_swiglu_bf16", "gemm_down_bf16", "gemm_gate_up_swiglu_mxfp8",
    "gemm_down_mxfp8", "mxfp8_quantize_rows", "mxfp8_quantize_cols",
    "mxfp8_quantize_segments", "mxfp8_quantize_segments_and_rows",
    "mxfp8_scales_retile", "unpermute",
    "gemm_dgrad_down_swiglu_bwd", "gemm_dgrad_gate_up", "gemm_wgrad_down",
    "gemm_wgrad_gate_up", "gemm_dgrad_down_swiglu_bwd_mxfp8",
    "gemm_dgrad_gate_up_mxfp8", "gemm_wgrad_down_mxfp8",
    "gemm_wgrad_gate_up_mxfp8", "gemm_gate_up_swiglu_fp8t", "gemm_down_fp8t",
    "fp8_amax", "fp8_tensor_quantize", "fp8_amax_clear",
    "routing_weight_grad_reduce", "probs_grad",
    "tile_table", "padded_offsets", "expert_order",
]
# algorithmic flop per step (each GEMM runs once per step)
_F4 = lambda c: 4.0 * c.rows * c.H * c.F
_F2 = lambda c: 2.0 * c.rows * c.H * c.F
KERNEL_FLOP = {
    "gemm_gate_up_swiglu_bf16": _F4, "gemm_gate_up_swiglu_mxfp8": _F4,
    "gemm_down_bf16": _F2, "gemm_down_mxfp8": _F2,
    "gemm_dgrad_down_swiglu_bwd": _F2, "gemm_dgrad_gate_up": _F4,
    "gemm_wgrad_down": _F2, "gemm_wgrad_gate_up": _F4,
    "gemm_dgrad_down_swiglu_bwd_mxfp8": _F2, "gemm_dgrad_gate_up_mxfp8": _F4,
    "gemm_wgrad_down_mxfp8": _F2, "gemm_wgrad_gate_up_mxfp8": _F4,
    "gemm_gate_up_swiglu_fp8t": _F4, "gemm_down_fp8t": _F2,
}
MX_BYTES = 2.0 + 1.0 + 1.0 / 32   # bf16 read, E4M3 code + E8M0/32 written


def _mx_rows_elems(c):
    """Values quantised row-wise alone per step: both weight tensors in the
    forward; with a backward pass also x_perm (forward).  dZ and dH1 are
    quantised row-wise by the pass that also quantises them along tokens."""
    n = c.E * 3.0 * c.H * c.F
    if c.backward:
        n += c.rows * c.H
    return n


# algorithmic HBM bytes per step (reads + writes)
KERNEL_BYTES = {
    # read x once, write k rows, + topk_w/row_map reads and w_perm writes;
    # with a backward pass dY is gathered the same way
    "permute_gather": lambda c: (2 if c.backward else 1) * (
        (1 + c.k) * c.T * c.H * 2.0 + c.rows * 12.0),
    "permute_gather_mxfp8": lambda c: c.T * c.H * (2.0 + c.k * 1.03125)
    + c.rows * 12.0,
    # read k rows, write one, + row_map (forward y, backward dx)
    "unpermute": lambda c: (2 if c.backward else 1) * (
        (c.k + 1) * c.T * c.H * 2.0 + c.rows * 4.0),
    "mxfp8_quantize_rows": lambda c: _mx_rows_elems(c) * MX_BYTES,
    # backward: both weight tensors along their other dimension
    "mxfp8_quantize_cols": lambda c: c.E * 3.0 * c.H * c.F * MX_BYTES,
    # backward: A and X along tokens (padding not counted)
    "mxfp8_quantize_segments": lambda c: c.rows * (c.H + c.F) * MX_BYTES,
    # backward: dZ and dH1 along tokens and row-wise in one pass (one bf16
    # read, two sets of codes and scales written)
    "mxfp8_quantize_segments_and_rows": lambda c: c.rows * (c.H + 2.0 * c.F)
    * (2.0 + 2.0 * (1.0 + 1.0 / 32)),
    # tensor-scaled FP8: an amax read and a quantising pass (read bf16,
    # write codes) over both weight tensors, x_perm and A
    "fp8_amax": lambda c: 2.0 * (3.0 * c.E * c.H * c.F + c.rows * (c.H + c.F)),
    "fp8_tensor_quantize": lambda c: 3.0 * (3.0 * c.E * c.H * c.F
                                            + c.rows * (c.H + c.F)),
}

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_gemm.json")
# the sources each precision's GEMM kernels are built from: a traffic record
# holds for the kernel only while their digest matches
_GEMM_DIR = os.path.join(ROOT, "mixture_experts_grouped_router_amd", "csrc")
_GEMM_HDRS = ("grouped_gemm.hpp", "grouped_gemm_w8.hpp",
              "grouped_gemm_w8q.hpp", "work_items.hpp", "common.hpp",
              "mx_codec.hpp")
GEMM_SOURCES = {"bf16": _GEMM_HDRS + ("gemm_bf16.hip",),
                "mxfp8": _GEMM_HDRS + ("gemm_mxfp8.hip",),
                "fp8t": _GEMM_HDRS + ("gemm_fp8t.hip",)}


def sources_digest(kernel):
    """Digest of the sources of `kernel` (named ..._bf16, _mxfp8, _fp8t)."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES[kernel.rsplit("_", 1)[-1]]:
        with open(os.path.join(_GEMM_DIR, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, cfg):
    """HBM bytes per launch of `kernel` on this workload from the committed
    rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, scaled by the copy
    calibration), or None when no record matches the current kernel
    sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            recs = json.load(fh)
    except (OSError, ValueError):
        return None
    dig = sources_digest(kernel)
    for r in recs.get("records", []):
        if r.get("kernel") == kernel and r.get("workload") == cfg.name and \
                r.get("source_digest") == dig:
            return r.get("bytes_per_launch")
    return None


def algorithmic(cfg):
    """Algorithmic work per op (flop or bytes, per launch of that op)."""
    T, H, F, k = cfg.T, cfg.H, cfg.F, cfg.k
    rows = T * k
    w = {
        "grouped_mlp_fwd": ("flop", 6.0 * rows * H * F),
        "grouped_mlp_bwd": ("flop", 12.0 * rows * H * F),
        # permute: read x once, write k rows (+ 4-byte index/weight traffic)
        "permute": ("bytes", (1 + k) * T * H * 2.0 + rows * 16.0),
        "unpermute": ("bytes", (k + 1) * T * H * 2.0 + rows * 4.0),
        "gather_dy": ("bytes", (1 + k) * T * H * 2.0 + rows * 4.0),
        "unpermute_dx": ("bytes", (k + 1) * T * H * 2.0 + rows * 4.0),
    }
    return w


def cpu_baseline(cfg, d, n_tokens):
    """The oracle as it stands, timed on the host on a bounded sample of the
    same workload.  bf16: the first n_tokens, whole layer (route, permute,
    per-expert MLP in float64, combine).  MXFP8 (whose oracle quantises every
    block in numpy): the first n_tokens are routed and permuted, then the
    MLP of expert 0 alone on its rows, restricted to FFN columns [0, Fs)
    (gate and up rows and down columns of those f; the MLP is a sum of such
    column slices, and 32-aligned slices keep every quantisation block
    whole)."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] +
                      [1])
    except Exception:
        threads = os.cpu_count() or 1
    x = d["x"][:n_tokens]
    lg = d["logits"][:n_tokens]
    passes = "fwd+bwd" if cfg.backward else "fwd"
    per_flop = 6.0 + (12.0 if cfg.backward else 0.0)
    t0 = time.perf_counter()
    if cfg.mode == "bf16":
        if cfg.backward:
            O.layer_bwd(x, lg, d["w_gu"], d["w_dn"], d["dy"][:n_tokens],
                        cfg.k)
        else:
            O.layer_fwd(x, lg, d["w_gu"], d["w_dn"], cfg.k)
        flop = per_flop * n_tokens * cfg.k * cfg.H * cfg.F
        what = (f"first {n_tokens} of {cfg.T} tokens of the {cfg.name} "
                f"workload, whole layer {passes} in float64 numpy")
    elif cfg.mode == "fp8t":
        F, Fs = cfg.F, min(cfg.F, 7168)
        idx, w = O.route_topk(lg, cfg.k)
        mp = O.permute_index(idx, d["w_gu"].shape[0])
        lo, hi = int(mp["offsets"][0]), int(mp["offsets"][1])
        sr = mp["src_row"][lo:hi]
        xp = O.permute_rows(x, sr, cfg.k)
        wp = O.permute_weights(w, sr)
        off = np.array([0, hi - lo], dtype=np.int32)
        wgu = np.concatenate([d["w_gu"][0, :Fs], d["w_gu"][0, F:F + Fs]])[None]
        wdn = np.ascontiguousarray(d["w_dn"][0][:, :Fs])[None]
        O.grouped_mlp_fwd_fp8_tensor(xp, wgu, wdn, wp, off)
        flop = per_flop * (hi - lo) * cfg.H * Fs
        what = (f"tensor-scaled FP8 MLP fwd (quantisation included; each "
                f"sampled operand scaled as its own tensor) of expert 0 on "
                f"its {hi - lo} rows among the first {n_tokens} of {cfg.T} "
                f"tokens of the {cfg.name} workload, FFN columns [0, {Fs}) "
                f"of {F}, float64 numpy")
    else:
        F, Fs = cfg.F, min(cfg.F, 3584 if cfg.backward else 7168)
        idx, w = O.route_topk(lg, cfg.k)
        mp = O.permute_index(idx, d["w_gu"].shape[0])
        lo, hi = int(mp["offsets"][0]), int(mp["offsets"][1])
        sr = mp["src_row"][lo:hi]
        xp = O.permute_rows(x, sr, cfg.k)
        wp = O.permute_weights(w, sr)
        off = np.array([0, hi - lo], dtype=np.int32)
        wgu = np.concatenate([d["w_gu"][0, :Fs], d["w_gu"][0, F:F + Fs]])[None]
        wdn = np.ascontiguousarray(d["w_dn"][0][:, :Fs])[None]
        O.grouped_mlp_fwd_mxfp8(xp, wgu, wdn, wp, off)
        if cfg.backward:
            dz = O.gather_rows(d["dy"][:n_tokens], sr, cfg.k)
            O.grouped_mlp_bwd_mxfp8(dz, xp, wgu, wdn, wp, off)
        flop = per_flop * (hi - lo) * cfg.H * Fs
        what = (f"MXFP8 MLP {passes} (quantisation included) of expert 0 "
                f"on its {hi - lo} rows among the first {n_tokens} of "
                f"{cfg.T} tokens of the {cfg.name} workload, FFN columns "
                f"[0, {Fs}) of {F}, float64 numpy")
    dt = time.perf_counter() - t0
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "sample": f"{what} ({dt:.1f} s wall)",
            "seconds": dt}


def hbm_extras(m, layer, cfg, st):
    """HBM-bound kernels timed alone after writing a 1 GiB buffer (which
    evicts L2 and the 256 MB Infinity Cache), next to the library's stream
    kernel with the permute's traffic shape as the achievable reference."""
    import torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    stages = dict(layer.stages())
    res = {}
    work = {
        "permute_gather": KERNEL_BYTES["permute_gather"],
        "permute_gather_mxfp8": KERNEL_BYTES["permute_gather_mxfp8"],
        "unpermute": KERNEL_BYTES["unpermute"],
    }
    fwd_only = lambda c: dataclasses_replace(c)
    for stage, kname in (("permute", "permute_gather_mxfp8"
                          if layer.mx_codes else "permute_gather"),
                         ("unpermute", "unpermute")):
        times = []
        for _ in range(5):
            flush.fill_(1.0)
            m.reset_kernel_timing()
            m.set_kernel_timing(True)
            stages[stage](st)
            m.set_kernel_timing(False)
            torch.cuda.synchronize()
            n, tot = m.kernel_time(kname)
            times.append(tot / max(n, 1))
        ms = float(np.median(times))
        b = work[kname](fwd_only(cfg))
        res[kname] = {"ms": round(ms, 4), "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                      "frac_hbm": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    m.reset_kernel_timing()
    # the achievable reference: the library's stream kernel reading the
    # gather's bytes once and writing k copies (its traffic shape, no
    # indexing), caches flushed the same way
    nbytes = cfg.T * cfg.H * 2
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty(cfg.k * nbytes, dtype=torch.uint8, device="cuda")
    ctx = m._context(torch.device("cuda"))
    cts = []
    for _ in range(5):
        flush.fill_(1.0)
        m.reset_kernel_timing()
        m.set_kernel_timing(True)
        m._check(layer.lib.moe_hbm_stream_reference(
            ctx, src.data_ptr(), nbytes, cfg.k, dst.data_ptr(), st))
        m.set_kernel_timing(False)
        torch.cuda.synchronize()
        n, tot = m.kernel_time("hbm_stream_reference")
        cts.append(tot / max(n, 1))
    m.reset_kernel_timing()
    cms = float(np.median(cts))
    cb = (1 + cfg.k) * nbytes
    ref = round(cb / (cms * 1e-3) / 1e9, 1)
    for v in res.values():
        v["frac_of_stream"] = round(v["GB/s"] / ref, 4)
    del src, dst
    # the device's ceiling for each traffic mix: 256 MiB buffers (larger
    # than the Infinity Cache), read r and write w of them, caches flushed
    mb = 1 << 28
    msrc = torch.empty(2 * mb, dtype=torch.uint8, device="cuda")
    msrc.fill_(3)
    mdst = torch.empty(2 * mb, dtype=torch.uint8, device="cuda")
    mix = {}
    for name, r, w in (("read", 1, 0), ("write", 0, 1), ("copy", 1, 1),
                       ("1 read 2 writes (gather, k = 2)", 1, 2),
                       ("2 reads 1 write (combine, k = 2)", 2, 1)):
        ts = []
        for _ in range(5):
            flush.fill_(1.0)
            m.reset_kernel_timing()
            m.set_kernel_timing(True)
            m._check(layer.lib.moe_hbm_stream_mix(
                ctx, msrc.data_ptr(), mb, r, w, mdst.data_ptr(), st))
            m.set_kernel_timing(False)
            torch.cuda.synchronize()
            n, tot = m.kernel_time("hbm_stream_mix")
            ts.append(tot / max(n, 1))
        gbs = (r + w) * mb / (float(np.median(ts)) * 1e-3) / 1e9
        mix[name] = {"GB/s": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    m.reset_kernel_timing()
    del flush, msrc, mdst
    if cfg.k == 2:
        # the MXFP8 gather writes about as many bytes as it reads
        ceil = {"permute_gather": "1 read 2 writes (gather, k = 2)",
                "permute_gather_mxfp8": "copy",
                "unpermute": "2 reads 1 write (combine, k = 2)"}
        for kname, v in res.items():
            v["frac_of_mix_ceiling"] = round(
                v["GB/s"] / mix[ceil[kname]]["GB/s"], 4)
    return {"kernels": res,
            "stream_reference": {
                "GB/s": ref, "frac_hbm": round(ref / PEAK_HBM_GBS, 4),
                "bytes": cb, "what": f"moe_hbm_stream_reference: read "
                f"{nbytes} bytes once, write {cfg.k} copies, caches flushed"},
            "mix_ceilings": dict(
                mix, what="moe_hbm_stream_mix: 256 MiB buffers, read r and "
                "write w of them with 16-byte nontemporal vectors, caches "
                "flushed (GB/s of bytes read + written)")}


def dataclasses_replace(c):
    """The config with the backward pass off (per-call forward bytes)."""
    import dataclasses
    return dataclasses.replace(c, backward=False)


def prequantised_step(m, layer, cfg, st, K):
    """8-bit step with the weights quantised once beforehand (as a trainer
    does once per weight update and reuses for every micro-batch) instead
    of inside every call: MXFP8 row-wise codes for the forward call and
    column-wise codes for the backward; tensor-scaled FP8 codes with one
    scale per expert."""
    import torch
    E, H, F = cfg.E, cfg.H, cfg.F
    fa = layer.fa
    saved = (fa.w_gu_q, fa.w_gu_s, fa.w_dn_q, fa.w_dn_s, fa.w_gu_ts,
             fa.w_dn_ts, fa.ws, fa.ws_bytes)
    if cfg.mode == "fp8t":
        gq = m.fp8_tensor_quantize(layer.w_gu, E)
        dq = m.fp8_tensor_quantize(layer.w_dn, E)
        fa.w_gu_q, fa.w_gu_ts = gq[0].data_ptr(), gq[1].data_ptr()
        fa.w_dn_q, fa.w_dn_ts = dq[0].data_ptr(), dq[1].data_ptr()
    else:
        gq = m.mxfp8_quantize(layer.w_gu.reshape(E * 2 * F, H), m.ROWWISE)
        dq = m.mxfp8_quantize(layer.w_dn.reshape(E * H, F), m.ROWWISE)
        fa.w_gu_q, fa.w_gu_s = gq[0].data_ptr(), gq[1].data_ptr()
        fa.w_dn_q, fa.w_dn_s = dq[0].data_ptr(), dq[1].data_ptr()
    n = ctypes.c_size_t()
    m._check(layer.lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(fa),
                                                          ctypes.byref(n)))
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device="cuda")
    fa.ws, fa.ws_bytes = ws.data_ptr(), ws.numel()
    if layer.bwd:
        ba = layer.ba
        bsaved = (ba.w_gu_qt, ba.w_gu_st, ba.w_dn_qt, ba.w_dn_st, ba.ws,
                  ba.ws_bytes)
        gqt = m.mxfp8_quantize(layer.w_gu, m.COLWISE)
        dqt = m.mxfp8_quantize(layer.w_dn, m.COLWISE)
        ba.w_gu_qt, ba.w_gu_st = gqt[0].data_ptr(), gqt[1].data_ptr()
        ba.w_dn_qt, ba.w_dn_st = dqt[0].data_ptr(), dqt[1].data_ptr()
        m._check(layer.lib.moe_grouped_mlp_bwd_workspace_size(
            ctypes.byref(ba), ctypes.byref(n)))
        bws = torch.empty(max(n.value, 256), dtype=torch.uint8,
                          device="cuda")
        ba.ws, ba.ws_bytes = bws.data_ptr(), bws.numel()
    stages = layer.stages()
    for _ in range(2):
        for _, fn in stages:
            fn(st)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        for _, fn in stages:
            fn(st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    (fa.w_gu_q, fa.w_gu_s, fa.w_dn_q, fa.w_dn_s, fa.w_gu_ts, fa.w_dn_ts,
     fa.ws, fa.ws_bytes) = saved
    if layer.bwd:
        (ba.w_gu_qt, ba.w_gu_st, ba.w_dn_qt, ba.w_dn_st, ba.ws,
         ba.ws_bytes) = bsaved
    flop = cfg.fwd_flop() + (cfg.bwd_flop() if cfg.backward else 0.0)
    return {"ms_per_step": round(ms, 4),
            "value": round(flop / (ms * 1e-3) / 1e12, 2),
            "what": "weights quantised once outside the timed step (" +
                    ("one scale per expert" if cfg.mode == "fp8t" else
                     "row-wise for the forward" +
                     (", column-wise for the backward" if layer.bwd
                      else "")) + ")"}


def expert_loop_extra(m, layer, cfg, st, K):
    """The grouped MLP against the per-expert loop baseline on the same
    permuted inputs: wall time per call, stream synchronised around each
    run (the loop waits for the stream itself to read the row counts)."""
    import torch
    fa = layer.fa
    la = m._FwdArgs()
    for f, _ in m._FwdArgs._fields_:
        setattr(la, f, getattr(fa, f))
    la.h1_save, la.a_save = None, None
    n = ctypes.c_size_t()
    m._check(layer.lib.moe_expert_loop_mlp_fwd_workspace_size(
        ctypes.byref(la), ctypes.byref(n)))
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device="cuda")
    la.ws, la.ws_bytes = ws.data_ptr(), ws.numel()
    z_loop = torch.empty_like(layer.z)
    la.z_perm = z_loop.data_ptr()
    for _, fn in layer.stages():     # valid x_perm / offsets / w_perm
        fn(st)

    def loop():
        m._check(layer.lib.moe_expert_loop_mlp_fwd(layer.ctx, ctypes.byref(la),
                                                   st))

    def grouped():
        m._check(layer.lib.moe_grouped_mlp_fwd(layer.ctx, ctypes.byref(fa),
                                               st))

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / K * 1e3

    t_loop, t_grp = timed(loop), timed(grouped)
    diff = (z_loop.float() - layer.z.float()).norm() / layer.z.float().norm()
    return {"loop_ms": round(t_loop, 4), "grouped_ms": round(t_grp, 4),
            "speedup_grouped_vs_loop": round(t_loop / t_grp, 3),
            "rel_diff_z": float(f"{diff.item():.3e}"),
            "what": "moe_expert_loop_mlp_fwd (per expert: gate/up GEMM, "
                    "SwiGLU kernel, down GEMM; host reads the row counts) "
                    "vs moe_grouped_mlp_fwd, wall ms per call"}


def ep_share_extra(m, layer, cfg, st, K, G=8):
    """One GPU's share of an expert-parallel layer over G GPUs: experts
    [g E/G, (g+1) E/G) live on GPU g and every GPU routes T tokens like this
    workload, so GPU g receives G times the rows its experts get here (the
    other GPUs' tokens are drawn alike; their rows are stood in for by G
    copies of the local ones).  The grouped MLP forward on the heaviest
    GPU's share (it bounds the step), timed with HIP events; the all-to-all
    exchanges around it are not run (one GPU)."""
    import torch
    E, H, F = cfg.E, cfg.H, cfg.F
    if E % G:
        return None
    for _, fn in layer.stages():     # valid x_perm / offsets / w_perm
        fn(st)
    torch.cuda.synchronize()
    off = layer.offsets.cpu().numpy().astype(np.int64)
    el = E // G
    loads = [int(off[(g + 1) * el] - off[g * el]) for g in range(G)]
    g = int(np.argmax(loads))
    e0 = g * el
    cnt = np.diff(off[e0:e0 + el + 1]) * G
    offl = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    rows = int(offl[-1])
    dev = layer.x_perm.device
    x = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    wp = torch.empty(rows, dtype=torch.float32, device=dev)
    for i in range(el):
        a, b = int(off[e0 + i]), int(off[e0 + i + 1])
        x[offl[i]:offl[i + 1]] = layer.x_perm[a:b].repeat(G, 1)
        wp[offl[i]:offl[i + 1]] = layer.w_perm[a:b].repeat(G)
    z = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    offs = torch.from_numpy(offl).to(dev)
    fa = m._FwdArgs()
    fa.E, fa.H, fa.F, fa.rows = el, H, F, rows
    fa.precision = m.PREC_BF16
    fa.x_perm, fa.x_perm_scale = x.data_ptr(), None
    fa.w_gu = layer.w_gu[e0:e0 + el].data_ptr()
    fa.w_dn = layer.w_dn[e0:e0 + el].data_ptr()
    fa.w_perm, fa.offsets, fa.z_perm = wp.data_ptr(), offs.data_ptr(), \
        z.data_ptr()
    fa.h1_save, fa.a_save = None, None
    n = ctypes.c_size_t()
    m._check(layer.lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(fa),
                                                          ctypes.byref(n)))
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
    fa.ws, fa.ws_bytes = ws.data_ptr(), ws.numel()

    def run():
        m._check(layer.lib.moe_grouped_mlp_fwd(layer.ctx, ctypes.byref(fa),
                                               st))

    run()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(K):
        run()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    tf = 6.0 * rows * H * F / (ms * 1e-3) / 1e12
    return {"gpus": G, "gpu": g, "experts": [e0, e0 + el],
            "rows": rows, "rows_per_gpu": [r * G for r in loads],
            "grouped_mlp_ms": round(ms, 4), "TFLOP/s": round(tf, 1),
            "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4),
            "what": "grouped MLP forward (bf16) on the heaviest GPU's "
                    "experts of an expert-parallel split over 8 GPUs, "
                    "8x this workload's rows for them; exchanges not run"}


def graph_extra(layer, st, K):
    """The step captured once in a HIP graph and replayed, against the same
    stages launched eagerly: what launch overhead costs at this size."""
    import torch
    stages = layer.stages()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, fn in stages:
            fn(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for _, fn in stages:
            fn(cs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(run):
        run()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    def eager():
        for _, fn in stages:
            fn(st)

    t_graph, t_eager = timed(g.replay), timed(eager)
    return {"graph_ms_per_step": round(t_graph, 4),
            "eager_ms_per_step": round(t_eager, 4),
            "what": "the whole step captured in one HIP graph and replayed "
                    "vs launched call by call (HIP events, same stream)"}


def router_extra(m, layer, cfg, d, st, K):
    """Router projection (and, with a backward pass, the router backward)
    on the workload's tokens, timed with HIP events on the library stream;
    reported beside the step, not inside it."""
    import torch
    E, H, T, k = cfg.E, cfg.H, cfg.T, cfg.k
    w_r = torch.from_numpy(d["w_r"].view(np.int16)).view(torch.bfloat16).cuda()
    bias = None
    if cfg.zipf > 0.0:
        bias = torch.from_numpy(d["bias"].astype(np.float32)).cuda()
    out = torch.empty((T, E), dtype=torch.float32, device="cuda")
    P = lambda t: t.data_ptr() if t is not None else None
    lib = layer.lib

    def logits():
        m._check(lib.moe_router_logits(layer.ctx, P(layer.x), P(w_r), P(bias),
                                       T, H, E, P(out), st))

    def timed(fn):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    ms = timed(logits)
    fl = 2.0 * T * E * H
    res = {"logits_ms": round(ms, 4),
           "logits_fp64_TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2),
           "fp64_peak_TFLOP/s": PEAK_FP64_TFLOPS}
    if bias is None:   # the generator's bias is float64, the call's float32
        res["logits_equal_to_input_logits"] = float(
            (out.cpu().numpy() == d["logits"]).mean())
    if cfg.backward:
        idx = layer.idx
        dw = torch.randn((T, k), dtype=torch.float32, device="cuda")
        dl = torch.empty((T, E), dtype=torch.float32, device="cuda")
        dW = torch.empty((E, H), dtype=torch.float32, device="cuda")
        dx = torch.empty((T, H), dtype=torch.float32, device="cuda")
        n = ctypes.c_size_t()
        m._check(lib.moe_router_bwd_workspace_size(T, H, E, ctypes.byref(n)))
        ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device="cuda")

        def bwd():
            m._check(lib.moe_router_bwd(layer.ctx, P(out), P(idx), P(dw),
                                        P(layer.x), P(w_r), T, H, E, k, 1,
                                        P(dl), P(dW), P(dx), P(ws), ws.numel(),
                                        st))
        msb = timed(bwd)
        res["bwd_ms"] = round(msb, 4)
        res["bwd_fp32_TFLOP/s"] = round(4.0 * T * E * H / (msb * 1e-3) / 1e12,
                                        2)
    res["what"] = ("moe_router_logits (float64, ascending h, bit-exact) and "
                   "moe_router_bwd (dlogits + dW_r + dx, float32) per call; "
                   "logits_equal_to_input_logits (no bias): share of the "
                   "workload's generated logits (numpy float64 matmul) "
                   "reproduced bit for bit")
    return res


# the other workloads, each timed in the default run after the headline one
CONFIG_EXTRAS = ("tiny", "qwen3", "mixtral_mxfp8", "mixtral_mxfp8_bwd",
                 "mixtral_fp8t", "qwen3_long")


def _config_data(cfg, base_cfg, base_d):
    """Inputs of cfg; a workload with the headline's shapes and router reuses
    its tensors (same seed, same streams), drawing only dY if needed."""
    from synthetic import generate, generate_config
    same = all(getattr(cfg, a) == getattr(base_cfg, a)
               for a in ("T", "H", "F", "E", "k", "zipf"))
    if not same:
        return generate_config(cfg, seed=0)
    d = dict(base_d)
    if cfg.backward and d.get("dy") is None:
        d["dy"] = generate(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, zipf=cfg.zipf,
                           seed=0, want=("dy",))["dy"]
    return d


def config_run(m, cfg, d, dev, K, W):
    """One workload's step, timed like the headline run (K steps after W
    warm-up steps, every library kernel bracketed by HIP events): step time,
    TFLOP/s, tokens/s, and each GEMM's and HBM kernel's roofline fraction."""
    import torch
    layer = Layer(m, cfg, d, dev)
    stages = layer.stages()
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(W):
        for _, fn in stages:
            fn(st)
    torch.cuda.synchronize()
    m.reset_kernel_timing()
    m.set_kernel_timing(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        for _, fn in stages:
            fn(st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    m.set_kernel_timing(False)
    peak = PEAK_BF16_TFLOPS if cfg.mode == "bf16" else PEAK_FP8_TFLOPS
    gemms, hbm = {}, {}
    for name in KERNELS:
        n, tot = m.kernel_time(name)
        if not n:
            continue
        ms_s = tot / K
        if name in KERNEL_FLOP:
            tf = KERNEL_FLOP[name](cfg) / (ms_s * 1e-3) / 1e12
            gemms[name] = {"ms_per_step": round(ms_s, 4),
                           "TFLOP/s": round(tf, 1),
                           "frac_mfma": round(tf / peak, 4)}
        elif name in KERNEL_BYTES:
            gb = KERNEL_BYTES[name](cfg) / (ms_s * 1e-3) / 1e9
            hbm[name] = {"ms_per_step": round(ms_s, 4), "GB/s": round(gb, 1),
                         "frac_hbm": round(gb / PEAK_HBM_GBS, 4)}
    m.reset_kernel_timing()
    if m.check_device_status() != 0:
        raise RuntimeError(f"device status set by {cfg.name}")
    flop = cfg.fwd_flop() + (cfg.bwd_flop() if cfg.backward else 0.0)
    tf = flop / (ms * 1e-3) / 1e12
    dom = "gemm_gate_up_swiglu_" + {"mxfp8": "mxfp8", "fp8t": "fp8t"}.get(
        cfg.mode, "bf16")
    out = {"workload": f"{cfg.name}: {cfg.description}",
           "passes": "fwd+bwd" if cfg.backward else "fwd",
           "steps": K, "warmup": W, "ms_per_step": round(ms, 4),
           "TFLOP/s": round(tf, 2), "tokens_per_s": round(cfg.T / (ms * 1e-3),
                                                            1),
           "mfma_frac_step": round(tf / peak, 4),
           "dominant": {"kernel": dom, **gemms.get(dom, {})},
           "gemms": gemms, "hbm_kernels": hbm}
    if cfg.mode in ("mxfp8", "fp8t"):
        out["prequantised_weights"] = prequantised_step(m, layer, cfg, st,
                                                        max(2, K // 2))
    del layer
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def configs_extra(m, base_cfg, base_d, dev, K):
    from synthetic import CONFIGS
    res = {}
    for name in CONFIG_EXTRAS:
        if name == base_cfg.name:
            continue
        cfg = CONFIGS[name]
        t0 = time.time()
        d = _config_data(cfg, base_cfg, base_d)
        print(f"[bench] configs: {name} inputs in {time.time() - t0:.1f} s",
              file=sys.stderr, flush=True)
        res[name] = config_run(m, cfg, d, dev, K, 2)
        del d
        print(f"[bench] configs: {name} {res[name]['ms_per_step']} ms/step",
              file=sys.stderr, flush=True)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding of this path is a design note, not a "
              "runnable configuration.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.write_traffic:
        write_traffic(args.workload, args.write_traffic,
                      "rocprofv3 --pmc FETCH_SIZE | WRITE_SIZE "
                      "--kernel-include-regex grouped_gemm -- python3 "
                      f"bench.py --workload {args.workload} --steps 1 "
                      "--warmup 0 --no-cpu-baseline --no-extras")
        return
    import torch
    import mixture_experts_grouped_router_amd as m
    from synthetic import CONFIGS, generate_config

    cfg = CONFIGS[args.workload]
    m.load_library()
    t0 = time.time()
    d = generate_config(cfg, seed=0)
    gen_s = time.time() - t0
    print(f"[bench] inputs for {cfg.name} generated in {gen_s:.1f} s",
          file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layer = Layer(m, cfg, d, dev)
    stages = layer.stages()
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream

    for _ in range(args.warmup):
        for _, fn in stages:
            fn(st)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # every library kernel of the timed region is bracketed by HIP events on
    # the stream it runs on (the library's own timing facility)
    m.reset_kernel_timing()
    m.set_kernel_timing(True)
    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in stages]
          for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for s in range(K):
        for i, (_, fn) in enumerate(stages):
            ev[s][i][0].record(stream)
            fn(st)
            ev[s][i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / K
    per_stage = {name: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1])
                                      for s in range(K)]))
                 for i, (name, _) in enumerate(stages)}
    step_ms = [ev[s][0][0].elapsed_time(ev[s][-1][1]) for s in range(K)]
    m.set_kernel_timing(False)
    ktimes = {}      # name -> (launches, average ms, ms per step)
    for name in KERNELS:
        n, tot = m.kernel_time(name)
        if n:
            ktimes[name] = (n, tot / n, tot / K)
    m.reset_kernel_timing()
    status = m.check_device_status()
    if status != 0:
        raise RuntimeError(f"device status {status}")
    peak_mem = torch.cuda.max_memory_allocated()
    extras = {"peak_device_mem_GiB": round(peak_mem / 2**30, 2)}
    if not args.no_extras:
        extras["hbm_flushed"] = hbm_extras(m, layer, cfg, st)
        if cfg.mode in ("mxfp8", "fp8t"):
            extras["prequantised_weights"] = prequantised_step(
                m, layer, cfg, st, max(1, K // 2))
        if cfg.mode == "bf16" and not cfg.backward:
            extras["expert_loop"] = expert_loop_extra(m, layer, cfg, st,
                                                      max(2, K // 4))
            extras["ep_share"] = ep_share_extra(m, layer, cfg, st,
                                                max(2, K // 4))
        extras["router"] = router_extra(m, layer, cfg, d, st, max(2, K // 2))
        extras["graph"] = graph_extra(layer, st, max(2, K // 2))
    if not args.no_extras and not args.no_configs:
        del layer, stages
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        extras["configs"] = configs_extra(m, cfg, d, dev, max(4, K // 2))

    flop = cfg.fwd_flop() + (cfg.bwd_flop() if cfg.backward else 0.0)
    tflops = flop / (ms_step * 1e-3) / 1e12
    tokens_s = cfg.T / (ms_step * 1e-3)
    work = algorithmic(cfg)
    peak = PEAK_BF16_TFLOPS if cfg.mode == "bf16" else PEAK_FP8_TFLOPS
    # dominant kernel: the grouped gate/up GEMM with the ScaledSwiGLU
    # epilogue; one launch covers all T*k routed rows: 4*T*k*H*F flop
    dom = "gemm_gate_up_swiglu_" + {"mxfp8": "mxfp8", "fp8t": "fp8t"}.get(
        cfg.mode, "bf16")
    dom_flop = 4.0 * cfg.rows * cfg.H * cfg.F
    n_dom, dom_ms, _ = ktimes[dom]
    ach = dom_flop / (dom_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1),
            "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
            "traffic": traffic_for(dom, cfg),
            "avg_launch_ms": round(dom_ms, 4), "launches": n_dom,
            "work_per_launch": f"4*T*k*H*F = {dom_flop:.4e} flop"}
    kernels = {}
    for name, (n, ms, ms_s) in ktimes.items():
        # rates from the kernel's time per step and its work per step
        kd = {"launches": n, "avg_ms": round(ms, 4), "ms_per_step":
              round(ms_s, 4)}
        if name in KERNEL_FLOP:
            f = KERNEL_FLOP[name](cfg)
            kd["TFLOP/s"] = round(f / (ms_s * 1e-3) / 1e12, 1)
            kd["frac_mfma"] = round(f / (ms_s * 1e-3) / 1e12 / peak, 4)
        if name in KERNEL_BYTES:
            b = KERNEL_BYTES[name](cfg)
            kd["GB/s"] = round(b / (ms_s * 1e-3) / 1e9, 1)
            kd["frac_hbm"] = round(b / (ms_s * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        kernels[name] = kd
    stage_rates = {}
    for name, ms in per_stage.items():
        if name in work:
            kind, amt = work[name]
            if kind == "bytes":
                stage_rates[name] = {"ms": round(ms, 4), "GB/s": round(
                    amt / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(
                    amt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            else:
                stage_rates[name] = {"ms": round(ms, 4), "TFLOP/s": round(
                    amt / (ms * 1e-3) / 1e12, 1), "frac_mfma": round(
                    amt / (ms * 1e-3) / 1e12 / peak, 4)}
        else:
            stage_rates[name] = {"ms": round(ms, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens
        if n_tok <= 0:
            # about 10-30 s of host work for the oracle (float64 BLAS on
            # 16 host threads runs the per-expert matmuls at ~0.4 TFLOP/s)
            per_tok = (18.0 if cfg.backward else 6.0) * cfg.k * cfg.H * cfg.F
            n_tok = max(16, min(cfg.T, int(6e12 / per_tok)))
            if cfg.mode != "bf16":   # one expert, one FFN slice (above)
                n_tok = min(cfg.T, 8192)
        cpu = cpu_baseline(cfg, d, n_tok)

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp8": "mxfp8-e4m3", "fp8t": "fp8-e4m3-tensor-scaled"}.get(
            cfg.mode, "bf16"),
        "data": "synthetic (seeded; random-init expert weights)",
        "config": {"workload": f"{cfg.name}: {cfg.description}",
                   "T": cfg.T, "H": cfg.H, "F": cfg.F, "E": cfg.E,
                   "k": cfg.k, "mode": cfg.mode,
                   "passes": "fwd+bwd" if cfg.backward else "fwd",
                   "parallelism": "single GPU"},
        "step_ms_spread": {"min": round(min(step_ms), 4),
                           "median": round(float(np.median(step_ms)), 4),
                           "max": round(max(step_ms), 4)},
        "tokens_per_s": round(tokens_s, 1),
        "mfma_frac_step": round(tflops / peak, 4),
        "roofline": roof,
        "stages": stage_rates,
        "kernels": kernels,
        "wall_s_timed": round(wall, 3),
        "cpu_baseline": cpu,
        **extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
