"""Python binding of libmoe, the MoE expert-MLP hot path on MI355X (gfx950).

Thin ctypes layer over the C ABI in ``include/moe.h``: every function here
has the name of the C entry point it wraps, checks tensor shapes/dtypes,
allocates outputs with torch (device memory only) and passes raw pointers and
the current HIP stream.  All arithmetic runs in the HIP kernels of
``libmoe.so``; there is no CPU or torch fallback -- if the library is missing
the import of any entry point raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Optional, Tuple

import torch

__all__ = [
    "lib_path", "load_library", "MoEError", "PREC_BF16", "PREC_MXFP8",
    "PREC_FP8_TENSOR", "fp8_tensor_quantize",
    "ROWWISE", "COLWISE", "moe_router_logits", "moe_router_bwd",
    "moe_route_topk", "moe_permute", "moe_permute_noalloc",
    "moe_gather_rows",
    "moe_unpermute", "moe_unpermute_probs_grad", "mxfp8_quantize",
    "mxfp8_quantize_f32",
    "moe_grouped_mlp_fwd", "moe_expert_loop_mlp_fwd", "moe_grouped_mlp_bwd",
    "check_device_status",
    "mx_segment_ld", "set_kernel_timing", "reset_kernel_timing",
    "kernel_time",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmoe.so")

PREC_BF16 = 0
PREC_MXFP8 = 1
PREC_FP8_TENSOR = 2
ROWWISE = 0
COLWISE = 1

_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_c_sz = ctypes.c_size_t


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libmoe status {status}: {msg}")
        self.status = status


class _FwdArgs(ctypes.Structure):
    _fields_ = [
        ("E", _c_i32), ("H", _c_i32), ("F", _c_i32), ("rows", _c_i64),
        ("precision", ctypes.c_int),
        ("x_perm", _c_p), ("x_perm_scale", _c_p),
        ("w_gu", _c_p), ("w_dn", _c_p),
        ("w_gu_q", _c_p), ("w_gu_s", _c_p), ("w_dn_q", _c_p), ("w_dn_s", _c_p),
        ("w_perm", _c_p), ("offsets", _c_p),
        ("z_perm", _c_p), ("h1_save", _c_p), ("a_save", _c_p),
        ("ws", _c_p), ("ws_bytes", _c_sz),
        ("a_q_save", _c_p), ("a_s_save", _c_p),
        ("w_gu_ts", _c_p), ("w_dn_ts", _c_p),
    ]


class _BwdArgs(ctypes.Structure):
    _fields_ = [
        ("E", _c_i32), ("H", _c_i32), ("F", _c_i32), ("rows", _c_i64),
        ("precision", ctypes.c_int),
        ("x_perm", _c_p), ("w_gu", _c_p), ("w_dn", _c_p), ("w_perm", _c_p),
        ("offsets", _c_p), ("h1_save", _c_p), ("a_save", _c_p),
        ("dz_perm", _c_p), ("dx_perm", _c_p), ("dw_gu", _c_p),
        ("dw_dn", _c_p), ("dw_perm", _c_p),
        ("ws", _c_p), ("ws_bytes", _c_sz),
        ("w_gu_qt", _c_p), ("w_gu_st", _c_p), ("w_dn_qt", _c_p),
        ("w_dn_st", _c_p),
    ]


_SIGS = {
    "moe_ctx_create": [ctypes.c_int, ctypes.POINTER(_c_p)],
    "moe_ctx_destroy": [_c_p],
    "moe_ctx_check_device_status": [_c_p, _c_p, ctypes.POINTER(_c_i32)],
    "moe_route_topk": [_c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_i32, _c_p, _c_p,
                       _c_p],
    "moe_router_logits": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32,
                          _c_p, _c_p],
    "moe_fp8_tensor_quantize_workspace_size": [_c_i64, ctypes.POINTER(_c_sz)],
    "moe_fp8_tensor_quantize": [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                                _c_sz, _c_p],
    "moe_router_bwd_workspace_size": [_c_i64, _c_i32, _c_i32,
                                      ctypes.POINTER(_c_sz)],
    "moe_router_bwd": [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32,
                       _c_i32, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_sz,
                       _c_p],
    "moe_permute_workspace_size": [_c_i64, _c_i32, _c_i32,
                                   ctypes.POINTER(_c_sz)],
    "moe_permute": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_i32,
                    ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                    _c_p, _c_sz, _c_p],
    "moe_permute_noalloc": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32,
                            _c_i32, ctypes.c_int, _c_p, _c_p, _c_p, _c_p,
                            _c_p, _c_p, _c_p, _c_p],
    "moe_gather_rows": [_c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p],
    "moe_unpermute": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_p,
                      _c_p],
    "moe_unpermute_probs_grad": [_c_p, _c_p, _c_p, _c_i64, _c_i32, _c_p,
                                 _c_p],
    "mxfp8_quantize": [_c_p, _c_p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_p,
                       _c_i32, _c_p, _c_p, _c_p],
    "mxfp8_quantize_f32": [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "moe_grouped_mlp_fwd_workspace_size": [ctypes.POINTER(_FwdArgs),
                                           ctypes.POINTER(_c_sz)],
    "moe_grouped_mlp_fwd": [_c_p, ctypes.POINTER(_FwdArgs), _c_p],
    "moe_expert_loop_mlp_fwd_workspace_size": [ctypes.POINTER(_FwdArgs),
                                               ctypes.POINTER(_c_sz)],
    "moe_expert_loop_mlp_fwd": [_c_p, ctypes.POINTER(_FwdArgs), _c_p],
    "moe_grouped_mlp_bwd_workspace_size": [ctypes.POINTER(_BwdArgs),
                                           ctypes.POINTER(_c_sz)],
    "moe_grouped_mlp_bwd": [_c_p, ctypes.POINTER(_BwdArgs), _c_p],
    "moe_hbm_stream_reference": [_c_p, _c_p, _c_i64, _c_i32, _c_p, _c_p],
    "moe_hbm_stream_mix": [_c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_p, _c_p],
    "moe_ctx_set_kernel_timing": [_c_p, _c_i32],
    "moe_ctx_reset_kernel_timing": [_c_p],
    "moe_ctx_kernel_time": [_c_p, ctypes.c_char_p, ctypes.POINTER(_c_i64),
                            ctypes.POINTER(ctypes.c_double)],
}

_lib = None
_lib_lock = threading.Lock()
_ctx: Dict[int, int] = {}


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built).  The environment
    variable MOE_LIBRARY_PATH selects another build of the same library."""
    global _lib
    with _lib_lock:
        if _lib is None:
            p = path or os.environ.get("MOE_LIBRARY_PATH") or lib_path
            if not os.path.exists(p):
                raise ImportError(
                    f"{p} not found: build it with "
                    "`python -m mixture_experts_grouped_router_amd.build`")
            lib = ctypes.CDLL(p)
            for name, argtypes in _SIGS.items():
                fn = getattr(lib, name)
                fn.argtypes = argtypes
                fn.restype = ctypes.c_int
            lib.moe_status_string.argtypes = [ctypes.c_int]
            lib.moe_status_string.restype = ctypes.c_char_p
            lib.moe_last_error.argtypes = []
            lib.moe_last_error.restype = ctypes.c_char_p
            _lib = lib
        return _lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        raise MoEError(status, lib.moe_last_error().decode())


def _context(device: torch.device) -> int:
    idx = device.index if device.index is not None else \
        torch.cuda.current_device()
    if idx not in _ctx:
        lib = load_library()
        h = _c_p()
        with torch.cuda.device(idx):
            _check(lib.moe_ctx_create(idx, ctypes.byref(h)))
        _ctx[idx] = h.value
    return _ctx[idx]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, shape, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def check_device_status(device=None) -> int:
    """Synchronise the current stream and return (and clear) the first
    device-side data error code (0 = none)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    lib = load_library()
    code = _c_i32(0)
    st = lib.moe_ctx_check_device_status(_context(dev), _stream(),
                                         ctypes.byref(code))
    if st not in (0, 5):
        _check(st)
    return int(code.value)


def set_kernel_timing(enable: bool, device=None) -> None:
    """Bracket every library kernel launch with HIP events (measurement)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    _check(load_library().moe_ctx_set_kernel_timing(_context(dev),
                                                    int(bool(enable))))


def reset_kernel_timing(device=None) -> None:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    _check(load_library().moe_ctx_reset_kernel_timing(_context(dev)))


def kernel_time(name: str, device=None) -> Tuple[int, float]:
    """(launches, summed milliseconds) of the library kernel `name` since the
    last reset (waits for the recorded events)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    n = _c_i64(0)
    ms = ctypes.c_double(0.0)
    _check(load_library().moe_ctx_kernel_time(_context(dev), name.encode(),
                                              ctypes.byref(n),
                                              ctypes.byref(ms)))
    return int(n.value), float(ms.value)


# --------------------------------------------------------------------------
def moe_route_topk(logits: torch.Tensor, k: int, renormalize: bool = True
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """logits float32 [T, E] -> (topk_idx int32 [T, k], topk_w float32 [T, k])."""
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    idx = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    lib = load_library()
    _check(lib.moe_route_topk(_context(logits.device), _ptr(logits), T, E, k,
                              int(bool(renormalize)), _ptr(idx), _ptr(w),
                              _stream()))
    return idx, w


def fp8_tensor_quantize(src: torch.Tensor, n_seg: int = 1
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 tensor holding n_seg equal tensors -> (E4M3 codes uint8 of the
    same shape, float32 scales [n_seg]); one scale amax / 448 per tensor."""
    if src.dtype != torch.bfloat16 or not src.is_contiguous():
        raise ValueError("src must be a contiguous bf16 tensor")
    n = src.numel()
    if n_seg < 1 or n % n_seg:
        raise ValueError("numel must split into n_seg equal tensors")
    dev = src.device
    codes = torch.empty(src.shape, dtype=torch.uint8, device=dev)
    scales = torch.empty(n_seg, dtype=torch.float32, device=dev)
    lib = load_library()
    nb = _c_sz(0)
    _check(lib.moe_fp8_tensor_quantize_workspace_size(n_seg, ctypes.byref(nb)))
    ws = torch.empty(max(int(nb.value), 256), dtype=torch.uint8, device=dev)
    _check(lib.moe_fp8_tensor_quantize(_context(dev), _ptr(src), n_seg,
                                       n // n_seg, _ptr(codes), _ptr(scales),
                                       _ptr(ws), ws.numel(), _stream()))
    return codes, scales


def moe_router_logits(x: torch.Tensor, w_r: torch.Tensor,
                      bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x bf16 [T, H], w_r bf16 [E, H], bias float32 [E] -> logits float32
    [T, E] (float64 accumulation in ascending h, one rounding)."""
    T, H = x.shape
    E = w_r.shape[0]
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_r, torch.bfloat16, (E, H), "w_r")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    lib = load_library()
    _check(lib.moe_router_logits(_context(x.device), _ptr(x), _ptr(w_r),
                                 _ptr(bias), T, H, E, _ptr(out), _stream()))
    return out


def moe_router_bwd(logits: torch.Tensor, topk_idx: torch.Tensor,
                   dtopk_w: torch.Tensor, x: torch.Tensor, w_r: torch.Tensor,
                   renormalize: bool = True, want_dw: bool = True,
                   want_dx: bool = True) -> Dict[str, torch.Tensor]:
    """Router backward: {"dlogits" [T, E]} (+ "dw_r" [E, H], "dx" [T, H]),
    float32."""
    T, E = logits.shape
    k = topk_idx.shape[1]
    H = x.shape[1]
    dev = logits.device
    _need(logits, torch.float32, (T, E), "logits")
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    _need(dtopk_w, torch.float32, (T, k), "dtopk_w")
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_r, torch.bfloat16, (E, H), "w_r")
    dl = torch.empty((T, E), dtype=torch.float32, device=dev)
    dw = torch.empty((E, H), dtype=torch.float32, device=dev) \
        if want_dw else None
    dx = torch.empty((T, H), dtype=torch.float32, device=dev) \
        if want_dx else None
    lib = load_library()
    n = _c_sz(0)
    _check(lib.moe_router_bwd_workspace_size(T, H, E, ctypes.byref(n)))
    ws = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)
    _check(lib.moe_router_bwd(_context(dev), _ptr(logits), _ptr(topk_idx),
                              _ptr(dtopk_w), _ptr(x), _ptr(w_r), T, H, E, k,
                              int(bool(renormalize)), _ptr(dl), _ptr(dw),
                              _ptr(dx), _ptr(ws), ws.numel(), _stream()))
    res = {"dlogits": dl}
    if want_dw:
        res["dw_r"] = dw
    if want_dx:
        res["dx"] = dx
    return res


def moe_permute(x: torch.Tensor, topk_idx: torch.Tensor, E: int,
                topk_w: Optional[torch.Tensor] = None,
                precision: int = PREC_BF16) -> Dict[str, torch.Tensor]:
    """Expert-order permutation + row gather.  Returns x_perm (bf16, or uint8
    E4M3 codes with x_perm_scale), w_perm (if topk_w), row_map, src_row,
    split_sizes, offsets."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    _need(x, torch.bfloat16, (T, H), "x")
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    if topk_w is not None:
        _need(topk_w, torch.float32, (T, k), "topk_w")
    rows = T * k
    if precision == PREC_BF16:
        x_perm = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
        xs = None
    else:
        x_perm = torch.empty((rows, H), dtype=torch.uint8, device=dev)
        xs = torch.empty((rows, H // 32), dtype=torch.uint8, device=dev)
    w_perm = torch.empty(rows, dtype=torch.float32, device=dev) \
        if topk_w is not None else None
    row_map = torch.empty(rows, dtype=torch.int32, device=dev)
    src_row = torch.empty(rows, dtype=torch.int32, device=dev)
    split = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    lib = load_library()
    nbytes = _c_sz(0)
    _check(lib.moe_permute_workspace_size(T, E, k, ctypes.byref(nbytes)))
    ws = torch.empty(max(int(nbytes.value), 16), dtype=torch.uint8, device=dev)
    _check(lib.moe_permute(
        _context(dev), _ptr(x), _ptr(topk_idx), _ptr(topk_w), T, H, E, k,
        precision, _ptr(x_perm), _ptr(xs), _ptr(w_perm), _ptr(row_map),
        _ptr(src_row), _ptr(split), _ptr(offsets), _ptr(ws), ws.numel(),
        _stream()))
    out = {"x_perm": x_perm, "row_map": row_map, "src_row": src_row,
           "split_sizes": split, "offsets": offsets}
    if xs is not None:
        out["x_perm_scale"] = xs
    if w_perm is not None:
        out["w_perm"] = w_perm
    return out


def moe_permute_noalloc(x: torch.Tensor, topk_idx: torch.Tensor,
                        topk_w: Optional[torch.Tensor],
                        out: Dict[str, torch.Tensor],
                        precision: int = PREC_BF16) -> Dict[str, torch.Tensor]:
    """moe_permute into caller-provided outputs ``out`` (keys x_perm, row_map,
    src_row, split_sizes, offsets, and x_perm_scale / w_perm as needed),
    with the library's static scratch instead of a workspace: the library
    call allocates nothing."""
    T, H = x.shape
    k = topk_idx.shape[1]
    E = out["split_sizes"].shape[0]
    rows = T * k
    _need(x, torch.bfloat16, (T, H), "x")
    _need(topk_idx, torch.int32, (T, k), "topk_idx")
    if topk_w is not None:
        _need(topk_w, torch.float32, (T, k), "topk_w")
    if precision == PREC_BF16:
        _need(out["x_perm"], torch.bfloat16, (rows, H), "x_perm")
    else:
        _need(out["x_perm"], torch.uint8, (rows, H), "x_perm")
        _need(out["x_perm_scale"], torch.uint8, (rows, H // 32),
              "x_perm_scale")
    for key in ("row_map", "src_row"):
        _need(out[key], torch.int32, (rows,), key)
    _need(out["split_sizes"], torch.int32, (E,), "split_sizes")
    _need(out["offsets"], torch.int32, (E + 1,), "offsets")
    if out.get("w_perm") is not None:
        _need(out["w_perm"], torch.float32, (rows,), "w_perm")
    lib = load_library()
    _check(lib.moe_permute_noalloc(
        _context(x.device), _ptr(x), _ptr(topk_idx), _ptr(topk_w), T, H, E,
        k, precision, _ptr(out["x_perm"]), _ptr(out.get("x_perm_scale")),
        _ptr(out.get("w_perm")), _ptr(out["row_map"]), _ptr(out["src_row"]),
        _ptr(out["split_sizes"]), _ptr(out["offsets"]), _stream()))
    return out


def moe_gather_rows(src: torch.Tensor, row_map: torch.Tensor, k: int
                    ) -> torch.Tensor:
    """dst[row_map[t*k+j]] = src[t] (bf16 [T, H] -> [T*k, H])."""
    T, H = src.shape
    _need(src, torch.bfloat16, (T, H), "src")
    _need(row_map, torch.int32, (T * k,), "row_map")
    dst = torch.empty((T * k, H), dtype=torch.bfloat16, device=src.device)
    lib = load_library()
    _check(lib.moe_gather_rows(_context(src.device), _ptr(src), _ptr(row_map),
                               T, H, k, _ptr(dst), _stream()))
    return dst


def moe_unpermute(z_perm: torch.Tensor, row_map: torch.Tensor, k: int,
                  topk_w: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[t] = sum_j c_j z_perm[row_map[t*k+j]] (c_j = 1 or topk_w[t, j])."""
    rows, H = z_perm.shape
    T = rows // k
    _need(z_perm, torch.bfloat16, (rows, H), "z_perm")
    _need(row_map, torch.int32, (rows,), "row_map")
    if topk_w is not None:
        _need(topk_w, torch.float32, (T, k), "topk_w")
    y = torch.empty((T, H), dtype=torch.bfloat16, device=z_perm.device)
    lib = load_library()
    _check(lib.moe_unpermute(_context(z_perm.device), _ptr(z_perm),
                             _ptr(row_map), _ptr(topk_w), T, H, k, _ptr(y),
                             _stream()))
    return y


def moe_unpermute_probs_grad(dw_perm: torch.Tensor, row_map: torch.Tensor,
                             k: int) -> torch.Tensor:
    rows = dw_perm.shape[0]
    _need(dw_perm, torch.float32, (rows,), "dw_perm")
    _need(row_map, torch.int32, (rows,), "row_map")
    out = torch.empty((rows // k, k), dtype=torch.float32,
                      device=dw_perm.device)
    lib = load_library()
    _check(lib.moe_unpermute_probs_grad(_context(dw_perm.device),
                                        _ptr(dw_perm), _ptr(row_map),
                                        rows // k, k, _ptr(out), _stream()))
    return out


def mx_segment_ld(rows: int, n_seg: int) -> int:
    """Row stride of the segment-wise column quantisation output."""
    return (rows + 32 * n_seg + 31) // 32 * 32


def mxfp8_quantize(src: torch.Tensor, axis: int = ROWWISE,
                   seg_offsets: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP8 codes + E8M0 scales of a bf16 tensor [.., rows, cols]."""
    if src.dim() == 2:
        batch, (rows, cols) = 1, src.shape
    elif src.dim() == 3:
        batch, rows, cols = src.shape
    else:
        raise ValueError("src must be 2-D or 3-D")
    _need(src, torch.bfloat16, tuple(src.shape), "src")
    dev = src.device
    lead = () if src.dim() == 2 else (batch,)
    n_seg = 0
    if axis == ROWWISE:
        codes = torch.empty(lead + (rows, cols), dtype=torch.uint8, device=dev)
        scales = torch.empty(lead + (rows, cols // 32), dtype=torch.uint8,
                             device=dev)
    elif seg_offsets is None:
        codes = torch.empty(lead + (cols, rows), dtype=torch.uint8, device=dev)
        scales = torch.empty(lead + (cols, rows // 32), dtype=torch.uint8,
                             device=dev)
    else:
        n_seg = seg_offsets.numel() - 1
        _need(seg_offsets, torch.int32, (n_seg + 1,), "seg_offsets")
        ld = mx_segment_ld(rows, n_seg)
        codes = torch.zeros((cols, ld), dtype=torch.uint8, device=dev)
        scales = torch.zeros((cols, ld // 32), dtype=torch.uint8, device=dev)
    lib = load_library()
    _check(lib.mxfp8_quantize(_context(dev), _ptr(src), batch, rows, cols,
                              axis, _ptr(seg_offsets), n_seg, _ptr(codes),
                              _ptr(scales), _stream()))
    return codes, scales


def mxfp8_quantize_f32(src: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Row-wise MXFP8 codes + E8M0 scales of a float32 tensor [rows, cols]
    (the encoder of the MXFP8 gate/up epilogue)."""
    rows, cols = src.shape
    _need(src, torch.float32, (rows, cols), "src")
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8,
                         device=src.device)
    lib = load_library()
    _check(lib.mxfp8_quantize_f32(_context(src.device), _ptr(src), rows, cols,
                                  _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def moe_grouped_mlp_fwd(x_perm: torch.Tensor, w_gu: torch.Tensor,
                        w_dn: torch.Tensor, offsets: torch.Tensor,
                        w_perm: Optional[torch.Tensor] = None,
                        precision: int = PREC_BF16,
                        x_perm_scale: Optional[torch.Tensor] = None,
                        w_gu_q: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                        w_dn_q: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                        save: bool = False,
                        out: Optional[torch.Tensor] = None,
                        ws: Optional[torch.Tensor] = None,
                        save_a_codes: bool = False,
                        ) -> Dict[str, torch.Tensor]:
    """Grouped gate/up GEMM -> ScaledSwiGLU x w -> grouped down GEMM.
    Returns {"z": bf16 [rows, H]} (+ "h1", "a" when save=True; + "a_q",
    "a_s", A's MXFP8 codes and row-major scales, when save_a_codes=True in
    MXFP8 mode).  w_gu_q / w_dn_q (optional, both or neither): the weights
    quantised beforehand, (codes, E8M0 scales) from mxfp8_quantize ROWWISE
    in MXFP8 mode, (codes, float32 scale per expert) from
    fp8_tensor_quantize(w, E) in tensor-scaled FP8 mode."""
    E, F2, H = w_gu.shape
    F = F2 // 2
    rows = x_perm.shape[0]
    dev = x_perm.device
    _need(w_gu, torch.bfloat16, (E, 2 * F, H), "w_gu")
    _need(w_dn, torch.bfloat16, (E, H, F), "w_dn")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    if precision == PREC_BF16 or x_perm_scale is None:
        _need(x_perm, torch.bfloat16, (rows, H), "x_perm")
    else:
        _need(x_perm, torch.uint8, (rows, H), "x_perm")
        _need(x_perm_scale, torch.uint8, (rows, H // 32), "x_perm_scale")
    if w_perm is not None:
        _need(w_perm, torch.float32, (rows,), "w_perm")
    z = out if out is not None else torch.empty((rows, H), dtype=torch.bfloat16,
                                                device=dev)
    _need(z, torch.bfloat16, (rows, H), "out")
    h1 = torch.empty((rows, 2 * F), dtype=torch.bfloat16, device=dev) \
        if save else None
    a = torch.empty((rows, F), dtype=torch.bfloat16, device=dev) \
        if save else None
    args = _FwdArgs()
    args.E, args.H, args.F, args.rows = E, H, F, rows
    args.precision = precision
    args.x_perm = _ptr(x_perm)
    args.x_perm_scale = _ptr(x_perm_scale)
    args.w_gu, args.w_dn = _ptr(w_gu), _ptr(w_dn)
    if precision == PREC_FP8_TENSOR:
        # (E4M3 codes, float32 scale per expert) as fp8_tensor_quantize
        # (w, n_seg=E) returns them
        if w_gu_q is not None:
            _need(w_gu_q[0], torch.uint8, (E, 2 * F, H), "w_gu_q codes")
            _need(w_gu_q[1], torch.float32, (E,), "w_gu_q scales")
            args.w_gu_q, args.w_gu_ts = _ptr(w_gu_q[0]), _ptr(w_gu_q[1])
        if w_dn_q is not None:
            _need(w_dn_q[0], torch.uint8, (E, H, F), "w_dn_q codes")
            _need(w_dn_q[1], torch.float32, (E,), "w_dn_q scales")
            args.w_dn_q, args.w_dn_ts = _ptr(w_dn_q[0]), _ptr(w_dn_q[1])
    else:
        if w_gu_q is not None:
            args.w_gu_q, args.w_gu_s = _ptr(w_gu_q[0]), _ptr(w_gu_q[1])
        if w_dn_q is not None:
            args.w_dn_q, args.w_dn_s = _ptr(w_dn_q[0]), _ptr(w_dn_q[1])
    args.w_perm = _ptr(w_perm)
    args.offsets = _ptr(offsets)
    args.z_perm = _ptr(z)
    args.h1_save, args.a_save = _ptr(h1), _ptr(a)
    aq = as_ = None
    if save_a_codes:
        aq = torch.empty((rows, F), dtype=torch.uint8, device=dev)
        as_ = torch.empty((rows, F // 32), dtype=torch.uint8, device=dev)
        args.a_q_save, args.a_s_save = _ptr(aq), _ptr(as_)
    lib = load_library()
    nbytes = _c_sz(0)
    _check(lib.moe_grouped_mlp_fwd_workspace_size(ctypes.byref(args),
                                                  ctypes.byref(nbytes)))
    if ws is None or ws.numel() < int(nbytes.value):
        ws = torch.empty(max(int(nbytes.value), 256), dtype=torch.uint8,
                         device=dev)
    args.ws, args.ws_bytes = _ptr(ws), ws.numel()
    _check(lib.moe_grouped_mlp_fwd(_context(dev), ctypes.byref(args),
                                   _stream()))
    res = {"z": z}
    if save:
        res["h1"], res["a"] = h1, a
    if save_a_codes:
        res["a_q"], res["a_s"] = aq, as_
    return res



def moe_expert_loop_mlp_fwd(x_perm: torch.Tensor, w_gu: torch.Tensor,
                            w_dn: torch.Tensor, offsets: torch.Tensor,
                            w_perm: Optional[torch.Tensor] = None,
                            save: bool = False,
                            out: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None,
                            ) -> Dict[str, torch.Tensor]:
    """The bf16 expert MLP as a per-expert loop (separate gate/up GEMM,
    SwiGLU and down GEMM launches per expert; the call waits for the
    stream to read the row counts): the baseline of moe_grouped_mlp_fwd.
    Returns {"z"} (+ "h1", "a" when save=True)."""
    E, F2, H = w_gu.shape
    F = F2 // 2
    rows = x_perm.shape[0]
    dev = x_perm.device
    _need(w_gu, torch.bfloat16, (E, 2 * F, H), "w_gu")
    _need(w_dn, torch.bfloat16, (E, H, F), "w_dn")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(x_perm, torch.bfloat16, (rows, H), "x_perm")
    if w_perm is not None:
        _need(w_perm, torch.float32, (rows,), "w_perm")
    z = out if out is not None else torch.empty((rows, H), dtype=torch.bfloat16,
                                                device=dev)
    _need(z, torch.bfloat16, (rows, H), "out")
    h1 = torch.empty((rows, 2 * F), dtype=torch.bfloat16, device=dev) \
        if save else None
    a = torch.empty((rows, F), dtype=torch.bfloat16, device=dev) \
        if save else None
    args = _FwdArgs()
    args.E, args.H, args.F, args.rows = E, H, F, rows
    args.precision = PREC_BF16
    args.x_perm = _ptr(x_perm)
    args.w_gu, args.w_dn = _ptr(w_gu), _ptr(w_dn)
    args.w_perm = _ptr(w_perm)
    args.offsets = _ptr(offsets)
    args.z_perm = _ptr(z)
    args.h1_save, args.a_save = _ptr(h1), _ptr(a)
    lib = load_library()
    nbytes = _c_sz(0)
    _check(lib.moe_expert_loop_mlp_fwd_workspace_size(ctypes.byref(args),
                                                      ctypes.byref(nbytes)))
    if ws is None or ws.numel() < int(nbytes.value):
        ws = torch.empty(max(int(nbytes.value), 256), dtype=torch.uint8,
                         device=dev)
    args.ws, args.ws_bytes = _ptr(ws), ws.numel()
    _check(lib.moe_expert_loop_mlp_fwd(_context(dev), ctypes.byref(args),
                                       _stream()))
    res = {"z": z}
    if save:
        res["h1"], res["a"] = h1, a
    return res

def moe_grouped_mlp_bwd(dz_perm: torch.Tensor, x_perm: torch.Tensor,
                        w_gu: torch.Tensor, w_dn: torch.Tensor,
                        offsets: torch.Tensor, h1: torch.Tensor,
                        a: torch.Tensor, w_perm: Optional[torch.Tensor] = None,
                        precision: int = PREC_BF16,
                        ws: Optional[torch.Tensor] = None,
                        w_gu_qt: Optional[Tuple[torch.Tensor,
                                                torch.Tensor]] = None,
                        w_dn_qt: Optional[Tuple[torch.Tensor,
                                                torch.Tensor]] = None,
                        ) -> Dict[str, torch.Tensor]:
    """Backward of moe_grouped_mlp_fwd: returns dx_perm, dw_gu, dw_dn (bf16)
    and dw_perm (float32, when w_perm is given).  MXFP8: w_gu_qt / w_dn_qt
    are optional (codes, scales) of the weights quantised COLWISE
    (mxfp8_quantize(w, COLWISE)), reused instead of quantised in the call."""
    E, F2, H = w_gu.shape
    F = F2 // 2
    rows = x_perm.shape[0]
    dev = x_perm.device
    _need(dz_perm, torch.bfloat16, (rows, H), "dz_perm")
    _need(x_perm, torch.bfloat16, (rows, H), "x_perm")
    _need(w_gu, torch.bfloat16, (E, 2 * F, H), "w_gu")
    _need(w_dn, torch.bfloat16, (E, H, F), "w_dn")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(h1, torch.bfloat16, (rows, 2 * F), "h1")
    _need(a, torch.bfloat16, (rows, F), "a")
    dx = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    dw_gu = torch.empty((E, 2 * F, H), dtype=torch.bfloat16, device=dev)
    dw_dn = torch.empty((E, H, F), dtype=torch.bfloat16, device=dev)
    dw_perm = torch.empty(rows, dtype=torch.float32, device=dev) \
        if w_perm is not None else None
    args = _BwdArgs()
    args.E, args.H, args.F, args.rows = E, H, F, rows
    args.precision = precision
    args.x_perm, args.w_gu, args.w_dn = _ptr(x_perm), _ptr(w_gu), _ptr(w_dn)
    args.w_perm, args.offsets = _ptr(w_perm), _ptr(offsets)
    args.h1_save, args.a_save = _ptr(h1), _ptr(a)
    args.dz_perm, args.dx_perm = _ptr(dz_perm), _ptr(dx)
    args.dw_gu, args.dw_dn, args.dw_perm = _ptr(dw_gu), _ptr(dw_dn), \
        _ptr(dw_perm)
    if w_gu_qt is not None:
        _need(w_gu_qt[0], torch.uint8, (E, H, 2 * F), "w_gu_qt codes")
        _need(w_gu_qt[1], torch.uint8, (E, H, 2 * F // 32), "w_gu_qt scales")
        args.w_gu_qt, args.w_gu_st = _ptr(w_gu_qt[0]), _ptr(w_gu_qt[1])
    if w_dn_qt is not None:
        _need(w_dn_qt[0], torch.uint8, (E, F, H), "w_dn_qt codes")
        _need(w_dn_qt[1], torch.uint8, (E, F, H // 32), "w_dn_qt scales")
        args.w_dn_qt, args.w_dn_st = _ptr(w_dn_qt[0]), _ptr(w_dn_qt[1])
    lib = load_library()
    nbytes = _c_sz(0)
    _check(lib.moe_grouped_mlp_bwd_workspace_size(ctypes.byref(args),
                                                  ctypes.byref(nbytes)))
    if ws is None or ws.numel() < int(nbytes.value):
        ws = torch.empty(max(int(nbytes.value), 256), dtype=torch.uint8,
                         device=dev)
    args.ws, args.ws_bytes = _ptr(ws), ws.numel()
    _check(lib.moe_grouped_mlp_bwd(_context(dev), ctypes.byref(args),
                                   _stream()))
    res = {"dx_perm": dx, "dw_gu": dw_gu, "dw_dn": dw_dn}
    if dw_perm is not None:
        res["dw_perm"] = dw_perm
    return res
