"""CPU oracle for the MoE expert-MLP path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The GPU library never calls it and
shares no code with it.

Plain, slow, obviously correct: numpy in float64, one Python loop per expert,
a library matmul / stable sort as the only "fast" primitives.  No blocking, no
fusion and no reordering beyond what the definitions below state.

Sources (web pages; titles as published, sections as headed on the page):

[PG1] "NVIDIA presents an efficient path for training biological MoE models"
      (sitech.ge).  Sections: "Grouped experts instead of a Python loop",
      "Reducing memory and quantisation cost".
[PG2] "Efficient MoE training for biological foundation models (NVIDIA)"
      (news.bpdata.com).  Sections: "Why dense and MoE models differ",
      "1) Fragmented expert kernels", "2) Model size and activation memory",
      "3) Quantisation overhead in low-precision training".
[PG3] "Nous Research scales expert parallelism with DeepEP" (seventnews.com),
      paragraph on practical implications (Top-k, capacity factor).
[PG4] "NVIDIA NeMo AutoModel: 3.7x faster MoE fine-tuning with expert
      parallelism and DeepEP" (seventnews.com).  Sections "Background",
      "Using Transformers v5 features" (eager / batched_mm / grouped_mm).

The pages state the problem (tokens, per-expert weights, split_sizes,
routing weights scaled inside the grouped MLP, MXFP8 = 8-bit elements with one
scale per 32 consecutive values, 16-bit master weights) but not every formula.
Where they are silent this module takes the readings listed here:

  R1  router: softmax over the E logits, keep the k largest; weights are the
      softmax restricted to the chosen set (renormalize=True) or the plain
      softmax over all E (renormalize=False); evaluated in float64, stored
      float32.
  R2  selection order: larger logit first; equal logits -> lower expert id;
      +0 == -0.  Slot j=0 holds the top expert.
  R3  permutation: pair p = t*k + j; stable by expert, then by p.
  R4  expert weights nn.Linear-style [out, in]: W_gu [E, 2F, H] with gate rows
      0..F-1 and up rows F..2F-1; W_dn [E, H, F]; no biases.
  R5  SwiGLU(g, u) = silu(g) * u, silu(z) = z / (1 + exp(-z)).
  R6  ScaledSwiGLU: the routing weight of the (token, expert) pair multiplies
      the SwiGLU output before the down projection; the combine is then a
      plain sum over the k slots.
  R7  MXFP8 (OCP Microscaling reading): per block of 32 values along the
      GEMM's K, scale exponent s = floor(log2 amax) - 8 clamped to
      [-127, 127] (amax = 0 -> -127), stored E8M0 as s + 127; elements
      E4M3 (bias 7, max 448, no infinities) of v * 2^-s, round to nearest
      even, saturating at +-448, sign kept on zero.
  R8  MXFP8 layer: quantise x_perm and W_gu along H, A and W_dn along F, GEMMs
      on the dequantised values; backward quantises each GEMM operand along
      that GEMM's K, token-direction blocks restarting at each expert segment
      and zero-padded at its end.
  R9  router projection: logits = x W_r^T (+ optional per-expert bias), the
      gate W_r [E, H] bf16; each logit is accumulated in float64 one term at
      a time in ascending h (products of two bf16 values are exact in
      float64), the bias added last, then rounded once to float32.  The
      fixed order makes the result a function of the inputs alone, so the
      routing it feeds can be compared bit for bit.
  R10 router backward: the routing-weight gradient reaches the logits only
      through the softmax the forward used (over the chosen set, or over all
      E without renormalisation); the top-k selection itself is piecewise
      constant and passes no gradient.  dW_r = dlogits^T x, and the router's
      share of dx = dlogits W_r.
  R11 tensor-scaled FP8 (the other 8-bit mode the pages name): one float32
      scale per tensor, s = amax / 448 from an amax pass (s = 1 for an
      all-zero tensor), codes = E4M3(float32(v / s)) (round to nearest even,
      saturating), value = decode(code) * s.  A "tensor" is x_perm, each
      expert's W_gu[e] and W_dn[e] (separate weight tensors per expert, as
      in a grouped linear layer), and the SwiGLU output A stored as bf16
      (its amax taken over the bf16 values).  GEMMs run on the codes and
      multiply by the two scales.

Pins of this module against things other than itself live in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

f64 = np.float64


# --------------------------------------------------------------------------
# Router top-k  [PG3 practical implications: Top-k routing;
#                PG2 "Why dense and MoE models differ": a small subset of
#                experts is active per token]
# --------------------------------------------------------------------------
def route_topk(logits: np.ndarray, k: int, renormalize: bool = True
               ) -> Tuple[np.ndarray, np.ndarray]:
    """logits float32 [T, E] -> (topk_idx int32 [T, k], topk_w float32 [T, k]).

    Readings R1, R2.  The selection compares the float32 logits exactly.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(lg)):
        # a precondition of the routing: no selection is defined for them
        raise ValueError("router logits must be finite")
    lv = lg.astype(f64) + 0.0          # -0.0 + 0.0 == +0.0 (R2)
    # a stable sort keeps the lower expert id first among equal logits
    order = np.argsort(-lv, axis=1, kind="stable")
    idx = order[:, :k]
    m = lv.max(axis=1, keepdims=True)
    ex = np.exp(lv - m)
    sel = np.take_along_axis(ex, idx, axis=1)
    denom = sel.sum(axis=1, keepdims=True) if renormalize else \
        ex.sum(axis=1, keepdims=True)
    w = sel / denom
    return idx.astype(np.int32), w.astype(np.float32)


# --------------------------------------------------------------------------
# Permutation into expert-contiguous order with split_sizes
# [PG1 "Grouped experts instead of a Python loop"; PG2 "1) Fragmented expert
#  kernels": the grouped call receives the per-expert token counts
#  (split_sizes); PG4 "Using Transformers v5 features": grouped_mm runs on
#  sorted tokens]
# --------------------------------------------------------------------------
def permute_index(topk_idx: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    """topk_idx int [T, k] -> split_sizes [E], offsets [E+1], row_map [T*k],
    src_row [T*k] (all int32).  Reading R3.

    row_map[p] is the expert-ordered row of pair p; src_row is its inverse.
    """
    e = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    if e.size and (e.min() < 0 or e.max() >= E):
        raise ValueError("expert id out of range")
    split = np.bincount(e, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(split)
    src_row = np.argsort(e, kind="stable")   # by expert, then by pair index
    row_map = np.empty_like(src_row)
    row_map[src_row] = np.arange(e.size)
    return {
        "split_sizes": split.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "row_map": row_map.astype(np.int32),
        "src_row": src_row.astype(np.int32),
    }


def permute_rows(x: np.ndarray, src_row: np.ndarray, k: int) -> np.ndarray:
    """x_perm[r] = x[src_row[r] // k] (a row copy, any dtype)."""
    return np.asarray(x)[np.asarray(src_row, dtype=np.int64) // k]


def permute_weights(topk_w: np.ndarray, src_row: np.ndarray) -> np.ndarray:
    """w_perm[r] = topk_w.flat[src_row[r]] (float32)."""
    return np.asarray(topk_w, dtype=np.float32).reshape(-1)[
        np.asarray(src_row, dtype=np.int64)]


# --------------------------------------------------------------------------
# Grouped MLP forward: grouped GEMM gate/up -> ScaledSwiGLU -> grouped GEMM
# down  [PG1 "Reducing memory and quantisation cost": GroupedLinear ->
#  ScaledSwiGLU -> GroupedLinear; PG1 "Grouped experts instead of a Python
#  loop": routing weights scaled inside the grouped MLP]
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """R5: z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _as_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or any float array -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(f64)
    return a.astype(f64)


def grouped_mlp_fwd(x_perm, w_gu, w_dn, w_perm, offsets,
                    keep: bool = False) -> Dict[str, np.ndarray]:
    """Per expert e (ascending), rows [offsets[e], offsets[e+1]):
         h1 = X_e W_gu[e]^T ; g = h1[:, :F] ; u = h1[:, F:]
         a  = w * silu(g) * u           (R6: scaled before the down proj)
         z  = a W_dn[e]^T
    Returns z (float64 [rows, H]); with keep=True also h1 and a.
    ``w_perm`` None means weight 1 (unweighted MLP).
    """
    E = len(offsets) - 1
    rows = np.asarray(x_perm).shape[0]
    F = np.asarray(w_gu).shape[1] // 2
    H = np.asarray(w_dn).shape[1]
    z = np.zeros((rows, H), dtype=f64)
    h1_all = np.zeros((rows, 2 * F), dtype=f64) if keep else None
    a_all = np.zeros((rows, F), dtype=f64) if keep else None
    w = np.ones(rows) if w_perm is None else np.asarray(w_perm, dtype=f64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = _as_f64(x_perm[lo:hi])
        h1 = X @ _as_f64(w_gu[e]).T
        g, u = h1[:, :F], h1[:, F:]
        a = w[lo:hi, None] * silu(g) * u
        z[lo:hi] = a @ _as_f64(w_dn[e]).T
        if keep:
            h1_all[lo:hi] = h1
            a_all[lo:hi] = a
    out = {"z": z}
    if keep:
        out["h1"] = h1_all
        out["a"] = a_all
    return out


# --------------------------------------------------------------------------
# Unpermute / combine back to token order
# [PG4 "Sources of speedup": dispatch and combine around the expert compute]
# --------------------------------------------------------------------------
def unpermute(z_perm: np.ndarray, row_map: np.ndarray, k: int,
              topk_w: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t] = sum_{j ascending} c_j * z[row_map[t*k + j]], with c_j = 1
    (weights already applied in the MLP, R6) or c_j = topk_w[t, j]."""
    z = _as_f64(z_perm)
    rm = np.asarray(row_map, dtype=np.int64).reshape(-1, k)
    T = rm.shape[0]
    y = np.zeros((T, z.shape[1]), dtype=f64)
    for j in range(k):
        c = 1.0 if topk_w is None else \
            np.asarray(topk_w, dtype=f64).reshape(T, k)[:, j:j + 1]
        y += c * z[rm[:, j]]
    return y


def layer_fwd(x, logits, w_gu, w_dn, k: int, renormalize: bool = True,
              keep: bool = False) -> Dict[str, np.ndarray]:
    """Whole forward: route -> permute -> grouped MLP -> unpermute."""
    E = np.asarray(w_gu).shape[0]
    idx, w = route_topk(logits, k, renormalize)
    maps = permute_index(idx, E)
    x_perm = permute_rows(x, maps["src_row"], k)
    w_perm = permute_weights(w, maps["src_row"])
    mlp = grouped_mlp_fwd(x_perm, w_gu, w_dn, w_perm, maps["offsets"],
                          keep=keep)
    y = unpermute(mlp["z"], maps["row_map"], k)
    out = {"topk_idx": idx, "topk_w": w, "w_perm": w_perm, "x_perm": x_perm,
           "y": y, **maps, **mlp}
    return out


# --------------------------------------------------------------------------
# Backward  [PG1 "Reducing memory and quantisation cost": the fused forward
#  op has a counterpart in the backward pass]
# --------------------------------------------------------------------------
def grouped_mlp_bwd(dz_perm, x_perm, w_gu, w_dn, w_perm, offsets
                    ) -> Dict[str, np.ndarray]:
    """Gradients of grouped_mlp_fwd's z w.r.t. x_perm, W_gu, W_dn, w_perm.

    Per expert, with s = sigmoid(g):
      dA  = dZ W_dn[e]
      dg  = dA * w * u * s * (1 + g * (1 - s))   (d silu / dg)
      du  = dA * w * silu(g)
      dw  = sum_f dA * silu(g) * u
      dW_dn[e] = dZ^T A ;  dW_gu[e] = dH1^T X ;  dX = dH1 W_gu[e]
    Experts without tokens get dW = 0.
    """
    E = len(offsets) - 1
    rows = np.asarray(x_perm).shape[0]
    F = np.asarray(w_gu).shape[1] // 2
    H = np.asarray(w_dn).shape[1]
    w = np.ones(rows) if w_perm is None else np.asarray(w_perm, dtype=f64)
    dx = np.zeros((rows, H), dtype=f64)
    dh1_all = np.zeros((rows, 2 * F), dtype=f64)
    dw_perm = np.zeros(rows, dtype=f64)
    dw_gu = np.zeros((E, 2 * F, H), dtype=f64)
    dw_dn = np.zeros((E, H, F), dtype=f64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = _as_f64(x_perm[lo:hi])
        Wgu = _as_f64(w_gu[e])
        Wdn = _as_f64(w_dn[e])
        dZ = _as_f64(dz_perm[lo:hi])
        h1 = X @ Wgu.T
        g, u = h1[:, :F], h1[:, F:]
        we = w[lo:hi, None]
        A = we * (g * sigmoid(g)) * u
        dA = dZ @ Wdn
        dh1, dw_perm[lo:hi] = swiglu_bwd(dA, g, u, we)
        dw_dn[e] = dZ.T @ A
        dw_gu[e] = dh1.T @ X
        dx[lo:hi] = dh1 @ Wgu
        dh1_all[lo:hi] = dh1
    return {"dx_perm": dx, "dh1": dh1_all, "dw_perm": dw_perm,
            "dw_gu": dw_gu, "dw_dn": dw_dn}


def gather_rows(src: np.ndarray, src_row: np.ndarray, k: int) -> np.ndarray:
    """dst[r] = src[src_row[r] // k]  (dY -> dZ in the backward pass)."""
    return permute_rows(src, src_row, k)


def probs_grad(dw_perm: np.ndarray, row_map: np.ndarray, k: int
               ) -> np.ndarray:
    """dprobs[t, j] = dw_perm[row_map[t*k + j]]."""
    rm = np.asarray(row_map, dtype=np.int64)
    return np.asarray(dw_perm, dtype=f64)[rm].reshape(-1, k)


def layer_bwd(x, logits, w_gu, w_dn, dy, k: int, renormalize: bool = True
              ) -> Dict[str, np.ndarray]:
    """Backward of layer_fwd's y w.r.t. x, W_gu, W_dn and topk_w (routing
    indices held fixed): dZ = gather(dY); MLP backward; dx = unweighted
    combine of dX_perm; dprobs from dw_perm."""
    fwd = layer_fwd(x, logits, w_gu, w_dn, k, renormalize)
    dz = gather_rows(_as_f64(dy), fwd["src_row"], k)
    g = grouped_mlp_bwd(dz, fwd["x_perm"], w_gu, w_dn, fwd["w_perm"],
                        fwd["offsets"])
    dx = unpermute(g["dx_perm"], fwd["row_map"], k)
    dprobs = probs_grad(g["dw_perm"], fwd["row_map"], k)
    return {**fwd, "dz": dz, **g, "dx": dx, "dprobs": dprobs}


# --------------------------------------------------------------------------
# MXFP8: E4M3 elements, one E8M0 scale per 32 consecutive values
# [PG1 "Reducing memory and quantisation cost" and PG2 "2) Model size and
#  activation memory": 8-bit elements, one scale per block of 32 consecutive
#  values; PG2 "3) Quantisation overhead": 16-bit master weights quantised]
# --------------------------------------------------------------------------
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal (448 = 1.75 * 2^8)
MX_BLOCK = 32


def e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """R7 scale exponent s (int) from a block's amax >= 0 (float64).

    floor(log2 amax) comes from frexp (amax = m * 2^ex, m in [0.5, 1)), so it
    is exact; amax = 0 gives the clamp -127."""
    amax = np.asarray(amax, dtype=f64)
    _, ex = np.frexp(amax)
    s = ex.astype(np.int64) - 1 - E4M3_EMAX
    s = np.where(amax > 0, s, -127)
    return np.clip(s, -127, 127)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float64 (already scaled) -> OCP E4M3 code (uint8), round to nearest
    even, saturating at +-448, sign kept (also for zero results)."""
    v = np.asarray(v, dtype=f64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = ex.astype(np.int64) - 1                 # floor(log2 a) for a > 0
    e = np.where(a > 0, e, -7)
    e = np.maximum(e, -6)                       # below 2^-6: subnormal grid
    quantum = np.ldexp(1.0, e - 3)              # 3 mantissa bits
    q = np.rint(a / quantum).astype(np.int64)   # exact division; RNE
    # q in [0, 16]; q == 16 carries into the next binade
    carry = q >= 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    normal = q >= 8
    code = np.where(normal, ((e + 7) << 3) | (q - 8), q)
    code = np.where(a >= E4M3_MAX, 0x7E, code)  # saturation
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """OCP E4M3 code -> float64 (0x7F / 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    val = np.where(ef == 0, np.ldexp(m.astype(f64), -9),
                   np.ldexp((8 + m).astype(f64), ef - 10))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def mx_quantize_blocks(v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """v float64 [..., nb, 32] -> (codes uint8 same shape, scale u8 [..., nb]).
    R7 step by step: amax -> s -> E8M0 code s+127 -> E4M3(v * 2^-s)."""
    v = np.asarray(v, dtype=f64)
    amax = np.abs(v).max(axis=-1)
    s = e8m0_exponent(amax)
    scaled = np.ldexp(v, -s[..., None])
    codes = e4m3_encode(scaled)
    return codes, (s + 127).astype(np.uint8)


def mx_dequantize_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    s = np.asarray(scales, dtype=np.int64) - 127
    return np.ldexp(e4m3_decode(codes), s[..., None])


def mxfp8_quantize_rows(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row-wise: [R, C] (C % 32 == 0) -> codes u8 [R, C], scales u8 [R, C/32];
    blocks run along each row (the row is the GEMM's K)."""
    a = _as_f64(a)
    R, C = a.shape
    if C % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    codes, sc = mx_quantize_blocks(a.reshape(R, C // MX_BLOCK, MX_BLOCK))
    return codes.reshape(R, C), sc


def mxfp8_quantize_cols(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Column-wise: [R, C] (R % 32 == 0) -> codes u8 [C, R] (transposed so the
    blocked dimension is contiguous), scales u8 [C, R/32]."""
    return mxfp8_quantize_rows(_as_f64(a).T)


def mxfp8_quantize_segments(a: np.ndarray, seg_offsets: np.ndarray
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """Per-segment column-wise (token direction, R8): rows of ``a`` [R, C] are
    split at seg_offsets; within a segment blocks of 32 rows start at the
    segment start, the last one zero-padded.  Output codes u8 [C, Rp] and
    scales u8 [C, Rp/32], where each segment occupies ceil(n/32)*32 columns
    starting at padded offset sum_{e'<e} ceil(n_e'/32)*32."""
    a = _as_f64(a)
    C = a.shape[1]
    segs = []
    for e in range(len(seg_offsets) - 1):
        lo, hi = int(seg_offsets[e]), int(seg_offsets[e + 1])
        n = hi - lo
        npad = -(-n // MX_BLOCK) * MX_BLOCK
        blk = np.zeros((C, npad), dtype=f64)
        blk[:, :n] = a[lo:hi].T
        segs.append(blk)
    full = np.concatenate(segs, axis=1) if segs else np.zeros((C, 0))
    return mxfp8_quantize_rows(full)


def padded_offsets(offsets: np.ndarray) -> np.ndarray:
    """Offsets of the 32-padded token segments used by the segment layout."""
    n = np.diff(np.asarray(offsets, dtype=np.int64))
    p = np.zeros(len(n) + 1, dtype=np.int64)
    p[1:] = np.cumsum(-(-n // MX_BLOCK) * MX_BLOCK)
    return p


def _mx_rows_np(a):
    """quantise row-wise then dequantise (the value the MX GEMM consumes)."""
    c, s = mxfp8_quantize_rows(a)
    R, C = c.shape
    return mx_dequantize_blocks(c.reshape(R, C // 32, 32), s).reshape(R, C)


def _mx_rows(a):
    """_mx_rows_np; bf16 input (uint16 bit patterns, e.g. whole expert
    weights) goes through the C statement of the same rule in mx_fast.c,
    which is pinned bit for bit against the numpy one."""
    if np.asarray(a).dtype == np.uint16:
        from oracle import mx_fast
        return mx_fast.dequantized_rows(a)
    return _mx_rows_np(a)


def _mx_segment_cols(a, lo, hi):
    """Token-direction quantisation of rows [lo, hi) of a (one segment),
    returned dequantised in the original [n, C] orientation."""
    sub = _as_f64(a[lo:hi])
    n, C = sub.shape
    npad = -(-n // MX_BLOCK) * MX_BLOCK
    t = np.zeros((C, npad))
    t[:, :n] = sub.T
    return _mx_rows(t)[:, :n].T


def mx_gemm_rows(a, b) -> np.ndarray:
    """C = Q_K(a) Q_K(b)^T for a [M, K], b [N, K]: both operands quantised
    with blocks of 32 along their rows (the GEMM's K), then multiplied
    (float64).  The forward GEMMs: x_perm W_gu^T and A W_dn^T (R8)."""
    return _mx_rows(a) @ _mx_rows(b).T


def mx_dgrad(dy, w) -> np.ndarray:
    """dX = Q_N(dY) Q_N(W) for dY [M, N], W [N, K]: the contraction runs over
    N, so dY is quantised along its rows and W along its columns (blocks of
    32 consecutive rows of W).  dgrad of the down projection (N = H) and of
    the gate/up projection (N = 2F) (R8)."""
    return mx_gemm_rows(dy, np.asarray(w).T)


def mx_wgrad_segment(a, b, offsets, e: int) -> np.ndarray:
    """dW = Q_tok(A_e)^T Q_tok(B_e) for the rows [offsets[e], offsets[e+1])
    of a [R, M] and b [R, N]: the contraction runs over the expert's tokens,
    so both are quantised along tokens with blocks restarting at the
    segment's first row, the last block zero-padded (R8).  [M, N] float64;
    zeros for an expert without tokens."""
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    a = np.asarray(a)
    b = np.asarray(b)
    if hi == lo:
        return np.zeros((a.shape[1], b.shape[1]), dtype=f64)
    n = hi - lo
    return _mx_segment_cols(a, lo, hi).T @ _mx_segment_cols(b, lo, hi)


def swiglu_bwd(da, g, u, w) -> Tuple[np.ndarray, np.ndarray]:
    """SwiGLU backward of a = w * silu(g) * u (R5, R6), with s = sigmoid(g):
      dg = dA * w * u * s * (1 + g * (1 - s))      (d silu / dg)
      du = dA * w * silu(g)
      dw = sum_f dA * silu(g) * u
    Returns (dH1 = [dg, du] along columns, dw per row)."""
    s = sigmoid(g)
    sg = g * s
    dg = da * w * u * (s * (1.0 + g * (1.0 - s)))
    du = da * w * sg
    return np.concatenate([dg, du], axis=1), (da * sg * u).sum(axis=1)


def grouped_mlp_fwd_mxfp8(x_perm, w_gu, w_dn, w_perm, offsets,
                          keep: bool = False) -> Dict[str, np.ndarray]:
    """R8 forward: x_perm and W_gu quantised along H, the SwiGLU*w output A
    and W_dn along F; both GEMMs on the dequantised values (float64)."""
    E = len(offsets) - 1
    rows = np.asarray(x_perm).shape[0]
    F = np.asarray(w_gu).shape[1] // 2
    H = np.asarray(w_dn).shape[1]
    w = np.ones(rows) if w_perm is None else np.asarray(w_perm, dtype=f64)
    z = np.zeros((rows, H), dtype=f64)
    a_all = np.zeros((rows, F), dtype=f64) if keep else None
    h1_all = np.zeros((rows, 2 * F), dtype=f64) if keep else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        h1 = mx_gemm_rows(x_perm[lo:hi], w_gu[e])
        g, u = h1[:, :F], h1[:, F:]
        a = w[lo:hi, None] * silu(g) * u
        z[lo:hi] = mx_gemm_rows(a, w_dn[e])
        if keep:
            a_all[lo:hi] = a
            h1_all[lo:hi] = h1
    out = {"z": z}
    if keep:
        out["a"] = a_all
        out["h1"] = h1_all
    return out


def grouped_mlp_bwd_mxfp8(dz_perm, x_perm, w_gu, w_dn, w_perm, offsets
                          ) -> Dict[str, np.ndarray]:
    """R8 backward: every GEMM operand quantised along that GEMM's K.
      dgrad2  dA = Q_H(dZ) Q_H(W_dn)            (W_dn blocks along H: col-wise)
      wgrad2  dW_dn = Q_tok(dZ)^T Q_tok(A)
      dgrad1  dX = Q_2F(dH1) Q_2F(W_gu)         (W_gu blocks along 2F)
      wgrad1  dW_gu = Q_tok(dH1)^T Q_tok(X)
    The forward intermediates (h1, A) are recomputed as in the MXFP8 forward;
    SwiGLU backward and dw in float64."""
    E = len(offsets) - 1
    rows = np.asarray(x_perm).shape[0]
    F = np.asarray(w_gu).shape[1] // 2
    H = np.asarray(w_dn).shape[1]
    w = np.ones(rows) if w_perm is None else np.asarray(w_perm, dtype=f64)
    dx = np.zeros((rows, H))
    dw_perm = np.zeros(rows)
    dw_gu = np.zeros((E, 2 * F, H))
    dw_dn = np.zeros((E, H, F))
    X = _as_f64(x_perm)
    dZ = _as_f64(dz_perm)
    A = np.zeros((rows, F))
    dh1 = np.zeros((rows, 2 * F))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        h1 = mx_gemm_rows(X[lo:hi], w_gu[e])
        g, u = h1[:, :F], h1[:, F:]
        we = w[lo:hi, None]
        A[lo:hi] = we * silu(g) * u
        dA = mx_dgrad(dZ[lo:hi], w_dn[e])
        dh1[lo:hi], dw_perm[lo:hi] = swiglu_bwd(dA, g, u, we)
        dx[lo:hi] = mx_dgrad(dh1[lo:hi], w_gu[e])
    for e in range(E):
        dw_dn[e] = mx_wgrad_segment(dZ, A, offsets, e)
        dw_gu[e] = mx_wgrad_segment(dh1, X, offsets, e)
    return {"dx_perm": dx, "dw_perm": dw_perm, "dw_gu": dw_gu,
            "dw_dn": dw_dn}


# --------------------------------------------------------------------------
# Tensor-scaled FP8  [PG1 "Reducing memory and quantisation cost" and PG2
# "3) Quantisation overhead in low-precision training": 8-bit formats with
# scales, from 16-bit masters]; reading R11
# --------------------------------------------------------------------------
def fp8_tensor_scale(amax) -> np.float32:
    """s = amax / 448 in float32 (1 for amax == 0)."""
    a = np.float32(amax)
    return np.float32(a / np.float32(E4M3_MAX)) if a > 0 else np.float32(1.0)


def fp8_tensor_quantize(v) -> Tuple[np.ndarray, np.float32]:
    """One tensor (bf16 bit patterns or floats exactly representable in
    float32) -> (E4M3 codes, float32 scale)."""
    vf = _as_f64(v).astype(np.float32)
    s = fp8_tensor_scale(np.abs(vf).max() if vf.size else 0.0)
    q = (vf / s).astype(np.float32)              # IEEE float32 division
    return e4m3_encode(q.astype(f64)), s


def fp8_tensor_dequantize(codes, s) -> np.ndarray:
    return e4m3_decode(codes) * f64(s)


def grouped_mlp_fwd_fp8_tensor(x_perm, w_gu, w_dn, w_perm, offsets
                               ) -> Dict[str, np.ndarray]:
    """R11 forward: x_perm, each W_gu[e] and W_dn[e] quantised per tensor;
    h1 = Xq Wq^T (float64 on the dequantised values); A = w * silu(g) * u
    rounded to bf16, quantised per tensor over all rows; z = Aq Wdnq^T.
    Returns z, h1, A (rounded to bf16; all float64) and A's scale."""
    E = len(offsets) - 1
    rows = np.asarray(x_perm).shape[0]
    F = np.asarray(w_gu).shape[1] // 2
    H = np.asarray(w_dn).shape[1]
    w = np.ones(rows) if w_perm is None else np.asarray(w_perm, dtype=f64)
    xc, xs = fp8_tensor_quantize(x_perm)
    X = fp8_tensor_dequantize(xc, xs)
    a = np.zeros((rows, F), dtype=f64)
    h1_all = np.zeros((rows, 2 * F), dtype=f64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wc, ws = fp8_tensor_quantize(w_gu[e])
        h1 = X[lo:hi] @ fp8_tensor_dequantize(wc, ws).T
        g, u = h1[:, :F], h1[:, F:]
        a[lo:hi] = w[lo:hi, None] * silu(g) * u
        h1_all[lo:hi] = h1
    a16 = _as_f64(_bf16_round_bits(a))
    ac, as_ = fp8_tensor_quantize(a16)
    A = fp8_tensor_dequantize(ac, as_)
    z = np.zeros((rows, H), dtype=f64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        wc, ws = fp8_tensor_quantize(w_dn[e])
        z[lo:hi] = A[lo:hi] @ fp8_tensor_dequantize(wc, ws).T
    return {"z": z, "a": a16, "a_scale": as_, "h1": h1_all}


def _bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16): to float32, then round to
    nearest even on the upper 16 bits."""
    b = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


# --------------------------------------------------------------------------
# Router projection and router backward  [PG3 practical implications: Top-k
# routing; PG4 "Background": tokens are routed across many experts]
# --------------------------------------------------------------------------
def router_logits(x, w_r, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """x bf16 [T, H], w_r bf16 [E, H] (bit patterns or floats), bias [E] or
    None -> logits float32 [T, E].  Reading R9: float64, one term at a time
    in ascending h (ufunc accumulate adds left to right), bias last, one
    rounding to float32."""
    X = _as_f64(x)
    W = _as_f64(w_r)
    T = X.shape[0]
    E = W.shape[0]
    out = np.empty((T, E), dtype=f64)
    for t in range(T):
        prod = W * X[t][None, :]                 # exact products
        out[t] = np.add.accumulate(prod, axis=1)[:, -1]
    if bias is not None:
        out = out + np.asarray(bias, dtype=f64)[None, :]
    return out.astype(np.float32)


def router_bwd(logits: np.ndarray, topk_idx: np.ndarray, dtopk_w: np.ndarray,
               renormalize: bool = True) -> np.ndarray:
    """dlogits float64 [T, E] from the gradient of the routing weights
    dtopk_w [T, k] (reading R10).  With w the forward's softmax (over the
    chosen set S, or p over all E):
      renormalize:  dl_i = w_i (dw_i - sum_{j in S} w_j dw_j) for i in S, else 0
      otherwise:    dl_e = p_e (g_e - sum_{j in S} p_j dw_j), g = dw on S, 0 off S
    """
    lv = np.asarray(logits, dtype=np.float32).astype(f64) + 0.0
    idx = np.asarray(topk_idx).astype(np.int64)
    dw = np.asarray(dtopk_w, dtype=f64)
    T, E = lv.shape
    dl = np.zeros((T, E), dtype=f64)
    for t in range(T):
        S = idx[t]
        ex = np.exp(lv[t] - lv[t].max())
        if renormalize:
            w = ex[S] / ex[S].sum()
            dl[t, S] = w * (dw[t] - (w * dw[t]).sum())
        else:
            p = ex / ex.sum()
            g = np.zeros(E, dtype=f64)
            g[S] = dw[t]
            dl[t] = p * (g - (p * g).sum())
    return dl


def router_weight_grads(dlogits: np.ndarray, x, w_r
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """(dW_r [E, H], dx [T, H]) = (dlogits^T x, dlogits W_r), float64."""
    dl = np.asarray(dlogits, dtype=f64)
    return dl.T @ _as_f64(x), dl @ _as_f64(w_r)


# --------------------------------------------------------------------------
# Error metric used by the parity tests
# --------------------------------------------------------------------------
def rel_err(a: np.ndarray, b: np.ndarray) -> float:
    """Normwise ||a - b||_2 / ||b||_2 (0 when both are zero)."""
    a = np.asarray(a, dtype=f64)
    b = np.asarray(b, dtype=f64)
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    if nb == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return float(d / nb)
