"""Seeded synthetic inputs for the MoE expert-MLP path.

This module is the one piece shared by the CPU oracle and the GPU path: it
draws random tensors and nothing else.  It holds none of the method's
arithmetic (no routing, no permutation, no MLP, no quantisation).  The router
logits are an *input* of the path (the router projection itself is outside
the hot path), so they are synthesised here once, in float64, and rounded to
float32; both sides then read that one tensor.

Recipe (every config, seed 0 unless stated):
  * ``numpy.random.SeedSequence(seed).spawn(6)`` gives six independent PCG64
    streams, used in the order [x, W_r, rank, W_gu, W_dn, dY].
  * x ~ N(0, 1) float32, rounded once to bfloat16 (round-to-nearest-even).
  * W_r (router gate, [E, H]), W_gu ([E, 2F, H], gate rows 0..F-1, up rows
    F..2F-1) and W_dn ([E, H, F]) ~ 0.02 * N(0, 1), rounded to bfloat16.
  * Zipf-skewed configs add a per-expert bias -s*ln(rank_e) with s = 1.2 and
    rank a seeded permutation of 1..E, so the softmax prior over experts is
    proportional to rank^-s: ragged loads with some experts left empty.
  * logits = x @ W_r^T + bias evaluated in float64, rounded to float32.
  * dY (upstream gradient) ~ N(0, 1), rounded to bfloat16.

bfloat16 tensors are carried as ``uint16`` bit patterns in numpy.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "MoEConfig", "CONFIGS", "generate", "bf16_bits", "bf16_to_f32",
    "bf16_to_f64",
]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    H: int          # hidden size
    F: int          # expert FFN size
    E: int          # experts
    k: int          # experts per token
    mode: str       # "bf16", "mxfp8" or "fp8t" (tensor-scaled E4M3)
    backward: bool  # the workload includes the backward pass
    zipf: float     # Zipf exponent of the per-expert router bias (0 = none)
    renormalize: bool = True
    description: str = ""

    @property
    def rows(self) -> int:
        return self.T * self.k

    def fwd_flop(self) -> float:
        """Algorithmic forward flop: 2*rows*H*2F + 2*rows*F*H."""
        return 6.0 * self.rows * self.H * self.F

    def bwd_flop(self) -> float:
        """Algorithmic backward flop: dgrad + wgrad of both projections."""
        return 12.0 * self.rows * self.H * self.F


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig(
        "tiny", T=256, H=128, F=256, E=8, k=2, mode="bf16", backward=False,
        zipf=0.0,
        description="tiny MoE layer fwd, top-2 softmax routing, seed 0"),
    "mixtral": MoEConfig(
        "mixtral", T=8192, H=4096, F=14336, E=8, k=2, mode="bf16",
        backward=False, zipf=0.0,
        description="Mixtral-8x7B-shaped layer fwd, bf16, near-balanced"),
    "qwen3": MoEConfig(
        "qwen3", T=16384, H=2048, F=768, E=128, k=8, mode="bf16",
        backward=False, zipf=1.2,
        description="Qwen3-30B-A3B-shaped layer fwd, bf16, Zipf-skewed"),
    "mixtral_mxfp8": MoEConfig(
        "mixtral_mxfp8", T=8192, H=4096, F=14336, E=8, k=2, mode="mxfp8",
        backward=False, zipf=0.0,
        description="Mixtral-8x7B-shaped layer fwd, MXFP8 E4M3 + E8M0/32"),
    "mixtral_mxfp8_bwd": MoEConfig(
        "mixtral_mxfp8_bwd", T=8192, H=4096, F=14336, E=8, k=2, mode="mxfp8",
        backward=True, zipf=0.0,
        description="Mixtral-8x7B-shaped layer fwd + bwd, MXFP8, dY ~ N(0,1)"),
    "mixtral_fp8t": MoEConfig(
        "mixtral_fp8t", T=8192, H=4096, F=14336, E=8, k=2, mode="fp8t",
        backward=False, zipf=0.0,
        description="Mixtral-8x7B-shaped layer fwd, E4M3 with one float32 "
                    "scale per tensor"),
    "qwen3_long": MoEConfig(
        "qwen3_long", T=32768, H=2048, F=768, E=128, k=8, mode="bf16",
        backward=True, zipf=1.2,
        description="one 32768-token sequence, Qwen3 shape, fwd + bwd"),
}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    import torch  # CPU conversion only; multithreaded and RNE
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def _normal_bf16(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    """Draw N(0, scale^2) as float32 in chunks (same sequence as one draw)."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1)
    for i in range(shape[0]):
        v = rng.standard_normal(flat.shape[1], dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        flat[i] = bf16_bits(v)
    return out


def generate(T: int, H: int, F: int, E: int, k: int, *, zipf: float = 0.0,
             seed: int = 0, want=("x", "logits", "w_gu", "w_dn"),
             ) -> Dict[str, Optional[np.ndarray]]:
    """Draw one layer's inputs.  Keys (only those in ``want`` are drawn,
    streams are still consumed in order so each tensor is independent of
    which others were requested):

      x       uint16 bf16 [T, H]
      x_f32   float32 [T, H]  (the unrounded draw, for information)
      w_r     uint16 bf16 [E, H]
      bias    float64 [E]
      logits  float32 [T, E]
      w_gu    uint16 bf16 [E, 2F, H]
      w_dn    uint16 bf16 [E, H, F]
      dy      uint16 bf16 [T, H]
    """
    streams = np.random.SeedSequence(seed).spawn(6)
    rng = [np.random.Generator(np.random.PCG64(s)) for s in streams]
    out: Dict[str, Optional[np.ndarray]] = {}
    need_x = "x" in want or "logits" in want or "x_f32" in want
    if need_x:
        xf = rng[0].standard_normal((T, H), dtype=np.float32)
        out["x"] = bf16_bits(xf)
        if "x_f32" in want:
            out["x_f32"] = xf
    if "logits" in want or "w_r" in want:
        w_r = _normal_bf16(rng[1], (E, H), 0.02)
        out["w_r"] = w_r
        bias = np.zeros(E, dtype=np.float64)
        if zipf > 0.0:
            rank = rng[2].permutation(E).astype(np.float64) + 1.0
            bias = -zipf * np.log(rank)
        out["bias"] = bias
        if "logits" in want:
            lg = bf16_to_f64(out["x"]) @ bf16_to_f64(w_r).T + bias[None, :]
            out["logits"] = lg.astype(np.float32)
    if "w_gu" in want:
        out["w_gu"] = _normal_bf16(rng[3], (E, 2 * F, H), 0.02)
    if "w_dn" in want:
        out["w_dn"] = _normal_bf16(rng[4], (E, H, F), 0.02)
    if "dy" in want:
        out["dy"] = _normal_bf16(rng[5], (T, H), 1.0)
    return out


def generate_config(cfg: MoEConfig, seed: int = 0, want=None):
    if want is None:
        want = ("x", "logits", "w_gu", "w_dn") + (("dy",) if cfg.backward else ())
    return generate(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, zipf=cfg.zipf,
                    seed=seed, want=want)
