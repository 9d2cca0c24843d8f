"""Seeded synthetic inputs for the Gated DeltaNet (GDN) layer.

This module only draws random numbers and stores them in the element types
the kernels read (bf16 bit patterns as uint16, fp32, int32 offsets).  It holds
none of the layer's arithmetic: the recurrence lives in the HIP kernels and,
separately, in the fp64 oracle.  Both sides receive the same arrays from here.

The pages give no input distributions; these are the synthetic benchmark
recipe of this library (the pages fix only the workload's scale: a native
context of 262,144 tokens, studioglobal.ai, "Die wichtigsten technischen
Daten"):

* q, k ~ N(0, 1), L2-normalised over the head dimension in fp32 for each
  (token, head), then rounded to the I/O type;
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1)), g = -softplus(N(0, 1)) (so alpha = exp(g) < 1), fp32;
* non-zero initial states ~ N(0, 0.1^2) (variance 0.01), fp32.

Draw order is fixed (seeded ``numpy.random.default_rng``): sequence lengths
first (packed configuration), then q, k, v, beta logits, g logits, initial
state; for decode the state first, then per step q, k, v, beta, g.  Large
tensors are drawn in fixed slabs of tokens so that memory stays bounded; the
generator stream is sequential, so the slab size does not change the values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Tokens per slab when drawing large tensors (fixed: part of the recipe).
_SLAB_TOKENS = 8192


# --------------------------------------------------------------------------
# element-type helpers (storage conversions only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even); returns the uint16 bits.

    Inputs are finite by construction (no NaN handling needed here).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored inputs ("bf16" bits or "f32") to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclass
class Workload:
    """Shapes of one GDN call (or of a decode run)."""
    name: str
    dtype: str                 # "f32" or "bf16" (q/k/v/out element type)
    num_qk_heads: int
    num_v_heads: int
    head_dim_k: int
    head_dim_v: int
    seqlens: list              # per-sequence token counts (prefill)
    init_state: str = "zero"   # "zero" or "normal"
    decode_steps: int = 0      # >0: decode workload (each sequence advances 1 token per step)
    seed: int = 0
    packed: bool = False       # True: pass cu_seqlens (varlen packing)
    raw: bool = False          # True: q, k unnormalised (per-token scales), g and beta hold logits

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))


def _workload(cfg: str) -> Workload:
    if cfg == "tiny_f32":
        return Workload("tiny_f32", "f32", 2, 2, 64, 64, [256])
    if cfg == "prefill_4k":
        return Workload("prefill_4k", "bf16", 16, 16, 128, 128, [4096])
    if cfg == "varlen_8x":
        # lengths are drawn from the seed in make_inputs (first draw)
        return Workload("varlen_8x", "bf16", 16, 32, 128, 128, [], init_state="normal", packed=True)
    if cfg == "prefill_256k":
        return Workload("prefill_256k", "bf16", 16, 16, 128, 128, [262144])
    if cfg == "draft_256x4":
        # multi-token decode: 256 sequences advance 4 tokens each in one call
        return Workload("draft_256x4", "bf16", 16, 16, 128, 128, [4] * 256, init_state="normal")
    if cfg == "decode_256x64":
        return Workload("decode_256x64", "bf16", 16, 16, 128, 128, [1] * 256,
                        init_state="normal", decode_steps=64)
    raise KeyError(cfg)


CONFIGS = ("tiny_f32", "prefill_4k", "varlen_8x", "prefill_256k", "decode_256x64")


@dataclass
class Inputs:
    """Host arrays for one workload, in the element types the kernels read."""
    wl: Workload
    q: np.ndarray = None          # [tokens, Hqk, dk] (uint16 bf16 bits or float32)
    k: np.ndarray = None
    v: np.ndarray = None          # [tokens, Hv, dv]
    g: np.ndarray = None          # [tokens, Hv] float32, log alpha (<= 0)
    beta: np.ndarray = None       # [tokens, Hv] float32 in (0, 1)
    init_state: Optional[np.ndarray] = None   # [N, Hv, dv, dk] float32 or None (zero)
    cu_seqlens: Optional[np.ndarray] = None   # int32 [N+1] or None
    steps: list = field(default_factory=list)  # decode: per step dict(q,k,v,g,beta)


def _normal(rng, shape, dtype=np.float32):
    return rng.standard_normal(shape, dtype=dtype)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _draw_qk(rng, T, H, d, dtype):
    out = np.empty((T, H, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for t0 in range(0, T, _SLAB_TOKENS):
        t1 = min(T, t0 + _SLAB_TOKENS)
        out[t0:t1] = _store(_unit_rows(_normal(rng, (t1 - t0, H, d))), dtype)
    return out


def _draw_v(rng, T, H, d, dtype):
    out = np.empty((T, H, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for t0 in range(0, T, _SLAB_TOKENS):
        t1 = min(T, t0 + _SLAB_TOKENS)
        out[t0:t1] = _store(_normal(rng, (t1 - t0, H, d)), dtype)
    return out


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _neg_softplus(x):
    x = x.astype(np.float64)
    return (-(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))).astype(np.float32)


def make_inputs(cfg, seed: int = 0, seqlens=None) -> Inputs:
    """Draw the inputs of a named workload (or of a custom ``Workload``).

    ``seqlens`` overrides the per-sequence lengths of a prefill workload (used
    by tests that need a smaller instance with the same distributions).
    """
    wl = _workload(cfg) if isinstance(cfg, str) else cfg
    wl.seed = seed
    rng = np.random.default_rng(seed)
    if wl.packed and not wl.seqlens and seqlens is None:
        wl.seqlens = [int(x) for x in rng.integers(1024, 16384, endpoint=True, size=8)]
    if seqlens is not None:
        wl.seqlens = [int(x) for x in seqlens]
    Hqk, Hv, dk, dv, dt = wl.num_qk_heads, wl.num_v_heads, wl.head_dim_k, wl.head_dim_v, wl.dtype
    inp = Inputs(wl)
    if wl.decode_steps > 0:
        N = wl.num_seqs
        inp.init_state = (0.1 * _normal(rng, (N, Hv, dv, dk))).astype(np.float32)
        for _ in range(wl.decode_steps):
            q = _draw_qk(rng, N, Hqk, dk, dt)
            k = _draw_qk(rng, N, Hqk, dk, dt)
            v = _draw_v(rng, N, Hv, dv, dt)
            beta = _sigmoid(_normal(rng, (N, Hv)))
            g = _neg_softplus(_normal(rng, (N, Hv)))
            inp.steps.append(dict(q=q, k=k, v=v, g=g, beta=beta))
        return inp
    T = wl.total_tokens
    if wl.raw:
        # raw projections: N(0,1) rows times a per-(token, head) scale in [0.1, 10), logits N(0,1)
        def raw_rows(H, d):
            x = _normal(rng, (T, H, d)) * np.exp(rng.uniform(np.log(0.1), np.log(10.0), (T, H, 1))).astype(np.float32)
            return _store(x.astype(np.float32), dt)
        inp.q = raw_rows(Hqk, dk)
        inp.k = raw_rows(Hqk, dk)
        inp.v = _draw_v(rng, T, Hv, dv, dt)
        inp.beta = _normal(rng, (T, Hv))
        inp.g = _normal(rng, (T, Hv))
        if wl.init_state == "normal":
            inp.init_state = (0.1 * _normal(rng, (wl.num_seqs, Hv, dv, dk))).astype(np.float32)
        if wl.packed or wl.num_seqs > 1:
            inp.cu_seqlens = np.concatenate([[0], np.cumsum(wl.seqlens)]).astype(np.int32)
        return inp
    inp.q = _draw_qk(rng, T, Hqk, dk, dt)
    inp.k = _draw_qk(rng, T, Hqk, dk, dt)
    inp.v = _draw_v(rng, T, Hv, dv, dt)
    inp.beta = _sigmoid(_normal(rng, (T, Hv)))
    inp.g = _neg_softplus(_normal(rng, (T, Hv)))
    if wl.init_state == "normal":
        inp.init_state = (0.1 * _normal(rng, (wl.num_seqs, Hv, dv, dk))).astype(np.float32)
    if wl.packed or wl.num_seqs > 1:
        inp.cu_seqlens = np.concatenate([[0], np.cumsum(wl.seqlens)]).astype(np.int32)
    return inp


def custom(dtype="bf16", Hqk=2, Hv=2, dk=64, dv=64, seqlens=(100,), init_state="zero",
           decode_steps=0, name="custom", raw=False) -> Workload:
    """A workload of arbitrary (small) shape with the standard distributions
    (raw=True: the raw projections the *_raw entry points take)."""
    return Workload(name, dtype, Hqk, Hv, dk, dv, list(seqlens), init_state=init_state,
                    decode_steps=decode_steps, packed=len(seqlens) > 1, raw=raw)
