"""Seeded synthetic inputs for the gated delta-rule prefill and decode workloads.

This module is shared by the HIP path's tests and bench and by the CPU oracle's
tests.  It holds no arithmetic of the method itself: it only draws random
tensors, normalises q/k per token (the workload recipe asks for unit-norm keys
and queries), maps logits to beta = sigmoid(x) and g = log(alpha) =
-softplus(x), and rounds to the storage precision.  The library under test
receives these arrays as its inputs; it never normalises or applies gates
itself.

Shapes follow the packed layout of the C-ABI: q, k are [T_tot, Hk, Dk];
v is [T_tot, Hv, Dv]; g and beta are [T_tot, Hv]; states are
[N, Hv, Dv, Dk] (value index, then key index); cu_seqlens is [N+1] int32.
With a per-key-channel gate (the KDA variant) g is [T_tot, Hv, Dk], drawn from the
same distribution element by element.

Every array is numpy.  bf16 and fp16 values are carried as float32 arrays whose
values are exactly representable in the storage type (round-to-nearest-even from
float32), so an exact upcast to fp64 gives the oracle the very values the GPU
reads.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Seed of workload i is SEED_BASE + i.
SEED_BASE = 20260000


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16 expects finite values")
    # finite floats: u + 0x8000 stays below 2^32, so uint32 arithmetic cannot wrap
    bias = (u >> 16) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    u += bias
    u &= np.uint32(0xFFFF0000)
    return x


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest IEEE fp16 (ties to even); return float32."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) >= 65520.0):
        raise ValueError("round_to_f16 expects finite values inside the fp16 range")
    return x.astype(np.float16).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _l2_normalize(x: np.ndarray) -> np.ndarray:
    # per (token, head) vector, computed in float32
    x = np.asarray(x, dtype=np.float32)
    n = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float32))[..., None]
    x /= np.maximum(n, np.float32(1e-12))
    return x


def _sigmoid64(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def _softplus64(x: np.ndarray) -> np.ndarray:
    # log(1 + e^x) in a form that does not overflow for large x
    x = x.astype(np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


@dataclasses.dataclass
class GDNInputs:
    """One synthetic workload.  Arrays are float32 (exact in the storage type io)."""

    name: str
    io: str                      # 'bf16', 'f16' or 'f32': storage type of q, k, v, o
    q: np.ndarray                # [T_tot, Hk, Dk]
    k: np.ndarray                # [T_tot, Hk, Dk]
    v: np.ndarray                # [T_tot, Hv, Dv]
    g: np.ndarray                # [T_tot, Hv] (or [T_tot, Hv, Dk]) float32, log of the decay
    beta: np.ndarray             # [T_tot, Hv] float32
    cu_seqlens: np.ndarray       # [N+1] int32
    initial_state: Optional[np.ndarray]  # [N, Hv, Dv, Dk] float32 or None
    decode: Optional[dict] = None  # per-step decode inputs (q, k, v, g, beta lists)

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def T_tot(self) -> int:
        return int(self.q.shape[0])

    @property
    def Hk(self) -> int:
        return int(self.q.shape[1])

    @property
    def Hv(self) -> int:
        return int(self.v.shape[1])

    @property
    def Dk(self) -> int:
        return int(self.q.shape[2])

    @property
    def Dv(self) -> int:
        return int(self.v.shape[2])

    @property
    def per_channel(self) -> bool:
        return self.g.ndim == 3

    def seq_lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))


def draw_tokens(rng: np.random.Generator, T: int, Hk: int, Hv: int, Dk: int, Dv: int,
                io: str, g_shift: float = 0.0, per_channel: bool = False, raw: bool = False):
    """Draw q, k, v, beta, g for T tokens in the fixed order q, k, v, beta-logits, g-logits
    (g-logits [T, Hv, Dk] for a per-key-channel gate).  raw: return the draws as a
    linear-attention layer's projections would hand them over -- q, k not normalised,
    beta and g as their logits (g-logits plus g_shift) -- for the fused prologue."""
    q = rng.standard_normal((T, Hk, Dk), dtype=np.float32)
    k = rng.standard_normal((T, Hk, Dk), dtype=np.float32)
    v = rng.standard_normal((T, Hv, Dv), dtype=np.float32)
    beta_logit = rng.standard_normal((T, Hv), dtype=np.float32)
    g_logit = rng.standard_normal((T, Hv, Dk) if per_channel else (T, Hv), dtype=np.float32)
    if raw:
        beta = beta_logit
        g = (g_logit.astype(np.float64) + g_shift).astype(np.float32)
    else:
        q = _l2_normalize(q)
        k = _l2_normalize(k)
        beta = _sigmoid64(beta_logit).astype(np.float32)
        g = (-_softplus64(g_logit.astype(np.float64) + g_shift)).astype(np.float32)
    if io == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif io == "f16":
        q, k, v = round_to_f16(q), round_to_f16(k), round_to_f16(v)
    elif io != "f32":
        raise ValueError(f"unknown io type {io!r}")
    return q, k, v, g, beta


def make_custom(seed: int, lengths, Hk: int, Hv: int, Dk: int = 128, Dv: int = 128,
                io: str = "bf16", g_shift: float = 0.0, init_std: Optional[float] = None,
                name: str = "custom", per_channel: bool = False, raw: bool = False) -> GDNInputs:
    """Packed batch of sequences with the given lengths (any may be 0); raw as in
    draw_tokens."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(list(lengths), dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q, k, v, g, beta = draw_tokens(rng, T, Hk, Hv, Dk, Dv, io, g_shift, per_channel, raw)
    s0 = None
    if init_std is not None:
        s0 = (rng.standard_normal((len(lengths), Hv, Dv, Dk), dtype=np.float32)
              * np.float32(init_std)).astype(np.float32)
    return GDNInputs(name, io, q, k, v, g, beta, cu, s0)


def head_shard(x: GDNInputs, gpus: int) -> GDNInputs:
    """One GPU's share of x when its heads are split over `gpus` GPUs (tensor parallel over
    heads): key heads [0, Hk / gpus) and the value heads that read them, renumbered so that
    value head h' still reads key head h' % (Hk / gpus).  The decode steps are dropped."""
    if gpus == 1:
        return x
    if x.Hk % gpus:
        raise ValueError(f"Hk={x.Hk} heads do not split over {gpus} GPUs")
    hk = x.Hk // gpus
    vheads = [j + x.Hk * m for m in range(x.Hv // x.Hk) for j in range(hk)]
    take = lambda a: None if a is None else np.ascontiguousarray(a[:, vheads])  # noqa: E731
    s0 = None if x.initial_state is None else np.ascontiguousarray(x.initial_state[:, vheads])
    return GDNInputs(f"{x.name}_shard{gpus}", x.io, np.ascontiguousarray(x.q[:, :hk]),
                     np.ascontiguousarray(x.k[:, :hk]), take(x.v), take(x.g), take(x.beta),
                     x.cu_seqlens, s0)


# The five workloads.  Index i uses seed SEED_BASE + i.
WORKLOADS = {
    0: dict(name="tiny_f32_H1_T256", desc="B=1, H=1, T=256, d=128, fp32 I/O, zero initial state"),
    1: dict(name="prefill_bf16_H16_T4096", desc="B=1, H=16, T=4096, d=128, bf16 q/k/v/o, fp32 g/beta/state"),
    2: dict(name="gqa_bf16_Hv32_Hk16_T16384",
            desc="B=1, Hv=32 value heads over Hk=16 key heads (hv % Hk), T=16384, g=-softplus(N(0,1)+2)"),
    3: dict(name="varlen8_bf16_H16_L512-8192",
            desc="8 packed sequences, lengths U[512, 8192], H=16, initial states N(0, 0.02^2)"),
    4: dict(name="long_bf16_H32_T65536_decode256",
            desc="B=1, H=32, T=65536, then 256 single-token decode steps"),
}


def make_workload(i: int, decode_steps: Optional[int] = None, io: Optional[str] = None,
                  per_channel: bool = False, raw: bool = False) -> GDNInputs:
    """Build workload i (0..4) from its seed.  Draw order is fixed per workload.

    io overrides the storage type of q, k, v, o (default: the workload's own, fp32 for
    workload 0 and bf16 for the rest); the draws are the same, only the rounding
    differs, and the name then carries the new type.  per_channel draws one gate per
    key channel (the KDA variant; g-logits [T, Hv, Dk] in place of [T, Hv], so the later
    draws differ too) and prefixes the name with "kda_".  raw returns the draws before
    the input prologue (as draw_tokens) and prefixes the name with "raw_"."""
    rng = np.random.default_rng(SEED_BASE + i)
    own = "f32" if i == 0 else "bf16"
    name = WORKLOADS[i]["name"]
    if io is not None and io != own:
        name = name.replace(own, io)
    if per_channel:
        name = "kda_" + name
    if raw:
        name = "raw_" + name
    io = io or own
    pc = per_channel
    if raw:
        def draw_tokens(*args, **kw):   # noqa: E306 -- the same draws, before the prologue
            return _draw_tokens(*args, raw=True, **kw)
    else:
        draw_tokens = _draw_tokens
    D = 128
    if i == 0:
        q, k, v, g, beta = draw_tokens(rng, 256, 1, 1, D, D, io, per_channel=pc)
        return GDNInputs(name, io, q, k, v, g, beta, np.array([0, 256], np.int32), None)
    if i == 1:
        q, k, v, g, beta = draw_tokens(rng, 4096, 16, 16, D, D, io, per_channel=pc)
        return GDNInputs(name, io, q, k, v, g, beta, np.array([0, 4096], np.int32), None)
    if i == 2:
        q, k, v, g, beta = draw_tokens(rng, 16384, 16, 32, D, D, io, g_shift=2.0, per_channel=pc)
        return GDNInputs(name, io, q, k, v, g, beta, np.array([0, 16384], np.int32), None)
    if i == 3:
        # lengths are drawn first because they fix the packed token count
        lengths = rng.integers(512, 8192, size=8, endpoint=True)
        cu = np.zeros(9, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        T = int(cu[-1])
        q, k, v, g, beta = draw_tokens(rng, T, 16, 16, D, D, io, per_channel=pc)
        s0 = (rng.standard_normal((8, 16, D, D), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
        return GDNInputs(name, io, q, k, v, g, beta, cu, s0)
    if i == 4:
        q, k, v, g, beta = draw_tokens(rng, 65536, 32, 32, D, D, io, per_channel=pc)
        steps = 256 if decode_steps is None else decode_steps
        dq, dk_, dv, dg, db = draw_tokens(rng, steps, 32, 32, D, D, io, per_channel=pc)
        dec = dict(q=dq, k=dk_, v=dv, g=dg, beta=db, steps=steps)
        return GDNInputs(name, io, q, k, v, g, beta, np.array([0, 65536], np.int32), None, dec)
    raise KeyError(i)


_draw_tokens = draw_tokens


def select_heads(x: GDNInputs, heads) -> GDNInputs:
    """Restrict a workload to a subset of value heads (with their key heads h % Hk).

    Used to compute sampled oracle outputs at full sequence length.  The key heads of
    the subset are re-indexed so that value head j of the subset uses key head j of the
    subset; the GQA mapping is therefore resolved here by gathering, not by arithmetic.
    """
    heads = list(heads)
    kh = [h % x.Hk for h in heads]
    s0 = None if x.initial_state is None else np.ascontiguousarray(x.initial_state[:, heads])
    return GDNInputs(x.name + f"[heads={heads}]", x.io,
                     np.ascontiguousarray(x.q[:, kh]), np.ascontiguousarray(x.k[:, kh]),
                     np.ascontiguousarray(x.v[:, heads]), np.ascontiguousarray(x.g[:, heads]),
                     np.ascontiguousarray(x.beta[:, heads]), x.cu_seqlens.copy(), s0)
