"""Seeded synthetic inputs for causal grouped-query attention.

This module is shared by the CPU oracle's tests and the HIP path's tests and bench.
It holds none of the attention arithmetic: it only draws normal samples and rounds
them to bfloat16 bit patterns.

Workloads (sizes after the page "A transformer in PTX", section "The model", whose dev
preset maps six 64-wide query heads onto two key/value heads, plus larger shapes):
every input is drawn N(0, 1) in float32 with numpy's PCG64 ``default_rng(seed)`` in
the order Q, K, V, dO, optionally multiplied by a constant (2 for Q and K in the
"peaky" workload, exact in bf16), then rounded to bf16 by round-to-nearest-even.
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    qk_mult: float = 1.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        # 1/sqrt(d), rounded to float32: the value both sides receive.
        return float(np.float32(1.0 / np.sqrt(self.d)))

    @property
    def causal_pairs(self) -> int:
        return self.B * self.Hq * self.T * (self.T + 1) // 2


# The five workloads, smallest first.
WORKLOADS = [
    Workload("B1_T64_Hq6_Hkv2_d64", 1, 64, 6, 2, 64),
    Workload("B8_T512_Hq6_Hkv2_d64", 8, 512, 6, 2, 64),
    Workload("B16_T1024_Hq6_Hkv2_d64", 16, 1024, 6, 2, 64),
    Workload("B8_T2048_Hq12_Hkv4_d64_qk2", 8, 2048, 12, 4, 64, qk_mult=2.0),
    Workload("B4_T4096_Hq32_Hkv8_d128", 4, 4096, 32, 8, 128),
]
WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS}


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (uint16), round-to-nearest-even.

    Written from the IEEE 754 definition: bfloat16 keeps the upper 16 bits of the
    binary32 pattern; the discarded lower half is compared with one half-unit
    (0x8000), ties go to the even upper half. NaNs stay NaN (quiet bit set); the
    carry out of a finite maximum correctly overflows to infinity.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    upper = u >> np.uint32(16)
    lower = u & np.uint32(0xFFFF)
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint32(1)) == 1))
    out = (upper + round_up.astype(np.uint32)).astype(np.uint32)
    is_nan = ((u & np.uint32(0x7F800000)) == 0x7F800000) & ((u & np.uint32(0x007FFFFF)) != 0)
    out = np.where(is_nan, upper | np.uint32(0x0040), out)
    return out.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for test-side bookkeeping)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def make_inputs(B, T, Hq, Hkv, d, seed, qk_mult=1.0, with_do=True):
    """Q [B,T,Hq,d], K and V [B,T,Hkv,d], dO [B,T,Hq,d] as bf16 bit patterns (uint16)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, T, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, T, Hkv, d), dtype=np.float32)
    out = {}
    if qk_mult != 1.0:
        q = q * np.float32(qk_mult)
        k = k * np.float32(qk_mult)
    out["q"] = f32_to_bf16_bits(q)
    out["k"] = f32_to_bf16_bits(k)
    out["v"] = f32_to_bf16_bits(v)
    if with_do:
        out["do"] = f32_to_bf16_bits(rng.standard_normal((B, T, Hq, d), dtype=np.float32))
    return out


def make_workload_inputs(w: Workload, seed, with_do=True):
    return make_inputs(w.B, w.T, w.Hq, w.Hkv, w.d, seed, w.qk_mult, with_do)


def slice_group(arrs, Hq, Hkv, b, g):
    """The inputs of one (batch, kv head) slice: batches and kv groups are independent,
    so attention on the slice equals the full result restricted to it."""
    G = Hq // Hkv
    out = {}
    for name, a in arrs.items():
        if a.shape[2] == Hq:
            out[name] = np.ascontiguousarray(a[b:b + 1, :, g * G:(g + 1) * G, :])
        else:
            out[name] = np.ascontiguousarray(a[b:b + 1, :, g:g + 1, :])
    return out


def rope_tables(T, d, base=10000.0):
    """Rotary position tables, inputs of the RoPE calls: cos and sin of t * base^(-2i/d)
    for positions t < T and pairs i < d/2 (angles in float64, rounded once to float32),
    each float32 [T][d/2]. The usual Llama choice of frequencies; the calls take any
    table."""
    t = np.arange(T, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)[None, :]
    ang = t * inv
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
