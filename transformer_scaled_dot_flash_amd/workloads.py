"""The five synthetic workloads, with their input seeds and work counts.

Shapes follow the pages: GPT-2 small head_dim 64 (learn-cuda-from-scratch
Ch. 11 "Attention", section 11.1), the multi-head exercise B=1 H=4 T=128 D=64
(same page, exercises), and the Llama-3-8B GQA shape n_q=32, n_kv=8,
d_head=128 (same page, sections 11.8.1 and 11.11).  Every tensor is i.i.d.
N(0,1) from its own seeded stream: seed = 1000*c + {1: Q, 2: K, 3: V} for the
workload with ordinal c (1..5).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import inputs


def f32(x: float) -> float:
    """Round a Python float to the nearest float32 value."""
    return float(np.float32(x))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    ordinal: int
    kind: str  # "prefill" or "decode"
    B: int
    H_q: int
    H_kv: int
    T_q: int
    T_kv: int
    D: int
    causal: bool
    dtype: str  # "f32" or "bf16"
    scale: float  # a float32 value

    @property
    def seeds(self):
        return tuple(1000 * self.ordinal + i for i in (1, 2, 3))

    def visible_pairs(self) -> int:
        """Number of (query row, key) pairs that take part, per (b, h_q)."""
        if not self.causal:
            return self.T_q * self.T_kv
        off = self.T_kv - self.T_q
        # row i sees keys 0..i+off
        return sum(min(self.T_kv, i + off + 1) for i in range(self.T_q))

    def flops(self) -> int:
        """4*D flops per visible pair per (b, h_q): one multiply-add for the
        score and one for the weighted sum, per component."""
        return 4 * self.B * self.H_q * self.D * self.visible_pairs()

    def bytes(self) -> int:
        """Algorithmic HBM bytes: Q and O at H_q, K and V at H_kv, once each."""
        e = 4 if self.dtype == "f32" else 2
        q = self.B * self.H_q * self.T_q * self.D
        kv = self.B * self.H_kv * self.T_kv * self.D
        return e * (2 * q + 2 * kv)

    def make_inputs(self):
        """(Q, K, V) as numpy arrays: float32 values or bfloat16 bit patterns."""
        sq, sk, sv = self.seeds
        q = inputs.normal(sq, (self.B, self.H_q, self.T_q, self.D), self.dtype)
        k = inputs.normal(sk, (self.B, self.H_kv, self.T_kv, self.D), self.dtype)
        v = inputs.normal(sv, (self.B, self.H_kv, self.T_kv, self.D), self.dtype)
        return q, k, v


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_f32_T128_D64", 1, "prefill", 1, 1, 1, 128, 128, 64,
                 False, "f32", f32(1.0 / 8.0)),
        Workload("mha_causal_bf16_B1_H4_T128_D64", 2, "prefill", 1, 4, 4, 128, 128, 64,
                 True, "bf16", f32(1.0 / math.sqrt(64))),
        Workload("gpt2s_causal_bf16_B4_H12_T1024_D64", 3, "prefill", 4, 12, 12, 1024, 1024, 64,
                 True, "bf16", f32(1.0 / math.sqrt(64))),
        Workload("llama3_8b_gqa_causal_bf16_B1_Hq32_Hkv8_T8192_D128", 4, "prefill", 1, 32, 8,
                 8192, 8192, 128, True, "bf16", f32(1.0 / math.sqrt(128))),
        Workload("gqa_decode_bf16_B64_Hq32_Hkv8_Tkv4096_D128", 5, "decode", 64, 32, 8, 1, 4096,
                 128, False, "bf16", f32(1.0 / math.sqrt(128))),
    ]
}

BY_ORDINAL = {w.ordinal: w for w in WORKLOADS.values()}
PREFILL_HEADLINE = BY_ORDINAL[4]
DECODE_HEADLINE = BY_ORDINAL[5]
