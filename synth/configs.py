"""Shapes of the five seeded workloads of the CCA / CCGQA forward pass.

Notation follows the method's description: residual width ``E``, latent
query width ``e_q = H_q * d``, latent key/value width ``e_kv = H_kv * d``,
``G = H_q / H_kv`` query heads per shared key/value head (CCGQA; ``G = 1`` is
plain CCA), ``k_s`` / ``k_c`` taps of the sequence / channel convolutions.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, asdict, replace


@dataclass(frozen=True)
class CCAShape:
    batch: int
    seq_len: int            # prefill tokens per sequence (T); 1 for a decode step
    d_model: int            # E
    n_q_heads: int          # H_q
    n_kv_heads: int         # H_kv
    head_dim: int           # d
    seq_conv_k: int = 4     # k_s
    chan_conv_k: int = 4    # k_c
    use_qk_mean: int = 1
    use_value_shift: int = 1
    use_qk_norm: int = 1
    rope_base: float = 10000.0   # 0 switches RoPE off
    norm_eps: float = 1e-6
    dtype: str = "bf16"     # storage / MFMA operand type of activations and weights: "bf16" | "f32"
    cache_len: int = 0      # decode only: number of past tokens already in the cache (L)

    # ---- derived sizes -------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def e_q(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def e_kv(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_qkv(self) -> int:
        return self.e_q + 2 * self.e_kv

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def tau(self) -> list:
        """Synthetic per-query-head logit temperature: sqrt(d) for every head."""
        return [math.sqrt(self.head_dim)] * self.n_q_heads

    def with_(self, **kw) -> "CCAShape":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


def shape_from_dict(d: dict) -> CCAShape:
    return CCAShape(**d)


# The five workloads.  0-3 are prefill, 4 is one decode step against a cache of
# 32768 past tokens.  The decode workload shares the head shapes of workload 2
# and therefore its RoPE base.
WORKLOADS = {
    "cca_prefill_tiny_f32": CCAShape(
        batch=1, seq_len=256, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=16,
        rope_base=10000.0, dtype="f32"),
    "cca_prefill_b4_t2048": CCAShape(
        batch=4, seq_len=2048, d_model=2048, n_q_heads=8, n_kv_heads=8, head_dim=64,
        rope_base=10000.0, dtype="bf16"),
    "ccgqa_prefill_t8192": CCAShape(
        batch=1, seq_len=8192, d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=64,
        rope_base=500000.0, dtype="bf16"),
    "ccgqa_prefill_t16384": CCAShape(
        batch=1, seq_len=16384, d_model=4096, n_q_heads=8, n_kv_heads=2, head_dim=64,
        rope_base=500000.0, dtype="bf16"),
    "ccgqa_decode_b64_l32768": CCAShape(
        batch=64, seq_len=1, d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=64,
        rope_base=500000.0, dtype="bf16", cache_len=32768),
}

WORKLOAD_ORDER = list(WORKLOADS)

# Full-width baselines for the prefill comparison against ccgqa_prefill_t16384
# (same T, E and head size): the same kernels with the extras off, i.e. one
# unit tap in each convolution, no q-k-mean, value-shift or L2 norm, and a
# logit scale of 1/sqrt(d) (see COMPARISON_OVERRIDES).  "GQA-8" is read as 8
# key/value heads shared by the 64 query heads.
COMPARISONS = {
    "mha_prefill_t16384": CCAShape(
        batch=1, seq_len=16384, d_model=4096, n_q_heads=64, n_kv_heads=64, head_dim=64,
        seq_conv_k=1, chan_conv_k=1, use_qk_mean=0, use_value_shift=0, use_qk_norm=0,
        rope_base=500000.0, dtype="bf16"),
    "gqa8_prefill_t16384": CCAShape(
        batch=1, seq_len=16384, d_model=4096, n_q_heads=64, n_kv_heads=8, head_dim=64,
        seq_conv_k=1, chan_conv_k=1, use_qk_mean=0, use_value_shift=0, use_qk_norm=0,
        rope_base=500000.0, dtype="bf16"),
}
# Weights the comparison baselines use in place of the drawn ones.
COMPARISON_OVERRIDES = {"taps": 1.0, "tau": "1/sqrt(d)"}


def workload(name_or_index) -> CCAShape:
    if isinstance(name_or_index, int):
        return WORKLOADS[WORKLOAD_ORDER[name_or_index]]
    if name_or_index in COMPARISONS:
        return COMPARISONS[name_or_index]
    return WORKLOADS[name_or_index]
