"""Seeded synthetic inputs for the CCA / CCGQA forward pass.

Every value is drawn from one NumPy ``Generator(PCG64(seed))`` in a fixed
order, then rounded to the storage precision of the workload (bf16 with
round-to-nearest-even, or fp32).  The rounded values are the inputs of BOTH
the GPU path and the fp64 oracle, so input quantisation is never counted as
error.  Distributions:

* hidden states ``x ~ N(0, 1)``
* projection weights ``~ N(0, 1/fan_in)``
* convolution taps ``~ N(0, 1/k)`` (always fp32)
* temperature ``tau_h = sqrt(d)`` (fp32, deterministic)
* decode only: latent key/value cache, carried convolution window and the
  previous token's value, all ``~ N(0, 1)``.
* backward only: the upstream gradient ``dy ~ N(0, 1)`` of the layer output,
  drawn from its own generator (seed + 7919) so the prefill draws above
  are unchanged.

Draw order (prefill): x, W_q, W_k, W_v, W_o, q seq taps, k seq taps,
q channel taps, k channel taps.  Decode draws the same list (x is the new
token of each sequence) and then, per sequence b in order, K[b] and V[b] of
the cache, followed by the q and k convolution windows and the value-shift
state.

Nothing here computes any step of the method.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import CCAShape


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to bf16 (RNE) and return the raw 16-bit patterns as uint16.

    The value is first rounded to fp32 (NumPy's RNE cast), then the fp32 bit
    pattern is rounded to its upper 16 bits with ties to even.  Inputs are
    finite draws far from the bf16 overflow threshold.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float64."""
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32)


def f64_to_bf16_f64(a: np.ndarray) -> np.ndarray:
    """Round to bf16 and return the rounded values as float64."""
    return bf16_bits_to_f64(round_to_bf16_bits(a))


def _store(a: np.ndarray, dtype: str):
    """Return (storage array, exact float64 value of the storage)."""
    if dtype == "bf16":
        bits = round_to_bf16_bits(a)
        return bits, bf16_bits_to_f64(bits)
    if dtype == "f32":
        f = np.ascontiguousarray(a, dtype=np.float32)
        return f, f.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _f32(a: np.ndarray):
    f = np.ascontiguousarray(a, dtype=np.float32)
    return f, f.astype(np.float64)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclass
class Weights:
    """Weights in storage form (``*_s``: uint16 bf16 bits or float32) and as
    exact float64 values.  Matrices are [out, in] row-major."""
    w_qkv_s: np.ndarray        # [e_q + 2 e_kv, E]  rows: q | k | v
    w_o_s: np.ndarray          # [E, e_q]
    q_seq_taps: np.ndarray     # [e_q, k_s] fp32, taps indexed by lag
    k_seq_taps: np.ndarray     # [e_kv, k_s]
    q_chan_taps: np.ndarray    # [H_q, k_c] fp32, taps indexed by lag
    k_chan_taps: np.ndarray    # [H_kv, k_c]
    tau: np.ndarray            # [H_q] fp32
    w_qkv: np.ndarray          # float64 values of the above
    w_o: np.ndarray
    # grouped channel conv only: [H, d_out, k_c, d_in] fp32 (add_chan_dense)
    q_chan_dense: Optional[np.ndarray] = None
    k_chan_dense: Optional[np.ndarray] = None

    def f64(self):
        """The weights as float64 arrays, in the order the oracle takes them."""
        out = dict(w_qkv=self.w_qkv, w_o=self.w_o,
                   q_seq_taps=self.q_seq_taps.astype(np.float64),
                   k_seq_taps=self.k_seq_taps.astype(np.float64),
                   q_chan_taps=self.q_chan_taps.astype(np.float64),
                   k_chan_taps=self.k_chan_taps.astype(np.float64),
                   tau=self.tau.astype(np.float64))
        if self.q_chan_dense is not None:
            out["q_chan_dense"] = self.q_chan_dense.astype(np.float64)
            out["k_chan_dense"] = self.k_chan_dense.astype(np.float64)
        return out


@dataclass
class Prefill:
    shape: CCAShape
    x_s: np.ndarray            # [B, T, E] storage
    x: np.ndarray              # float64
    weights: Weights


@dataclass
class Decode:
    shape: CCAShape
    capacity: int
    x_s: np.ndarray            # [B, E] storage (new token per sequence)
    x: np.ndarray
    weights: Weights
    k_cache_s: np.ndarray      # [B, H_kv, capacity, d] storage; slots >= cache_len are zero
    v_cache_s: np.ndarray
    conv_q_s: np.ndarray       # [B, k_s - 1, e_q]   slot 0 = oldest token
    conv_k_s: np.ndarray       # [B, k_s - 1, e_kv]
    vshift_s: np.ndarray       # [B, H_kv // 2, d]

    def cache_f64(self, b: int, which: str, upto: Optional[int] = None) -> np.ndarray:
        """float64 values of K or V of sequence b, slots [0, upto)."""
        src = self.k_cache_s if which == "k" else self.v_cache_s
        upto = self.shape.cache_len if upto is None else upto
        return _to_f64(src[b, :, :upto, :], self.shape.dtype)

    def state_f64(self):
        dt = self.shape.dtype
        return (_to_f64(self.conv_q_s, dt), _to_f64(self.conv_k_s, dt),
                _to_f64(self.vshift_s, dt))


def _to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


def _draw_weights(rng: np.random.Generator, s: CCAShape) -> Weights:
    E, eq, ekv = s.d_model, s.e_q, s.e_kv
    wq = rng.standard_normal((eq, E)) * np.sqrt(1.0 / E)
    wk = rng.standard_normal((ekv, E)) * np.sqrt(1.0 / E)
    wv = rng.standard_normal((ekv, E)) * np.sqrt(1.0 / E)
    wo = rng.standard_normal((E, eq)) * np.sqrt(1.0 / eq)
    qs = rng.standard_normal((eq, s.seq_conv_k)) * np.sqrt(1.0 / s.seq_conv_k)
    ks = rng.standard_normal((ekv, s.seq_conv_k)) * np.sqrt(1.0 / s.seq_conv_k)
    qc = rng.standard_normal((s.n_q_heads, s.chan_conv_k)) * np.sqrt(1.0 / s.chan_conv_k)
    kc = rng.standard_normal((s.n_kv_heads, s.chan_conv_k)) * np.sqrt(1.0 / s.chan_conv_k)
    w_qkv_s, w_qkv = _store(np.concatenate([wq, wk, wv], axis=0), s.dtype)
    w_o_s, w_o = _store(wo, s.dtype)
    tau = np.asarray(s.tau(), dtype=np.float32)
    return Weights(w_qkv_s=w_qkv_s, w_o_s=w_o_s,
                   q_seq_taps=_f32(qs)[0], k_seq_taps=_f32(ks)[0],
                   q_chan_taps=_f32(qc)[0], k_chan_taps=_f32(kc)[0],
                   tau=tau, w_qkv=w_qkv, w_o=w_o)


def make_prefill(s: CCAShape, seed: int = 0) -> Prefill:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((s.batch, s.seq_len, s.d_model))
    w = _draw_weights(rng, s)
    x_s, x64 = _store(x, s.dtype)
    return Prefill(shape=s, x_s=x_s, x=x64, weights=w)


def make_decode(s: CCAShape, seed: int = 0, capacity: Optional[int] = None,
                cache_fill: str = "normal", window: Optional[int] = None) -> Decode:
    """A decode step against a cache of ``s.cache_len`` past tokens.

    ``window``: rows of the carried pre-conv window (default k_s - 1; the
    grouped channel conv carries (k_s - 1) + (k_c - 1)).

    ``cache_fill="normal"`` draws the cache and the carried state ~ N(0, 1)
    (the synthetic long-cache workload).  The cache is drawn per sequence in
    float32 to bound host memory (the full cache of the long workload is
    about 1.07e9 values)."""
    if s.use_value_shift and s.n_kv_heads % 2:
        raise ValueError("value-shift needs an even number of kv heads")
    L = s.cache_len
    cap = L + 1 if capacity is None else capacity
    if cap < L + 1:
        raise ValueError("capacity must hold the new token")
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((s.batch, s.d_model))
    w = _draw_weights(rng, s)
    x_s, x64 = _store(x, s.dtype)
    B, H, d = s.batch, s.n_kv_heads, s.head_dim
    sdt = np.uint16 if s.dtype == "bf16" else np.float32
    kc = np.zeros((B, H, cap, d), dtype=sdt)
    vc = np.zeros((B, H, cap, d), dtype=sdt)
    if cache_fill != "normal":
        raise ValueError(cache_fill)
    for b in range(B):
        kb = rng.standard_normal((H, L, d), dtype=np.float32)
        vb = rng.standard_normal((H, L, d), dtype=np.float32)
        kc[b, :, :L, :] = _store(kb, s.dtype)[0]
        vc[b, :, :L, :] = _store(vb, s.dtype)[0]
    ks1 = s.seq_conv_k - 1 if window is None else window
    cq = rng.standard_normal((B, ks1, s.e_q))
    ck = rng.standard_normal((B, ks1, s.e_kv))
    vs = rng.standard_normal((B, max(H // 2, 0), d))
    return Decode(shape=s, capacity=cap, x_s=x_s, x=x64, weights=w,
                  k_cache_s=kc, v_cache_s=vc,
                  conv_q_s=_store(cq, s.dtype)[0], conv_k_s=_store(ck, s.dtype)[0],
                  vshift_s=_store(vs, s.dtype)[0])


@dataclass
class Backward:
    """Upstream gradient of a prefill's output, for the backward pass."""
    dy_s: np.ndarray           # [B, T, E] storage
    dy: np.ndarray             # float64


def make_upstream_grad(s: CCAShape, seed: int = 0) -> Backward:
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    dy = rng.standard_normal((s.batch, s.seq_len, s.d_model))
    dy_s, dy64 = _store(dy, s.dtype)
    return Backward(dy_s=dy_s, dy=dy64)


def add_chan_dense(w: Weights, s: CCAShape, seed: int = 0) -> Weights:
    """Weights of the grouped channel conv, W[h, i, j, c] ~ N(0, 1 / (k_c d))
    (fan-in k_c d), fp32, drawn from their own stream so the other draws of
    a seed stay as they are."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    sc = np.sqrt(1.0 / (s.chan_conv_k * s.head_dim))
    d, kc = s.head_dim, s.chan_conv_k
    w.q_chan_dense = _f32(rng.standard_normal((s.n_q_heads, d, kc, d)) * sc)[0]
    w.k_chan_dense = _f32(rng.standard_normal((s.n_kv_heads, d, kc, d)) * sc)[0]
    return w
