"""Shared plumbing of the GPU tests: upload seeded inputs, run libcca through
its C ABI, and compare with the fp64 oracle at the stated tolerances."""

from __future__ import annotations

import math

import numpy as np
import torch

from synth import CCAShape, make_decode, make_prefill

# bf16 I/O: max |err| <= 2e-2 and ||err|| / ||ref|| <= 5e-3; fp32 mode: rel L2 <= 1e-5.
BF16_MAXABS, BF16_REL, F32_REL = 2e-2, 5e-3, 1e-5


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_parity(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if got.size else 0.0
    print(f"[parity] {what}: max-abs {m:.3e} rel-L2 {r:.3e} ({dtype})", flush=True)
    if dtype == "bf16":
        assert m <= BF16_MAXABS and r <= BF16_REL, f"{what}: max-abs {m:.3e} rel-L2 {r:.3e}"
    else:
        assert r <= F32_REL, f"{what}: rel-L2 {r:.3e} (max-abs {m:.3e})"
    return m, r


def lib():
    from efficient_transformer_attention_amd import cca
    return cca


def tens():
    from efficient_transformer_attention_amd import tensors
    return tensors


def upload_weights(Wt, dev="cuda"):
    T = tens()
    L = lib()
    return L.Weights(
        w_qkv=T.to_device(Wt.w_qkv_s, dev), w_o=T.to_device(Wt.w_o_s, dev),
        q_seq_taps=torch.from_numpy(Wt.q_seq_taps).to(dev),
        k_seq_taps=torch.from_numpy(Wt.k_seq_taps).to(dev),
        q_chan_taps=torch.from_numpy(Wt.q_chan_taps).to(dev),
        k_chan_taps=torch.from_numpy(Wt.k_chan_taps).to(dev),
        tau=torch.from_numpy(Wt.tau).to(dev),
        q_chan_dense=None if Wt.q_chan_dense is None else torch.from_numpy(Wt.q_chan_dense).to(dev),
        k_chan_dense=None if Wt.k_chan_dense is None else torch.from_numpy(Wt.k_chan_dense).to(dev))


def set_taps(P, seq=None, chan=None, tau=None):
    """Override taps / temperatures of a generated workload (host side)."""
    w = P.weights
    if seq is not None:
        w.q_seq_taps = np.ascontiguousarray(seq[0], dtype=np.float32)
        w.k_seq_taps = np.ascontiguousarray(seq[1], dtype=np.float32)
    if chan is not None:
        w.q_chan_taps = np.ascontiguousarray(chan[0], dtype=np.float32)
        w.k_chan_taps = np.ascontiguousarray(chan[1], dtype=np.float32)
    if tau is not None:
        w.tau = np.ascontiguousarray(tau, dtype=np.float32)


class PrefillRun:
    """Device buffers and one prefill through cca_prefill_forward."""

    def __init__(self, shape: CCAShape, P, capacity: int = 0, dev="cuda", chan_conv="per_head",
                 qk_mean="pre_post", attn="auto"):
        L, T = lib(), tens()
        self.shape, self.P = shape, P
        self.cfg = L.make_config(shape, chan_conv=chan_conv, qk_mean=qk_mean, attn=attn)
        assert L.validate_config(self.cfg) == L.CCA_OK
        self.w = upload_weights(P.weights, dev)
        self.x = T.to_device(P.x_s, dev)
        self.y = torch.empty_like(self.x)
        self.ws = T.workspace(L.prefill_workspace_size(self.cfg), dev)
        self.layout = L.prefill_workspace_layout(self.cfg)
        self.state = None
        if capacity:
            s = shape
            sd = T.storage_dtype(s.dtype)
            # carried pre-conv rows: k_s - 1, plus k_c - 1 under the grouped channel conv
            win = s.seq_conv_k - 1 + (s.chan_conv_k - 1 if chan_conv == "grouped" else 0)
            self.state = L.State(
                k_cache=torch.zeros((s.batch, s.n_kv_heads, capacity, s.head_dim), dtype=sd, device=dev),
                v_cache=torch.zeros((s.batch, s.n_kv_heads, capacity, s.head_dim), dtype=sd, device=dev),
                capacity=capacity,
                conv_q=torch.zeros((s.batch, win, s.e_q), dtype=sd, device=dev),
                conv_k=torch.zeros((s.batch, win, s.e_kv), dtype=sd, device=dev),
                vshift=torch.zeros((s.batch, max(s.n_kv_heads // 2, 1), s.head_dim), dtype=sd, device=dev))

    def run(self):
        lib().prefill_forward(self.cfg, self.w, self.x, self.y, self.ws, self.state)
        torch.cuda.synchronize()
        return tens().to_f64(self.y)

    def ws_view(self, slot, dtype, shape):
        off = self.layout[slot]
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.ws[off:off + n].view(dtype).view(*shape)

    def qkv_dtype(self):
        """The down-projection output: fp16 in bf16 mode, fp32 in fp32 mode."""
        return torch.float32 if self.shape.dtype == "f32" else torch.float16

    def qk_dtype(self):
        s = self.shape
        if s.dtype == "f32":
            return torch.float32
        return torch.float16 if s.use_qk_norm else torch.bfloat16

    def padded_T(self):
        return (self.shape.seq_len + 127) // 128 * 128


def vt_unpermute(vt: np.ndarray) -> np.ndarray:
    """Inverse of the key order inside 16-token groups of the transposed value
    buffer (bits 2 and 3 of the token index exchanged; an involution)."""
    Tp = vt.shape[-1]
    t = np.arange(Tp)
    perm = (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1)
    return vt[..., perm]


def sample_rows(T: int, n: int, seed: int = 1):
    rng = np.random.default_rng(seed)
    fixed = set(range(min(T, 8))) | set(range(max(0, T - 8), T))
    extra = rng.choice(T, size=min(n, T), replace=False)
    return np.array(sorted(fixed | set(int(e) for e in extra)))


def tau_inv_sqrt_d(shape: CCAShape):
    return np.full(shape.n_q_heads, 1.0 / math.sqrt(shape.head_dim), dtype=np.float32)
