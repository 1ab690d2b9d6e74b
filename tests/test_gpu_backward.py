"""GPU parity of the backward pass (cca_prefill_forward_train +
cca_prefill_backward) against the fp64 backward oracle, through the C ABI.

Every gradient (x, both projection matrices, the four tap sets and the
temperatures) is compared element by element with oracle.backward on the
same seeded inputs and upstream gradient, by relative L2 (against an RMS
floor of 1e-3 where the exact gradient vanishes).

fp32 validation mode: <= 1e-4.

bf16 I/O: bounds derived per shape and per gradient from the oracle alone,
not from the kernels' measured errors.  delta_n is the relative L2 change of
gradient n when x, dy, W_qkv and W_o are each perturbed by independent
relative errors drawn uniformly from [-u, u], u = 2^-9 (one bf16 rounding),
with the fp64 oracle on the same shape: the gradient's own sensitivity to a
bf16-sized rounding of what feeds it, cancellation in its reductions
included.  The bf16 path rounds at R = 11 points in sequence, each a
rounding of the same relative size (qkv~ to fp16; q, k to fp16; v to bf16; P
to bf16 in P*V; the stored O; dO; P again for dV; dS for dQ and dK; the
stored dq/dk; dz for the weight gradients; x for dx), independent of one
another, so the expected error grows like sqrt(R) * delta_n.  The bound is
twice that, 2 * sqrt(11) * delta_n ~ 6.6 delta_n, and never below 1e-3.
"""

import sys

import numpy as np
import pytest
import torch

import oracle.backward as BW
from synth import CCAShape, make_prefill, make_upstream_grad, workload
from gpu_helpers import lib, set_taps, tau_inv_sqrt_d, tens, upload_weights

pytestmark = pytest.mark.gpu

GRADS = ["x", "w_qkv", "w_o", "q_seq_taps", "k_seq_taps", "q_chan_taps", "k_chan_taps", "tau"]
TOL_F32 = 1e-4
ROUNDING_POINTS = 11
BF16_U = 2.0 ** -9


def _rel(g, r):
    g, r = np.asarray(g, dtype=np.float64), np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-3 * np.sqrt(r.size)))


def bf16_bounds(P, dyB, shape, ref, readings=None, seed=11):
    """Per-gradient bf16 bounds from the oracle's sensitivity (module doc)."""
    rng = np.random.default_rng(seed)

    def pert(a):
        a = np.asarray(a, dtype=np.float64)
        return a * (1.0 + BF16_U * rng.uniform(-1.0, 1.0, size=a.shape))

    W = P.weights.f64()
    W2 = dict(W)
    for f in ("w_qkv", "w_o"):
        W2[f] = pert(W[f])
    kw = {} if readings is None else dict(readings=readings)
    g2 = BW.prefill_backward(pert(P.x), W2, shape, pert(dyB.dy), **kw)
    k = 2.0 * np.sqrt(ROUNDING_POINTS)
    return {n: max(k * _rel(g2[n], ref[n]), 1e-3) for n in GRADS}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class TrainRun:
    """Device buffers of one forward_train + backward."""

    def __init__(self, shape, P, dyB, dev="cuda", qk_mean="pre_post", attn="auto"):
        L, T = lib(), tens()
        self.shape, self.P = shape, P
        self.cfg = L.make_config(shape, qk_mean=qk_mean, attn=attn)
        assert L.validate_config(self.cfg) == L.CCA_OK
        self.w = upload_weights(P.weights, dev)
        self.x = T.to_device(P.x_s, dev)
        self.dy = T.to_device(dyB.dy_s, dev)
        self.y = torch.empty_like(self.x)
        self.ws = T.workspace(L.train_workspace_size(self.cfg), dev)
        s = shape
        f32 = dict(dtype=torch.float32, device=dev)
        self.g = L.Grads(
            x=torch.empty_like(self.x),
            w_qkv=torch.empty((s.e_q + 2 * s.e_kv, s.d_model), **f32),
            w_o=torch.empty((s.d_model, s.e_q), **f32),
            q_seq_taps=torch.empty((s.e_q, s.seq_conv_k), **f32),
            k_seq_taps=torch.empty((s.e_kv, s.seq_conv_k), **f32),
            q_chan_taps=torch.empty((s.n_q_heads, s.chan_conv_k), **f32),
            k_chan_taps=torch.empty((s.n_kv_heads, s.chan_conv_k), **f32),
            tau=torch.empty((s.n_q_heads,), **f32))

    def forward(self):
        lib().prefill_forward_train(self.cfg, self.w, self.x, self.y, self.ws)

    def backward(self):
        lib().prefill_backward(self.cfg, self.w, self.x, self.dy, self.g, self.ws)
        torch.cuda.synchronize()
        return {n: tens().to_f64(getattr(self.g, n)) for n in GRADS}


def check_grads(got, ref, dtype, what, bounds=None):
    """bounds: the per-gradient bf16 bounds (bf16_bounds); fp32 uses TOL_F32."""
    worst = {}
    for n in GRADS:
        g, r = got[n], np.asarray(ref[n], dtype=np.float64)
        assert g.shape == r.shape, (n, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{what}: non-finite d{n}"
        # relative L2, against an RMS floor of 1e-3 for gradients that are
        # zero in exact arithmetic (with T = 1 nothing reaches the q/k path)
        e = _rel(g, r)
        worst[n] = e
        tol = TOL_F32 if dtype == "f32" else bounds[n]
        _say(f"[grad] {what} d{n}: rel-L2 {e:.3e} bound {tol:.2e} max-abs {np.max(np.abs(g - r)):.3e} "
             f"(|ref| max {np.max(np.abs(r)):.3e})")
    for n, e in worst.items():
        tol = TOL_F32 if dtype == "f32" else bounds[n]
        assert e <= tol, f"{what}: d{n} rel-L2 {e:.3e} > {tol:.2e}"


SMALL = {
    "bf16_g2_ragged": (CCAShape(batch=2, seq_len=300, d_model=256, n_q_heads=4, n_kv_heads=2,
                                head_dim=64, rope_base=10000.0), None),
    # weight gradients read token-major in place, the 2100 tokens split into
    # two contraction slices, the second ending in a partial 32-row tile
    "bf16_split_ragged": (CCAShape(batch=1, seq_len=2100, d_model=256, n_q_heads=4, n_kv_heads=2,
                                   head_dim=64, rope_base=10000.0), None),
    "bf16_g4_base5e5": (CCAShape(batch=1, seq_len=200, d_model=512, n_q_heads=8, n_kv_heads=2,
                                 head_dim=64, rope_base=500000.0), None),
    "bf16_d16": (CCAShape(batch=2, seq_len=130, d_model=128, n_q_heads=2, n_kv_heads=2,
                          head_dim=16), None),
    "bf16_d32_t77": (CCAShape(batch=1, seq_len=77, d_model=256, n_q_heads=4, n_kv_heads=4,
                              head_dim=32), None),
    "bf16_d128": (CCAShape(batch=1, seq_len=150, d_model=256, n_q_heads=2, n_kv_heads=2,
                           head_dim=128), None),
    "f32_d32_g2_ragged": (CCAShape(batch=2, seq_len=190, d_model=128, n_q_heads=4, n_kv_heads=2,
                                   head_dim=32, dtype="f32"), None),
    "f32_d64_g4": (CCAShape(batch=1, seq_len=260, d_model=256, n_q_heads=8, n_kv_heads=2,
                            head_dim=64, rope_base=500000.0, dtype="f32"), None),
    "f32_d16_taps_2_3": (CCAShape(batch=1, seq_len=70, d_model=64, n_q_heads=2, n_kv_heads=2,
                                  head_dim=16, seq_conv_k=2, chan_conv_k=3, dtype="f32"), None),
    "bf16_taps_2_3": (CCAShape(batch=1, seq_len=140, d_model=256, n_q_heads=4, n_kv_heads=2,
                               head_dim=64, seq_conv_k=2, chan_conv_k=3), None),
    "bf16_single_token": (CCAShape(batch=3, seq_len=1, d_model=256, n_q_heads=4, n_kv_heads=2,
                                   head_dim=64), None),
    "bf16_g8": (CCAShape(batch=1, seq_len=100, d_model=256, n_q_heads=8, n_kv_heads=1,
                         head_dim=64, use_value_shift=0), None),
    "bf16_switches_off": (CCAShape(batch=1, seq_len=160, d_model=256, n_q_heads=4, n_kv_heads=4,
                                   head_dim=64, use_qk_mean=0, use_value_shift=0, use_qk_norm=0,
                                   rope_base=10000.0), "inv_sqrt_d"),
    "f32_switches_off": (CCAShape(batch=1, seq_len=96, d_model=128, n_q_heads=2, n_kv_heads=2,
                                  head_dim=32, use_qk_mean=0, use_value_shift=0, use_qk_norm=0,
                                  rope_base=0.0, dtype="f32"), "inv_sqrt_d"),
    "bf16_norm_mixed_tau": (CCAShape(batch=1, seq_len=210, d_model=256, n_q_heads=4, n_kv_heads=2,
                                     head_dim=64), "mixed"),
}


def _prepare(shape, tau, seed=0):
    P = make_prefill(shape, seed=seed)
    if tau == "inv_sqrt_d":
        set_taps(P, tau=tau_inv_sqrt_d(shape))
    elif tau == "mixed":
        set_taps(P, tau=np.array([8.0, 50.0, 0.5, 41.0], dtype=np.float32))
    return P, make_upstream_grad(shape, seed=seed)


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_small_parity(name):
    shape, tau = SMALL[name]
    _say(f"[backward] {name} {shape}")
    P, dyB = _prepare(shape, tau)
    run = TrainRun(shape, P, dyB)
    run.forward()
    got = run.backward()
    ref = BW.prefill_backward(P.x, P.weights.f64(), shape, dyB.dy)
    bounds = bf16_bounds(P, dyB, shape, ref) if shape.dtype == "bf16" else None
    check_grads(got, ref, shape.dtype, name, bounds)


def test_forward_train_output_equals_forward():
    """The training forward writes the same y as the inference forward, bit
    for bit (it only keeps extra activations)."""
    shape = SMALL["bf16_g2_ragged"][0]
    _say(f"[backward] forward_train == forward {shape}")
    P, dyB = _prepare(shape, None)
    run = TrainRun(shape, P, dyB)
    run.forward()
    torch.cuda.synchronize()
    y_train = run.y.clone()
    L, T = lib(), tens()
    ws = T.workspace(L.prefill_workspace_size(run.cfg))
    y = torch.empty_like(run.x)
    L.prefill_forward(run.cfg, run.w, run.x, y, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_train.view(torch.int16))


def test_backward_deterministic():
    """Fixed summation orders: two backward passes agree bit for bit."""
    shape = SMALL["bf16_g4_base5e5"][0]
    _say(f"[backward] repeat bitwise {shape}")
    P, dyB = _prepare(shape, None)
    run = TrainRun(shape, P, dyB)
    run.forward()
    run.backward()
    first = {n: getattr(run.g, n).clone() for n in GRADS}
    run.backward()
    for n in GRADS:
        a, b = first[n], getattr(run.g, n)
        iv = torch.int16 if a.element_size() == 2 else torch.int32
        assert torch.equal(a.view(iv), b.view(iv)), n


def test_backward_workload_full():
    """The full prefill workload (B=4, T=2048, E=2048, 8 heads of 64): every
    gradient element against the fp64 oracle."""
    shape = workload("cca_prefill_b4_t2048")
    _say(f"[backward] full workload {shape}")
    P, dyB = _prepare(shape, None)
    run = TrainRun(shape, P, dyB)
    run.forward()
    got = run.backward()
    ref = BW.prefill_backward(P.x, P.weights.f64(), shape, dyB.dy)
    check_grads(got, ref, shape.dtype, "cca_prefill_b4_t2048", bf16_bounds(P, dyB, shape, ref))
