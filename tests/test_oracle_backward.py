"""Pins of the fp64 backward oracle against things other than itself (CPU only).

* Every step's backward against central finite differences of the forward
  oracle's step (the forward is pinned separately by brute force, closed
  forms and the MHA reduction): for random cotangents g and directions v,
  <g, (f(x + h v) - f(x - h v)) / 2h> must equal <bwd(g), v>.
* The whole backward pass against finite differences of the whole forward,
  separately for x and every weight, under several switch settings.
* The attention step against torch.autograd through torch's own
  scaled_dot_product_attention in fp64 (a library routine the step reduces
  to when the temperature is folded into q).
* Planted mistakes in the backward oracle must fail one of these pins.
"""

import math

import numpy as np
import pytest
import torch

import oracle.backward as BW
import oracle.cca as O
from synth import CCAShape, make_prefill, make_upstream_grad

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

H_FD = 1e-6


def case(B=2, T=6, E=10, Hq=4, Hkv=2, d=4, base=100.0, seed=0, **kw):
    s = CCAShape(batch=B, seq_len=T, d_model=E, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                 rope_base=base, dtype="f32", **kw)
    P = make_prefill(s, seed)
    w = P.weights.f64()
    rng = np.random.default_rng(seed + 11)
    w["tau"] = rng.uniform(0.5, 2.0 * math.sqrt(d), size=Hq)
    dy = make_upstream_grad(s, seed).dy
    return s, P.x, w, dy


def fd_dir(f, args, i, v, h=H_FD):
    """Central difference of f along v in argument i (f returns a scalar)."""
    a_p = list(args); a_p[i] = args[i] + h * v
    a_m = list(args); a_m[i] = args[i] - h * v
    return (f(*a_p) - f(*a_m)) / (2 * h)


def check_dir(f, args, grads, rng, tol=1e-6, ntries=2):
    """<grad_i, v> against the finite difference for each argument i."""
    for i, g in enumerate(grads):
        if g is None:
            continue
        for _ in range(ntries):
            v = rng.standard_normal(np.shape(args[i]))
            num = fd_dir(f, args, i, v)
            ana = float(np.sum(g * v))
            scale = max(abs(num), abs(ana), 1e-3)
            assert abs(num - ana) <= tol * scale, (i, num, ana)


# ---------------------------------------------------------------------------
# step by step
# ---------------------------------------------------------------------------

def test_down_project_bwd():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 5, 6))
    eq, ekv = 8, 4
    w = rng.standard_normal((eq + 2 * ekv, 6))
    g = rng.standard_normal((2, 5, eq + 2 * ekv))

    def f(x, w):
        q, k, v = O.down_project(x, w, 2, 1, 4)
        z = np.concatenate([q.reshape(2, 5, -1), k.reshape(2, 5, -1), v.reshape(2, 5, -1)], -1)
        return float(np.sum(g * z))
    dx, dw = BW.down_project_bwd(x, w, g)
    check_dir(f, [x, w], [dx, dw], rng)


@pytest.mark.parametrize("ks,T", [(1, 5), (3, 6), (4, 3)])
def test_seq_conv_bwd(ks, T):
    rng = np.random.default_rng(ks)
    u = rng.standard_normal((2, T, 5)); taps = rng.standard_normal((5, ks))
    g = rng.standard_normal((2, T, 5))
    f = lambda u, taps: float(np.sum(g * O.seq_conv(u, taps)))
    du, dt = BW.seq_conv_bwd(u, taps, g)
    check_dir(f, [u, taps], [du, dt], rng)


@pytest.mark.parametrize("kc,d", [(1, 4), (3, 4), (4, 8), (3, 2)])
def test_chan_conv_bwd(kc, d):
    rng = np.random.default_rng(kc * 10 + d)
    a = rng.standard_normal((2, 3, 3, d)); taps = rng.standard_normal((3, kc))
    g = rng.standard_normal(a.shape)
    f = lambda a, taps: float(np.sum(g * O.chan_conv(a, taps)))
    da, dt = BW.chan_conv_bwd(a, taps, g)
    check_dir(f, [a, taps], [da, dt], rng)


@pytest.mark.parametrize("reading", ["M1", "M2"])
@pytest.mark.parametrize("G", [1, 3])
def test_qk_mean_bwd(reading, G):
    rng = np.random.default_rng(G)
    r = O.Readings(qk_mean=reading)
    Hkv, d = 2, 4
    bq = rng.standard_normal((2, 5, Hkv * G, d)); qp = rng.standard_normal(bq.shape)
    bk = rng.standard_normal((2, 5, Hkv, d)); kp = rng.standard_normal(bk.shape)
    gq = rng.standard_normal(bq.shape); gk = rng.standard_normal(bk.shape)

    def f(bq, bk, qp, kp):
        q, k = O.qk_mean(bq, bk, qp, kp, G, r)
        return float(np.sum(gq * q) + np.sum(gk * k))
    grads = BW.qk_mean_bwd(gq, gk, G, r)
    check_dir(f, [bq, bk, qp, kp], list(grads), rng)


@pytest.mark.parametrize("half", ["upper", "lower"])
def test_value_shift_bwd(half):
    rng = np.random.default_rng(5)
    r = O.Readings(shift_half=half)
    v = rng.standard_normal((2, 5, 4, 3)); g = rng.standard_normal(v.shape)
    f = lambda v: float(np.sum(g * O.value_shift(v, None, r)))
    check_dir(f, [v], [BW.value_shift_bwd(g, r)], rng)


def test_l2_normalize_bwd():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 4, 8))
    x[0, 0] *= 1e-3                       # below eps: the divisor is the constant eps
    x[1, 2] *= 1e-9
    eps = 0.05
    g = rng.standard_normal(x.shape)
    f = lambda x: float(np.sum(g * O.l2_normalize(x, eps)))
    check_dir(f, [x], [BW.l2_normalize_bwd(x, g, eps)], rng)


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_rope_bwd(pairing):
    rng = np.random.default_rng(7)
    r = O.Readings(rope_pairing=pairing)
    x = rng.standard_normal((2, 6, 3, 8)); g = rng.standard_normal(x.shape)
    pos = np.arange(6) + 3
    f = lambda x: float(np.sum(g * O.rope(x, pos, 50.0, r)))
    check_dir(f, [x], [BW.rope_bwd(g, pos, 50.0, r)], rng)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (3, 1)])
def test_causal_attention_bwd(Hq, Hkv):
    rng = np.random.default_rng(Hq * 3 + Hkv)
    B, T, d = 2, 7, 4
    q = rng.standard_normal((B, T, Hq, d)); k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d)); tau = rng.uniform(0.3, 2.0, size=Hq)
    g = rng.standard_normal((B, T, Hq, d))

    def f(q, k, v, tau):
        return float(np.sum(g * O.causal_attention(q, k, v, tau, np.arange(T))))
    dq, dk, dv, dtau = BW.causal_attention_bwd(q, k, v, tau, g, block=3)
    check_dir(f, [q, k, v, tau], [dq, dk, dv, dtau], rng)


def test_up_project_bwd():
    rng = np.random.default_rng(8)
    o = rng.standard_normal((2, 5, 3, 4)); w = rng.standard_normal((7, 12))
    g = rng.standard_normal((2, 5, 7))
    f = lambda o, w: float(np.sum(g * O.up_project(o, w)))
    do, dw = BW.up_project_bwd(o, w, g)
    check_dir(f, [o, w], [do, dw], rng)


# ---------------------------------------------------------------------------
# the library routine: torch's attention and autograd, fp64 on the CPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_attention_bwd_matches_torch_autograd(Hq, Hkv):
    rng = np.random.default_rng(21)
    B, T, d = 2, 9, 8
    G = Hq // Hkv
    q = rng.standard_normal((B, T, Hq, d)); k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d)); tau = rng.uniform(0.3, 2.0, size=Hq)
    g = rng.standard_normal((B, T, Hq, d))
    tq = torch.tensor(q, requires_grad=True); tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True); tt = torch.tensor(tau, requires_grad=True)
    qs = (tq * tt[None, None, :, None]).transpose(1, 2)
    kr = tk.repeat_interleave(G, dim=2).transpose(1, 2)
    vr = tv.repeat_interleave(G, dim=2).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qs, kr, vr, is_causal=True, scale=1.0)
    (o.transpose(1, 2) * torch.tensor(g)).sum().backward()
    dq, dk, dv, dtau = BW.causal_attention_bwd(q, k, v, tau, g)
    for a, b in [(dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (dtau, tt.grad)]:
        b = b.numpy()
        assert np.linalg.norm(a - b) <= 1e-12 * np.linalg.norm(b)


# ---------------------------------------------------------------------------
# the whole pass
# ---------------------------------------------------------------------------

WHOLE = [
    dict(),                                                       # every switch on, G = 2
    dict(Hq=2, Hkv=2),                                            # CCA (G = 1)
    dict(Hq=4, Hkv=1, use_value_shift=0),                         # one wide group
    dict(use_qk_mean=0, use_value_shift=0, use_qk_norm=0, base=0.0),
    dict(seq_conv_k=1, chan_conv_k=1, d=8),
    dict(seq_conv_k=4, chan_conv_k=4, T=5, d=8, E=8),
]


@pytest.mark.parametrize("kw", WHOLE)
def test_whole_backward_finite_differences(kw):
    s, x, w, dy = case(**kw)
    grads = BW.prefill_backward(x, w, s, dy)
    rng = np.random.default_rng(99)
    names = ["x"] + list(w.keys())

    def loss(*vals):
        xx = vals[0]
        ww = dict(zip(w.keys(), vals[1:]))
        return BW.prefill_loss(xx, ww, s, dy)
    args = [x] + [w[k] for k in w]
    check_dir(loss, args, [grads[n] for n in names], rng, tol=2e-6)


def test_whole_backward_reading_m2():
    s, x, w, dy = case()
    r = O.Readings(qk_mean="M2")
    grads = BW.prefill_backward(x, w, s, dy, readings=r)
    rng = np.random.default_rng(5)

    def loss(xx, wq):
        ww = dict(w); ww["w_qkv"] = wq
        return BW.prefill_loss(xx, ww, s, dy, readings=r)
    check_dir(loss, [x, w["w_qkv"]], [grads["x"], grads["w_qkv"]], rng, tol=2e-6)


def test_whole_backward_mha_reduction():
    """Mixing off, norm off, no RoPE: the layer is MHA in the latent space, so
    the gradient of x equals torch autograd through torch's SDPA."""
    s, x, w, dy = case(Hq=2, Hkv=2, use_qk_mean=0, use_value_shift=0, use_qk_norm=0, base=0.0,
                       seq_conv_k=1, chan_conv_k=1)
    w = dict(w)
    w["q_seq_taps"] = np.ones_like(w["q_seq_taps"]); w["k_seq_taps"] = np.ones_like(w["k_seq_taps"])
    w["q_chan_taps"] = np.ones_like(w["q_chan_taps"]); w["k_chan_taps"] = np.ones_like(w["k_chan_taps"])
    grads = BW.prefill_backward(x, w, s, dy)
    B, T, E = x.shape
    H, d = s.n_q_heads, s.head_dim
    tx = torch.tensor(x, requires_grad=True)
    wqkv = torch.tensor(w["w_qkv"]); wo = torch.tensor(w["w_o"]); tau = torch.tensor(w["tau"])
    z = tx @ wqkv.T
    q = z[..., :H * d].reshape(B, T, H, d) * tau[None, None, :, None]
    k = z[..., H * d:2 * H * d].reshape(B, T, H, d)
    v = z[..., 2 * H * d:].reshape(B, T, H, d)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=True, scale=1.0)
    y = o.transpose(1, 2).reshape(B, T, H * d) @ wo.T
    (y * torch.tensor(dy)).sum().backward()
    g = tx.grad.numpy()
    assert np.linalg.norm(grads["x"] - g) <= 1e-12 * np.linalg.norm(g)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

_ORIG = dict(seq_conv_bwd=BW.seq_conv_bwd, chan_conv_bwd=BW.chan_conv_bwd)


def _pins_hold():
    try:
        test_whole_backward_finite_differences(WHOLE[0])
        test_whole_backward_finite_differences(WHOLE[2])
    except AssertionError:
        return False
    return True


def _rope_bwd_forward_rotation(dr, pos, base, readings=O.DEFAULT_READINGS):
    return O.rope(dr, pos, base, readings)           # rotates the wrong way


def _qk_mean_bwd_no_group_division(dq, dk, group, readings=O.DEFAULT_READINGS):
    lead = dq.shape[:-2]
    Hkv, d = dk.shape[-2:]
    return (dq.copy(), dk.copy(), 0.5 * dq + 0.5 * np.repeat(dk, group, axis=-2),
            0.5 * dk + 0.5 * dq.reshape(*lead, Hkv, group, d).sum(axis=-2))


def _seq_conv_bwd_backwards_in_time(u, taps, da):
    B, T, C = u.shape
    du = np.zeros_like(u)
    for j in range(taps.shape[1]):
        du[:, j:, :] += taps[:, j] * da[:, :T - j, :]
    return du, _ORIG["seq_conv_bwd"](u, taps, da)[1]


def _value_shift_bwd_wrong_way(dv, readings=O.DEFAULT_READINGS):
    B, T, H, d = dv.shape
    sh = O.shifted_heads(H, readings)
    out = dv.copy()
    out[:, :, sh, :] = 0.0
    out[:, 1:, sh, :] = dv[:, :T - 1, sh, :]
    return out


def _l2_bwd_no_projection(x, dy, eps):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return dy / np.maximum(n, eps)


def _chan_conv_bwd_transposed_taps(a, taps, db):
    da, dt = _ORIG["chan_conv_bwd"](a, taps, db)
    return da, dt[:, ::-1].copy()


def _attention_bwd_no_rowsum(q, k, v, tau, do, block=512):
    """Softmax backward without the <do, o> subtraction (one head group)."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    qq = q.transpose(0, 2, 1, 3)
    kk = np.repeat(k, G, axis=2).transpose(0, 2, 1, 3)
    vv = np.repeat(v, G, axis=2).transpose(0, 2, 1, 3)
    gg = do.transpose(0, 2, 1, 3)
    raw = qq @ kk.transpose(0, 1, 3, 2)
    s = raw * tau[None, :, None, None]
    vis = np.tril(np.ones((T, T), bool))
    s = np.where(vis, s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    ds = p * (gg @ vv.transpose(0, 1, 3, 2))
    dq = (tau[None, :, None, None] * (ds @ kk)).transpose(0, 2, 1, 3)
    dk = (tau[None, :, None, None] * (ds.transpose(0, 1, 3, 2) @ qq)).transpose(0, 2, 1, 3)
    dv = (p.transpose(0, 1, 3, 2) @ gg).transpose(0, 2, 1, 3)
    dk = dk.reshape(B, T, Hkv, G, d).sum(3)
    dv = dv.reshape(B, T, Hkv, G, d).sum(3)
    return dq, dk, dv, np.sum(ds * np.where(vis, raw, 0.0), axis=(0, 2, 3))


MUTANTS = [
    ("rope_bwd", _rope_bwd_forward_rotation),
    ("qk_mean_bwd", _qk_mean_bwd_no_group_division),
    ("seq_conv_bwd", _seq_conv_bwd_backwards_in_time),
    ("value_shift_bwd", _value_shift_bwd_wrong_way),
    ("l2_normalize_bwd", _l2_bwd_no_projection),
    ("chan_conv_bwd", _chan_conv_bwd_transposed_taps),
    ("causal_attention_bwd", _attention_bwd_no_rowsum),
]


def test_pins_hold_unmutated():
    assert _pins_hold()


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, mutant, monkeypatch):
    monkeypatch.setattr(BW, name, mutant)
    assert not _pins_hold()
