"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each mutant replaces one step of ``oracle.cca`` with a plausible mistake (a
wrong sign, index, direction, dropped term, wrong coefficient or swapped
operand).  ``_pins_hold`` runs four independent pins -- the scalar brute
force, the textbook causal MHA reduction, the single-token closed form and
the closed form of the q-k-mean under scaled delta taps -- and every mutant
must make at least one of them fail.  Each pin also runs on the unmutated
oracle, where all four must hold.  The mistakes live only in this test, on
the CPU.
"""

import math

import numpy as np
import pytest

import oracle.cca as O
from oracle.brute import brute_prefill
from synth import CCAShape, make_prefill


def _case(Hq=4, Hkv=2, T=6, d=4, E=10, seed=3, **kw):
    s = CCAShape(batch=2, seq_len=T, d_model=E, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                 rope_base=100.0, dtype="f32", **kw)
    P = make_prefill(s, seed)
    w = P.weights.f64()
    w["tau"] = np.random.default_rng(seed).uniform(1.0, 4.0, size=Hq)
    return s, P.x, w


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def _delta(w, c=1.0, c2=1.0):
    w = dict(w)
    for name, scale in (("q_seq_taps", c), ("k_seq_taps", c), ("q_chan_taps", c2),
                        ("k_chan_taps", c2)):
        t = np.zeros_like(w[name])
        t[:, 0] = scale
        w[name] = t
    return w


def _pin_brute():
    s, x, w = _case()
    y = O.prefill(x, w, s)
    yb = np.array(brute_prefill(x.tolist(), {k: v.tolist() for k, v in w.items()}, s))
    return _rel(y, yb) <= 1e-12


def _pin_mha():
    """Compression 1, delta taps, extras off: textbook causal RoPE MHA with
    grouped kv heads, written here with explicit complex rotations."""
    Hq, Hkv, d, T, B, base = 4, 2, 4, 6, 2, 100.0
    s = CCAShape(batch=B, seq_len=T, d_model=Hq * d, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                 rope_base=base, dtype="f32", use_qk_mean=0, use_value_shift=0, use_qk_norm=0)
    P = make_prefill(s, 5)
    w = _delta(P.weights.f64())
    w["tau"] = np.full(Hq, 1.0 / math.sqrt(d))
    x = P.x
    eq, ekv, G = Hq * d, Hkv * d, Hq // Hkv
    Q = (x @ w["w_qkv"][:eq].T).reshape(B, T, Hq, d)
    K = (x @ w["w_qkv"][eq:eq + ekv].T).reshape(B, T, Hkv, d)
    V = (x @ w["w_qkv"][eq + ekv:].T).reshape(B, T, Hkv, d)
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    rot = np.exp(1j * np.outer(np.arange(T), theta))[None, :, None, :]

    def rope(u):
        z = (u[..., 0::2] + 1j * u[..., 1::2]) * rot
        r = np.empty_like(u)
        r[..., 0::2], r[..., 1::2] = z.real, z.imag
        return r
    Q, K = rope(Q), rope(K)
    o = np.zeros((B, T, Hq, d))
    for b in range(B):
        for h in range(Hq):
            S = Q[b, :, h] @ K[b, :, h // G].T / math.sqrt(d)
            S[np.triu_indices(T, 1)] = -np.inf
            p = np.exp(S - S.max(axis=1, keepdims=True))
            o[b, :, h] = (p / p.sum(axis=1, keepdims=True)) @ V[b, :, h // G]
    ref = o.reshape(B, T, eq) @ w["w_o"].T
    return _rel(O.prefill(x, w, s), ref) <= 1e-12


def _pin_single_token():
    """T = 1: o is the token's own value on unshifted kv heads, zero on the
    shifted (upper) ones, whatever q and k are."""
    s, x, w = _case(T=1)
    eq, ekv, d = s.e_q, s.e_kv, s.head_dim
    vbar = x[:, 0] @ w["w_qkv"][eq + ekv:].T
    vbar[:, d:] = 0.0
    o = np.repeat(vbar.reshape(2, 2, d), 2, axis=1).reshape(2, eq)
    return _rel(O.prefill(x, w, s)[:, 0], o @ w["w_o"].T) <= 1e-12


def _pin_qk_mean_closed_form():
    """Taps (c,0,0,0) and (c',0,0,0) make both convolutions a scaling by
    alpha = c c'; the mean of the pre- and post-convolution q and k then
    gives q = (alpha + (1+alpha)/4) q~ + ((1+alpha)/4) k~ per query head, and
    k = (alpha + (1+alpha)/4) k~ + ((1+alpha)/4) avg q~ per kv head."""
    s, x, w = _case(Hq=6, Hkv=2)
    s = s.with_(use_qk_norm=0, rope_base=0.0, use_value_shift=0)
    c, c2 = 1.5, -2.0
    w = _delta(w, c, c2)
    alpha = c * c2
    lat = O.latents(x, w, s)
    B, T, d, Hq, Hkv = 2, s.seq_len, s.head_dim, 6, 2
    G, eq, ekv = 3, s.e_q, s.e_kv
    qt = (x @ w["w_qkv"][:eq].T).reshape(B, T, Hq, d)
    kt = (x @ w["w_qkv"][eq:eq + ekv].T).reshape(B, T, Hkv, d)
    own, other = alpha + (1 + alpha) / 4, (1 + alpha) / 4
    ok = _rel(lat["q"], own * qt + other * kt[:, :, np.arange(Hq) // G]) <= 1e-12
    ok &= _rel(lat["k"], own * kt + other * qt.reshape(B, T, Hkv, G, d).mean(axis=3)) <= 1e-12
    return bool(ok)


PINS = (_pin_brute, _pin_mha, _pin_single_token, _pin_qk_mean_closed_form)


def _pins_hold():
    """True when every pin passes with the oracle as currently bound."""
    return all(bool(pin()) for pin in PINS)


def _rope_bad_sign(x, pos, base, readings=O.DEFAULT_READINGS):
    if base == 0:
        return x.copy()
    ang = O.rope_angles(pos, x.shape[-1], base)
    c, s = np.cos(ang)[None, :, None, :], np.sin(ang)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
    out[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _rope_bad_freq(x, pos, base, readings=O.DEFAULT_READINGS):
    d = x.shape[-1]
    i = np.arange(d // 2)
    ang = np.asarray(pos, float)[:, None] * base ** (-i / d)[None, :]
    c, s = np.cos(ang)[None, :, None, :], np.sin(ang)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _seq_conv_reversed_taps(u, taps, history=None):
    return _orig["seq_conv"](u, taps[:, ::-1].copy(), history)


def _seq_conv_anticausal(u, taps, history=None):
    B, T, C = u.shape
    out = np.zeros_like(u)
    for j in range(taps.shape[1]):
        out[:, :T - j] += taps[:, j] * u[:, j:]
    return out


def _chan_conv_wrong_direction(a, taps):
    d = a.shape[-1]
    out = np.zeros_like(a)
    for j in range(taps.shape[1]):
        out[..., :d - j] += taps[:, j][:, None] * a[..., j:]
    return out


def _qk_mean_drop_k(bq, bk, q_pre, k_pre, group, readings=O.DEFAULT_READINGS):
    # the query heads' mean forgets the key's pre-conv value
    q, _ = _orig["qk_mean"](bq, bk, q_pre, 0 * k_pre, group, readings)
    _, k = _orig["qk_mean"](bq, bk, q_pre, k_pre, group, readings)
    return q, k


def _qk_mean_wrong_group(bq, bk, q_pre, k_pre, group, readings=O.DEFAULT_READINGS):
    # query head h meets kv head h mod H_kv instead of h // G
    rep = lambda a: np.tile(a, (1,) * (a.ndim - 2) + (group, 1))
    lead = q_pre.shape[:-2]
    Hkv, d = k_pre.shape[-2:]
    mean = lambda a: a.reshape(*lead, Hkv, group, d).mean(axis=-2)
    return (bq + 0.25 * (q_pre + rep(k_pre) + bq + rep(bk)),
            bk + 0.25 * (k_pre + mean(q_pre) + bk + mean(bq)))


def _qk_mean_half_not_quarter(bq, bk, q_pre, k_pre, group, readings=O.DEFAULT_READINGS):
    # the four terms halved instead of averaged
    q, k = _orig["qk_mean"](bq, bk, q_pre, k_pre, group, readings)
    return 2 * q - bq, 2 * k - bk


def _qk_mean_first_head_not_group_mean(bq, bk, q_pre, k_pre, group, readings=O.DEFAULT_READINGS):
    # kv head g takes the post-conv q of the group's first head instead of the average
    lead = q_pre.shape[:-2]
    Hkv, d = k_pre.shape[-2:]
    mean = lambda a: a.reshape(*lead, Hkv, group, d).mean(axis=-2)
    first = bq.reshape(*lead, Hkv, group, d)[..., 0, :]
    q, _ = _orig["qk_mean"](bq, bk, q_pre, k_pre, group, readings)
    return q, bk + 0.25 * (k_pre + mean(q_pre) + bk + first)


def _qk_mean_pre_only(bq, bk, q_pre, k_pre, group, readings=O.DEFAULT_READINGS):
    # the other reading (pre-convolution mean only) in place of the default
    return _orig["qk_mean"](bq, bk, q_pre, k_pre, group, O.Readings(qk_mean="M1"))


def _value_shift_lower(vbar, prev=None, readings=O.DEFAULT_READINGS):
    return _orig["value_shift"](vbar, prev, O.Readings(shift_half="lower"))


def _value_shift_forward(vbar, prev=None, readings=O.DEFAULT_READINGS):
    H = vbar.shape[2]
    v = vbar.copy()
    v[:, :-1, H // 2:] = vbar[:, 1:, H // 2:]
    return v


def _no_norm(x, eps):
    return x


def _attn_strict_mask(q, k, v, tau, q_pos, block=512):
    qp = np.asarray(q_pos)
    o = _orig["causal_attention"](q, k, v, tau, np.maximum(qp - 1, 0), block)
    return o


def _attn_tiled_groups(q, k, v, tau, q_pos, block=512):
    G = q.shape[2] // k.shape[2]
    # kv head h % H_kv instead of h // G
    perm = np.arange(q.shape[2]).reshape(k.shape[2], G).T.ravel()
    inv = np.argsort(perm)
    o = _orig["causal_attention"](q[:, :, perm], k, v, tau[perm], q_pos, block)
    return o[:, :, inv]


def _down_project_swap_kv(x, w_qkv, Hq, Hkv, d):
    q, k, v = _orig["down_project"](x, w_qkv, Hq, Hkv, d)
    return q, v, k


def _up_project_transposed_heads(o, w_o):
    lead = o.shape[:-2]
    return o.swapaxes(-1, -2).reshape(*lead, -1) @ w_o.T


_orig = {n: getattr(O, n) for n in ("rope", "seq_conv", "chan_conv", "qk_mean", "value_shift",
                                     "l2_normalize", "causal_attention", "down_project",
                                     "up_project")}

MUTANTS = {
    "rope sign": ("rope", _rope_bad_sign),
    "rope frequency": ("rope", _rope_bad_freq),
    "seq conv reversed taps": ("seq_conv", _seq_conv_reversed_taps),
    "seq conv anti-causal": ("seq_conv", _seq_conv_anticausal),
    "chan conv direction": ("chan_conv", _chan_conv_wrong_direction),
    "q-k-mean drops k~": ("qk_mean", _qk_mean_drop_k),
    "q-k-mean wrong group": ("qk_mean", _qk_mean_wrong_group),
    "q-k-mean halves instead of averaging": ("qk_mean", _qk_mean_half_not_quarter),
    "q-k-mean first head not group mean": ("qk_mean", _qk_mean_first_head_not_group_mean),
    "q-k-mean pre-conv terms only": ("qk_mean", _qk_mean_pre_only),
    "value-shift lower half": ("value_shift", _value_shift_lower),
    "value-shift looks ahead": ("value_shift", _value_shift_forward),
    "no normalisation": ("l2_normalize", _no_norm),
    "diagonal masked": ("causal_attention", _attn_strict_mask),
    "kv head h mod H_kv": ("causal_attention", _attn_tiled_groups),
    "k and v swapped": ("down_project", _down_project_swap_kv),
    "head-major flatten transposed": ("up_project", _up_project_transposed_heads),
}


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_unmutated_pins_hold(pin):
    assert pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    fn_name, bad = MUTANTS[name]
    monkeypatch.setattr(O, fn_name, bad)
    assert not _pins_hold(), f"planted mistake '{name}' passed every pin"
