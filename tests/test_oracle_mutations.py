"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each mutant replaces one step of ``oracle.cca`` with a plausible mistake (a
wrong sign, index, direction, dropped term or swapped operand).  The test
runs the independent pins -- the scalar brute force, the textbook MHA
reduction and the single-token closed form -- and requires that one of them
notices.  The mistakes live only in this test, on the CPU.
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


def _pins_hold():
    """True when every pin passes with the oracle as currently bound."""
    ok = True
    s, x, w = _case()
    y = O.prefill(x, w, s)
    yb = np.array(brute_prefill(x.tolist(), {k: v.tolist() for k, v in w.items()}, s))
    ok &= np.linalg.norm(y - yb) <= 1e-12 * np.linalg.norm(yb)
    return bool(ok)


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
    q, k = _orig["qk_mean"](bq, bk, q_pre, 0 * k_pre, group, readings)
    return q, k + 0.5 * k_pre


def _qk_mean_wrong_group(bq, bk, q_pre, k_pre, group, readings=O.DEFAULT_READINGS):
    k_for_q = np.tile(k_pre, (1,) * (k_pre.ndim - 2) + (group, 1))
    lead = q_pre.shape[:-2]
    Hkv, d = k_pre.shape[-2:]
    qm = q_pre.reshape(*lead, Hkv, group, d).mean(axis=-2)
    return bq + 0.5 * (q_pre + k_for_q), bk + 0.5 * (k_pre + qm)


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
    "value-shift lower half": ("value_shift", _value_shift_lower),
    "value-shift looks ahead": ("value_shift", _value_shift_forward),
    "no normalisation": ("l2_normalize", _no_norm),
    "diagonal masked": ("causal_attention", _attn_strict_mask),
    "kv head h mod H_kv": ("causal_attention", _attn_tiled_groups),
    "k and v swapped": ("down_project", _down_project_swap_kv),
    "head-major flatten transposed": ("up_project", _up_project_transposed_heads),
}


def test_unmutated_pins_hold():
    assert _pins_hold()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    fn_name, bad = MUTANTS[name]
    monkeypatch.setattr(O, fn_name, bad)
    assert not _pins_hold(), f"planted mistake '{name}' passed every pin"
