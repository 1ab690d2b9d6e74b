"""fp64 oracle of the CCA / CCGQA backward pass (test infrastructure).

The pages define the forward pass and report that CCA also speeds up the
backward pass over MHA [GS-EN "3. Key Contributions"; EDG "How Compressed
Convolutional Attention Works"].  The backward pass is the derivative of
that forward pass, nothing more: every function below is the chain rule
applied to one step of ``oracle.cca`` and is named after it.  Steps run in
reverse order:

  up-projection -> causal attention -> RoPE -> L2 norm -> value-shift
  -> q-k-mean -> channel conv -> sequence conv -> down-projection.

Each function takes the forward step's inputs and the cotangent of its
output (``d*``: the gradient of a scalar loss with respect to that output)
and returns the cotangents of its inputs and parameters.  Plain NumPy in
float64, no blocking beyond the row blocks the forward attention also uses.

Pins (``tests/test_oracle_backward.py``): every step against central finite
differences of the forward oracle, the whole pass against finite
differences in each argument, and the attention step against
``torch.autograd`` through ``scaled_dot_product_attention`` in fp64.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import cca as F
from .cca import DEFAULT_READINGS, Readings


# ---------------------------------------------------------------------------
# a1 down-projection z = x W^T   (forward: oracle.cca.down_project)
# ---------------------------------------------------------------------------

def down_project_bwd(x: np.ndarray, w_qkv: np.ndarray, dz: np.ndarray):
    """x [..., E], dz [..., e_q + 2 e_kv] -> (dx [..., E], dw_qkv [e_q + 2 e_kv, E])."""
    E = x.shape[-1]
    dx = dz @ w_qkv
    dw = dz.reshape(-1, dz.shape[-1]).T @ x.reshape(-1, E)
    return dx, dw


# ---------------------------------------------------------------------------
# a2 causal sequence convolution a[t, c] = sum_j w[c, j] u[t - j, c]
# ---------------------------------------------------------------------------

def seq_conv_bwd(u: np.ndarray, taps: np.ndarray, da: np.ndarray):
    """u, da [B, T, C] (no carried history: prefill) -> (du [B, T, C], dtaps [C, k_s]).

    du[t, c] = sum_j w[c, j] da[t + j, c] for t + j < T;
    dtaps[c, j] = sum_{b, t >= j} da[t, c] u[t - j, c]."""
    B, T, C = u.shape
    du = np.zeros_like(u)
    dtaps = np.zeros_like(taps)
    for j in range(taps.shape[1]):
        if j >= T:
            continue
        du[:, :T - j, :] += taps[:, j] * da[:, j:, :]
        dtaps[:, j] = np.einsum("btc,btc->c", da[:, j:, :], u[:, :T - j, :])
    return du, dtaps


# ---------------------------------------------------------------------------
# a3 channel convolution b[t, h, i] = sum_j w[h, j] a[t, h, i - j]
# ---------------------------------------------------------------------------

def chan_conv_bwd(a: np.ndarray, taps: np.ndarray, db: np.ndarray):
    """a, db [..., H, d] -> (da [..., H, d], dtaps [H, k_c]).

    da[..., i] = sum_j w[h, j] db[..., i + j] for i + j < d;
    dtaps[h, j] = sum over tokens and i >= j of db[..., h, i] a[..., h, i - j]."""
    d = a.shape[-1]
    H = a.shape[-2]
    da = np.zeros_like(a)
    dtaps = np.zeros_like(taps)
    for j in range(min(taps.shape[1], d)):
        da[..., :d - j] += taps[:, j][:, None] * db[..., j:]
        prod = db[..., j:] * a[..., :d - j]
        dtaps[:, j] = prod.reshape(-1, H, d - j).sum(axis=(0, 2))
    return da, dtaps


# ---------------------------------------------------------------------------
# a4 q-k-mean (reading M1 or M2, as in oracle.cca.qk_mean)
# ---------------------------------------------------------------------------

def qk_mean_bwd(dq: np.ndarray, dk: np.ndarray, group: int,
                readings: Readings = DEFAULT_READINGS):
    """dq [..., H_q, d], dk [..., H_kv, d] ->
    (dbq, dbk, dq_pre, dk_pre) with the shapes of bq, bk, q_pre, k_pre.

    M1: q = bq + (q_pre + k_pre[g(h)]) / 2, k = bk + (k_pre + mean_g q_pre) / 2,
    so q_pre[h] collects dq[h] / 2 and dk[g(h)] / (2 G); k_pre[g] collects
    dk[g] / 2 and the sum of dq over the group / 2."""
    lead = dq.shape[:-2]
    Hq, d = dq.shape[-2:]
    Hkv = dk.shape[-2]
    dq_grp_sum = dq.reshape(*lead, Hkv, group, d).sum(axis=-2)      # [..., H_kv, d]
    dk_rep = np.repeat(dk, group, axis=-2)                            # [..., H_q, d]
    if readings.qk_mean == "M1":
        dq_pre = 0.5 * dq + 0.5 * dk_rep / group
        dk_pre = 0.5 * dk + 0.5 * dq_grp_sum
        return dq.copy(), dk.copy(), dq_pre, dk_pre
    if readings.qk_mean == "M2":
        # q = 1.25 bq + (q_pre + k_pre[g] + bk[g]) / 4,
        # k = 1.25 bk + (k_pre + mean q_pre + mean bq) / 4
        dbq = 1.25 * dq + 0.25 * dk_rep / group
        dbk = 1.25 * dk + 0.25 * dq_grp_sum
        dq_pre = 0.25 * dq + 0.25 * dk_rep / group
        dk_pre = 0.25 * dk + 0.25 * dq_grp_sum
        return dbq, dbk, dq_pre, dk_pre
    raise ValueError(readings.qk_mean)


# ---------------------------------------------------------------------------
# a5 value-shift: the shifted heads take the previous token's value
# ---------------------------------------------------------------------------

def value_shift_bwd(dv: np.ndarray, readings: Readings = DEFAULT_READINGS):
    """dv [B, T, H_kv, d] -> dvbar (prefill: nothing carried in)."""
    B, T, H, d = dv.shape
    sh = F.shifted_heads(H, readings)
    dvbar = dv.copy()
    dvbar[:, :, sh, :] = 0.0
    dvbar[:, :T - 1, sh, :] = dv[:, 1:, sh, :]
    return dvbar


# ---------------------------------------------------------------------------
# a6 L2 normalisation y = x / max(||x||, eps)
# ---------------------------------------------------------------------------

def l2_normalize_bwd(x: np.ndarray, dy: np.ndarray, eps: float):
    """x, dy [..., d] -> dx.  Where ||x|| > eps: (dy - y <y, dy>) / ||x||;
    elsewhere the divisor is the constant eps: dy / eps."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    big = n > eps
    y = x / np.where(big, n, 1.0)
    dx_big = (dy - y * np.sum(y * dy, axis=-1, keepdims=True)) / np.where(big, n, 1.0)
    return np.where(big, dx_big, dy / eps)


# ---------------------------------------------------------------------------
# a7 RoPE: a rotation per channel pair, so its transpose rotates back
# ---------------------------------------------------------------------------

def rope_bwd(dr: np.ndarray, pos: np.ndarray, base: float,
             readings: Readings = DEFAULT_READINGS):
    """dr [B, T, H, d] -> cotangent of the unrotated input."""
    if base == 0:
        return dr.copy()
    d = dr.shape[-1]
    ang = F.rope_angles(pos, d, base)
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    out = np.empty_like(dr)
    if readings.rope_pairing == "interleaved":
        g0, g1 = dr[..., 0::2], dr[..., 1::2]
        out[..., 0::2] = g0 * c + g1 * s
        out[..., 1::2] = -g0 * s + g1 * c
    elif readings.rope_pairing == "half":
        h = d // 2
        g0, g1 = dr[..., :h], dr[..., h:]
        out[..., :h] = g0 * c + g1 * s
        out[..., h:] = -g0 * s + g1 * c
    else:
        raise ValueError(readings.rope_pairing)
    return out


# ---------------------------------------------------------------------------
# a8 causal softmax attention (forward: oracle.cca.causal_attention with
#    q_pos = 0 .. T-1)
# ---------------------------------------------------------------------------

def causal_attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: np.ndarray,
                         do: np.ndarray, block: int = 512):
    """q [B, T, H_q, d], k, v [B, T, H_kv, d], do [B, T, H_q, d] ->
    (dq, dk, dv, dtau).

    With s = tau_h <q, k>, p = softmax over the visible keys and o = p v:
    dp = do v^T, ds = p (dp - <do, o>) (softmax's Jacobian), dq = tau ds k,
    dk = sum over the group's heads of tau ds^T q, dv = sum of p^T do, and
    dtau_h = sum of ds <q, k>."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    qq = q.transpose(0, 2, 1, 3)                          # [B, H_q, T, d]
    kk = np.repeat(k, G, axis=2).transpose(0, 2, 1, 3)
    vv = np.repeat(v, G, axis=2).transpose(0, 2, 1, 3)
    gg = do.transpose(0, 2, 1, 3)
    dqq = np.zeros_like(qq)
    dkk = np.zeros_like(kk)
    dvv = np.zeros_like(vv)
    dtau = np.zeros(Hq)
    t_all = np.arange(T)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        kmax = r1
        raw = qq[:, :, r0:r1, :] @ kk[:, :, :kmax, :].transpose(0, 1, 3, 2)   # <q, k>
        s = raw * tau[None, :, None, None]
        vis = t_all[None, :kmax] <= t_all[r0:r1, None]
        s = np.where(vis[None, None], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        o = p @ vv[:, :, :kmax, :]
        dp = gg[:, :, r0:r1, :] @ vv[:, :, :kmax, :].transpose(0, 1, 3, 2)
        dsum = np.sum(gg[:, :, r0:r1, :] * o, axis=-1, keepdims=True)
        ds = p * (dp - dsum)
        dqq[:, :, r0:r1, :] += tau[None, :, None, None] * (ds @ kk[:, :, :kmax, :])
        dkk[:, :, :kmax, :] += tau[None, :, None, None] * (ds.transpose(0, 1, 3, 2) @ qq[:, :, r0:r1, :])
        dvv[:, :, :kmax, :] += p.transpose(0, 1, 3, 2) @ gg[:, :, r0:r1, :]
        dtau += np.sum(ds * np.where(vis[None, None], raw, 0.0), axis=(0, 2, 3))
    dq = dqq.transpose(0, 2, 1, 3)
    dk = dkk.transpose(0, 2, 1, 3).reshape(B, T, Hkv, G, d).sum(axis=3)
    dv = dvv.transpose(0, 2, 1, 3).reshape(B, T, Hkv, G, d).sum(axis=3)
    return dq, dk, dv, dtau


# ---------------------------------------------------------------------------
# a9 up-projection y = o W_o^T
# ---------------------------------------------------------------------------

def up_project_bwd(o: np.ndarray, w_o: np.ndarray, dy: np.ndarray):
    """o [B, T, H_q, d], dy [B, T, E] -> (do [B, T, H_q, d], dw_o [E, e_q])."""
    lead = o.shape[:-2]
    of = o.reshape(*lead, -1)
    do = (dy @ w_o).reshape(o.shape)
    dw = dy.reshape(-1, dy.shape[-1]).T @ of.reshape(-1, of.shape[-1])
    return do, dw


# ---------------------------------------------------------------------------
# the whole backward pass of a prefill
# ---------------------------------------------------------------------------

def prefill_backward(x: np.ndarray, w: dict, cfg, dy: np.ndarray,
                     readings: Readings = DEFAULT_READINGS,
                     intermediates: bool = False):
    """Gradients of sum(dy * prefill(x)) with respect to x and every weight.

    Returns a dict with ``x`` [B, T, E] and the weight names of
    ``synth.Weights.f64()`` (``w_qkv``, ``w_o``, ``q_seq_taps``,
    ``k_seq_taps``, ``q_chan_taps``, ``k_chan_taps``, ``tau``), each the shape
    of its argument.  With ``intermediates`` also the cotangents of the
    latent q, k (rotated), v and of the mixed, pre-norm q and k."""
    if readings.chan_conv != "per_head":
        raise NotImplementedError("the backward follows the per-head channel conv reading")
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    B, T, E = x.shape
    G = Hq // Hkv
    _, lat = F.prefill(x, w, cfg, readings=readings, intermediates=True)
    pos = np.arange(T)

    do, dw_o = up_project_bwd(lat["o"], w["w_o"], dy)
    dq_r, dk_r, dv, dtau = causal_attention_bwd(lat["q"], lat["k"], lat["v"], w["tau"], do)

    dn_q = rope_bwd(dq_r, pos, cfg.rope_base, readings)
    dn_k = rope_bwd(dk_r, pos, cfg.rope_base, readings)
    if cfg.use_qk_norm:
        dm_q = l2_normalize_bwd(lat["q_mix"], dn_q, cfg.norm_eps)
        dm_k = l2_normalize_bwd(lat["k_mix"], dn_k, cfg.norm_eps)
    else:
        dm_q, dm_k = dn_q, dn_k

    if cfg.use_qk_mean:
        db_q, db_k, dq_pre, dk_pre = qk_mean_bwd(dm_q, dm_k, G, readings)
    else:
        db_q, db_k = dm_q, dm_k
        dq_pre, dk_pre = np.zeros_like(dm_q), np.zeros_like(dm_k)

    dvbar = value_shift_bwd(dv, readings) if cfg.use_value_shift else dv

    # channel conv: its input is the sequence conv's output
    a_q = F.seq_conv(lat["q_pre"].reshape(B, T, Hq * d), w["q_seq_taps"]).reshape(B, T, Hq, d)
    a_k = F.seq_conv(lat["k_pre"].reshape(B, T, Hkv * d), w["k_seq_taps"]).reshape(B, T, Hkv, d)
    da_q, dqc = chan_conv_bwd(a_q, w["q_chan_taps"], db_q)
    da_k, dkc = chan_conv_bwd(a_k, w["k_chan_taps"], db_k)

    du_q, dqs = seq_conv_bwd(lat["q_pre"].reshape(B, T, Hq * d), w["q_seq_taps"],
                             da_q.reshape(B, T, Hq * d))
    du_k, dks = seq_conv_bwd(lat["k_pre"].reshape(B, T, Hkv * d), w["k_seq_taps"],
                             da_k.reshape(B, T, Hkv * d))
    dq_pre = dq_pre.reshape(B, T, Hq * d) + du_q
    dk_pre = dk_pre.reshape(B, T, Hkv * d) + du_k

    dz = np.concatenate([dq_pre, dk_pre, dvbar.reshape(B, T, Hkv * d)], axis=-1)
    dx, dw_qkv = down_project_bwd(x, w["w_qkv"], dz)

    g = dict(x=dx, w_qkv=dw_qkv, w_o=dw_o, q_seq_taps=dqs, k_seq_taps=dks,
             q_chan_taps=dqc, k_chan_taps=dkc, tau=dtau)
    if intermediates:
        g.update(d_o=do, d_q_rot=dq_r, d_k_rot=dk_r, d_v=dv, d_q_mix=dm_q, d_k_mix=dm_k,
                 d_z=dz)
    return g


def prefill_loss(x: np.ndarray, w: dict, cfg, dy: np.ndarray,
                 readings: Readings = DEFAULT_READINGS) -> float:
    """sum(dy * prefill(x)): the scalar whose gradient prefill_backward returns."""
    return float(np.sum(dy * F.prefill(x, w, cfg, readings=readings)))
