"""Vectorised fp64 oracle of the CCA / CCGQA forward pass (test infrastructure).

Plain NumPy in float64, in the order the pages describe the method:

  down-projection -> sequence conv -> channel conv -> q-k-mean -> value-shift
  -> L2 norm with temperature -> RoPE -> causal softmax attention inside the
  latent heads (kv heads shared by groups of G query heads) -> up-projection.

Inputs are the exact values the GPU receives (bf16 or fp32 upcast to fp64), so
the only differences to the GPU are its roundings and summation order.

This module is test infrastructure: only the tests, the smoke check and the
benchmark's CPU baseline import it; the library never does.

Array conventions: tokens are ``[B, T, ...]``; latent heads are ``[..., H, d]``
with flat channel index ``h * d + i``; weights are ``[out, in]``.

Parity status of each step (see the tests under ``tests/test_oracle_*.py``):
pinned by closed forms, brute force, the MHA reduction and invariants; the
readings of the channel convolution, tau, the RoPE pair convention and the
shifted half are parity unpinned against the original paper (the pages fix
none of them); the q-k-mean follows the pages' wording (the mean of the pre-
and post-convolution q and k) and is pinned by the brute-force twin and
closed forms of that reading, not by a number from the paper.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


@dataclass(frozen=True)
class Readings:
    """Switches for the steps the pages leave open.

    qk_mean:       "M2" (default) the mean of the pre- and post-convolution q
                   and k, a quarter of their sum, added to the convolved q and
                   k; "M1" the mean of the pre-convolution q and k only.
    rope_pairing:  "interleaved" (default, pairs (2i, 2i+1)) or "half"
                   (pairs (i, i + d/2)).
    shift_half:    "upper" (default: kv heads H_kv/2 .. H_kv-1 take token t-1)
                   or "lower".
    chan_conv:     "per_head" (default: one k_c-tap filter per head sliding
                   along the channel index) or "grouped" (a k_c-lag causal
                   convolution over tokens that mixes all d channels of a
                   head, weights ``q_chan_dense`` / ``k_chan_dense``).  With
                   "grouped" the carried decode window holds the last
                   (k_s - 1) + (k_c - 1) pre-conv rows.
    """
    qk_mean: str = "M2"
    rope_pairing: str = "interleaved"
    shift_half: str = "upper"
    chan_conv: str = "per_head"


DEFAULT_READINGS = Readings()


# ---------------------------------------------------------------------------
# a1  down-projection  [GS-EN "2. Methodology" / Down-Projection;
#     GS-DE "2. Methodik" / Down-Projektion; ABS]
# Three learnable matrices map width E to the latent; no bias.  The three are
# stored stacked as one [e_q + 2 e_kv, E] matrix (rows q | k | v).
# ---------------------------------------------------------------------------

def down_project(x: np.ndarray, w_qkv: np.ndarray, n_q_heads: int, n_kv_heads: int,
                 head_dim: int):
    """x [..., E] -> (q~ [..., H_q, d], k~ [..., H_kv, d], vbar [..., H_kv, d])."""
    eq, ekv = n_q_heads * head_dim, n_kv_heads * head_dim
    z = x @ w_qkv.T
    lead = z.shape[:-1]
    q = z[..., :eq].reshape(*lead, n_q_heads, head_dim)
    k = z[..., eq:eq + ekv].reshape(*lead, n_kv_heads, head_dim)
    v = z[..., eq + ekv:].reshape(*lead, n_kv_heads, head_dim)
    return q, k, v


# ---------------------------------------------------------------------------
# a2  causal sequence convolution  [GS-EN "2. Methodology" / Convolutional
#     Mixing; EDG "How Compressed Convolutional Attention Works"]
# Depthwise along the token axis, one k_s-tap filter per latent channel, taps
# indexed by lag: a[t, c] = sum_j w[c, j] * u[t - j, c], with u = 0 before the
# sequence start (or the carried window in decode).
# ---------------------------------------------------------------------------

def seq_conv(u: np.ndarray, taps: np.ndarray, history: Optional[np.ndarray] = None):
    """u [B, T, C], taps [C, k_s], history [B, k_s-1, C] (slot 0 oldest) -> [B, T, C]."""
    B, T, C = u.shape
    ks = taps.shape[1]
    if history is None:
        history = np.zeros((B, ks - 1, C), dtype=u.dtype)
    ext = np.concatenate([history, u], axis=1)      # ext[:, t + ks - 1] = u[:, t]
    out = np.zeros_like(u)
    for j in range(ks):
        out += taps[:, j] * ext[:, ks - 1 - j: ks - 1 - j + T, :]
    return out


# ---------------------------------------------------------------------------
# a3  channel convolution  [GS-EN "2. Methodology" / Convolutional Mixing;
#     GS-DE "2. Methodik" / Faltungen]
# Reading (parity unpinned): one k_c-tap filter per head that slides along the
# head's channel index, taps indexed by lag, zero padding inside the head:
# b[t, h, i] = sum_j w[h, j] * a[t, h, i - j].
# ---------------------------------------------------------------------------

def chan_conv(a: np.ndarray, taps: np.ndarray):
    """a [..., H, d], taps [H, k_c] -> [..., H, d]."""
    d = a.shape[-1]
    out = np.zeros_like(a)
    for j in range(min(taps.shape[1], d)):
        out[..., j:] += taps[:, j][:, None] * a[..., :d - j]
    return out


# Alternative reading of a3 (parity unpinned, selected by Readings.chan_conv
# = "grouped"): the channel dimension is mixed by a dense d x d matrix per lag
# and head, a causal convolution over tokens grouped by head:
# b[t, h, i] = sum_j sum_c W[h, i, j, c] * a[t - j, h, c], a = 0 before the
# sequence start (or the carried values in decode).
# ---------------------------------------------------------------------------

def chan_conv_grouped(a: np.ndarray, w: np.ndarray, history: Optional[np.ndarray] = None):
    """a [B, T, H, d], w [H, d_out, k_c, d_in], history [B, k_c-1, H, d]
    (a of the tokens before t = 0, slot 0 oldest) -> [B, T, H, d]."""
    B, T, H, d = a.shape
    kc = w.shape[2]
    if history is None:
        history = np.zeros((B, kc - 1, H, d), dtype=a.dtype)
    ext = np.concatenate([history, a], axis=1)       # ext[:, t + kc - 1] = a[:, t]
    out = np.zeros_like(a)
    for j in range(kc):
        lagged = ext[:, kc - 1 - j: kc - 1 - j + T]  # a[t - j]
        out += np.einsum("hic,bthc->bthi", w[:, :, j, :], lagged)
    return out


def conv_window_rows(cfg, readings: "Readings" = None) -> int:
    """Pre-conv rows the decode state carries: k_s - 1, plus k_c - 1 under
    the grouped channel conv (its lagged inputs a[t-j] need them)."""
    readings = DEFAULT_READINGS if readings is None else readings
    extra = cfg.chan_conv_k - 1 if readings.chan_conv == "grouped" else 0
    return cfg.seq_conv_k - 1 + extra


# ---------------------------------------------------------------------------
# a4  q-k-mean  [GS-EN "2. Methodology" / Q-K-Mean; EDG "How Compressed
#     Convolutional Attention Works"; GS-DE "2. Methodik" / Q-K-Mean]
# All three pages describe one operation: the mean of the query and key
# values taken before and after the convolutions is added back to the
# convolved tensors, a skip path that lets q and k share information.
# Reading M2 (the default; parity unpinned against the paper itself): the
# mean of the four tensors q~, k~ (pre-conv) and b_q, b_k (post-conv),
#   m = (q~ + k~ + b_q + b_k) / 4,   q = b_q + m,   k = b_k + m.
# With G query heads per kv head (CCGQA) q head h meets the k~ and b_k of its
# group g(h) = floor(h / G), and kv head g meets the averages of q~ and b_q
# over its G query heads.  Reading M1 (a switch) keeps only the pre-conv
# terms: q = b_q + (q~ + k~) / 2, k = b_k + (k~ + q~) / 2.
# ---------------------------------------------------------------------------

def qk_mean(bq, bk, q_pre, k_pre, group: int, readings: Readings = DEFAULT_READINGS):
    """bq, q_pre [..., H_q, d]; bk, k_pre [..., H_kv, d] -> (q, k)."""
    k_for_q = np.repeat(k_pre, group, axis=-2)                       # [..., H_q, d]
    lead = q_pre.shape[:-2]
    Hkv, d = k_pre.shape[-2:]
    q_grp_mean = q_pre.reshape(*lead, Hkv, group, d).mean(axis=-2)  # [..., H_kv, d]
    if readings.qk_mean == "M1":
        return bq + 0.5 * (q_pre + k_for_q), bk + 0.5 * (k_pre + q_grp_mean)
    if readings.qk_mean == "M2":
        bk_for_q = np.repeat(bk, group, axis=-2)
        bq_grp_mean = bq.reshape(*lead, Hkv, group, d).mean(axis=-2)
        q = bq + 0.25 * (q_pre + k_for_q + bq + bk_for_q)
        k = bk + 0.25 * (k_pre + q_grp_mean + bk + bq_grp_mean)
        return q, k
    raise ValueError(readings.qk_mean)


# ---------------------------------------------------------------------------
# a5  value-shift  [GS-EN "2. Methodology" / Value-Shift; EDG "How Compressed
#     Convolutional Attention Works"; GS-DE "2. Methodik" / Value-Shift]
# Half of the value heads take the previous token's projected value, so they
# cannot see the present token (zero before the sequence start, or the
# carried value in decode).  Which half: the upper one (a labelling choice).
# ---------------------------------------------------------------------------

def shifted_heads(n_kv_heads: int, readings: Readings = DEFAULT_READINGS):
    h2 = n_kv_heads // 2
    if readings.shift_half == "upper":
        return list(range(h2, n_kv_heads))
    return list(range(0, h2))


def value_shift(vbar: np.ndarray, prev: Optional[np.ndarray] = None,
                readings: Readings = DEFAULT_READINGS):
    """vbar [B, T, H_kv, d]; prev [B, H_kv/2, d] = vbar of the token before t=0."""
    B, T, H, d = vbar.shape
    sh = shifted_heads(H, readings)
    v = vbar.copy()
    before = np.zeros((B, len(sh), d)) if prev is None else prev
    v[:, 0, sh, :] = before
    v[:, 1:, sh, :] = vbar[:, :-1, sh, :]
    return v


# ---------------------------------------------------------------------------
# a6  L2 normalisation + temperature  [GS-EN "2. Methodology" / Q-K-Mean
#     mentions the normalisation; the per-head temperature tau_h scales the
#     logits.  Reading: x / max(||x||_2, eps) per head.]
# ---------------------------------------------------------------------------

def l2_normalize(x: np.ndarray, eps: float):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


# ---------------------------------------------------------------------------
# a7  RoPE on the latent q and k  [GS-EN "2. Methodology" / RoPE Integration;
#     GS-DE "2. Methodik" / Integration von RoPE; EDG]
# Rotary embedding over all d channels of each latent head, position = token
# index from 0, frequency of pair i = base^(-2i/d), angles in fp64.
# Reading (parity unpinned): pairs (2i, 2i+1) as in RoFormer.
# ---------------------------------------------------------------------------

def rope_angles(pos: np.ndarray, head_dim: int, base: float):
    """pos [T] -> angles [T, d/2] in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, pos: np.ndarray, base: float,
         readings: Readings = DEFAULT_READINGS):
    """x [B, T, H, d] rotated at positions pos [T]."""
    if base == 0:
        return x.copy()
    d = x.shape[-1]
    ang = rope_angles(pos, d, base)                    # [T, d/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    out = np.empty_like(x)
    if readings.rope_pairing == "interleaved":
        x0, x1 = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = x0 * c - x1 * s
        out[..., 1::2] = x0 * s + x1 * c
    elif readings.rope_pairing == "half":
        h = d // 2
        x0, x1 = x[..., :h], x[..., h:]
        out[..., :h] = x0 * c - x1 * s
        out[..., h:] = x0 * s + x1 * c
    else:
        raise ValueError(readings.rope_pairing)
    return out


# ---------------------------------------------------------------------------
# a8  causal softmax attention inside the latent heads  [GS-EN "2. Methodology"
#     / Latent Space Operations and "Extension: CCGQA"; GS-DE "2. Methodik" /
#     Attention im latenten Raum; ABS]
# s[t, u] = tau_h <q_h(t), k_g(u)> for u <= pos(t), g = floor(h / G), softmax
# over u with the max subtracted, o = sum_u p v.  No dropout, bias or window.
# ---------------------------------------------------------------------------

def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: np.ndarray,
                     q_pos: Sequence[int], block: int = 512):
    """q [B, Tq, H_q, d] at positions q_pos; k, v [B, Tk, H_kv, d] at 0..Tk-1.

    Returns o [B, Tq, H_q, d].  Query rows are processed in blocks so long
    sequences fit in memory; each row sees keys 0..q_pos[row]."""
    B, Tq, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    q_pos = np.asarray(q_pos)
    o = np.zeros_like(q)
    kk = np.repeat(k, G, axis=2).transpose(0, 2, 1, 3)   # [B, H_q, Tk, d]
    vv = np.repeat(v, G, axis=2).transpose(0, 2, 1, 3)
    qq = q.transpose(0, 2, 1, 3)                          # [B, H_q, Tq, d]
    for r0 in range(0, Tq, block):
        r1 = min(Tq, r0 + block)
        kmax = int(q_pos[r0:r1].max()) + 1
        s = qq[:, :, r0:r1, :] @ kk[:, :, :kmax, :].transpose(0, 1, 3, 2)
        s = s * tau[None, :, None, None]
        vis = np.arange(kmax)[None, :] <= q_pos[r0:r1, None]  # [rows, kmax]
        s = np.where(vis[None, None], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        o[:, r0:r1, :, :] = (p @ vv[:, :, :kmax, :]).transpose(0, 2, 1, 3)
    return o


# ---------------------------------------------------------------------------
# a9  up-projection  (the latent output returns to width E after attention:
#     GS-EN "2. Methodology" / Latent Space Operations says it is not done
#     before attention).  y = o W_o^T with o flattened head-major; no bias.
# ---------------------------------------------------------------------------

def up_project(o: np.ndarray, w_o: np.ndarray):
    lead = o.shape[:-2]
    return o.reshape(*lead, -1) @ w_o.T


# ---------------------------------------------------------------------------
# composite passes
# ---------------------------------------------------------------------------

def latents(x, w, cfg, pos0: int = 0, history=None, readings: Readings = DEFAULT_READINGS):
    """Steps a1-a7 for tokens x [B, T, E] at positions pos0 .. pos0+T-1.

    ``w`` holds float64 weights (keys of ``synth.Weights.f64()``), ``cfg`` a
    shape with the method switches.  ``history`` = (conv_q [B, W, e_q],
    conv_k [B, W, e_kv], vshift [B, H_kv/2, d]) of the tokens before pos0,
    W = conv_window_rows(cfg, readings).  Returns a dict of every
    intermediate."""
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    B, T, _ = x.shape
    G = Hq // Hkv
    qt, kt, vbar = down_project(x, w["w_qkv"], Hq, Hkv, d)
    hq = hk = hv = None
    if history is not None:
        hq, hk, hv = history
    if readings.chan_conv == "grouped":
        # a over the carried rows and the new ones; the rows before the first
        # k_s - 1 carried ones are unknown, so the first k_s - 1 results are
        # dropped and the next k_c - 1 are the lagged inputs of the first token
        W = conv_window_rows(cfg, readings)
        ks1, kc1 = cfg.seq_conv_k - 1, cfg.chan_conv_k - 1

        def grouped(pre, hist, seq_taps, dense, H):
            hist = np.zeros((B, W, H * d)) if hist is None else hist
            ext = np.concatenate([hist, pre.reshape(B, T, H * d)], axis=1)
            a_ext = seq_conv(ext, seq_taps).reshape(B, W + T, H, d)
            a_hist = a_ext[:, ks1:ks1 + kc1]
            a = a_ext[:, W:]
            return a, chan_conv_grouped(a, dense, a_hist)

        a_q, b_q = grouped(qt, hq, w["q_seq_taps"], w["q_chan_dense"], Hq)
        a_k, b_k = grouped(kt, hk, w["k_seq_taps"], w["k_chan_dense"], Hkv)
    elif readings.chan_conv == "per_head":
        a_q = seq_conv(qt.reshape(B, T, Hq * d), w["q_seq_taps"], hq).reshape(B, T, Hq, d)
        a_k = seq_conv(kt.reshape(B, T, Hkv * d), w["k_seq_taps"], hk).reshape(B, T, Hkv, d)
        b_q = chan_conv(a_q, w["q_chan_taps"])
        b_k = chan_conv(a_k, w["k_chan_taps"])
    else:
        raise ValueError(readings.chan_conv)
    if cfg.use_qk_mean:
        m_q, m_k = qk_mean(b_q, b_k, qt, kt, G, readings)
    else:
        m_q, m_k = b_q, b_k
    if cfg.use_value_shift:
        v = value_shift(vbar, hv, readings)
    else:
        v = vbar
    if cfg.use_qk_norm:
        n_q, n_k = l2_normalize(m_q, cfg.norm_eps), l2_normalize(m_k, cfg.norm_eps)
    else:
        n_q, n_k = m_q, m_k
    pos = np.arange(pos0, pos0 + T)
    r_q = rope(n_q, pos, cfg.rope_base, readings)
    r_k = rope(n_k, pos, cfg.rope_base, readings)
    return dict(q_pre=qt, k_pre=kt, vbar=vbar, q_conv=b_q, k_conv=b_k,
                q_mix=m_q, k_mix=m_k, q=r_q, k=r_k, v=v)


def prefill(x, w, cfg, rows: Optional[Sequence[int]] = None,
            readings: Readings = DEFAULT_READINGS, intermediates: bool = False):
    """Whole forward pass over x [B, T, E].

    ``rows``: optional sorted token positions whose outputs are wanted (the
    latents are still computed for every token, attention only for ``rows``).
    Returns y [B, T or len(rows), E] (and the intermediates if asked)."""
    lat = latents(x, w, cfg, readings=readings)
    T = x.shape[1]
    q_pos = np.arange(T) if rows is None else np.asarray(rows)
    o = causal_attention(lat["q"][:, q_pos], lat["k"], lat["v"], w["tau"], q_pos)
    y = up_project(o, w["w_o"])
    if intermediates:
        lat["o"] = o
        lat["y"] = y
        return y, lat
    return y


def prefill_state(lat: dict, cfg, readings: Readings = DEFAULT_READINGS):
    """Decode state after a prefill: (K cache, V cache, conv_q, conv_k, vshift).

    K holds the normalised, rotated k (tau not folded in), V the post-shift v,
    both [B, H_kv, T, d]; the convolution window holds the pre-conv q~, k~ of
    the last k_s - 1 tokens (slot 0 oldest, zeros before the sequence start);
    vshift holds vbar of the last token on the shifted heads.  Under the
    grouped channel conv the window holds conv_window_rows() tokens."""
    B, T = lat["q_pre"].shape[:2]
    ks1 = conv_window_rows(cfg, readings)
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    cq = np.zeros((B, ks1, Hq * d))
    ck = np.zeros((B, ks1, Hkv * d))
    for s in range(ks1):
        t = T - ks1 + s
        if t >= 0:
            cq[:, s] = lat["q_pre"][:, t].reshape(B, -1)
            ck[:, s] = lat["k_pre"][:, t].reshape(B, -1)
    sh = shifted_heads(Hkv, readings)
    vs = lat["vbar"][:, T - 1][:, sh, :]
    return (lat["k"].transpose(0, 2, 1, 3).copy(), lat["v"].transpose(0, 2, 1, 3).copy(),
            cq, ck, vs)


def decode_step(x_t, w, cfg, k_cache, v_cache, conv_q, conv_k, vshift,
                readings: Readings = DEFAULT_READINGS):
    """One token per sequence against a cache of L = k_cache.shape[2] past tokens.

    x_t [B, E]; k_cache, v_cache [B, H_kv, L, d]; conv_q [B, W, e_q];
    conv_k [B, W, e_kv] (W = conv_window_rows(cfg, readings)); vshift
    [B, H_kv/2, d].
    The new token sits at position L: steps a1-a7 run there with the carried
    window, its k and v are appended at cache index L, attention runs over the
    L + 1 keys, then the up-projection.  Returns (y_t [B, E], dict with the new
    k row, v row [B, H_kv, d], q [B, H_q, d] and the rolled state)."""
    B = x_t.shape[0]
    L = k_cache.shape[2]
    lat = latents(x_t[:, None, :], w, cfg, pos0=L, history=(conv_q, conv_k, vshift),
                  readings=readings)
    k_new = lat["k"][:, 0]                    # [B, H_kv, d]
    v_new = lat["v"][:, 0]
    kk = np.concatenate([k_cache, k_new[:, :, None, :]], axis=2).transpose(0, 2, 1, 3)
    vv = np.concatenate([v_cache, v_new[:, :, None, :]], axis=2).transpose(0, 2, 1, 3)
    o = causal_attention(lat["q"], kk, vv, w["tau"], [L])
    y = up_project(o, w["w_o"])[:, 0]
    W = conv_window_rows(cfg, readings)
    cq_all = np.concatenate([conv_q, lat["q_pre"].reshape(B, 1, -1)], axis=1)
    ck_all = np.concatenate([conv_k, lat["k_pre"].reshape(B, 1, -1)], axis=1)
    new_cq, new_ck = cq_all[:, cq_all.shape[1] - W:], ck_all[:, ck_all.shape[1] - W:]
    sh = shifted_heads(cfg.n_kv_heads, readings)
    new_vs = lat["vbar"][:, 0][:, sh, :]
    return y, dict(k_new=k_new, v_new=v_new, q=lat["q"][:, 0], o=o[:, 0],
                   conv_q=new_cq, conv_k=new_ck, vshift=new_vs)


def decode_multi(x_new, w, cfg, k_cache, v_cache, conv_q, conv_k, vshift,
                 readings: Readings = DEFAULT_READINGS):
    """m new tokens per sequence against a cache of L = k_cache.shape[2] past
    tokens (a speculative-verification or chunked step): x_new [B, m, E]; the
    new tokens sit at positions L .. L+m-1.  Steps a1-a7 run over the m tokens
    with the carried window (the same code path as a prefill that continues
    from that state), their k and v are appended at slots L .. L+m-1, query j
    attends to keys 0 .. L+j, then the up-projection.  Returns (y [B, m, E],
    dict with k_new, v_new [B, H_kv, m, d] and the rolled state)."""
    B, m, _ = x_new.shape
    L = k_cache.shape[2]
    lat = latents(x_new, w, cfg, pos0=L, history=(conv_q, conv_k, vshift), readings=readings)
    k_new = lat["k"].transpose(0, 2, 1, 3)            # [B, H_kv, m, d]
    v_new = lat["v"].transpose(0, 2, 1, 3)
    kk = np.concatenate([k_cache, k_new], axis=2).transpose(0, 2, 1, 3)
    vv = np.concatenate([v_cache, v_new], axis=2).transpose(0, 2, 1, 3)
    o = causal_attention(lat["q"], kk, vv, w["tau"], list(range(L, L + m)))
    y = up_project(o, w["w_o"])
    ks1 = conv_window_rows(cfg, readings)
    cq_all = np.concatenate([conv_q, lat["q_pre"].reshape(B, m, -1)], axis=1)
    ck_all = np.concatenate([conv_k, lat["k_pre"].reshape(B, m, -1)], axis=1)
    sh = shifted_heads(cfg.n_kv_heads, readings)
    return y, dict(k_new=k_new, v_new=v_new, q=lat["q"],
                   conv_q=cq_all[:, cq_all.shape[1] - ks1:], conv_k=ck_all[:, ck_all.shape[1] - ks1:],
                   vshift=lat["vbar"][:, -1][:, sh, :])
