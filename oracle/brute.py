"""Scalar brute-force twin of the oracle for tiny inputs (test infrastructure).

Written separately from ``oracle.cca`` from the same readings, with explicit
Python loops over every index and ``math`` functions, so that an indexing,
sign or transposition mistake in the vectorised oracle shows up as a
mismatch.  Same page citations as ``oracle.cca``: down-projection, sequence
and channel convolution, q-k-mean, value-shift, normalisation, RoPE, latent
attention and up-projection [GS-EN "2. Methodology"; GS-DE "2. Methodik";
EDG "How Compressed Convolutional Attention Works"; ABS].

Sizes: B <= 2, T <= 8, E <= 16, d <= 8 keep it under a second.
"""

from __future__ import annotations

import math


def _matvec(w, x):
    return [sum(w[r][c] * x[c] for c in range(len(x))) for r in range(len(w))]


def brute_prefill(x, w, cfg, chan_conv="per_head", qk_mean="M2"):
    """x: nested lists [B][T][E] (floats); w: dict of nested lists.
    ``chan_conv="grouped"`` takes the dense lag-by-channel reading of the
    channel convolution (weights ``q_chan_dense`` / ``k_chan_dense``
    [H][d_out][k_c][d_in]).  ``qk_mean``: "M2" adds the average of the four
    values q~, k~ (before the convolutions) and bq, bk (after them) to each
    convolved value; "M1" the average of q~ and k~ only.

    Returns y as nested lists [B][T][E]."""
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = Hq // Hkv
    ks, kc = cfg.seq_conv_k, cfg.chan_conv_k
    eq, ekv = Hq * d, Hkv * d
    B, T = len(x), len(x[0])
    half = Hkv // 2
    out = []
    for b in range(B):
        # projections, token by token
        z = [_matvec(w["w_qkv"], x[b][t]) for t in range(T)]
        qt = [[z[t][c] for c in range(eq)] for t in range(T)]
        kt = [[z[t][eq + c] for c in range(ekv)] for t in range(T)]
        vb = [[z[t][eq + ekv + c] for c in range(ekv)] for t in range(T)]

        def conv_seq(u, taps, C):
            a = [[0.0] * C for _ in range(T)]
            for t in range(T):
                for c in range(C):
                    acc = 0.0
                    for j in range(ks):
                        if t - j >= 0:
                            acc += taps[c][j] * u[t - j][c]
                    a[t][c] = acc
            return a

        def conv_chan(a, taps, H):
            r = [[0.0] * (H * d) for _ in range(T)]
            for t in range(T):
                for h in range(H):
                    for i in range(d):
                        acc = 0.0
                        for j in range(kc):
                            if i - j >= 0:
                                acc += taps[h][j] * a[t][h * d + i - j]
                        r[t][h * d + i] = acc
            return r

        def conv_grouped(a, dense, H):
            # b[t][h, i] = sum over lags j and input channels c of
            # dense[h][i][j][c] * a[t - j][h, c] (nothing before t = 0)
            r = [[0.0] * (H * d) for _ in range(T)]
            for t in range(T):
                for h in range(H):
                    for i in range(d):
                        acc = 0.0
                        for j in range(kc):
                            if t - j < 0:
                                continue
                            for c in range(d):
                                acc += dense[h][i][j][c] * a[t - j][h * d + c]
                        r[t][h * d + i] = acc
            return r

        if chan_conv == "grouped":
            bq = conv_grouped(conv_seq(qt, w["q_seq_taps"], eq), w["q_chan_dense"], Hq)
            bk = conv_grouped(conv_seq(kt, w["k_seq_taps"], ekv), w["k_chan_dense"], Hkv)
        else:
            bq = conv_chan(conv_seq(qt, w["q_seq_taps"], eq), w["q_chan_taps"], Hq)
            bk = conv_chan(conv_seq(kt, w["k_seq_taps"], ekv), w["k_chan_taps"], Hkv)

        q = [row[:] for row in bq]
        k = [row[:] for row in bk]
        if cfg.use_qk_mean:
            for t in range(T):
                for h in range(Hq):
                    g = h // G
                    for i in range(d):
                        qc, kc_ = h * d + i, g * d + i
                        if qk_mean == "M2":
                            mean = (qt[t][qc] + kt[t][kc_] + bq[t][qc] + bk[t][kc_]) / 4.0
                        else:
                            mean = (qt[t][qc] + kt[t][kc_]) / 2.0
                        q[t][qc] = bq[t][qc] + mean
                for g in range(Hkv):
                    for i in range(d):
                        # the group's query heads enter through their average
                        pre_q = sum(qt[t][(g * G + m) * d + i] for m in range(G)) / G
                        post_q = sum(bq[t][(g * G + m) * d + i] for m in range(G)) / G
                        kc_ = g * d + i
                        if qk_mean == "M2":
                            mean = (pre_q + kt[t][kc_] + post_q + bk[t][kc_]) / 4.0
                        else:
                            mean = (pre_q + kt[t][kc_]) / 2.0
                        k[t][kc_] = bk[t][kc_] + mean

        v = [[0.0] * ekv for _ in range(T)]
        for t in range(T):
            for g in range(Hkv):
                shifted = cfg.use_value_shift and g >= half
                for i in range(d):
                    if shifted:
                        v[t][g * d + i] = vb[t - 1][g * d + i] if t >= 1 else 0.0
                    else:
                        v[t][g * d + i] = vb[t][g * d + i]

        def norm_rope(u, H, t):
            res = [0.0] * (H * d)
            for h in range(H):
                vec = u[h * d:(h + 1) * d]
                if cfg.use_qk_norm:
                    nrm = math.sqrt(sum(e * e for e in vec))
                    vec = [e / max(nrm, cfg.norm_eps) for e in vec]
                for p in range(d // 2):
                    a0, a1 = vec[2 * p], vec[2 * p + 1]
                    if cfg.rope_base:
                        ang = t * cfg.rope_base ** (-(2.0 * p) / d)
                        c, s = math.cos(ang), math.sin(ang)
                    else:
                        c, s = 1.0, 0.0
                    res[h * d + 2 * p] = a0 * c - a1 * s
                    res[h * d + 2 * p + 1] = a0 * s + a1 * c
            return res

        qr = [norm_rope(q[t], Hq, t) for t in range(T)]
        kr = [norm_rope(k[t], Hkv, t) for t in range(T)]

        yb = []
        for t in range(T):
            o = [0.0] * eq
            for h in range(Hq):
                g = h // G
                sc = []
                for u in range(t + 1):
                    dot = 0.0
                    for i in range(d):
                        dot += qr[t][h * d + i] * kr[u][g * d + i]
                    sc.append(w["tau"][h] * dot)
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                den = sum(ex)
                for i in range(d):
                    o[h * d + i] = sum(ex[u] * v[u][g * d + i] for u in range(t + 1)) / den
            yb.append(_matvec(w["w_o"], o))
        out.append(yb)
    return out
