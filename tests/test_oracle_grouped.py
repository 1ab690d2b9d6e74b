"""Pins of the oracle's grouped channel-conv reading (Readings.chan_conv =
"grouped"): a k_c-lag causal convolution over tokens that mixes the d
channels of each head with a dense matrix per lag.  The pages only say that
1-D convolutions run across the sequence and the channel dimensions [GS-EN
"2. Methodology" / Convolutional Mixing], so the reading itself is parity
unpinned; these tests pin the oracle's arithmetic for it:

* the vectorised step against explicit loops, with weights that are not
  symmetric in (output, input) channel so a transposed matrix fails;
* the scalar twin (oracle.brute) against the vectorised forward end to end;
* special weights that reduce it to known operations: the identity (no
  channel mixing) and a diagonal per lag (a per-head depthwise temporal
  convolution, i.e. oracle.seq_conv with per-head taps);
* causality, and decode steps against the prefill over the same tokens
  (the carried window of (k_s - 1) + (k_c - 1) pre-conv rows).
"""

import numpy as np
import pytest

import oracle.cca as O
from oracle.brute import brute_prefill
from synth import CCAShape, add_chan_dense, make_prefill

GROUPED = O.Readings(chan_conv="grouped")


def _loops(a, w):
    B, T, H, d = a.shape
    kc = w.shape[2]
    out = np.zeros_like(a)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                for i in range(d):
                    acc = 0.0
                    for j in range(kc):
                        if t - j >= 0:
                            for c in range(d):
                                acc += w[h, i, j, c] * a[b, t - j, h, c]
                    out[b, t, h, i] = acc
    return out


@pytest.mark.parametrize("kc", [1, 2, 4])
def test_grouped_step_matches_loops(kc):
    rng = np.random.default_rng(kc)
    a = rng.standard_normal((2, 6, 3, 4))
    w = rng.standard_normal((3, 4, kc, 4))
    np.testing.assert_allclose(O.chan_conv_grouped(a, w), _loops(a, w), rtol=1e-12, atol=1e-12)
    # the test has power: the transposed matrix gives a different result
    assert not np.allclose(O.chan_conv_grouped(a, w.transpose(0, 3, 2, 1)), _loops(a, w))


def test_grouped_history_is_the_previous_tokens():
    """history = a of the k_c - 1 tokens before t = 0: the result over the
    last T tokens of a longer sequence equals the one computed with the
    earlier tokens passed as history."""
    rng = np.random.default_rng(3)
    a = rng.standard_normal((1, 9, 2, 4))
    w = rng.standard_normal((2, 4, 3, 4))
    full = O.chan_conv_grouped(a, w)
    part = O.chan_conv_grouped(a[:, 5:], w, history=a[:, 3:5])
    np.testing.assert_allclose(part, full[:, 5:], rtol=1e-12, atol=1e-12)


def _shape(**kw):
    base = dict(batch=2, seq_len=7, d_model=16, n_q_heads=2, n_kv_heads=2, head_dim=4,
                seq_conv_k=3, chan_conv_k=3, dtype="f32", rope_base=10000.0)
    base.update(kw)
    return CCAShape(**base)


def _weights(s, seed):
    P = make_prefill(s, seed=seed)
    add_chan_dense(P.weights, s, seed)
    return P, P.weights.f64()


@pytest.mark.parametrize("shape_kw", [dict(), dict(n_q_heads=4, n_kv_heads=2, chan_conv_k=2),
                                      dict(seq_conv_k=4, chan_conv_k=4, use_qk_mean=0)])
def test_grouped_forward_matches_brute(shape_kw):
    s = _shape(**shape_kw)
    P, w = _weights(s, seed=11)
    y = O.prefill(P.x, w, s, readings=GROUPED)
    yb = np.array(brute_prefill(P.x.tolist(), {k: v.tolist() for k, v in w.items()}, s,
                                chan_conv="grouped"))
    np.testing.assert_allclose(y, yb, rtol=1e-9, atol=1e-11)


def test_grouped_identity_is_no_channel_mixing():
    """W[h, i, 0, c] = [i == c], zero at the other lags: the channel step is
    the identity, as the per-head filter with taps (1, 0, ...) is."""
    s = _shape()
    P, w = _weights(s, seed=5)
    d, kc = s.head_dim, s.chan_conv_k
    eye = np.zeros((d, kc, d))
    eye[:, 0, :] = np.eye(d)
    w["q_chan_dense"] = np.broadcast_to(eye, (s.n_q_heads, d, kc, d)).copy()
    w["k_chan_dense"] = np.broadcast_to(eye, (s.n_kv_heads, d, kc, d)).copy()
    w["q_chan_taps"] = np.zeros_like(w["q_chan_taps"])
    w["k_chan_taps"] = np.zeros_like(w["k_chan_taps"])
    w["q_chan_taps"][:, 0] = 1.0
    w["k_chan_taps"][:, 0] = 1.0
    yg, lg = O.prefill(P.x, w, s, readings=GROUPED, intermediates=True)
    yp, lp = O.prefill(P.x, w, s, intermediates=True)
    np.testing.assert_allclose(lg["q_conv"], lp["q_conv"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(yg, yp, rtol=1e-12, atol=1e-12)


def test_grouped_diagonal_is_a_temporal_depthwise_conv():
    """W[h, i, j, c] = f[h, j] [i == c]: each channel of head h is filtered
    over tokens by f[h, :], which is oracle.seq_conv with those taps."""
    rng = np.random.default_rng(9)
    B, T, H, d, kc = 2, 8, 3, 4, 3
    a = rng.standard_normal((B, T, H, d))
    f = rng.standard_normal((H, kc))
    w = np.zeros((H, d, kc, d))
    for h in range(H):
        for j in range(kc):
            w[h, :, j, :] = f[h, j] * np.eye(d)
    taps = np.repeat(f, d, axis=0)                      # [H * d, kc], per channel
    want = O.seq_conv(a.reshape(B, T, H * d), taps).reshape(B, T, H, d)
    np.testing.assert_allclose(O.chan_conv_grouped(a, w), want, rtol=1e-12, atol=1e-12)


def test_grouped_is_causal():
    s = _shape(batch=1, seq_len=8)
    P, w = _weights(s, seed=2)
    _, l1 = O.prefill(P.x, w, s, readings=GROUPED, intermediates=True)
    x2 = P.x.copy()
    x2[:, 5:] += 1.0
    _, l2 = O.prefill(x2, w, s, readings=GROUPED, intermediates=True)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(l1[key][:, :5], l2[key][:, :5])
        assert not np.allclose(l1[key][:, 5:], l2[key][:, 5:])


@pytest.mark.parametrize("T0,m", [(0, 1), (1, 1), (5, 1), (3, 4), (6, 2)])
def test_grouped_decode_matches_prefill(T0, m):
    """Prefill T0 tokens, then decode m more from the carried state: the
    outputs and the new cache rows equal the prefill over T0 + m tokens."""
    s_all = _shape(batch=2, seq_len=T0 + m, seq_conv_k=3, chan_conv_k=4)
    P, w = _weights(s_all, seed=21)
    y_all, lat_all = O.prefill(P.x, w, s_all, readings=GROUPED, intermediates=True)
    s0 = s_all.with_(seq_len=T0)
    Wrows = O.conv_window_rows(s0, GROUPED)
    assert Wrows == (3 - 1) + (4 - 1)
    if T0 > 0:
        _, lat0 = O.prefill(P.x[:, :T0], w, s0, readings=GROUPED, intermediates=True)
        K, V, cq, ck, vs = O.prefill_state(lat0, s0, GROUPED)
    else:
        K = np.zeros((2, s0.n_kv_heads, 0, s0.head_dim))
        V = K.copy()
        cq = np.zeros((2, Wrows, s0.e_q))
        ck = np.zeros((2, Wrows, s0.e_kv))
        vs = np.zeros((2, s0.n_kv_heads // 2, s0.head_dim))
    assert cq.shape[1] == Wrows
    if m == 1:
        y, new = O.decode_step(P.x[:, T0], w, s0, K, V, cq, ck, vs, readings=GROUPED)
        np.testing.assert_allclose(y, y_all[:, T0], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(new["k_new"], lat_all["k"][:, T0], rtol=1e-10, atol=1e-12)
        assert new["conv_q"].shape[1] == Wrows
    else:
        y, new = O.decode_multi(P.x[:, T0:], w, s0, K, V, cq, ck, vs, readings=GROUPED)
        np.testing.assert_allclose(y, y_all[:, T0:], rtol=1e-10, atol=1e-12)
        assert new["conv_q"].shape[1] == Wrows


def test_backward_rejects_grouped():
    import oracle.backward as BW
    s = _shape(batch=1, seq_len=3)
    P, w = _weights(s, seed=1)
    with pytest.raises(NotImplementedError):
        BW.prefill_backward(P.x, w, s, np.ones((1, 3, s.d_model)), readings=GROUPED)
