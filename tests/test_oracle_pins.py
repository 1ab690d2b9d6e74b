"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a textbook or library routine
the method reduces to, a closed form, an invariant the pages imply, or the
scalar brute-force twin written separately.  Together they are chosen so a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle.cca as O
from oracle.brute import brute_prefill
from synth import CCAShape, make_prefill

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def tiny(B=2, T=7, E=12, Hq=2, Hkv=2, d=4, base=100.0, seed=0, **kw):
    s = CCAShape(batch=B, seq_len=T, d_model=E, n_q_heads=Hq, n_kv_heads=Hkv,
                 head_dim=d, rope_base=base, dtype="f32", **kw)
    P = make_prefill(s, seed)
    w = P.weights.f64()
    rng = np.random.default_rng(seed + 100)
    w["tau"] = rng.uniform(1.0, 2.0 * math.sqrt(d), size=Hq)   # random temperatures
    return s, P.x, w


def delta_taps(w, s):
    w = dict(w)
    w["q_seq_taps"] = np.zeros_like(w["q_seq_taps"]); w["q_seq_taps"][:, 0] = 1.0
    w["k_seq_taps"] = np.zeros_like(w["k_seq_taps"]); w["k_seq_taps"][:, 0] = 1.0
    w["q_chan_taps"] = np.zeros_like(w["q_chan_taps"]); w["q_chan_taps"][:, 0] = 1.0
    w["k_chan_taps"] = np.zeros_like(w["k_chan_taps"]); w["k_chan_taps"][:, 0] = 1.0
    return w


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


# ---------------------------------------------------------------------------
# brute force: every step, all switches on, several head layouts
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("reading", ["M2", "M1"])
@pytest.mark.parametrize("Hq,Hkv,T,d", [(2, 2, 7, 4), (4, 2, 6, 4), (4, 4, 5, 2), (2, 1, 8, 4), (4, 1, 3, 8)])
def test_brute_force_matches_oracle(Hq, Hkv, T, d, reading):
    shift = 1 if Hkv % 2 == 0 else 0
    s, x, w = tiny(T=T, Hq=Hq, Hkv=Hkv, d=d, E=10, use_value_shift=shift, seed=Hq * 7 + T)
    y = O.prefill(x, w, s, readings=O.Readings(qk_mean=reading))
    yb = np.array(brute_prefill(x.tolist(), {k: v.tolist() for k, v in w.items()}, s,
                                qk_mean=reading))
    assert rel(y, yb) < 1e-12


def test_qk_mean_readings_differ():
    """The two readings give different outputs on the same inputs (so the
    brute-force comparison above can tell them apart)."""
    s, x, w = tiny(T=6, Hq=4, Hkv=2)
    y2 = O.prefill(x, w, s, readings=O.Readings(qk_mean="M2"))
    y1 = O.prefill(x, w, s, readings=O.Readings(qk_mean="M1"))
    assert rel(y1, y2) > 1e-3


def test_brute_force_switches_off():
    s, x, w = tiny(use_qk_mean=0, use_value_shift=0, use_qk_norm=0, base=0.0)
    y = O.prefill(x, w, s)
    yb = np.array(brute_prefill(x.tolist(), {k: v.tolist() for k, v in w.items()}, s))
    assert rel(y, yb) < 1e-12


# ---------------------------------------------------------------------------
# MHA reduction: compression 1, delta conv taps, mean and shift off,
# normalisation off, tau = 1/sqrt(d) -> textbook causal RoPE multi-head
# attention.  Two independent references: a textbook implementation with RoPE
# as complex rotation, and torch's scaled_dot_product_attention in fp64.
# ---------------------------------------------------------------------------

def textbook_rope_complex(x, base):
    """x [B, T, H, d]; pairs (2i, 2i+1) as complex numbers times e^{i t theta_i}."""
    B, T, H, d = x.shape
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.array([base ** (-(2.0 * i) / d) for i in range(d // 2)])
    rot = np.exp(1j * np.outer(np.arange(T), theta))[None, :, None, :]
    z = z * rot
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def textbook_mha(x, wq, wk, wv, wo, H, Hkv, d, base, scale, qk_l2=False):
    B, T, _ = x.shape
    Q = (x @ wq.T).reshape(B, T, H, d)
    K = (x @ wk.T).reshape(B, T, Hkv, d)
    V = (x @ wv.T).reshape(B, T, Hkv, d)
    if qk_l2:
        Q = Q / np.linalg.norm(Q, axis=-1, keepdims=True)
        K = K / np.linalg.norm(K, axis=-1, keepdims=True)
    Q, K = textbook_rope_complex(Q, base), textbook_rope_complex(K, base)
    G = H // Hkv
    out = np.zeros((B, T, H, d))
    for b in range(B):
        for h in range(H):
            g = h // G
            S = scale[h] * Q[b, :, h] @ K[b, :, g].T
            S[np.triu_indices(T, 1)] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[b, :, h] = P @ V[b, :, g]
    return out.reshape(B, T, H * d) @ wo.T


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (4, 1)])
def test_mha_reduction_textbook(Hq, Hkv):
    d = 8
    E = Hq * d                                       # compression factor 1 for queries
    s, x, w = tiny(B=2, T=9, E=E, Hq=Hq, Hkv=Hkv, d=d, base=500.0,
                   use_qk_mean=0, use_value_shift=0, use_qk_norm=0)
    w = delta_taps(w, s)
    w["tau"] = np.full(Hq, 1.0 / math.sqrt(d))
    y = O.prefill(x, w, s)
    eq, ekv = Hq * d, Hkv * d
    wq, wk, wv = w["w_qkv"][:eq], w["w_qkv"][eq:eq + ekv], w["w_qkv"][eq + ekv:]
    ref = textbook_mha(x, wq, wk, wv, w["w_o"], Hq, Hkv, d, 500.0, w["tau"])
    assert rel(y, ref) < 1e-12


def test_mha_reduction_with_qk_norm():
    d, H = 8, 4
    s, x, w = tiny(B=1, T=9, E=H * d, Hq=H, Hkv=H, d=d, base=10000.0,
                   use_qk_mean=0, use_value_shift=0, use_qk_norm=1)
    w = delta_taps(w, s)
    eq = H * d
    ref = textbook_mha(x, w["w_qkv"][:eq], w["w_qkv"][eq:2 * eq], w["w_qkv"][2 * eq:],
                       w["w_o"], H, H, d, 10000.0, w["tau"], qk_l2=True)
    assert rel(O.prefill(x, w, s), ref) < 1e-12


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2)])
def test_mha_reduction_torch_sdpa(Hq, Hkv):
    d = 8
    s, x, w = tiny(B=2, T=11, E=Hq * d, Hq=Hq, Hkv=Hkv, d=d, base=0.0,
                   use_qk_mean=0, use_value_shift=0, use_qk_norm=0)
    w = delta_taps(w, s)
    w["tau"] = np.full(Hq, 1.0 / math.sqrt(d))
    y = O.prefill(x, w, s)
    eq, ekv = Hq * d, Hkv * d
    xt = torch.from_numpy(x)
    B, T = x.shape[:2]
    Q = (xt @ torch.from_numpy(w["w_qkv"][:eq]).T).reshape(B, T, Hq, d).transpose(1, 2)
    K = (xt @ torch.from_numpy(w["w_qkv"][eq:eq + ekv]).T).reshape(B, T, Hkv, d).transpose(1, 2)
    V = (xt @ torch.from_numpy(w["w_qkv"][eq + ekv:]).T).reshape(B, T, Hkv, d).transpose(1, 2)
    K = K.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    V = V.repeat_interleave(Hq // Hkv, dim=1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(Q.contiguous(), K, V, is_causal=True)
    ref = o.transpose(1, 2).reshape(B, T, eq) @ torch.from_numpy(w["w_o"]).T
    assert rel(y, ref.numpy()) < 1e-12


# ---------------------------------------------------------------------------
# causality and batch independence
# ---------------------------------------------------------------------------

def test_causality_exact():
    s, x, w = tiny(B=2, T=8, Hq=4, Hkv=2)
    y = O.prefill(x, w, s)
    rng = np.random.default_rng(3)
    for t in range(s.seq_len - 1):
        x2 = x.copy()
        x2[:, t + 1:, :] += rng.standard_normal(x2[:, t + 1:, :].shape)
        y2 = O.prefill(x2, w, s)
        np.testing.assert_array_equal(y[:, :t + 1], y2[:, :t + 1])
        assert np.abs(y[:, t + 1:] - y2[:, t + 1:]).max() > 1e-6   # the future does change


def test_batch_independence():
    s, x, w = tiny(B=3, T=6)
    y = O.prefill(x, w, s)
    x2 = x.copy()
    x2[1] = np.random.default_rng(4).standard_normal(x2[1].shape)
    y2 = O.prefill(x2, w, s)
    np.testing.assert_array_equal(y[0], y2[0])
    np.testing.assert_array_equal(y[2], y2[2])


# ---------------------------------------------------------------------------
# convolutions: delta taps are the identity, a single tap at lag j is an exact
# shift by j (zeros before the sequence start / the head's first channel)
# ---------------------------------------------------------------------------

def test_seq_conv_delta_and_shift():
    rng = np.random.default_rng(5)
    u = rng.standard_normal((2, 9, 6))
    for j in range(4):
        taps = np.zeros((6, 4)); taps[:, j] = 1.0
        a = O.seq_conv(u, taps)
        exp = np.zeros_like(u); exp[:, j:] = u[:, :9 - j]
        np.testing.assert_array_equal(a, exp)
    # per-channel taps scale per channel; history feeds the first tokens
    taps = np.zeros((6, 4)); taps[:, 2] = np.arange(1, 7)
    hist = rng.standard_normal((2, 3, 6))
    a = O.seq_conv(u, taps, hist)
    np.testing.assert_array_equal(a[:, 0], hist[:, 1] * np.arange(1, 7))
    np.testing.assert_array_equal(a[:, 1], hist[:, 2] * np.arange(1, 7))
    np.testing.assert_array_equal(a[:, 2], u[:, 0] * np.arange(1, 7))


def test_chan_conv_delta_and_shift():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((2, 5, 3, 8))
    for j in range(4):
        taps = np.zeros((3, 4)); taps[:, j] = 1.0
        b = O.chan_conv(a, taps)
        exp = np.zeros_like(a); exp[..., j:] = a[..., :8 - j]
        np.testing.assert_array_equal(b, exp)
    # taps differ per head, never mix heads
    taps = np.zeros((3, 4)); taps[:, 1] = [1.0, 2.0, 3.0]
    b = O.chan_conv(a, taps)
    for h in range(3):
        np.testing.assert_array_equal(b[..., h, 0], 0.0)
        np.testing.assert_array_equal(b[..., h, 1:], (h + 1) * a[..., h, :7])


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_single_token_closed_form():
    """T = 1: softmax over one key is 1, so o = v_0; shifted heads see zeros."""
    s, x, w = tiny(B=2, T=1, Hq=4, Hkv=2)
    y = O.prefill(x, w, s)
    eq, ekv, d = s.e_q, s.e_kv, s.head_dim
    vbar = x[:, 0] @ w["w_qkv"][eq + ekv:].T            # [B, e_kv]
    vbar[:, d:] = 0.0                                     # kv head 1 (upper half) is shifted
    o = np.repeat(vbar.reshape(2, 2, d), 2, axis=1).reshape(2, eq)
    np.testing.assert_allclose(y[:, 0], o @ w["w_o"].T, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("shift", [0, 1])
def test_zero_temperature_is_prefix_mean(shift):
    """tau = 0 makes attention uniform over the visible keys: o_t is the mean of
    v_0..v_t; a shifted head averages vbar_{-1}=0, vbar_0, .., vbar_{t-1}."""
    s, x, w = tiny(B=2, T=6, Hq=4, Hkv=2, use_value_shift=shift)
    w["tau"] = np.zeros(4)
    y = O.prefill(x, w, s)
    eq, ekv, d = s.e_q, s.e_kv, s.head_dim
    wv = w["w_qkv"][eq + ekv:]
    T = s.seq_len
    for t in range(T):
        cur = x[:, :t + 1].sum(axis=1) / (t + 1)          # mean of x_0..x_t
        prev = x[:, :t].sum(axis=1) / (t + 1)             # (x_0..x_{t-1}) / (t+1)
        vv = np.empty((2, ekv))
        vv[:, :d] = cur @ wv[:d].T
        vv[:, d:] = (prev if shift else cur) @ wv[d:].T
        o = np.repeat(vv.reshape(2, 2, d), 2, axis=1).reshape(2, eq)
        np.testing.assert_allclose(y[:, t], o @ w["w_o"].T, rtol=1e-12, atol=1e-13)


def test_scale_equivariance_with_norm():
    """With q, k normalised, scaling x by a > 0 leaves every attention weight
    unchanged and scales the values, so y scales by a."""
    s, x, w = tiny(B=1, T=7, Hq=4, Hkv=2)
    y = O.prefill(x, w, s)
    np.testing.assert_allclose(O.prefill(3.5 * x, w, s), 3.5 * y, rtol=1e-12, atol=1e-13)


def test_qk_norm_gives_unit_heads():
    s, x, w = tiny(B=1, T=5, Hq=4, Hkv=2)
    lat = O.latents(x, w, s)
    np.testing.assert_allclose(np.linalg.norm(lat["q"], axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(lat["k"], axis=-1), 1.0, rtol=1e-13)


def test_value_shift_index_form():
    s, x, w = tiny(B=2, T=5, Hq=4, Hkv=4)
    lat = O.latents(x, w, s)
    np.testing.assert_array_equal(lat["v"][:, :, :2], lat["vbar"][:, :, :2])
    np.testing.assert_array_equal(lat["v"][:, 1:, 2:], lat["vbar"][:, :-1, 2:])
    np.testing.assert_array_equal(lat["v"][:, 0, 2:], 0.0)


# ---------------------------------------------------------------------------
# RoPE invariants
# ---------------------------------------------------------------------------

def test_rope_invariants():
    rng = np.random.default_rng(7)
    d = 16
    a = rng.standard_normal((1, 1, 1, d))
    b = rng.standard_normal((1, 1, 1, d))
    for base in (1e4, 5e5):
        # position 0 is the identity, norms are preserved
        np.testing.assert_array_equal(O.rope(a, np.array([0]), base), a)
        for p in (1, 37, 32768):
            r = O.rope(a, np.array([p]), base)
            assert abs(np.linalg.norm(r) - np.linalg.norm(a)) < 1e-12
        # relative position: <R_m a, R_n b> = <R_{m-n} a, b>
        for m, n in ((5, 2), (1000, 999), (16383, 100)):
            lhs = np.sum(O.rope(a, np.array([m]), base) * O.rope(b, np.array([n]), base))
            rhs = np.sum(O.rope(a, np.array([m - n]), base) * b)
            assert abs(lhs - rhs) < 1e-9
        # a quarter turn of pair 0 at the position whose angle is pi/2
        e = np.zeros((1, 1, 1, d)); e[..., 0] = 1.0
        r = O.rope(e, np.array([math.pi / 2]), base)   # pair 0 has frequency 1
        np.testing.assert_allclose(r[..., :2].ravel(), [0.0, 1.0], atol=1e-15)


def test_norm_and_rope_commute():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 6, 2, 8))
    pos = np.arange(6)
    a = O.rope(O.l2_normalize(x, 1e-6), pos, 1e4)
    b = O.l2_normalize(O.rope(x, pos, 1e4), 1e-6)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# decode: one step after a prefill of L tokens equals a prefill of L + 1
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L", [0, 1, 2, 3, 6])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2)])
def test_decode_after_prefill(L, Hq, Hkv):
    s, x, w = tiny(B=2, T=L + 1, Hq=Hq, Hkv=Hkv, d=4, E=10)
    y_full = O.prefill(x, w, s)
    if L > 0:
        _, lat = O.prefill(x[:, :L], w, s.with_(seq_len=L), intermediates=True)
        K, V, cq, ck, vs = O.prefill_state(lat, s)
    else:
        K = np.zeros((2, Hkv, 0, 4)); V = np.zeros((2, Hkv, 0, 4))
        cq = np.zeros((2, 3, s.e_q)); ck = np.zeros((2, 3, s.e_kv)); vs = np.zeros((2, Hkv // 2, 4))
    y_t, new = O.decode_step(x[:, L], w, s, K, V, cq, ck, vs)
    assert rel(y_t, y_full[:, L]) < 1e-12
    # the rolled state equals the state of the longer prefill
    _, lat2 = O.prefill(x, w, s.with_(seq_len=L + 1), intermediates=True)
    K2, V2, cq2, ck2, vs2 = O.prefill_state(lat2, s)
    np.testing.assert_allclose(new["k_new"], K2[:, :, L], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["v_new"], V2[:, :, L], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["conv_q"], cq2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["conv_k"], ck2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["vshift"], vs2, rtol=1e-12, atol=1e-14)


def test_multi_step_decode_matches_prefill():
    s, x, w = tiny(B=2, T=9, Hq=4, Hkv=2)
    y_full = O.prefill(x, w, s)
    L0 = 4
    _, lat = O.prefill(x[:, :L0], w, s.with_(seq_len=L0), intermediates=True)
    K, V, cq, ck, vs = O.prefill_state(lat, s)
    for L in range(L0, 9):
        y_t, new = O.decode_step(x[:, L], w, s, K, V, cq, ck, vs)
        assert rel(y_t, y_full[:, L]) < 1e-12
        K = np.concatenate([K, new["k_new"][:, :, None]], axis=2)
        V = np.concatenate([V, new["v_new"][:, :, None]], axis=2)
        cq, ck, vs = new["conv_q"], new["conv_k"], new["vshift"]


@pytest.mark.parametrize("L0,m", [(0, 1), (0, 3), (2, 2), (4, 5), (6, 1)])
def test_multi_token_decode_matches_prefill(L0, m):
    """m new tokens at once after a prefill of L0 equal a prefill of L0 + m
    (outputs, appended k / v rows and the rolled state)."""
    s, x, w = tiny(B=2, T=L0 + m, Hq=4, Hkv=2)
    y_full = O.prefill(x, w, s)
    Hkv, d = s.n_kv_heads, s.head_dim
    if L0 > 0:
        _, lat = O.prefill(x[:, :L0], w, s.with_(seq_len=L0), intermediates=True)
        K, V, cq, ck, vs = O.prefill_state(lat, s)
    else:
        K = np.zeros((2, Hkv, 0, d)); V = np.zeros((2, Hkv, 0, d))
        cq = np.zeros((2, 3, s.e_q)); ck = np.zeros((2, 3, s.e_kv)); vs = np.zeros((2, Hkv // 2, d))
    y, new = O.decode_multi(x[:, L0:], w, s, K, V, cq, ck, vs)
    assert rel(y, y_full[:, L0:]) < 1e-12
    _, lat2 = O.prefill(x, w, s, intermediates=True)
    K2, V2, cq2, ck2, vs2 = O.prefill_state(lat2, s)
    np.testing.assert_allclose(new["k_new"], K2[:, :, L0:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["v_new"], V2[:, :, L0:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["conv_q"], cq2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["conv_k"], ck2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(new["vshift"], vs2, rtol=1e-12, atol=1e-14)


def test_sampled_rows_match_full():
    s, x, w = tiny(B=2, T=12, Hq=4, Hkv=2)
    y = O.prefill(x, w, s)
    rows = [0, 3, 4, 11]
    np.testing.assert_allclose(O.prefill(x, w, s, rows=rows), y[:, rows], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# qualitative pin of the q-k-mean: with normalisation it strengthens the
# attention diagonal (q_t and k_t share a term), so the mean cosine between
# q_t and k_t over random inputs is clearly higher with the mean on.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("reading", ["M2", "M1"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_qk_mean_strengthens_diagonal(reading, Hq, Hkv):
    s, x, w = tiny(B=4, T=64, E=64, Hq=Hq, Hkv=Hkv, d=16, base=0.0, seed=11)
    r = O.Readings(qk_mean=reading)
    on = O.latents(x, w, s, readings=r)
    off = O.latents(x, w, s.with_(use_qk_mean=0), readings=r)
    G = Hq // Hkv
    cos_on = np.mean(np.sum(on["q"] * np.repeat(on["k"], G, axis=2), axis=-1))
    cos_off = np.mean(np.sum(off["q"] * np.repeat(off["k"], G, axis=2), axis=-1))
    assert cos_on > cos_off + 0.2


# ---------------------------------------------------------------------------
# closed form of the q-k-mean under scaled delta taps.  With the sequence and
# channel taps (c, 0, 0, 0) and (c', 0, 0, 0) both convolutions are a scaling
# by alpha = c * c': b_q = alpha q~, b_k = alpha k~.  The mean of the pre- and
# post-convolution q and k of a CCA head is then (1 + alpha)(q~ + k~) / 4, so
#   q = (alpha + (1 + alpha) / 4) q~ + ((1 + alpha) / 4) k~          (M2)
# and with only the pre-convolution mean (q~ + k~) / 2,
#   q = (alpha + 1 / 2) q~ + (1 / 2) k~                                (M1).
# For CCGQA the kv head meets the average q~ of its G query heads.  At
# alpha = 1 the two readings coincide; at alpha = 3 they do not.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("reading", ["M2", "M1"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (6, 2)])
@pytest.mark.parametrize("c,c2", [(1.0, 1.0), (1.5, 2.0), (-0.5, 3.0)])
def test_qk_mean_closed_form_scaled_delta(reading, Hq, Hkv, c, c2):
    s, x, w = tiny(B=2, T=5, E=10, Hq=Hq, Hkv=Hkv, d=4, base=0.0, use_value_shift=0,
                   use_qk_norm=0, seed=Hq + 3)
    w = delta_taps(w, s)
    w["q_seq_taps"] *= c
    w["k_seq_taps"] *= c
    w["q_chan_taps"] *= c2
    w["k_chan_taps"] *= c2
    alpha = c * c2
    lat = O.latents(x, w, s, readings=O.Readings(qk_mean=reading))
    d, G, eq, ekv = s.head_dim, Hq // Hkv, s.e_q, s.e_kv
    qt = (x @ w["w_qkv"][:eq].T).reshape(2, 5, Hq, d)
    kt = (x @ w["w_qkv"][eq:eq + ekv].T).reshape(2, 5, Hkv, d)
    k_of_q = kt[:, :, np.arange(Hq) // G]                  # kv head of each query head
    q_avg = qt.reshape(2, 5, Hkv, G, d).mean(axis=3)      # average q~ of each group
    if reading == "M2":
        own, other = alpha + (1 + alpha) / 4, (1 + alpha) / 4
    else:
        own, other = alpha + 0.5, 0.5
    np.testing.assert_allclose(lat["q"], own * qt + other * k_of_q, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lat["k"], own * kt + other * q_avg, rtol=1e-12, atol=1e-13)
