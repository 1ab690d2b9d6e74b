"""GPU parity of libcca against the fp64 oracle, through the C ABI.

Small shapes are compared element by element (several tiles and a ragged
tail); the full-size workloads are compared on sampled query rows that the
oracle computes one by one.  Tolerances: bf16 I/O max-abs <= 2e-2 and
relative L2 <= 5e-3; fp32 validation mode relative L2 <= 1e-5.
"""

import sys

import numpy as np
import pytest
import torch

import oracle.cca as O
from synth import COMPARISON_OVERRIDES, COMPARISONS, CCAShape, make_decode, make_prefill, workload
from gpu_helpers import (PrefillRun, assert_parity, lib, rel_l2, sample_rows, set_taps,
                         tau_inv_sqrt_d, tens, upload_weights, vt_unpermute)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = {
    # name: (shape, tau override)
    "tiny_f32_workload": (workload("cca_prefill_tiny_f32"), None),
    "bf16_g2_ragged": (CCAShape(batch=2, seq_len=300, d_model=256, n_q_heads=4, n_kv_heads=2,
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
    "bf16_taps_2_3": (CCAShape(batch=1, seq_len=140, d_model=256, n_q_heads=4, n_kv_heads=2,
                               head_dim=64, seq_conv_k=2, chan_conv_k=3), None),
    "bf16_single_token": (CCAShape(batch=3, seq_len=1, d_model=256, n_q_heads=4, n_kv_heads=2,
                                   head_dim=64), None),
    "bf16_g8": (CCAShape(batch=1, seq_len=100, d_model=256, n_q_heads=8, n_kv_heads=1,
                         head_dim=64, use_value_shift=0), None),
    "bf16_switches_off": (CCAShape(batch=1, seq_len=160, d_model=256, n_q_heads=4, n_kv_heads=4,
                                   head_dim=64, use_qk_mean=0, use_value_shift=0, use_qk_norm=0,
                                   rope_base=10000.0), "inv_sqrt_d"),
    # norm on with per-head temperatures on both sides of the constant-shift
    # limit (tau * log2(e) <= 60 uses the fixed shift, above it the running max)
    "bf16_norm_mixed_tau": (CCAShape(batch=1, seq_len=210, d_model=256, n_q_heads=4, n_kv_heads=2,
                                     head_dim=64), "mixed"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_small_parity(name):
    shape, tau = SMALL[name]
    _say(f"[prefill] {name} {shape}")
    P = make_prefill(shape, seed=0)
    if tau == "inv_sqrt_d":
        set_taps(P, tau=tau_inv_sqrt_d(shape))
    elif tau == "mixed":
        set_taps(P, tau=np.array([8.0, 50.0, 0.5, 41.0], dtype=np.float32))
    run = PrefillRun(shape, P)
    y = run.run()
    ref = O.prefill(P.x, P.weights.f64(), shape)
    assert_parity(y, ref, shape.dtype, name)


def test_prefill_mha_reduction_gpu():
    """Compression 1, delta taps, mean / shift / norm off, tau = 1/sqrt(d):
    the GPU path computes textbook causal RoPE MHA (oracle pinned to it)."""
    shape = CCAShape(batch=1, seq_len=192, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                     use_qk_mean=0, use_value_shift=0, use_qk_norm=0, rope_base=10000.0)
    _say(f"[prefill] mha reduction {shape}")
    P = make_prefill(shape, seed=3)
    qs = np.zeros((shape.e_q, 4), np.float32); qs[:, 0] = 1
    ks = np.zeros((shape.e_kv, 4), np.float32); ks[:, 0] = 1
    qc = np.zeros((4, 4), np.float32); qc[:, 0] = 1
    set_taps(P, seq=(qs, ks), chan=(qc, qc.copy()), tau=tau_inv_sqrt_d(shape))
    y = PrefillRun(shape, P).run()
    assert_parity(y, O.prefill(P.x, P.weights.f64(), shape), "bf16", "mha")


@pytest.mark.parametrize("name", list(COMPARISONS))
def test_comparison_baseline_parity(name):
    """The full-width baselines of the prefill comparison at their own head
    shapes (E = 4096, 64 query heads over 64 or 8 kv heads, d = 64), shortened
    to T = 1024: taps of length one set to 1 (identity convolutions), mean,
    shift and norm off, tau = 1/sqrt(d), exactly as the comparison runs them.
    Sampled rows against the oracle."""
    import math
    shape = COMPARISONS[name].with_(seq_len=1024)
    _say(f"[prefill] comparison baseline {name} {shape}")
    P = make_prefill(shape, seed=5)
    W = P.weights
    for a in (W.q_seq_taps, W.k_seq_taps, W.q_chan_taps, W.k_chan_taps):
        a[...] = COMPARISON_OVERRIDES["taps"]
    W.tau = np.full(shape.n_q_heads, 1.0 / math.sqrt(shape.head_dim), dtype=np.float32)
    y = PrefillRun(shape, P).run()
    rows = sample_rows(shape.seq_len, 40, seed=2)
    ref = O.prefill(P.x, W.f64(), shape, rows=rows)
    assert_parity(y[:, rows], ref, "bf16", name)


def test_prefill_stage_intermediates():
    """Each kernel's output against the oracle's intermediate of the same step."""
    shape = CCAShape(batch=2, seq_len=150, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64)
    _say(f"[stages] {shape}")
    P = make_prefill(shape, seed=5)
    run = PrefillRun(shape, P)
    y = run.run()
    ref_y, lat = O.prefill(P.x, P.weights.f64(), shape, intermediates=True)
    s, T = shape, tens()
    B, Tn, Tp, d = s.batch, s.seq_len, run.padded_T(), s.head_dim
    L = lib()
    qkv = T.to_f64(run.ws_view(L.WS_QKV, run.qkv_dtype(), (B, Tn, s.n_qkv)))
    ref_qkv = np.concatenate([lat["q_pre"].reshape(B, Tn, -1), lat["k_pre"].reshape(B, Tn, -1),
                              lat["vbar"].reshape(B, Tn, -1)], axis=-1)
    # the fp16 output rounding moves each element by at most 2^-11 of itself
    # (fp32 accumulation adds ~1e-7)
    assert rel_l2(qkv, ref_qkv) < 2.0 ** -11 + 1e-6, "down-projection"
    q = T.to_f64(run.ws_view(L.WS_Q, run.qk_dtype(), (B, s.n_q_heads, Tp, d)))
    k = T.to_f64(run.ws_view(L.WS_K, run.qk_dtype(), (B, s.n_kv_heads, Tp, d)))
    scale = (P.weights.tau.astype(np.float64) * np.log2(np.e))[None, :, None, None]
    assert rel_l2(q[:, :, :Tn] / scale, lat["q"].transpose(0, 2, 1, 3)) < 1e-3, "mixed q"
    assert rel_l2(k[:, :, :Tn], lat["k"].transpose(0, 2, 1, 3)) < 1e-3, "mixed k"
    assert np.all(q[:, :, Tn:] == 0) and np.all(k[:, :, Tn:] == 0), "padding rows"
    vt = vt_unpermute(T.to_f64(run.ws_view(L.WS_VT, torch.bfloat16, (B, s.n_kv_heads, d, Tp))))
    assert rel_l2(vt[..., :Tn], lat["v"].transpose(0, 2, 3, 1)) < 5e-3, "shifted v"
    assert np.all(vt[..., Tn:] == 0)
    o = T.to_f64(run.ws_view(L.WS_O, torch.bfloat16, (B, Tn, s.e_q)))
    assert rel_l2(o, lat["o"].reshape(B, Tn, -1)) < 5e-3, "attention output"
    assert_parity(y, ref_y, "bf16", "y")


@pytest.mark.parametrize("name,nrows", [("cca_prefill_b4_t2048", 48),
                                        ("ccgqa_prefill_t8192", 48),
                                        ("ccgqa_prefill_t16384", 48)])
def test_prefill_workload_sampled(name, nrows):
    shape = workload(name)
    _say(f"[workload] {name}")
    P = make_prefill(shape, seed=0)
    run = PrefillRun(shape, P)
    y = run.run()
    rows = sample_rows(shape.seq_len, nrows)
    ref = O.prefill(P.x, P.weights.f64(), shape, rows=rows)
    assert_parity(y[:, rows], ref, "bf16", name)


def test_prefill_causality_bitwise():
    shape = CCAShape(batch=2, seq_len=300, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64)
    _say("[causality]")
    P = make_prefill(shape, seed=7)
    run = PrefillRun(shape, P)
    y0 = run.run().copy()
    for t in (0, 63, 64, 127, 200, 298):
        x2 = P.x_s.copy()
        rng = np.random.default_rng(t)
        x2[:, t + 1:] = rng.integers(0, 2 ** 16, size=x2[:, t + 1:].shape, dtype=np.uint16) & 0xBFFF
        run.x.copy_(tens().to_device(x2))
        y1 = run.run()
        np.testing.assert_array_equal(y1[:, :t + 1], y0[:, :t + 1])
        assert np.any(y1[:, t + 1:] != y0[:, t + 1:])


def test_prefill_repeat_bitwise():
    shape = CCAShape(batch=1, seq_len=513, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64)
    P = make_prefill(shape, seed=8)
    run = PrefillRun(shape, P)
    a = run.run().copy()
    b = run.run()
    np.testing.assert_array_equal(a, b)


def test_prefill_state_then_decode():
    """prefill(x[:L]) with state -> decode(x[L]) -> decode(x[L+1]) equals the
    oracle prefill over L+1 / L+2 tokens at the last position."""
    full = CCAShape(batch=2, seq_len=39, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64)
    _say("[prefill->decode]")
    P = make_prefill(full, seed=9)
    Lp = 37
    pshape = full.with_(seq_len=Lp)
    Pp = make_prefill(full, seed=9)
    Pp.x_s = np.ascontiguousarray(P.x_s[:, :Lp])
    Pp.x = P.x[:, :Lp]
    run = PrefillRun(pshape, Pp, capacity=64)
    run.run()
    # the state the GPU wrote equals the oracle's (after bf16 rounding)
    _, lat = O.prefill(Pp.x, P.weights.f64(), pshape, intermediates=True)
    K, V, cq, ck, vs = O.prefill_state(lat, pshape)
    T = tens()
    st = run.state
    assert rel_l2(T.to_f64(st.k_cache)[:, :, :Lp], K) < 5e-3
    assert rel_l2(T.to_f64(st.v_cache)[:, :, :Lp], V) < 5e-3
    assert rel_l2(T.to_f64(st.conv_q), cq) < 5e-3
    assert rel_l2(T.to_f64(st.conv_k), ck) < 5e-3
    assert rel_l2(T.to_f64(st.vshift), vs) < 5e-3
    L = lib()
    dshape = full.with_(seq_len=1)
    cfg = L.make_config(dshape)
    ref_full = O.prefill(P.x, P.weights.f64(), full)
    for step, pos in enumerate((Lp, Lp + 1)):
        x_t = T.to_device(np.ascontiguousarray(P.x_s[:, pos]))
        y_t = torch.empty_like(x_t)
        ws = T.workspace(L.decode_workspace_size(cfg, pos))
        L.decode_step(cfg, run.w, x_t, pos, st, st, y_t, ws)
        torch.cuda.synchronize()
        assert_parity(T.to_f64(y_t), ref_full[:, pos], "bf16", f"decode step {step}")


def _upload_decode(D, dev="cuda"):
    T, L = tens(), lib()
    s = D.shape
    st = L.State(k_cache=T.to_device(D.k_cache_s, dev), v_cache=T.to_device(D.v_cache_s, dev),
                 capacity=D.capacity, conv_q=T.to_device(D.conv_q_s, dev),
                 conv_k=T.to_device(D.conv_k_s, dev), vshift=T.to_device(D.vshift_s, dev))
    return st


def _oracle_decode(D, b_list=None):
    s = D.shape
    w = D.weights.f64()
    cq, ck, vs = D.state_f64()
    B = s.batch
    bs = range(B) if b_list is None else b_list
    ys, news = [], []
    for b in bs:
        K = D.cache_f64(b, "k")[None]
        V = D.cache_f64(b, "v")[None]
        y, new = O.decode_step(D.x[b:b + 1], w, s, K, V, cq[b:b + 1], ck[b:b + 1], vs[b:b + 1])
        ys.append(y[0])
        news.append(new)
    return np.stack(ys), news


@pytest.mark.parametrize("L_", [0, 1, 5, 1023, 1024, 1025, 3000])
def test_decode_small_parity(L_):
    shape = CCAShape(batch=3, seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                     rope_base=500000.0, cache_len=L_)
    _say(f"[decode] L={L_}")
    D = make_decode(shape, seed=L_, capacity=L_ + 3)
    T, Lb = tens(), lib()
    st = _upload_decode(D)
    w = upload_weights(D.weights)
    cfg = Lb.make_config(shape)
    x_t = T.to_device(D.x_s)
    y_t = torch.empty_like(x_t)
    ws = T.workspace(Lb.decode_workspace_size(cfg, L_))
    Lb.decode_step(cfg, w, x_t, L_, st, st, y_t, ws)
    torch.cuda.synchronize()
    ref, news = _oracle_decode(D)
    assert_parity(T.to_f64(y_t), ref, "bf16", "y_t")
    kc = T.to_f64(st.k_cache)
    vc = T.to_f64(st.v_cache)
    for b, new in enumerate(news):
        assert rel_l2(kc[b, :, L_], new["k_new"][0]) < 5e-3
        assert rel_l2(vc[b, :, L_], new["v_new"][0]) < 5e-3
        assert rel_l2(T.to_f64(st.conv_q)[b], new["conv_q"][0]) < 5e-3
        assert rel_l2(T.to_f64(st.conv_k)[b], new["conv_k"][0]) < 5e-3
        assert rel_l2(T.to_f64(st.vshift)[b], new["vshift"][0]) < 5e-3
    # cache slots before L are untouched
    for b in range(shape.batch):
        np.testing.assert_array_equal(kc[b, :, :L_], D.cache_f64(b, "k"))
        np.testing.assert_array_equal(vc[b, :, :L_], D.cache_f64(b, "v"))


def test_decode_varlen_parity():
    """Per-sequence cache lengths: every sequence against the oracle with its
    own cache prefix, the new rows at its own slot, the rest untouched."""
    lens = [0, 1, 37, 1024, 2999]
    Lmax = 3000
    shape = CCAShape(batch=len(lens), seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2,
                     head_dim=64, rope_base=500000.0, cache_len=Lmax)
    _say(f"[decode varlen] lens={lens}")
    D = make_decode(shape, seed=11, capacity=Lmax + 3)
    T, Lb = tens(), lib()
    st = _upload_decode(D)
    cfg = Lb.make_config(shape)
    x_t = T.to_device(D.x_s)
    y_t = torch.empty_like(x_t)
    ws = T.workspace(Lb.decode_workspace_size(cfg, Lmax))
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    Lb.decode_step_varlen(cfg, upload_weights(D.weights), x_t, dl, Lmax, st, st, y_t, ws)
    torch.cuda.synchronize()
    w = D.weights.f64()
    cq, ck, vs = D.state_f64()
    kc, vc, y = T.to_f64(st.k_cache), T.to_f64(st.v_cache), T.to_f64(y_t)
    for b, L_ in enumerate(lens):
        K = D.cache_f64(b, "k")[None, :, :L_]
        V = D.cache_f64(b, "v")[None, :, :L_]
        ref, new = O.decode_step(D.x[b:b + 1], w, shape, K, V, cq[b:b + 1], ck[b:b + 1], vs[b:b + 1])
        assert_parity(y[b:b + 1], ref, "bf16", f"varlen b={b} L={L_}")
        assert rel_l2(kc[b, :, L_], new["k_new"][0]) < 5e-3
        assert rel_l2(vc[b, :, L_], new["v_new"][0]) < 5e-3
        assert rel_l2(T.to_f64(st.conv_q)[b], new["conv_q"][0]) < 5e-3
        assert rel_l2(T.to_f64(st.vshift)[b], new["vshift"][0]) < 5e-3
        keep = [i for i in range(Lmax) if i != L_]
        np.testing.assert_array_equal(kc[b][:, keep], D.cache_f64(b, "k")[:, keep])
        np.testing.assert_array_equal(vc[b][:, keep], D.cache_f64(b, "v")[:, keep])


def test_decode_varlen_uniform_bitwise():
    """With every length equal, the varlen step is the uniform step, bit for bit."""
    L_ = 777
    shape = CCAShape(batch=3, seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                     rope_base=500000.0, cache_len=L_)
    D = make_decode(shape, seed=12, capacity=L_ + 2)
    T, Lb = tens(), lib()
    cfg = Lb.make_config(shape)
    w = upload_weights(D.weights)
    x_t = T.to_device(D.x_s)
    outs = []
    for varlen in (False, True):
        st = _upload_decode(D)
        y_t = torch.empty_like(x_t)
        ws = T.workspace(Lb.decode_workspace_size(cfg, L_))
        if varlen:
            dl = torch.full((shape.batch,), L_, dtype=torch.int32, device="cuda")
            Lb.decode_step_varlen(cfg, w, x_t, dl, L_, st, st, y_t, ws)
        else:
            Lb.decode_step(cfg, w, x_t, L_, st, st, y_t, ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (y_t, st.k_cache, st.v_cache, st.conv_q, st.conv_k, st.vshift)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_decode_f32_validation_mode():
    shape = CCAShape(batch=2, seq_len=1, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=16,
                     dtype="f32", cache_len=700)
    D = make_decode(shape, seed=4)
    T, Lb = tens(), lib()
    st = _upload_decode(D)
    cfg = Lb.make_config(shape)
    x_t = T.to_device(D.x_s)
    y_t = torch.empty_like(x_t)
    ws = T.workspace(Lb.decode_workspace_size(cfg, shape.cache_len))
    Lb.decode_step(cfg, upload_weights(D.weights), x_t, shape.cache_len, st, st, y_t, ws)
    torch.cuda.synchronize()
    ref, _ = _oracle_decode(D)
    assert_parity(T.to_f64(y_t), ref, "f32", "decode f32")


def test_decode_workload_full():
    shape = workload("ccgqa_decode_b64_l32768")
    _say("[decode] full workload B=64 L=32768")
    D = make_decode(shape, seed=0)
    T, Lb = tens(), lib()
    st = _upload_decode(D)
    cfg = Lb.make_config(shape)
    x_t = T.to_device(D.x_s)
    y_t = torch.empty_like(x_t)
    ws = T.workspace(Lb.decode_workspace_size(cfg, shape.cache_len))
    Lb.decode_step(cfg, upload_weights(D.weights), x_t, shape.cache_len, st, st, y_t, ws)
    torch.cuda.synchronize()
    ref, news = _oracle_decode(D)
    assert_parity(T.to_f64(y_t), ref, "bf16", "decode workload")
    L_ = shape.cache_len
    kc = st.k_cache[:, :, L_].float().cpu().numpy()
    vc = st.v_cache[:, :, L_].float().cpu().numpy()
    assert rel_l2(kc, np.stack([n["k_new"][0] for n in news])) < 5e-3
    assert rel_l2(vc, np.stack([n["v_new"][0] for n in news])) < 5e-3


FUSED = {
    "g1_norm_t256": CCAShape(batch=2, seq_len=256, d_model=256, n_q_heads=4, n_kv_heads=4,
                             head_dim=64, rope_base=10000.0),
    "g1_nonorm_noshift_t384": CCAShape(batch=1, seq_len=384, d_model=512, n_q_heads=2, n_kv_heads=2,
                                       head_dim=64, use_qk_norm=0, use_value_shift=0,
                                       seq_conv_k=2, chan_conv_k=3),
}


@pytest.mark.parametrize("name", list(FUSED))
def test_prefill_fused_matches_stages_and_oracle(name):
    """cca_prefill_forward_fused (down-projection + mixing in one kernel) gives
    the q, k, v^T of the separate stage kernels and the oracle's output."""
    shape = FUSED[name]
    _say(f"[fused] {name} {shape}")
    P = make_prefill(shape, seed=2)
    if not shape.use_qk_norm:
        set_taps(P, tau=tau_inv_sqrt_d(shape))
    run = PrefillRun(shape, P)
    L = lib()
    y = torch.empty_like(run.x)
    L.prefill_forward_fused(run.cfg, run.w, run.x, y, run.ws)
    torch.cuda.synchronize()
    B, T, d = shape.batch, shape.seq_len, shape.head_dim
    Tp = run.padded_T()
    qv = lambda: run.ws_view(L.WS_Q, run.qk_dtype(), (B, shape.n_q_heads, Tp, d)).clone()
    kv = lambda: run.ws_view(L.WS_K, run.qk_dtype(), (B, shape.n_kv_heads, Tp, d)).clone()
    vv = lambda: run.ws_view(L.WS_VT, torch.bfloat16, (B, shape.n_kv_heads, d, Tp)).clone()
    fused = (qv(), kv(), vv())
    L.stage_downproj(run.cfg, run.w, run.x, run.ws)
    L.stage_convmix(run.cfg, run.w, run.ws)
    torch.cuda.synchronize()
    staged = (qv(), kv(), vv())
    # the fused kernel keeps qkv~ in fp32, the staged path rounds it to fp16
    # (2^-11 relative) before mixing; both round their outputs (fp16 q, k:
    # 2^-11; bf16 v: 2^-8, where the fp16 step can tip a tie): the two agree
    # to 2e-3 relative L2
    for what, a, b in zip(("q", "k", "vt"), fused, staged):
        fa, fb = a.double().cpu().numpy(), b.double().cpu().numpy()
        r = rel_l2(fa, fb)
        _say(f"[fused] {what}: rel-L2 |fused - staged| = {r:.3e}, bitwise {torch.equal(a, b)}")
        assert r <= 2e-3, what
    ref = O.prefill(P.x, P.weights.f64(), shape)
    assert_parity(tens().to_f64(y), ref, "bf16", name)
