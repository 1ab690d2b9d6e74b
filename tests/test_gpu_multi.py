"""GPU tests of the multi-token decode step (cca_decode_multi and its paged
form) through the C ABI, against oracle.decode_multi sequence by sequence:
outputs, the k / v rows written at slots L .. L+m-1, the rolled state, and
the untouched rest of the cache."""

import sys

import numpy as np
import pytest
import torch

import oracle.cca as O
from synth import CCAShape, make_decode
from gpu_helpers import assert_parity, lib, rel_l2, tens, upload_weights

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _upload(D, dev="cuda"):
    T, L = tens(), lib()
    return L.State(k_cache=T.to_device(D.k_cache_s, dev), v_cache=T.to_device(D.v_cache_s, dev),
                   capacity=D.capacity, conv_q=T.to_device(D.conv_q_s, dev),
                   conv_k=T.to_device(D.conv_k_s, dev), vshift=T.to_device(D.vshift_s, dev))


def _new_tokens(shape, m, seed):
    """x_new [B, m, E] in storage precision and as float64."""
    from synth.generate import round_to_bf16_bits, bf16_bits_to_f64
    x = np.random.default_rng(seed).standard_normal((shape.batch, m, shape.d_model))
    if shape.dtype == "bf16":
        bits = round_to_bf16_bits(x)
        return bits, bf16_bits_to_f64(bits)
    f = x.astype(np.float32)
    return f, f.astype(np.float64)


CASES = {
    # name: (shape, lens, m)
    "bf16_g4_m2": (CCAShape(batch=5, seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                            rope_base=500000.0, cache_len=3000), [0, 1, 62, 1024, 2999], 2),
    "bf16_g4_m5": (CCAShape(batch=4, seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                            rope_base=500000.0, cache_len=700), [0, 60, 123, 700], 5),
    "bf16_g1_m16": (CCAShape(batch=3, seq_len=1, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                             cache_len=300), [3, 128, 300], 16),
    "bf16_d128_m3": (CCAShape(batch=2, seq_len=1, d_model=256, n_q_heads=2, n_kv_heads=2,
                              head_dim=128, cache_len=200), [17, 200], 3),
    "f32_d16_m4": (CCAShape(batch=3, seq_len=1, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=16,
                            dtype="f32", cache_len=500), [0, 250, 500], 4),
}


def _run_multi(shape, D, lens, m, seed, paged=False, page=64, qk_mean="pre_post"):
    T, Lb = tens(), lib()
    Lmax = shape.cache_len
    cfg = Lb.make_config(shape, qk_mean=qk_mean)
    st = _upload(D)
    xs, x64 = _new_tokens(shape, m, seed)
    x_new = T.to_device(xs)
    y = torch.empty_like(x_new)
    ws = T.workspace(Lb.decode_multi_workspace_size(cfg, m, Lmax))
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    if not paged:
        Lb.decode_multi(cfg, upload_weights(D.weights), x_new, m, dl, Lmax, st, st, y, ws)
        torch.cuda.synchronize()
        return y, st, x64
    from test_gpu_paged import _paged_from
    mpps = (D.capacity + page - 1) // page
    kp, table = _paged_from(st.k_cache, page, mpps, seed=seed)
    vp, _ = _paged_from(st.v_cache, page, mpps, seed=seed)
    ps = Lb.PagedState(kp, vp, table, page, st.conv_q, st.conv_k, st.vshift)
    Lb.decode_multi_paged(cfg, upload_weights(D.weights), x_new, m, dl, Lmax, ps, ps, y, ws)
    torch.cuda.synchronize()
    return y, (ps, kp, vp, table), x64


@pytest.mark.parametrize("name", list(CASES))
def test_decode_multi_parity(name):
    shape, lens, m = CASES[name]
    _say(f"[multi] {name} lens={lens} m={m}")
    D = make_decode(shape, seed=31, capacity=shape.cache_len + m)
    y, st, x64 = _run_multi(shape, D, lens, m, seed=5)
    T = tens()
    w = D.weights.f64()
    cq, ck, vs = D.state_f64()
    yy = T.to_f64(y)
    kc, vc = T.to_f64(st.k_cache), T.to_f64(st.v_cache)
    tol = 5e-3 if shape.dtype == "bf16" else 1e-5
    for b, L_ in enumerate(lens):
        K = D.cache_f64(b, "k")[None, :, :L_]
        V = D.cache_f64(b, "v")[None, :, :L_]
        ref, new = O.decode_multi(x64[b:b + 1], w, shape, K, V, cq[b:b + 1], ck[b:b + 1], vs[b:b + 1])
        assert_parity(yy[b:b + 1], ref, shape.dtype, f"multi b={b} L={L_}")
        assert rel_l2(kc[b, :, L_:L_ + m], new["k_new"][0]) < tol
        assert rel_l2(vc[b, :, L_:L_ + m], new["v_new"][0]) < tol
        assert rel_l2(T.to_f64(st.conv_q)[b], new["conv_q"][0]) < tol
        assert rel_l2(T.to_f64(st.conv_k)[b], new["conv_k"][0]) < tol
        if shape.n_kv_heads % 2 == 0:
            assert rel_l2(T.to_f64(st.vshift)[b], new["vshift"][0]) < tol
        keep = [i for i in range(D.capacity) if not (L_ <= i < L_ + m)]
        full_k = T.to_f64(T.to_device(D.k_cache_s))[b]
        np.testing.assert_array_equal(kc[b][:, keep], full_k[:, keep])


def test_decode_multi_one_token_equals_varlen_step():
    """n_new = 1 is the per-sequence-length single-token step, bit for bit."""
    shape, lens, _ = CASES["bf16_g4_m2"]
    D = make_decode(shape, seed=32, capacity=shape.cache_len + 1)
    T, Lb = tens(), lib()
    y1, st1, _ = _run_multi(shape, D, lens, 1, seed=6)
    cfg = Lb.make_config(shape)
    st2 = _upload(D)
    xs, _ = _new_tokens(shape, 1, 6)
    x_t = T.to_device(xs[:, 0])
    y2 = torch.empty_like(x_t)
    ws = T.workspace(Lb.decode_workspace_size(cfg, shape.cache_len))
    Lb.decode_step_varlen(cfg, upload_weights(D.weights), x_t,
                          torch.tensor(lens, dtype=torch.int32, device="cuda"), shape.cache_len,
                          st2, st2, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1[:, 0].view(torch.int16), y2.view(torch.int16))
    assert torch.equal(st1.k_cache.view(torch.int16), st2.k_cache.view(torch.int16))
    assert torch.equal(st1.conv_q.view(torch.int16), st2.conv_q.view(torch.int16))


def test_decode_multi_paged_equals_contiguous():
    shape, lens, m = CASES["bf16_g4_m5"]
    _say(f"[multi] paged lens={lens} m={m}")
    D = make_decode(shape, seed=33, capacity=shape.cache_len + m)
    y1, st1, _ = _run_multi(shape, D, lens, m, seed=7)
    y2, (ps, kp, vp, table), _ = _run_multi(shape, D, lens, m, seed=7, paged=True, page=32)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    from test_gpu_paged import _gather
    for b, L_ in enumerate(lens):
        rows = list(range(L_, L_ + m))
        assert torch.equal(_gather(kp, table, b, rows).view(torch.int16),
                           st1.k_cache[b, :, L_:L_ + m].view(torch.int16))
        assert torch.equal(_gather(vp, table, b, rows).view(torch.int16),
                           st1.v_cache[b, :, L_:L_ + m].view(torch.int16))


def test_decode_multi_full_length():
    """Four new tokens per sequence at the decode workload's shape (B=64,
    16 query / 4 kv heads of 64) with lengths up to 32764, so the 32768 keys
    split into two 16384-key chunks: contiguous and paged (32-row pages, 513
    per chunk) agree bit for bit, and 6 sequences match the oracle."""
    from synth import workload
    m, Lmax = 4, 32764
    shape = workload("ccgqa_decode_b64_l32768").with_(cache_len=Lmax)
    rng = np.random.default_rng(61)
    lens = rng.integers(30000, Lmax + 1, size=shape.batch).astype(np.int32).tolist()
    lens[0] = Lmax
    _say(f"[multi] full length B={shape.batch} Lmax={Lmax} m={m}")
    D = make_decode(shape, seed=61, capacity=Lmax + m)
    y1, st1, x64 = _run_multi(shape, D, lens, m, seed=62)
    y2, (ps, kp, vp, table), _ = _run_multi(shape, D, lens, m, seed=62, paged=True, page=32)
    _say("[multi] full length: steps done")
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    from test_gpu_paged import _gather
    for b in (0, 1, 63):
        rows = list(range(lens[b], lens[b] + m))
        assert torch.equal(_gather(kp, table, b, rows).view(torch.int16),
                           st1.k_cache[b, :, lens[b]:lens[b] + m].view(torch.int16))
    T = tens()
    w = D.weights.f64()
    cq, ck, vs = D.state_f64()
    yy = T.to_f64(y1)
    for b in [0] + sorted(rng.choice(np.arange(1, shape.batch), size=5, replace=False).tolist()):
        L_ = lens[b]
        ref, _ = O.decode_multi(x64[b:b + 1], w, shape, D.cache_f64(b, "k")[None, :, :L_],
                                D.cache_f64(b, "v")[None, :, :L_], cq[b:b + 1], ck[b:b + 1],
                                vs[b:b + 1])
        assert_parity(yy[b:b + 1], ref, "bf16", f"multi full b={b} L={L_}")
