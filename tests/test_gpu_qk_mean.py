"""GPU parity of the q-k-mean's second reading, through the C ABI.

The library's default (cca_config.qk_mean_mode = CCA_QK_MEAN_PRE_POST) adds
the mean of the pre- and post-convolution q and k to the convolved tensors,
the oracle's Readings(qk_mean="M2"); every other GPU test runs it.  Here the
switch CCA_QK_MEAN_PRE (the mean of the pre-convolution values only) is
checked against Readings(qk_mean="M1") on prefill, the decode state a
prefill leaves, single- and multi-token decode steps and the backward pass;
and the two readings are shown to give different results on the GPU, each
matching its own oracle.
"""

import sys

import numpy as np
import pytest
import torch

import oracle.backward as BW
import oracle.cca as O
from synth import CCAShape, make_decode, make_prefill, make_upstream_grad
from gpu_helpers import PrefillRun, assert_parity, lib, rel_l2, tens, upload_weights
from test_gpu_backward import TrainRun, bf16_bounds, check_grads
from test_gpu_multi import _run_multi

pytestmark = pytest.mark.gpu

PRE = O.Readings(qk_mean="M1")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SHAPES = {
    "bf16_g1": CCAShape(batch=2, seq_len=200, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64),
    "bf16_g2_ragged": CCAShape(batch=2, seq_len=300, d_model=256, n_q_heads=4, n_kv_heads=2,
                               head_dim=64, rope_base=10000.0),
    "bf16_g4_base5e5": CCAShape(batch=1, seq_len=200, d_model=512, n_q_heads=8, n_kv_heads=2,
                                head_dim=64, rope_base=500000.0),
    "bf16_d16": CCAShape(batch=2, seq_len=130, d_model=128, n_q_heads=2, n_kv_heads=2, head_dim=16),
    "bf16_d128": CCAShape(batch=1, seq_len=150, d_model=256, n_q_heads=2, n_kv_heads=2,
                          head_dim=128),
    "f32_d32_g2_ragged": CCAShape(batch=2, seq_len=190, d_model=128, n_q_heads=4, n_kv_heads=2,
                                  head_dim=32, dtype="f32"),
    "f32_d64_g4": CCAShape(batch=1, seq_len=260, d_model=256, n_q_heads=8, n_kv_heads=2,
                           head_dim=64, rope_base=500000.0, dtype="f32"),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_prefill_pre_reading(name):
    shape = SHAPES[name]
    _say(f"[qk-mean pre] prefill {name} {shape}")
    P = make_prefill(shape, seed=4)
    y = PrefillRun(shape, P, qk_mean="pre").run()
    assert_parity(y, O.prefill(P.x, P.weights.f64(), shape, readings=PRE), shape.dtype, name)


@pytest.mark.parametrize("name", ["bf16_g4_base5e5", "f32_d64_g4"])
def test_readings_differ_on_gpu(name):
    """Each reading matches its own oracle, and the two outputs differ by far
    more than the parity tolerance."""
    shape = SHAPES[name]
    _say(f"[qk-mean] both readings {name}")
    P = make_prefill(shape, seed=6)
    w = P.weights.f64()
    y_pp = PrefillRun(shape, P).run()
    y_pre = PrefillRun(shape, P, qk_mean="pre").run()
    assert_parity(y_pp, O.prefill(P.x, w, shape), shape.dtype, f"{name} pre+post")
    assert_parity(y_pre, O.prefill(P.x, w, shape, readings=PRE), shape.dtype, f"{name} pre")
    assert rel_l2(y_pre, y_pp) > 5e-2


def test_prefill_state_then_decode_pre():
    """prefill(x[:L]) with state -> two decode steps, all under the pre-only
    reading, against the oracle prefill over L+1 / L+2 tokens."""
    full = CCAShape(batch=2, seq_len=39, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                    rope_base=500000.0)
    P = make_prefill(full, seed=9)
    Lp = 37
    pshape = full.with_(seq_len=Lp)
    Pp = make_prefill(full, seed=9)
    Pp.x_s = np.ascontiguousarray(P.x_s[:, :Lp])
    Pp.x = P.x[:, :Lp]
    run = PrefillRun(pshape, Pp, capacity=64, qk_mean="pre")
    run.run()
    _, lat = O.prefill(Pp.x, P.weights.f64(), pshape, readings=PRE, intermediates=True)
    K, V, cq, ck, vs = O.prefill_state(lat, pshape, PRE)
    T, L = tens(), lib()
    st = run.state
    assert rel_l2(T.to_f64(st.k_cache)[:, :, :Lp], K) < 5e-3
    assert rel_l2(T.to_f64(st.v_cache)[:, :, :Lp], V) < 5e-3
    dcfg = L.make_config(full.with_(seq_len=1), qk_mean="pre")
    ref_full = O.prefill(P.x, P.weights.f64(), full, readings=PRE)
    for step, pos in enumerate((Lp, Lp + 1)):
        x_t = T.to_device(np.ascontiguousarray(P.x_s[:, pos]))
        y_t = torch.empty_like(x_t)
        ws = T.workspace(L.decode_workspace_size(dcfg, pos))
        L.decode_step(dcfg, run.w, x_t, pos, st, st, y_t, ws)
        torch.cuda.synchronize()
        assert_parity(T.to_f64(y_t), ref_full[:, pos], "bf16", f"pre decode step {step}")


@pytest.mark.parametrize("L_", [0, 5, 1025])
def test_decode_pre_reading(L_):
    shape = CCAShape(batch=3, seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                     rope_base=500000.0, cache_len=L_)
    _say(f"[qk-mean pre] decode L={L_}")
    D = make_decode(shape, seed=L_ + 40, capacity=L_ + 2)
    T, Lb = tens(), lib()
    st = Lb.State(k_cache=T.to_device(D.k_cache_s), v_cache=T.to_device(D.v_cache_s),
                  capacity=D.capacity, conv_q=T.to_device(D.conv_q_s),
                  conv_k=T.to_device(D.conv_k_s), vshift=T.to_device(D.vshift_s))
    cfg = Lb.make_config(shape, qk_mean="pre")
    x_t = T.to_device(D.x_s)
    y_t = torch.empty_like(x_t)
    ws = T.workspace(Lb.decode_workspace_size(cfg, L_))
    Lb.decode_step(cfg, upload_weights(D.weights), x_t, L_, st, st, y_t, ws)
    torch.cuda.synchronize()
    w = D.weights.f64()
    cq, ck, vs = D.state_f64()
    kc = T.to_f64(st.k_cache)
    for b in range(shape.batch):
        ref, new = O.decode_step(D.x[b:b + 1], w, shape, D.cache_f64(b, "k")[None],
                                 D.cache_f64(b, "v")[None], cq[b:b + 1], ck[b:b + 1], vs[b:b + 1],
                                 readings=PRE)
        assert_parity(T.to_f64(y_t)[b:b + 1], ref, "bf16", f"pre decode b={b}")
        assert rel_l2(kc[b, :, L_], new["k_new"][0]) < 5e-3


def test_decode_multi_pre_reading():
    shape = CCAShape(batch=4, seq_len=1, d_model=256, n_q_heads=8, n_kv_heads=2, head_dim=64,
                     rope_base=500000.0, cache_len=700)
    lens, m = [0, 60, 123, 700], 3
    _say("[qk-mean pre] multi-token decode")
    D = make_decode(shape, seed=17, capacity=shape.cache_len + m)
    y, st, x64 = _run_multi(shape, D, lens, m, seed=17, qk_mean="pre")
    y = tens().to_f64(y)
    w = D.weights.f64()
    cq, ck, vs = D.state_f64()
    for b, L_ in enumerate(lens):
        ref, _ = O.decode_multi(x64[b:b + 1], w, shape, D.cache_f64(b, "k")[None, :, :L_],
                                D.cache_f64(b, "v")[None, :, :L_], cq[b:b + 1], ck[b:b + 1],
                                vs[b:b + 1], readings=PRE)
        assert_parity(y[b:b + 1], ref, "bf16", f"pre multi b={b} L={L_}")


@pytest.mark.parametrize("name", ["bf16_g2_ragged", "bf16_g4_base5e5", "f32_d64_g4"])
def test_backward_pre_reading(name):
    shape = SHAPES[name]
    _say(f"[qk-mean pre] backward {name}")
    P = make_prefill(shape, seed=0)
    dyB = make_upstream_grad(shape, seed=0)
    run = TrainRun(shape, P, dyB, qk_mean="pre")
    run.forward()
    got = run.backward()
    ref = BW.prefill_backward(P.x, P.weights.f64(), shape, dyB.dy, readings=PRE)
    bounds = bf16_bounds(P, dyB, shape, ref, readings=PRE) if shape.dtype == "bf16" else None
    check_grads(got, ref, shape.dtype, f"pre {name}", bounds)
