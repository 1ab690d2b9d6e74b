"""GPU parity of the grouped channel-conv reading (cca_config.chan_conv_mode
= CCA_CHAN_GROUPED) against the fp64 oracle's Readings(chan_conv="grouped"),
through the C ABI: prefill outputs, the decode state a prefill leaves (a
window of (k_s - 1) + (k_c - 1) pre-conv rows), single- and multi-token
decode steps from it.  Tolerances as for the default reading: bf16 I/O
max-abs <= 2e-2 and relative L2 <= 5e-3; fp32 relative L2 <= 1e-5.  In bf16
mode the channel conv multiplies fp16 copies of a and W (fp32 accumulation),
the precision the stored q and k have anyway."""

import sys

import numpy as np
import pytest
import torch

import oracle.cca as O
from synth import CCAShape, add_chan_dense, make_prefill
from gpu_helpers import PrefillRun, assert_parity, lib, rel_l2, tens

pytestmark = pytest.mark.gpu
GROUPED = O.Readings(chan_conv="grouped")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _prefill(shape, seed):
    P = make_prefill(shape, seed=seed)
    add_chan_dense(P.weights, shape, seed)
    return P


CASES = {
    "bf16_g1_d64_ragged": CCAShape(batch=2, seq_len=300, d_model=256, n_q_heads=4, n_kv_heads=4,
                                   head_dim=64, rope_base=10000.0),
    "bf16_g2_d32_kc2": CCAShape(batch=1, seq_len=200, d_model=256, n_q_heads=8, n_kv_heads=4,
                                head_dim=32, chan_conv_k=2),
    "bf16_d16_ks2_kc3": CCAShape(batch=2, seq_len=130, d_model=128, n_q_heads=2, n_kv_heads=2,
                                 head_dim=16, seq_conv_k=2, chan_conv_k=3),
    "bf16_kc1": CCAShape(batch=1, seq_len=129, d_model=256, n_q_heads=4, n_kv_heads=2,
                         head_dim=64, chan_conv_k=1),
    "bf16_switches_off": CCAShape(batch=1, seq_len=160, d_model=256, n_q_heads=4, n_kv_heads=4,
                                  head_dim=64, use_qk_mean=0, use_value_shift=0),
    "f32_d64_g2": CCAShape(batch=2, seq_len=190, d_model=128, n_q_heads=4, n_kv_heads=2,
                           head_dim=64, dtype="f32"),
    "f32_d16_g4": CCAShape(batch=1, seq_len=70, d_model=64, n_q_heads=4, n_kv_heads=1,
                           head_dim=16, dtype="f32", use_value_shift=0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_grouped_prefill_parity(name):
    shape = CASES[name]
    _say(f"[grouped prefill] {name} {shape}")
    P = _prefill(shape, seed=3)
    run = PrefillRun(shape, P, chan_conv="grouped")
    y = run.run()
    ref = O.prefill(P.x, P.weights.f64(), shape, readings=GROUPED)
    assert_parity(y, ref, shape.dtype, name)
    # and it is not the default reading's result
    other = O.prefill(P.x, P.weights.f64(), shape)
    assert rel_l2(y, other) > 1e-2


def test_grouped_prefill_workload_rows():
    """The prefill workload's shape (B4, T2048, E2048, 8 + 8 heads of 64) under
    the grouped reading, on sampled query rows of the first sequence."""
    shape = CCAShape(batch=1, seq_len=2048, d_model=2048, n_q_heads=8, n_kv_heads=8, head_dim=64)
    _say(f"[grouped prefill] workload rows {shape}")
    P = _prefill(shape, seed=4)
    run = PrefillRun(shape, P, chan_conv="grouped")
    y = run.run()
    rows = [0, 1, 2, 3, 127, 128, 1000, 2047]
    ref = O.prefill(P.x, P.weights.f64(), shape, rows=rows, readings=GROUPED)
    assert_parity(y[:, rows], ref, "bf16", "grouped workload rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_grouped_prefill_state_then_decode(dtype):
    """prefill(x[:Lp]) with state -> decode(x[Lp]) -> decode_multi(x[Lp+1 ..
    Lp+3]) equals the oracle prefill over the longer sequence at those
    positions; the state the prefill wrote equals the oracle's."""
    full = CCAShape(batch=2, seq_len=43, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    seq_conv_k=3, chan_conv_k=4, dtype=dtype)
    _say(f"[grouped prefill->decode] {dtype}")
    P = _prefill(full, seed=9)
    Lp = 39
    pshape = full.with_(seq_len=Lp)
    Pp = _prefill(full, seed=9)
    Pp.x_s = np.ascontiguousarray(P.x_s[:, :Lp])
    Pp.x = P.x[:, :Lp]
    run = PrefillRun(pshape, Pp, capacity=64, chan_conv="grouped")
    run.run()
    w = P.weights.f64()
    _, lat = O.prefill(Pp.x, w, pshape, readings=GROUPED, intermediates=True)
    K, V, cq, ck, vs = O.prefill_state(lat, pshape, GROUPED)
    T = tens()
    st = run.state
    assert cq.shape[1] == (3 - 1) + (4 - 1) == st.conv_q.shape[1]
    tol = 5e-3 if dtype == "bf16" else 1e-5
    assert rel_l2(T.to_f64(st.k_cache)[:, :, :Lp], K) < tol
    assert rel_l2(T.to_f64(st.v_cache)[:, :, :Lp], V) < tol
    assert rel_l2(T.to_f64(st.conv_q), cq) < tol
    assert rel_l2(T.to_f64(st.conv_k), ck) < tol
    assert rel_l2(T.to_f64(st.vshift), vs) < tol
    L = lib()
    ref_full = O.prefill(P.x, w, full, readings=GROUPED)
    dshape = full.with_(seq_len=1)
    cfg = L.make_config(dshape, chan_conv="grouped")
    x_t = T.to_device(np.ascontiguousarray(P.x_s[:, Lp]))
    y_t = torch.empty_like(x_t)
    ws = T.workspace(L.decode_workspace_size(cfg, Lp))
    L.decode_step(cfg, run.w, x_t, Lp, st, st, y_t, ws)
    torch.cuda.synchronize()
    assert_parity(T.to_f64(y_t), ref_full[:, Lp], dtype, "grouped decode step")
    m = 3
    x_new = T.to_device(np.ascontiguousarray(P.x_s[:, Lp + 1:Lp + 1 + m]))
    y_new = torch.empty_like(x_new)
    ws = T.workspace(L.decode_multi_workspace_size(cfg, m, Lp + 1))
    lens = torch.full((full.batch,), Lp + 1, dtype=torch.int32, device="cuda")
    L.decode_multi(cfg, run.w, x_new, m, lens, Lp + 1, st, st, y_new, ws)
    torch.cuda.synchronize()
    assert_parity(T.to_f64(y_new), ref_full[:, Lp + 1:Lp + 1 + m], dtype, "grouped decode multi")
    # the rolled window after all Lp + 1 + m tokens
    _, lat_all = O.prefill(P.x, w, full, readings=GROUPED, intermediates=True)
    _, _, cq2, ck2, _ = O.prefill_state(lat_all, full, GROUPED)
    assert rel_l2(T.to_f64(st.conv_q), cq2) < tol
    assert rel_l2(T.to_f64(st.conv_k), ck2) < tol


def test_grouped_paged_and_varlen_equal_contiguous():
    """Under the grouped reading the paged prefill writes the same cache rows
    and window as the contiguous one, and the per-sequence-length and paged
    decode steps equal the uniform step bit for bit when every length is the
    same."""
    from test_gpu_paged import _gather, _paged_from
    shape = CCAShape(batch=2, seq_len=150, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64)
    _say(f"[grouped] paged / varlen {shape}")
    P = _prefill(shape, seed=12)
    T, L = tens(), lib()
    run = PrefillRun(shape, P, capacity=160, chan_conv="grouped")
    run.run()
    st = run.state
    page = 32
    mpps = (160 + page - 1) // page
    kp, table = _paged_from(torch.zeros_like(st.k_cache), page, mpps, seed=3)
    vp, _ = _paged_from(torch.zeros_like(st.v_cache), page, mpps, seed=3)
    pst = L.PagedState(kp, vp, table, page, torch.zeros_like(st.conv_q), torch.zeros_like(st.conv_k),
                       torch.zeros_like(st.vshift))
    y2 = torch.empty_like(run.y)
    L.prefill_forward_paged(run.cfg, run.w, run.x, y2, run.ws, pst)
    torch.cuda.synchronize()
    assert torch.equal(run.y.view(torch.int16), y2.view(torch.int16))
    for b in range(shape.batch):
        rows = list(range(shape.seq_len))
        assert torch.equal(_gather(kp, table, b, rows).view(torch.int16),
                           st.k_cache[b, :, :shape.seq_len].view(torch.int16))
    assert torch.equal(pst.conv_q.view(torch.int16), st.conv_q.view(torch.int16))
    # one more token: uniform, per-sequence-length and paged steps agree
    dcfg = L.make_config(shape.with_(seq_len=1), chan_conv="grouped")
    xt = T.to_device(np.ascontiguousarray(
        np.random.default_rng(2).standard_normal((shape.batch, shape.d_model)).astype(np.float32)))
    xt = xt.to(torch.bfloat16)
    Lc = shape.seq_len
    st_u = L.State(st.k_cache.clone(), st.v_cache.clone(), st.capacity, st.conv_q.clone(),
                   st.conv_k.clone(), st.vshift.clone())
    ya, yb, yc = torch.empty_like(xt), torch.empty_like(xt), torch.empty_like(xt)
    ws = T.workspace(L.decode_workspace_size(dcfg, Lc))
    L.decode_step(dcfg, run.w, xt, Lc, st_u, st_u, ya, ws)
    dl = torch.full((shape.batch,), Lc, dtype=torch.int32, device="cuda")
    L.decode_step_varlen(dcfg, run.w, xt, dl, Lc, st, st, yb, ws)
    L.decode_step_paged(dcfg, run.w, xt, dl, Lc, pst, pst, yc, ws)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    assert torch.equal(ya.view(torch.int16), yc.view(torch.int16))
    assert torch.equal(st_u.conv_q.view(torch.int16), pst.conv_q.view(torch.int16))
