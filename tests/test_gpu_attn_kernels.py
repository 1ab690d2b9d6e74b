"""The two prefill attention kernels, through the C ABI.

cca_config.attn_kernel selects the four-wave kernel (128 query rows per
workgroup) or the eight-wave ping-pong kernel (256 rows, two halves of the
workgroup alternating softmax and matrix products).  Both take the same
tiles in the same order with the same per-lane summation, so their outputs
(y, and the attention output and log-sum-exp kept for the backward pass) must
agree bit for bit; the ping-pong path is also compared with the fp64 oracle
at the bf16 tolerances (max-abs <= 2e-2, relative L2 <= 5e-3).

The shapes cover the ways the 256-row blocks meet the sequence: one query
head per kv head (a block of 256 positions, reaching past the 128-padded
rows), 2, 3 (not a divisor of 4: one head per block), 4 and 8 (two blocks
per kv head) query heads per kv head; lengths of 1, one tile, a ragged tail;
the constant logit shift and the running maximum (norm off, or a temperature
above the shift limit) in one workgroup.
"""

import sys

import numpy as np
import pytest
import torch

import oracle.cca as O
import oracle.backward as BW
from synth import CCAShape, make_prefill, make_upstream_grad, workload
from gpu_helpers import PrefillRun, assert_parity, lib, sample_rows, set_taps, tau_inv_sqrt_d, tens

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    "g1_b2_t300": (CCAShape(batch=2, seq_len=300, d_model=256, n_q_heads=2, n_kv_heads=2,
                            head_dim=64), None),
    "g2_t513": (CCAShape(batch=1, seq_len=513, d_model=256, n_q_heads=4, n_kv_heads=2,
                         head_dim=64), None),
    "g3_t130": (CCAShape(batch=1, seq_len=130, d_model=384, n_q_heads=6, n_kv_heads=2,
                         head_dim=64), None),
    "g4_t1000_base5e5": (CCAShape(batch=1, seq_len=1000, d_model=512, n_q_heads=8, n_kv_heads=2,
                                  head_dim=64, rope_base=500000.0), None),
    "g8_t200": (CCAShape(batch=1, seq_len=200, d_model=256, n_q_heads=8, n_kv_heads=1,
                         head_dim=64, use_value_shift=0), None),
    "t1": (CCAShape(batch=3, seq_len=1, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64), None),
    "t64": (CCAShape(batch=1, seq_len=64, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64), None),
    "norm_off": (CCAShape(batch=1, seq_len=333, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
                          use_qk_mean=0, use_value_shift=0, use_qk_norm=0, rope_base=10000.0),
                 "inv_sqrt_d"),
    "mixed_tau": (CCAShape(batch=1, seq_len=410, d_model=256, n_q_heads=4, n_kv_heads=2,
                           head_dim=64), "mixed"),
}


def _prepare(shape, tau, seed=0):
    P = make_prefill(shape, seed=seed)
    if tau == "inv_sqrt_d":
        set_taps(P, tau=tau_inv_sqrt_d(shape))
    elif tau == "mixed":
        # tau * log2(e) of 11.5 and 72: the constant shift on heads 0 and 2,
        # the running maximum on heads 1 and 3 (one kv head's pair each)
        set_taps(P, tau=np.array([8.0, 50.0, 8.0, 50.0], dtype=np.float32))
    return P


def _o_view(run):
    s = run.shape
    return run.ws_view(lib().WS_O, torch.int16, (s.batch * s.seq_len * s.n_q_heads * s.head_dim,))


@pytest.mark.parametrize("name", list(CASES))
def test_ping_pong_matches_four_wave_and_oracle(name):
    shape, tau = CASES[name]
    _say(f"[attn-kernels] {name} {shape}")
    P = _prepare(shape, tau)
    four = PrefillRun(shape, P, attn="four_wave")
    y4 = four.run()
    o4 = _o_view(four).clone()
    pp = PrefillRun(shape, P, attn="ping_pong")
    ypp = pp.run()
    assert torch.equal(_o_view(pp), o4), f"{name}: attention outputs differ"
    np.testing.assert_array_equal(ypp, y4)
    ref = O.prefill(P.x, P.weights.f64(), shape)
    assert_parity(ypp, ref, shape.dtype, name)


@pytest.mark.parametrize("name", ["cca_prefill_b4_t2048", "ccgqa_prefill_t8192"])
def test_ping_pong_workload(name):
    """Full-size workloads: bitwise against the four-wave kernel, and sampled
    rows against the oracle."""
    shape = workload(name)
    _say(f"[attn-kernels] workload {name}")
    P = make_prefill(shape, seed=0)
    four = PrefillRun(shape, P, attn="four_wave")
    y4 = four.run()
    del four
    torch.cuda.empty_cache()
    pp = PrefillRun(shape, P, attn="ping_pong")
    ypp = pp.run()
    np.testing.assert_array_equal(ypp, y4)
    rows = sample_rows(shape.seq_len, 24)
    ref = O.prefill(P.x, P.weights.f64(), shape, rows=rows)
    assert_parity(ypp[:, rows], ref, "bf16", name)


def test_ping_pong_training_lse_and_gradients():
    """forward_train keeps the log-sum-exp that the backward pass reads: with
    the ping-pong kernel every gradient equals the four-wave one bit for bit,
    and the parameter gradients match the fp64 backward oracle."""
    from test_gpu_backward import GRADS, TrainRun, bf16_bounds, check_grads
    shape = CCAShape(batch=1, seq_len=300, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64)
    _say(f"[attn-kernels] training {shape}")
    P = make_prefill(shape, seed=3)
    dyB = make_upstream_grad(shape, seed=3)
    got = {}
    for kern in ("four_wave", "ping_pong"):
        run = TrainRun(shape, P, dyB, attn=kern)
        run.forward()
        run.backward()
        torch.cuda.synchronize()
        got[kern] = {n: getattr(run.g, n).clone() for n in GRADS}
    for n in GRADS:
        a, b = got["four_wave"][n], got["ping_pong"][n]
        iv = torch.int16 if a.element_size() == 2 else torch.int32
        assert torch.equal(a.view(iv), b.view(iv)), n
    ref = BW.prefill_backward(P.x, P.weights.f64(), shape, dyB.dy)
    check_grads({n: tens().to_f64(got["ping_pong"][n]) for n in GRADS}, ref, "bf16", "ping_pong",
                bf16_bounds(P, dyB, shape, ref))
