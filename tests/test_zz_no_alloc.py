"""The allocation-free decode step (cca_decode_step_noalloc) against
cca_decode_step with a caller workspace, through the C ABI: two calls in a
row, the decode workload's shape (64 sequences, 32768 cached tokens) and then
a smaller one (8 sequences, 1000 cached tokens), each bit for bit equal to
the workspace entry point in its output, its new cache rows and its rolled
state.  The two share every kernel; only the workspace differs."""

import sys

import numpy as np
import pytest
import torch

from synth import make_decode, workload
from gpu_helpers import lib, tens, upload_weights

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _state(D):
    T, L = tens(), lib()
    return L.State(k_cache=T.to_device(D.k_cache_s), v_cache=T.to_device(D.v_cache_s),
                   capacity=D.capacity, conv_q=T.to_device(D.conv_q_s),
                   conv_k=T.to_device(D.conv_k_s), vshift=T.to_device(D.vshift_s))


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_decode_matches_workspace_step(order):
    T, L = tens(), lib()
    base = workload("ccgqa_decode_b64_l32768")
    for step, shape in enumerate((base, base.with_(batch=8, cache_len=1000))):
        _say(f"[noalloc] call {step}: B={shape.batch} L={shape.cache_len}")
        D = make_decode(shape, seed=70 + step, capacity=shape.cache_len + 1)
        cfg = L.make_config(shape)
        assert L.decode_workspace_size(cfg, shape.cache_len) <= L.NOALLOC_SCRATCH_BYTES
        w = upload_weights(D.weights)
        x_t = T.to_device(D.x_s)
        ref_st, st = _state(D), _state(D)
        y_ref, y = torch.empty_like(x_t), torch.empty_like(x_t)
        ws = T.workspace(L.decode_workspace_size(cfg, shape.cache_len))
        L.decode_step(cfg, w, x_t, shape.cache_len, ref_st, ref_st, y_ref, ws)
        L.decode_step_noalloc(cfg, w, x_t, shape.cache_len, st, st, y)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref)), "y_t"
        Lc = shape.cache_len
        assert torch.equal(_bits(st.k_cache[:, :, Lc]), _bits(ref_st.k_cache[:, :, Lc]))
        assert torch.equal(_bits(st.v_cache[:, :, Lc]), _bits(ref_st.v_cache[:, :, Lc]))
        for a, b in ((st.conv_q, ref_st.conv_q), (st.conv_k, ref_st.conv_k),
                     (st.vshift, ref_st.vshift)):
            assert torch.equal(_bits(a), _bits(b))
        assert np.all(np.isfinite(tens().to_f64(y)))
        del ws, st, ref_st
        torch.cuda.empty_cache()
