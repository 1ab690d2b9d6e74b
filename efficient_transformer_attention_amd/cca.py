"""ctypes binding of libcca (include/cca.h).

Argument marshalling only: torch tensors are passed as device pointers and
torch's current HIP stream as the stream; every step of the forward and
backward passes runs in the library's HIP kernels.  There is no fallback: if libcca.so is missing
or a call returns a non-OK status, this module raises.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
# CCA_LIBRARY may name another build of the same library (same ABI).
LIB_PATH = os.environ.get("CCA_LIBRARY") or os.path.join(PKG, "libcca.so")

CCA_OK, CCA_ERR_INVALID_ARG, CCA_ERR_UNSUPPORTED, CCA_ERR_WORKSPACE, CCA_ERR_HIP = range(5)
CCA_BF16, CCA_F32 = 0, 1
CCA_CHAN_PER_HEAD, CCA_CHAN_GROUPED = 0, 1
CCA_QK_MEAN_PRE_POST, CCA_QK_MEAN_PRE = 0, 1
CCA_ATTN_AUTO, CCA_ATTN_FOUR_WAVE, CCA_ATTN_PING_PONG = 0, 1, 2
WS_QKV, WS_Q, WS_K, WS_VT, WS_O, WS_PART, WS_SPLITK, WS_COUNT = range(8)
NOALLOC_SCRATCH_BYTES = 16 << 20       # CCA_NOALLOC_SCRATCH

# Every entry point declared in include/cca.h.
EXPORTS = (
    "cca_validate_config", "cca_prefill_workspace_size", "cca_decode_workspace_size",
    "cca_prefill_forward", "cca_decode_step", "cca_decode_step_varlen", "cca_status_string",
    "cca_prefill_workspace_layout", "cca_decode_workspace_layout",
    "cca_stage_downproj", "cca_stage_convmix", "cca_stage_attention", "cca_stage_upproj",
    "cca_stage_decode_downproj", "cca_stage_decode_mix", "cca_stage_decode_attention",
    "cca_stage_decode_upproj",
    "cca_train_workspace_size", "cca_prefill_forward_train", "cca_prefill_backward",
    "cca_decode_step_paged", "cca_prefill_forward_paged",
    "cca_decode_multi_workspace_size", "cca_decode_multi", "cca_decode_multi_paged",
    "cca_prefill_forward_fused", "cca_decode_step_noalloc",
)


class CCAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Config(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("seq_len", C.c_int32), ("d_model", C.c_int32),
        ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("seq_conv_k", C.c_int32), ("chan_conv_k", C.c_int32),
        ("use_qk_mean", C.c_int32), ("use_value_shift", C.c_int32), ("use_qk_norm", C.c_int32),
        ("rope_base", C.c_float), ("norm_eps", C.c_float), ("dtype", C.c_int32),
        ("chan_conv_mode", C.c_int32), ("qk_mean_mode", C.c_int32), ("attn_kernel", C.c_int32),
    ]


class _Weights(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_o", C.c_void_p),
                ("q_seq_taps", C.c_void_p), ("k_seq_taps", C.c_void_p),
                ("q_chan_taps", C.c_void_p), ("k_chan_taps", C.c_void_p), ("tau", C.c_void_p),
                ("q_chan_dense", C.c_void_p), ("k_chan_dense", C.c_void_p)]


class _Grads(C.Structure):
    _fields_ = [("x", C.c_void_p), ("w_qkv", C.c_void_p), ("w_o", C.c_void_p),
                ("q_seq_taps", C.c_void_p), ("k_seq_taps", C.c_void_p),
                ("q_chan_taps", C.c_void_p), ("k_chan_taps", C.c_void_p), ("tau", C.c_void_p)]


class _State(C.Structure):
    _fields_ = [("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("capacity", C.c_int32),
                ("reserved", C.c_int32), ("conv_q", C.c_void_p), ("conv_k", C.c_void_p),
                ("vshift", C.c_void_p)]


class _PagedState(C.Structure):
    _fields_ = [("k_pages", C.c_void_p), ("v_pages", C.c_void_p), ("block_table", C.c_void_p),
                ("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("max_pages_per_seq", C.c_int32), ("reserved", C.c_int32),
                ("conv_q", C.c_void_p), ("conv_k", C.c_void_p), ("vshift", C.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m efficient_transformer_attention_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P = C.POINTER
    cfgp, wp, sp, vp, sz = P(Config), P(_Weights), P(_State), C.c_void_p, C.c_size_t
    sig = {
        "cca_validate_config": (C.c_int, [cfgp]),
        "cca_prefill_workspace_size": (sz, [cfgp]),
        "cca_decode_workspace_size": (sz, [cfgp, C.c_int32]),
        "cca_prefill_workspace_layout": (C.c_int, [cfgp, P(sz)]),
        "cca_decode_workspace_layout": (C.c_int, [cfgp, C.c_int32, P(sz)]),
        "cca_prefill_forward": (C.c_int, [cfgp, wp, vp, vp, sp, vp, sz, vp]),
        "cca_decode_step": (C.c_int, [cfgp, wp, vp, C.c_int32, sp, sp, vp, vp, sz, vp]),
        "cca_decode_step_noalloc": (C.c_int, [cfgp, wp, vp, C.c_int32, sp, sp, vp, vp]),
        "cca_decode_step_varlen": (C.c_int, [cfgp, wp, vp, vp, C.c_int32, sp, sp, vp, vp, sz, vp]),
        "cca_status_string": (C.c_char_p, [C.c_int]),
        "cca_stage_downproj": (C.c_int, [cfgp, wp, vp, vp, sz, vp]),
        "cca_stage_convmix": (C.c_int, [cfgp, wp, sp, vp, sz, vp]),
        "cca_stage_attention": (C.c_int, [cfgp, wp, vp, sz, vp]),
        "cca_stage_upproj": (C.c_int, [cfgp, wp, vp, vp, sz, vp]),
        "cca_stage_decode_downproj": (C.c_int, [cfgp, wp, vp, C.c_int32, vp, sz, vp]),
        "cca_stage_decode_mix": (C.c_int, [cfgp, wp, C.c_int32, sp, sp, vp, sz, vp]),
        "cca_stage_decode_attention": (C.c_int, [cfgp, wp, C.c_int32, sp, vp, sz, vp]),
        "cca_stage_decode_upproj": (C.c_int, [cfgp, wp, C.c_int32, vp, vp, sz, vp]),
        "cca_train_workspace_size": (sz, [cfgp]),
        "cca_prefill_forward_train": (C.c_int, [cfgp, wp, vp, vp, vp, sz, vp]),
        "cca_prefill_backward": (C.c_int, [cfgp, wp, vp, vp, P(_Grads), vp, sz, vp]),
        "cca_decode_step_paged": (C.c_int, [cfgp, wp, vp, vp, C.c_int32, P(_PagedState),
                                            P(_PagedState), vp, vp, sz, vp]),
        "cca_prefill_forward_paged": (C.c_int, [cfgp, wp, vp, vp, P(_PagedState), vp, sz, vp]),
        "cca_decode_multi_workspace_size": (sz, [cfgp, C.c_int32, C.c_int32]),
        "cca_prefill_forward_fused": (C.c_int, [cfgp, wp, vp, vp, vp, sz, vp]),
        "cca_decode_multi": (C.c_int, [cfgp, wp, vp, C.c_int32, vp, C.c_int32, sp, sp, vp, vp, sz,
                                       vp]),
        "cca_decode_multi_paged": (C.c_int, [cfgp, wp, vp, C.c_int32, vp, C.c_int32,
                                             P(_PagedState), P(_PagedState), vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.cca_status_string(int(status)).decode()


def make_config(shape, chan_conv: str = "per_head", qk_mean: str = "pre_post",
                attn: str = "auto") -> Config:
    """Config from any object with the cca_config field names (dtype given as
    "bf16" / "f32" or as the enum value); ``chan_conv`` "per_head" or
    "grouped" selects the channel-conv reading, ``qk_mean`` "pre_post" or
    "pre" the q-k-mean reading, ``attn`` "auto", "four_wave" or "ping_pong"
    the prefill attention kernel."""
    dt = shape.dtype
    if isinstance(dt, str):
        dt = {"bf16": CCA_BF16, "f32": CCA_F32}[dt]
    mode = {"per_head": CCA_CHAN_PER_HEAD, "grouped": CCA_CHAN_GROUPED}[chan_conv]
    mean = {"pre_post": CCA_QK_MEAN_PRE_POST, "pre": CCA_QK_MEAN_PRE}[qk_mean]
    ak = {"auto": CCA_ATTN_AUTO, "four_wave": CCA_ATTN_FOUR_WAVE, "ping_pong": CCA_ATTN_PING_PONG}[attn]
    return Config(int(shape.batch), int(shape.seq_len), int(shape.d_model), int(shape.n_q_heads),
                  int(shape.n_kv_heads), int(shape.head_dim), int(shape.seq_conv_k),
                  int(shape.chan_conv_k), int(shape.use_qk_mean), int(shape.use_value_shift),
                  int(shape.use_qk_norm), float(shape.rope_base), float(shape.norm_eps), int(dt),
                  mode, mean, ak)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("libcca takes contiguous device tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    import torch
    return torch.cuda.current_stream().cuda_stream


@dataclass
class Weights:
    """Device tensors of one layer's weights (see cca_weights in include/cca.h)."""
    w_qkv: object
    w_o: object
    q_seq_taps: object
    k_seq_taps: object
    q_chan_taps: object
    k_chan_taps: object
    tau: object
    q_chan_dense: object = None      # grouped channel conv only: [H_q, d, k_c, d] fp32
    k_chan_dense: object = None      # [H_kv, d, k_c, d] fp32

    def struct(self) -> _Weights:
        return _Weights(_ptr(self.w_qkv), _ptr(self.w_o), _ptr(self.q_seq_taps),
                        _ptr(self.k_seq_taps), _ptr(self.q_chan_taps), _ptr(self.k_chan_taps),
                        _ptr(self.tau), _ptr(self.q_chan_dense), _ptr(self.k_chan_dense))


@dataclass
class State:
    """Device tensors of a decode state (see cca_state in include/cca.h)."""
    k_cache: object = None
    v_cache: object = None
    capacity: int = 0
    conv_q: object = None
    conv_k: object = None
    vshift: object = None

    def struct(self) -> _State:
        return _State(_ptr(self.k_cache), _ptr(self.v_cache), int(self.capacity), 0,
                      _ptr(self.conv_q), _ptr(self.conv_k), _ptr(self.vshift))


@dataclass
class PagedState:
    """Device tensors of a paged decode state (see cca_paged_state in include/cca.h)."""
    k_pages: object
    v_pages: object
    block_table: object
    page_size: int
    conv_q: object = None
    conv_k: object = None
    vshift: object = None

    def struct(self) -> _PagedState:
        return _PagedState(_ptr(self.k_pages), _ptr(self.v_pages), _ptr(self.block_table),
                           int(self.k_pages.shape[0]) if self.k_pages is not None else 0,
                           int(self.page_size),
                           int(self.block_table.shape[1]) if self.block_table is not None else 0, 0,
                           _ptr(self.conv_q), _ptr(self.conv_k), _ptr(self.vshift))


@dataclass
class Grads:
    """Device tensors receiving the gradients (see cca_grads in include/cca.h)."""
    x: object
    w_qkv: object
    w_o: object
    q_seq_taps: object
    k_seq_taps: object
    q_chan_taps: object
    k_chan_taps: object
    tau: object

    def struct(self) -> _Grads:
        return _Grads(_ptr(self.x), _ptr(self.w_qkv), _ptr(self.w_o), _ptr(self.q_seq_taps),
                      _ptr(self.k_seq_taps), _ptr(self.q_chan_taps), _ptr(self.k_chan_taps),
                      _ptr(self.tau))


def _check(status: int, where: str):
    if status != CCA_OK:
        raise CCAError(status, where)


def validate_config(cfg: Config) -> int:
    return lib.cca_validate_config(C.byref(cfg))


def prefill_workspace_size(cfg: Config) -> int:
    return lib.cca_prefill_workspace_size(C.byref(cfg))


def decode_workspace_size(cfg: Config, cache_len: int) -> int:
    return lib.cca_decode_workspace_size(C.byref(cfg), int(cache_len))


def prefill_workspace_layout(cfg: Config) -> list:
    off = (C.c_size_t * WS_COUNT)()
    _check(lib.cca_prefill_workspace_layout(C.byref(cfg), off), "cca_prefill_workspace_layout")
    return list(off)


def decode_workspace_layout(cfg: Config, cache_len: int) -> list:
    off = (C.c_size_t * WS_COUNT)()
    _check(lib.cca_decode_workspace_layout(C.byref(cfg), int(cache_len), off),
           "cca_decode_workspace_layout")
    return list(off)


def prefill_forward(cfg: Config, w: Weights, x, y, workspace, state_out: Optional[State] = None,
                    stream=None):
    so = C.byref(state_out.struct()) if state_out is not None else None
    _check(lib.cca_prefill_forward(C.byref(cfg), C.byref(w.struct()), _ptr(x), _ptr(y), so,
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "cca_prefill_forward")


def decode_step(cfg: Config, w: Weights, x_t, cache_len: int, state_in: State, state_out: State,
                y_t, workspace, stream=None):
    _check(lib.cca_decode_step(C.byref(cfg), C.byref(w.struct()), _ptr(x_t), int(cache_len),
                               C.byref(state_in.struct()), C.byref(state_out.struct()), _ptr(y_t),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "cca_decode_step")


def decode_step_noalloc(cfg: Config, w: Weights, x_t, cache_len: int, state_in: State,
                        state_out: State, y_t, stream=None):
    """cca_decode_step with the library's own per-GPU scratch array as the
    workspace (no allocation; calls that overlap on one GPU race)."""
    _check(lib.cca_decode_step_noalloc(C.byref(cfg), C.byref(w.struct()), _ptr(x_t), int(cache_len),
                                       C.byref(state_in.struct()), C.byref(state_out.struct()),
                                       _ptr(y_t), _stream(stream)), "cca_decode_step_noalloc")


def decode_step_varlen(cfg: Config, w: Weights, x_t, cache_lens, max_cache_len: int,
                       state_in: State, state_out: State, y_t, workspace, stream=None):
    """cache_lens: device int32 tensor [B] of per-sequence cache lengths."""
    _check(lib.cca_decode_step_varlen(C.byref(cfg), C.byref(w.struct()), _ptr(x_t), _ptr(cache_lens),
                                      int(max_cache_len), C.byref(state_in.struct()),
                                      C.byref(state_out.struct()), _ptr(y_t), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)),
           "cca_decode_step_varlen")


def _wsb(ws):
    return ws.numel() * ws.element_size()


def stage_downproj(cfg, w, x, workspace, stream=None):
    _check(lib.cca_stage_downproj(C.byref(cfg), C.byref(w.struct()), _ptr(x), _ptr(workspace),
                                  _wsb(workspace), _stream(stream)), "cca_stage_downproj")


def stage_convmix(cfg, w, workspace, state_out: Optional[State] = None, stream=None):
    so = C.byref(state_out.struct()) if state_out is not None else None
    _check(lib.cca_stage_convmix(C.byref(cfg), C.byref(w.struct()), so, _ptr(workspace),
                                 _wsb(workspace), _stream(stream)), "cca_stage_convmix")


def stage_attention(cfg, w, workspace, stream=None):
    _check(lib.cca_stage_attention(C.byref(cfg), C.byref(w.struct()), _ptr(workspace),
                                   _wsb(workspace), _stream(stream)), "cca_stage_attention")


def stage_upproj(cfg, w, y, workspace, stream=None):
    _check(lib.cca_stage_upproj(C.byref(cfg), C.byref(w.struct()), _ptr(y), _ptr(workspace),
                                _wsb(workspace), _stream(stream)), "cca_stage_upproj")


def stage_decode_downproj(cfg, w, x_t, cache_len, workspace, stream=None):
    _check(lib.cca_stage_decode_downproj(C.byref(cfg), C.byref(w.struct()), _ptr(x_t),
                                         int(cache_len), _ptr(workspace), _wsb(workspace),
                                         _stream(stream)), "cca_stage_decode_downproj")


def stage_decode_mix(cfg, w, cache_len, state_in: State, state_out: State, workspace, stream=None):
    _check(lib.cca_stage_decode_mix(C.byref(cfg), C.byref(w.struct()), int(cache_len),
                                    C.byref(state_in.struct()), C.byref(state_out.struct()),
                                    _ptr(workspace), _wsb(workspace), _stream(stream)),
           "cca_stage_decode_mix")


def stage_decode_attention(cfg, w, cache_len, state_in: State, workspace, stream=None):
    _check(lib.cca_stage_decode_attention(C.byref(cfg), C.byref(w.struct()), int(cache_len),
                                          C.byref(state_in.struct()), _ptr(workspace),
                                          _wsb(workspace), _stream(stream)),
           "cca_stage_decode_attention")


def stage_decode_upproj(cfg, w, cache_len, y_t, workspace, stream=None):
    _check(lib.cca_stage_decode_upproj(C.byref(cfg), C.byref(w.struct()), int(cache_len), _ptr(y_t),
                                       _ptr(workspace), _wsb(workspace), _stream(stream)),
           "cca_stage_decode_upproj")


def train_workspace_size(cfg: Config) -> int:
    return lib.cca_train_workspace_size(C.byref(cfg))


def prefill_forward_train(cfg: Config, w: Weights, x, y, workspace, stream=None):
    _check(lib.cca_prefill_forward_train(C.byref(cfg), C.byref(w.struct()), _ptr(x), _ptr(y),
                                         _ptr(workspace), _wsb(workspace), _stream(stream)),
           "cca_prefill_forward_train")


def prefill_backward(cfg: Config, w: Weights, x, dy, grads: Grads, workspace, stream=None):
    _check(lib.cca_prefill_backward(C.byref(cfg), C.byref(w.struct()), _ptr(x), _ptr(dy),
                                    C.byref(grads.struct()), _ptr(workspace), _wsb(workspace),
                                    _stream(stream)), "cca_prefill_backward")


def decode_step_paged(cfg: Config, w: Weights, x_t, cache_lens, max_cache_len: int,
                      state_in: PagedState, state_out: PagedState, y_t, workspace, stream=None):
    """cache_lens: device int32 [B]; the pages and block table live in the states."""
    _check(lib.cca_decode_step_paged(C.byref(cfg), C.byref(w.struct()), _ptr(x_t), _ptr(cache_lens),
                                     int(max_cache_len), C.byref(state_in.struct()),
                                     C.byref(state_out.struct()), _ptr(y_t), _ptr(workspace),
                                     _wsb(workspace), _stream(stream)), "cca_decode_step_paged")


def prefill_forward_paged(cfg: Config, w: Weights, x, y, workspace, state_out: PagedState,
                          stream=None):
    _check(lib.cca_prefill_forward_paged(C.byref(cfg), C.byref(w.struct()), _ptr(x), _ptr(y),
                                         C.byref(state_out.struct()), _ptr(workspace),
                                         _wsb(workspace), _stream(stream)),
           "cca_prefill_forward_paged")


def decode_multi_workspace_size(cfg: Config, n_new: int, max_cache_len: int) -> int:
    return lib.cca_decode_multi_workspace_size(C.byref(cfg), int(n_new), int(max_cache_len))


def decode_multi(cfg: Config, w: Weights, x_new, n_new: int, cache_lens, max_cache_len: int,
                 state_in: State, state_out: State, y_new, workspace, stream=None):
    """x_new, y_new: [B, n_new, E]; cache_lens: device int32 [B]."""
    _check(lib.cca_decode_multi(C.byref(cfg), C.byref(w.struct()), _ptr(x_new), int(n_new),
                                _ptr(cache_lens), int(max_cache_len), C.byref(state_in.struct()),
                                C.byref(state_out.struct()), _ptr(y_new), _ptr(workspace),
                                _wsb(workspace), _stream(stream)), "cca_decode_multi")


def decode_multi_paged(cfg: Config, w: Weights, x_new, n_new: int, cache_lens, max_cache_len: int,
                       state_in: PagedState, state_out: PagedState, y_new, workspace, stream=None):
    _check(lib.cca_decode_multi_paged(C.byref(cfg), C.byref(w.struct()), _ptr(x_new), int(n_new),
                                      _ptr(cache_lens), int(max_cache_len),
                                      C.byref(state_in.struct()), C.byref(state_out.struct()),
                                      _ptr(y_new), _ptr(workspace), _wsb(workspace),
                                      _stream(stream)), "cca_decode_multi_paged")


def prefill_forward_fused(cfg: Config, w: Weights, x, y, workspace, stream=None):
    _check(lib.cca_prefill_forward_fused(C.byref(cfg), C.byref(w.struct()), _ptr(x), _ptr(y),
                                         _ptr(workspace), _wsb(workspace), _stream(stream)),
           "cca_prefill_forward_fused")
