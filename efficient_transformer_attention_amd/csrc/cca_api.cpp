// Host side of libcca: argument validation, workspace layout and the launch
// sequence of the prefill and decode passes.  Every check runs before the
// first launch; launches are asynchronous on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "cca.h"
#include "cca_device.h"
#include "cca_launch.h"

using namespace cca;

#define CCA_TRY(expr)                 \
  do {                                \
    cca_status _r = (expr);           \
    if (_r != CCA_OK) return _r;      \
  } while (0)

namespace {

constexpr size_t WS_ALIGN = 256;
constexpr int TILE_T = 128;   // token padding of the attention operands

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool debug_sync() {
  static int v = -1;
  if (v < 0) {
    const char *e = getenv("CCA_DEBUG_SYNC");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

cca_status check_launch(hipError_t e, hipStream_t stream) {
  if (e != hipSuccess) return CCA_ERR_HIP;
  if (debug_sync()) {
    if (hipStreamSynchronize(stream) != hipSuccess) return CCA_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return CCA_ERR_HIP;
  }
  return CCA_OK;
}

size_t elem_size(int dtype) { return dtype == CCA_F32 ? 4 : 2; }

// The down-projection output qkv~: fp16 in bf16 mode (10 mantissa bits, half
// the bytes of fp32 for the mixing kernel to read), fp32 in fp32 mode.
size_t qkv_elem_size(int dtype) { return dtype == CCA_F32 ? 4 : 2; }

// Storage type of the normalised, rotated q and k handed to the attention
// kernel: fp16 when they are unit vectors (10 mantissa bits instead of
// bf16's 7, no range concern), else the storage dtype.
size_t qk_elem_size(const cca_config &c) {
  if (c.dtype == CCA_F32) return 4;
  return 2;
}
bool qk_is_f16(const cca_config &c) { return c.dtype == CCA_BF16 && c.use_qk_norm; }

int padded_T(int T) { return (T + TILE_T - 1) / TILE_T * TILE_T; }

// The prefill attention kernel for c: 1 four-wave, 2 ping-pong, 0 chosen at
// launch from the grid size.  The ping-pong kernel takes bf16 with d = 64.
int attn_kernel_for(const cca_config &c) {
  const bool pp_ok = c.dtype == CCA_BF16 && c.head_dim == 64;
  if (!pp_ok || c.attn_kernel == CCA_ATTN_FOUR_WAVE) return 1;
  if (c.attn_kernel == CCA_ATTN_PING_PONG) return 2;
  return 0;
}

MixShape mix_shape(const cca_config &c) {
  MixShape s;
  s.B = c.batch;
  s.T = c.seq_len;
  s.Tp = padded_T(c.seq_len);
  s.Hq = c.n_q_heads;
  s.Hkv = c.n_kv_heads;
  s.G = c.n_q_heads / c.n_kv_heads;
  s.d = c.head_dim;
  s.ks = c.seq_conv_k;
  s.kc = c.chan_conv_k;
  // q-k-mean: 0 off, 1 the pre-convolution values, 2 the pre- and post-convolution values
  s.use_mean = c.use_qk_mean ? (c.qk_mean_mode == CCA_QK_MEAN_PRE ? 1 : 2) : 0;
  s.use_shift = c.use_value_shift;
  s.use_norm = c.use_qk_norm;
  s.grouped = c.chan_conv_mode == CCA_CHAN_GROUPED ? 1 : 0;
  s.rope_base = c.rope_base;
  s.eps = c.norm_eps;
  s.attn_kernel = attn_kernel_for(c);
  for (int i = 0; i < 64; ++i)
    s.theta[i] = (c.rope_base > 0.f && 2 * i < c.head_dim)
                     ? std::pow((double)c.rope_base, -2.0 * (double)i / (double)c.head_dim)
                     : 0.0;
  return s;
}

cca_status validate_shape(const cca_config *c, bool need_seq) {
  if (!c) return CCA_ERR_INVALID_ARG;
  if (c->batch < 1 || c->d_model < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1)
    return CCA_ERR_INVALID_ARG;
  if (need_seq && c->seq_len < 1) return CCA_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads) return CCA_ERR_INVALID_ARG;
  if (c->d_model % 8) return CCA_ERR_INVALID_ARG;
  if (c->use_value_shift && (c->n_kv_heads % 2)) return CCA_ERR_INVALID_ARG;
  if (!(c->norm_eps > 0.f) || !(c->rope_base >= 0.f)) return CCA_ERR_INVALID_ARG;
  if ((unsigned)c->use_qk_mean > 1u || (unsigned)c->use_value_shift > 1u ||
      (unsigned)c->use_qk_norm > 1u)
    return CCA_ERR_INVALID_ARG;
  if (c->dtype != CCA_BF16 && c->dtype != CCA_F32) return CCA_ERR_UNSUPPORTED;
  if (c->chan_conv_mode != CCA_CHAN_PER_HEAD && c->chan_conv_mode != CCA_CHAN_GROUPED)
    return CCA_ERR_INVALID_ARG;
  if (c->qk_mean_mode != CCA_QK_MEAN_PRE_POST && c->qk_mean_mode != CCA_QK_MEAN_PRE)
    return CCA_ERR_INVALID_ARG;
  if (c->attn_kernel != CCA_ATTN_AUTO && c->attn_kernel != CCA_ATTN_FOUR_WAVE &&
      c->attn_kernel != CCA_ATTN_PING_PONG)
    return CCA_ERR_INVALID_ARG;
  const int d = c->head_dim;
  if (d != 16 && d != 32 && d != 64 && d != 128) return CCA_ERR_UNSUPPORTED;
  if (c->seq_conv_k < 1 || c->seq_conv_k > 4 || c->chan_conv_k < 1 || c->chan_conv_k > 4)
    return CCA_ERR_UNSUPPORTED;
  if (!convmix_fits(c->n_q_heads / c->n_kv_heads, d)) return CCA_ERR_UNSUPPORTED;
  if (c->chan_conv_mode == CCA_CHAN_GROUPED &&
      (!grouped_conv_supported(d, c->dtype == CCA_F32) ||
       !convmix_decode_grouped_fits(c->n_q_heads / c->n_kv_heads, d, 1, c->seq_conv_k, c->chan_conv_k)))
    return CCA_ERR_UNSUPPORTED;
  if (need_seq && !attention_supported(d, c->dtype == CCA_F32)) return CCA_ERR_UNSUPPORTED;
  // index arithmetic stays in 32-bit for per-row offsets
  const long long N = (long long)(c->n_q_heads + 2 * c->n_kv_heads) * d;
  if ((long long)c->batch * (need_seq ? padded_T(c->seq_len) : 1) * (N > c->d_model ? N : c->d_model) >
      (1ll << 40))
    return CCA_ERR_UNSUPPORTED;
  if ((long long)c->batch * (need_seq ? c->seq_len : 1) > (1ll << 31) - 1) return CCA_ERR_UNSUPPORTED;
  // one sequence's down-projection rows are addressed by 32-bit buffer offsets
  if (need_seq && (long long)padded_T(c->seq_len) * N * 4 >= (1ll << 31)) return CCA_ERR_UNSUPPORTED;
  return CCA_OK;
}

// Shapes cca_prefill_forward_fused takes: bf16 kv groups of one query head
// with d = 64 and T a multiple of 128.
bool fused_downproj_mix(const cca_config &c) {
  if (c.dtype != CCA_BF16 || c.chan_conv_mode != CCA_CHAN_PER_HEAD) return false;
  const int G = c.n_q_heads / c.n_kv_heads;
  if (!downproj_mix_supported(G, c.head_dim, c.seq_len, c.d_model)) return false;
  const size_t N = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t lim = (1ull << 32) - 2 * (size_t)c.d_model;
  return (size_t)c.batch * c.seq_len * c.d_model * 2 < lim && N * c.d_model * 2 < lim;
}

struct Layout {
  size_t off[CCA_WS_COUNT];
  size_t total;
};

Layout prefill_layout(const cca_config &c) {
  Layout L;
  for (int i = 0; i < CCA_WS_COUNT; ++i) L.off[i] = SIZE_MAX;
  const size_t B = c.batch, T = c.seq_len, Tp = padded_T(c.seq_len), d = c.head_dim;
  const size_t eq = (size_t)c.n_q_heads * d, ekv = (size_t)c.n_kv_heads * d;
  const size_t N = eq + 2 * ekv;
  size_t o = 0;
  L.off[CCA_WS_QKV] = o; o = align_up(o + B * T * N * qkv_elem_size(c.dtype), WS_ALIGN);
  L.off[CCA_WS_Q] = o;   o = align_up(o + B * c.n_q_heads * Tp * d * qk_elem_size(c), WS_ALIGN);
  L.off[CCA_WS_K] = o;   o = align_up(o + B * c.n_kv_heads * Tp * d * qk_elem_size(c), WS_ALIGN);
  L.off[CCA_WS_VT] = o;  o = align_up(o + B * c.n_kv_heads * d * Tp * elem_size(c.dtype), WS_ALIGN);
  L.off[CCA_WS_O] = o;   o = align_up(o + B * T * eq * elem_size(c.dtype), WS_ALIGN);
  if (fused_downproj_mix(c)) {   // halo rows of the fused down-projection + mixing
    L.off[CCA_WS_PART] = o;
    o = align_up(o + downproj_mix_halo_bytes(c.batch, c.seq_len, c.d_model, (int)N), WS_ALIGN);
  } else if (c.chan_conv_mode == CCA_CHAN_GROUPED) {   // the grouped channel conv's output
    L.off[CCA_WS_PART] = o;
    o = align_up(o + B * T * (eq + ekv) * 4, WS_ALIGN);
  }
  L.total = o;
  return L;
}

// m new tokens per sequence (1 for the single-token step): the projections
// see B*m rows.
Layout decode_layout(const cca_config &c, int cache_len, int m = 1) {
  Layout L;
  for (int i = 0; i < CCA_WS_COUNT; ++i) L.off[i] = SIZE_MAX;
  const size_t B = (size_t)c.batch * m, d = c.head_dim;
  const size_t eq = (size_t)c.n_q_heads * d, ekv = (size_t)c.n_kv_heads * d;
  const size_t N = eq + 2 * ekv;
  size_t o = 0;
  L.off[CCA_WS_QKV] = o;  o = align_up(o + B * N * 4, WS_ALIGN);
  L.off[CCA_WS_Q] = o;    o = align_up(o + B * c.n_q_heads * d * 4, WS_ALIGN);
  L.off[CCA_WS_PART] = o;
  o = align_up(o + decode_partial_floats(c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim,
                                         cache_len + m, m) * 4, WS_ALIGN);
  L.off[CCA_WS_O] = o;    o = align_up(o + B * eq * elem_size(c.dtype), WS_ALIGN);
  if (B <= 64) {   // split-contraction partial sums of the two skinny projections
    const int es = (int)elem_size(c.dtype);
    const size_t down = (size_t)gemm_splitk_slices((int)B, (int)N, c.d_model, es) * B * N;
    const size_t up = (size_t)gemm_splitk_slices((int)B, c.d_model, (int)eq, es) * B * c.d_model;
    L.off[CCA_WS_SPLITK] = o;
    o = align_up(o + (down > up ? down : up) * 4, WS_ALIGN);
  }
  L.total = o;
  return L;
}

// Training workspace: the prefill layout (same offsets), then what the
// backward pass keeps or builds.  Slots of the backward, in order.
enum {
  TR_LSE, TR_BPOST, TR_DO, TR_DSUM, TR_QT, TR_KT, TR_DOT, TR_VR, TR_GQ, TR_DK, TR_DV, TR_DM, TR_DA,
  TR_DZ, TR_MIXS, TR_WOT, TR_WQKVT, TR_DYT, TR_OT, TR_DZT, TR_XT, TR_SPLITK, TR_COUNT
};

// Whether the training forward keeps the channel-conv output b (fp32) for the
// backward: the q-k-mean of the pre- and post-convolution values mixes b of
// the group's heads.
bool keeps_bpost(const cca_config &c) {
  return c.use_qk_mean && c.qk_mean_mode == CCA_QK_MEAN_PRE_POST;
}

struct TrainLayout {
  Layout pre;
  size_t off[TR_COUNT];
  size_t total;
  int BTp;   // B*T rounded up to 64: contraction length of the weight gradients
};

// fp32 partials of the two weight-gradient products (contraction over B*T)
size_t splitk_floats(const cca_config &c, int BTp) {
  const int E = c.d_model, eq = c.n_q_heads * c.head_dim;
  const int N = eq + 2 * c.n_kv_heads * c.head_dim;
  // the token-major products contract over B*T rows, the transposed ones over BTp
  const int BT = c.batch * c.seq_len;
  auto sl = [](int m, int n, int k1, int k2) {
    const int a = gemm_long_k_slices(m, n, k1), b = gemm_long_k_slices(m, n, k2);
    return (size_t)(a > b ? a : b);
  };
  const size_t a = sl(E, eq, BTp, BT) * E * eq;
  const size_t b = sl(N, E, BTp, BT) * N * E;
  return a > b ? a : b;
}

TrainLayout train_layout(const cca_config &c) {
  TrainLayout L;
  L.pre = prefill_layout(c);
  const size_t B = c.batch, T = c.seq_len, Tp = padded_T(c.seq_len), d = c.head_dim;
  const size_t Hq = c.n_q_heads, Hkv = c.n_kv_heads, E = c.d_model;
  const size_t eq = Hq * d, ekv = Hkv * d, N = eq + 2 * ekv, BT = B * T;
  const size_t es = elem_size(c.dtype);
  L.BTp = (int)((BT + 63) / 64 * 64);
  const size_t BTp = (size_t)L.BTp;
  const size_t sz[TR_COUNT] = {
      B * Hq * Tp * 4,            // TR_LSE
      keeps_bpost(c) ? BT * (eq + ekv) * 4 : 0,   // TR_BPOST
      BT * eq * es,               // TR_DO
      B * Hq * Tp * 4,            // TR_DSUM
      B * Hq * d * Tp * es,       // TR_QT
      B * Hkv * d * Tp * es,      // TR_KT
      B * Hq * d * Tp * es,       // TR_DOT
      B * Hkv * Tp * d * es,      // TR_VR
      BT * eq * 4,                // TR_GQ
      BT * ekv * 4,               // TR_DK
      BT * ekv * 4,               // TR_DV
      BT * (eq + ekv) * 4,        // TR_DM
      BT * (eq + ekv) * 4,        // TR_DA
      BT * N * es,                // TR_DZ
      mix_backward_scratch_floats(mix_shape(c)) * 4,   // TR_MIXS
      eq * E * es,                // TR_WOT
      E * N * es,                 // TR_WQKVT
      E * BTp * es,               // TR_DYT
      eq * BTp * es,              // TR_OT
      N * BTp * es,               // TR_DZT
      E * BTp * es,               // TR_XT
      splitk_floats(c, (int)BTp) * 4,   // TR_SPLITK
  };
  size_t o = L.pre.total;
  for (int i = 0; i < TR_COUNT; ++i) {
    L.off[i] = o;
    o = align_up(o + sz[i], WS_ALIGN);
  }
  L.total = o;
  return L;
}

// fp32 scratch of the split-contraction GEMM path (decode only).
float *splitk_ptr(void *ws, const Layout &L, size_t *floats) {
  if (L.off[CCA_WS_SPLITK] == SIZE_MAX) { *floats = 0; return nullptr; }
  *floats = (L.total - L.off[CCA_WS_SPLITK]) / 4;
  return reinterpret_cast<float *>(static_cast<unsigned char *>(ws) + L.off[CCA_WS_SPLITK]);
}

cca_status check_weights(const cca_config &c, const cca_weights *w) {
  if (!w || !w->w_qkv || !w->w_o || !w->q_seq_taps || !w->k_seq_taps || !w->q_chan_taps ||
      !w->k_chan_taps || !w->tau)
    return CCA_ERR_INVALID_ARG;
  if (!aligned16(w->w_qkv) || !aligned16(w->w_o)) return CCA_ERR_INVALID_ARG;
  if (c.chan_conv_mode == CCA_CHAN_GROUPED &&
      (!w->q_chan_dense || !w->k_chan_dense || !aligned16(w->q_chan_dense) ||
       !aligned16(w->k_chan_dense)))
    return CCA_ERR_INVALID_ARG;
  return CCA_OK;
}

cca_status check_ws(void *ws, size_t bytes, size_t need) {
  if (bytes < need) return CCA_ERR_WORKSPACE;
  if (need && !ws) return CCA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & (WS_ALIGN - 1)) return CCA_ERR_WORKSPACE;
  return CCA_OK;
}

MixTaps taps_of(const cca_weights *w) {
  MixTaps t;
  t.q_seq = w->q_seq_taps;
  t.k_seq = w->k_seq_taps;
  t.q_chan = w->q_chan_taps;
  t.k_chan = w->k_chan_taps;
  t.tau = w->tau;
  return t;
}

StateOut state_of(const cca_state *st) {
  StateOut s;
  std::memset(&s, 0, sizeof(s));
  if (st) {
    s.k_cache = st->k_cache;
    s.v_cache = st->v_cache;
    s.capacity = st->capacity;
    s.conv_q = st->conv_q;
    s.conv_k = st->conv_k;
    s.vshift = st->vshift;
  }
  return s;
}

StateOut state_of(const cca_paged_state *st) {
  StateOut s;
  std::memset(&s, 0, sizeof(s));
  if (st) {
    s.k_cache = st->k_pages;
    s.v_cache = st->v_pages;
    s.conv_q = st->conv_q;
    s.conv_k = st->conv_k;
    s.vshift = st->vshift;
    s.table = st->block_table;
    s.page = st->page_size;
    s.mpps = st->max_pages_per_seq;
    s.npages = st->num_pages;
  }
  return s;
}

unsigned char *wsp(void *ws, const Layout &L, int slot) {
  return static_cast<unsigned char *>(ws) + L.off[slot];
}

// ---- prefill stages --------------------------------------------------------

cca_status run_downproj(const cca_config &c, const cca_weights *w, const void *x, void *ws,
                        const Layout &L, hipStream_t st) {
  const int M = c.batch * c.seq_len, E = c.d_model;
  const int N = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  void *qkv = wsp(ws, L, CCA_WS_QKV);
  hipError_t e;
  if (c.dtype == CCA_BF16)
    e = launch_gemm_nt<bf16, f16>((const bf16 *)x, (const bf16 *)w->w_qkv, (f16 *)qkv, M, N, E, E,
                                  E, N, st);
  else
    e = launch_gemm_nt<float, float>((const float *)x, (const float *)w->w_qkv, (float *)qkv, M, N,
                                     E, E, E, N, st);
  return check_launch(e, st);
}

// bout (nullable): receives the channel-conv output of every q and k head
// (the training forward under the pre- and post-convolution mean).
cca_status run_convmix(const cca_config &c, const cca_weights *w, const StateOut &so, void *ws,
                       const Layout &L, hipStream_t st, float *bout = nullptr) {
  const MixShape s = mix_shape(c);
  const void *qkv = wsp(ws, L, CCA_WS_QKV);
  float *r1b = nullptr;
  hipError_t e;
  if (c.chan_conv_mode == CCA_CHAN_GROUPED) {   // the channel conv on MFMA first
    r1b = reinterpret_cast<float *>(wsp(ws, L, CCA_WS_PART));
    e = launch_grouped_conv_prefill(s, taps_of(w), w->q_chan_dense, w->k_chan_dense, qkv, r1b,
                                    c.dtype == CCA_F32, st);
    CCA_TRY(check_launch(e, st));
  }
  if (c.dtype == CCA_F32) {
    e = launch_convmix_prefill<float, float, float>(
        s, taps_of(w), (const float *)qkv, (float *)wsp(ws, L, CCA_WS_Q),
        (float *)wsp(ws, L, CCA_WS_K), (float *)wsp(ws, L, CCA_WS_VT), so, st, r1b, bout);
  } else if (qk_is_f16(c)) {
    e = launch_convmix_prefill<f16, f16, bf16>(
        s, taps_of(w), (const f16 *)qkv, (f16 *)wsp(ws, L, CCA_WS_Q), (f16 *)wsp(ws, L, CCA_WS_K),
        (bf16 *)wsp(ws, L, CCA_WS_VT), so, st, r1b, bout);
  } else {
    e = launch_convmix_prefill<f16, bf16, bf16>(
        s, taps_of(w), (const f16 *)qkv, (bf16 *)wsp(ws, L, CCA_WS_Q),
        (bf16 *)wsp(ws, L, CCA_WS_K), (bf16 *)wsp(ws, L, CCA_WS_VT), so, st, r1b, bout);
  }
  return check_launch(e, st);
}

cca_status run_downproj_mix(const cca_config &c, const cca_weights *w, const void *x, void *ws,
                            const Layout &L, hipStream_t st) {
  const MixShape s = mix_shape(c);
  hipError_t e;
  if (qk_is_f16(c))
    e = launch_downproj_mix<f16, bf16>(s, taps_of(w), (const bf16 *)x, (const bf16 *)w->w_qkv,
                                       c.d_model, wsp(ws, L, CCA_WS_PART),
                                       (f16 *)wsp(ws, L, CCA_WS_Q), (f16 *)wsp(ws, L, CCA_WS_K),
                                       (bf16 *)wsp(ws, L, CCA_WS_VT), st);
  else
    e = launch_downproj_mix<bf16, bf16>(s, taps_of(w), (const bf16 *)x, (const bf16 *)w->w_qkv,
                                        c.d_model, wsp(ws, L, CCA_WS_PART),
                                        (bf16 *)wsp(ws, L, CCA_WS_Q), (bf16 *)wsp(ws, L, CCA_WS_K),
                                        (bf16 *)wsp(ws, L, CCA_WS_VT), st);
  return check_launch(e, st);
}

cca_status run_attention(const cca_config &c, const cca_weights *w, void *ws, const Layout &L,
                         hipStream_t st, float *lse = nullptr) {
  const MixShape s = mix_shape(c);
  hipError_t e;
  if (c.dtype == CCA_F32) {
    e = launch_attention_prefill<float, float>(s, (const float *)wsp(ws, L, CCA_WS_Q),
                                               (const float *)wsp(ws, L, CCA_WS_K),
                                               (const float *)wsp(ws, L, CCA_WS_VT), w->tau,
                                               (float *)wsp(ws, L, CCA_WS_O), lse, st);
  } else if (qk_is_f16(c)) {
    e = launch_attention_prefill<f16, bf16>(s, (const f16 *)wsp(ws, L, CCA_WS_Q),
                                            (const f16 *)wsp(ws, L, CCA_WS_K),
                                            (const bf16 *)wsp(ws, L, CCA_WS_VT), w->tau,
                                            (bf16 *)wsp(ws, L, CCA_WS_O), lse, st);
  } else {
    e = launch_attention_prefill<bf16, bf16>(s, (const bf16 *)wsp(ws, L, CCA_WS_Q),
                                             (const bf16 *)wsp(ws, L, CCA_WS_K),
                                             (const bf16 *)wsp(ws, L, CCA_WS_VT), w->tau,
                                             (bf16 *)wsp(ws, L, CCA_WS_O), lse, st);
  }
  return check_launch(e, st);
}

cca_status run_upproj(const cca_config &c, const cca_weights *w, void *y, void *ws,
                      const Layout &L, int M, hipStream_t st) {
  const int E = c.d_model, eq = c.n_q_heads * c.head_dim;
  size_t skf;
  float *sk = splitk_ptr(ws, L, &skf);
  hipError_t e;
  if (c.dtype == CCA_BF16)
    e = launch_gemm_nt<bf16, bf16>((const bf16 *)wsp(ws, L, CCA_WS_O), (const bf16 *)w->w_o,
                                   (bf16 *)y, M, E, eq, eq, eq, E, st, sk, skf);
  else
    e = launch_gemm_nt<float, float>((const float *)wsp(ws, L, CCA_WS_O), (const float *)w->w_o,
                                     (float *)y, M, E, eq, eq, eq, E, st, sk, skf);
  return check_launch(e, st);
}

cca_status check_state_out(const cca_config &c, const cca_state *so) {
  if (!so) return CCA_OK;
  if ((so->k_cache || so->v_cache) && so->capacity < c.seq_len) return CCA_ERR_INVALID_ARG;
  if ((so->k_cache && !aligned16(so->k_cache)) || (so->v_cache && !aligned16(so->v_cache)))
    return CCA_ERR_INVALID_ARG;
  return CCA_OK;
}

// ---- decode stages ---------------------------------------------------------

cca_status check_decode_state(const cca_config &c, int32_t L, const cca_state *si,
                              const cca_state *so) {
  if (L < 0 || !si || !so) return CCA_ERR_INVALID_ARG;
  if (!si->k_cache || !si->v_cache || si->capacity <= L) return CCA_ERR_INVALID_ARG;
  if (!aligned16(si->k_cache) || !aligned16(si->v_cache)) return CCA_ERR_INVALID_ARG;
  if ((so->k_cache && so->k_cache != si->k_cache) || (so->v_cache && so->v_cache != si->v_cache))
    return CCA_ERR_INVALID_ARG;
  if (c.seq_conv_k > 1 && (!si->conv_q || !si->conv_k || !so->conv_q || !so->conv_k))
    return CCA_ERR_INVALID_ARG;
  if (c.use_value_shift && (!si->vshift || !so->vshift)) return CCA_ERR_INVALID_ARG;
  if ((long long)c.batch * c.n_kv_heads * si->capacity * c.head_dim > (1ll << 40))
    return CCA_ERR_UNSUPPORTED;
  return CCA_OK;
}

// ---- backward pass ---------------------------------------------------------

template <typename T> T *trp(void *ws, const TrainLayout &L, int slot) {
  return reinterpret_cast<T *>(static_cast<unsigned char *>(ws) + L.off[slot]);
}

// g[M, N] = a^T b for token-major a [BT, M], b [BT, N] (a weight gradient):
// read in place (bf16, tile-aligned M and N), else transposed to [M, BTp] and
// [N, BTp] copies (rows past BT zero) for the K-contiguous product.
template <typename TV>
hipError_t weight_grad(const TV *a, const TV *b, float *g, int M, int N, int BT, int BTp, TV *aT,
                       TV *bT, float *splitk, size_t skf, hipStream_t st) {
  if constexpr (std::is_same<TV, bf16>::value) {
    const hipError_t e = launch_gemm_tn_long_k(a, b, g, M, N, BT, M, N, splitk, skf, st);
    if (e != hipErrorNotSupported) return e;
  }
  hipError_t e = launch_transpose_2d<TV, TV>(a, aT, BTp, BT, M, M, BTp, st);
  if (e != hipSuccess) return e;
  e = launch_transpose_2d<TV, TV>(b, bT, BTp, BT, N, N, BTp, st);
  if (e != hipSuccess) return e;
  return launch_gemm_nt_long_k<TV>(aT, bT, g, M, N, BTp, BTp, BTp, splitk, skf, st);
}

template <typename TQ, typename TV>
cca_status run_backward(const cca_config &c, const cca_weights *w, const void *x, const void *dy,
                        const cca_grads *gr, void *ws, const TrainLayout &L, hipStream_t st) {
  const MixShape s = mix_shape(c);
  const int BT = c.batch * c.seq_len, E = c.d_model, d = c.head_dim;
  const int eq = c.n_q_heads * d, ekv = c.n_kv_heads * d, N = eq + 2 * ekv;
  const int BTp = L.BTp;
  const Layout &P = L.pre;
  TV *dO = trp<TV>(ws, L, TR_DO);
  TV *dz = trp<TV>(ws, L, TR_DZ);
  const TV *O = reinterpret_cast<const TV *>(wsp(ws, P, CCA_WS_O));
  // up-projection: dO = dy W_o, dW_o = dy^T O (contraction over tokens)
  CCA_TRY(check_launch(launch_transpose_2d<TV, TV>((const TV *)w->w_o, trp<TV>(ws, L, TR_WOT), E, E,
                                                   eq, eq, E, st), st));
  CCA_TRY(check_launch(launch_gemm_nt<TV, TV>((const TV *)dy, trp<TV>(ws, L, TR_WOT), dO, BT, eq, E,
                                              E, E, eq, st), st));
  const size_t skf = splitk_floats(c, BTp);
  CCA_TRY(check_launch(weight_grad<TV>((const TV *)dy, O, gr->w_o, E, eq, BT, BTp,
                                       trp<TV>(ws, L, TR_DYT), trp<TV>(ws, L, TR_OT),
                                       trp<float>(ws, L, TR_SPLITK), skf, st), st));
  // attention
  AttnBwdArgs<TQ, TV> aa;
  aa.q = reinterpret_cast<const TQ *>(wsp(ws, P, CCA_WS_Q));
  aa.k = reinterpret_cast<const TQ *>(wsp(ws, P, CCA_WS_K));
  aa.vt = reinterpret_cast<const TV *>(wsp(ws, P, CCA_WS_VT));
  aa.O = O;
  aa.dO = dO;
  aa.lse = trp<float>(ws, L, TR_LSE);
  aa.qT = trp<TV>(ws, L, TR_QT);
  aa.kT = trp<TV>(ws, L, TR_KT);
  aa.dOT = trp<TV>(ws, L, TR_DOT);
  aa.vr = trp<TV>(ws, L, TR_VR);
  aa.dsum = trp<float>(ws, L, TR_DSUM);
  aa.dk = trp<float>(ws, L, TR_DK);
  aa.dv = trp<float>(ws, L, TR_DV);
  aa.gq = trp<float>(ws, L, TR_GQ);
  CCA_TRY(check_launch(launch_attention_backward<TQ, TV>(s, aa, st), st));
  // mixing steps
  typedef typename std::conditional<std::is_same<TV, float>::value, float, f16>::type TI;
  MixBwdArgs<TI, TV> ma;
  ma.qkv = reinterpret_cast<const TI *>(wsp(ws, P, CCA_WS_QKV));
  ma.bpost = keeps_bpost(c) ? trp<float>(ws, L, TR_BPOST) : nullptr;
  ma.gq = aa.gq;
  ma.dk = aa.dk;
  ma.dv = aa.dv;
  ma.dm = trp<float>(ws, L, TR_DM);
  ma.da = trp<float>(ws, L, TR_DA);
  ma.scratch = trp<float>(ws, L, TR_MIXS);
  ma.dz = dz;
  ma.d_tau = gr->tau;
  ma.d_q_chan = gr->q_chan_taps;
  ma.d_k_chan = gr->k_chan_taps;
  ma.d_q_seq = gr->q_seq_taps;
  ma.d_k_seq = gr->k_seq_taps;
  CCA_TRY(check_launch(launch_mix_backward<TI, TV>(s, taps_of(w), ma, st), st));
  // down-projection: dx = dz W_qkv, dW_qkv = dz^T x
  CCA_TRY(check_launch(launch_transpose_2d<TV, TV>((const TV *)w->w_qkv, trp<TV>(ws, L, TR_WQKVT),
                                                   N, N, E, E, N, st), st));
  CCA_TRY(check_launch(launch_gemm_nt<TV, TV>(dz, trp<TV>(ws, L, TR_WQKVT), (TV *)gr->x, BT, E, N,
                                              N, N, E, st), st));
  return check_launch(weight_grad<TV>(dz, (const TV *)x, gr->w_qkv, N, E, BT, BTp,
                                      trp<TV>(ws, L, TR_DZT), trp<TV>(ws, L, TR_XT),
                                      trp<float>(ws, L, TR_SPLITK), skf, st), st);
}

cca_config decode_cfg(const cca_config *c) {
  cca_config d = *c;
  d.seq_len = 1;
  return d;
}

}  // namespace

// ============================================================================
extern "C" {

const char *cca_status_string(cca_status s) {
  switch (s) {
    case CCA_OK: return "CCA_OK";
    case CCA_ERR_INVALID_ARG: return "CCA_ERR_INVALID_ARG: invalid argument";
    case CCA_ERR_UNSUPPORTED: return "CCA_ERR_UNSUPPORTED: configuration not supported";
    case CCA_ERR_WORKSPACE: return "CCA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case CCA_ERR_HIP: return "CCA_ERR_HIP: HIP launch or runtime error";
  }
  return "CCA_ERR_UNKNOWN";
}

cca_status cca_validate_config(const cca_config *cfg) { return validate_shape(cfg, true); }

size_t cca_prefill_workspace_size(const cca_config *cfg) {
  if (validate_shape(cfg, true) != CCA_OK) return 0;
  return prefill_layout(*cfg).total;
}

size_t cca_decode_workspace_size(const cca_config *cfg, int32_t cache_len) {
  if (validate_shape(cfg, false) != CCA_OK || cache_len < 0) return 0;
  return decode_layout(decode_cfg(cfg), cache_len).total;
}

cca_status cca_prefill_workspace_layout(const cca_config *cfg, size_t offsets[CCA_WS_COUNT]) {
  cca_status r = validate_shape(cfg, true);
  if (r != CCA_OK) return r;
  if (!offsets) return CCA_ERR_INVALID_ARG;
  Layout L = prefill_layout(*cfg);
  for (int i = 0; i < CCA_WS_COUNT; ++i) offsets[i] = L.off[i];
  return CCA_OK;
}

cca_status cca_decode_workspace_layout(const cca_config *cfg, int32_t cache_len,
                                       size_t offsets[CCA_WS_COUNT]) {
  cca_status r = validate_shape(cfg, false);
  if (r != CCA_OK) return r;
  if (!offsets || cache_len < 0) return CCA_ERR_INVALID_ARG;
  Layout L = decode_layout(decode_cfg(cfg), cache_len);
  for (int i = 0; i < CCA_WS_COUNT; ++i) offsets[i] = L.off[i];
  return CCA_OK;
}

static cca_status prefill_checks(const cca_config *cfg, const cca_weights *w, void *ws,
                                 size_t wsb, Layout *L) {
  CCA_TRY(validate_shape(cfg, true));
  CCA_TRY(check_weights(*cfg, w));
  *L = prefill_layout(*cfg);
  return check_ws(ws, wsb, L->total);
}

cca_status cca_prefill_forward(const cca_config *cfg, const cca_weights *w, const void *x, void *y,
                               const cca_state *state_out, void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(prefill_checks(cfg, w, ws, wsb, &L));
  if (!x || !y || !aligned16(x) || !aligned16(y)) return CCA_ERR_INVALID_ARG;
  CCA_TRY(check_state_out(*cfg, state_out));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CCA_TRY(run_downproj(*cfg, w, x, ws, L, st));
  CCA_TRY(run_convmix(*cfg, w, state_of(state_out), ws, L, st));
  CCA_TRY(run_attention(*cfg, w, ws, L, st));
  return run_upproj(*cfg, w, y, ws, L, cfg->batch * cfg->seq_len, st);
}

cca_status cca_prefill_forward_fused(const cca_config *cfg, const cca_weights *w, const void *x,
                                     void *y, void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(prefill_checks(cfg, w, ws, wsb, &L));
  if (!x || !y || !aligned16(x) || !aligned16(y)) return CCA_ERR_INVALID_ARG;
  if (!fused_downproj_mix(*cfg)) return CCA_ERR_UNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CCA_TRY(run_downproj_mix(*cfg, w, x, ws, L, st));
  CCA_TRY(run_attention(*cfg, w, ws, L, st));
  return run_upproj(*cfg, w, y, ws, L, cfg->batch * cfg->seq_len, st);
}

cca_status cca_stage_downproj(const cca_config *cfg, const cca_weights *w, const void *x,
                              void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(prefill_checks(cfg, w, ws, wsb, &L));
  if (!x || !aligned16(x)) return CCA_ERR_INVALID_ARG;
  return run_downproj(*cfg, w, x, ws, L, reinterpret_cast<hipStream_t>(stream));
}

cca_status cca_stage_convmix(const cca_config *cfg, const cca_weights *w, const cca_state *so,
                             void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(prefill_checks(cfg, w, ws, wsb, &L));
  CCA_TRY(check_state_out(*cfg, so));
  return run_convmix(*cfg, w, state_of(so), ws, L, reinterpret_cast<hipStream_t>(stream));
}

cca_status cca_stage_attention(const cca_config *cfg, const cca_weights *w, void *ws, size_t wsb,
                               void *stream) {
  Layout L;
  CCA_TRY(prefill_checks(cfg, w, ws, wsb, &L));
  return run_attention(*cfg, w, ws, L, reinterpret_cast<hipStream_t>(stream));
}

cca_status cca_stage_upproj(const cca_config *cfg, const cca_weights *w, void *y, void *ws,
                            size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(prefill_checks(cfg, w, ws, wsb, &L));
  if (!y || !aligned16(y)) return CCA_ERR_INVALID_ARG;
  return run_upproj(*cfg, w, y, ws, L, cfg->batch * cfg->seq_len,
                    reinterpret_cast<hipStream_t>(stream));
}

// ---- decode ----------------------------------------------------------------

static cca_status decode_checks(const cca_config *cfg, const cca_weights *w, int32_t L,
                                void *ws, size_t wsb, Layout *lay) {
  CCA_TRY(validate_shape(cfg, false));
  CCA_TRY(check_weights(*cfg, w));
  if (L < 0) return CCA_ERR_INVALID_ARG;
  *lay = decode_layout(decode_cfg(cfg), L);
  return check_ws(ws, wsb, lay->total);
}

// The decode down-projection.  With few rows it leaves the split-contraction
// partials in CCA_WS_SPLITK for the mixing kernel to sum (no reduction
// launch); dec_qkv() describes what it left.
static cca_status dec_downproj(const cca_config &c, const cca_weights *w, const void *x_t,
                               void *ws, const Layout &L, hipStream_t st, int m = 1) {
  const int M = c.batch * m, E = c.d_model;
  const int N = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  float *qkv = reinterpret_cast<float *>(wsp(ws, L, CCA_WS_QKV));
  size_t skf;
  float *sk = splitk_ptr(ws, L, &skf);
  int slices = 0;
  hipError_t e;
  if (c.dtype == CCA_BF16)
    e = launch_gemm_nt_partials<bf16>((const bf16 *)x_t, (const bf16 *)w->w_qkv, qkv, M, N, E, E,
                                      E, sk, skf, &slices, st);
  else
    e = launch_gemm_nt_partials<float>((const float *)x_t, (const float *)w->w_qkv, qkv, M, N, E,
                                       E, E, sk, skf, &slices, st);
  return check_launch(e, st);
}

static DecQkv dec_qkv(const cca_config &c, void *ws, const Layout &L, int m) {
  const int M = c.batch * m, E = c.d_model;
  const int N = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  size_t skf;
  float *sk = splitk_ptr(ws, L, &skf);
  DecQkv d;
  d.qkv = reinterpret_cast<const float *>(wsp(ws, L, CCA_WS_QKV));
  d.parts = sk;
  d.slices = sk ? gemm_nt_partial_slices(M, N, E, (int)elem_size(c.dtype), skf) : 0;
  return d;
}

static cca_status dec_mix(const cca_config &c, const cca_weights *w, int32_t Lc,
                          const int32_t *lens, const StateOut &si, const StateOut &so, void *ws,
                          const Layout &L, hipStream_t st, int m = 1) {
  MixShape s = mix_shape(c);
  s.T = m;                       // new tokens per sequence
  s.Tp = m;
  const DecQkv qkv = dec_qkv(c, ws, L, m);
  float *q = reinterpret_cast<float *>(wsp(ws, L, CCA_WS_Q));
  hipError_t e;
  if (c.chan_conv_mode == CCA_CHAN_GROUPED) {
    if (c.dtype == CCA_BF16)
      e = launch_convmix_decode_grouped<bf16>(s, taps_of(w), w->q_chan_dense, w->k_chan_dense, qkv,
                                              Lc, lens, si, so, q, st);
    else
      e = launch_convmix_decode_grouped<float>(s, taps_of(w), w->q_chan_dense, w->k_chan_dense, qkv,
                                               Lc, lens, si, so, q, st);
  } else if (c.dtype == CCA_BF16) {
    e = launch_convmix_decode<bf16>(s, taps_of(w), qkv, Lc, lens, si, so, q, st);
  } else {
    e = launch_convmix_decode<float>(s, taps_of(w), qkv, Lc, lens, si, so, q, st);
  }
  return check_launch(e, st);
}

static cca_status dec_attn(const cca_config &c, const cca_weights *w, int32_t Lc,
                           const int32_t *lens, const StateOut &cache, void *ws, const Layout &L,
                           hipStream_t st, int m = 1) {
  MixShape s = mix_shape(c);
  s.T = m;                       // new tokens per sequence
  s.Tp = m;
  const float *q = reinterpret_cast<const float *>(wsp(ws, L, CCA_WS_Q));
  float *part = reinterpret_cast<float *>(wsp(ws, L, CCA_WS_PART));
  hipError_t e;
  if (c.dtype == CCA_BF16)
    e = launch_attention_decode<bf16>(s, q, cache, Lc + m, lens, w->tau, part,
                                      (bf16 *)wsp(ws, L, CCA_WS_O), st);
  else
    e = launch_attention_decode<float>(s, q, cache, Lc + m, lens, w->tau, part,
                                       (float *)wsp(ws, L, CCA_WS_O), st);
  return check_launch(e, st);
}

cca_status cca_decode_step(const cca_config *cfg, const cca_weights *w, const void *x_t,
                           int32_t cache_len, const cca_state *si, const cca_state *so, void *y_t,
                           void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(decode_checks(cfg, w, cache_len, ws, wsb, &L));
  if (!x_t || !y_t || !aligned16(x_t) || !aligned16(y_t)) return CCA_ERR_INVALID_ARG;
  const cca_config c = decode_cfg(cfg);
  CCA_TRY(check_decode_state(c, cache_len, si, so));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CCA_TRY(dec_downproj(c, w, x_t, ws, L, st));
  CCA_TRY(dec_mix(c, w, cache_len, nullptr, state_of(si), state_of(so), ws, L, st));
  CCA_TRY(dec_attn(c, w, cache_len, nullptr, state_of(si), ws, L, st));
  return run_upproj(c, w, y_t, ws, L, c.batch, st);
}

cca_status cca_decode_step_varlen(const cca_config *cfg, const cca_weights *w, const void *x_t,
                                  const int32_t *cache_lens, int32_t max_cache_len,
                                  const cca_state *si, const cca_state *so, void *y_t, void *ws,
                                  size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(decode_checks(cfg, w, max_cache_len, ws, wsb, &L));
  if (!x_t || !y_t || !aligned16(x_t) || !aligned16(y_t)) return CCA_ERR_INVALID_ARG;
  if (!cache_lens || reinterpret_cast<uintptr_t>(cache_lens) % 4) return CCA_ERR_INVALID_ARG;
  const cca_config c = decode_cfg(cfg);
  CCA_TRY(check_decode_state(c, max_cache_len, si, so));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CCA_TRY(dec_downproj(c, w, x_t, ws, L, st));
  CCA_TRY(dec_mix(c, w, max_cache_len, cache_lens, state_of(si), state_of(so), ws, L, st));
  CCA_TRY(dec_attn(c, w, max_cache_len, cache_lens, state_of(si), ws, L, st));
  return run_upproj(c, w, y_t, ws, L, c.batch, st);
}

cca_status cca_stage_decode_downproj(const cca_config *cfg, const cca_weights *w, const void *x_t,
                                     int32_t cache_len, void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(decode_checks(cfg, w, cache_len, ws, wsb, &L));
  if (!x_t || !aligned16(x_t)) return CCA_ERR_INVALID_ARG;
  return dec_downproj(decode_cfg(cfg), w, x_t, ws, L, reinterpret_cast<hipStream_t>(stream));
}

cca_status cca_stage_decode_mix(const cca_config *cfg, const cca_weights *w, int32_t cache_len,
                                const cca_state *si, const cca_state *so, void *ws, size_t wsb,
                                void *stream) {
  Layout L;
  CCA_TRY(decode_checks(cfg, w, cache_len, ws, wsb, &L));
  const cca_config c = decode_cfg(cfg);
  CCA_TRY(check_decode_state(c, cache_len, si, so));
  return dec_mix(c, w, cache_len, nullptr, state_of(si), state_of(so), ws, L,
                 reinterpret_cast<hipStream_t>(stream));
}

cca_status cca_stage_decode_attention(const cca_config *cfg, const cca_weights *w,
                                      int32_t cache_len, const cca_state *si, void *ws,
                                      size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(decode_checks(cfg, w, cache_len, ws, wsb, &L));
  const cca_config c = decode_cfg(cfg);
  CCA_TRY(check_decode_state(c, cache_len, si, si));
  return dec_attn(c, w, cache_len, nullptr, state_of(si), ws, L,
                  reinterpret_cast<hipStream_t>(stream));
}

cca_status cca_stage_decode_upproj(const cca_config *cfg, const cca_weights *w, int32_t cache_len,
                                   void *y_t, void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(decode_checks(cfg, w, cache_len, ws, wsb, &L));
  if (!y_t || !aligned16(y_t)) return CCA_ERR_INVALID_ARG;
  const cca_config c = decode_cfg(cfg);
  return run_upproj(c, w, y_t, ws, L, c.batch, reinterpret_cast<hipStream_t>(stream));
}

// ---- training ----------------------------------------------------------------

size_t cca_train_workspace_size(const cca_config *cfg) {
  if (validate_shape(cfg, true) != CCA_OK || cfg->chan_conv_mode != CCA_CHAN_PER_HEAD) return 0;
  return train_layout(*cfg).total;
}

cca_status cca_prefill_forward_train(const cca_config *cfg, const cca_weights *w, const void *x,
                                     void *y, void *ws, size_t wsb, void *stream) {
  CCA_TRY(validate_shape(cfg, true));
  if (cfg->chan_conv_mode != CCA_CHAN_PER_HEAD) return CCA_ERR_UNSUPPORTED;
  CCA_TRY(check_weights(*cfg, w));
  const TrainLayout TL = train_layout(*cfg);
  CCA_TRY(check_ws(ws, wsb, TL.total));
  if (!x || !y || !aligned16(x) || !aligned16(y)) return CCA_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Layout &L = TL.pre;
  CCA_TRY(run_downproj(*cfg, w, x, ws, L, st));
  CCA_TRY(run_convmix(*cfg, w, state_of((const cca_state *)nullptr), ws, L, st,
                      keeps_bpost(*cfg) ? trp<float>(ws, TL, TR_BPOST) : nullptr));
  CCA_TRY(run_attention(*cfg, w, ws, L, st, trp<float>(ws, TL, TR_LSE)));
  return run_upproj(*cfg, w, y, ws, L, cfg->batch * cfg->seq_len, st);
}

cca_status cca_prefill_backward(const cca_config *cfg, const cca_weights *w, const void *x,
                                const void *dy, const cca_grads *g, void *ws, size_t wsb,
                                void *stream) {
  CCA_TRY(validate_shape(cfg, true));
  if (cfg->chan_conv_mode != CCA_CHAN_PER_HEAD) return CCA_ERR_UNSUPPORTED;
  CCA_TRY(check_weights(*cfg, w));
  const TrainLayout TL = train_layout(*cfg);
  CCA_TRY(check_ws(ws, wsb, TL.total));
  if (!x || !dy || !aligned16(x) || !aligned16(dy)) return CCA_ERR_INVALID_ARG;
  if (!g || !g->x || !g->w_qkv || !g->w_o || !g->q_seq_taps || !g->k_seq_taps ||
      !g->q_chan_taps || !g->k_chan_taps || !g->tau)
    return CCA_ERR_INVALID_ARG;
  if (!aligned16(g->x) || !aligned16(g->w_qkv) || !aligned16(g->w_o)) return CCA_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (cfg->dtype == CCA_F32) return run_backward<float, float>(*cfg, w, x, dy, g, ws, TL, st);
  if (qk_is_f16(*cfg)) return run_backward<f16, bf16>(*cfg, w, x, dy, g, ws, TL, st);
  return run_backward<bf16, bf16>(*cfg, w, x, dy, g, ws, TL, st);
}

}  // extern "C"

// ---- paged cache -------------------------------------------------------------

static cca_status check_paged(const cca_config &c, const cca_paged_state *p, long long need_rows) {
  if (!p) return CCA_ERR_INVALID_ARG;
  if (!p->k_pages || !p->v_pages || !p->block_table) return CCA_ERR_INVALID_ARG;
  if (!aligned16(p->k_pages) || !aligned16(p->v_pages) ||
      reinterpret_cast<uintptr_t>(p->block_table) % 4)
    return CCA_ERR_INVALID_ARG;
  if (p->page_size < 32 || p->page_size % 32 || p->num_pages < 1 || p->max_pages_per_seq < 1)
    return CCA_ERR_INVALID_ARG;
  if ((long long)p->max_pages_per_seq * p->page_size < need_rows) return CCA_ERR_INVALID_ARG;
  if ((long long)p->num_pages * c.n_kv_heads * p->page_size * c.head_dim > (1ll << 40))
    return CCA_ERR_UNSUPPORTED;
  return CCA_OK;
}

extern "C" {

cca_status cca_decode_step_paged(const cca_config *cfg, const cca_weights *w, const void *x_t,
                                 const int32_t *cache_lens, int32_t max_cache_len,
                                 const cca_paged_state *si, const cca_paged_state *so, void *y_t,
                                 void *ws, size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(decode_checks(cfg, w, max_cache_len, ws, wsb, &L));
  if (!x_t || !y_t || !aligned16(x_t) || !aligned16(y_t)) return CCA_ERR_INVALID_ARG;
  if (!cache_lens || reinterpret_cast<uintptr_t>(cache_lens) % 4) return CCA_ERR_INVALID_ARG;
  const cca_config c = decode_cfg(cfg);
  CCA_TRY(check_paged(c, si, (long long)max_cache_len + 1));
  if (!so) return CCA_ERR_INVALID_ARG;
  if ((so->k_pages && so->k_pages != si->k_pages) || (so->v_pages && so->v_pages != si->v_pages) ||
      (so->block_table && so->block_table != si->block_table))
    return CCA_ERR_INVALID_ARG;
  if (c.seq_conv_k > 1 && (!si->conv_q || !si->conv_k || !so->conv_q || !so->conv_k))
    return CCA_ERR_INVALID_ARG;
  if (c.use_value_shift && (!si->vshift || !so->vshift)) return CCA_ERR_INVALID_ARG;
  if (c.dtype == CCA_BF16 && !decode_pages_fit(c.batch, c.n_kv_heads, max_cache_len + 1, si->page_size))
    return CCA_ERR_UNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const StateOut in = state_of(si), out = state_of(so);
  CCA_TRY(dec_downproj(c, w, x_t, ws, L, st));
  CCA_TRY(dec_mix(c, w, max_cache_len, cache_lens, in, out, ws, L, st));
  CCA_TRY(dec_attn(c, w, max_cache_len, cache_lens, in, ws, L, st));
  return run_upproj(c, w, y_t, ws, L, c.batch, st);
}

cca_status cca_prefill_forward_paged(const cca_config *cfg, const cca_weights *w, const void *x,
                                     void *y, const cca_paged_state *so, void *ws, size_t wsb,
                                     void *stream) {
  Layout L;
  CCA_TRY(prefill_checks(cfg, w, ws, wsb, &L));
  if (!x || !y || !aligned16(x) || !aligned16(y)) return CCA_ERR_INVALID_ARG;
  if (!so) return CCA_ERR_INVALID_ARG;
  if (so->k_pages || so->v_pages) CCA_TRY(check_paged(*cfg, so, cfg->seq_len));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CCA_TRY(run_downproj(*cfg, w, x, ws, L, st));
  CCA_TRY(run_convmix(*cfg, w, state_of(so), ws, L, st));
  CCA_TRY(run_attention(*cfg, w, ws, L, st));
  return run_upproj(*cfg, w, y, ws, L, cfg->batch * cfg->seq_len, st);
}

}  // extern "C"

// ---- several new tokens per sequence -----------------------------------------

static constexpr int MAX_NEW_TOKENS = 16;

static cca_status multi_checks(const cca_config *cfg, const cca_weights *w, int32_t n_new,
                               int32_t Lmax, void *ws, size_t wsb, Layout *lay) {
  CCA_TRY(validate_shape(cfg, false));
  CCA_TRY(check_weights(*cfg, w));
  if (n_new < 1 || Lmax < 0) return CCA_ERR_INVALID_ARG;
  const int G = cfg->n_q_heads / cfg->n_kv_heads;
  const bool fits = cfg->chan_conv_mode == CCA_CHAN_GROUPED
                        ? convmix_decode_grouped_fits(G, cfg->head_dim, n_new, cfg->seq_conv_k,
                                                      cfg->chan_conv_k)
                        : convmix_decode_fits(G, cfg->head_dim, n_new);
  if (n_new > MAX_NEW_TOKENS || !fits) return CCA_ERR_UNSUPPORTED;
  *lay = decode_layout(decode_cfg(cfg), Lmax, n_new);
  return check_ws(ws, wsb, lay->total);
}

extern "C" {

size_t cca_decode_multi_workspace_size(const cca_config *cfg, int32_t n_new, int32_t max_cache_len) {
  if (validate_shape(cfg, false) != CCA_OK || n_new < 1 || n_new > MAX_NEW_TOKENS ||
      max_cache_len < 0)
    return 0;
  return decode_layout(decode_cfg(cfg), max_cache_len, n_new).total;
}

cca_status cca_decode_multi(const cca_config *cfg, const cca_weights *w, const void *x_new,
                            int32_t n_new, const int32_t *cache_lens, int32_t max_cache_len,
                            const cca_state *si, const cca_state *so, void *y_new, void *ws,
                            size_t wsb, void *stream) {
  Layout L;
  CCA_TRY(multi_checks(cfg, w, n_new, max_cache_len, ws, wsb, &L));
  if (!x_new || !y_new || !aligned16(x_new) || !aligned16(y_new)) return CCA_ERR_INVALID_ARG;
  if (!cache_lens || reinterpret_cast<uintptr_t>(cache_lens) % 4) return CCA_ERR_INVALID_ARG;
  const cca_config c = decode_cfg(cfg);
  // the last new token's slot must fit: capacity > max_cache_len + n_new - 1
  CCA_TRY(check_decode_state(c, max_cache_len + n_new - 1, si, so));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CCA_TRY(dec_downproj(c, w, x_new, ws, L, st, n_new));
  CCA_TRY(dec_mix(c, w, max_cache_len, cache_lens, state_of(si), state_of(so), ws, L, st, n_new));
  CCA_TRY(dec_attn(c, w, max_cache_len, cache_lens, state_of(si), ws, L, st, n_new));
  return run_upproj(c, w, y_new, ws, L, c.batch * n_new, st);
}

cca_status cca_decode_multi_paged(const cca_config *cfg, const cca_weights *w, const void *x_new,
                                  int32_t n_new, const int32_t *cache_lens,
                                  int32_t max_cache_len, const cca_paged_state *si,
                                  const cca_paged_state *so, void *y_new, void *ws, size_t wsb,
                                  void *stream) {
  Layout L;
  CCA_TRY(multi_checks(cfg, w, n_new, max_cache_len, ws, wsb, &L));
  if (!x_new || !y_new || !aligned16(x_new) || !aligned16(y_new)) return CCA_ERR_INVALID_ARG;
  if (!cache_lens || reinterpret_cast<uintptr_t>(cache_lens) % 4) return CCA_ERR_INVALID_ARG;
  const cca_config c = decode_cfg(cfg);
  CCA_TRY(check_paged(c, si, (long long)max_cache_len + n_new));
  if (!so) return CCA_ERR_INVALID_ARG;
  if ((so->k_pages && so->k_pages != si->k_pages) || (so->v_pages && so->v_pages != si->v_pages) ||
      (so->block_table && so->block_table != si->block_table))
    return CCA_ERR_INVALID_ARG;
  if (c.seq_conv_k > 1 && (!si->conv_q || !si->conv_k || !so->conv_q || !so->conv_k))
    return CCA_ERR_INVALID_ARG;
  if (c.use_value_shift && (!si->vshift || !so->vshift)) return CCA_ERR_INVALID_ARG;
  if (c.dtype == CCA_BF16 &&
      !decode_pages_fit(c.batch, c.n_kv_heads, max_cache_len + n_new, si->page_size))
    return CCA_ERR_UNSUPPORTED;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const StateOut in = state_of(si), out = state_of(so);
  CCA_TRY(dec_downproj(c, w, x_new, ws, L, st, n_new));
  CCA_TRY(dec_mix(c, w, max_cache_len, cache_lens, in, out, ws, L, st, n_new));
  CCA_TRY(dec_attn(c, w, max_cache_len, cache_lens, in, ws, L, st, n_new));
  return run_upproj(c, w, y_new, ws, L, c.batch * n_new, st);
}

}  // extern "C"

// ---- decode step without a caller workspace ----------------------------------
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the decode
// step's workspace lives in a file-scope device array of CCA_NOALLOC_SCRATCH
// bytes.  Each GPU the library runs on holds its own copy until the process
// ends.  Host code never uses the array's name as an address: the first call
// on a device takes the array's device address with hipGetSymbolAddress
// (that device current) and keeps it per device.

static constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)CCA_NOALLOC_SCRATCH;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptrs[MAX_DEVICES] = {};

// The current device's copy of `scratch`.
cca_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CCA_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return CCA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptrs[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CCA_ERR_HIP;
    scratch_ptrs[dev] = p;
  }
  *out = scratch_ptrs[dev];
  return CCA_OK;
}

}  // namespace

extern "C" {

cca_status cca_decode_step_noalloc(const cca_config *cfg, const cca_weights *w, const void *x_t,
                                   int32_t cache_len, const cca_state *si, const cca_state *so,
                                   void *y_t, void *stream) {
  CCA_TRY(validate_shape(cfg, false));
  if (cache_len < 0) return CCA_ERR_INVALID_ARG;
  // the workspace the step needs must fit the array; checked before any HIP call
  const size_t need = decode_layout(decode_cfg(cfg), cache_len).total;
  if (need > NOALLOC_SCRATCH_BYTES) return CCA_ERR_WORKSPACE;
  void *ws = nullptr;
  CCA_TRY(scratch_of_current_device(&ws));
  return cca_decode_step(cfg, w, x_t, cache_len, si, so, y_t, ws, NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
