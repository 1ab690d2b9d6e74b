// Internal launchers of the libcca kernels.  Every launcher only enqueues
// work on `stream` and returns hipGetLastError(); shapes have been validated
// by the host API before any of them is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cca {

// C[M,N] = A[M,K] * B[N,K]^T, fp32 accumulation.  K * sizeof(Tin) must be a
// multiple of 16 bytes and every row 16-byte aligned.  With M <= 64 and a
// fp32 scratch of splitk_floats floats, the contraction is split over
// workgroups and reduced by a second kernel (deterministic order).
template <typename Tin, typename Tout>
hipError_t launch_gemm_nt(const Tin *A, const Tin *B, Tout *C, int M, int N, int K, int lda,
                          int ldb, int ldc, hipStream_t stream, float *splitk_ws = nullptr,
                          size_t splitk_floats = 0);

// Contraction slices the skinny path uses for an M x N x K product.
int gemm_splitk_slices(int M, int N, int K, int elem_bytes);

// The skinny split-contraction product without its reduction kernel: with
// M <= 64 and room in splitk_ws, writes the S fp32 partial products
// [S][M][N] there and sets *slices = S (gemm_nt_partial_slices); otherwise
// writes the fp32 product to C (ldc = N) and sets *slices = 0.  Consumers sum
// slice 0 .. S-1 in that order.
int gemm_nt_partial_slices(int M, int N, int K, int elem_bytes, size_t splitk_floats);
template <typename Tin>
hipError_t launch_gemm_nt_partials(const Tin *A, const Tin *B, float *C, int M, int N, int K,
                                   int lda, int ldb, float *splitk_ws, size_t splitk_floats,
                                   int *slices, hipStream_t stream);

// C[M,N] (fp32, ldc = N) = A[M,K] * B[N,K]^T for few output tiles and a long
// contraction (weight gradients): the contraction is split over
// gemm_long_k_slices() workgroup slices whose fp32 partials go to ws
// (slices * M * N floats) and are summed in a fixed order; without room in
// ws it is one plain product.
int gemm_long_k_slices(int M, int N, int K);
template <typename Tin>
hipError_t launch_gemm_nt_long_k(const Tin *A, const Tin *B, float *C, int M, int N, int K, int lda,
                                 int ldb, float *ws, size_t ws_floats, hipStream_t stream);

// C[M,N] (fp32, ldc = N) = A^T B for row-major A [K][lda] and B [K][ldb]
// (bf16), the contraction over rows (tokens): the same slices as above, the
// operands read in place through LDS transpose reads.  hipErrorNotSupported
// (nothing launched) unless M and N are multiples of 128, lda and ldb
// multiples of 8 (16-byte rows), A and B 16-byte aligned and (K + 64) rows of
// either operand under 2 GiB.
hipError_t launch_gemm_tn_long_k(const bf16 *A, const bf16 *B, float *C, int M, int N, int K,
                                 int lda, int ldb, float *ws, size_t ws_floats,
                                 hipStream_t stream);

// Sizes shared by the mixing and attention kernels.
struct MixShape {
  int B, T, Tp;            // batch, tokens, tokens padded to the query tile
  int Hq, Hkv, G, d;       // heads and head dim
  int ks, kc;              // conv taps (1..4)
  int use_mean;            // q-k-mean: 0 off, 1 pre-conv q and k, 2 pre- and post-conv q and k
  int use_shift, use_norm;
  int grouped;             // channel conv: 0 per-head filter along channels, 1 dense per lag
  float rope_base, eps;
  int attn_kernel;         // prefill attention: 1 four-wave, 2 eight-wave ping-pong, 0 by grid size
  // RoPE frequencies base^(-2i/d), i < d/2, evaluated on the host in double
  // precision (all zero when RoPE is off); passed by value with the launch.
  double theta[64];
};

struct MixTaps {
  const float *q_seq, *k_seq, *q_chan, *k_chan;
  const float *tau;   // [H_q]; the prefill mixing stores tau_h * log2(e) * q_hat
};

// A latent KV cache and the carried conv window / value-shift state (any
// pointer may be null).  The cache is either contiguous, [B, Hkv, capacity,
// d], or paged: pages [npages, Hkv, page, d] with table[b * mpps + key /
// page] the page that holds sequence b's keys [page * j, page * (j + 1));
// table entries outside [0, npages) are clamped (wrong rows, never a fault).
struct StateOut {
  void *k_cache, *v_cache;
  int capacity;
  void *conv_q, *conv_k, *vshift;
  const int *table;     // null: contiguous
  int page, mpps, npages;
};

// Row index (times d gives the element offset) of sequence b's key `key` of
// kv head g in the cache described by st.  For reads: a block-table entry
// outside [0, npages) is clamped (a wrong row, never a fault).
__host__ __device__ inline size_t cache_row(const StateOut &st, int b, int Hkv, int g, int key) {
  if (!st.table) return (size_t)(b * Hkv + g) * st.capacity + key;
  int pg = st.table[(size_t)b * st.mpps + key / st.page];
  pg = pg < 0 ? 0 : (pg >= st.npages ? st.npages - 1 : pg);
  return ((size_t)pg * Hkv + g) * st.page + key % st.page;
}

// The same row for a store, or false when the block-table entry lies outside
// [0, npages): then nothing is written (a clamped row would belong to another
// sequence).
__host__ __device__ inline bool cache_row_store(const StateOut &st, int b, int Hkv, int g, int key,
                                                size_t *row) {
  if (!st.table) {
    *row = (size_t)(b * Hkv + g) * st.capacity + key;
    return true;
  }
  const int pg = st.table[(size_t)b * st.mpps + key / st.page];
  if (pg < 0 || pg >= st.npages) return false;
  *row = ((size_t)pg * Hkv + g) * st.page + key % st.page;
  return true;
}

// Fused sequence conv + channel conv + q-k-mean + value-shift + L2 norm + RoPE
// over a prefill.  qkv: [B*T, e_q + 2 e_kv] in TI (fp16 in bf16 mode, fp32 in
// fp32 mode).  Writes q [B,Hq,Tp,d] and k [B,Hkv,Tp,d] in TQ, vt [B,Hkv,d,Tp]
// in TV (token order permuted inside 16-token groups), zeros in the padding
// tokens [T, Tp).  With r1b (the grouped channel conv's output, fp32
// [B*T, e_q + e_kv]) the two convolutions are taken from there instead.
// bout (nullable): receives the channel-conv output b of every q and k head,
// fp32 [B*T, e_q + e_kv] (the backward of the pre- and post-convolution mean
// reads it).
template <typename TI, typename TQ, typename TV>
hipError_t launch_convmix_prefill(const MixShape &s, const MixTaps &w, const TI *qkv, TQ *q,
                                  TQ *k, TV *vt, const StateOut &st, hipStream_t stream,
                                  const float *r1b = nullptr, float *bout = nullptr);

// Grouped reading of the channel conv over a prefill (d in {16, 32, 64}):
// outb[b*T + t, col] = sum over lags j < k_c and channels c of
// W[h, i, j, c] * a[t - j, h, c], a the sequence conv of qkv's q / k columns,
// for every q head (columns h*d + i) and k head (e_q + g*d + i); W is fp32
// [H, d, k_c, d] per kind (dense_q for the H_q query heads, dense_k for the
// H_kv key heads).  bf16 mode multiplies in fp16 on MFMA, fp32 mode on the
// VALU in fp32.
// qkv: fp32 in fp32 mode, fp16 in bf16 mode (the down-projection's output).
hipError_t launch_grouped_conv_prefill(const MixShape &s, const MixTaps &w, const float *dense_q,
                                       const float *dense_k, const void *qkv, float *outb,
                                       bool f32, hipStream_t stream);
bool grouped_conv_supported(int d, bool f32);

// The down-projection output of a decode step: qkv [M, N] fp32 when
// slices == 0, else the sum over s < slices of parts [slices][M][N] (the
// split-contraction partials, summed in slice order).
struct DecQkv {
  const float *qkv, *parts;
  int slices;
};

// The same mixing for m = s.T new tokens per sequence at positions L .. L+m-1
// (L per sequence lens[b], clamped to [0, L], when lens is not null), using
// the carried window / vshift of state_in; the down-projection output has
// rows [B*m, e_q + 2 e_kv]; writes q (fp32 [B, m, Hq, d]), the k and v rows
// at those cache slots, and the rolled state into state_out.
template <typename TV>
hipError_t launch_convmix_decode(const MixShape &s, const MixTaps &w, const DecQkv &qkv, int L,
                                 const int *lens, const StateOut &in, const StateOut &out,
                                 float *q, hipStream_t stream);

// The decode mixing under the grouped channel conv: the same outputs as
// launch_convmix_decode, with the window of (k_s - 1) + (k_c - 1) pre-conv
// rows and the dense per-lag channel weights (fp32 [H, d, k_c, d]).
template <typename TV>
hipError_t launch_convmix_decode_grouped(const MixShape &s, const MixTaps &w, const float *dense_q,
                                         const float *dense_k, const DecQkv &qkv, int L,
                                         const int *lens, const StateOut &in, const StateOut &out,
                                         float *q, hipStream_t stream);
bool convmix_decode_grouped_fits(int G, int d, int m, int ks, int kc);

// Causal flash attention inside the latent heads; q holds tau_h * log2(e) *
// q_hat (the mixing kernel applies the temperature); tau [Hq] (device) bounds
// the logits when the L2 norm is on.  o [B*T, Hq*d] in TV.  lse (nullable):
// fp32 [B, Hq, Tp], log2 of each query's softmax denominator in the exp2
// domain (rows t < T), for the backward pass.
template <typename TQ, typename TV>
hipError_t launch_attention_prefill(const MixShape &s, const TQ *q, const TQ *k, const TV *vt,
                                    const float *tau, TV *o, float *lse, hipStream_t stream);
bool attention_supported(int d, bool f32);

// Split-KV decode attention of m = s.T new tokens per sequence (q [B, m, Hq,
// d]) over Lk = L + m cached keys (per sequence lens[b] + m, lens clamped to
// [0, Lk - m], when lens is not null; the chunking follows Lk) of the cache
// `cache` (contiguous or paged); new token j sees keys 0 .. L + j.  Then the
// log-sum-exp combine into o [B*m, Hq*d].  part: fp32 scratch of
// decode_partial_floats(..., m) floats.
template <typename TV>
hipError_t launch_attention_decode(const MixShape &s, const float *q, const StateOut &cache, int Lk,
                                   const int *lens, const float *tau, float *part, TV *o,
                                   hipStream_t stream);

// Down-projection fused with the mixing steps (bf16 x and W_qkv; kv groups
// of one query head, d = 64, T a multiple of 128): writes q, k, vt as
// launch_convmix_prefill does, without the fp32 qkv~ in HBM.  halo_ws:
// downproj_mix_halo_bytes() bytes of scratch (the 3 rows before each
// 128-token tile, through a small GEMM).
bool downproj_mix_supported(int G, int d, int T, int E);
size_t downproj_mix_halo_bytes(int B, int T, int E, int N);
template <typename TQ, typename TV>
hipError_t launch_downproj_mix(const MixShape &s, const MixTaps &w, const bf16 *x,
                               const bf16 *wqkv, int E, void *halo_ws, TQ *q, TQ *k, TV *vt,
                               hipStream_t stream);

// Whether the mixing kernels' fp32 LDS tiles of one kv group (G query heads
// + k + v; 19 prefill tokens, 4 decode rows) fit the 64 KiB they may use.
bool convmix_fits(int G, int d);
// Whether the decode mixing tile of m new tokens fits its LDS.
bool convmix_decode_fits(int G, int d, int m);

// Keys handled by one workgroup of the split-KV decode attention, and the
// partial-state scratch it needs.
int decode_chunk_keys(int d);
// Whether one key chunk of a decode over Lk keys spans few enough pages of
// `page` rows for the page list the attention kernel keeps in LDS.
bool decode_pages_fit(int B, int Hkv, int Lk, int page);
size_t decode_partial_floats(int B, int Hq, int Hkv, int d, int Lk, int m = 1);

// ---- backward pass ---------------------------------------------------------

// Buffers of the attention backward.  Inputs: q, k (the forward's attention
// operands, [B,H,Tp,d]), vt ([B,Hkv,d,Tp], token-permuted), O and dO
// ([B*T, Hq*d]), lse ([B,Hq,Tp], exp2 domain).  Scratch it fills first: qT,
// dOT [B,Hq,d,Tp] and kT [B,Hkv,d,Tp] (token-permuted), vr [B,Hkv,Tp,d],
// dsum [B,Hq,Tp].  Outputs (fp32, token-major): gq [B*T, Hq*d] =
// sum_u ds k_hat (tau not applied), dk and dv [B*T, Hkv*d].
template <typename TQ, typename TV> struct AttnBwdArgs {
  const TQ *q, *k;
  const TV *vt, *O, *dO;
  const float *lse;
  TV *qT, *kT, *dOT, *vr;
  float *dsum, *dk, *dv, *gq;
};
template <typename TQ, typename TV>
hipError_t launch_attention_backward(const MixShape &s, const AttnBwdArgs<TQ, TV> &a,
                                     hipStream_t stream);

// Buffers of the mixing backward.  Inputs: qkv (the down-projection output,
// TI: fp16 in bf16 mode, fp32 in fp32 mode),
// gq, dk, dv from the attention backward.  Scratch: dm, da (fp32
// [B*T, e_q + e_kv]) and mix_backward_scratch_floats() floats.  Outputs: dz
// ([B*T, e_q + 2 e_kv], the down-projection output's cotangent) and the
// gradients of tau [Hq], the channel taps [Hq|Hkv, kc] and the sequence taps
// [e_q|e_kv, ks] (fp32, overwritten).
template <typename TI, typename TZ> struct MixBwdArgs {
  const TI *qkv;
  const float *bpost;   // q-k-mean of pre- and post-conv values: the forward's channel-conv output
  const float *gq, *dk, *dv;
  float *dm, *da, *scratch;
  TZ *dz;
  float *d_tau, *d_q_chan, *d_k_chan, *d_q_seq, *d_k_seq;
};
size_t mix_backward_scratch_floats(const MixShape &s);
template <typename TI, typename TZ>
hipError_t launch_mix_backward(const MixShape &s, const MixTaps &w, const MixBwdArgs<TI, TZ> &a,
                               hipStream_t stream);

// out[c * out_rs + r] = in[r * in_rs + c] for r < R, c < C; rows r >= Rvalid
// read as zero.
template <typename Tin, typename Tout>
hipError_t launch_transpose_2d(const Tin *in, Tout *out, int R, int Rvalid, int C, long long in_rs,
                               long long out_rs, hipStream_t stream);

}  // namespace cca
