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

// Sizes shared by the mixing and attention kernels.
struct MixShape {
  int B, T, Tp;            // batch, tokens, tokens padded to the query tile
  int Hq, Hkv, G, d;       // heads and head dim
  int ks, kc;              // conv taps (1..4)
  int use_mean, use_shift, use_norm;
  float rope_base, eps;
  // RoPE frequencies base^(-2i/d), i < d/2, evaluated on the host in double
  // precision (all zero when RoPE is off); passed by value with the launch.
  double theta[64];
};

struct MixTaps {
  const float *q_seq, *k_seq, *q_chan, *k_chan;
  const float *tau;   // [H_q]; the prefill mixing stores tau_h * log2(e) * q_hat
};

// Optional prefill outputs that seed a decode: cache rows [0, T) and the
// carried conv window / value-shift state (any pointer may be null).
struct StateOut {
  void *k_cache, *v_cache;
  int capacity;
  void *conv_q, *conv_k, *vshift;
};

// Fused sequence conv + channel conv + q-k-mean + value-shift + L2 norm + RoPE
// over a prefill.  qkv: fp32 [B*T, e_q + 2 e_kv].  Writes q [B,Hq,Tp,d] and
// k [B,Hkv,Tp,d] in TQ, vt [B,Hkv,d,Tp] in TV (token order permuted inside
// 16-token groups), zeros in the padding tokens [T, Tp).
template <typename TQ, typename TV>
hipError_t launch_convmix_prefill(const MixShape &s, const MixTaps &w, const float *qkv, TQ *q,
                                  TQ *k, TV *vt, const StateOut &st, hipStream_t stream);

// The same mixing for one new token per sequence at position L (per
// sequence lens[b], clamped to [0, L], when lens is not null), using the
// carried window / vshift of state_in; writes q (fp32 [B,Hq,d]), the k and v
// rows at that cache slot, and the rolled state into state_out.
template <typename TV>
hipError_t launch_convmix_decode(const MixShape &s, const MixTaps &w, const float *qkv, int L,
                                 const int *lens, const StateOut &in, const StateOut &out,
                                 float *q, hipStream_t stream);

// Causal flash attention inside the latent heads; q holds tau_h * log2(e) *
// q_hat (the mixing kernel applies the temperature); tau [Hq] (device) bounds
// the logits when the L2 norm is on.  o [B*T, Hq*d] in TV.
template <typename TQ, typename TV>
hipError_t launch_attention_prefill(const MixShape &s, const TQ *q, const TQ *k, const TV *vt,
                                    const float *tau, TV *o, hipStream_t stream);
bool attention_supported(int d, bool f32);

// Split-KV decode attention over Lk = L + 1 cached keys (per sequence
// lens[b] + 1, clamped to [1, Lk], when lens is not null; the chunking
// follows Lk), then the log-sum-exp combine.  part: fp32 scratch of
// decode_partial_floats() floats.
template <typename TV>
hipError_t launch_attention_decode(const MixShape &s, const float *q, const TV *k_cache,
                                   const TV *v_cache, int capacity, int Lk, const int *lens,
                                   const float *tau, float *part, TV *o, hipStream_t stream);

// Whether the mixing kernel's LDS tile of one kv group (G query heads + k +
// v, 19 tokens) fits the 64 KiB it may use.
bool convmix_fits(int G, int d);

// Keys handled by one workgroup of the split-KV decode attention, and the
// partial-state scratch it needs.
int decode_chunk_keys(int d);
size_t decode_partial_floats(int B, int Hq, int Hkv, int d, int Lk);

}  // namespace cca
