/*
 * libcca -- Compressed Convolutional Attention (CCA) and its grouped-query
 * variant (CCGQA), forward and backward pass on AMD Instinct MI355X (gfx950).
 *
 * The method (page tags as in the oracle's header):
 *   down-projection of hidden states to a latent q, k, v
 *       [GS-EN "2. Methodology" / Down-Projection; ABS]
 *   causal sequence convolution and channel convolution of q and k
 *       [GS-EN "2. Methodology" / Convolutional Mixing]
 *   q-k-mean, value-shift
 *       [GS-EN "2. Methodology" / Q-K-Mean, Value-Shift; EDG "How Compressed
 *        Convolutional Attention Works"]
 *   L2 normalisation with a per-head temperature, RoPE on the latent q, k
 *       [GS-EN "2. Methodology" / RoPE Integration]
 *   causal softmax attention inside the latent heads, kv heads shared by
 *   groups of G = H_q / H_kv query heads
 *       [GS-EN "2. Methodology" / Latent Space Operations, "Extension: CCGQA"]
 *   up-projection back to the residual width.
 * The two workloads are prefill over whole sequences and one autoregressive
 * decode step against a latent KV cache [GS-EN "1. Problem Statement"].
 *
 * Page tags: [ABS] mlsanity.com paper index, "Abstract (arXiv)"; [GS-EN]
 * gist.science English explainer of "Compressed Convolutional Attention:
 * Efficient Attention in a Compressed Latent Space"; [EDG]
 * blogs.edgentiq.com, "Boosting Transformer Efficiency with Compressed
 * Convolutional Attention".
 *
 * Readings where the pages leave a step open (they are the library's
 * definition of the operation):
 *   - convolution taps are indexed by lag: a[t,c] = sum_j w[c,j] u[t-j,c];
 *   - the channel convolution is one k_c-tap filter per head sliding along
 *     the head's channel index, zero padded inside the head;
 *   - q-k-mean adds the mean of the query and key values before and after
 *     the convolutions to the convolved q and k [GS-EN "2. Methodology" /
 *     Q-K-Mean; EDG "How Compressed Convolutional Attention Works"; GS-DE
 *     "2. Methodik"]: m = (q~ + k~ + b_q + b_k) / 4, q = b_q + m, k = b_k + m,
 *     with b the convolutions' output and ~ the down-projection's; for CCGQA
 *     query head h meets kv head h/G and kv head g the averages over its G
 *     query heads.  cca_config.qk_mean_mode selects the other reading, the
 *     mean of the pre-convolution values only;
 *   - value-shift: kv heads H_kv/2 .. H_kv-1 take the previous token's value
 *     (zero before the first token);
 *   - q and k are divided by max(||.||_2, norm_eps) per head; the logit of
 *     query head h is tau[h] * <q_h, k_g>;
 *   - RoPE rotates channel pairs (2i, 2i+1) by pos * base^(-2i/d), pos = token
 *     index from 0, angles evaluated in double precision.
 *
 * Conventions for every call
 *   - All tensor arguments are device pointers to caller-owned, contiguous,
 *     16-byte aligned memory.  The library never allocates device memory,
 *     never synchronises the stream and keeps no mutable global state; calls
 *     on different streams with distinct workspaces may run concurrently.
 *   - Every launch is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Argument errors are detected on the host before any
 *     launch and returned as a status; a failed launch returns CCA_ERR_HIP.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - No C++ exception crosses this interface.
 *   - Matrices are row-major [out, in].  Activations and weights use the
 *     storage type cfg.dtype (bf16 or fp32); taps and tau are always fp32.
 *     Accumulation is always fp32.
 */
#ifndef CCA_H
#define CCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CCA_OK = 0,
  CCA_ERR_INVALID_ARG = 1,   /* null pointer, inconsistent sizes, misaligned pointer */
  CCA_ERR_UNSUPPORTED = 2,   /* a legal configuration this build does not implement */
  CCA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the *_workspace_size */
  CCA_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} cca_status;

typedef enum { CCA_BF16 = 0, CCA_F32 = 1 } cca_dtype;

/* Reading of the channel convolution [GS-EN "2. Methodology" / Convolutional
 * Mixing: 1-D convolutions across the sequence and channel dimensions].
 * CCA_CHAN_PER_HEAD: one k_c-tap filter per head sliding along the head's
 *   channel index, b[t,h,i] = sum_j w[h,j] a[t,h,i-j] (the default).
 * CCA_CHAN_GROUPED: a k_c-lag causal convolution over tokens that mixes the
 *   d channels of each head densely, b[t,h,i] = sum_j sum_c W[h,i,j,c]
 *   a[t-j,h,c], a = 0 before the sequence start. */
typedef enum { CCA_CHAN_PER_HEAD = 0, CCA_CHAN_GROUPED = 1 } cca_chan_conv;

/* Reading of the q-k-mean [GS-EN "2. Methodology" / Q-K-Mean: q and k each
 * receive an average of the query and key values taken before and after the
 * convolutions].
 * CCA_QK_MEAN_PRE_POST: q += (q~ + b_q + k~ + b_k) / 4, k += (k~ + b_k +
 *   avg q~ + avg b_q) / 4 (avg over the kv head's G query heads) -- the
 *   default.
 * CCA_QK_MEAN_PRE: the pre-convolution values only, q += (q~ + k~) / 2,
 *   k += (k~ + avg q~) / 2. */
typedef enum { CCA_QK_MEAN_PRE_POST = 0, CCA_QK_MEAN_PRE = 1 } cca_qk_mean;

/* Prefill attention kernel.  Both compute the same values in the same
 * summation order; they differ in how the work maps onto the CU.
 * CCA_ATTN_FOUR_WAVE: 4 waves (128 query rows) per workgroup, 2 per CU.
 * CCA_ATTN_PING_PONG: 8 waves (256 query rows) per workgroup, 1 per CU, two
 *   halves alternating between the softmax and the matrix products; bf16
 *   with head_dim 64 only (other configurations use the four-wave kernel).
 * CCA_ATTN_AUTO takes the ping-pong kernel where it applies and its grid
 *   (one workgroup per CU) needs more than one round of the device's CUs,
 *   else the four-wave kernel. */
typedef enum { CCA_ATTN_AUTO = 0, CCA_ATTN_FOUR_WAVE = 1, CCA_ATTN_PING_PONG = 2 } cca_attn_kernel;

/* Shape and switches of one attention layer.  C (compression) and G are
 * derived: e_q = n_q_heads*head_dim, e_kv = n_kv_heads*head_dim,
 * G = n_q_heads / n_kv_heads. */
typedef struct {
  int32_t batch;          /* B  >= 1 */
  int32_t seq_len;        /* T  >= 1 (prefill); ignored by cca_decode_step */
  int32_t d_model;        /* E  >= 8, multiple of 8 */
  int32_t n_q_heads;      /* H_q, multiple of n_kv_heads */
  int32_t n_kv_heads;     /* H_kv >= 1; even when use_value_shift */
  int32_t head_dim;       /* d in {16, 32, 64, 128} */
  int32_t seq_conv_k;     /* k_s in 1..4 */
  int32_t chan_conv_k;    /* k_c in 1..4 */
  int32_t use_qk_mean;    /* 0 / 1 */
  int32_t use_value_shift;/* 0 / 1 */
  int32_t use_qk_norm;    /* 0 / 1 */
  float rope_base;        /* > 0, or 0 to switch RoPE off */
  float norm_eps;         /* > 0 (1e-6 by default) */
  int32_t dtype;          /* cca_dtype: storage of x, y, weights, cache, state */
  int32_t chan_conv_mode; /* cca_chan_conv; 0 (zero-initialised) is the per-head filter.
                           * CCA_CHAN_GROUPED needs d in {16, 32, 64}; the training and
                           * fused prefill entry points reject it (CCA_ERR_UNSUPPORTED) */
  int32_t qk_mean_mode;   /* cca_qk_mean; 0 (zero-initialised) is the pre- and
                           * post-convolution mean.  Only read when use_qk_mean is 1. */
  int32_t attn_kernel;    /* cca_attn_kernel; 0 (zero-initialised) is CCA_ATTN_AUTO */
} cca_config;

/* Weights.  w_qkv: [e_q + 2*e_kv, E] in cfg.dtype, rows q | k | v.
 * w_o: [E, e_q] in cfg.dtype (latent output flattened head-major, h*d+i).
 * q_seq_taps [e_q, k_s], k_seq_taps [e_kv, k_s]: fp32, lag-indexed.
 * q_chan_taps [H_q, k_c], k_chan_taps [H_kv, k_c]: fp32, lag-indexed (the
 *   per-head channel filter; unused under CCA_CHAN_GROUPED).
 * tau [H_q]: fp32 logit temperature per query head.
 * q_chan_dense [H_q, d, k_c, d], k_chan_dense [H_kv, d, k_c, d]: fp32, the
 *   grouped channel conv's W[h, i_out, lag, c_in], 16-byte aligned; read only
 *   under CCA_CHAN_GROUPED (NULL otherwise is fine).  bf16 configurations
 *   multiply them in fp16 (MFMA, fp32 accumulation). */
typedef struct {
  const void *w_qkv;
  const void *w_o;
  const float *q_seq_taps;
  const float *k_seq_taps;
  const float *q_chan_taps;
  const float *k_chan_taps;
  const float *tau;
  const float *q_chan_dense;
  const float *k_chan_dense;
} cca_weights;

/* Decode state, caller-owned, all in cfg.dtype.
 * k_cache, v_cache: [B, H_kv, capacity, d].  K holds the normalised, rotated
 *   k (tau not folded in); V the value after value-shift.
 * conv_q [B, W, e_q], conv_k [B, W, e_kv]: pre-convolution q~, k~ of the
 *   last W tokens, slot 0 the oldest; zeros stand for tokens before the
 *   sequence start.  W = k_s-1, or (k_s-1) + (k_c-1) under CCA_CHAN_GROUPED
 *   (its lagged inputs a[t-j] need the extra rows).
 * vshift [B, H_kv/2, d]: pre-shift value of the last token on the shifted
 *   (upper) kv heads; unused (may be NULL) when use_value_shift is 0. */
typedef struct {
  void *k_cache;
  void *v_cache;
  int32_t capacity;
  int32_t reserved;
  void *conv_q;
  void *conv_k;
  void *vshift;
} cca_state;

/* Host-only check of a configuration; needs no device.  Returns CCA_OK,
 * CCA_ERR_INVALID_ARG (null cfg, non-positive sizes, H_q % H_kv != 0, odd
 * H_kv with value-shift, E not a multiple of 8, bad eps/base) or
 * CCA_ERR_UNSUPPORTED (d outside {16,32,64,128}, fp32 prefill with d = 128,
 * taps outside 1..4, dtype, a kv group too wide for the mixing kernel).
 * A qk_mean_mode, chan_conv_mode or attn_kernel outside its enum is
 * CCA_ERR_INVALID_ARG. */
cca_status cca_validate_config(const cca_config *cfg);

/* Bytes of device workspace cca_prefill_forward needs for cfg (0 if cfg is
 * invalid).  Host-only. */
size_t cca_prefill_workspace_size(const cca_config *cfg);

/* Bytes of device workspace cca_decode_step needs for cfg and a cache of
 * cache_len past tokens (0 if invalid).  Host-only. */
size_t cca_decode_workspace_size(const cca_config *cfg, int32_t cache_len);

/* Prefill: the whole forward pass over x [B, T, E] -> y [B, T, E]
 * (x, y in cfg.dtype; they must not overlap): down-projection, the
 * convolutions, q-k-mean, value-shift, norm and RoPE in the latent space,
 * causal attention among the latent heads, up-projection [GS-EN "1. Problem
 * Statement" (training and prefill over whole sequences); GS-EN "2.
 * Methodology" (the steps)].
 * state_out (nullable): when given, also writes the decode state after the
 * T tokens: k_cache / v_cache slots [0, T) (capacity >= T), conv_q, conv_k
 * and (with value-shift) vshift.  Members left NULL are skipped.
 * workspace: >= cca_prefill_workspace_size(cfg) bytes, 256-byte aligned; its
 * contents are scratch and are overwritten. */
cca_status cca_prefill_forward(const cca_config *cfg, const cca_weights *w,
                               const void *x, void *y, const cca_state *state_out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* cca_prefill_forward with the down-projection and the mixing steps fused
 * into one kernel, so qkv~ stays on chip (the deeper fusion the pages' own
 * kernel uses [GS-EN "3. Key Contributions"]).  Same outputs up to fp32
 * rounding order; no decode state.  CCA_ERR_UNSUPPORTED unless cfg.dtype is
 * bf16, H_q == H_kv, head_dim == 64, seq_len is a multiple of 128 and
 * d_model a multiple of 32.  On MI355X it measures slower than the separate
 * kernels that cca_prefill_forward uses; it is kept for comparison.
 * workspace: >= cca_prefill_workspace_size(cfg) bytes. */
cca_status cca_prefill_forward_fused(const cca_config *cfg, const cca_weights *w, const void *x,
                                     void *y, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Decode step: one new token per sequence at position cache_len (uniform over
 * the batch).  x_t [B, E] -> y_t [B, E].  The new token's latent k and v join
 * the compressed cache, which its query heads attend over [GS-EN "1. Problem
 * Statement" (the cache read at every decoding step); GS-EN "2. Methodology"
 * / Extension: CCGQA (one compressed kv head per query group)].
 * state_in: cache slots [0, cache_len) and the carried conv window / vshift.
 *   The new k and v rows are written into state_in's cache at slot cache_len
 *   (capacity must exceed cache_len).
 * state_out: receives the rolled conv window and vshift; it may alias
 *   state_in.  Its k_cache / v_cache must be NULL or equal to state_in's.
 * workspace: >= cca_decode_workspace_size(cfg, cache_len) bytes. */
cca_status cca_decode_step(const cca_config *cfg, const cca_weights *w,
                           const void *x_t, int32_t cache_len,
                           const cca_state *state_in, const cca_state *state_out,
                           void *y_t, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Decode step with a cache length per sequence, for batches whose sequences
 * sit at different positions (continuous batching) [GS-EN "1. Problem
 * Statement": the decode-time cache grows per sequence].
 * cache_lens: device int32 [B]; sequence b's new token is at position
 *   cache_lens[b], attends to cache slots [0, cache_lens[b]] and is written
 *   at slot cache_lens[b].  Values are clamped to [0, max_cache_len].
 * max_cache_len: host bound on the lengths; it sizes the launch and the
 *   workspace (capacity must exceed it).  The key chunking follows it, so
 *   with every cache_lens[b] == max_cache_len the result equals
 *   cca_decode_step(..., max_cache_len, ...) bit for bit.
 * Everything else as cca_decode_step; workspace: >=
 * cca_decode_workspace_size(cfg, max_cache_len) bytes.  CCA_ERR_INVALID_ARG
 * for a null or misaligned cache_lens. */
cca_status cca_decode_step_varlen(const cca_config *cfg, const cca_weights *w,
                                  const void *x_t, const int32_t *cache_lens,
                                  int32_t max_cache_len, const cca_state *state_in,
                                  const cca_state *state_out, void *y_t, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Training: the forward pass keeping what its backward pass needs, and the
 * backward pass [GS-EN "3. Key Contributions": CCA speeds up training as
 * well as inference; the gradients are the derivative of the forward pass
 * defined above, step by step in reverse order].
 * ---------------------------------------------------------------------- */

/* Gradients of sum(dy * y) for one cca_prefill_forward_train call.  All are
 * written (overwritten, never accumulated) by cca_prefill_backward.
 * x: [B, T, E] in cfg.dtype.  w_qkv [e_q + 2*e_kv, E] and w_o [E, e_q]: fp32.
 * q_seq_taps [e_q, k_s], k_seq_taps [e_kv, k_s], q_chan_taps [H_q, k_c],
 * k_chan_taps [H_kv, k_c], tau [H_q]: fp32.  x, w_qkv and w_o 16-byte
 * aligned. */
typedef struct {
  void *x;
  float *w_qkv;
  float *w_o;
  float *q_seq_taps;
  float *k_seq_taps;
  float *q_chan_taps;
  float *k_chan_taps;
  float *tau;
} cca_grads;

/* Bytes of device workspace the two training calls need (0 if cfg is
 * invalid).  Its first cca_prefill_workspace_size(cfg) bytes have the
 * prefill layout.  Host-only. */
size_t cca_train_workspace_size(const cca_config *cfg);

/* Forward pass of a training step: y = the prefill of x, as
 * cca_prefill_forward (no decode state), and in the workspace the
 * activations the backward pass reads: the down-projection output, the
 * attention operands and output, and the log2 of every query's softmax
 * denominator.  workspace: >= cca_train_workspace_size(cfg) bytes,
 * 256-byte aligned. */
cca_status cca_prefill_forward_train(const cca_config *cfg, const cca_weights *w, const void *x,
                                     void *y, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Backward pass: given dy [B, T, E] (cfg.dtype), the cotangent of the y of
 * the cca_prefill_forward_train call that last wrote `workspace` with the
 * same cfg, w and x, writes every gradient of *g.  The workspace must hold
 * that call's activations (stream order; nothing else may write it in
 * between); its backward scratch is overwritten.  Argument errors as for
 * the forward; a null member of g is CCA_ERR_INVALID_ARG.  Deterministic:
 * no atomics, fixed summation orders. */
cca_status cca_prefill_backward(const cca_config *cfg, const cca_weights *w, const void *x,
                                const void *dy, const cca_grads *g, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Paged latent cache, for serving many sequences from one pool of pages
 * [GS-EN "1. Problem Statement": the cache grows per sequence; CCGQA keeps it
 * small, GS-EN "2. Methodology" / "Extension: CCGQA"].  Caller-owned.
 * k_pages, v_pages: [num_pages, H_kv, page_size, d] in cfg.dtype, 16-byte
 *   aligned; page p holds page_size consecutive tokens of one sequence.
 * block_table: device int32 [B, max_pages_per_seq]; entry [b, j] is the page
 *   that holds sequence b's tokens [j * page_size, (j + 1) * page_size).
 *   Entries outside [0, num_pages) are clamped (wrong rows, never a fault).
 * page_size: a multiple of 32.  conv_q, conv_k, vshift as in cca_state. */
typedef struct {
  void *k_pages;
  void *v_pages;
  const int32_t *block_table;
  int32_t num_pages;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t reserved;
  void *conv_q;
  void *conv_k;
  void *vshift;
} cca_paged_state;

/* cca_decode_step_varlen on a paged cache: sequence b's new token at
 * position cache_lens[b] attends to its rows [0, cache_lens[b]] found through
 * the block table, and its k, v rows are written into the page that holds
 * position cache_lens[b].  state_in and state_out share pages and table
 * (state_out's k_pages / v_pages / block_table must be NULL or equal);
 * conv_q / conv_k / vshift roll as in cca_decode_step.  With the same rows,
 * lengths and max_cache_len the result equals cca_decode_step_varlen on a
 * contiguous cache bit for bit.  CCA_ERR_INVALID_ARG when page_size is not a
 * positive multiple of 32, max_pages_per_seq * page_size <= max_cache_len,
 * num_pages < 1, or a pointer is null or misaligned. */
cca_status cca_decode_step_paged(const cca_config *cfg, const cca_weights *w, const void *x_t,
                                 const int32_t *cache_lens, int32_t max_cache_len,
                                 const cca_paged_state *state_in,
                                 const cca_paged_state *state_out, void *y_t, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* cca_prefill_forward writing its decode state into a paged cache: rows
 * [0, T) of every sequence go to the pages its block-table row names
 * (max_pages_per_seq * page_size >= T).  Members left NULL are skipped as in
 * cca_prefill_forward. */
cca_status cca_prefill_forward_paged(const cca_config *cfg, const cca_weights *w, const void *x,
                                     void *y, const cca_paged_state *state_out, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Several new tokens per sequence in one step (speculative verification,
 * chunked appends) [GS-EN "1. Problem Statement": autoregressive decode
 * against the cache].  x_new [B, n_new, E] -> y_new [B, n_new, E].
 * Sequence b's new tokens sit at positions cache_lens[b] .. cache_lens[b] +
 * n_new - 1: steps a1-a7 run over them with the carried window, their k and
 * v rows are written at those slots, new token j attends to keys
 * 0 .. cache_lens[b] + j, and the state rolls past the last one.  The result
 * equals n_new single-token steps.  cache_lens: device int32 [B], clamped to
 * [0, max_cache_len]; capacity must exceed max_cache_len + n_new - 1.
 * 1 <= n_new <= 16 (CCA_ERR_UNSUPPORTED beyond, or when the kv group's
 * mixing tile does not fit).  workspace: >=
 * cca_decode_multi_workspace_size(cfg, n_new, max_cache_len) bytes. */
size_t cca_decode_multi_workspace_size(const cca_config *cfg, int32_t n_new,
                                       int32_t max_cache_len);
cca_status cca_decode_multi(const cca_config *cfg, const cca_weights *w, const void *x_new,
                            int32_t n_new, const int32_t *cache_lens, int32_t max_cache_len,
                            const cca_state *state_in, const cca_state *state_out, void *y_new,
                            void *workspace, size_t workspace_bytes, void *stream);

/* cca_decode_multi on a paged cache (max_pages_per_seq * page_size >=
 * max_cache_len + n_new); as cca_decode_step_paged otherwise. */
cca_status cca_decode_multi_paged(const cca_config *cfg, const cca_weights *w, const void *x_new,
                                  int32_t n_new, const int32_t *cache_lens,
                                  int32_t max_cache_len, const cca_paged_state *state_in,
                                  const cca_paged_state *state_out, void *y_new, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* cca_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the step's workspace is a device array of
 * CCA_NOALLOC_SCRATCH bytes inside the library, one per GPU, held until the
 * process ends.  The call allocates nothing.  Its first call on a device
 * looks up that device's array (hipGetSymbolAddress, the device current).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, different threads) race and must be serialised by the
 * caller.  Arguments and results as cca_decode_step.  CCA_ERR_WORKSPACE,
 * before any launch, when cca_decode_workspace_size(cfg, cache_len) exceeds
 * CCA_NOALLOC_SCRATCH (the decode workload of 64 sequences, 16 query / 4 kv
 * heads of 64, E = 2048 and a 32768-token cache needs 7.8 MiB). */
#define CCA_NOALLOC_SCRATCH (16u << 20)
cca_status cca_decode_step_noalloc(const cca_config *cfg, const cca_weights *w, const void *x_t,
                                   int32_t cache_len, const cca_state *state_in,
                                   const cca_state *state_out, void *y_t, void *stream);

/* Static description of a status code. */
const char *cca_status_string(cca_status s);

/* ------------------------------------------------------------------------
 * Stage calls.  Each launches exactly the kernel(s) of one step of the
 * forward pass on the buffers of a prefill or decode workspace, so the steps
 * can be checked against the oracle's intermediates and timed one by one:
 * downproj [GS-EN "2. Methodology" / Down-Projection]; convmix
 * [/ Convolutional Mixing, / Q-K-Mean, / Value-Shift, / RoPE Integration];
 * attention [/ Latent Space Operations, / Extension: CCGQA]; upproj (the
 * projection back to the model width after the latent attention [/ Latent
 * Space Operations]).
 * cca_prefill_forward == downproj, convmix, attention, upproj in this order
 * on the same workspace; cca_decode_step == decode_downproj, decode_mix,
 * decode_attention, decode_upproj.
 *
 * Prefill workspace layout (offsets from cca_prefill_workspace_layout; Tp is
 * T rounded up to 128):
 *   CCA_WS_QKV  [B*T, e_q + 2*e_kv]   down-projection output: fp16 when
 *               cfg.dtype is bf16 (10 mantissa bits; |values| above 65504
 *               overflow), fp32 when it is fp32
 *   CCA_WS_Q    [B, H_q, Tp, d]   normalised, rotated q times tau_h*log2(e)
 *               (logits in the exp2 domain); fp16 when cfg.dtype is bf16 and
 *               use_qk_norm is 1, else cfg.dtype
 *   CCA_WS_K    [B, H_kv, Tp, d]  same type as CCA_WS_Q
 *   CCA_WS_VT   [B, H_kv, d, Tp]  value after shift, transposed, cfg.dtype;
 *               inside each group of 16 tokens, positions 4..7 and 8..11 are
 *               swapped (bits 2 and 3 of the token index exchanged)
 *   CCA_WS_O    [B*T, e_q] latent attention output, cfg.dtype
 *   CCA_WS_PART scratch of cca_prefill_forward_fused (the 3 rows before each
 *               128-token tile), for the shapes it takes; under
 *               CCA_CHAN_GROUPED fp32 [B*T, e_q + e_kv], the channel conv's
 *               output (q heads, then k heads)
 * Decode workspace layout:
 *   CCA_WS_QKV  fp32 [B, e_q + 2*e_kv]
 *   CCA_WS_Q    fp32 [B, H_q, d]  normalised, rotated q of the new token
 *   CCA_WS_PART fp32 partial softmax states of the split-KV attention
 *   CCA_WS_O    [B, e_q] cfg.dtype
 *   CCA_WS_SPLITK fp32 partial sums of the two projections, whose contraction
 *               is split over workgroups when B <= 64
 * ---------------------------------------------------------------------- */
enum { CCA_WS_QKV = 0, CCA_WS_Q = 1, CCA_WS_K = 2, CCA_WS_VT = 3, CCA_WS_O = 4,
       CCA_WS_PART = 5, CCA_WS_SPLITK = 6, CCA_WS_COUNT = 7 };

/* Byte offsets of the buffers above (the intermediates between the steps of
 * GS-EN "2. Methodology") inside a prefill (decode: cache_len >= 0)
 * workspace; unused slots are set to SIZE_MAX.  Returns the status
 * cca_validate_config gives an invalid cfg, CCA_ERR_INVALID_ARG for a NULL
 * offsets or a negative cache_len.  Host-only. */
cca_status cca_prefill_workspace_layout(const cca_config *cfg, size_t offsets[CCA_WS_COUNT]);
cca_status cca_decode_workspace_layout(const cca_config *cfg, int32_t cache_len,
                                       size_t offsets[CCA_WS_COUNT]);

cca_status cca_stage_downproj(const cca_config *cfg, const cca_weights *w, const void *x,
                              void *workspace, size_t workspace_bytes, void *stream);
cca_status cca_stage_convmix(const cca_config *cfg, const cca_weights *w,
                             const cca_state *state_out, void *workspace,
                             size_t workspace_bytes, void *stream);
cca_status cca_stage_attention(const cca_config *cfg, const cca_weights *w,
                               void *workspace, size_t workspace_bytes, void *stream);
cca_status cca_stage_upproj(const cca_config *cfg, const cca_weights *w, void *y,
                            void *workspace, size_t workspace_bytes, void *stream);

cca_status cca_stage_decode_downproj(const cca_config *cfg, const cca_weights *w,
                                     const void *x_t, int32_t cache_len, void *workspace,
                                     size_t workspace_bytes, void *stream);
cca_status cca_stage_decode_mix(const cca_config *cfg, const cca_weights *w, int32_t cache_len,
                                const cca_state *state_in, const cca_state *state_out,
                                void *workspace, size_t workspace_bytes, void *stream);
cca_status cca_stage_decode_attention(const cca_config *cfg, const cca_weights *w,
                                      int32_t cache_len, const cca_state *state_in,
                                      void *workspace, size_t workspace_bytes, void *stream);
cca_status cca_stage_decode_upproj(const cca_config *cfg, const cca_weights *w,
                                   int32_t cache_len, void *y_t, void *workspace,
                                   size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CCA_H */
