// Fused latent mixing of the CCA forward pass (gfx950), memory bound.
//
// For every token and latent head, from the down-projection output:
//   a2 causal sequence conv, depthwise, lag-indexed k_s taps per channel
//   a3 channel conv: one k_c-tap filter per head sliding along the channel
//      index, zero padded inside the head
//      [GS-EN "2. Methodology" / Convolutional Mixing]
//   a4 q-k-mean: the mean of the query and key values before and after the
//      convolutions is added to the convolved q and k,
//        m = (q~ + k~ + b_q + b_k) / 4,  q = b_q + m,  k = b_k + m
//      (mean mode 2, the default), or the mean of the pre-convolution values
//      only, (q~ + k~) / 2 (mean mode 1).  With G query heads per kv head,
//      query head h meets its group's key head, and the key head meets the
//      average over the group's query heads
//      [GS-EN "2. Methodology" / Q-K-Mean; EDG "How Compressed Convolutional
//       Attention Works"; GS-DE "2. Methodik"]
//   a5 value-shift: the upper half of the kv heads take the previous token's
//      value [GS-EN "2. Methodology" / Value-Shift]
//   a6 L2 normalisation per head, x / max(||x||, eps)
//   a7 RoPE, pairs (2i, 2i+1), angle pos * base^(-2i/d) evaluated in double
//      and reduced modulo 2*pi before the fp32 sin/cos
//      [GS-EN "2. Methodology" / RoPE Integration]
//
// Work split (prefill): one workgroup per (batch b, kv group g, chunk of TC
// tokens).  The group's pre-conv columns (G query heads, its key head, its
// value head) for tokens t0-3 .. t0+TC-1 move HBM -> LDS by LDS-DMA in the
// type the down-projection wrote (fp16 in bf16 mode), together with the
// group's taps; the 3-token halo of the causal window comes along.  A lane group of d/4 lanes takes one token row and walks every head
// slot of the group, 4 channels per lane: the channel convolution is three
// lane shifts, RoPE pairs stay inside a lane, the L2 norm is a reduction over
// the d/4 lanes, and the q-k-mean finds the pre- and post-convolution values
// of the other heads of its group in its own registers (key head first, then
// the query heads with a running sum for the key head's mean).  The value
// head is written transposed (d-major) for the attention kernel, straight
// from the LDS tile.
#include "cca_device.h"
#include "gemm_tile.h"
#include "cca_launch.h"

namespace cca {

static constexpr int HALO = 3;   // k_s - 1 for the largest supported k_s = 4

template <typename T> struct Store4;
template <> struct Store4<float> {
  __device__ __forceinline__ static void st(float *p, const float *v) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
};
template <> struct Store4<f16> {
  // the values are rounded to fp32 first, then to fp16: the empty asm keeps
  // the compiler from folding the conversion into the producing fma (one
  // rounding instead of two), which it does in some instantiations and not in
  // others, so every kernel writes the same bits
  __device__ __forceinline__ static void st(f16 *p, const float *v) {
    float a = v[0], b = v[1], c = v[2], d = v[3];
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
    *reinterpret_cast<f16x4 *>(p) = f16x4{(f16)a, (f16)b, (f16)c, (f16)d};
  }
};
template <> struct Store4<bf16> {
  __device__ __forceinline__ static void st(bf16 *p, const float *v) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  }
};

// a6 and a7 on this lane's 4 channels of one head: sc * b / max(||b||, eps)
// over the d/4 lanes of the head (sc * b without the norm), then the rotation
// of the pairs (4li, 4li+1) and (4li+2, 4li+3) by (cos, sin) = cs0, cs1.  sc
// carries an output scale into the normalisation's factor (1 for none).
template <int D>
__device__ __forceinline__ void norm_rope(const MixShape &s, float2 cs0, float2 cs1, float sc,
                                          float (&b)[4], float y[4]) {
  constexpr int LPU = D / 4;
  float f = sc;
  if (s.use_norm) {
    // 1 / max(||b||, eps) == rsqrt(max(||b||^2, eps^2))
    const float ss = group_sum<LPU>(b[0] * b[0] + b[1] * b[1] + b[2] * b[2] + b[3] * b[3]);
    f *= __builtin_amdgcn_rsqf(fmaxf(ss, s.eps * s.eps));
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) b[c] *= f;
  y[0] = b[0] * cs0.x - b[1] * cs0.y;
  y[1] = b[0] * cs0.y + b[1] * cs0.x;
  y[2] = b[2] * cs1.x - b[3] * cs1.y;
  y[3] = b[2] * cs1.y + b[3] * cs1.x;
}

// a2 and a3 of one head slot at one token: `tile` rows are tokens (row `row`
// the current one, the rows above it the earlier ones), columns [q heads | k
// head | v head] of the group, CW elements wide; slot 0..G-1 are the query
// heads, slot G the key head.  staps [(G+1) d][4] and ctaps [G+1][4] hold the
// group's taps (zero past k_s / k_c).  The lane holds channels 4li .. 4li+3.
template <int D, typename TT>
__device__ __forceinline__ void conv_slot(const TT *tile, int CW, int row, int slot, int li,
                                          const float *staps, const float *ctaps, float (&b)[4],
                                          f32x4 &pre) {
  constexpr int LPU = D / 4;
  const int col = slot * D + 4 * li;
  f32x4 u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = ld4f<TT>(tile + (row - j) * CW + col);
  pre = u[0];
  float a[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(staps + (col + c) * 4);
    float acc = t[0] * u[0][c];
#pragma unroll
    for (int j = 1; j < 4; ++j) acc = fmaf(t[j], u[j][c], acc);
    a[c] = acc;
  }
  // values of the three channels below this lane's first one (previous lane;
  // zero for the head's first lane)
  float p1, p2, p3;
  if constexpr (LPU <= 16) {
    p1 = dpp_shr1(a[1]);
    p2 = dpp_shr1(a[2]);
    p3 = dpp_shr1(a[3]);
  } else {
    p1 = __shfl_up(a[1], 1, LPU);
    p2 = __shfl_up(a[2], 1, LPU);
    p3 = __shfl_up(a[3], 1, LPU);
  }
  // with 16 lanes per head the DPP row is the head: its lane 0 already reads 0
  if (LPU != 16 && li == 0) p1 = p2 = p3 = 0.f;
  const f32x4 w = *reinterpret_cast<const f32x4 *>(ctaps + slot * 4);
  b[0] = w[0] * a[0] + w[1] * p3 + w[2] * p2 + w[3] * p1;
  b[1] = w[0] * a[1] + w[1] * a[0] + w[2] * p3 + w[3] * p2;
  b[2] = w[0] * a[2] + w[1] * a[1] + w[2] * a[0] + w[3] * p3;
  b[3] = w[0] * a[3] + w[1] * a[2] + w[2] * a[1] + w[3] * a[0];
}

// a4, a6, a7 for every head slot of one kv group at one token, this lane's 4
// channels: the key head (slot G) first, then the G query heads.
//   conv(slot, b, p)  the slot's channel-conv output b and its
//                     pre-convolution values p (f32x4)
//   emit(slot, y)     receives the normalised, rotated result
//   scale(slot)       a factor applied to the slot's output (see norm_rope)
// s.use_mean: 0 off; 1 q += (q~ + k~)/2, k += (k~ + avg q~)/2; 2 q += (q~ + b_q
// + k~ + b_k)/4, k += (k~ + b_k + avg q~ + avg b_q)/4.
template <int D, typename ConvFn, typename EmitFn, typename ScaleFn>
__device__ __forceinline__ void mix_row(int G, const MixShape &s, float2 cs0, float2 cs1,
                                        ConvFn &&conv, EmitFn &&emit, ScaleFn &&scale) {
  const bool mean = s.use_mean != 0, post = s.use_mean == 2;
  const float coef = post ? 0.25f : 0.5f;
  float bk[4];
  f32x4 kp;
  conv(G, bk, kp);
  float sk[4] = {0.f, 0.f, 0.f, 0.f}, sq[4] = {0.f, 0.f, 0.f, 0.f};
  if (mean) {
#pragma unroll
    for (int c = 0; c < 4; ++c) sk[c] = post ? kp[c] + bk[c] : kp[c];
  }
  for (int h = 0; h < G; ++h) {
    float b[4];
    f32x4 qp;
    conv(h, b, qp);
    if (mean) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float own = post ? qp[c] + b[c] : qp[c];
        sq[c] += own;
        b[c] += coef * (own + sk[c]);
      }
    }
    float y[4];
    norm_rope<D>(s, cs0, cs1, scale(h), b, y);
    emit(h, y);
  }
  if (mean) {
    const float invg = 1.f / (float)G;
#pragma unroll
    for (int c = 0; c < 4; ++c) bk[c] += coef * (sk[c] + sq[c] * invg);
  }
  float y[4];
  norm_rope<D>(s, cs0, cs1, scale(G), bk, y);
  emit(G, y);
}

// Group taps into LDS: seq taps [(G+1)*D][4] (q channels, then k), channel
// taps [(G+1)][4], taps beyond k_s / k_c zero; tsc [G] = tau_h * log2(e) of
// the group's query heads (the attention kernel takes exp2-domain logits).
template <int D>
__device__ __forceinline__ void load_taps(const MixShape &s, const MixTaps &w, int g, float *staps,
                                          float *ctaps, float *tsc) {
  const int G = s.G;
  for (int c = threadIdx.x; c < (G + 1) * D; c += blockDim.x) {
    const float *src = c < G * D ? w.q_seq + (size_t)(g * G * D + c) * s.ks
                                 : w.k_seq + (size_t)(g * D + c - G * D) * s.ks;
#pragma unroll
    for (int j = 0; j < 4; ++j) staps[c * 4 + j] = j < s.ks ? src[j] : 0.f;
  }
  for (int c = threadIdx.x; c < G + 1; c += blockDim.x) {
    const float *src = c < G ? w.q_chan + (size_t)(g * G + c) * s.kc : w.k_chan + (size_t)g * s.kc;
#pragma unroll
    for (int j = 0; j < 4; ++j) ctaps[c * 4 + j] = j < s.kc ? src[j] : 0.f;
  }
  for (int h = threadIdx.x; h < G; h += blockDim.x) tsc[h] = w.tau[g * G + h] * 1.4426950408889634f;
}

// The group's taps and tau scales held in registers between their loads and
// their LDS stores (the layout of load_taps), so that the loads can be
// issued before other work: thread t owns seq-tap channels t + 256 i
// ((G + 1) d < 1024 when (G + 2) d / 4 <= 256, which the host checks;
// zero-padded past k_s), channel-tap / tau slot t.
template <int D> struct TapRegs {
  static constexpr int NS = 4;
  f32x4 sq[NS];
  f32x4 ch;
  float tau;
  __device__ __forceinline__ void load(const MixShape &s, const MixTaps &w, int g) {
    const int G = s.G, t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = t + 256 * i;
      sq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c < (G + 1) * D) {
        const float *src = c < G * D ? w.q_seq + (size_t)(g * G * D + c) * s.ks
                                     : w.k_seq + (size_t)(g * D + c - G * D) * s.ks;
#pragma unroll
        for (int j = 0; j < 4; ++j) sq[i][j] = j < s.ks ? src[j] : 0.f;
      }
    }
    ch = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < G + 1) {
      const float *src = t < G ? w.q_chan + (size_t)(g * G + t) * s.kc : w.k_chan + (size_t)g * s.kc;
#pragma unroll
      for (int j = 0; j < 4; ++j) ch[j] = j < s.kc ? src[j] : 0.f;
    }
    tau = t < G ? w.tau[g * G + t] * 1.4426950408889634f : 0.f;
  }
  __device__ __forceinline__ void store(const MixShape &s, float *staps, float *ctaps, float *tsc) const {
    const int G = s.G, t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (t + 256 * i < (G + 1) * D) *reinterpret_cast<f32x4 *>(staps + (t + 256 * i) * 4) = sq[i];
    if (t < G + 1) *reinterpret_cast<f32x4 *>(ctaps + t * 4) = ch;
    if (t < G) tsc[t] = tau;
  }
};

// Floats of the tap area after the tile: seq taps, channel taps, tau scales.
__host__ __device__ inline int taps_floats(int G, int D) {
  return (G + 1) * D * 4 + (G + 1) * 4 + (G + 3) / 4 * 4;
}

// Element i of a decode step's down-projection output (see DecQkv).
// The slices are summed in order; their loads go out four at a time.
__device__ __forceinline__ float dec_qkv(const DecQkv &d, size_t i, size_t mn) {
  if (d.slices == 0) return d.qkv[i];
  const float *p = d.parts + i;
  float acc = p[0];
  int sl = 1;
  for (; sl + 4 <= d.slices; sl += 4) {
    const float a0 = p[sl * mn], a1 = p[(sl + 1) * mn], a2 = p[(sl + 2) * mn], a3 = p[(sl + 3) * mn];
    acc += a0;
    acc += a1;
    acc += a2;
    acc += a3;
  }
  for (; sl < d.slices; ++sl) acc += p[sl * mn];
  return acc;
}

// Map a column of the group tile to its column in the qkv row.
__device__ __forceinline__ int group_col(int col, int g, int G, int D, int eq, int ekv) {
  if (col < G * D) return g * G * D + col;
  if (col < (G + 1) * D) return eq + g * D + (col - G * D);
  return eq + ekv + g * D + (col - (G + 1) * D);
}

// Bytes of a tile of `rows` token rows of one group (16-byte multiple).
__host__ __device__ inline size_t tile_bytes(int rows, int G, int D, int es) {
  return ((size_t)rows * (G + 2) * D * es + 15) / 16 * 16;
}

// MEAN: the q-k-mean mode (s.use_mean: 0 off, 1 pre-conv, 2 pre- and
// post-conv); R1B: the channel conv's output comes from r1b (the grouped
// reading) instead of the two convolutions; OUT: some of the cache, the
// conv window, vshift or bout is written (without it none of that code is
// in the kernel).
template <typename TI, typename TQ, typename TV, int D, int MEAN, bool R1B, bool OUT>
__global__ __launch_bounds__(256) void convmix_prefill_kernel(MixShape s, MixTaps w,
                                                              const TI *__restrict__ qkv,
                                                              TQ *__restrict__ q, TQ *__restrict__ k,
                                                              TV *__restrict__ vt, StateOut st,
                                                              const float *__restrict__ r1b,
                                                              float *__restrict__ bout, int TC) {
  extern __shared__ __attribute__((aligned(16))) unsigned char mix_smem[];
  const int G = s.G, CW = (G + 2) * D;
  // LDS: the tile (rows: tokens t0-HALO .. t0+TC-1), then the group's seq
  // taps [(G+1) D][4], channel taps [G+1][4], tau [G] (rounded up to 4
  // floats) and the RoPE frequencies [D/2] (double)
  TI *tile = reinterpret_cast<TI *>(mix_smem);
  float *staps = reinterpret_cast<float *>(mix_smem + tile_bytes(TC + HALO, G, D, sizeof(TI)));
  float *ctaps = staps + (G + 1) * D * 4;
  float *ltau = ctaps + (G + 1) * 4;
  double *lth = reinterpret_cast<double *>(ltau + (G + 3) / 4 * 4);

  const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const int nchunks = s.Tp / TC;
  // consecutive chunks of a (b, g) on one XCD: the halo rows and the value
  // tile's partial lines meet in one L2
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int chunk = lid % nchunks, bg = lid / nchunks;
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int t0 = chunk * TC;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int shifted = (s.use_shift && g >= s.Hkv / 2) ? 1 : 0;
  const int vcol = (G + 1) * D;
  const TI *src = qkv + (size_t)b * s.T * N;

  // Everything the mixing reads reaches LDS by LDS-DMA, with no register
  // staging: the taps and tau, then the tile.  Out-of-range offsets (taps
  // past k_s / k_c, tokens outside [0, T)) land as zeros.
  {
    const int ks = s.ks, kc = s.kc;
    const unsigned qb = (unsigned)(G * D * ks * 4), kb = (unsigned)(D * ks * 4);
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void *)(w.q_seq + (size_t)g * G * D * ks), 0, qb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void *)(w.k_seq + (size_t)g * D * ks), 0, kb, 0x00020000);
    const int nq = G * D / 16, nk = D / 16;               // 64-float instructions ([c][4] rows)
    for (int i = wv; i < nq + nk; i += 4) {
      const bool isq = i < nq;
      const int f = (isq ? i : i - nq) * 64 + lane, c = f >> 2, j = f & 3;
      const unsigned off = j < ks ? (unsigned)((c * ks + j) * 4) : (isq ? qb : kb);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isq ? rq : rk, as_lds(staps + i * 64), 4, (int)off, 0, 0, 0);
    }
    if (wv == 3) {
      const unsigned cqb = (unsigned)(G * kc * 4), ckb = (unsigned)(kc * 4), tb = (unsigned)(G * 4);
      const __amdgpu_buffer_rsrc_t rcq =
          __builtin_amdgcn_make_buffer_rsrc((void *)(w.q_chan + (size_t)g * G * kc), 0, cqb, 0x00020000);
      const __amdgpu_buffer_rsrc_t rck =
          __builtin_amdgcn_make_buffer_rsrc((void *)(w.k_chan + (size_t)g * kc), 0, ckb, 0x00020000);
      const __amdgpu_buffer_rsrc_t rt =
          __builtin_amdgcn_make_buffer_rsrc((void *)(w.tau + (size_t)g * G), 0, tb, 0x00020000);
      const int c = lane >> 2, j = lane & 3;
      if (lane < G * 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rcq, as_lds(ctaps), 4,
                                                 j < kc ? (int)((c * kc + j) * 4) : (int)cqb, 0, 0, 0);
      if (lane < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rck, as_lds(ctaps + G * 4), 4,
                                                 j < kc ? (int)(j * 4) : (int)ckb, 0, 0, 0);
      if (lane < G)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, as_lds(ltau), 4, lane * 4, 0, 0, 0);
    }
  }
  // the tile: row-major [TC + HALO][CW] without padding.  It arrives in
  // steps of srows token rows (upp, the rows the lane groups take in one pass
  // of the row loop, when the chunk holds four or more such passes): the
  // halo and the first step's rows before the loop, then the next step's
  // rows while this step's are mixed, so with the input in HBM the rows of
  // the first step start before the rest of the tile has arrived (a 64-token
  // chunk at G = 1: 16.3 against 17.8 us for one wait at B = 4, T = 2048; in
  // the two-step case of 32-token chunks the extra barrier cost as much as it
  // saved).
  // issue_rows(rlo, rhi) moves tile rows [rlo, rhi): 16-byte chunk c of the
  // tile (row c / cpr) goes to LDS byte 16 c; instruction i of the range
  // starts at its chunk c_lo + 64 i, lane l moves chunk c_lo + 64 i + l (lanes
  // past the range stay idle), and instruction i goes out from wave i % 4.
  constexpr int LPU = D / 4;
  const int upp = 256 / LPU;
  const int li = tid % LPU, ui = tid / LPU;
  constexpr int EPC = 16 / (int)sizeof(TI);
  const int cpr = CW / EPC;
  const int tlo = max(t0 - HALO, 0), thi = min(t0 + TC, s.T);
  const unsigned nbytes = thi > tlo ? (unsigned)((size_t)(thi - tlo) * N * sizeof(TI)) : 0u;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(src + (size_t)tlo * N), 0, nbytes, 0x00020000);
  auto issue_rows = [&](int rlo, int rhi) {
    const int c_lo = rlo * cpr, c_hi = rhi * cpr;
    for (int i = wv; c_lo + i * 64 < c_hi; i += 4) {
      const int c = c_lo + i * 64 + lane;
      const int row = c / cpr, tok = t0 - HALO + row;
      const unsigned off =
          tok >= tlo && tok < thi
              ? (unsigned)(((size_t)(tok - tlo) * N + group_col((c - row * cpr) * EPC, g, G, D, eq, ekv)) *
                           sizeof(TI))
              : nbytes;
      if (c < c_hi)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, as_lds(mix_smem + (size_t)(c_lo + i * 64) * 16), 16,
                                                 (int)off, 0, 0, 0);
    }
  };
  // steps of upp rows when a chunk holds at least four of them, else the
  // whole chunk at once (always under the grouped channel conv, whose rows
  // also read the MFMA kernel's output)
  const int srows = !R1B && TC >= 4 * upp ? upp : TC;
  issue_rows(0, min(HALO + srows, TC + HALO));
  // the RoPE frequencies come from the kernel arguments (scalar loads)
  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < D / 2; ++i) lth[i] = s.theta[i];
  }
  wait_vmcnt<0>();
  lds_barrier();
  const double th0 = lth[2 * li], th1 = lth[2 * li + 1];

  // one token row per lane group, every head slot of the group
  MixShape sm = s;
  sm.use_mean = MEAN;
  // per-lane bases: row r of this chunk adds r * D to the q / k offsets
  TQ *qlane = q + ((size_t)(b * s.Hq + g * G) * s.Tp + t0) * D + 4 * li;
  TQ *klane = k + ((size_t)(b * s.Hkv + g) * s.Tp + t0) * D + 4 * li;
  const size_t qhead = (size_t)s.Tp * D;               // between the group's query heads
  TV *kcache = OUT ? reinterpret_cast<TV *>(st.k_cache) : nullptr;
  float *blane = OUT && bout ? bout + (size_t)b * s.T * (eq + ekv) + 4 * li : nullptr;
  for (int r0 = 0; r0 < TC; r0 += srows) {
    if (r0 > 0) {
      wait_vmcnt<0>();
      lds_barrier();
    }
    if (r0 + srows < TC) issue_rows(HALO + r0 + srows, min(HALO + r0 + 2 * srows, TC + HALO));
    const int rend = min(r0 + srows, TC);
    for (int r = r0 + ui; r < rend; r += upp) {
      const int tok = t0 + r;
      const float2 cs0 = rope_cs_theta(tok, th0, s.rope_base);
      const float2 cs1 = rope_cs_theta(tok, th1, s.rope_base);
      const TI *cur = tile + (r + HALO) * CW + 4 * li;
      // q leaves scaled by tau_h * log2(e); rows past the sequence's end are
      // zero: both factors ride on the normalisation's
      const bool live = tok < s.T;
      auto scale = [&](int slot) __attribute__((always_inline)) {
        return live ? (slot < G ? ltau[slot] * 1.4426950408889634f : 1.f) : 0.f;
      };
      auto emit = [&](int slot, float *y) __attribute__((always_inline)) {
        if (slot < G) {
          Store4<TQ>::st(qlane + slot * qhead + r * D, y);
        } else {
          Store4<TQ>::st(klane + r * D, y);
          if constexpr (OUT) {
            size_t row;
            if (kcache && tok < s.T && cache_row_store(st, b, s.Hkv, g, tok, &row))
              Store4<TV>::st(kcache + row * D + 4 * li, y);
          }
        }
      };
      if constexpr (R1B) {
        // grouped channel conv: b comes from the MFMA kernel's output rows
        const float *brow = r1b + (size_t)(b * s.T + min(tok, s.T - 1)) * (eq + ekv) + 4 * li;
        auto conv = [&](int slot, float (&bb)[4], f32x4 &pre) __attribute__((always_inline)) {
          const f32x4 v = tok < s.T ? *reinterpret_cast<const f32x4 *>(
                                          brow + (slot < G ? (g * G + slot) * D : eq + g * D))
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int c = 0; c < 4; ++c) bb[c] = v[c];
          pre = ld4f<TI>(cur + slot * D);
        };
        mix_row<D>(G, sm, cs0, cs1, conv, emit, scale);
      } else {
        auto conv = [&](int slot, float (&bb)[4], f32x4 &pre) __attribute__((always_inline)) {
          conv_slot<D, TI>(tile, CW, r + HALO, slot, li, staps, ctaps, bb, pre);
          if (OUT && blane && tok < s.T)
            *reinterpret_cast<f32x4 *>(blane + (size_t)tok * (eq + ekv) +
                                       (slot < G ? (g * G + slot) * D : eq + g * D)) =
                f32x4{bb[0], bb[1], bb[2], bb[3]};
        };
        mix_row<D>(G, sm, cs0, cs1, conv, emit, scale);
      }
    }
  }

  // value head, transposed: vt[b, g, dd, p] holds token vt_perm(p) of the
  // chunk.  A thread takes 4 channels at the 8 positions 8 grp .. 8 grp + 7,
  // i.e. tokens tb + {0, 1, 2, 3, 8, 9, 10, 11} with tb = 16 (grp >> 1) +
  // 4 (grp & 1): 8 LDS reads of 4 elements at fixed row strides, every row
  // inside the tile.  Only the chunk holding the sequence's end zeroes the
  // positions past it.
  auto write_vt = [&](auto tail) {
    const int rb = CW * (int)sizeof(TI);
    for (int e = tid; e < (D / 4) * (TC / 8); e += 256) {
      const int d4 = e / (TC / 8), grp = e % (TC / 8);
      const int tb = 16 * (grp >> 1) + 4 * (grp & 1);
      const unsigned char *base = reinterpret_cast<const unsigned char *>(tile) +
                                  (tb + HALO - shifted) * rb + (vcol + 4 * d4) * (int)sizeof(TI);
      float vals[4][8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int dt = jj < 4 ? jj : jj + 4;
        f32x4 v = ld4f<TI>(reinterpret_cast<const TI *>(base + dt * rb));
        if constexpr (decltype(tail)::value)
          if (t0 + tb + dt >= s.T) v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) vals[c][jj] = v[c];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        TV *dst = vt + ((size_t)(b * s.Hkv + g) * D + 4 * d4 + c) * s.Tp + t0 + 8 * grp;
        Store4<TV>::st(dst, vals[c]);
        Store4<TV>::st(dst + 4, vals[c] + 4);
      }
    }
  };
  if (t0 + TC > s.T) write_vt(std::true_type{});
  else write_vt(std::false_type{});
  if (OUT && st.v_cache) {
    for (int e = tid; e < TC * (D / 4); e += 256) {
      const int r = e / (D / 4), c4 = e % (D / 4), tok = t0 + r;
      if (tok >= s.T) continue;
      size_t row;
      if (!cache_row_store(st, b, s.Hkv, g, tok, &row)) continue;
      const f32x4 v = ld4f<TI>(tile + (r + HALO - shifted) * CW + vcol + 4 * c4);
      const float vv[4] = {v[0], v[1], v[2], v[3]};
      Store4<TV>::st(reinterpret_cast<TV *>(st.v_cache) + row * D + 4 * c4, vv);
    }
  }

  // decode state after the last token: conv window (k_s - 1 pre-conv rows,
  // plus k_c - 1 under the grouped channel conv) and value-shift state
  if (OUT && chunk == 0) {
    const int ks1 = s.ks - 1 + (s.grouped ? s.kc - 1 : 0);
    if (st.conv_q)
      for (int e = tid; e < ks1 * G * D; e += 256) {
        const int sl = e / (G * D), c = e % (G * D), tok = s.T - ks1 + sl;
        const float v = tok >= 0 ? to_f32(src[(size_t)tok * N + g * G * D + c]) : 0.f;
        reinterpret_cast<TV *>(st.conv_q)[(size_t)(b * ks1 + sl) * eq + g * G * D + c] = from_f32<TV>(v);
      }
    if (st.conv_k)
      for (int e = tid; e < ks1 * D; e += 256) {
        const int sl = e / D, c = e % D, tok = s.T - ks1 + sl;
        const float v = tok >= 0 ? to_f32(src[(size_t)tok * N + eq + g * D + c]) : 0.f;
        reinterpret_cast<TV *>(st.conv_k)[(size_t)(b * ks1 + sl) * ekv + g * D + c] = from_f32<TV>(v);
      }
    if (st.vshift && shifted)
      for (int c = tid; c < D; c += 256)
        reinterpret_cast<TV *>(st.vshift)[(size_t)(b * (s.Hkv / 2) + g - s.Hkv / 2) * D + c] =
            from_f32<TV>(to_f32(src[(size_t)(s.T - 1) * N + eq + ekv + g * D + c]));
  }
}

// m = s.T new tokens per sequence at positions L .. L+m-1 (L = lens[b] when
// lens is given, clamped to [0, L]).  One workgroup per (b, g); the fp32 tile
// holds tokens L-3 .. L+m-1: three rows from the carried window, then the m
// new rows from the down-projection.  All state reads finish before the
// barrier, so state_out may alias state_in.
template <typename TV, int D>
__global__ __launch_bounds__(256) void convmix_decode_kernel(MixShape s, MixTaps w,
                                                             DecQkv qkv, int Lmax,
                                                             const int *__restrict__ lens,
                                                             StateOut in, StateOut out,
                                                             float *__restrict__ qout) {
  extern __shared__ __attribute__((aligned(16))) unsigned char mix_smem[];
  const int G = s.G, CW = (G + 2) * D;
  const int m = s.T, R = 3 + m;
  float *tile = reinterpret_cast<float *>(mix_smem);    // R rows
  float *staps = reinterpret_cast<float *>(mix_smem + tile_bytes(R, G, D, 4));
  float *ctaps = staps + (G + 1) * D * 4;
  float *tsc = ctaps + (G + 1) * 4;

  const int tid = threadIdx.x;
  const int g = blockIdx.x % s.Hkv, b = blockIdx.x / s.Hkv;
  const int L = lens ? min(max(lens[b], 0), Lmax) : Lmax;   // this sequence's position
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int ks1 = s.ks - 1;
  const int shifted = (s.use_shift && g >= s.Hkv / 2) ? 1 : 0;
  const TV *cq = reinterpret_cast<const TV *>(in.conv_q);
  const TV *ck = reinterpret_cast<const TV *>(in.conv_k);
  const TV *vs = reinterpret_cast<const TV *>(in.vshift);
  // taps, tau and this lane's RoPE frequencies first: their latency overlaps the tile's
  TapRegs<D> tr;
  tr.load(s, w, g);
  constexpr int LPU = D / 4;
  const int li = tid % LPU, ui = tid / LPU;
  const double th0 = s.theta[2 * li], th1 = s.theta[2 * li + 1];

  // the tile: the three carried rows, then the m new rows (the down-
  // projection output, or the sum of its split-contraction slices in slice
  // order).  Each pass issues every load of LB carried and NU new elements
  // per thread before the first LDS store: one pass at the decode shapes.
  constexpr int LB = 8, NU = 2;
  const size_t mn = (size_t)s.B * m * N;
  for (int p = 0; p * 256 * LB < 3 * CW || p * 256 * NU < m * CW; ++p) {
    float v[LB];
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int e = p * 256 * LB + tid + 256 * u;
      const int r = e / CW, col = e % CW;
      v[u] = 0.f;
      if (e >= 3 * CW) continue;
      if (r >= 4 - s.ks && col < (G + 1) * D) {
        const int sl = r - (4 - s.ks);           // window slot of token L-3+r
        v[u] = col < G * D ? to_f32(cq[(size_t)(b * ks1 + sl) * eq + g * G * D + col])
                           : to_f32(ck[(size_t)(b * ks1 + sl) * ekv + g * D + col - G * D]);
      } else if (r == 2 && shifted && col >= (G + 1) * D) {
        v[u] = to_f32(vs[(size_t)(b * (s.Hkv / 2) + g - s.Hkv / 2) * D + col - (G + 1) * D]);
      }
    }
    float a[NU][16];
#pragma unroll
    for (int n = 0; n < NU; ++n) {
      const int e = p * 256 * NU + tid + 256 * n;
#pragma unroll
      for (int sl = 0; sl < 16; ++sl) a[n][sl] = 0.f;
      if (e >= m * CW) continue;
      const int j = e / CW, col = e % CW;
      const size_t i = (size_t)(b * m + j) * N + group_col(col, g, G, D, eq, ekv);
      if (qkv.slices == 0) {
        a[n][0] = qkv.qkv[i];
      } else {
#pragma unroll
        for (int sl = 0; sl < 16; ++sl)
          if (sl < qkv.slices) a[n][sl] = qkv.parts[sl * mn + i];
      }
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int e = p * 256 * LB + tid + 256 * u;
      if (e < 3 * CW) tile[e] = v[u];
    }
#pragma unroll
    for (int n = 0; n < NU; ++n) {
      const int e = p * 256 * NU + tid + 256 * n;
      if (e >= m * CW) continue;
      float acc = a[n][0];
      if (qkv.slices > 0) {
#pragma unroll
        for (int sl = 1; sl < 16; ++sl)
          if (sl < qkv.slices) acc += a[n][sl];
      }
      tile[3 * CW + e] = acc;
    }
  }
  tr.store(s, staps, ctaps, tsc);
  __syncthreads();

  const int upp = 256 / LPU;
  TV *kc = reinterpret_cast<TV *>(in.k_cache);
  TV *vc = reinterpret_cast<TV *>(in.v_cache);
  // the value rows of the new tokens and the rolled state depend on the tile
  // only: their stores go out before the mixing
  for (int e = tid; e < m * (D / 4); e += 256) {
    const int j = e / (D / 4), c4 = e % (D / 4);
    size_t row;
    if (cache_row_store(in, b, s.Hkv, g, L + j, &row))
      Store4<TV>::st(vc + row * D + 4 * c4, tile + (3 + j - shifted) * CW + (G + 1) * D + 4 * c4);
  }
  // rolled state: slot sl holds token L + m - ks1 + sl = tile row m + 3 - ks1 + sl
  {
    TV *oq = reinterpret_cast<TV *>(out.conv_q);
    TV *ok = reinterpret_cast<TV *>(out.conv_k);
    for (int e = tid; e < ks1 * G * D; e += 256) {
      const int sl = e / (G * D), c = e % (G * D);
      oq[(size_t)(b * ks1 + sl) * eq + g * G * D + c] = from_f32<TV>(tile[(m + 3 - ks1 + sl) * CW + c]);
    }
    for (int e = tid; e < ks1 * D; e += 256) {
      const int sl = e / D, c = e % D;
      ok[(size_t)(b * ks1 + sl) * ekv + g * D + c] = from_f32<TV>(tile[(m + 3 - ks1 + sl) * CW + G * D + c]);
    }
    if (shifted && out.vshift)
      for (int c = tid; c < D; c += 256)
        reinterpret_cast<TV *>(out.vshift)[(size_t)(b * (s.Hkv / 2) + g - s.Hkv / 2) * D + c] =
            from_f32<TV>(tile[(m + 2) * CW + (G + 1) * D + c]);
  }

  auto emit_to = [&](int j, int slot, float *y) {
    size_t row;
    if (slot < G)
      Store4<float>::st(qout + ((size_t)(b * m + j) * s.Hq + g * G + slot) * D + 4 * li, y);
    else if (cache_row_store(in, b, s.Hkv, g, L + j, &row))
      Store4<TV>::st(kc + row * D + 4 * li, y);
  };
  if (m * (G + 1) <= upp) {
    // one (token, head slot) unit per lane group, all in parallel: the
    // convolutions, then the q-k-mean terms exchanged through LDS (own[u]:
    // the values unit u contributes to the mean), then norm and RoPE.  The
    // same arithmetic, in the same order, as mix_row.
    float *own = tsc + (G + 3) / 4 * 4;
    const int units = m * (G + 1), u = ui < units ? ui : units - 1;
    const int j = u / (G + 1), sl = u % (G + 1);
    const float2 cs0 = rope_cs_theta(L + j, th0, s.rope_base);
    const float2 cs1 = rope_cs_theta(L + j, th1, s.rope_base);
    float bb[4];
    f32x4 pre;
    conv_slot<D, float>(tile, CW, 3 + j, sl, li, staps, ctaps, bb, pre);
    const bool mean = s.use_mean != 0, post = s.use_mean == 2;
    float o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = post ? pre[c] + bb[c] : pre[c];
    if (ui < units) *reinterpret_cast<f32x4 *>(own + u * D + 4 * li) = f32x4{o[0], o[1], o[2], o[3]};
    __syncthreads();
    if (mean) {
      const float coef = post ? 0.25f : 0.5f;
      const f32x4 sk = *reinterpret_cast<const f32x4 *>(own + (j * (G + 1) + G) * D + 4 * li);
      if (sl < G) {
#pragma unroll
        for (int c = 0; c < 4; ++c) bb[c] += coef * (o[c] + sk[c]);
      } else {
        float sq[4] = {0.f, 0.f, 0.f, 0.f};
        for (int h = 0; h < G; ++h) {
          const f32x4 oh = *reinterpret_cast<const f32x4 *>(own + (j * (G + 1) + h) * D + 4 * li);
#pragma unroll
          for (int c = 0; c < 4; ++c) sq[c] += oh[c];
        }
        const float invg = 1.f / (float)G;
#pragma unroll
        for (int c = 0; c < 4; ++c) bb[c] += coef * (sk[c] + sq[c] * invg);
      }
    }
    float y[4];
    norm_rope<D>(s, cs0, cs1, 1.f, bb, y);
    if (ui < units) emit_to(j, sl, y);
    return;
  }
  // one new token per lane group; groups past the last token compute on row
  // 0 and store nothing
  for (int j0 = 0; j0 < m; j0 += upp) {
    const int j = j0 + ui;
    const bool active = j < m;
    const int jr = active ? j : 0;
    const float2 cs0 = rope_cs_theta(L + jr, th0, s.rope_base);
    const float2 cs1 = rope_cs_theta(L + jr, th1, s.rope_base);
    auto conv = [&](int slot, float (&bb)[4], f32x4 &pre) {
      conv_slot<D, float>(tile, CW, 3 + jr, slot, li, staps, ctaps, bb, pre);
    };
    auto emit = [&](int slot, float *y) {
      if (active) emit_to(j, slot, y);
    };
    mix_row<D>(G, s, cs0, cs1, conv, emit, [](int) { return 1.f; });
  }
}

// The decode mixing under the grouped channel conv (m = s.T new tokens per
// sequence at positions L .. L+m-1).  The carried window holds W = (k_s - 1)
// + (k_c - 1) pre-conv rows; one workgroup per (b, g) stages them with the m
// new rows, computes a (the sequence conv) for tokens L-k_c+1 .. L+m-1 into
// LDS, then one thread per output forms b = sum_j W[h, i, j, :] . a[t - j]
// on the VALU (one (sequence, group) holds at most a few thousand of them)
// into LDS, and each (new token) row finishes with mix_row.  All state reads
// finish before the first barrier, so state_out may alias state_in.
template <typename TV, int D>
__global__ __launch_bounds__(256) void convmix_decode_grouped_kernel(
    MixShape s, MixTaps w, const float *__restrict__ dense_q, const float *__restrict__ dense_k,
    DecQkv qkv, int Lmax, const int *__restrict__ lens, StateOut in,
    StateOut out, float *__restrict__ qout) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int G = s.G, CW = (G + 2) * D, QK = (G + 1) * D;
  const int m = s.T;
  const int ks1 = s.ks - 1, kc1 = s.kc - 1, W = ks1 + kc1;
  const int Wt = W > 0 ? W : 1;          // carried tile rows (one at least, for the shifted value)
  const int R = Wt + m, AR = kc1 + m;
  float *tile = lds;                     // [R][CW]: rows 0..Wt-1 carried, then the new tokens
  float *at = tile + R * CW;             // [AR][QK]: a of tokens L-kc1 .. L+m-1
  float *bt = at + AR * QK;              // [m][QK]: b of the new tokens

  const int tid = threadIdx.x;
  const int g = blockIdx.x % s.Hkv, b = blockIdx.x / s.Hkv;
  const int L = lens ? min(max(lens[b], 0), Lmax) : Lmax;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int shifted = (s.use_shift && g >= s.Hkv / 2) ? 1 : 0;
  const TV *cq = reinterpret_cast<const TV *>(in.conv_q);
  const TV *ck = reinterpret_cast<const TV *>(in.conv_k);
  const TV *vs = reinterpret_cast<const TV *>(in.vshift);

  for (int e = tid; e < R * CW; e += 256) {
    const int r = e / CW, col = e % CW;
    float v = 0.f;
    if (r >= Wt) {
      v = dec_qkv(qkv, (size_t)(b * m + r - Wt) * N + group_col(col, g, G, D, eq, ekv),
                  (size_t)s.B * m * N);
    } else if (col < QK) {
      const int sl = r - (Wt - W);               // window slot of token L - Wt + r
      if (sl >= 0)
        v = col < G * D ? to_f32(cq[(size_t)(b * W + sl) * eq + g * G * D + col])
                        : to_f32(ck[(size_t)(b * W + sl) * ekv + g * D + col - G * D]);
    } else if (r == Wt - 1 && shifted) {
      v = to_f32(vs[(size_t)(b * (s.Hkv / 2) + g - s.Hkv / 2) * D + col - QK]);
    }
    tile[e] = v;
  }
  __syncthreads();

  // a of token L - kc1 + r' is tile row Wt - kc1 + r'; its k_s inputs reach
  // back to row Wt - W >= 0
  for (int e = tid; e < AR * QK; e += 256) {
    const int rr = e / QK, c = e % QK, row = Wt - kc1 + rr;
    const float *tp = c < G * D ? w.q_seq + (size_t)(g * G * D + c) * s.ks
                                : w.k_seq + (size_t)(g * D + c - G * D) * s.ks;
    float acc = 0.f;
    for (int j = 0; j < s.ks; ++j) acc = fmaf(tp[j], tile[(row - j) * CW + c], acc);
    at[e] = acc;
  }
  __syncthreads();

  // b of every (new token j, head slot, channel i): one thread per output,
  // a dot product of the row W[h, i, :, :] (k_c * d contiguous floats) with
  // the a rows of the k_c lags
  for (int e = tid; e < m * QK; e += 256) {
    const int j = e / QK, col = e % QK, slot = col / D, i = col % D;
    const float *wrow = (slot < G ? dense_q + (size_t)(g * G + slot) * D * s.kc * D
                                  : dense_k + (size_t)g * D * s.kc * D) + (size_t)i * s.kc * D;
    float acc = 0.f;
    for (int lag = 0; lag < s.kc; ++lag) {
      const float *arow = at + (kc1 + j - lag) * QK + slot * D;   // a of token L + j - lag
#pragma unroll
      for (int c4 = 0; c4 < D; c4 += 4) {
        const f32x4 wv = *reinterpret_cast<const f32x4 *>(wrow + lag * D + c4);
        const f32x4 av = *reinterpret_cast<const f32x4 *>(arow + c4);
        acc += wv[0] * av[0] + wv[1] * av[1] + wv[2] * av[2] + wv[3] * av[3];
      }
    }
    bt[e] = acc;
  }
  __syncthreads();

  constexpr int LPU = D / 4;
  const int upp = 256 / LPU;
  const int li = tid % LPU, ui = tid / LPU;
  TV *kc = reinterpret_cast<TV *>(in.k_cache);
  TV *vc = reinterpret_cast<TV *>(in.v_cache);
  for (int j0 = 0; j0 < m; j0 += upp) {
    const int j = j0 + ui;
    const bool active = j < m;
    const int jr = active ? j : 0;
    const float2 cs0 = rope_cs_theta(L + jr, s.theta[2 * li], s.rope_base);
    const float2 cs1 = rope_cs_theta(L + jr, s.theta[2 * li + 1], s.rope_base);
    const float *cur = tile + (Wt + jr) * CW + 4 * li;
    auto conv = [&](int slot, float (&bb)[4], f32x4 &pre) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(bt + jr * QK + slot * D + 4 * li);
#pragma unroll
      for (int c = 0; c < 4; ++c) bb[c] = v[c];
      pre = *reinterpret_cast<const f32x4 *>(cur + slot * D);
    };
    auto emit = [&](int slot, float *y) {
      if (!active) return;
      size_t row;
      if (slot < G)
        Store4<float>::st(qout + ((size_t)(b * m + j) * s.Hq + g * G + slot) * D + 4 * li, y);
      else if (cache_row_store(in, b, s.Hkv, g, L + j, &row))
        Store4<TV>::st(kc + row * D + 4 * li, y);
    };
    mix_row<D>(G, s, cs0, cs1, conv, emit, [](int) { return 1.f; });
  }
  for (int e = tid; e < m * (D / 4); e += 256) {
    const int j = e / (D / 4), c4 = e % (D / 4);
    size_t row;
    if (cache_row_store(in, b, s.Hkv, g, L + j, &row))
      Store4<TV>::st(vc + row * D + 4 * c4, tile + (Wt + j - shifted) * CW + QK + 4 * c4);
  }
  // rolled window: slot sl holds token L + m - W + sl = tile row Wt + m - W + sl
  TV *oq = reinterpret_cast<TV *>(out.conv_q);
  TV *ok = reinterpret_cast<TV *>(out.conv_k);
  for (int e = tid; e < W * G * D; e += 256) {
    const int sl = e / (G * D), c = e % (G * D);
    oq[(size_t)(b * W + sl) * eq + g * G * D + c] = from_f32<TV>(tile[(Wt + m - W + sl) * CW + c]);
  }
  for (int e = tid; e < W * D; e += 256) {
    const int sl = e / D, c = e % D;
    ok[(size_t)(b * W + sl) * ekv + g * D + c] = from_f32<TV>(tile[(Wt + m - W + sl) * CW + G * D + c]);
  }
  if (shifted && out.vshift)
    for (int c = tid; c < D; c += 256)
      reinterpret_cast<TV *>(out.vshift)[(size_t)(b * (s.Hkv / 2) + g - s.Hkv / 2) * D + c] =
          from_f32<TV>(tile[(Wt + m - 1) * CW + QK + c]);
}

// ---------------------------------------------------------------------------
// Down-projection fused with the mixing steps (a1 + a2..a7) for kv groups of
// one query head (G = 1), d = 64 and sequences of a multiple of 128 tokens.
// A workgroup computes the 128-token x (q | k | v columns of one kv group)
// tile of qkv~ = x W_qkv^T with the DMA GEMM main loop, leaves it in LDS as
// fp32 below the 3-token halo that the previous tile's tokens form (computed
// beforehand by a small GEMM over just those rows), and runs the mixing of
// convmix_prefill_kernel on it: qkv~ never goes to HBM.
// ---------------------------------------------------------------------------
static constexpr int FUSE_BM = 128;

// xh[mt * 3 + r] = x row of token t0 - 3 + r of tile mt (t0 = its first token;
// zero rows for the first tile of a sequence)
__global__ __launch_bounds__(256) void halo_rows_kernel(const bf16 *__restrict__ x,
                                                        bf16 *__restrict__ xh, int T, int E,
                                                        int nrows) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per = E / 8;
  if (e >= (long long)nrows * per) return;
  const int row = (int)(e / per), c8 = (int)(e % per);
  const int tps = T / FUSE_BM;
  const int mt = row / HALO, r = row % HALO, b = mt / tps, tt = mt % tps;
  const u32x4 v = tt > 0 ? ld16(x + ((size_t)b * T + tt * FUSE_BM - HALO + r) * E + 8 * c8)
                         : zero_u32x4();
  st16(xh + (size_t)row * E + 8 * c8, v);
}

template <typename TQ, typename TV>
__global__ __launch_bounds__(256, 1) void downproj_mix_kernel(MixShape s, MixTaps w,
                                                             const bf16 *__restrict__ x,
                                                             const bf16 *__restrict__ wqkv,
                                                             const float *__restrict__ halo,
                                                             TQ *__restrict__ q,
                                                             TQ *__restrict__ k,
                                                             TV *__restrict__ vt, int E) {
  constexpr int D = 64, G = 1, BM = FUSE_BM, CW = (G + 2) * D, BN = CW, BK = 32, STAGES = 5;
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int RING = STAGES * (BM + BN) * 2 * BK;
  constexpr int TILE_F = (BM + HALO) * CW;
  constexpr int TAPS_F = (G + 1) * D * 4 + (G + 1) * 4 + 4;
  constexpr int EPI = (TILE_F + TAPS_F) * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[RING > EPI ? RING : EPI];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, hl = lane >> 5;
  const int tps = s.T / BM;
  const int lid = xcd_remap(blockIdx.x, s.B * tps * s.Hkv);
  const int g = lid % s.Hkv, mt = lid / s.Hkv;
  const int b = mt / tps, tt = mt % tps;
  const int t0 = tt * BM;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;

  f32x16 acc[TM][TN];
  dma_gemm_tile<BM, BN, BK, STAGES>(x, wqkv, s.B * s.T, N, E, E, b * s.T + t0,
                                    [&](int r) { return group_col(r, g, G, D, eq, ekv); }, 0, E,
                                    smem, acc);
  __syncthreads();                                  // every wave is done with the ring

  float *tile = reinterpret_cast<float *>(smem);    // rows: tokens t0-HALO .. t0+BM-1
  float *staps = tile + TILE_F;
  float *ctaps = staps + (G + 1) * D * 4;
  float *tsc = ctaps + (G + 1) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int row = wm * (BM / 2) + i * 32 + 8 * (a >> 2) + 4 * hl + (a & 3);
        tile[(HALO + row) * CW + wn * (BN / 2) + j * 32 + l32] = acc[i][j][a];
      }
  for (int e = tid; e < HALO * CW; e += 256) {
    const int r = e / CW, c = e % CW;
    tile[e] = tt > 0 ? halo[((size_t)mt * HALO + r) * N + group_col(c, g, G, D, eq, ekv)] : 0.f;
  }
  load_taps<D>(s, w, g, staps, ctaps, tsc);
  __syncthreads();

  // the mixing of convmix_prefill_kernel on the tile's rows
  constexpr int LPU = D / 4;
  const int upp = 256 / LPU;
  const int li = tid % LPU, ui = tid / LPU;
  for (int r = ui; r < BM; r += upp) {
    const int tok = t0 + r;
    const float2 cs0 = rope_cs_theta(tok, s.theta[2 * li], s.rope_base);
    const float2 cs1 = rope_cs_theta(tok, s.theta[2 * li + 1], s.rope_base);
    auto conv = [&](int slot, float (&bb)[4], f32x4 &pre) {
      conv_slot<D, float>(tile, CW, r + HALO, slot, li, staps, ctaps, bb, pre);
    };
    auto emit = [&](int slot, float *y) {
      if (slot < G)
        Store4<TQ>::st(q + ((size_t)(b * s.Hq + g * G + slot) * s.Tp + tok) * D + 4 * li, y);
      else
        Store4<TQ>::st(k + ((size_t)(b * s.Hkv + g) * s.Tp + tok) * D + 4 * li, y);
    };
    // q leaves scaled by tau_h * log2(e), folded into the normalisation
    mix_row<D>(G, s, cs0, cs1, conv, emit, [&](int slot) { return slot < G ? tsc[slot] : 1.f; });
  }
  // value head, transposed: vt[b, g, dd, perm(t)]
  const int shifted = (s.use_shift && g >= s.Hkv / 2) ? 1 : 0;
  const int vcol = (G + 1) * D;
  for (int e = tid; e < D * (BM / 8); e += 256) {
    const int dd = e / (BM / 8), grp = e % (BM / 8);
    float vals[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      vals[jj] = tile[(vt_perm(8 * grp + jj) + HALO - shifted) * CW + vcol + dd];
    TV *dst = vt + ((size_t)(b * s.Hkv + g) * D + dd) * s.Tp + t0 + 8 * grp;
    Store4<TV>::st(dst, vals);
    Store4<TV>::st(dst + 4, vals + 4);
  }
}

bool downproj_mix_supported(int G, int d, int T, int E) {
  return G == 1 && d == 64 && T % FUSE_BM == 0 && E % 32 == 0;
}

size_t downproj_mix_halo_bytes(int B, int T, int E, int N) {
  const size_t rows = (size_t)B * (T / FUSE_BM) * HALO;
  return rows * E * 2 + rows * N * 4 + 256;
}

template <typename TQ, typename TV>
hipError_t launch_downproj_mix(const MixShape &s, const MixTaps &w, const bf16 *x,
                               const bf16 *wqkv, int E, void *halo_ws, TQ *q, TQ *k, TV *vt,
                               hipStream_t stream) {
  const int N = (s.Hq + 2 * s.Hkv) * s.d;
  const int nrows = s.B * (s.T / FUSE_BM) * HALO;
  bf16 *xh = reinterpret_cast<bf16 *>(halo_ws);
  float *hq = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(halo_ws) +
                                        ((size_t)nrows * E * 2 + 255) / 256 * 256);
  const long long nthr = (long long)nrows * (E / 8);
  hipLaunchKernelGGL(halo_rows_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream,
                     x, xh, s.T, E, nrows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gemm_nt<bf16, float>(xh, wqkv, hq, nrows, N, E, E, E, N, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((downproj_mix_kernel<TQ, TV>), dim3(s.B * (s.T / FUSE_BM) * s.Hkv), dim3(256),
                     0, stream, s, w, x, wqkv, hq, q, k, vt, E);
  return hipGetLastError();
}

template hipError_t launch_downproj_mix<f16, bf16>(const MixShape &, const MixTaps &, const bf16 *,
                                                   const bf16 *, int, void *, f16 *, f16 *, bf16 *,
                                                   hipStream_t);
template hipError_t launch_downproj_mix<bf16, bf16>(const MixShape &, const MixTaps &, const bf16 *,
                                                    const bf16 *, int, void *, bf16 *, bf16 *,
                                                    bf16 *, hipStream_t);

// LDS of the prefill kernel for chunks of TC tokens (fp32 tile).
static size_t mix_lds_bytes(int TC, int G, int D, int es) {
  return tile_bytes(TC + HALO, G, D, es) + (size_t)taps_floats(G, D) * 4 + (size_t)D / 2 * 8;
}

// Tokens per workgroup: the largest of 64 / 32 / 16 whose LDS stays within
// 40 KiB (several workgroups per CU keep many rows in flight).
static int mix_chunk(int G, int D, int es) {
  for (int tc = 64; tc > 16; tc /= 2)
    if (mix_lds_bytes(tc, G, D, es) <= 40 * 1024) return tc;
  return 16;
}

// tile, taps, and the q-k-mean exchange of the parallel path (256 / (D/4)
// lane groups x D floats = 4 KiB)
static size_t decode_lds_bytes(int rows, int G, int D) {
  return tile_bytes(rows, G, D, 4) + (size_t)taps_floats(G, D) * 4 + 4096;
}

bool convmix_decode_fits(int G, int d, int m) {
  return m >= 1 && decode_lds_bytes(3 + m, G, d) <= 65536;
}

bool convmix_fits(int G, int d) {
  // the prefill staging gives each thread one 16-byte column chunk of a row
  return (G + 2) * d / 4 <= 256 && mix_lds_bytes(16, G, d, 4) <= 65536 && convmix_decode_fits(G, d, 1);
}

template <typename TI, typename TQ, typename TV, int D, int MEAN, bool R1B, bool OUT>
static hipError_t convmix_prefill_launch(const MixShape &s, const MixTaps &w, const TI *qkv, TQ *q,
                                         TQ *k, TV *vt, const StateOut &st, const float *r1b,
                                         float *bout, hipStream_t stream) {
  const int TC = mix_chunk(s.G, D, sizeof(TI));
  const long long grid = (long long)s.B * s.Hkv * (s.Tp / TC);
  if (grid >= (1ll << 31)) return hipErrorInvalidValue;
  const size_t lds = mix_lds_bytes(TC, s.G, D, sizeof(TI));
  hipLaunchKernelGGL((convmix_prefill_kernel<TI, TQ, TV, D, MEAN, R1B, OUT>), dim3((unsigned)grid),
                     dim3(256), lds, stream, s, w, qkv, q, k, vt, st, r1b, bout, TC);
  return hipGetLastError();
}

template <typename TI, typename TQ, typename TV, int D>
static hipError_t convmix_prefill_d(const MixShape &s, const MixTaps &w, const TI *qkv, TQ *q,
                                    TQ *k, TV *vt, const StateOut &st, const float *r1b,
                                    float *bout, hipStream_t stream) {
#define CCA_MIX_LAUNCH(M, R, O) \
  convmix_prefill_launch<TI, TQ, TV, D, M, R, O>(s, w, qkv, q, k, vt, st, r1b, bout, stream)
  const bool out = st.k_cache || st.v_cache || st.conv_q || st.conv_k || st.vshift || bout;
  if (r1b) {   // the grouped reading, always with the outputs switch on
    switch (s.use_mean) {
      case 0: return CCA_MIX_LAUNCH(0, true, true);
      case 1: return CCA_MIX_LAUNCH(1, true, true);
      default: return CCA_MIX_LAUNCH(2, true, true);
    }
  }
  if (out) {
    switch (s.use_mean) {
      case 0: return CCA_MIX_LAUNCH(0, false, true);
      case 1: return CCA_MIX_LAUNCH(1, false, true);
      default: return CCA_MIX_LAUNCH(2, false, true);
    }
  }
  switch (s.use_mean) {
    case 0: return CCA_MIX_LAUNCH(0, false, false);
    case 1: return CCA_MIX_LAUNCH(1, false, false);
    default: return CCA_MIX_LAUNCH(2, false, false);
  }
#undef CCA_MIX_LAUNCH
}

template <typename TI, typename TQ, typename TV>
hipError_t launch_convmix_prefill(const MixShape &s, const MixTaps &w, const TI *qkv, TQ *q,
                                  TQ *k, TV *vt, const StateOut &st, hipStream_t stream,
                                  const float *r1b, float *bout) {
  switch (s.d) {
    case 16: return convmix_prefill_d<TI, TQ, TV, 16>(s, w, qkv, q, k, vt, st, r1b, bout, stream);
    case 32: return convmix_prefill_d<TI, TQ, TV, 32>(s, w, qkv, q, k, vt, st, r1b, bout, stream);
    case 64: return convmix_prefill_d<TI, TQ, TV, 64>(s, w, qkv, q, k, vt, st, r1b, bout, stream);
    case 128: return convmix_prefill_d<TI, TQ, TV, 128>(s, w, qkv, q, k, vt, st, r1b, bout, stream);
  }
  return hipErrorInvalidValue;
}

template <typename TV, int D>
static hipError_t convmix_decode_d(const MixShape &s, const MixTaps &w, const DecQkv &qkv, int L,
                                   const int *lens,
                                   const StateOut &in, const StateOut &out, float *q,
                                   hipStream_t stream) {
  const size_t lds = decode_lds_bytes(3 + s.T, s.G, D);
  hipLaunchKernelGGL((convmix_decode_kernel<TV, D>), dim3(s.B * s.Hkv), dim3(256), lds, stream, s,
                     w, qkv, L, lens, in, out, q);
  return hipGetLastError();
}

template <typename TV>
hipError_t launch_convmix_decode(const MixShape &s, const MixTaps &w, const DecQkv &qkv, int L,
                                 const int *lens, const StateOut &in, const StateOut &out, float *q,
                                 hipStream_t stream) {
  switch (s.d) {
    case 16: return convmix_decode_d<TV, 16>(s, w, qkv, L, lens, in, out, q, stream);
    case 32: return convmix_decode_d<TV, 32>(s, w, qkv, L, lens, in, out, q, stream);
    case 64: return convmix_decode_d<TV, 64>(s, w, qkv, L, lens, in, out, q, stream);
    case 128: return convmix_decode_d<TV, 128>(s, w, qkv, L, lens, in, out, q, stream);
  }
  return hipErrorInvalidValue;
}

static size_t decode_grouped_lds_bytes(int G, int D, int m, int ks, int kc) {
  const int W = ks - 1 + kc - 1, Wt = W > 0 ? W : 1;
  return ((size_t)(Wt + m) * (G + 2) * D + (size_t)(kc - 1 + m) * (G + 1) * D +
          (size_t)m * (G + 1) * D) * 4;
}

bool convmix_decode_grouped_fits(int G, int d, int m, int ks, int kc) {
  return m >= 1 && decode_grouped_lds_bytes(G, d, m, ks, kc) <= 65536;
}

template <typename TV, int D>
static hipError_t convmix_decode_grouped_d(const MixShape &s, const MixTaps &w, const float *dq,
                                           const float *dk, const DecQkv &qkv, int L,
                                           const int *lens, const StateOut &in,
                                           const StateOut &out, float *q, hipStream_t stream) {
  const size_t lds = decode_grouped_lds_bytes(s.G, D, s.T, s.ks, s.kc);
  if (lds > 65536) return hipErrorInvalidValue;
  hipLaunchKernelGGL((convmix_decode_grouped_kernel<TV, D>), dim3(s.B * s.Hkv), dim3(256), lds,
                     stream, s, w, dq, dk, qkv, L, lens, in, out, q);
  return hipGetLastError();
}

template <typename TV>
hipError_t launch_convmix_decode_grouped(const MixShape &s, const MixTaps &w, const float *dense_q,
                                         const float *dense_k, const DecQkv &qkv, int L,
                                         const int *lens, const StateOut &in, const StateOut &out,
                                         float *q, hipStream_t stream) {
  switch (s.d) {
    case 16: return convmix_decode_grouped_d<TV, 16>(s, w, dense_q, dense_k, qkv, L, lens, in, out, q, stream);
    case 32: return convmix_decode_grouped_d<TV, 32>(s, w, dense_q, dense_k, qkv, L, lens, in, out, q, stream);
    case 64: return convmix_decode_grouped_d<TV, 64>(s, w, dense_q, dense_k, qkv, L, lens, in, out, q, stream);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_convmix_decode_grouped<bf16>(const MixShape &, const MixTaps &,
                                                        const float *, const float *, const DecQkv &,
                                                        int, const int *, const StateOut &,
                                                        const StateOut &, float *, hipStream_t);
template hipError_t launch_convmix_decode_grouped<float>(const MixShape &, const MixTaps &,
                                                         const float *, const float *, const DecQkv &,
                                                         int, const int *, const StateOut &,
                                                         const StateOut &, float *, hipStream_t);

template hipError_t launch_convmix_prefill<f16, f16, bf16>(const MixShape &, const MixTaps &,
                                                           const f16 *, f16 *, f16 *, bf16 *,
                                                           const StateOut &, hipStream_t,
                                                           const float *, float *);
template hipError_t launch_convmix_prefill<f16, bf16, bf16>(const MixShape &, const MixTaps &,
                                                            const f16 *, bf16 *, bf16 *, bf16 *,
                                                            const StateOut &, hipStream_t,
                                                            const float *, float *);
template hipError_t launch_convmix_prefill<float, float, float>(const MixShape &, const MixTaps &,
                                                                const float *, float *, float *,
                                                                float *, const StateOut &,
                                                                hipStream_t, const float *, float *);
template hipError_t launch_convmix_decode<bf16>(const MixShape &, const MixTaps &, const DecQkv &,
                                                int, const int *, const StateOut &, const StateOut &, float *,
                                                hipStream_t);
template hipError_t launch_convmix_decode<float>(const MixShape &, const MixTaps &, const DecQkv &,
                                                int, const int *, const StateOut &, const StateOut &, float *,
                                                 hipStream_t);

}  // namespace cca
