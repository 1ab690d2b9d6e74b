// Fused latent mixing of the CCA forward pass (gfx950), memory bound.
//
// For every token and latent head, from the fp32 down-projection output:
//   a2 causal sequence conv, depthwise, lag-indexed k_s taps per channel
//   a3 channel conv: one k_c-tap filter per head sliding along the channel
//      index, zero padded inside the head
//      [GS-EN "2. Methodology" / Convolutional Mixing]
//   a4 q-k-mean: the mean of the pre-convolution q~ and k~ added to the
//      convolved q and k; with G query heads per kv head, q head h meets k~ of
//      its group and kv head g meets the average q~ of its G heads
//      [GS-EN "2. Methodology" / Q-K-Mean]
//   a5 value-shift: the upper half of the kv heads take the previous token's
//      value [GS-EN "2. Methodology" / Value-Shift]
//   a6 L2 normalisation per head, x / max(||x||, eps)
//   a7 RoPE, pairs (2i, 2i+1), angle pos * base^(-2i/d) evaluated in double
//      and reduced modulo 2*pi before the fp32 sin/cos
//      [GS-EN "2. Methodology" / RoPE Integration]
//
// Work split: one workgroup per (batch b, kv group g, chunk of TC tokens).
// The group's pre-conv columns (G query heads, its key head, its value head)
// for tokens t0-3 .. t0+TC-1 are staged in LDS with coalesced 16-byte loads
// (the 3-token halo of the causal window comes along), together with the
// group's taps and a cos/sin table of the chunk.  A head of d channels is
// handled by d/4 lanes of 4 consecutive channels each, so the channel
// convolution needs only three lane shifts and the RoPE pairs stay inside a
// lane; the L2 norm is a reduction over the d/4 lanes.  The value head is
// written transposed (d-major) for the attention kernel, straight from the
// LDS tile.
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
  __device__ __forceinline__ static void st(f16 *p, const float *v) {
    *reinterpret_cast<f16x4 *>(p) = f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
  }
};
template <> struct Store4<bf16> {
  __device__ __forceinline__ static void st(bf16 *p, const float *v) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  }
};

template <int D>
__device__ __forceinline__ void mix_tail(const float *cur, int slot, int G, const MixShape &s,
                                         float2 cs0, float2 cs1, float (&b)[4], float y[4]);

// Steps a2-a7 for one (token row r of the LDS tile, head slot) unit.  Slot
// 0..G-1 are the group's query heads, slot G its key head.  The lane holds
// channels 4*li .. 4*li+3.  `tile` rows are tokens (row r+HALO is the current
// token), columns [q heads | k head | v head] of the group, CW floats wide.
template <int D>
__device__ __forceinline__ void mix_unit(const float *tile, int CW, int r, int slot, int G,
                                         int li, const float (&st)[4][4], const float (&ct)[4],
                                         const MixShape &s, float2 cs0, float2 cs1, float y[4]) {
  constexpr int LPU = D / 4;
  const int col = slot * D + 4 * li;
  float a[4];
  {
    f32x4 row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) row[j] = *reinterpret_cast<const f32x4 *>(tile + (r + HALO - j) * CW + col);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(st[c][j], row[j][c], acc);
      a[c] = acc;
    }
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
  if (li == 0) p1 = p2 = p3 = 0.f;
  const float w0 = ct[0], w1 = ct[1], w2 = ct[2], w3 = ct[3];
  float b[4];
  b[0] = w0 * a[0] + w1 * p3 + w2 * p2 + w3 * p1;
  b[1] = w0 * a[1] + w1 * a[0] + w2 * p3 + w3 * p2;
  b[2] = w0 * a[2] + w1 * a[1] + w2 * a[0] + w3 * p3;
  b[3] = w0 * a[3] + w1 * a[2] + w2 * a[1] + w3 * a[0];
  mix_tail<D>(tile + (r + HALO) * CW + 4 * li, slot, G, s, cs0, cs1, b, y);
}

// Steps a4, a6, a7 after the channel conv: b (the channel-conv output of this
// lane's 4 channels) plus the q-k-mean skip from the pre-conv row `cur` (the
// token's tile row, offset to this lane's channels), normalised and rotated.
template <int D>
__device__ __forceinline__ void mix_tail(const float *cur, int slot, int G, const MixShape &s,
                                         float2 cs0, float2 cs1, float (&b)[4], float y[4]) {
  constexpr int LPU = D / 4;
  if (s.use_mean) {
    const f32x4 kpre = *reinterpret_cast<const f32x4 *>(cur + G * D);
    if (slot < G) {
      const f32x4 qpre = *reinterpret_cast<const f32x4 *>(cur + slot * D);
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] += 0.5f * (qpre[c] + kpre[c]);
    } else {
      f32x4 m = *reinterpret_cast<const f32x4 *>(cur);
      for (int h = 1; h < G; ++h) m += *reinterpret_cast<const f32x4 *>(cur + h * D);
      const float invg = 1.f / (float)G;
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] += 0.5f * (kpre[c] + m[c] * invg);
    }
  }
  if (s.use_norm) {
    // 1 / max(||b||, eps) == rsqrt(max(||b||^2, eps^2))
    const float ss = group_sum<LPU>(b[0] * b[0] + b[1] * b[1] + b[2] * b[2] + b[3] * b[3]);
    const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, s.eps * s.eps));
#pragma unroll
    for (int c = 0; c < 4; ++c) b[c] *= inv;
  }
  y[0] = b[0] * cs0.x - b[1] * cs0.y;
  y[1] = b[0] * cs0.y + b[1] * cs0.x;
  y[2] = b[2] * cs1.x - b[3] * cs1.y;
  y[3] = b[2] * cs1.y + b[3] * cs1.x;
}

// Group taps into LDS: seq taps [(G+1)*D][4] (q channels, then k), channel
// taps [(G+1)][4]; taps beyond k_s / k_c are zero.
template <int D>
__device__ __forceinline__ void load_taps(const MixShape &s, const MixTaps &w, int g, float *staps,
                                          float *ctaps) {
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
}

// This lane's taps for head slot `slot` (channels 4*li .. 4*li+3) from the
// LDS copies made by load_taps.
template <int D>
__device__ __forceinline__ void lane_taps(const float *staps, const float *ctaps, int slot, int li,
                                          float (&st)[4][4], float (&ct)[4]) {
  const int col = slot * D + 4 * li;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const f32x4 t = *reinterpret_cast<const f32x4 *>(staps + (col + c) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) st[c][j] = t[j];
  }
  const f32x4 t = *reinterpret_cast<const f32x4 *>(ctaps + slot * 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) ct[j] = t[j];
}

// Map a column of the group tile to its column in the qkv row.
__device__ __forceinline__ int group_col(int col, int g, int G, int D, int eq, int ekv) {
  if (col < G * D) return g * G * D + col;
  if (col < (G + 1) * D) return eq + g * D + (col - G * D);
  return eq + ekv + g * D + (col - (G + 1) * D);
}

// Rows of the next chunk each thread prefetches into registers (16 bytes each).
static constexpr int MIX_PF = 8;

template <typename TQ, typename TV, int D>
__global__ __launch_bounds__(256) void convmix_prefill_kernel(MixShape s, MixTaps w,
                                                              const float *__restrict__ qkv,
                                                              TQ *__restrict__ q, TQ *__restrict__ k,
                                                              TV *__restrict__ vt, StateOut st,
                                                              const float *__restrict__ r1b,
                                                              int TC, int nchunks, int cpw,
                                                              int nseg) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int G = s.G, CW = (G + 2) * D;
  float *tile = lds;                                   // rows: tokens t0-HALO .. t0+TC-1
  float *staps = tile + (TC + HALO) * CW;
  float *ctaps = staps + (G + 1) * D * 4;
  float2 *rot = reinterpret_cast<float2 *>(ctaps + ((G + 1) * 4 + 3) / 4 * 4);

  const int tid = threadIdx.x;
  const int seg = blockIdx.x % nseg;
  const int bg = blockIdx.x / nseg;
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int c_beg = seg * cpw, c_end = min(nchunks, c_beg + cpw);
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int shifted = (s.use_shift && g >= s.Hkv / 2) ? 1 : 0;
  const int vcol = (G + 1) * D;

  // each thread owns one 16-byte column chunk of the group and walks rows
  // with a fixed stride (CW/4 <= 256 chunks per row)
  const int cpr = CW / 4;
  const int rstep = 256 / cpr;
  const int my_col = (tid % cpr) * 4, my_row0 = tid / cpr;
  const bool col_active = my_row0 < rstep;
  const float *src_col = qkv + group_col(my_col, g, G, D, eq, ekv) + (size_t)b * s.T * N;
  auto row_load = [&](int tok) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (tok >= 0 && tok < s.T) v = *reinterpret_cast<const f32x4 *>(src_col + (size_t)tok * N);
    return v;
  };

  load_taps<D>(s, w, g, staps, ctaps);

  // first chunk: halo and rows straight into LDS
  {
    const int t0 = c_beg * TC;
    for (int r0 = my_row0; r0 < TC + HALO; r0 += rstep * MIX_PF) {
      f32x4 v[MIX_PF];
#pragma unroll
      for (int u = 0; u < MIX_PF; ++u) {
        const int r = r0 + rstep * u;
        v[u] = (col_active && r < TC + HALO) ? row_load(t0 - HALO + r) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < MIX_PF; ++u) {
        const int r = r0 + rstep * u;
        if (col_active && r < TC + HALO) *reinterpret_cast<f32x4 *>(tile + r * CW + my_col) = v[u];
      }
    }
  }

  constexpr int LPU = D / 4;
  const int upp = 256 / LPU;
  const int li = tid % LPU, ui = tid / LPU;
  f32x4 pf[MIX_PF];

  for (int ch = c_beg; ch < c_end; ++ch) {
    const int t0 = ch * TC;
    // rotation table of the chunk: one double multiply and reduction per entry
    for (int e = tid; e < TC * (D / 2); e += 256)
      rot[e] = rope_cs_theta(t0 + e / (D / 2), s.theta[e % (D / 2)], s.rope_base);
    __syncthreads();

    // prefetch the next chunk's rows; their latency overlaps this chunk's math
    const bool more = ch + 1 < c_end;
    if (more) {
#pragma unroll
      for (int u = 0; u < MIX_PF; ++u) {
        const int r = my_row0 + rstep * u;
        pf[u] = (col_active && r < TC) ? row_load(t0 + TC + r) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

    // query and key heads, slot-major so each lane keeps its head's taps in
    // registers: slot 0..G-1 are the query heads, slot G the key head
    for (int slot = 0; slot <= G; ++slot) {
      float stp[4][4], ctp[4];
      lane_taps<D>(staps, ctaps, slot, li, stp, ctp);
      const float qscale = slot < G ? w.tau[g * G + slot] * 1.4426950408889634f : 1.f;
      for (int r = ui; r < TC; r += upp) {
        const int tok = t0 + r;
        float y[4];
        if (r1b) {
          // grouped channel conv: b comes from the MFMA kernel's output rows
          float bb[4] = {0.f, 0.f, 0.f, 0.f};
          if (tok < s.T) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(
                r1b + (size_t)(b * s.T + tok) * (eq + ekv) + (slot < G ? (g * G + slot) * D : eq + g * D) + 4 * li);
#pragma unroll
            for (int c = 0; c < 4; ++c) bb[c] = v[c];
          }
          mix_tail<D>(tile + (r + HALO) * CW + 4 * li, slot, G, s, rot[r * (D / 2) + 2 * li],
                      rot[r * (D / 2) + 2 * li + 1], bb, y);
        } else {
          mix_unit<D>(tile, CW, r, slot, G, li, stp, ctp, s, rot[r * (D / 2) + 2 * li],
                      rot[r * (D / 2) + 2 * li + 1], y);
        }
        if (tok >= s.T) y[0] = y[1] = y[2] = y[3] = 0.f;
        if (slot < G) {
          // the attention kernel takes q scaled by tau_h * log2(e) (exp2-domain logits)
#pragma unroll
          for (int c = 0; c < 4; ++c) y[c] *= qscale;
          Store4<TQ>::st(q + ((size_t)(b * s.Hq + g * G + slot) * s.Tp + tok) * D + 4 * li, y);
        } else {
          Store4<TQ>::st(k + ((size_t)(b * s.Hkv + g) * s.Tp + tok) * D + 4 * li, y);
          if (st.k_cache && tok < s.T)
            Store4<TV>::st(reinterpret_cast<TV *>(st.k_cache) + cache_row(st, b, s.Hkv, g, tok) * D +
                               4 * li, y);
        }
      }
    }

    // value head, transposed: vt[b, g, dd, perm(t)] for the chunk's tokens
    for (int e = tid; e < D * (TC / 8); e += 256) {
      const int dd = e / (TC / 8), grp = e % (TC / 8);
      float vals[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int tl = vt_perm(8 * grp + jj);
        vals[jj] = (t0 + tl < s.T) ? tile[(tl + HALO - shifted) * CW + vcol + dd] : 0.f;
      }
      TV *dst = vt + ((size_t)(b * s.Hkv + g) * D + dd) * s.Tp + t0 + 8 * grp;
      Store4<TV>::st(dst, vals);
      Store4<TV>::st(dst + 4, vals + 4);
    }
    if (st.v_cache) {
      for (int e = tid; e < TC * (D / 4); e += 256) {
        const int r = e / (D / 4), c4 = e % (D / 4), tok = t0 + r;
        if (tok >= s.T) continue;
        const float *src = tile + (r + HALO - shifted) * CW + vcol + 4 * c4;
        Store4<TV>::st(reinterpret_cast<TV *>(st.v_cache) + cache_row(st, b, s.Hkv, g, tok) * D +
                           4 * c4, src);
      }
    }
    __syncthreads();                                 // every read of this tile is done

    if (more) {
      // carry the halo (last HALO rows) to the top, then the prefetched rows
      for (int e = tid; e < HALO * CW / 4; e += 256) {
        const int r = e / (CW / 4), c4 = (e % (CW / 4)) * 4;
        *reinterpret_cast<f32x4 *>(tile + r * CW + c4) =
            *reinterpret_cast<const f32x4 *>(tile + (TC + r) * CW + c4);
      }
      __syncthreads();                               // halo rows read before they are overwritten
#pragma unroll
      for (int u = 0; u < MIX_PF; ++u) {
        const int r = my_row0 + rstep * u;
        if (col_active && r < TC) *reinterpret_cast<f32x4 *>(tile + (HALO + r) * CW + my_col) = pf[u];
      }
      // the rotation table is rewritten after the next barrier-protected use
    }
  }

  // decode state after the last token: conv window (k_s - 1 pre-conv rows,
  // plus k_c - 1 under the grouped channel conv) and value-shift state
  if (seg == 0) {
    const int ks1 = s.ks - 1 + (s.grouped ? s.kc - 1 : 0);
    const float *qb = qkv + (size_t)b * s.T * N;
    if (st.conv_q)
      for (int e = tid; e < ks1 * G * D; e += 256) {
        const int sl = e / (G * D), c = e % (G * D), tok = s.T - ks1 + sl;
        const float v = tok >= 0 ? qb[(size_t)tok * N + g * G * D + c] : 0.f;
        reinterpret_cast<TV *>(st.conv_q)[(size_t)(b * ks1 + sl) * eq + g * G * D + c] = from_f32<TV>(v);
      }
    if (st.conv_k)
      for (int e = tid; e < ks1 * D; e += 256) {
        const int sl = e / D, c = e % D, tok = s.T - ks1 + sl;
        const float v = tok >= 0 ? qb[(size_t)tok * N + eq + g * D + c] : 0.f;
        reinterpret_cast<TV *>(st.conv_k)[(size_t)(b * ks1 + sl) * ekv + g * D + c] = from_f32<TV>(v);
      }
    if (st.vshift && shifted)
      for (int c = tid; c < D; c += 256)
        reinterpret_cast<TV *>(st.vshift)[(size_t)(b * (s.Hkv / 2) + g - s.Hkv / 2) * D + c] =
            from_f32<TV>(qb[(size_t)(s.T - 1) * N + eq + ekv + g * D + c]);
  }
}

// m = s.T new tokens per sequence at positions L .. L+m-1 (L = lens[b] when
// lens is given, clamped to [0, L]).  One workgroup per (b, g); the tile
// holds tokens L-3 .. L+m-1: three rows from the carried window, then the m
// new rows from the down-projection.  All state reads finish before the
// barrier, so state_out may alias state_in.
template <typename TV, int D>
__global__ __launch_bounds__(256) void convmix_decode_kernel(MixShape s, MixTaps w,
                                                             const float *__restrict__ qkv,
                                                             int Lmax,
                                                             const int *__restrict__ lens,
                                                             StateOut in, StateOut out,
                                                             float *__restrict__ qout) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int G = s.G, CW = (G + 2) * D;
  const int m = s.T, R = 3 + m;
  float *tile = lds;                               // R rows
  float *staps = tile + R * CW;
  float *ctaps = staps + (G + 1) * D * 4;
  float2 *rot = reinterpret_cast<float2 *>(ctaps + ((G + 1) * 4 + 3) / 4 * 4);

  const int tid = threadIdx.x;
  const int g = blockIdx.x % s.Hkv, b = blockIdx.x / s.Hkv;
  const int L = lens ? min(max(lens[b], 0), Lmax) : Lmax;   // this sequence's position
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int ks1 = s.ks - 1;
  const int shifted = (s.use_shift && g >= s.Hkv / 2) ? 1 : 0;
  const TV *cq = reinterpret_cast<const TV *>(in.conv_q);
  const TV *ck = reinterpret_cast<const TV *>(in.conv_k);
  const TV *vs = reinterpret_cast<const TV *>(in.vshift);

  // all loads of the tile are issued before their LDS stores
  constexpr int LB = 8;
  for (int e0 = 0; e0 < R * CW; e0 += 256 * LB) {
    float v[LB];
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int e = e0 + tid + 256 * u;
      const int r = e / CW, col = e % CW;
      v[u] = 0.f;
      if (e >= R * CW) continue;
      if (r >= 3) {
        v[u] = qkv[(size_t)(b * m + r - 3) * N + group_col(col, g, G, D, eq, ekv)];
      } else if (r >= 4 - s.ks && col < (G + 1) * D) {
        const int sl = r - (4 - s.ks);           // window slot of token L-3+r
        v[u] = col < G * D ? to_f32(cq[(size_t)(b * ks1 + sl) * eq + g * G * D + col])
                           : to_f32(ck[(size_t)(b * ks1 + sl) * ekv + g * D + col - G * D]);
      } else if (r == 2 && shifted && col >= (G + 1) * D) {
        v[u] = to_f32(vs[(size_t)(b * (s.Hkv / 2) + g - s.Hkv / 2) * D + col - (G + 1) * D]);
      }
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int e = e0 + tid + 256 * u;
      if (e < R * CW) tile[e] = v[u];
    }
  }
  load_taps<D>(s, w, g, staps, ctaps);
  for (int e = tid; e < m * (D / 2); e += 256)
    rot[e] = rope_cs_theta(L + e / (D / 2), s.theta[e % (D / 2)], s.rope_base);
  __syncthreads();

  constexpr int LPU = D / 4;
  const int upp = 256 / LPU;
  const int li = tid % LPU, ui = tid / LPU;
  TV *kc = reinterpret_cast<TV *>(in.k_cache);
  TV *vc = reinterpret_cast<TV *>(in.v_cache);
  // units: (new token j, head slot), slot 0..G-1 the query heads, G the key head
  for (int u0 = 0; u0 < m * (G + 1); u0 += upp) {
    const int unit = u0 + ui;
    const bool active = unit < m * (G + 1);
    const int j = active ? unit / (G + 1) : 0, slot = active ? unit % (G + 1) : 0;
    float stp[4][4], ctp[4];
    lane_taps<D>(staps, ctaps, slot, li, stp, ctp);
    float y[4];
    mix_unit<D>(tile, CW, j, slot, G, li, stp, ctp, s, rot[j * (D / 2) + 2 * li],
                rot[j * (D / 2) + 2 * li + 1], y);
    if (!active) continue;
    if (slot < G) {
      Store4<float>::st(qout + ((size_t)(b * m + j) * s.Hq + g * G + slot) * D + 4 * li, y);
    } else {
      Store4<TV>::st(kc + cache_row(in, b, s.Hkv, g, L + j) * D + 4 * li, y);
    }
  }
  // value rows of the new tokens into the cache
  for (int e = tid; e < m * (D / 4); e += 256) {
    const int j = e / (D / 4), c4 = e % (D / 4);
    Store4<TV>::st(vc + cache_row(in, b, s.Hkv, g, L + j) * D + 4 * c4,
                   tile + (3 + j - shifted) * CW + (G + 1) * D + 4 * c4);
  }
  // rolled state: slot sl holds token L + m - ks1 + sl = tile row m + 3 - ks1 + sl
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

// The decode mixing under the grouped channel conv (m = s.T new tokens per
// sequence at positions L .. L+m-1).  The carried window holds W = (k_s - 1)
// + (k_c - 1) pre-conv rows; one workgroup per (b, g) stages them with the m
// new rows, computes a (the sequence conv) for tokens L-k_c+1 .. L+m-1 into
// LDS, then one thread per output forms b = sum_j W[h, i, j, :] . a[t - j]
// on the VALU (one (sequence, group) holds at most a few thousand of them)
// into LDS, and each (new token, head) unit finishes with mix_tail.  All state reads
// finish before the first barrier, so state_out may alias state_in.
template <typename TV, int D>
__global__ __launch_bounds__(256) void convmix_decode_grouped_kernel(
    MixShape s, MixTaps w, const float *__restrict__ dense_q, const float *__restrict__ dense_k,
    const float *__restrict__ qkv, int Lmax, const int *__restrict__ lens, StateOut in,
    StateOut out, float *__restrict__ qout) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int G = s.G, CW = (G + 2) * D, QK = (G + 1) * D;
  const int m = s.T;
  const int ks1 = s.ks - 1, kc1 = s.kc - 1, W = ks1 + kc1;
  const int Wt = W > 0 ? W : 1;          // carried tile rows (one at least, for the shifted value)
  const int R = Wt + m, AR = kc1 + m;
  float *tile = lds;                     // [R][CW]: rows 0..Wt-1 carried, then the new tokens
  float *at = tile + R * CW;             // [AR][QK]: a of tokens L-kc1 .. L+m-1
  float2 *rot = reinterpret_cast<float2 *>(at + AR * QK);   // [m][D/2], then b [m][QK]

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
      v = qkv[(size_t)(b * m + r - Wt) * N + group_col(col, g, G, D, eq, ekv)];
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
  for (int e = tid; e < m * (D / 2); e += 256)
    rot[e] = rope_cs_theta(L + e / (D / 2), s.theta[e % (D / 2)], s.rope_base);
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
  // the a rows of the k_c lags; results to LDS for the per-head tails below
  float *bt = reinterpret_cast<float *>(rot + m * (D / 2));
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
  for (int u0 = 0; u0 < m * (G + 1); u0 += upp) {
    const int unit = u0 + ui;
    const bool active = unit < m * (G + 1);
    const int j = active ? unit / (G + 1) : 0, slot = active ? unit % (G + 1) : 0;
    const f32x4 bv = *reinterpret_cast<const f32x4 *>(bt + j * QK + slot * D + 4 * li);
    float bb[4] = {bv[0], bv[1], bv[2], bv[3]};
    float y[4];
    mix_tail<D>(tile + (Wt + j) * CW + 4 * li, slot, G, s, rot[j * (D / 2) + 2 * li],
                rot[j * (D / 2) + 2 * li + 1], bb, y);
    if (!active) continue;
    if (slot < G) {
      Store4<float>::st(qout + ((size_t)(b * m + j) * s.Hq + g * G + slot) * D + 4 * li, y);
    } else {
      Store4<TV>::st(kc + cache_row(in, b, s.Hkv, g, L + j) * D + 4 * li, y);
    }
  }
  for (int e = tid; e < m * (D / 4); e += 256) {
    const int j = e / (D / 4), c4 = e % (D / 4);
    Store4<TV>::st(vc + cache_row(in, b, s.Hkv, g, L + j) * D + 4 * c4,
                   tile + (Wt + j - shifted) * CW + QK + 4 * c4);
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
  constexpr int TAPS_F = (G + 1) * D * 4 + ((G + 1) * 4 + 3) / 4 * 4;
  constexpr int EPI = (TILE_F + TAPS_F) * 4 + BM * (D / 2) * 8;
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
  float2 *rot = reinterpret_cast<float2 *>(staps + TAPS_F);
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
  load_taps<D>(s, w, g, staps, ctaps);
  for (int e = tid; e < BM * (D / 2); e += 256)
    rot[e] = rope_cs_theta(t0 + e / (D / 2), s.theta[e % (D / 2)], s.rope_base);
  __syncthreads();

  // the mixing of convmix_prefill_kernel on the tile's rows
  constexpr int LPU = D / 4;
  const int upp = 256 / LPU;
  const int li = tid % LPU, ui = tid / LPU;
  for (int slot = 0; slot <= G; ++slot) {
    float stp[4][4], ctp[4];
    lane_taps<D>(staps, ctaps, slot, li, stp, ctp);
    const float qscale = slot < G ? w.tau[g * G + slot] * 1.4426950408889634f : 1.f;
    for (int r = ui; r < BM; r += upp) {
      const int tok = t0 + r;
      float y[4];
      mix_unit<D>(tile, CW, r, slot, G, li, stp, ctp, s, rot[r * (D / 2) + 2 * li],
                  rot[r * (D / 2) + 2 * li + 1], y);
      if (slot < G) {
#pragma unroll
        for (int c = 0; c < 4; ++c) y[c] *= qscale;
        Store4<TQ>::st(q + ((size_t)(b * s.Hq + g * G + slot) * s.Tp + tok) * D + 4 * li, y);
      } else {
        Store4<TQ>::st(k + ((size_t)(b * s.Hkv + g) * s.Tp + tok) * D + 4 * li, y);
      }
    }
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

static size_t mix_lds_bytes(int rows, int G, int D, int TC) {
  const int CW = (G + 2) * D;
  size_t f = (size_t)rows * CW + (size_t)(G + 1) * D * 4 + ((G + 1) * 4 + 3) / 4 * 4;
  return f * 4 + (size_t)TC * (D / 2) * 8;
}

// Tokens per chunk: 32 when the tile fits in LDS, else 16.
static int mix_chunk(int G, int D) { return mix_lds_bytes(32 + HALO, G, D, 32) <= 65536 ? 32 : 16; }

// Whether a thread's share of one chunk's rows fits the prefetch registers;
// otherwise each workgroup handles a single chunk and nothing is prefetched.
static bool mix_prefetch_fits(int G, int D, int TC) {
  const int cpr = (G + 2) * D / 4, rstep = 256 / cpr;
  return (TC + rstep - 1) / rstep <= MIX_PF;
}

bool convmix_decode_fits(int G, int d, int m) {
  return m >= 1 && mix_lds_bytes(3 + m, G, d, m) <= 65536;
}

bool convmix_fits(int G, int d) {
  return (G + 2) * d / 4 <= 256 && mix_lds_bytes(16 + HALO, G, d, 16) <= 65536;
}

template <typename TQ, typename TV, int D>
static hipError_t convmix_prefill_d(const MixShape &s, const MixTaps &w, const float *qkv, TQ *q,
                                    TQ *k, TV *vt, const StateOut &st, const float *r1b,
                                    hipStream_t stream) {
  const int TC = mix_chunk(s.G, D);
  const int nchunks = s.Tp / TC;
  // about 4 chunks per workgroup (the prefetch of chunk i+1 hides behind the
  // mixing of chunk i), at least ~512 workgroups when the work allows
  const int streams = s.B * s.Hkv;
  int cpw = (nchunks / 4 > 0 && mix_prefetch_fits(s.G, D, TC)) ? 4 : 1;
  while (cpw > 1 && (long long)streams * ((nchunks + cpw - 1) / cpw) < 512) --cpw;
  const int nseg = (nchunks + cpw - 1) / cpw;
  const size_t lds = mix_lds_bytes(TC + HALO, s.G, D, TC);
  hipLaunchKernelGGL((convmix_prefill_kernel<TQ, TV, D>), dim3(streams * nseg), dim3(256), lds,
                     stream, s, w, qkv, q, k, vt, st, r1b, TC, nchunks, cpw, nseg);
  return hipGetLastError();
}

template <typename TQ, typename TV>
hipError_t launch_convmix_prefill(const MixShape &s, const MixTaps &w, const float *qkv, TQ *q,
                                  TQ *k, TV *vt, const StateOut &st, hipStream_t stream,
                                  const float *r1b) {
  switch (s.d) {
    case 16: return convmix_prefill_d<TQ, TV, 16>(s, w, qkv, q, k, vt, st, r1b, stream);
    case 32: return convmix_prefill_d<TQ, TV, 32>(s, w, qkv, q, k, vt, st, r1b, stream);
    case 64: return convmix_prefill_d<TQ, TV, 64>(s, w, qkv, q, k, vt, st, r1b, stream);
    case 128: return convmix_prefill_d<TQ, TV, 128>(s, w, qkv, q, k, vt, st, r1b, stream);
  }
  return hipErrorInvalidValue;
}

template <typename TV, int D>
static hipError_t convmix_decode_d(const MixShape &s, const MixTaps &w, const float *qkv, int L,
                                   const int *lens,
                                   const StateOut &in, const StateOut &out, float *q,
                                   hipStream_t stream) {
  const size_t lds = mix_lds_bytes(3 + s.T, s.G, D, s.T);
  hipLaunchKernelGGL((convmix_decode_kernel<TV, D>), dim3(s.B * s.Hkv), dim3(256), lds, stream, s,
                     w, qkv, L, lens, in, out, q);
  return hipGetLastError();
}

template <typename TV>
hipError_t launch_convmix_decode(const MixShape &s, const MixTaps &w, const float *qkv, int L,
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
          (size_t)m * (G + 1) * D) * 4 + (size_t)m * (D / 2) * 8;
}

bool convmix_decode_grouped_fits(int G, int d, int m, int ks, int kc) {
  return m >= 1 && decode_grouped_lds_bytes(G, d, m, ks, kc) <= 65536;
}

template <typename TV, int D>
static hipError_t convmix_decode_grouped_d(const MixShape &s, const MixTaps &w, const float *dq,
                                           const float *dk, const float *qkv, int L,
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
                                         const float *dense_k, const float *qkv, int L,
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
                                                        const float *, const float *, const float *,
                                                        int, const int *, const StateOut &,
                                                        const StateOut &, float *, hipStream_t);
template hipError_t launch_convmix_decode_grouped<float>(const MixShape &, const MixTaps &,
                                                         const float *, const float *, const float *,
                                                         int, const int *, const StateOut &,
                                                         const StateOut &, float *, hipStream_t);

template hipError_t launch_convmix_prefill<f16, bf16>(const MixShape &, const MixTaps &,
                                                      const float *, f16 *, f16 *, bf16 *,
                                                      const StateOut &, hipStream_t, const float *);
template hipError_t launch_convmix_prefill<bf16, bf16>(const MixShape &, const MixTaps &,
                                                       const float *, bf16 *, bf16 *, bf16 *,
                                                       const StateOut &, hipStream_t, const float *);
template hipError_t launch_convmix_prefill<float, float>(const MixShape &, const MixTaps &,
                                                         const float *, float *, float *, float *,
                                                         const StateOut &, hipStream_t, const float *);
template hipError_t launch_convmix_decode<bf16>(const MixShape &, const MixTaps &, const float *,
                                                int, const int *, const StateOut &, const StateOut &, float *,
                                                hipStream_t);
template hipError_t launch_convmix_decode<float>(const MixShape &, const MixTaps &, const float *,
                                                int, const int *, const StateOut &, const StateOut &, float *,
                                                 hipStream_t);

}  // namespace cca
