// Decode attention over the latent KV cache (gfx950, HBM bound).
//
// One new query token per sequence attends to the Lk = L + 1 cached latent
// keys of its kv head; the G query heads of a group read each K/V row once.
// The cache grows with the sequence and decode is limited by memory
// bandwidth [GS-EN "1. Problem Statement"]; CCGQA's shared latent kv heads
// make that cache small [GS-EN "2. Methodology" / "Extension: CCGQA"].
//
// Design (MI355X): split-KV.  A workgroup (4 waves) streams one chunk of
// keys of one (sequence, kv head, up to 4 query heads).  A lane reads 16
// contiguous bytes of a K row and of the matching V row, so one wave load
// instruction covers whole consecutive 128-byte rows (coalesced); the dot
// products are reduced across the d/8 lanes of a row, and each lane keeps its
// own online-softmax state (max, sum, unnormalised output of its 8 channels)
// over blocks of NB keys, so the rescale costs one exp per block.  The lane
// states are merged with cross-lane exchanges, the 4 waves through LDS, and
// each chunk leaves (m, l, o) in fp32 scratch.  A second small kernel merges
// the chunks with the log-sum-exp rule and writes the latent output.
#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

static constexpr int DEC_CHUNK = 1024;   // keys per workgroup
static constexpr int NB = 4;             // keys per lane per softmax block

int decode_chunk_keys(int) { return DEC_CHUNK; }

size_t decode_partial_floats(int B, int Hq, int d, int Lk) {
  const int nch = (Lk + DEC_CHUNK - 1) / DEC_CHUNK;
  return (size_t)B * Hq * nch * (d + 2);
}

template <typename TV> struct Row16;
template <> struct Row16<bf16> {
  static constexpr int E = 8;
  __device__ __forceinline__ static void cvt(u32x4 r, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
};
template <> struct Row16<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static void cvt(u32x4 r, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
  }
};

__device__ __forceinline__ float safe_exp2_diff(float a, float m) {
  return a == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(a - m);
}

template <typename TV, int D, int GH>
__global__ __launch_bounds__(256) void attn_decode_kernel(const float *__restrict__ q,
                                                          const float *__restrict__ tau,
                                                          const TV *__restrict__ kc,
                                                          const TV *__restrict__ vc, int cap,
                                                          int Lk, int Hq, int Hkv, int G,
                                                          int nquad, int nch,
                                                          float *__restrict__ part) {
  constexpr int E = Row16<TV>::E;          // elements per 16-byte lane load
  constexpr int DS = D / E;                // lanes per key row
  constexpr int KPS = 64 / DS;             // keys per wave load
  __shared__ float red[4][GH][D + 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int id = blockIdx.x;
  const int c = id % nch; id /= nch;
  const int quad = id % nquad; id /= nquad;
  const int g = id % Hkv, b = id / Hkv;
  const int h0 = g * G + quad * GH;
  const int seg = lane % DS, ksub = lane / DS;

  float qv[GH][E];
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
    const float sc = tau[h0 + hh] * 1.4426950408889634f;
#pragma unroll
    for (int e = 0; e < E; ++e) qv[hh][e] = q[(size_t)(b * Hq + h0 + hh) * D + seg * E + e] * sc;
  }

  const int kbeg = c * DEC_CHUNK;
  const int kend = min(kbeg + DEC_CHUNK, Lk);
  const TV *kb = kc + (size_t)(b * Hkv + g) * cap * D;
  const TV *vb = vc + (size_t)(b * Hkv + g) * cap * D;

  float m[GH], l[GH], acc[GH][E];
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[hh][e] = 0.f;
  }

  const int per_iter = 4 * NB * KPS;
  for (int base = kbeg; base < kend; base += per_iter) {
    float kf[NB][E], vf[NB][E];
    bool valid[NB];
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      const int key = base + (wave * NB + s) * KPS + ksub;
      valid[s] = key < kend;
      const int kk = valid[s] ? key : kbeg;
      Row16<TV>::cvt(ld16(kb + (size_t)kk * D + seg * E), kf[s]);
      Row16<TV>::cvt(ld16(vb + (size_t)kk * D + seg * E), vf[s]);
    }
    float sc[NB][GH];
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot = fmaf(qv[hh][e], kf[s][e], dot);
#pragma unroll
        for (int o = DS / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
        sc[s][hh] = valid[s] ? dot : -INFINITY;
      }
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      float mb = sc[0][hh];
#pragma unroll
      for (int s = 1; s < NB; ++s) mb = fmaxf(mb, sc[s][hh]);
      const float m_new = fmaxf(m[hh], mb);
      if (m_new == -INFINITY) continue;          // no valid key seen yet by this lane
      const float alpha = safe_exp2_diff(m[hh], m_new);
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[hh][e] *= alpha;
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const float p = safe_exp2_diff(sc[s][hh], m_new);
        l[hh] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = fmaf(p, vf[s][e], acc[hh][e]);
      }
      m[hh] = m_new;
    }
  }

  // merge the lanes that share a channel segment (different keys)
#pragma unroll
  for (int o = DS; o < 64; o <<= 1) {
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      const float mo = __shfl_xor(m[hh], o, 64);
      const float lo = __shfl_xor(l[hh], o, 64);
      const float mn = fmaxf(m[hh], mo);
      const float a = mn == -INFINITY ? 0.f : safe_exp2_diff(m[hh], mn);
      const float bo = mn == -INFINITY ? 0.f : safe_exp2_diff(mo, mn);
      l[hh] = l[hh] * a + lo * bo;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float ao = __shfl_xor(acc[hh][e], o, 64);
        acc[hh][e] = acc[hh][e] * a + ao * bo;
      }
      m[hh] = mn;
    }
  }
  if (ksub == 0) {
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      if (seg == 0) {
        red[wave][hh][0] = m[hh];
        red[wave][hh][1] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) red[wave][hh][2 + seg * E + e] = acc[hh][e];
    }
  }
  __syncthreads();
  // merge the 4 waves and write the chunk's partial state
  for (int e = tid; e < GH * D; e += 256) {
    const int hh = e / D, dd = e % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][hh][0]);
    float ll = 0.f, oo = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = safe_exp2_diff(red[w][hh][0], mm);
      ll += red[w][hh][1] * f;
      oo += red[w][hh][2 + dd] * f;
    }
    float *dst = part + ((size_t)(b * Hq + h0 + hh) * nch + c) * (D + 2);
    dst[2 + dd] = oo;
    if (dd == 0) {
      dst[0] = mm;
      dst[1] = ll;
    }
  }
}

// o[b, h*D + dd] = sum_c 2^(m_c - M) o_c[dd] / sum_c 2^(m_c - M) l_c
template <typename TV, int D>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(const float *__restrict__ part,
                                                                 int nch, int Hq,
                                                                 TV *__restrict__ o) {
  const int bh = blockIdx.x;   // b * Hq + h
  const float *p = part + (size_t)bh * nch * (D + 2);
  float mm = -INFINITY;
  for (int c = 0; c < nch; ++c) mm = fmaxf(mm, p[c * (D + 2)]);
  for (int dd = threadIdx.x; dd < D; dd += 64) {
    float ll = 0.f, oo = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float f = safe_exp2_diff(p[c * (D + 2)], mm);
      ll += p[c * (D + 2) + 1] * f;
      oo += p[c * (D + 2) + 2 + dd] * f;
    }
    o[(size_t)bh * D + dd] = from_f32<TV>(oo / ll);
  }
}

static int group_heads(int G) {
  for (int gh = 4; gh >= 1; --gh)
    if (G % gh == 0) return gh;
  return 1;
}

template <typename TV, int D, int GH>
static hipError_t dec_dgh(const MixShape &s, const float *q, const TV *kc, const TV *vc, int cap,
                          int Lk, const float *tau, float *part, TV *o, hipStream_t stream) {
  const int nch = (Lk + DEC_CHUNK - 1) / DEC_CHUNK;
  const int nquad = s.G / GH;
  hipLaunchKernelGGL((attn_decode_kernel<TV, D, GH>), dim3(nch * nquad * s.B * s.Hkv), dim3(256),
                     0, stream, q, tau, kc, vc, cap, Lk, s.Hq, s.Hkv, s.G, nquad, nch, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_combine_kernel<TV, D>), dim3(s.B * s.Hq), dim3(64), 0, stream,
                     part, nch, s.Hq, o);
  return hipGetLastError();
}

template <typename TV, int D>
static hipError_t dec_d(const MixShape &s, const float *q, const TV *kc, const TV *vc, int cap,
                        int Lk, const float *tau, float *part, TV *o, hipStream_t stream) {
  switch (group_heads(s.G)) {
    case 4: return dec_dgh<TV, D, 4>(s, q, kc, vc, cap, Lk, tau, part, o, stream);
    case 3: return dec_dgh<TV, D, 3>(s, q, kc, vc, cap, Lk, tau, part, o, stream);
    case 2: return dec_dgh<TV, D, 2>(s, q, kc, vc, cap, Lk, tau, part, o, stream);
    default: return dec_dgh<TV, D, 1>(s, q, kc, vc, cap, Lk, tau, part, o, stream);
  }
}

template <typename TV>
hipError_t launch_attention_decode(const MixShape &s, const float *q, const TV *k_cache,
                                   const TV *v_cache, int capacity, int Lk, const float *tau,
                                   float *part, TV *o, hipStream_t stream) {
  switch (s.d) {
    case 16: return dec_d<TV, 16>(s, q, k_cache, v_cache, capacity, Lk, tau, part, o, stream);
    case 32: return dec_d<TV, 32>(s, q, k_cache, v_cache, capacity, Lk, tau, part, o, stream);
    case 64: return dec_d<TV, 64>(s, q, k_cache, v_cache, capacity, Lk, tau, part, o, stream);
    case 128: return dec_d<TV, 128>(s, q, k_cache, v_cache, capacity, Lk, tau, part, o, stream);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_attention_decode<bf16>(const MixShape &, const float *, const bf16 *,
                                                  const bf16 *, int, int, const float *, float *,
                                                  bf16 *, hipStream_t);
template hipError_t launch_attention_decode<float>(const MixShape &, const float *, const float *,
                                                   const float *, int, int, const float *,
                                                   float *, float *, hipStream_t);

}  // namespace cca
