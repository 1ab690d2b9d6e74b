// Grouped reading of the channel convolution (gfx950): per head h, a causal
// convolution over tokens whose taps are dense d x d matrices, one per lag,
// applied to the sequence-conv output a:
//   b[t, h, i] = sum_{j < k_c} sum_c W[h, i, j, c] * a[t - j, h, c]
// [GS-EN "2. Methodology" / Convolutional Mixing: 1-D convolutions across the
//  sequence and the channel dimensions; this is the reading that mixes the
//  channels of a head densely, next to the default per-head filter that
//  slides along the channel index.]
//
// Prefill: a dense contraction of k_c * d inputs into d outputs per (token,
// head), so it runs on MFMA.  One workgroup per (sequence, head, 128 tokens)
// recomputes a (the k_s-tap sequence conv of the down-projection output,
// fp16 in bf16 mode) for its tokens and the k_c - 1 before them into LDS as fp16, stages
// the head's W as fp16 rows [i][lag-major, channel], and multiplies: row t of
// the A operand is the k_c consecutive a rows t-k_c+1 .. t, read straight
// from the tile (overlapping rows, no copy).  v_mfma_f32_32x32x16_f16, fp32
// accumulation; b goes to HBM in fp32 for the mixing kernel, which adds the
// q-k-mean skip, normalises and rotates.  The fp32 validation mode runs the
// same tile on the VALU in fp32.
#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

static constexpr int GC_RB = 128;   // tokens per workgroup (4 waves x 32)

template <int D>
struct GcTile {
  static constexpr int DP = D < 32 ? 32 : D;   // output rows of W, padded to one MFMA tile
  static constexpr int KMAX = 4 * D;           // k_c * d at k_c = 4
  static constexpr int AROWS = GC_RB + 3;
};

template <int D, bool F32>
__global__ __launch_bounds__(256) void grouped_conv_prefill_kernel(MixShape s, MixTaps w,
                                                                   const float *__restrict__ dense_q,
                                                                   const float *__restrict__ dense_k,
                                                                   const void *__restrict__ qkv_v,
                                                                   float *__restrict__ outb) {
  typedef GcTile<D> TL;
  typedef typename std::conditional<F32, float, f16>::type TE;
  typedef TE TI;   // the down-projection output: fp32 in fp32 mode, fp16 in bf16 mode
  const TI *qkv = reinterpret_cast<const TI *>(qkv_v);
  constexpr int DP = TL::DP;
  // LDS rows padded by 16 bytes (fp16) so that lanes reading the same
  // columns of consecutive rows spread over the banks
  constexpr int APAD = F32 ? D : D + 8;
  constexpr int WPAD = F32 ? DP : TL::KMAX + 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char gc_smem[];
  TE *a_lds = reinterpret_cast<TE *>(gc_smem);                    // [AROWS][APAD]
  TE *w_lds = a_lds + TL::AROWS * APAD;                           // fp16: [DP][WPAD]; fp32: [K][DP]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = s.Hq + s.Hkv;
  const int ntb = (s.T + GC_RB - 1) / GC_RB;
  int id = blockIdx.x;
  const int tb = id % ntb;
  id /= ntb;
  const int hh = id % H, b = id / H;
  const bool is_q = hh < s.Hq;
  const int g = is_q ? hh / s.G : hh - s.Hq;
  const int eq = s.Hq * D, ekv = s.Hkv * D, N = eq + 2 * ekv;
  const int colbase = is_q ? hh * D : eq + g * D;   // in the qkv row and in b rows (width e_q + e_kv)
  const int kc = s.kc, ks = s.ks, KD = kc * D;
  const int t0 = tb * GC_RB;
  const int arows = GC_RB + kc - 1;                  // a of tokens t0-kc+1 .. t0+GC_RB-1
  const float *dense = is_q ? dense_q + (size_t)hh * D * kc * D : dense_k + (size_t)g * D * kc * D;
  const float *seqw = is_q ? w.q_seq + (size_t)hh * D * ks : w.k_seq + (size_t)g * D * ks;
  const TI *u0 = qkv + (size_t)b * s.T * N + colbase;

  // W: column K = jp * d + c of output row i holds W[h, i, kc-1-jp, c] (A
  // row t, column jp * d + c, is a[t - kc + 1 + jp, c]).  Four channels per
  // item; every load of a thread is issued before the first store.
  {
    constexpr int NW4 = (DP * TL::KMAX / 4 + 255) / 256;   // items per thread at k_c = 4
    const int kd4 = KD / 4, nw4 = DP * kd4;
    f32x4 wv[NW4];
#pragma unroll
    for (int k = 0; k < NW4; ++k) {
      const int e = tid + 256 * k;
      wv[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (e < nw4) {
        const int i = e / kd4, K = 4 * (e - i * kd4), jp = K / D, c = K % D;
        if (i < D) wv[k] = *reinterpret_cast<const f32x4 *>(dense + ((size_t)i * kc + (kc - 1 - jp)) * D + c);
      }
    }
#pragma unroll
    for (int k = 0; k < NW4; ++k) {
      const int e = tid + 256 * k;
      if (e < nw4) {
        const int i = e / kd4, K = 4 * (e - i * kd4);
        if constexpr (F32) {
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) w_lds[(K + cc) * DP + i] = wv[k][cc];
        } else {
          *reinterpret_cast<f16x4 *>(w_lds + i * WPAD + K) =
              f16x4{(f16)wv[k][0], (f16)wv[k][1], (f16)wv[k][2], (f16)wv[k][3]};
        }
      }
    }
  }
  // a rows (zero outside [0, T)).  A thread always owns the same 4 channels
  // (256 is a multiple of d / 4), so its taps load once; the pre-conv rows of
  // three items at a time are in flight together.
  {
    const int c0 = 4 * (tid % (D / 4)), r0 = tid / (D / 4);
    constexpr int RSTEP = 256 / (D / 4);
    float tp[4][4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int j = 0; j < 4; ++j) tp[cc][j] = j < ks ? seqw[(c0 + cc) * ks + j] : 0.f;
    constexpr int NA = (TL::AROWS + RSTEP - 1) / RSTEP, BATCH = 3;
#pragma unroll
    for (int k0 = 0; k0 < NA; k0 += BATCH) {
      f32x4 u[BATCH][4];
#pragma unroll
      for (int kb = 0; kb < BATCH; ++kb) {
        const int r = r0 + RSTEP * (k0 + kb), t = t0 - (kc - 1) + r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = k0 + kb < NA && r < arows && j < ks && t - j >= 0 && t < s.T;
          u[kb][j] = ok ? ld4f<TI>(u0 + (size_t)(t - j) * N + c0) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int kb = 0; kb < BATCH; ++kb) {
        const int r = r0 + RSTEP * (k0 + kb);
        if (k0 + kb >= NA || r >= arows) continue;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc = fmaf(tp[cc][j], u[kb][j][cc], acc);
          a_lds[r * APAD + c0 + cc] = (TE)acc;
        }
      }
    }
  }
  __syncthreads();

  float *orow = outb + (size_t)b * s.T * (eq + ekv) + colbase;
  if constexpr (!F32) {
    // wave w: tokens t0 + 32w .. +31, all d outputs (DP / 32 tiles)
    constexpr int NT = DP / 32;
    const int l32 = lane & 31, hl = lane >> 5;
    f32x16 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = zero16();
    const int row = wave * 32 + l32;
    for (int k0 = 0; k0 < KD; k0 += 16) {
      const int K = k0 + 8 * hl, jp = K / D, c = K % D;
      const f16x8 af = *reinterpret_cast<const f16x8 *>(a_lds + (row + jp) * APAD + c);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const f16x8 bf = *reinterpret_cast<const f16x8 *>(w_lds + (n * 32 + l32) * WPAD + K);
        acc[n] = Mfma32<f16>::mma(af, bf, acc[n]);
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int i = n * 32 + l32;
      if (i >= D) continue;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int t = t0 + wave * 32 + 8 * (a >> 2) + 4 * hl + (a & 3);
        if (t < s.T) orow[(size_t)t * (eq + ekv) + i] = acc[n][a];
      }
    }
  } else {
    // thread: output channel i = tid % D of rows tid / D + (256 / D) * k
    constexpr int RSTEP = 256 / D, NR = GC_RB / RSTEP;
    const int i = tid % D, r0 = tid / D;
    float acc[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] = 0.f;
    for (int K = 0; K < KD; ++K) {
      const int jp = K / D, c = K % D;
      const float wv = w_lds[K * DP + i];
#pragma unroll
      for (int k = 0; k < NR; ++k) acc[k] = fmaf(wv, a_lds[(r0 + RSTEP * k + jp) * APAD + c], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int t = t0 + r0 + RSTEP * k;
      if (t < s.T) orow[(size_t)t * (eq + ekv) + i] = acc[k];
    }
  }
}

template <int D, bool F32>
static size_t gc_lds_bytes() {
  typedef GcTile<D> TL;
  constexpr int APAD = F32 ? D : D + 8;
  constexpr int WPAD = F32 ? TL::DP : TL::KMAX + 8;
  const size_t es = F32 ? 4 : 2;
  return es * ((size_t)TL::AROWS * APAD + (F32 ? (size_t)TL::KMAX * TL::DP : (size_t)TL::DP * WPAD));
}

bool grouped_conv_supported(int d, bool f32) {
  if (d != 16 && d != 32 && d != 64) return false;
  const size_t lds = f32 ? (d == 16 ? gc_lds_bytes<16, true>() : d == 32 ? gc_lds_bytes<32, true>() : gc_lds_bytes<64, true>())
                         : (d == 16 ? gc_lds_bytes<16, false>() : d == 32 ? gc_lds_bytes<32, false>() : gc_lds_bytes<64, false>());
  return lds <= 160 * 1024;
}

template <int D, bool F32>
static hipError_t gc_launch(const MixShape &s, const MixTaps &w, const float *dq, const float *dk,
                            const void *qkv, float *outb, hipStream_t stream) {
  const size_t lds = gc_lds_bytes<D, F32>();
  if (lds > 65536) {   // above the default dynamic LDS limit (the fp32 mode); set on every call,
                       // so each device the library runs on gets it
    hipError_t e = hipFuncSetAttribute((const void *)grouped_conv_prefill_kernel<D, F32>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int ntb = (s.T + GC_RB - 1) / GC_RB;
  const long long grid = (long long)s.B * (s.Hq + s.Hkv) * ntb;
  if (grid >= (1ll << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_conv_prefill_kernel<D, F32>), dim3((unsigned)grid), dim3(256), lds,
                     stream, s, w, dq, dk, qkv, outb);
  return hipGetLastError();
}

hipError_t launch_grouped_conv_prefill(const MixShape &s, const MixTaps &w, const float *dense_q,
                                       const float *dense_k, const void *qkv, float *outb,
                                       bool f32, hipStream_t stream) {
  if (s.kc < 1 || s.kc > 4 || s.ks < 1 || s.ks > 4) return hipErrorInvalidValue;
  switch (s.d) {
    case 16: return f32 ? gc_launch<16, true>(s, w, dense_q, dense_k, qkv, outb, stream)
                        : gc_launch<16, false>(s, w, dense_q, dense_k, qkv, outb, stream);
    case 32: return f32 ? gc_launch<32, true>(s, w, dense_q, dense_k, qkv, outb, stream)
                        : gc_launch<32, false>(s, w, dense_q, dense_k, qkv, outb, stream);
    case 64: return f32 ? gc_launch<64, true>(s, w, dense_q, dense_k, qkv, outb, stream)
                        : gc_launch<64, false>(s, w, dense_q, dense_k, qkv, outb, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace cca
