// Causal softmax attention inside the latent heads (gfx950, MFMA bound).
//
// o[t, h] = sum_{u <= t} softmax_u(tau_h <q(t, h), k(u, g)>) v(u, g), g = h / G
// [GS-EN "2. Methodology" / Latent Space Operations and "Extension: CCGQA";
//  GS-EN "3. Key Contributions" describes a fused kernel with an online
//  softmax in the style of Flash Attention.]
//
// Design (MI355X):
//  * One workgroup = 4 waves = 128 query rows: the query heads of one kv head
//    that share K/V tiles are packed side by side (hq = gcd(G, 4) heads x
//    128/hq positions), so each K/V tile staged in LDS serves every head of
//    the group that the block holds.
//  * Each wave owns 32 query rows and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16 (keys on M, queries on N).  In that accumulator
//    layout every lane holds 16 scores of ONE query (keys 8j+4h+i), so the
//    softmax row statistics need a single cross-half exchange and the
//    probabilities are already in the B-operand layout of O^T = V^T P^T: no
//    LDS round trip for P.  The O^T accumulator again holds one query per
//    lane, so the online-softmax rescale and the final 1/l stay in-lane.
//  * K tiles [64 keys][d] and transposed V tiles [d][64 keys] are double
//    buffered in LDS with a 16-byte XOR swizzle; the value tile's key order
//    is permuted inside 16-key groups (bits 2 and 3 swapped, done once by the
//    mixing kernel) so one lane's 8 keys are contiguous.
//  * tau_h * log2(e) scales the fp32 scores, exp2 is the native v_exp_f32.
//  * Causal blocks: tiles above the diagonal are skipped per wave; the heavy
//    (late) position blocks are dispatched first.
#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

static constexpr int KB = 64;   // keys per tile

template <typename TQ, typename TV, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const TQ *__restrict__ q,
                                                       const TQ *__restrict__ k,
                                                       const TV *__restrict__ vt,
                                                       const float *__restrict__ tau,
                                                       TV *__restrict__ o, int B, int T, int Tp,
                                                       int Hq, int Hkv, int G, int hq, int nsub,
                                                       int npb) {
  typedef Mfma32<TQ> MQ;
  typedef Mfma32<TV> MV;
  constexpr int KSQ = MQ::KS, KSV = MV::KS;
  constexpr int DP = D < 32 ? 32 : D;                 // V^T rows (padded to one MFMA tile)
  constexpr int ND = DP / 32;                         // O^T row blocks of 32
  constexpr int KROW = D * (int)sizeof(TQ);           // bytes per K tile row
  constexpr int KCPR = KROW / 16;
  constexpr int VROW = KB * (int)sizeof(TV);          // bytes per V^T tile row
  constexpr int VCPR = VROW / 16;
  constexpr int KTILE = KB * KROW, VTILE = DP * VROW;
  constexpr int K_CH = (KB * KCPR + 255) / 256;       // 16-byte chunks per thread
  constexpr int V_CH = (D * VCPR + 255) / 256;
  constexpr int QC = D / (2 * KSQ);                   // QK^T contraction chunks
  constexpr int PC = 16 / KSV;                        // P*V chunks per 32-key half

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * (KTILE + VTILE)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int pos_per = 128 / hq;

  // heavy-first: logical block order walks position blocks from the end
  int id = blockIdx.x;
  const int rest = B * Hkv * nsub;
  const int pb = npb - 1 - id / rest;
  id %= rest;
  const int sub = id % nsub;
  id /= nsub;
  const int g = id % Hkv, b = id / Hkv;

  const int hslot = wave % hq, rchunk = wave / hq;
  const int h = g * G + sub * hq + hslot;
  const int blk0 = pb * pos_per;
  const int p0 = blk0 + 32 * rchunk;                  // first query row of this wave
  const int qpos = p0 + l32;                          // this lane's query
  const int last_row = min(blk0 + pos_per, T) - 1;    // last valid query of the block
  const int ntiles = last_row / KB + 1;
  const int wave_last = p0 + 31;

  const float scale = tau[h] * 1.4426950408889634f;

  // zero the padding rows of the V^T tiles (d < 32)
  if (D < DP) {
    for (int e = tid; e < 2 * (DP - D) * VROW / 16; e += 256) {
      const int buf = e / ((DP - D) * VROW / 16), c = e % ((DP - D) * VROW / 16);
      st16(smem + buf * (KTILE + VTILE) + KTILE + D * VROW + c * 16, zero_u32x4());
    }
  }

  // Q fragments of this lane's query (B operand of S^T = K Q^T)
  typename MQ::frag qf[QC];
  {
    const TQ *qrow = q + ((size_t)(b * Hq + h) * Tp + qpos) * D;
#pragma unroll
    for (int c = 0; c < QC; ++c) qf[c] = load_frag<TQ>(qrow + c * 2 * KSQ + hl * KSQ);
  }

  const TQ *kbase = k + (size_t)(b * Hkv + g) * Tp * D;
  const TV *vbase = vt + (size_t)(b * Hkv + g) * D * Tp;
  u32x4 rk[K_CH], rv[V_CH];

  auto gload = [&](int kt) {
    const int k0 = kt * KB;
#pragma unroll
    for (int r = 0; r < K_CH; ++r) {
      const int c = tid + 256 * r;
      if (c < KB * KCPR) rk[r] = ld16(reinterpret_cast<const unsigned char *>(kbase + (size_t)k0 * D) + c * 16);
    }
#pragma unroll
    for (int r = 0; r < V_CH; ++r) {
      const int c = tid + 256 * r;
      if (c < D * VCPR) {
        const int row = c / VCPR, ch = c % VCPR;
        rv[r] = ld16(reinterpret_cast<const unsigned char *>(vbase + (size_t)row * Tp + k0) + ch * 16);
      }
    }
  };
  auto lstore = [&](int buf) {
    unsigned char *sk = smem + buf * (KTILE + VTILE);
    unsigned char *sv = sk + KTILE;
#pragma unroll
    for (int r = 0; r < K_CH; ++r) {
      const int c = tid + 256 * r;
      if (c < KB * KCPR) {
        const int row = c / KCPR, ch = c % KCPR;
        st16(sk + row * KROW + swz(row, ch * 16, KCPR), rk[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < V_CH; ++r) {
      const int c = tid + 256 * r;
      if (c < D * VCPR) {
        const int row = c / VCPR, ch = c % VCPR;
        st16(sv + row * VROW + swz(row, ch * 16, VCPR), rv[r]);
      }
    }
  };

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
    const int k0 = kt * KB;
    if (k0 <= wave_last) {
      const unsigned char *sk = smem + cur * (KTILE + VTILE);
      const unsigned char *sv = sk + KTILE;
      // S^T for keys k0 .. k0+63 as two 32-key halves
      f32x16 s[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        s[hf] = zero16();
        const int row = hf * 32 + l32;
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          const int kb = (c * 2 * KSQ + hl * KSQ) * (int)sizeof(TQ);
          typename MQ::frag kf = load_frag<TQ>(reinterpret_cast<const TQ *>(sk + row * KROW + swz(row, kb, KCPR)));
          s[hf] = MQ::mma(kf, qf[c], s[hf]);
        }
      }
      // scale, causal mask, row max
      const bool diag = k0 + KB - 1 > p0;
      float mx = -INFINITY;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          float v = s[hf][a] * scale;
          if (diag) {
            const int key = k0 + hf * 32 + 8 * (a >> 2) + 4 * hl + (a & 3);
            if (key > qpos) v = -INFINITY;
          }
          s[hf][a] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const float p = __builtin_amdgcn_exp2f(s[hf][a] - m_new);
          s[hf][a] = p;
          psum += p;
        }
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < ND; ++i)
#pragma unroll
        for (int a = 0; a < 16; ++a) acc[i][a] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int cc = 0; cc < PC; ++cc) {
          float pv[KSV];
#pragma unroll
          for (int sl = 0; sl < KSV; ++sl) pv[sl] = s[hf][KSV * cc + sl];
          const typename MV::frag pf = pack_frag<TV>(pv);
          // first key of this lane's k-slots, in the permuted tile order
          const int a0 = KSV * cc;
          const int key_rel = 8 * (a0 >> 2) + 4 * hl + (a0 & 3);
          const int kb = (hf * 32 + vt_perm(key_rel)) * (int)sizeof(TV);
#pragma unroll
          for (int i = 0; i < ND; ++i) {
            const int row = i * 32 + l32;
            typename MV::frag vf = load_frag<TV>(reinterpret_cast<const TV *>(sv + row * VROW + swz(row, kb, VCPR)));
            acc[i] = MV::mma(vf, pf, acc[i]);
          }
        }
    }
    if (kt + 1 < ntiles) lstore(cur ^ 1);
    __syncthreads();
  }

  if (qpos >= T) return;
  const float inv_l = 1.f / l_run;
  TV *orow = o + ((size_t)(b * T + qpos)) * (Hq * D) + h * D;
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dd = i * 32 + 8 * j + 4 * hl;
      if (dd >= D) continue;
      TV v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = from_f32<TV>(acc[i][4 * j + e] * inv_l);
      if constexpr (sizeof(TV) == 2) {
        *reinterpret_cast<u32x2 *>(orow + dd) = *reinterpret_cast<u32x2 *>(v4);
      } else {
        *reinterpret_cast<u32x4 *>(orow + dd) = *reinterpret_cast<u32x4 *>(v4);
      }
    }
}

static int gcd_int(int a, int b) {
  while (b) { int t = a % b; a = b; b = t; }
  return a;
}

template <typename TQ, typename TV, int D>
static hipError_t attn_d(const MixShape &s, const TQ *q, const TQ *k, const TV *vt,
                         const float *tau, TV *o, hipStream_t stream) {
  const int hq = gcd_int(s.G, 4);
  const int nsub = s.G / hq;
  const int pos_per = 128 / hq;
  const int npb = (s.T + pos_per - 1) / pos_per;
  const int grid = npb * s.B * s.Hkv * nsub;
  hipLaunchKernelGGL((attn_fwd_kernel<TQ, TV, D>), dim3(grid), dim3(256), 0, stream, q, k, vt, tau,
                     o, s.B, s.T, s.Tp, s.Hq, s.Hkv, s.G, hq, nsub, npb);
  return hipGetLastError();
}

template <typename TQ, typename TV>
hipError_t launch_attention_prefill(const MixShape &s, const TQ *q, const TQ *k, const TV *vt,
                                    const float *tau, TV *o, hipStream_t stream) {
  switch (s.d) {
    case 16: return attn_d<TQ, TV, 16>(s, q, k, vt, tau, o, stream);
    case 32: return attn_d<TQ, TV, 32>(s, q, k, vt, tau, o, stream);
    case 64: return attn_d<TQ, TV, 64>(s, q, k, vt, tau, o, stream);
    case 128: return attn_d<TQ, TV, 128>(s, q, k, vt, tau, o, stream);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_attention_prefill<f16, bf16>(const MixShape &, const f16 *, const f16 *,
                                                        const bf16 *, const float *, bf16 *,
                                                        hipStream_t);
template hipError_t launch_attention_prefill<bf16, bf16>(const MixShape &, const bf16 *,
                                                         const bf16 *, const bf16 *, const float *,
                                                         bf16 *, hipStream_t);
template hipError_t launch_attention_prefill<float, float>(const MixShape &, const float *,
                                                           const float *, const float *,
                                                           const float *, float *, hipStream_t);

}  // namespace cca
