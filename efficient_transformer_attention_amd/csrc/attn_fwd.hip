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
//  * K tiles [64 keys][d] and transposed V tiles [d][64 keys] (32 keys when
//    d = 128) are staged in LDS with a 16-byte XOR swizzle; the value tile's key order
//    is permuted inside 16-key groups (bits 2 and 3 swapped, done once by the
//    mixing kernel) so one lane's 8 keys are contiguous.
//  * The mixing kernel stores q already scaled by tau_h * log2(e), so the
//    scores come out of the MFMA in the exp2 domain (native v_exp_f32).
//  * K/V^T tiles travel HBM -> LDS by buffer_load ... lds (no register
//    staging): every lane fetches the logical chunk that belongs at its
//    physical slot of the swizzled tile.  A ring of four tiles: while a wave
//    runs the softmax and P*V of tile j it has already issued the QK^T MFMAs
//    of tile j+1, and tiles j+2 and j+3 are in flight; one barrier per tile.
//  * With the L2 norm on, |q_hat| <= 1 and |k_hat| <= 1, so every exp2-domain
//    logit lies in [-c_h, c_h] with c_h = tau_h * log2(e).  Softmax is
//    unchanged by a constant shift, so for c_h <= 60 the kernel subtracts c_h
//    instead of the running row maximum: 2^(s - c_h) stays within
//    [2^-120, ~1], normal in fp32 and bf16, and no row maximum, rescale or
//    cross-lane exchange is needed.  The shift enters as the MFMA's initial
//    accumulator, so the probabilities are one v_exp_f32 away from the
//    product.  Otherwise the usual online softmax runs: the rescale of O runs
//    only when some row's running max grew (a wave-uniform vote).
//  * The row sums add the bf16-rounded probabilities that the P*V product
//    consumes (v_dot2_f32_bf16); each half-wave keeps its own partial sum
//    until the end.
//  * Causal blocks: a workgroup walks the key tiles up to its last query;
//    only tiles that reach past a wave's first query are masked (tiles past
//    its last query come out fully masked and add nothing), and the heavy
//    (late) position blocks are dispatched first.
#include <type_traits>

#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

// Keys per tile: 64 when the ring of four K/V^T tiles fits in 64 KiB of LDS
// (two workgroups per CU), else 32.
template <typename TQ, typename TV, int D> struct AttnTile {
  static constexpr int NBUF = 4;
  static constexpr int DP = D < 32 ? 32 : D;
  static constexpr int bytes(int kb) { return kb * D * (int)sizeof(TQ) + DP * kb * (int)sizeof(TV); }
  static constexpr int KB = NBUF * bytes(64) <= 65536 ? 64 : 32;
  static constexpr bool fits = NBUF * bytes(KB) <= 65536;
};

template <typename TQ, typename TV, int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const TQ *__restrict__ q,
                                                          const TQ *__restrict__ k,
                                                          const TV *__restrict__ vt,
                                                          const float *__restrict__ tau,
                                                          TV *__restrict__ o,
                                                          float *__restrict__ lse, int B, int T, int Tp,
                                                          int Hq, int Hkv, int G, int hq, int nsub,
                                                          int npb, int use_norm) {
  typedef Mfma32<TQ> MQ;
  typedef Mfma32<TV> MV;
  typedef AttnTile<TQ, TV, D> TL;
  constexpr int KB = TL::KB;                          // keys per tile
  constexpr int NH = KB / 32;                         // 32-key halves per tile
  constexpr int KSQ = MQ::KS, KSV = MV::KS;
  constexpr int DP = TL::DP;                          // V^T rows (padded to one MFMA tile)
  constexpr int ND = DP / 32;                         // O^T row blocks of 32
  constexpr int KROW = D * (int)sizeof(TQ);           // bytes per K tile row
  constexpr int KCPR = KROW / 16;
  constexpr int VROW = KB * (int)sizeof(TV);          // bytes per V^T tile row
  constexpr int VCPR = VROW / 16;
  constexpr int KTILE = KB * KROW, VTILE = DP * VROW, BUF = KTILE + VTILE;
  constexpr int NBUF = TL::NBUF;
  constexpr int K_INS = KB * KCPR / 64;               // DMA instructions per K tile
  constexpr int V_INS = D * VCPR / 64;                // and per V^T tile
  constexpr int PER_WAVE = (K_INS + V_INS) / 4;
  static_assert(K_INS * 64 == KB * KCPR && V_INS * 64 == D * VCPR && (K_INS + V_INS) % 4 == 0,
                "tiles split into whole DMA instructions over 4 waves");
  static_assert(2 * PER_WAVE < 16, "vmcnt field");
  constexpr int QC = D / (2 * KSQ);                   // QK^T contraction chunks
  constexpr int PC = 16 / KSV;                        // P*V chunks per 32-key half
  static_assert(TL::fits, "K/V tiles exceed the LDS budget");

  __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
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

  // constant logit shift when the normalised logits are bounded by c_h
  const float c_h = tau[h] * 1.4426950408889634f;
  const bool fixed_shift = use_norm && c_h >= 0.f && c_h <= 60.f;   // wave-uniform
  f32x16 s_init;
#pragma unroll
  for (int a = 0; a < 16; ++a) s_init[a] = fixed_shift ? -c_h : 0.f;

  // zero the padding rows of the V^T tiles (d < 32)
  if (D < DP) {
    constexpr int PADC = (DP - D) * VROW / 16;
    for (int e = tid; e < NBUF * PADC; e += 256)
      st16(smem + (e / PADC) * BUF + KTILE + D * VROW + (e % PADC) * 16, zero_u32x4());
  }

  // Q fragments of this lane's query (B operand of S^T = K Q^T); q is stored
  // already scaled by tau_h * log2(e)
  typename MQ::frag qf[QC];
  {
    const TQ *qrow = q + ((size_t)(b * Hq + h) * Tp + qpos) * D;
#pragma unroll
    for (int c = 0; c < QC; ++c) qf[c] = load_frag<TQ>(qrow + c * 2 * KSQ + hl * KSQ);
  }

  const TQ *kbase = k + (size_t)(b * Hkv + g) * Tp * D;
  const TV *vbase = vt + (size_t)(b * Hkv + g) * D * Tp;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void *)kbase, 0, (unsigned)(Tp * KROW), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void *)vbase, 0, (unsigned)(D * Tp * (int)sizeof(TV)), 0x00020000);
  // DMA instruction u of wave w moves 1 KiB chunk u*4 + w of a K/V^T tile
  // pair (K first).  Per lane: the byte offset (inside tile 0) of the logical
  // chunk that belongs at its physical slot.
  auto is_k = [&](int u) {
    if constexpr (K_INS % 4 == 0) return u < K_INS / 4;   // compile-time
    else return u * 4 + wave < K_INS;
  };
  unsigned voff[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int ins = u * 4 + wave;
    if (is_k(u)) {
      const int c = ins * 64 + lane, row = c / KCPR, ch = (c % KCPR) ^ swz_key(row, KCPR);
      voff[u] = (unsigned)(row * KROW + ch * 16);
    } else {
      const int c = (ins - K_INS) * 64 + lane, row = c / VCPR, ch = (c % VCPR) ^ swz_key(row, VCPR);
      voff[u] = (unsigned)(row * Tp * (int)sizeof(TV) + ch * 16);
    }
  }
  auto issue = [&](int kt, int buf) {
    unsigned char *sk = smem + buf * BUF;
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int ins = u * 4 + wave;                    // wave-uniform
      if (is_k(u))
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, as_lds(sk + ins * 1024), 16, (int)voff[u],
                                                 (unsigned)(kt * KB * KROW), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, as_lds(sk + KTILE + (ins - K_INS) * 1024), 16, (int)voff[u],
                                                 (unsigned)(kt * KB * (int)sizeof(TV)), 0, 0);
    }
  };
  // S^T = K Q^T for one tile: NH accumulators of 32 keys x 32 queries
  auto qk = [&](int buf, f32x16 *s) {
    const unsigned char *sk = smem + buf * BUF;
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      s[hf] = s_init;
      const int row = hf * 32 + l32;
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const int kb = (c * 2 * KSQ + hl * KSQ) * (int)sizeof(TQ);
        typename MQ::frag kf = load_frag<TQ>(reinterpret_cast<const TQ *>(sk + row * KROW + swz(row, kb, KCPR)));
        s[hf] = MQ::mma(kf, qf[c], s[hf]);
      }
    }
  };

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  // the whole key loop is instantiated once per softmax form, so that the
  // branch between them stays outside the loop
  auto run = [&](auto fixed_tag) {
    constexpr bool FIXED = decltype(fixed_tag)::value;
    // one tile: tiles kt and kt + 1 are resident, kt + 2 is in flight
    auto step = [&](int kt, f32x16 (&s_cur)[NH], f32x16 (&s_nxt)[NH]) {
      // the slot of tile kt - 1 is free since the last barrier
      if (kt + 3 < ntiles) issue(kt + 3, (kt + 3) % NBUF);
      // one basic block per tile kind, so that the scheduler can interleave
      // the look-ahead QK^T MFMAs with this tile's softmax VALU work
      auto tile = [&](auto diag_tag) {
        constexpr bool DIAG = decltype(diag_tag)::value;
        const int k0 = kt * KB;
        const unsigned char *sv = smem + (kt % NBUF) * BUF + KTILE;
        // look ahead (past the last tile the ring slot still holds some
        // tile; that result is never used)
        qk((kt + 1) % NBUF, s_nxt);
        if constexpr (DIAG) {                          // causal mask
#pragma unroll
          for (int hf = 0; hf < NH; ++hf)
#pragma unroll
            for (int a = 0; a < 16; ++a) {
              const int key = k0 + hf * 32 + 8 * (a >> 2) + 4 * hl + (a & 3);
              if (key > qpos) s_cur[hf][a] = -INFINITY;
            }
        }
        if constexpr (!FIXED) {
          float mx = s_cur[0][0];
#pragma unroll
          for (int hf = 0; hf < NH; ++hf)
#pragma unroll
            for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s_cur[hf][a]);
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          // rescale only when some row's running max grew (alpha = 1 otherwise)
          if (__any(mx > m_run)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < ND; ++i)
#pragma unroll
              for (int a = 0; a < 16; ++a) acc[i][a] *= alpha;
            m_run = m_new;
          }
        }
#pragma unroll
        for (int hf = 0; hf < NH; ++hf)
#pragma unroll
          for (int cc = 0; cc < PC; ++cc) {
            float pv[KSV];
#pragma unroll
            for (int sl = 0; sl < KSV; ++sl)
              pv[sl] = __builtin_amdgcn_exp2f(FIXED ? s_cur[hf][KSV * cc + sl]
                                                    : s_cur[hf][KSV * cc + sl] - m_run);
            const typename MV::frag pf = pack_frag<TV>(pv);
            if constexpr (KSV == 8) {
              // row sum of the rounded probabilities the P*V product uses
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 pair = {pf[2 * e], pf[2 * e + 1]};
                const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
                l_run = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, l_run, false);
              }
            } else {
#pragma unroll
              for (int sl = 0; sl < KSV; ++sl) l_run += pv[sl];
            }
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
      };
      // tiles past this wave's last query are fully masked: they add nothing
      if (kt * KB + KB - 1 > p0) tile(std::true_type{});
      else tile(std::false_type{});
      // tile kt + 2 visible to every wave before the next step's look-ahead
      if (kt + 3 < ntiles) wait_vmcnt<PER_WAVE>();
      else wait_vmcnt<0>();
      lds_barrier();
    };

    // prologue: tiles 0..2 issued, 0 and 1 resident, S of tile 0 computed
    issue(0, 0);
    if (ntiles > 1) issue(1, 1);
    if (ntiles > 2) {
      issue(2, 2);
      wait_vmcnt<PER_WAVE>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    f32x16 s_a[NH], s_b[NH];
    qk(0, s_a);
    for (int kt = 0; kt < ntiles; kt += 2) {
      step(kt, s_a, s_b);
      if (kt + 1 < ntiles) step(kt + 1, s_b, s_a);
    }
  };
  if (fixed_shift) run(std::true_type{});
  else run(std::false_type{});

  // each half-wave summed its own keys (and both saw the same rescales)
  l_run += __shfl_xor(l_run, 32, 64);
  if (qpos >= T) return;
  // log2 of the softmax denominator in the exp2 domain, kept for the backward
  if (lse && hl == 0) lse[(size_t)(b * Hq + h) * Tp + qpos] = (fixed_shift ? c_h : m_run) + __log2f(l_run);
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
                         const float *tau, TV *o, float *lse, hipStream_t stream) {
  const int hq = gcd_int(s.G, 4);
  const int nsub = s.G / hq;
  const int pos_per = 128 / hq;
  const int npb = (s.T + pos_per - 1) / pos_per;
  const int grid = npb * s.B * s.Hkv * nsub;
  hipLaunchKernelGGL((attn_fwd_kernel<TQ, TV, D>), dim3(grid), dim3(256), 0, stream, q, k, vt, tau,
                     o, lse, s.B, s.T, s.Tp, s.Hq, s.Hkv, s.G, hq, nsub, npb, s.use_norm);
  return hipGetLastError();
}

template <typename TQ, typename TV>
hipError_t launch_attention_prefill(const MixShape &s, const TQ *q, const TQ *k, const TV *vt,
                                    const float *tau, TV *o, float *lse, hipStream_t stream) {
  switch (s.d) {
    case 16: return attn_d<TQ, TV, 16>(s, q, k, vt, tau, o, lse, stream);
    case 32: return attn_d<TQ, TV, 32>(s, q, k, vt, tau, o, lse, stream);
    case 64: return attn_d<TQ, TV, 64>(s, q, k, vt, tau, o, lse, stream);
    case 128:
      if constexpr (AttnTile<TQ, TV, 128>::fits) return attn_d<TQ, TV, 128>(s, q, k, vt, tau, o, lse, stream);
      break;
  }
  return hipErrorInvalidValue;
}

bool attention_supported(int d, bool f32) {
  return d == 16 || d == 32 || d == 64 || (d == 128 && !f32);
}

template hipError_t launch_attention_prefill<f16, bf16>(const MixShape &, const f16 *, const f16 *,
                                                        const bf16 *, const float *, bf16 *,
                                                        float *, hipStream_t);
template hipError_t launch_attention_prefill<bf16, bf16>(const MixShape &, const bf16 *,
                                                         const bf16 *, const bf16 *,
                                                         const float *, bf16 *, float *,
                                                         hipStream_t);
template hipError_t launch_attention_prefill<float, float>(const MixShape &, const float *,
                                                           const float *, const float *,
                                                           const float *, float *, float *,
                                                           hipStream_t);

}  // namespace cca
