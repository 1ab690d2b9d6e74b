// Backward of the causal softmax attention inside the latent heads (gfx950,
// MFMA).  The forward pass is o[t] = sum_{u <= t} p[t,u] v[u] with
// p = softmax_u(tau_h <q_hat(t), k_hat(u)>) [GS-EN "2. Methodology" / Latent
// Space Operations and "Extension: CCGQA"]; the pages credit CCA with a
// faster backward pass as well [GS-EN "3. Key Contributions"].  Its
// derivative, with the softmax Jacobian written out:
//   dv[u]   = sum_t p[t,u] do[t]
//   dp[t,u] = <do[t], v[u]>,   ds[t,u] = p[t,u] (dp[t,u] - <do[t], o[t]>)
//   dq[t]   = tau_h sum_u ds[t,u] k_hat[u]
//   dk[u]   = sum over the group's heads of tau_h sum_t ds[t,u] q_hat[t]
//
// Design (MI355X):
//  * p is recomputed from the forward's exp2-domain logits and the log2 of
//    each row's denominator that the forward kept (no T x T matrix in HBM).
//  * Two kernels, no atomics (deterministic sums):
//    - dK/dV: one workgroup per (sequence, kv head, 128 keys); each wave keeps
//      its 32 keys' k and v in registers and walks the query tiles of every
//      head of the group.  S = Q K^T puts one key per lane (its column) and
//      16 queries per lane, which is the B-operand layout of dV^T = dO^T P
//      and dK^T = Q^T dS: no LDS round trip for P or dS.
//    - dQ: one workgroup per (sequence, query head, 128 queries); each wave
//      keeps its 32 queries' q and dO in registers and walks the key tiles;
//      S^T = K Q^T puts one query per lane, so the row statistics are one
//      register each and dS^T is the B operand of dQ^T = K^T dS^T.
//  * The operands whose contraction runs over tokens (Q^T, dO^T, K^T) are
//    transposed once by a prep kernel, with the token order permuted inside
//    16-token groups (bits 2 and 3 swapped), so each lane's 8 tokens of an
//    MFMA k-slot run are contiguous in LDS.
//  * p and ds enter their MFMAs as the value type (bf16: fp32 range, so small
//    gradients do not underflow); the logits keep the forward's q/k type.
#include <type_traits>

#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

// ---------------------------------------------------------------------------
// prep: batched 2-D transpose with optional token permutation, and the row
// dot products <do, o>
// ---------------------------------------------------------------------------

// out[z][c'][r'] = in[z][r][c] for r < R, c < C, with r' = vt_perm(r) when
// perm_r (else r) and c' = vt_perm(c) when perm_c; rows r >= Rvalid read as
// zero.  z = z1 * nz2 + z2 selects the strides of both sides.
//
// Vector form (16-byte aligned sizes and strides): no LDS.  Each lane loads a
// VEC x VEC block (VEC rows of 16 bytes), transposes it in registers and
// stores VEC rows of 16 bytes; a wave covers a 64 x 64 (16-bit) or 32 x 32
// (32-bit) tile, and a workgroup holds one or four waves.  Lanes 8j .. 8j+7
// take consecutive row blocks of one column block, so each store instruction
// writes eight 128-byte output segments (the load instructions read eight
// 128-byte input segments either way).  The
// permutations only move whole 4-row groups, so they become load / store
// addresses.
template <typename T> struct TrBits;
template <> struct TrBits<bf16> { using U = unsigned short; };
template <> struct TrBits<f16> { using U = unsigned short; };
template <> struct TrBits<float> { using U = unsigned int; };

// One transpose of the vector form: sizes, strides and tile counts.
struct TrJob {
  const void *in;
  void *out;
  int R, Rvalid, C;
  long long in_rs, in_bs1, in_bs2, out_rs, out_bs1, out_bs2;
  int nz2, ncx, nry, perm_r, perm_c;
};

// The wave's part of one 64 x 64 (16-bit) or 32 x 32 (32-bit) tile of job t.
template <typename Tin, typename Tout>
__device__ __forceinline__ void transpose_vec_tile(const TrJob &t, int tile) {
  static_assert(sizeof(Tin) == sizeof(Tout), "same element size on both sides");
  constexpr int VEC = 16 / (int)sizeof(Tout);   // elements per 16 bytes
  constexpr int TS = 8 * VEC;                   // tile side
  const Tin *__restrict__ in = static_cast<const Tin *>(t.in);
  Tout *__restrict__ out = static_cast<Tout *>(t.out);
  const int R = t.R, Rvalid = t.Rvalid, C = t.C, nz2 = t.nz2, ncx = t.ncx, nry = t.nry;
  const int perm_r = t.perm_r, perm_c = t.perm_c;
  const long long in_rs = t.in_rs, in_bs1 = t.in_bs1, in_bs2 = t.in_bs2;
  const long long out_rs = t.out_rs, out_bs1 = t.out_bs1, out_bs2 = t.out_bs2;
  const int lane = threadIdx.x & 63, rb = lane & 7, cc = lane >> 3;
  const int cx = tile % ncx, rest = tile / ncx, ry = rest % nry, z = rest / nry;
  const int z1 = z / nz2, z2 = z % nz2;
  const int r0 = ry * TS + rb * VEC, col = cx * TS + cc * VEC;
  if (r0 >= R || col >= C) return;
  const Tin *src = in + z1 * in_bs1 + z2 * in_bs2 + col;
  Tout *dst = out + z1 * out_bs1 + z2 * out_bs2 + r0;
  using U = typename TrBits<Tout>::U;
  U e[VEC][VEC];                                // e[k][j]: input row r0 + k, column col + j
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    // input row that lands at output position r0 + k
    const int gr = perm_r ? vt_perm(r0 + k) : r0 + k;
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (gr < Rvalid) raw = ld16(src + gr * in_rs);
    if constexpr (std::is_same<Tin, Tout>::value) {
      const U *u = reinterpret_cast<const U *>(&raw);
#pragma unroll
      for (int j = 0; j < VEC; ++j) e[k][j] = u[j];
    } else {
      const Tin *iv = reinterpret_cast<const Tin *>(&raw);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const Tout o = from_f32<Tout>(to_f32(iv[j]));
        e[k][j] = *reinterpret_cast<const U *>(&o);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    u32x4 o;
    if constexpr (sizeof(U) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = (unsigned)e[2 * w][j] | ((unsigned)e[2 * w + 1][j] << 16);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = e[w][j];
    }
    const int gc = col + j;
    st16(dst + (perm_c ? vt_perm(gc) : gc) * out_rs, o);
  }
}

template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void transpose_vec_kernel(TrJob t, int ntiles) {
  const int tile = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (tile < ntiles) transpose_vec_tile<Tin, Tout>(t, tile);
}

// Several transposes in one launch: job k owns tiles [first[k], first[k+1]);
// jobs with conv set read TQ and write TV, the others read and write TV.
struct TrJobs {
  TrJob j[4];
  int conv[4];
  int first[5];
  int n;
};
template <typename TQ, typename TV>
__global__ __launch_bounds__(256) void transpose_multi_kernel(TrJobs jobs) {
  const int tile = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (tile >= jobs.first[jobs.n]) return;
  int k = 0;
  while (k + 1 < jobs.n && tile >= jobs.first[k + 1]) ++k;
  if (jobs.conv[k]) transpose_vec_tile<TQ, TV>(jobs.j[k], tile - jobs.first[k]);
  else transpose_vec_tile<TV, TV>(jobs.j[k], tile - jobs.first[k]);
}

// element-wise form for unaligned sizes or strides: 64 x 64 tiles through LDS
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void transpose_kernel(const Tin *__restrict__ in,
                                                        Tout *__restrict__ out, int R, int Rvalid,
                                                        int C, long long in_rs, long long in_bs1,
                                                        long long in_bs2, long long out_rs,
                                                        long long out_bs1, long long out_bs2,
                                                        int nz2, int perm_r, int perm_c) {
  __shared__ Tout tile[64][65];
  const int z = blockIdx.z, z1 = z / nz2, z2 = z % nz2;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const Tin *src = in + z1 * in_bs1 + z2 * in_bs2;
  Tout *dst = out + z1 * out_bs1 + z2 * out_bs2;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64, gr = r0 + r, gc = c0 + c;
    tile[r][c] = (gr < Rvalid && gr < R && gc < C) ? from_f32<Tout>(to_f32(src[gr * in_rs + gc]))
                                                   : from_f32<Tout>(0.f);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int c = e / 64, r = e % 64, gr = r0 + r, gc = c0 + c;
    if (gr < R && gc < C) {
      const int orr = perm_r ? vt_perm(gr) : gr, occ = perm_c ? vt_perm(gc) : gc;
      dst[occ * out_rs + orr] = tile[r][c];
    }
  }
}

// The vector form's job for a transpose, or false when sizes, strides or
// alignment need the element-wise form (the permutations act inside aligned
// groups of 16, which the tiles keep whole).
template <typename Tin, typename Tout>
static bool transpose_job(const Tin *in, Tout *out, int R, int Rvalid, int C, long long in_rs,
                          long long in_bs1, long long in_bs2, long long out_rs, long long out_bs1,
                          long long out_bs2, int nz1, int nz2, int perm_r, int perm_c, TrJob &j,
                          long long &ntiles) {
  constexpr int VEC = 16 / (int)sizeof(Tout);
  const bool vec = (reinterpret_cast<uintptr_t>(in) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(out) % 16 == 0) && R % VEC == 0 && C % VEC == 0 &&
                   in_rs % VEC == 0 && in_bs1 % VEC == 0 && in_bs2 % VEC == 0 &&
                   out_rs % VEC == 0 && out_bs1 % VEC == 0 && out_bs2 % VEC == 0 &&
                   (!perm_r || R % 16 == 0) && (!perm_c || C % 16 == 0);
  if (!vec) return false;
  constexpr int TS = 8 * VEC;
  j = TrJob{in, out, R, Rvalid, C, in_rs, in_bs1, in_bs2, out_rs, out_bs1, out_bs2, nz2,
            (C + TS - 1) / TS, (R + TS - 1) / TS, perm_r, perm_c};
  ntiles = (long long)j.ncx * j.nry * nz1 * nz2;
  return true;
}

// one wave per workgroup for small transposes, so they still reach every CU
static int transpose_waves_per_wg(long long ntiles) { return ntiles >= 4096 ? 4 : 1; }

template <typename Tin, typename Tout>
hipError_t launch_transpose(const Tin *in, Tout *out, int R, int Rvalid, int C, long long in_rs,
                            long long in_bs1, long long in_bs2, long long out_rs,
                            long long out_bs1, long long out_bs2, int nz1, int nz2, int perm_r,
                            int perm_c, hipStream_t stream) {
  if (R <= 0 || C <= 0 || nz1 * nz2 <= 0) return hipSuccess;
  TrJob j;
  long long nt;
  if (transpose_job(in, out, R, Rvalid, C, in_rs, in_bs1, in_bs2, out_rs, out_bs1, out_bs2, nz1,
                    nz2, perm_r, perm_c, j, nt)) {
    if (nt > (1ll << 31) - 4) return hipErrorInvalidValue;
    const int wpg = transpose_waves_per_wg(nt);
    hipLaunchKernelGGL((transpose_vec_kernel<Tin, Tout>), dim3((unsigned)((nt + wpg - 1) / wpg)),
                       dim3(64 * wpg), 0, stream, j, (int)nt);
    return hipGetLastError();
  }
  dim3 grid((C + 63) / 64, (R + 63) / 64, nz1 * nz2);
  hipLaunchKernelGGL((transpose_kernel<Tin, Tout>), grid, dim3(256), 0, stream, in, out, R, Rvalid,
                     C, in_rs, in_bs1, in_bs2, out_rs, out_bs1, out_bs2, nz2, perm_r, perm_c);
  return hipGetLastError();
}

// dsum[b, h, t] = <do[b, t, h], o[b, t, h]> for t < T, 0 for T <= t < Tp.
// LPR lanes share a row (16 bytes each, then a lane reduction); rows are
// walked token-major, the order of the [B*T, Hq*d] buffers.
template <typename TV, int D>
__global__ __launch_bounds__(256) void attn_bwd_rowdot_kernel(const TV *__restrict__ dO,
                                                              const TV *__restrict__ O,
                                                              float *__restrict__ dsum, int B,
                                                              int T, int Tp, int Hq) {
  constexpr int VEC = 16 / (int)sizeof(TV), LPR = D / VEC;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = i / LPR;                 // (b, t, h), t < Tp
  const int part = (int)(i % LPR);
  const bool ok = row < (long long)B * Tp * Hq;
  const int h = (int)(row % Hq);
  const int t = (int)((row / Hq) % Tp);
  const int b = (int)(row / ((long long)Hq * Tp));
  float acc = 0.f;
  if (ok && t < T) {
    const size_t off = ((size_t)b * T + t) * (size_t)(Hq * D) + (size_t)h * D + part * VEC;
    const u32x4 a = ld16(dO + off), c = ld16(O + off);
    const TV *av = reinterpret_cast<const TV *>(&a);
    const TV *cv = reinterpret_cast<const TV *>(&c);
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc += to_f32(av[k]) * to_f32(cv[k]);
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (ok && part == 0) dsum[((size_t)b * Hq + h) * Tp + t] = acc;
}

// ---------------------------------------------------------------------------
// shared pieces of the two main kernels
// ---------------------------------------------------------------------------

template <typename TQ, typename TV, int D> struct BwdTile {
  static constexpr int DP = D < 32 ? 32 : D;               // transposed rows, one MFMA tile min
  static constexpr int PADQ = 16 / (int)sizeof(TQ);        // 16 bytes of padding per row
  static constexpr int PADV = 16 / (int)sizeof(TV);
  static constexpr int RQ = D + PADQ;                      // row-major q/k tile row (elements)
  static constexpr int RV = D + PADV;                      // row-major v/dO tile row
  static constexpr int RT = 32 + PADV;                     // transposed tile row (32 tokens)
};

// Copy n16 16-byte chunks described by `chunk(e, &src, &dst)` into LDS through
// registers: load() issues the global reads, store() writes them to LDS.
template <int NPT> struct Staging {
  u32x4 r[NPT];
};

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

template <typename TQ, typename TV, int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TV *__restrict__ vr,
    const TV *__restrict__ qT, const TV *__restrict__ dO, const TV *__restrict__ dOT,
    const float *__restrict__ lse, const float *__restrict__ dsum, float *__restrict__ dk,
    float *__restrict__ dv, int B, int T, int Tp, int Hq, int Hkv, int G, int nkb) {
  typedef Mfma32<TQ> MQ;
  typedef Mfma32<TV> MV;
  typedef BwdTile<TQ, TV, D> TL;
  constexpr int KSQ = MQ::KS, KSV = MV::KS;
  constexpr int QC = D / (2 * KSQ), VC = D / (2 * KSV), PC = 16 / KSV;
  constexpr int DP = TL::DP, ND = DP / 32;
  constexpr int RQ = TL::RQ, RV = TL::RV, RT = TL::RT;
  // LDS of one stage: Q [32][RQ], Q^T [DP][RT], dO [32][RV], dO^T [DP][RT], lse, dsum
  constexpr int OFF_QT = 32 * RQ * (int)sizeof(TQ);
  constexpr int OFF_DO = OFF_QT + DP * RT * (int)sizeof(TV);
  constexpr int OFF_DOT = OFF_DO + 32 * RV * (int)sizeof(TV);
  constexpr int OFF_L = OFF_DOT + DP * RT * (int)sizeof(TV);
  constexpr int STAGE = OFF_L + 64 * 4;
  // 16-byte chunks per stage (global side): Q rows, Q^T rows, dO rows, dO^T rows
  constexpr int CQ = 32 * D * (int)sizeof(TQ) / 16;
  constexpr int CT = D * 32 * (int)sizeof(TV) / 16;
  constexpr int CO = 32 * D * (int)sizeof(TV) / 16;
  constexpr int NCH = CQ + CT + CO + CT;
  constexpr int NPT = (NCH + 255) / 256;
  constexpr int QCPR = D * (int)sizeof(TQ) / 16;           // chunks per Q / dO row
  constexpr int VCPR = D * (int)sizeof(TV) / 16;
  constexpr int TCPR = 32 * (int)sizeof(TV) / 16;          // chunks per transposed row

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hl = lane >> 5;
  const int rest = B * Hkv;
  const int kb = blockIdx.x / rest;                        // low key blocks (most work) first
  const int g = (blockIdx.x % rest) % Hkv, b = (blockIdx.x % rest) / Hkv;
  const int kblk0 = kb * 128;
  const int u0 = kblk0 + 32 * wave;                        // this wave's first key
  const int eq = Hq * D, ekv = Hkv * D;

  // zero the padding rows of the transposed tiles (d < 32)
  if (D < DP) {
    for (int s = 0; s < 2; ++s)
      for (int e = tid; e < (DP - D) * RT; e += 256) {
        reinterpret_cast<TV *>(smem + s * STAGE + OFF_QT)[D * RT + e] = from_f32<TV>(0.f);
        reinterpret_cast<TV *>(smem + s * STAGE + OFF_DOT)[D * RT + e] = from_f32<TV>(0.f);
      }
  }

  // this wave's keys and values (B operands: lane = key column, k-slots = dims)
  typename MQ::frag kf[QC];
  typename MV::frag vf[VC];
  {
    const int u = min(u0 + l32, Tp - 1);
    const TQ *krow = k + ((size_t)(b * Hkv + g) * Tp + u) * D;
    const TV *vrow = vr + ((size_t)(b * Hkv + g) * Tp + u) * D;
#pragma unroll
    for (int c = 0; c < QC; ++c) kf[c] = load_frag<TQ>(krow + c * 2 * KSQ + hl * KSQ);
#pragma unroll
    for (int c = 0; c < VC; ++c) vf[c] = load_frag<TV>(vrow + c * 2 * KSV + hl * KSV);
  }

  f32x16 dvt[ND], dkt[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) dvt[i] = dkt[i] = zero16();

  const int ntq = (T - kblk0 + 31) / 32;                   // query tiles per head
  const int nit = ntq * G;

  // global -> register staging of one (head, query tile) stage
  u32x4 pre[NPT];
  float pl = 0.f, pd = 0.f;
  auto gload = [&](int it) {
    const int hh = it / ntq, t0 = kblk0 + (it % ntq) * 32;
    const int h = g * G + hh;
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int e = tid + 256 * p;
      u32x4 v = zero_u32x4();
      if (e < CQ) {
        const int row = e / QCPR, c16 = e % QCPR;
        v = ld16(reinterpret_cast<const unsigned char *>(q + ((size_t)(b * Hq + h) * Tp + t0 + row) * D) + 16 * c16);
      } else if (e < CQ + CT) {
        const int e2 = e - CQ, row = e2 / TCPR, c16 = e2 % TCPR;
        v = ld16(reinterpret_cast<const unsigned char *>(qT + ((size_t)(b * Hq + h) * D + row) * Tp + t0) + 16 * c16);
      } else if (e < CQ + CT + CO) {
        const int e2 = e - CQ - CT, row = e2 / VCPR, c16 = e2 % VCPR;
        if (t0 + row < T)
          v = ld16(reinterpret_cast<const unsigned char *>(dO + ((size_t)b * T + t0 + row) * eq + (size_t)h * D) + 16 * c16);
      } else if (e < NCH) {
        const int e2 = e - CQ - CT - CO, row = e2 / TCPR, c16 = e2 % TCPR;
        v = ld16(reinterpret_cast<const unsigned char *>(dOT + ((size_t)(b * Hq + h) * D + row) * Tp + t0) + 16 * c16);
      }
      pre[p] = v;
    }
    if (tid < 32) {
      const int t = t0 + tid;
      const size_t o = (size_t)(b * Hq + h) * Tp + t;
      pl = t < T ? lse[o] : 0.f;
      pd = t < T ? dsum[o] : 0.f;
    }
  };
  auto sstore = [&](int s) {
    unsigned char *st = smem + s * STAGE;
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int e = tid + 256 * p;
      if (e < CQ) {
        const int row = e / QCPR, c16 = e % QCPR;
        st16(st + row * RQ * (int)sizeof(TQ) + 16 * c16, pre[p]);
      } else if (e < CQ + CT) {
        const int e2 = e - CQ, row = e2 / TCPR, c16 = e2 % TCPR;
        st16(st + OFF_QT + row * RT * (int)sizeof(TV) + 16 * c16, pre[p]);
      } else if (e < CQ + CT + CO) {
        const int e2 = e - CQ - CT, row = e2 / VCPR, c16 = e2 % VCPR;
        st16(st + OFF_DO + row * RV * (int)sizeof(TV) + 16 * c16, pre[p]);
      } else if (e < NCH) {
        const int e2 = e - CQ - CT - CO, row = e2 / TCPR, c16 = e2 % TCPR;
        st16(st + OFF_DOT + row * RT * (int)sizeof(TV) + 16 * c16, pre[p]);
      }
    }
    if (tid < 32) {
      reinterpret_cast<float *>(st + OFF_L)[tid] = pl;
      reinterpret_cast<float *>(st + OFF_L)[32 + tid] = pd;
    }
  };

  if (nit > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int cur = it & 1;
    if (it + 1 < nit) gload(it + 1);
    const int t0 = kblk0 + (it % ntq) * 32;
    // tiles that end before this wave's first key are fully masked
    if (t0 + 31 >= u0 && u0 < T) {
      const unsigned char *st = smem + cur * STAGE;
      const TQ *sq = reinterpret_cast<const TQ *>(st);
      const TV *sqt = reinterpret_cast<const TV *>(st + OFF_QT);
      const TV *sdo = reinterpret_cast<const TV *>(st + OFF_DO);
      const TV *sdot = reinterpret_cast<const TV *>(st + OFF_DOT);
      const float *sl = reinterpret_cast<const float *>(st + OFF_L);
      // S = Q K^T and dP = dO V^T: rows = queries 8j + 4hl + i, column = key l32
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int c = 0; c < QC; ++c)
        sacc = MQ::mma(load_frag<TQ>(sq + l32 * RQ + c * 2 * KSQ + hl * KSQ), kf[c], sacc);
#pragma unroll
      for (int c = 0; c < VC; ++c)
        dpacc = MV::mma(load_frag<TV>(sdo + l32 * RV + c * 2 * KSV + hl * KSV), vf[c], dpacc);
      const int u = u0 + l32;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int tr = 8 * (a >> 2) + 4 * hl + (a & 3);
        const int t = t0 + tr;
        const bool ok = t >= u && t < T;
        const float p = ok ? __builtin_amdgcn_exp2f(sacc[a] - sl[tr]) : 0.f;
        const float ds = ok ? p * (dpacc[a] - sl[32 + tr]) : 0.f;
        sacc[a] = p;
        dpacc[a] = ds;
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the tile's 32 queries
#pragma unroll
      for (int cc = 0; cc < PC; ++cc) {
        float pv[KSV], dsv[KSV];
#pragma unroll
        for (int s = 0; s < KSV; ++s) {
          pv[s] = sacc[KSV * cc + s];
          dsv[s] = dpacc[KSV * cc + s];
        }
        const typename MV::frag pf = pack_frag<TV>(pv), df = pack_frag<TV>(dsv);
        const int a0 = KSV * cc;
        const int col = vt_perm(8 * (a0 >> 2) + 4 * hl + (a0 & 3));
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          const int row = 32 * i + l32;
          dvt[i] = MV::mma(load_frag<TV>(sdot + row * RT + col), pf, dvt[i]);
          dkt[i] = MV::mma(load_frag<TV>(sqt + row * RT + col), df, dkt[i]);
        }
      }
    }
    if (it + 1 < nit) sstore(cur ^ 1);
    __syncthreads();
  }

  // lane: key u0 + l32, dims 32i + 8j + 4hl + (0..3); dK carries ln(2) since
  // the stored q is tau * log2(e) * q_hat
  const int u = u0 + l32;
  if (u >= T) return;
  float *dkrow = dk + ((size_t)b * T + u) * ekv + (size_t)g * D;
  float *dvrow = dv + ((size_t)b * T + u) * ekv + (size_t)g * D;
  const float ln2 = 0.6931471805599453f;
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dd = 32 * i + 8 * j + 4 * hl;
      if (dd >= D) continue;
      *reinterpret_cast<f32x4 *>(dkrow + dd) =
          f32x4{dkt[i][4 * j] * ln2, dkt[i][4 * j + 1] * ln2, dkt[i][4 * j + 2] * ln2,
                dkt[i][4 * j + 3] * ln2};
      *reinterpret_cast<f32x4 *>(dvrow + dd) =
          f32x4{dvt[i][4 * j], dvt[i][4 * j + 1], dvt[i][4 * j + 2], dvt[i][4 * j + 3]};
    }
}

// ---------------------------------------------------------------------------
// dQ (unscaled: gq[t] = sum_u ds[t,u] k_hat[u]; the caller applies tau_h)
// ---------------------------------------------------------------------------

template <typename TQ, typename TV, int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TV *__restrict__ kT,
    const TV *__restrict__ vr, const TV *__restrict__ dO, const float *__restrict__ lse,
    const float *__restrict__ dsum, float *__restrict__ gq, int B, int T, int Tp, int Hq, int Hkv,
    int G, int nqb) {
  typedef Mfma32<TQ> MQ;
  typedef Mfma32<TV> MV;
  typedef BwdTile<TQ, TV, D> TL;
  constexpr int KSQ = MQ::KS, KSV = MV::KS;
  constexpr int QC = D / (2 * KSQ), VC = D / (2 * KSV), PC = 16 / KSV;
  constexpr int DP = TL::DP, ND = DP / 32;
  constexpr int RQ = TL::RQ, RV = TL::RV, RT = TL::RT;
  // LDS of one stage: K [32][RQ], K^T [DP][RT], V [32][RV]
  constexpr int OFF_KT = 32 * RQ * (int)sizeof(TQ);
  constexpr int OFF_V = OFF_KT + DP * RT * (int)sizeof(TV);
  constexpr int STAGE = (OFF_V + 32 * RV * (int)sizeof(TV) + 15) / 16 * 16;
  constexpr int CK = 32 * D * (int)sizeof(TQ) / 16;
  constexpr int CT = D * 32 * (int)sizeof(TV) / 16;
  constexpr int CV = 32 * D * (int)sizeof(TV) / 16;
  constexpr int NCH = CK + CT + CV;
  constexpr int NPT = (NCH + 255) / 256;
  constexpr int QCPR = D * (int)sizeof(TQ) / 16;
  constexpr int VCPR = D * (int)sizeof(TV) / 16;
  constexpr int TCPR = 32 * (int)sizeof(TV) / 16;

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hl = lane >> 5;
  const int rest = B * Hq;
  const int qb = nqb - 1 - blockIdx.x / rest;              // late queries (most keys) first
  const int h = (blockIdx.x % rest) % Hq, b = (blockIdx.x % rest) / Hq;
  const int g = h / G;
  const int t0w = qb * 128 + 32 * wave;                    // this wave's first query
  const int t = t0w + l32;                                 // this lane's query
  const int eq = Hq * D;

  if (D < DP) {
    for (int s = 0; s < 2; ++s)
      for (int e = tid; e < (DP - D) * RT; e += 256)
        reinterpret_cast<TV *>(smem + s * STAGE + OFF_KT)[D * RT + e] = from_f32<TV>(0.f);
  }

  // this lane's query and output gradient (B operands: lane = query column)
  typename MQ::frag qf[QC];
  typename MV::frag of[VC];
  {
    const TQ *qrow = q + ((size_t)(b * Hq + h) * Tp + min(t, Tp - 1)) * D;
#pragma unroll
    for (int c = 0; c < QC; ++c) qf[c] = load_frag<TQ>(qrow + c * 2 * KSQ + hl * KSQ);
    const TV *orow = dO + ((size_t)b * T + min(t, T - 1)) * eq + (size_t)h * D;
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      of[c] = load_frag<TV>(orow + c * 2 * KSV + hl * KSV);
      if (t >= T) {
        const float zz[KSV] = {};
        of[c] = pack_frag<TV>(zz);
      }
    }
  }
  const size_t so = (size_t)(b * Hq + h) * Tp + min(t, Tp - 1);
  const float lq = t < T ? lse[so] : 0.f;
  const float dq_sum = t < T ? dsum[so] : 0.f;

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();

  const int last = min(qb * 128 + 127, T - 1);             // last query of the block
  const int nkt = last / 32 + 1;                           // key tiles 0 .. last

  u32x4 pre[NPT];
  auto gload = [&](int kt) {
    const int k0 = kt * 32;
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int e = tid + 256 * p;
      u32x4 v = zero_u32x4();
      if (e < CK) {
        const int row = e / QCPR, c16 = e % QCPR;
        v = ld16(reinterpret_cast<const unsigned char *>(k + ((size_t)(b * Hkv + g) * Tp + k0 + row) * D) + 16 * c16);
      } else if (e < CK + CT) {
        const int e2 = e - CK, row = e2 / TCPR, c16 = e2 % TCPR;
        v = ld16(reinterpret_cast<const unsigned char *>(kT + ((size_t)(b * Hkv + g) * D + row) * Tp + k0) + 16 * c16);
      } else if (e < NCH) {
        const int e2 = e - CK - CT, row = e2 / VCPR, c16 = e2 % VCPR;
        v = ld16(reinterpret_cast<const unsigned char *>(vr + ((size_t)(b * Hkv + g) * Tp + k0 + row) * D) + 16 * c16);
      }
      pre[p] = v;
    }
  };
  auto sstore = [&](int s) {
    unsigned char *st = smem + s * STAGE;
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
      const int e = tid + 256 * p;
      if (e < CK) {
        const int row = e / QCPR, c16 = e % QCPR;
        st16(st + row * RQ * (int)sizeof(TQ) + 16 * c16, pre[p]);
      } else if (e < CK + CT) {
        const int e2 = e - CK, row = e2 / TCPR, c16 = e2 % TCPR;
        st16(st + OFF_KT + row * RT * (int)sizeof(TV) + 16 * c16, pre[p]);
      } else if (e < NCH) {
        const int e2 = e - CK - CT, row = e2 / VCPR, c16 = e2 % VCPR;
        st16(st + OFF_V + row * RV * (int)sizeof(TV) + 16 * c16, pre[p]);
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const int k0 = kt * 32;
    // tiles that start after this wave's last query are fully masked
    if (k0 <= t0w + 31 && t0w < T) {
      const unsigned char *st = smem + cur * STAGE;
      const TQ *sk = reinterpret_cast<const TQ *>(st);
      const TV *skt = reinterpret_cast<const TV *>(st + OFF_KT);
      const TV *sv = reinterpret_cast<const TV *>(st + OFF_V);
      // S^T = K Q^T and dP^T = V dO^T: rows = keys 8j + 4hl + i, column = query l32
      f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
      for (int c = 0; c < QC; ++c)
        sacc = MQ::mma(load_frag<TQ>(sk + l32 * RQ + c * 2 * KSQ + hl * KSQ), qf[c], sacc);
#pragma unroll
      for (int c = 0; c < VC; ++c)
        dpacc = MV::mma(load_frag<TV>(sv + l32 * RV + c * 2 * KSV + hl * KSV), of[c], dpacc);
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int u = k0 + 8 * (a >> 2) + 4 * hl + (a & 3);
        const bool ok = u <= t && t < T;
        const float p = ok ? __builtin_amdgcn_exp2f(sacc[a] - lq) : 0.f;
        dpacc[a] = ok ? p * (dpacc[a] - dq_sum) : 0.f;
      }
      // dQ^T += K^T dS^T over the tile's 32 keys
#pragma unroll
      for (int cc = 0; cc < PC; ++cc) {
        float dsv[KSV];
#pragma unroll
        for (int s = 0; s < KSV; ++s) dsv[s] = dpacc[KSV * cc + s];
        const typename MV::frag df = pack_frag<TV>(dsv);
        const int a0 = KSV * cc;
        const int col = vt_perm(8 * (a0 >> 2) + 4 * hl + (a0 & 3));
#pragma unroll
        for (int i = 0; i < ND; ++i)
          acc[i] = MV::mma(load_frag<TV>(skt + (32 * i + l32) * RT + col), df, acc[i]);
      }
    }
    if (kt + 1 < nkt) sstore(cur ^ 1);
    __syncthreads();
  }

  if (t >= T) return;
  float *grow = gq + ((size_t)b * T + t) * eq + (size_t)h * D;
#pragma unroll
  for (int i = 0; i < ND; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dd = 32 * i + 8 * j + 4 * hl;
      if (dd >= D) continue;
      *reinterpret_cast<f32x4 *>(grow + dd) =
          f32x4{acc[i][4 * j], acc[i][4 * j + 1], acc[i][4 * j + 2], acc[i][4 * j + 3]};
    }
}

// ---------------------------------------------------------------------------
// d = 64 with 16-bit operands: the same two products with the streamed tiles
// moved HBM -> LDS by buffer_load ... lds (no register staging) through a
// ring of stages of 64 tokens, one barrier per stage.  Every tile row is 128
// bytes (64 elements), stored with the 16-byte chunk swizzle swz_key(row, 8);
// DMA instruction u of wave w fills 1 KiB chunk 4u + w of the stage, and
// each lane fetches the global chunk the swizzle places at its slot.
// ---------------------------------------------------------------------------

// the LDS bytes of the 16-byte piece starting at element `col` of row `row`
__device__ __forceinline__ int tile_off(int row, int col) { return row * 128 + swz(row, col * 2, 8); }

template <typename TQ, typename TV>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_dma_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TV *__restrict__ vr,
    const TV *__restrict__ qT, const TV *__restrict__ dO, const TV *__restrict__ dOT,
    const float *__restrict__ lse, const float *__restrict__ dsum, float *__restrict__ dk,
    float *__restrict__ dv, int B, int T, int Tp, int Hq, int Hkv, int G, int nkb) {
  typedef Mfma32<TQ> MQ;
  typedef Mfma32<TV> MV;
  static_assert(MQ::KS == 8 && MV::KS == 8, "16-bit operands");
  constexpr int D = 64, TILE = 64 * 128;
  constexpr int OFF_QT = TILE, OFF_DO = 2 * TILE, OFF_DOT = 3 * TILE, OFF_LD = 4 * TILE;
  constexpr int STAGE = 4 * TILE + 1024, NBUF = 4;
  constexpr int PER_WAVE = 9;              // 8 tile instructions + 1 for lse / dsum
  __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hl = lane >> 5;
  const int rest = B * Hkv;
  const int kb = blockIdx.x / rest;                        // low key blocks (most work) first
  const int g = (blockIdx.x % rest) % Hkv, b = (blockIdx.x % rest) / Hkv;
  const int kblk0 = kb * 128;
  const int u0 = kblk0 + 32 * wave;                        // this wave's first key
  const int eq = Hq * D, ekv = Hkv * D;
  (void)tid;

  typename MQ::frag kf[4];
  typename MV::frag vf[4];
  {
    const int u = min(u0 + l32, Tp - 1);
    const TQ *krow = k + ((size_t)(b * Hkv + g) * Tp + u) * D;
    const TV *vrow = vr + ((size_t)(b * Hkv + g) * Tp + u) * D;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kf[c] = load_frag<TQ>(krow + c * 16 + hl * 8);
      vf[c] = load_frag<TV>(vrow + c * 16 + hl * 8);
    }
  }

  // buffer resources over the group's G query heads
  const size_t hq0 = (size_t)b * Hq + (size_t)g * G;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(q + hq0 * Tp * D), 0, (unsigned)((size_t)G * Tp * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rqt = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(qT + hq0 * D * Tp), 0, (unsigned)((size_t)G * D * Tp * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rdo = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(dO + (size_t)b * T * eq + (size_t)g * G * D), 0,
      (unsigned)((size_t)T * eq * 2 - (size_t)g * G * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rdot = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(dOT + hq0 * D * Tp), 0, (unsigned)((size_t)G * D * Tp * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rld = __builtin_amdgcn_make_buffer_rsrc(
      (void *)((wave < 2 ? lse : dsum) + hq0 * Tp), 0, (unsigned)((size_t)G * Tp * 4), 0x00020000);

  // per-lane static offsets: instruction u covers tile u / 2, rows
  // ((u % 2) * 4 + wave) * 8 + lane / 8, physical chunk lane % 8
  unsigned vst[8];
  int rowv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int row = ((u & 1) * 4 + wave) * 8 + lane / 8;
    const int ch = (lane % 8) ^ swz_key(row, 8);
    const int tile = u >> 1;
    const unsigned rs = tile == 0 ? 128u : tile == 2 ? (unsigned)eq * 2 : (unsigned)Tp * 2;
    vst[u] = row * rs + ch * 16;
    rowv[u] = row;
  }

  const int ntq = (T - kblk0 + 63) / 64;                   // query stages per head
  const int nst = ntq * G;
  auto issue = [&](int it, int slot) {
    const int hh = it / ntq, t0 = kblk0 + (it % ntq) * 64;
    unsigned char *sb = smem + slot * STAGE;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tile = u >> 1;
      lds_void *dst = as_lds(sb + (u * 4 + wave) * 1024);
      if (tile == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dst, 16, (int)(vst[u] + t0 * 128),
                                                 (unsigned)(hh * Tp * 128), 0, 0);
      else if (tile == 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rqt, dst, 16, (int)(vst[u] + t0 * 2),
                                                 (unsigned)(hh * D * Tp * 2), 0, 0);
      else if (tile == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rdo, dst, 16, (int)(t0 + rowv[u] < T ? vst[u] + (unsigned)t0 * eq * 2 : 0x7FFFFFF0u),
            (unsigned)(hh * D * 2), 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rdot, dst, 16, (int)(vst[u] + t0 * 2),
                                                 (unsigned)(hh * D * Tp * 2), 0, 0);
    }
    // lse (waves 0, 1) and dsum (waves 2, 3): 32 floats per wave, lanes 0..7
    if (lane < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rld, as_lds(sb + OFF_LD + wave * 128), 16,
                                               (int)((t0 + 32 * (wave & 1)) * 4 + lane * 16),
                                               (unsigned)(hh * Tp * 4), 0, 0);
  };

  f32x16 dvt[2], dkt[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) dvt[i] = dkt[i] = zero16();

  // one 32-query half of a stage, in three steps: S = Q K^T and dP = dO V^T
  // (mm1), P and dS (sm), dV^T += dO^T P and dK^T += Q^T dS (mm2)
  auto mm1 = [&](const unsigned char *st, int sh, f32x16 &sacc, f32x16 &dpacc) {
    const int row = 32 * sh + l32;
    sacc = zero16();
    dpacc = zero16();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = c * 16 + hl * 8;
      sacc = MQ::mma(*reinterpret_cast<const typename MQ::frag *>(st + tile_off(row, col)), kf[c], sacc);
      dpacc = MV::mma(*reinterpret_cast<const typename MV::frag *>(st + OFF_DO + tile_off(row, col)),
                      vf[c], dpacc);
    }
  };
  auto sm = [&](const unsigned char *st, int t0, int sh, f32x16 &sacc, f32x16 &dpacc, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const float *ld = reinterpret_cast<const float *>(st + OFF_LD);
    const int u = u0 + l32;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int tr = 32 * sh + 8 * (a >> 2) + 4 * hl + (a & 3);
      const float p = __builtin_amdgcn_exp2f(sacc[a] - ld[tr]);
      const float ds = p * (dpacc[a] - ld[64 + tr]);
      if constexpr (EDGE) {
        const int t = t0 + tr;
        const bool ok = t >= u && t < T;
        sacc[a] = ok ? p : 0.f;
        dpacc[a] = ok ? ds : 0.f;
      } else {
        sacc[a] = p;
        dpacc[a] = ds;
      }
    }
  };
  auto mm2 = [&](const unsigned char *st, int sh, const f32x16 &sacc, const f32x16 &dpacc) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      float pv[8], dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = sacc[8 * cc + e];
        dsv[e] = dpacc[8 * cc + e];
      }
      const typename MV::frag pf = pack_frag<TV>(pv), df = pack_frag<TV>(dsv);
      const int col = 32 * sh + 16 * cc + 8 * hl;          // vt_perm(16 cc + 4 hl) inside the half
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rd = 32 * i + l32;
        dvt[i] = MV::mma(*reinterpret_cast<const typename MV::frag *>(st + OFF_DOT + tile_off(rd, col)),
                         pf, dvt[i]);
        dkt[i] = MV::mma(*reinterpret_cast<const typename MV::frag *>(st + OFF_QT + tile_off(rd, col)),
                         df, dkt[i]);
      }
    }
  };
  auto half = [&](const unsigned char *st, int t0, int sh, auto edge_tag) {
    f32x16 sacc, dpacc;
    mm1(st, sh, sacc, dpacc);
    sm(st, t0, sh, sacc, dpacc, edge_tag);
    mm2(st, sh, sacc, dpacc);
  };
  // both halves away from the diagonal and the sequence end, in one block:
  // the second half's S and dP MFMAs run under the first half's exponentials
  // and its dV / dK MFMAs under the second half's (same sums, same order)
  auto both = [&](const unsigned char *st, int t0) {
    f32x16 s0, d0, s1, d1;
    mm1(st, 0, s0, d0);
    mm1(st, 1, s1, d1);
    sm(st, t0, 0, s0, d0, std::false_type{});
    mm2(st, 0, s0, d0);
    sm(st, t0, 1, s1, d1, std::false_type{});
    mm2(st, 1, s1, d1);
  };

  // ring: at the top of stage it, stages it + 1 .. it + NBUF - 1 may be in
  // flight; wait_ahead(n): this wave's DMA of all but the last n issued
  // stages has landed
  auto wait_ahead = [&](int n) {
    if (n >= 2) wait_vmcnt<2 * PER_WAVE>();
    else if (n == 1) wait_vmcnt<PER_WAVE>();
    else wait_vmcnt<0>();
  };
  for (int s0 = 0; s0 < NBUF - 1 && s0 < nst; ++s0) issue(s0, s0);
  wait_ahead(min(nst, NBUF - 1) - 1);
  lds_barrier();
  for (int it = 0; it < nst; ++it) {
    // the slot of stage it - 1 is free since the last barrier
    if (it + NBUF - 1 < nst) issue(it + NBUF - 1, (it + NBUF - 1) % NBUF);
    const int t0 = kblk0 + (it % ntq) * 64;
    const unsigned char *st = smem + (it % NBUF) * STAGE;
    if (u0 < T) {
      if (t0 >= u0 + 32 && t0 + 63 < T) {
        both(st, t0);
      } else {
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const int ts = t0 + 32 * sh;
          if (ts + 31 < u0) continue;                      // every query before this wave's keys
          if (ts < u0 + 32 || ts + 31 >= T) half(st, t0, sh, std::true_type{});
          else half(st, t0, sh, std::false_type{});
        }
      }
    }
    // stage it + 1 landed (this wave's part), then every wave's part
    wait_ahead(min(nst, it + NBUF) - (it + 2));
    lds_barrier();
  }

  const int u = u0 + l32;
  if (u >= T) return;
  float *dkrow = dk + ((size_t)b * T + u) * ekv + (size_t)g * D;
  float *dvrow = dv + ((size_t)b * T + u) * ekv + (size_t)g * D;
  const float ln2 = 0.6931471805599453f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dd = 32 * i + 8 * j + 4 * hl;
      *reinterpret_cast<f32x4 *>(dkrow + dd) =
          f32x4{dkt[i][4 * j] * ln2, dkt[i][4 * j + 1] * ln2, dkt[i][4 * j + 2] * ln2,
                dkt[i][4 * j + 3] * ln2};
      *reinterpret_cast<f32x4 *>(dvrow + dd) =
          f32x4{dvt[i][4 * j], dvt[i][4 * j + 1], dvt[i][4 * j + 2], dvt[i][4 * j + 3]};
    }
}

template <typename TQ, typename TV>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_dma_kernel(
    const TQ *__restrict__ q, const TQ *__restrict__ k, const TV *__restrict__ kT,
    const TV *__restrict__ vr, const TV *__restrict__ dO, const float *__restrict__ lse,
    const float *__restrict__ dsum, float *__restrict__ gq, int B, int T, int Tp, int Hq, int Hkv,
    int G, int nqb) {
  typedef Mfma32<TQ> MQ;
  typedef Mfma32<TV> MV;
  static_assert(MQ::KS == 8 && MV::KS == 8, "16-bit operands");
  constexpr int D = 64, TILE = 64 * 128;
  constexpr int OFF_KT = TILE, OFF_V = 2 * TILE;
  constexpr int STAGE = 3 * TILE, NBUF = 3;
  constexpr int PER_WAVE = 6;
  __shared__ __attribute__((aligned(16))) unsigned char smem[NBUF * STAGE];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int l32 = lane & 31, hl = lane >> 5;
  const int rest = B * Hq;
  const int qb = nqb - 1 - blockIdx.x / rest;              // late queries (most keys) first
  const int h = (blockIdx.x % rest) % Hq, b = (blockIdx.x % rest) / Hq;
  const int g = h / G;
  const int t0w = qb * 128 + 32 * wave;
  const int t = t0w + l32;
  const int eq = Hq * D;

  typename MQ::frag qf[4];
  typename MV::frag of[4];
  {
    const TQ *qrow = q + ((size_t)(b * Hq + h) * Tp + min(t, Tp - 1)) * D;
    const TV *orow = dO + ((size_t)b * T + min(t, T - 1)) * eq + (size_t)h * D;
    const float zz[8] = {};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[c] = load_frag<TQ>(qrow + c * 16 + hl * 8);
      of[c] = t < T ? load_frag<TV>(orow + c * 16 + hl * 8) : pack_frag<TV>(zz);
    }
  }
  const size_t so = (size_t)(b * Hq + h) * Tp + min(t, Tp - 1);
  const float lq = t < T ? lse[so] : 0.f;
  const float dq_sum = t < T ? dsum[so] : 0.f;

  const size_t kv0 = (size_t)b * Hkv + g;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(k + kv0 * Tp * D), 0, (unsigned)((size_t)Tp * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rkt = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(kT + kv0 * D * Tp), 0, (unsigned)((size_t)D * Tp * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vr + kv0 * Tp * D), 0, (unsigned)((size_t)Tp * D * 2), 0x00020000);
  unsigned vst[6];
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int row = ((u & 1) * 4 + wave) * 8 + lane / 8;
    const int ch = (lane % 8) ^ swz_key(row, 8);
    vst[u] = row * ((u >> 1) == 1 ? (unsigned)Tp * 2 : 128u) + ch * 16;
  }
  auto issue = [&](int kt, int slot) {
    const int k0 = kt * 64;
    unsigned char *sb = smem + slot * STAGE;
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int tile = u >> 1;
      lds_void *dst = as_lds(sb + (u * 4 + wave) * 1024);
      if (tile == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dst, 16, (int)(vst[u] + k0 * 128), 0, 0, 0);
      else if (tile == 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rkt, dst, 16, (int)(vst[u] + k0 * 2), 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, (int)(vst[u] + k0 * 128), 0, 0, 0);
    }
  };

  f32x16 acc[2];
  acc[0] = acc[1] = zero16();

  // one 32-key half of a stage: S^T and dP^T (mm1), dS (sm), dQ^T += K^T
  // dS^T (mm2)
  auto mm1 = [&](const unsigned char *st, int sh, f32x16 &sacc, f32x16 &dpacc) {
    const int row = 32 * sh + l32;
    sacc = zero16();
    dpacc = zero16();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = c * 16 + hl * 8;
      sacc = MQ::mma(*reinterpret_cast<const typename MQ::frag *>(st + tile_off(row, col)), qf[c], sacc);
      dpacc = MV::mma(*reinterpret_cast<const typename MV::frag *>(st + OFF_V + tile_off(row, col)),
                      of[c], dpacc);
    }
  };
  auto sm = [&](int k0, int sh, const f32x16 &sacc, f32x16 &dpacc, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const float p = __builtin_amdgcn_exp2f(sacc[a] - lq);
      const float ds = p * (dpacc[a] - dq_sum);
      if constexpr (EDGE) {
        const int u = k0 + 32 * sh + 8 * (a >> 2) + 4 * hl + (a & 3);
        dpacc[a] = (u <= t && t < T) ? ds : 0.f;
      } else {
        dpacc[a] = ds;
      }
    }
  };
  auto mm2 = [&](const unsigned char *st, int sh, const f32x16 &dpacc) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      float dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) dsv[e] = dpacc[8 * cc + e];
      const typename MV::frag df = pack_frag<TV>(dsv);
      const int col = 32 * sh + 16 * cc + 8 * hl;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rd = 32 * i + l32;
        acc[i] = MV::mma(*reinterpret_cast<const typename MV::frag *>(st + OFF_KT + tile_off(rd, col)),
                         df, acc[i]);
      }
    }
  };
  auto half = [&](const unsigned char *st, int k0, int sh, auto edge_tag) {
    f32x16 sacc, dpacc;
    mm1(st, sh, sacc, dpacc);
    sm(k0, sh, sacc, dpacc, edge_tag);
    mm2(st, sh, dpacc);
  };
  // both halves below the diagonal, in one block: the second half's S and
  // dP MFMAs run under the first half's exponentials, its dQ MFMAs under the
  // second half's (same sums, same order)
  auto both = [&](const unsigned char *st, int k0) {
    f32x16 s0, d0, s1, d1;
    mm1(st, 0, s0, d0);
    mm1(st, 1, s1, d1);
    sm(k0, 0, s0, d0, std::false_type{});
    mm2(st, 0, d0);
    sm(k0, 1, s1, d1, std::false_type{});
    mm2(st, 1, d1);
  };

  const int last = min(qb * 128 + 127, T - 1);
  const int nkt = last / 64 + 1;
  issue(0, 0);
  if (nkt > 1) {
    issue(1, 1);
    wait_vmcnt<PER_WAVE>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 2 < nkt) issue(kt + 2, (kt + 2) % NBUF);
    const int k0 = kt * 64;
    const unsigned char *st = smem + (kt % NBUF) * STAGE;
    if (t0w < T) {
      if (k0 + 63 <= t0w && t0w + 31 < T) {
        both(st, k0);
      } else {
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const int ks = k0 + 32 * sh;
          if (ks > t0w + 31) continue;                     // every key after this wave's queries
          if (ks + 31 > t0w || t0w + 31 >= T) half(st, k0, sh, std::true_type{});
          else half(st, k0, sh, std::false_type{});
        }
      }
    }
    if (kt + 2 < nkt) wait_vmcnt<PER_WAVE>();
    else wait_vmcnt<0>();
    lds_barrier();
  }

  if (t >= T) return;
  float *grow = gq + ((size_t)b * T + t) * eq + (size_t)h * D;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dd = 32 * i + 8 * j + 4 * hl;
      *reinterpret_cast<f32x4 *>(grow + dd) =
          f32x4{acc[i][4 * j], acc[i][4 * j + 1], acc[i][4 * j + 2], acc[i][4 * j + 3]};
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <typename TQ, typename TV, int D>
static hipError_t attn_bwd_d(const MixShape &s, const AttnBwdArgs<TQ, TV> &a, hipStream_t stream) {
  const int eq = s.Hq * D;
  hipError_t e;
  // transposed, token-permuted copies: q^T and dO^T per query head, k^T per kv
  // head; v back to row-major
  {
    // the four as one launch when all take the vector form (their waits overlap)
    TrJobs jobs{};
    long long nt[4];
    bool all = transpose_job<TQ, TV>(a.q, a.qT, s.Tp, s.Tp, D, D, (long long)s.Hq * s.Tp * D,
                                     (long long)s.Tp * D, s.Tp, (long long)s.Hq * D * s.Tp,
                                     (long long)D * s.Tp, s.B, s.Hq, 1, 0, jobs.j[0], nt[0]);
    all = all && transpose_job<TQ, TV>(a.k, a.kT, s.Tp, s.Tp, D, D, (long long)s.Hkv * s.Tp * D,
                                       (long long)s.Tp * D, s.Tp, (long long)s.Hkv * D * s.Tp,
                                       (long long)D * s.Tp, s.B, s.Hkv, 1, 0, jobs.j[1], nt[1]);
    all = all && transpose_job<TV, TV>(a.dO, a.dOT, s.Tp, s.T, D, eq, (long long)s.T * eq, D, s.Tp,
                                       (long long)s.Hq * D * s.Tp, (long long)D * s.Tp, s.B, s.Hq,
                                       1, 0, jobs.j[2], nt[2]);
    all = all && transpose_job<TV, TV>(a.vt, a.vr, D, D, s.Tp, s.Tp, (long long)s.Hkv * D * s.Tp,
                                       (long long)D * s.Tp, D, (long long)s.Hkv * s.Tp * D,
                                       (long long)s.Tp * D, s.B, s.Hkv, 0, 1, jobs.j[3], nt[3]);
    const long long total = all ? nt[0] + nt[1] + nt[2] + nt[3] : 0;
    if (all && total > 0 && total <= (1ll << 31) - 4) {
      jobs.n = 4;
      jobs.first[0] = 0;
      for (int k = 0; k < 4; ++k) {
        jobs.conv[k] = k < 2 && !std::is_same<TQ, TV>::value;
        jobs.first[k + 1] = jobs.first[k] + (int)nt[k];
      }
      const int wpg = transpose_waves_per_wg(total);
      hipLaunchKernelGGL((transpose_multi_kernel<TQ, TV>), dim3((unsigned)((total + wpg - 1) / wpg)),
                         dim3(64 * wpg), 0, stream, jobs);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      e = launch_transpose<TQ, TV>(a.q, a.qT, s.Tp, s.Tp, D, D, (long long)s.Hq * s.Tp * D,
                                   (long long)s.Tp * D, s.Tp, (long long)s.Hq * D * s.Tp,
                                   (long long)D * s.Tp, s.B, s.Hq, 1, 0, stream);
      if (e != hipSuccess) return e;
      e = launch_transpose<TQ, TV>(a.k, a.kT, s.Tp, s.Tp, D, D, (long long)s.Hkv * s.Tp * D,
                                   (long long)s.Tp * D, s.Tp, (long long)s.Hkv * D * s.Tp,
                                   (long long)D * s.Tp, s.B, s.Hkv, 1, 0, stream);
      if (e != hipSuccess) return e;
      e = launch_transpose<TV, TV>(a.dO, a.dOT, s.Tp, s.T, D, eq, (long long)s.T * eq, D, s.Tp,
                                   (long long)s.Hq * D * s.Tp, (long long)D * s.Tp, s.B, s.Hq, 1, 0,
                                   stream);
      if (e != hipSuccess) return e;
      e = launch_transpose<TV, TV>(a.vt, a.vr, D, D, s.Tp, s.Tp, (long long)s.Hkv * D * s.Tp,
                                   (long long)D * s.Tp, D, (long long)s.Hkv * s.Tp * D,
                                   (long long)s.Tp * D, s.B, s.Hkv, 0, 1, stream);
      if (e != hipSuccess) return e;
    }
  }
  constexpr int LPR = D * (int)sizeof(TV) / 16;
  const long long nthr = (long long)s.B * s.Hq * s.Tp * LPR;
  hipLaunchKernelGGL((attn_bwd_rowdot_kernel<TV, D>), dim3((unsigned)((nthr + 255) / 256)),
                     dim3(256), 0, stream, a.dO, a.O, a.dsum, s.B, s.T, s.Tp, s.Hq);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (s.T + 127) / 128;
  if constexpr (D == 64 && sizeof(TQ) == 2 && sizeof(TV) == 2) {
    hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<TQ, TV>), dim3(nkb * s.B * s.Hkv), dim3(256), 0,
                       stream, a.q, a.k, a.vr, a.qT, a.dO, a.dOT, a.lse, a.dsum, a.dk, a.dv, s.B,
                       s.T, s.Tp, s.Hq, s.Hkv, s.G, nkb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dq_dma_kernel<TQ, TV>), dim3(nkb * s.B * s.Hq), dim3(256), 0,
                       stream, a.q, a.k, a.kT, a.vr, a.dO, a.lse, a.dsum, a.gq, s.B, s.T, s.Tp,
                       s.Hq, s.Hkv, s.G, nkb);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<TQ, TV, D>), dim3(nkb * s.B * s.Hkv), dim3(256), 0,
                     stream, a.q, a.k, a.vr, a.qT, a.dO, a.dOT, a.lse, a.dsum, a.dk, a.dv, s.B,
                     s.T, s.Tp, s.Hq, s.Hkv, s.G, nkb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<TQ, TV, D>), dim3(nkb * s.B * s.Hq), dim3(256), 0, stream,
                     a.q, a.k, a.kT, a.vr, a.dO, a.lse, a.dsum, a.gq, s.B, s.T, s.Tp, s.Hq, s.Hkv,
                     s.G, nkb);
  return hipGetLastError();
}

template <typename TQ, typename TV>
hipError_t launch_attention_backward(const MixShape &s, const AttnBwdArgs<TQ, TV> &a,
                                     hipStream_t stream) {
  switch (s.d) {
    case 16: return attn_bwd_d<TQ, TV, 16>(s, a, stream);
    case 32: return attn_bwd_d<TQ, TV, 32>(s, a, stream);
    case 64: return attn_bwd_d<TQ, TV, 64>(s, a, stream);
    case 128:
      if constexpr (sizeof(TV) == 2) return attn_bwd_d<TQ, TV, 128>(s, a, stream);
      break;
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_attention_backward<f16, bf16>(const MixShape &,
                                                         const AttnBwdArgs<f16, bf16> &,
                                                         hipStream_t);
template hipError_t launch_attention_backward<bf16, bf16>(const MixShape &,
                                                          const AttnBwdArgs<bf16, bf16> &,
                                                          hipStream_t);
template hipError_t launch_attention_backward<float, float>(const MixShape &,
                                                            const AttnBwdArgs<float, float> &,
                                                            hipStream_t);

template <typename Tin, typename Tout>
hipError_t launch_transpose_2d(const Tin *in, Tout *out, int R, int Rvalid, int C, long long in_rs,
                               long long out_rs, hipStream_t stream) {
  return launch_transpose<Tin, Tout>(in, out, R, Rvalid, C, in_rs, 0, 0, out_rs, 0, 0, 1, 1, 0, 0,
                                     stream);
}
template hipError_t launch_transpose_2d<bf16, bf16>(const bf16 *, bf16 *, int, int, int, long long,
                                                    long long, hipStream_t);
template hipError_t launch_transpose_2d<float, float>(const float *, float *, int, int, int,
                                                      long long, long long, hipStream_t);

}  // namespace cca
