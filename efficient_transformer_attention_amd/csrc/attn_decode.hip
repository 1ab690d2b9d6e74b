// Decode attention over the latent KV cache (gfx950, HBM bound).
//
// One new query token per sequence attends to the Lk = L + 1 cached latent
// keys of its kv head; the G query heads of a group read each K/V row once.
// The cache grows with the sequence and decode is limited by memory
// bandwidth [GS-EN "1. Problem Statement"]; CCGQA's shared latent kv heads
// make that cache small [GS-EN "2. Methodology" / "Extension: CCGQA"].
//
// Design (MI355X): split-KV with the arithmetic on the matrix cores, so the
// kernel is bound by HBM and not by VALU issue.
//  * A workgroup (4 waves) streams one chunk of keys of one (sequence, kv
//    head); its G query heads (up to 32) are the N columns of the MFMA tiles.
//  * Per 32-key tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16:
//    the K rows are loaded from HBM straight into the A-operand layout (lane:
//    one key row, 16 contiguous bytes).  q is fp32; it is split into a bf16
//    high part and a bf16 remainder, two MFMAs, so the logits keep ~16 bits
//    more than a single bf16 rounding of q would.
//  * The S^T accumulator holds one query head per lane, which is the B-operand
//    layout of O^T = V^T P^T; V rows go through a wave-private LDS tile
//    (coalesced 16-byte writes, 16-bit transposed reads).
//  * The next tiles' V rows are requested as soon as this tile's V is staged
//    in LDS, their K rows as soon as the QK^T MFMAs have read K, so each
//    load has most of an iteration to land.
//  * Online softmax per lane in fp32 (exp2, tau * log2(e) folded into q);
//    the 4 waves merge through LDS and each chunk leaves (m, l, o) in fp32
//    scratch; a second kernel merges the chunks with the log-sum-exp rule.
#include "cca_device.h"
#include "cca_launch.h"

namespace cca {

static constexpr int DEC_CHUNK = 4096;   // keys per workgroup
static constexpr int DEC_TILE = 32;      // keys per MFMA tile
static constexpr int DEC_F32_MAXG = 8;   // query heads per workgroup, fp32 path
// Pages one chunk of keys can span: chunks hold at most 4 * DEC_CHUNK + 63
// keys (dec_num_chunks starts at Lk / (4 * DEC_CHUNK)) and pages are at least
// 32 rows.
static constexpr int DEC_MAX_PAGES = (4 * DEC_CHUNK + 64) / 32 + 2;

// Query heads per workgroup of the MFMA path (the N columns of a 32x32 tile);
// capped lower at d = 128 so the merge buffer stays within 64 KiB of LDS.
template <int D> struct DecMaxG { static constexpr int value = D <= 64 ? 32 : 16; };

int decode_chunk_keys(int) { return DEC_CHUNK; }

static int dec_num_chunks(int B, int Hkv, int Lk);
static int dec_chunk_len(int Lk, int nch);

bool decode_pages_fit(int B, int Hkv, int Lk, int page) {
  const int chunk = dec_chunk_len(Lk, dec_num_chunks(B, Hkv, Lk));
  return page >= 1 && (chunk + page - 1) / page + 1 <= DEC_MAX_PAGES;
}

// Largest divisor of G that is <= cap.
static int dec_heads_per_wg(int G, int cap) {
  for (int gh = cap < G ? cap : G; gh >= 1; --gh)
    if (G % gh == 0) return gh;
  return 1;
}

// Number of key chunks per (sequence, kv head): DEC_CHUNK / 2 to 4 DEC_CHUNK
// keys each, chosen so the grid fills whole rounds of the workgroups the chip
// holds at once (256 CUs x 2 resident workgroups) when that costs little.
static int dec_num_chunks(int B, int Hkv, int Lk) {
  const int streams = B * Hkv, slots = 512;
  const int lo = (Lk + 4 * DEC_CHUNK - 1) / (4 * DEC_CHUNK);
  const int hi = (Lk + DEC_CHUNK / 2 - 1) / (DEC_CHUNK / 2);
  auto cost = [&](int n) {
    const long long rounds = ((long long)streams * n + slots - 1) / slots;
    return rounds * ((Lk + n - 1) / n);
  };
  long long best = -1;
  for (int n = lo < 1 ? 1 : lo; n <= hi; ++n)
    if (best < 0 || cost(n) < best) best = cost(n);
  // the fewest chunks within 1% of the best: longer chunks carry less
  // per-chunk overhead (B64 x L32768: 4 chunks measured 2% faster than 6)
  for (int n = lo < 1 ? 1 : lo; n <= hi; ++n)
    if (cost(n) * 100 <= best * 101) return n;
  return 1;
}

static int dec_chunk_len(int Lk, int nch) {
  const int per = (Lk + nch - 1) / nch;
  return (per + 2 * DEC_TILE - 1) / (2 * DEC_TILE) * (2 * DEC_TILE);
}

size_t decode_partial_floats(int B, int Hq, int Hkv, int d, int Lk, int m) {
  return (size_t)B * Hq * m * dec_num_chunks(B, Hkv, Lk) * (d + 2);
}

__device__ __forceinline__ float exp2_or_zero(float a, float m) {
  return a == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(a - m);
}

// ---------------------------------------------------------------------------
// bf16 cache: MFMA path
// ---------------------------------------------------------------------------
// VARLEN: the cache length comes per sequence from lens[] (a separate
// instantiation, so the uniform-length kernel carries no per-sequence load).
// PAGED: cache rows are found through the page table of `cm` (one table
// lookup per row gather); otherwise cm is contiguous.
// MULTI: m new tokens per sequence; the MFMA columns are (query head, new
// token) pairs, GH of them per workgroup, and column j of a sequence at
// length L sees keys 0 .. L + j (causal among the new tokens).
template <int D, bool VARLEN, bool PAGED, bool MULTI>
__global__ __launch_bounds__(256) void attn_decode_mfma_kernel(const float *__restrict__ q,
                                                               const float *__restrict__ tau,
                                                               const bf16 *__restrict__ kc,
                                                               const bf16 *__restrict__ vc, StateOut cm,
                                                               int Lk, const int *__restrict__ lens,
                                                               int chunk, int Hq, int Hkv,
                                                               int G, int GH, int nsub, int nch,
                                                               int m, float *__restrict__ part) {
  constexpr int QC = D / 16;                 // contraction chunks of S^T
  constexpr int ND = D < 32 ? 1 : D / 32;    // O^T row blocks
  constexpr int MAXG = DecMaxG<D>::value;
  constexpr int TPI = D <= 64 ? 2 : 1;       // 32-key tiles per wave iteration
  // LDS V row stride: 16 bytes of padding put rows r and r+4 (the two lane
  // halves of one transposed read) on disjoint banks.
  constexpr int VROW = D * 2 + 16;
  constexpr int VTILE = DEC_TILE * VROW;
  constexpr int VBYTES = 2 * 4 * TPI * VTILE;      // V tiles, then K tiles (same row stride)
  constexpr int RBYTES = 4 * MAXG * (D + 2) * 4;
  // the per-wave V tiles and, after the key loop, the wave-merge buffer
  __shared__ __attribute__((aligned(16))) unsigned char smem[VBYTES > RBYTES ? VBYTES : RBYTES];
  typedef float RedRow[D + 2];
  RedRow *red = reinterpret_cast<RedRow *>(smem);   // [wave * MAXG + column]

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hl = lane >> 5;
  int id = blockIdx.x;
  const int c = id % nch; id /= nch;
  const int sub = id % nsub; id /= nsub;
  const int g = id % Hkv, b = id / Hkv;
  const int h0 = g * G + sub * GH;
  // this lane's column: query head hcol (of new token jcol)
  bool col_ok;
  int hcol, jcol;
  if constexpr (MULTI) {
    const int pr = sub * GH + l32;
    col_ok = l32 < GH && pr < G * m;
    hcol = g * G + (col_ok ? pr : 0) / m;
    jcol = (col_ok ? pr : 0) % m;
  } else {
    col_ok = l32 < GH;
    hcol = h0 + (col_ok ? l32 : 0);
    jcol = 0;
  }

  // q of head hcol scaled by tau*log2(e), split into bf16 hi + lo
  bf16x8 qhi[QC], qlo[QC];
  {
    const float sc = col_ok ? tau[hcol] * 1.4426950408889634f : 0.f;
    const float *qr = MULTI ? q + ((size_t)(b * m + jcol) * Hq + hcol) * D
                            : q + (size_t)(b * Hq + hcol) * D;
#pragma unroll
    for (int cc = 0; cc < QC; ++cc)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float v = col_ok ? qr[16 * cc + 8 * hl + s] * sc : 0.f;
        const bf16 hi = (bf16)v;
        qhi[cc][s] = hi;
        qlo[cc][s] = (bf16)(v - (float)hi);
      }
  }

  // keys of this sequence: lens[b] + M (lens clamped to [0, Lk - M]) when
  // given, M = the new tokens; column jcol sees keys below klim
  const int M = MULTI ? m : 1;
  const int Lkb = VARLEN ? min(max(lens[b], 0), Lk - M) + M : Lk;
  const int kbeg = c * chunk;
  const int kend = min(kbeg + chunk, Lkb);
  const int klim = min(kend, Lkb - M + jcol + 1);
  const int kcut = MULTI ? min(kend, Lkb - M + 1) : kend;   // first key some column masks
  const int ntile = (kend - kbeg + DEC_TILE - 1) / DEC_TILE;
  const bf16 *kb = kc + (size_t)(b * Hkv + g) * cm.capacity * D;
  const bf16 *vb = vc + (size_t)(b * Hkv + g) * cm.capacity * D;
  unsigned char *myv = smem + wave * TPI * VTILE;
  unsigned char *myk = smem + (4 + wave) * TPI * VTILE;
  // transpose-read address of this lane inside a V tile (d a multiple of 32):
  // lane 16 gq + 4 j + q fetches key row 4 (gq >> 1) + j, columns
  // 16 (gq & 1) + 4 q .. + 3
  const int vtr_off = (4 * (lane >> 5) + ((lane >> 2) & 3)) * VROW + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  // paged: the pages of this chunk's rows, staged once in LDS (a chunk is at
  // most DEC_MAX_PAGES pages), so a row's page is an LDS read
  __shared__ int spages[PAGED ? DEC_MAX_PAGES : 1];
  const int pb0 = PAGED ? kbeg / cm.page : 0;
  if constexpr (PAGED) {
    const int npb = kend > kbeg ? (kend - 1) / cm.page - pb0 + 1 : 0;
    for (int i = tid; i < npb; i += 256) {
      const int pg = cm.table[(size_t)b * cm.mpps + pb0 + i];
      spages[i] = pg < 0 ? 0 : (pg >= cm.npages ? cm.npages - 1 : pg);
    }
    __syncthreads();
  }
  // element offset of a cache row: contiguous from this (b, g) base, or paged
  auto krow_ptr = [&](const bf16 *base_c, const bf16 *pool, int row) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int pi = row / cm.page;
      return pool + (((size_t)spages[pi - pb0] * Hkv + g) * cm.page + (row - pi * cm.page)) * D;
    } else {
      return base_c + (size_t)row * D;
    }
  };

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  // tiles of wave w: w*TPI + 4*TPI*it + u; rows past the chunk end are clamped
  // to its last key (finite data, masked below)
  constexpr int VPL = (DEC_TILE * D / 8 + 63) / 64;   // 16-byte V pieces per lane per tile
  u32x4 kreg[TPI][QC], vreg[TPI][VPL];
  static_assert(VPL == QC, "K and V tiles load as the same 16-byte pieces");
  // K and V rows load whole (D / 8 consecutive lanes per row, so every load
  // instruction reads whole 128-byte lines), marked non-temporal
  auto gload_k = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < TPI; ++u) {
      const int k0 = kbeg + (t0 + u) * DEC_TILE;
#pragma unroll
      for (int r = 0; r < VPL; ++r) {
        const int e = lane + 64 * r;
        if (e < DEC_TILE * D / 8) {
          const int row = e / (D / 8), seg = e % (D / 8);
          kreg[u][r] = ld16_nt(krow_ptr(kb, kc, min(k0 + row, kend - 1)) + 8 * seg);
        }
      }
    }
  };
  auto gload_v = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < TPI; ++u) {
      const int k0 = kbeg + (t0 + u) * DEC_TILE;
#pragma unroll
      for (int r = 0; r < VPL; ++r) {
        const int e = lane + 64 * r;
        if (e < DEC_TILE * D / 8) {
          const int row = e / (D / 8), seg = e % (D / 8);
          vreg[u][r] = ld16_nt(krow_ptr(vb, vc, min(k0 + row, kend - 1)) + 8 * seg);
        }
      }
    }
  };
  auto gload = [&](int t0) __attribute__((always_inline)) { gload_k(t0); gload_v(t0); };

  const int step = 4 * TPI;
  int t = wave * TPI;
  if (t < ntile) gload(t);
  for (; t < ntile; t += step) {
    // stage K and V (wave-private), then S^T = K Q^T for the TPI tiles
#pragma unroll
    for (int u = 0; u < TPI; ++u)
#pragma unroll
      for (int r = 0; r < VPL; ++r) {
        const int e = lane + 64 * r;
        if (e < DEC_TILE * D / 8) {
          const int row = e / (D / 8), seg = e % (D / 8);
          unsigned char *dv = myv + u * VTILE + row * VROW + seg * 16;
          *reinterpret_cast<u32x2 *>(dv) = u32x2{vreg[u][r][0], vreg[u][r][1]};
          *reinterpret_cast<u32x2 *>(dv + 8) = u32x2{vreg[u][r][2], vreg[u][r][3]};
          unsigned char *dk = myk + u * VTILE + row * VROW + seg * 16;
          *reinterpret_cast<u32x2 *>(dk) = u32x2{kreg[u][r][0], kreg[u][r][1]};
          *reinterpret_cast<u32x2 *>(dk + 8) = u32x2{kreg[u][r][2], kreg[u][r][3]};
        }
      }
    __builtin_amdgcn_wave_barrier();
    if (t + step < ntile) gload(t + step);     // K / V registers are free once staged
    f32x16 s[TPI];
#pragma unroll
    for (int u = 0; u < TPI; ++u) {
      s[u] = zero16();
#pragma unroll
      for (int cc = 0; cc < QC; ++cc) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(myk + u * VTILE + l32 * VROW + 32 * cc + 16 * hl);
        s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qhi[cc], s[u], 0, 0, 0);
        s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qlo[cc], s[u], 0, 0, 0);
      }
    }
    // mask keys past the chunk end, online softmax per column over TPI*32 keys
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < TPI; ++u) {
      const int k0 = kbeg + (t + u) * DEC_TILE;
      const bool tail = k0 + DEC_TILE > kcut;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        float v = s[u][a];
        if (tail && k0 + 8 * (a >> 2) + 4 * hl + (a & 3) >= (MULTI ? klim : kend)) v = -INFINITY;
        s[u][a] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    // a column can see no key yet only with several new tokens: keep its
    // state at (-inf, 0) instead of exp2(-inf + inf)
    const float m_use = (MULTI && m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < TPI; ++u)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float p = __builtin_amdgcn_exp2f(s[u][a] - m_use);
        s[u][a] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[i][a] *= alpha;
    // O^T += V^T P^T: k-slot sl of lane half hl <-> key 16*cc2 + 8*(sl/4) + 4*hl + sl%4
#pragma unroll
    for (int u = 0; u < TPI; ++u)
#pragma unroll
      for (int cc2 = 0; cc2 < 2; ++cc2) {
        bf16x8 pf;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) pf[sl] = (bf16)s[u][8 * cc2 + sl];
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          bf16x8 vf;
          if constexpr (D % 32 == 0) {
            // two transpose reads: keys 16 cc2 + 4 hl + 0..3 and + 8..11 of column 32 i + l32
            const unsigned char *p0 = myv + u * VTILE + 16 * cc2 * VROW + 64 * i + vtr_off;
            vf = tr_frag<bf16x8>(p0, p0 + 8 * VROW);
          } else {
            const int dd = 32 * i + l32;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
              const int key = 16 * cc2 + 8 * (sl >> 2) + 4 * hl + (sl & 3);
              vf[sl] = dd < D ? *reinterpret_cast<const bf16 *>(myv + u * VTILE + key * VROW + dd * 2)
                              : (bf16)0.f;
            }
          }
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[i], 0, 0, 0);
        }
      }
  }

  // merge the 4 waves: lane (column l32, half hl) holds O^T rows 8j + 4hl + i
  __syncthreads();                            // every wave is done with its V tiles
  if (col_ok) {
    RedRow &row = red[wave * MAXG + l32];
    if (hl == 0) {
      row[0] = m_run;
      row[1] = l_run;
    }
#pragma unroll
    for (int i = 0; i < ND; ++i)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int dd = 32 * i + 8 * (a >> 2) + 4 * hl + (a & 3);
        if (dd < D) row[2 + dd] = acc[i][a];
      }
  }
  __syncthreads();
  for (int e = tid; e < GH * D; e += 256) {
    const int hh = e / D, dd = e % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w * MAXG + hh][0]);
    float ll = 0.f, oo = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2_or_zero(red[w * MAXG + hh][0], mm);
      ll += red[w * MAXG + hh][1] * f;
      oo += red[w * MAXG + hh][2 + dd] * f;
    }
    size_t prow;
    if constexpr (MULTI) {
      const int pr = sub * GH + hh;
      if (pr >= G * m) continue;
      prow = (size_t)(b * Hq + g * G + pr / m) * m + pr % m;
    } else {
      prow = (size_t)(b * Hq + h0 + hh);
    }
    float *dst = part + (prow * nch + c) * (D + 2);
    dst[2 + dd] = oo;
    if (dd == 0) {
      dst[0] = mm;
      dst[1] = ll;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 cache (validation mode): same split and merge, VALU arithmetic
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_decode_f32_kernel(const float *__restrict__ q,
                                                              const float *__restrict__ tau,
                                                              const float *__restrict__ kc,
                                                              const float *__restrict__ vc,
                                                              StateOut cm, int Lk,
                                                              const int *__restrict__ lens, int chunk,
                                                              int Hq,
                                                              int Hkv, int G, int GH, int nsub,
                                                              int nch, int m,
                                                              float *__restrict__ part) {
  // one thread per (column, key) score, a column being a (query head, new
  // token) pair; waves walk the chunk in 256-key steps
  __shared__ float qs[DEC_F32_MAXG][D];
  __shared__ float pbuf[DEC_F32_MAXG][256];
  __shared__ float mst[DEC_F32_MAXG], lst[DEC_F32_MAXG], alph[DEC_F32_MAXG];
  __shared__ float oacc[DEC_F32_MAXG][D];
  const int tid = threadIdx.x;
  int id = blockIdx.x;
  const int c = id % nch; id /= nch;
  const int sub = id % nsub; id /= nsub;
  const int g = id % Hkv, b = id / Hkv;
  const int P = G * m;                           // columns of this (b, g)
  auto col_head = [&](int hh) { return g * G + min(sub * GH + hh, P - 1) / m; };
  auto col_tok = [&](int hh) { return min(sub * GH + hh, P - 1) % m; };
  for (int e = tid; e < GH * D; e += 256) {
    const int hh = e / D, dd = e % D;
    const int h = col_head(hh), j = col_tok(hh);
    qs[hh][dd] = q[((size_t)(b * m + j) * Hq + h) * D + dd] * tau[h] * 1.4426950408889634f;
    oacc[hh][dd] = 0.f;
  }
  for (int e = tid; e < GH; e += 256) { mst[e] = -INFINITY; lst[e] = 0.f; }
  __syncthreads();
  const int Lkb = lens ? min(max(lens[b], 0), Lk - m) + m : Lk;
  const int kbeg = c * chunk, kend = min(kbeg + chunk, Lkb);
  auto row_of = [&](int key) { return cache_row(cm, b, Hkv, g, key); };
  for (int k0 = kbeg; k0 < kend; k0 += 256) {
    const int key = k0 + tid;
    for (int hh = 0; hh < GH; ++hh) {
      float s = -INFINITY;
      if (key < min(kend, Lkb - m + col_tok(hh) + 1)) {
        s = 0.f;
        const float *kr = kc + row_of(key) * D;
        for (int dd = 0; dd < D; ++dd) s = fmaf(qs[hh][dd], kr[dd], s);
      }
      pbuf[hh][tid] = s;
    }
    __syncthreads();
    for (int hh = tid; hh < GH; hh += 256) {
      float mx = mst[hh];
      for (int j = 0; j < 256; ++j) mx = fmaxf(mx, pbuf[hh][j]);
      const float a = exp2_or_zero(mst[hh], mx);
      float ls = 0.f;
      for (int j = 0; j < 256; ++j) {
        const float p = exp2_or_zero(pbuf[hh][j], mx);
        pbuf[hh][j] = p;
        ls += p;
      }
      lst[hh] = lst[hh] * a + ls;
      mst[hh] = mx;
      alph[hh] = a;
    }
    __syncthreads();
    for (int e = tid; e < GH * D; e += 256) {
      const int hh = e / D, dd = e % D;
      float o = oacc[hh][dd] * alph[hh];
      const int n = min(256, kend - k0);
      for (int j = 0; j < n; ++j) o = fmaf(pbuf[hh][j], vc[row_of(k0 + j) * D + dd], o);
      oacc[hh][dd] = o;
    }
    __syncthreads();
  }
  for (int e = tid; e < GH * D; e += 256) {
    const int hh = e / D, dd = e % D;
    if (sub * GH + hh >= P) continue;
    const size_t prow = (size_t)(b * Hq + col_head(hh)) * m + col_tok(hh);
    float *dst = part + (prow * nch + c) * (D + 2);
    dst[2 + dd] = oacc[hh][dd];
    if (dd == 0) { dst[0] = mst[hh]; dst[1] = lst[hh]; }
  }
}

// o[b, h*D + dd] = sum_c 2^(m_c - M) o_c[dd] / sum_c 2^(m_c - M) l_c
// (part row (b*Hq + h)*m + j holds new token j of head h; o is [B*m, Hq*D])
template <typename TV, int D>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(const float *__restrict__ part,
                                                                  int nch, int Hq, int m,
                                                                  TV *__restrict__ o) {
  __shared__ float wts[1024];
  __shared__ float red[256 / D > 0 ? 256 / D : 1][D];
  __shared__ float s_m, s_l;
  const int bh = blockIdx.x, tid = threadIdx.x;   // bh = (b * Hq + h) * m + j
  const float *p = part + (size_t)bh * nch * (D + 2);
  if (tid < 64) {
    float mm = -INFINITY;
    for (int c = tid; c < nch; c += 64) mm = fmaxf(mm, p[(size_t)c * (D + 2)]);
    for (int o2 = 32; o2 >= 1; o2 >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o2, 64));
    float ll = 0.f;
    for (int c = tid; c < nch; c += 64) {
      const float w = exp2_or_zero(p[(size_t)c * (D + 2)], mm);
      if (c < 1024) wts[c] = w;
      ll += w * p[(size_t)c * (D + 2) + 1];
    }
    for (int o2 = 32; o2 >= 1; o2 >>= 1) ll += __shfl_xor(ll, o2, 64);
    if (tid == 0) { s_m = mm; s_l = ll; }
  }
  __syncthreads();
  constexpr int NG = 256 / D > 0 ? 256 / D : 1;   // chunk groups
  const int dd = tid % D, grp = tid / D;
  if (grp < NG) {
    float oo = 0.f;
    for (int c = grp; c < nch; c += NG) {
      const float w = c < 1024 ? wts[c] : exp2_or_zero(p[(size_t)c * (D + 2)], s_m);
      oo += w * p[(size_t)c * (D + 2) + 2 + dd];
    }
    red[grp][dd] = oo;
  }
  __syncthreads();
  if (tid < D) {
    float oo = 0.f;
    for (int gi = 0; gi < NG; ++gi) oo += red[gi][tid];
    const int bb = bh / (Hq * m), h = (bh / m) % Hq, j = bh % m;
    o[((size_t)(bb * m + j) * Hq + h) * D + tid] = from_f32<TV>(oo / s_l);
  }
}

template <int D>
static hipError_t dec_bf16(const MixShape &s, const float *q, const StateOut &cm, int Lk,
                           const int *lens, const float *tau, float *part, bf16 *o,
                           hipStream_t stream) {
  const int m = s.T;                                   // new tokens per sequence
  const int nch = dec_num_chunks(s.B, s.Hkv, Lk);
  const int chunk = dec_chunk_len(Lk, nch);
  const int GH = m == 1 ? dec_heads_per_wg(s.G, DecMaxG<D>::value)
                        : (s.G * m < DecMaxG<D>::value ? s.G * m : DecMaxG<D>::value);
  const int nsub = (s.G * m + GH - 1) / GH;
  const bf16 *kc = reinterpret_cast<const bf16 *>(cm.k_cache);
  const bf16 *vc = reinterpret_cast<const bf16 *>(cm.v_cache);
  const dim3 grid(nch * nsub * s.B * s.Hkv);
  if (cm.table && (chunk + cm.page - 1) / cm.page + 1 > DEC_MAX_PAGES) return hipErrorInvalidValue;
#define DEC_LAUNCH(VL, PG, MU)                                                                  \
  hipLaunchKernelGGL((attn_decode_mfma_kernel<D, VL, PG, MU>), grid, dim3(256), 0, stream, q, tau, \
                     kc, vc, cm, Lk, lens, chunk, s.Hq, s.Hkv, s.G, GH, nsub, nch, m, part)
  if (m > 1) {   // several new tokens: per-sequence lengths, contiguous or paged
    if (cm.table) DEC_LAUNCH(true, true, true);
    else DEC_LAUNCH(true, false, true);
  } else if (cm.table) {   // paged caches serve batches of per-sequence lengths
    DEC_LAUNCH(true, true, false);
  } else if (lens) {
    DEC_LAUNCH(true, false, false);
  } else {
    DEC_LAUNCH(false, false, false);
  }
#undef DEC_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_combine_kernel<bf16, D>), dim3(s.B * s.Hq * m), dim3(256), 0,
                     stream, part, nch, s.Hq, m, o);
  return hipGetLastError();
}

template <int D>
static hipError_t dec_f32(const MixShape &s, const float *q, const StateOut &cm, int Lk,
                          const int *lens, const float *tau, float *part, float *o,
                          hipStream_t stream) {
  const int m = s.T;
  const int nch = dec_num_chunks(s.B, s.Hkv, Lk);
  const int chunk = dec_chunk_len(Lk, nch);
  const int GH = m == 1 ? dec_heads_per_wg(s.G, DEC_F32_MAXG)
                        : (s.G * m < DEC_F32_MAXG ? s.G * m : DEC_F32_MAXG);
  const int nsub = (s.G * m + GH - 1) / GH;
  hipLaunchKernelGGL((attn_decode_f32_kernel<D>), dim3(nch * nsub * s.B * s.Hkv), dim3(256), 0,
                     stream, q, tau, reinterpret_cast<const float *>(cm.k_cache),
                     reinterpret_cast<const float *>(cm.v_cache), cm, Lk, lens, chunk, s.Hq, s.Hkv,
                     s.G, GH, nsub, nch, m, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_combine_kernel<float, D>), dim3(s.B * s.Hq * m), dim3(256), 0,
                     stream, part, nch, s.Hq, m, o);
  return hipGetLastError();
}

template <>
hipError_t launch_attention_decode<bf16>(const MixShape &s, const float *q, const StateOut &cm,
                                         int Lk, const int *lens, const float *tau, float *part,
                                         bf16 *o, hipStream_t stream) {
  switch (s.d) {
    case 16: return dec_bf16<16>(s, q, cm, Lk, lens, tau, part, o, stream);
    case 32: return dec_bf16<32>(s, q, cm, Lk, lens, tau, part, o, stream);
    case 64: return dec_bf16<64>(s, q, cm, Lk, lens, tau, part, o, stream);
    case 128: return dec_bf16<128>(s, q, cm, Lk, lens, tau, part, o, stream);
  }
  return hipErrorInvalidValue;
}

template <>
hipError_t launch_attention_decode<float>(const MixShape &s, const float *q, const StateOut &cm,
                                          int Lk, const int *lens, const float *tau, float *part,
                                          float *o, hipStream_t stream) {
  switch (s.d) {
    case 16: return dec_f32<16>(s, q, cm, Lk, lens, tau, part, o, stream);
    case 32: return dec_f32<32>(s, q, cm, Lk, lens, tau, part, o, stream);
    case 64: return dec_f32<64>(s, q, cm, Lk, lens, tau, part, o, stream);
    case 128: return dec_f32<128>(s, q, cm, Lk, lens, tau, part, o, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace cca
