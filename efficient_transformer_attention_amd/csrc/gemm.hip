// Projection GEMMs of the CCA forward pass (gfx950).
//
//   down-projection  qkv~[M, N] = x[M, E] * W_qkv[N, E]^T      (N = e_q + 2 e_kv)
//   up-projection    y[M, E]    = O[M, e_q] * W_o[E, e_q]^T
// [GS-EN "2. Methodology" / Down-Projection; the output returns to width E
//  after attention, which happens entirely in the latent space.]
//
// Both are "NT" products C = A * B^T with A and B contiguous along the
// contraction index, the native operand layout of MFMA.  One kernel serves
// bf16 (v_mfma_f32_32x32x16_bf16) and fp32 (v_mfma_f32_32x32x2_f32) inputs with
// fp32 accumulation.  Block tile BM x BN x BK with 4 waves (2 x 2), each wave
// owning (BM/2) x (BN/2) as 32 x 32 MFMA tiles; A and B tiles are staged in
// LDS with a 16-byte XOR swizzle, double buffered, one barrier per K step.
// Rows of 128 bytes per tile row: BK = 64 (bf16) or 32 (fp32).
#include "cca_device.h"
#include "gemm_tile.h"
#include "cca_launch.h"

namespace cca {

// blockIdx.y selects a slice [y*kchunk, (y+1)*kchunk) of the contraction;
// with more than one slice, C points at fp32 partial sums laid out
// [gridDim.y][M][ldc] and a reduction kernel finishes the product.
template <typename Tin, typename Tout, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const Tin *__restrict__ A,
                                                      const Tin *__restrict__ Bm,
                                                      Tout *__restrict__ C, int M, int N,
                                                      int K, int lda, int ldb, int ldc,
                                                      int kchunk) {
  typedef Mfma32<Tin> MF;
  constexpr int KS = MF::KS;
  constexpr int ROWB = 128;                       // bytes per LDS tile row
  constexpr int BK = ROWB / (int)sizeof(Tin);     // 64 (bf16) / 32 (fp32)
  constexpr int EPC = 16 / (int)sizeof(Tin);      // elements per 16-byte chunk
  constexpr int CPR = ROWB / 16;                  // chunks per row (8)
  constexpr int WM = BM / 2, WN = BN / 2;         // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;       // MFMA tiles per wave
  constexpr int A_CH = BM * CPR / 256;            // 16-byte chunks per thread
  constexpr int B_CH = BN * CPR / 256;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * (BM + BN) * ROWB];
  // buffer `buf`: A tile at smem + buf*(BM+BN)*ROWB, B tile right after it
  auto sA = [&](int buf) { return smem + buf * (BM + BN) * ROWB; };
  auto sB = [&](int buf) { return smem + buf * (BM + BN) * ROWB + BM * ROWB; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hl = lane >> 5;

  const int ntn = (N + BN - 1) / BN;
  const int ntm = (M + BM - 1) / BM;
  const int lid = xcd_remap(blockIdx.x, ntn * ntm);
  const int m0 = (lid / ntn) * BM;
  const int n0 = (lid % ntn) * BN;

  // prefetched global data of the next K tile
  u32x4 ra[A_CH], rb[B_CH];

  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < A_CH; ++r) {
      int c = tid + 256 * r;
      int row = c / CPR, ch = c % CPR;
      int gm = m0 + row, gk = k0 + ch * EPC;
      ra[r] = (gm < M && gk < K) ? ld16(A + (size_t)gm * lda + gk) : zero_u32x4();
    }
#pragma unroll
    for (int r = 0; r < B_CH; ++r) {
      int c = tid + 256 * r;
      int row = c / CPR, ch = c % CPR;
      int gn = n0 + row, gk = k0 + ch * EPC;
      rb[r] = (gn < N && gk < K) ? ld16(Bm + (size_t)gn * ldb + gk) : zero_u32x4();
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < A_CH; ++r) {
      int c = tid + 256 * r;
      int row = c / CPR, ch = c % CPR;
      st16(sA(buf) + row * ROWB + swz(row, ch * 16, CPR), ra[r]);
    }
#pragma unroll
    for (int r = 0; r < B_CH; ++r) {
      int c = tid + 256 * r;
      int row = c / CPR, ch = c % CPR;
      st16(sB(buf) + row * ROWB + swz(row, ch * 16, CPR), rb[r]);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero16();

  constexpr int KK = BK / (2 * KS);               // MFMA steps per K tile
  const int kbeg = blockIdx.y * kchunk;
  const int nk = (min(K, kbeg + kchunk) - kbeg + BK - 1) / BK;
  C += (size_t)blockIdx.y * M * ldc;
  gload(kbeg);
  lstore(0);
  __syncthreads();

  // one K tile: the fragments of MFMA step kk+1 are read from LDS while the
  // MFMAs of step kk run (two fragment sets)
  auto ktile = [&](int cur) {
    typename MF::frag fa[2][TM], fb[2][TN];
    auto fread = [&](int kk, int set) {
      const int kb = (kk * 2 * KS + hl * KS) * (int)sizeof(Tin);   // byte offset in row
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int row = wm * WM + i * 32 + l32;
        fa[set][i] = load_frag<Tin>(reinterpret_cast<const Tin *>(sA(cur) + row * ROWB + swz(row, kb, CPR)));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int row = wn * WN + j * 32 + l32;
        fb[set][j] = load_frag<Tin>(reinterpret_cast<const Tin *>(sB(cur) + row * ROWB + swz(row, kb, CPR)));
      }
    };
    fread(0, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) fread(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(fa[kk & 1][i], fb[kk & 1][j], acc[i][j]);
    }
  };

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kbeg + (kt + 1) * BK);
    ktile(cur);
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[8j + 4*hl + i][l32] of each 32x32 tile
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int gn = n0 + wn * WN + j * 32 + l32;
      if (gn >= N) continue;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int gm = m0 + wm * WM + i * 32 + 8 * (a >> 2) + 4 * hl + (a & 3);
        if (gm < M) C[(size_t)gm * ldc + gn] = from_f32<Tout>(acc[i][j][a]);
      }
    }
}

// ---------------------------------------------------------------------------
// bf16 inputs, whole 32-element K tiles: the same product with the A and B
// tiles streamed straight from HBM into LDS (buffer_load ... lds, no register
// staging) through a ring of STAGES tiles, and the MFMA fragments double
// buffered in registers: while the MFMAs of K tile k run, the fragments of
// tile k + 1 are read from LDS and tiles up to k + STAGES - 2 are in flight.
//   K tile = 32 elements: LDS rows of 64 bytes (4 chunks of 16 bytes), chunk
//   swizzle f(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1) (no bank conflicts for 8-
//   or 16-lane phases).  A DMA instruction fills 1 KiB = 16 rows; lane l
//   writes LDS bytes [16 l, 16 l + 16) of it, so each lane fetches the global
//   chunk that the swizzle places there.  Rows past M / N read as zero (buffer
//   range check).
// ---------------------------------------------------------------------------
// Tile (tm, tn) of workgroup bid on a tile grid of ntm x ntn.  The hardware
// deals workgroup ids round-robin to the 8 XCDs; with py in {1, 2, 4, 8} the
// XCDs form a (8/py) x py grid over the tiles, XCD bid % 8 owning a band of
// ntm/(8/py) x ntn/py tiles that it walks row by row in dispatch order
// (bid / 8), so its L2 holds the band's columns of B while rows of A stream
// through.  py = 0: each XCD takes a contiguous run of tiles in row-major
// order (grids that do not split evenly).
__device__ __forceinline__ void xcd_tile(int bid, int ntm, int ntn, int py, int &tm, int &tn) {
  if (py == 0) {
    const int lid = xcd_remap(bid, ntm * ntn);
    tm = lid / ntn;
    tn = lid % ntn;
    return;
  }
  const int px = 8 / py, bm = ntm / px, bn = ntn / py;
  const int x = bid & 7, slot = bid >> 3;
  tm = (x / py) * bm + slot / bn;
  tn = (x % py) * bn + slot % bn;
}

// The XCD split for xcd_tile: among the splits that divide the tile grid, the
// one with the fewest bytes brought into the L2s, py |A| + (8/py) |B| (each
// XCD reads its rows of A and its columns of B once); ties go to the larger
// py, whose narrower band of B is likelier to stay in L2.  0 when none
// divides the grid.
static int xcd_split(int ntm, int ntn, double abytes, double bbytes) {
  int best = 0;
  double bc = 0.0;
  for (int py = 1; py <= 8; py *= 2) {
    const int px = 8 / py;
    if (ntm % px || ntn % py) continue;
    const double c = py * abytes + px * bbytes;
    if (best == 0 || c <= bc * (1.0 + 1e-9)) {
      best = py;
      bc = c;
    }
  }
  return best;
}

template <typename Tout, int BM, int BN, int BK, int STAGES, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_nt_dma_kernel(const bf16 *__restrict__ A,
                                                             const bf16 *__restrict__ Bm,
                                                             Tout *__restrict__ C, int M, int N,
                                                             int K, int lda, int ldb, int ldc,
                                                             int kchunk, int xsplit) {
  typedef Mfma32<bf16> MF;
  typedef MF::frag Frag;
  constexpr int ROWB = BK * 2, CPR = ROWB / 16, KK = BK / 16;   // row bytes, chunks, k-chunks
  static_assert(BK == 32 || BK == 64, "K tile");
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int A_INS = BM * ROWB / 1024, B_INS = BN * ROWB / 1024;   // DMA instructions per stage
  constexpr int PER_WAVE = (A_INS + B_INS) / 4;
  static_assert(A_INS % 4 == 0 && B_INS % 4 == 0, "DMA split over 4 waves");
  static_assert(STAGES >= 3 && (STAGES - 3) * PER_WAVE < 16, "vmcnt field");
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGES * STAGE];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hl = lane >> 5;
  const int ntn = (N + BN - 1) / BN, ntm = (M + BM - 1) / BM;
  int tm, tn;
  xcd_tile(blockIdx.x, ntm, ntn, xsplit, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  // split contraction: slice blockIdx.y covers K range [kbeg, kbeg + kchunk)
  // and writes its own M x ldc block of C
  const int kbeg = blockIdx.y * kchunk;
  C += (size_t)blockIdx.y * M * ldc;

  f32x16 acc[TM][TN];
  dma_gemm_tile<BM, BN, BK, STAGES>(A, Bm, M, N, lda, ldb, m0, [&](int r) { return n0 + r; },
                                    kbeg, min(kchunk, K - kbeg), smem, acc);

  const bool full = m0 + BM <= M && n0 + BN <= N;   // workgroup-uniform
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int gn = n0 + wn * WN + j * 32 + l32;
      Tout *cp = C + (size_t)(m0 + wm * WM + i * 32 + 4 * hl) * ldc + gn;
      if (full) {
#pragma unroll
        for (int a = 0; a < 16; ++a)
          cp[(size_t)(8 * (a >> 2) + (a & 3)) * ldc] = from_f32<Tout>(acc[i][j][a]);
      } else if (gn < N) {
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int r = 8 * (a >> 2) + (a & 3);
          if (m0 + wm * WM + i * 32 + 4 * hl + r < M) cp[(size_t)r * ldc] = from_f32<Tout>(acc[i][j][a]);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Token-major operands: C[m][n] = sum_k A[k][m] B[k][n] with A [K][lda] and
// B [K][ldb] row-major, i.e. the contraction runs over rows (the weight
// gradients dW_o = dy^T O and dW_qkv = dz^T x contract over tokens).  Same
// ring, barriers and MFMA schedule as gemm_nt_dma_kernel; what changes is the
// layout:
//   * a stage holds 32 k-rows of BM (A) and BN (B) elements as they lie in
//     memory (rows of 256 bytes for 128 columns), 16-byte chunks XOR-swizzled
//     by ((k & 3) << 2), so the four k-rows that one fragment read touches sit
//     in four different 64-byte bank groups;
//   * the fragments come out with ds_read_b64_tr_b16: inside each 16-lane
//     group, lane 4j + q fetches columns [c + 4q, c + 4q + 4) of k-row k0 + j
//     and the instruction hands lane i the four k-rows k0 .. k0 + 3 of column
//     c + i.  Two such reads (k0 and k0 + 4) give a lane the 8 consecutive k
//     of one column that the 32 x 32 x 16 MFMA operand holds.
// k-rows at or past K read as zero through the buffer range check, so K needs
// no padding; M and N must be multiples of the block tile.
// ---------------------------------------------------------------------------
template <int BM, int BN, int STAGES>
__device__ __forceinline__ void dma_gemm_tile_tn(const bf16 *__restrict__ A,
                                                 const bf16 *__restrict__ Bm, int K, int lda,
                                                 int ldb, int m0, int n0, int kbeg, int klen,
                                                 unsigned char *smem,
                                                 f32x16 (&acc)[BM / 64][BN / 64]) {
  typedef Mfma32<bf16> MF;
  typedef MF::frag Frag;
  constexpr int BK = 32, KK = 2;
  constexpr int ROWA = BM * 2, ROWB = BN * 2;          // bytes per k-row
  constexpr int CPA = ROWA / 16, CPB = ROWB / 16;      // 16-byte chunks per k-row
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int ATILE = BK * ROWA, STAGE = BK * (ROWA + ROWB);
  constexpr int A_INS = ATILE / 1024, B_INS = BK * ROWB / 1024;   // DMA instructions per stage
  constexpr int PER_WAVE = (A_INS + B_INS) / 4;
  static_assert(CPA >= 16 && CPB >= 16 && 1024 % ROWA == 0 && 1024 % ROWB == 0,
                "the swizzle moves chunk bits 2..3 inside rows of 16 or more chunks");
  static_assert(A_INS % 4 == 0 && B_INS % 4 == 0, "DMA split over 4 waves");
  static_assert(STAGES >= 3 && (STAGES - 3) * PER_WAVE < 16, "vmcnt field");
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const unsigned a_bytes = (unsigned)((size_t)K * lda * 2), b_bytes = (unsigned)((size_t)K * ldb * 2);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)Bm, 0, b_bytes, 0x00020000);

  // DMA instruction u of wave w moves 1 KiB piece u*4 + w of a stage (A
  // first).  Lane l writes LDS bytes [16 l, 16 l + 16) of the piece: k-row
  // l / CP of it, physical chunk l % CP, which holds logical chunk
  // (l % CP) ^ ((row & 3) << 2).  Per lane: the byte offset inside k-tile 0.
  unsigned doff[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    constexpr int AU = A_INS / 4;
    const bool isA = u < AU;
    const int cp = isA ? CPA : CPB;
    const int row = ((isA ? u : u - AU) * 4 + wave) * (64 / cp) + lane / cp;
    const int chunk = (lane % cp) ^ ((row & 3) << 2);
    doff[u] = isA ? (unsigned)(((size_t)row * lda + m0 + chunk * 8) * 2)
                  : (unsigned)(((size_t)row * ldb + n0 + chunk * 8) * 2);
  }
  auto issue = [&](int kt, int slot) {
    unsigned char *base = smem + slot * STAGE + wave * 1024;
    const int krow = kbeg + kt * BK;
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const bool isA = u < A_INS / 4;
      unsigned char *dst = isA ? base + u * 4096 : base + ATILE + (u - A_INS / 4) * 4096;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? ra : rb, as_lds(dst), 16, (int)doff[u],
                                               krow * (isA ? lda : ldb) * 2, 0, 0);
    }
  };

  // per-lane LDS byte offsets of the transpose reads for k-chunk 0, first
  // half: lane 16g + 4j + q reads k-row 8 (g >> 1) + j at column
  // 16 (g & 1) + 4q of its 32-column MFMA tile.  The other k-chunk and half
  // are +16 and +4 rows, which leave the swizzle unchanged.
  const int g = lane >> 4, jr = (lane >> 2) & 3, q = lane & 3;
  const int krow0 = 8 * (g >> 1) + jr;
  int aoff[TM], boff[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int col = wm * WM + i * 32 + 16 * (g & 1) + 4 * q;
    aoff[i] = krow0 * ROWA + (((col >> 3) ^ ((krow0 & 3) << 2)) << 4) + (col & 7) * 2;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = wn * WN + j * 32 + 16 * (g & 1) + 4 * q;
    boff[j] = ATILE + krow0 * ROWB + (((col >> 3) ^ ((krow0 & 3) << 2)) << 4) + (col & 7) * 2;
  }
  auto frag = [&](const unsigned char *p, int rowbytes, int kk) {
    return tr_frag<Frag>(p + kk * 16 * rowbytes, p + (kk * 16 + 4) * rowbytes);
  };
  auto load = [&](int slot, Frag (&fa)[KK][TM], Frag (&fb)[KK][TN]) {
    const unsigned char *sbase = smem + slot * STAGE;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[kk][i] = frag(sbase + aoff[i], ROWA, kk);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[kk][j] = frag(sbase + boff[j], ROWB, kk);
    }
  };

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero16();
  auto mma = [&](Frag (&fa)[KK][TM], Frag (&fb)[KK][TN]) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(fa[kk][i], fb[kk][j], acc[i][j]);
  };
  auto wait_stages = [&](int n) {
    if constexpr (STAGES >= 5) {
      if (n >= 2) { wait_vmcnt<2 * PER_WAVE>(); return; }
    }
    if constexpr (STAGES >= 4) {
      if (n >= 1) { wait_vmcnt<PER_WAVE>(); return; }
    }
    wait_vmcnt<0>();
  };

  const int nk = (klen + BK - 1) / BK;
  auto iter = [&](int kt, Frag (&ca)[KK][TM], Frag (&cb)[KK][TN], Frag (&na)[KK][TM],
                  Frag (&nb)[KK][TN]) {
    wait_stages(min(nk, kt + STAGES - 1) - (kt + 2));
    lds_barrier();
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    load((kt + 1) % STAGES, na, nb);
    mma(ca, cb);
  };

#pragma unroll
  for (int s0 = 0; s0 < STAGES - 1; ++s0)
    if (s0 < nk) issue(s0, s0);
  wait_stages(min(nk, STAGES - 1) - 1);
  lds_barrier();
  Frag fa0[KK][TM], fb0[KK][TN], fa1[KK][TM], fb1[KK][TN];
  load(0, fa0, fb0);
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    iter(kt, fa0, fb0, fa1, fb1);
    iter(kt + 1, fa1, fb1, fa0, fb0);
  }
  if (kt + 1 < nk) {
    iter(kt, fa0, fb0, fa1, fb1);
    mma(fa1, fb1);
  } else {
    mma(fa0, fb0);
  }
}

// C (+ blockIdx.y * M * ldc with split slices) = A^T B over the k-rows
// [blockIdx.y * kchunk, min(K, (blockIdx.y + 1) * kchunk)); fp32 out.
template <int BM, int BN, int STAGES, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_tn_dma_kernel(const bf16 *__restrict__ A,
                                                             const bf16 *__restrict__ Bm,
                                                             float *__restrict__ C, int M, int N,
                                                             int K, int lda, int ldb, int ldc,
                                                             int kchunk) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGES * 32 * (BM + BN) * 2];
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hl = lane >> 5;
  const int ntn = N / BN, ntm = M / BM;
  const int lid = xcd_remap(blockIdx.x, ntn * ntm);
  const int m0 = (lid / ntn) * BM, n0 = (lid % ntn) * BN;
  const int kbeg = blockIdx.y * kchunk;
  C += (size_t)blockIdx.y * M * ldc;
  f32x16 acc[TM][TN];
  dma_gemm_tile_tn<BM, BN, STAGES>(A, Bm, K, lda, ldb, m0, n0, kbeg, min(kchunk, K - kbeg), smem,
                                   acc);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float *cp = C + (size_t)(m0 + wm * WM + i * 32 + 4 * hl) * ldc + n0 + wn * WN + j * 32 + l32;
#pragma unroll
      for (int a = 0; a < 16; ++a) cp[(size_t)(8 * (a >> 2) + (a & 3)) * ldc] = acc[i][j][a];
    }
}

// out[i] = sum over the S slices of part[s][i], i < n (n a multiple of 4)
template <typename Tout>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part,
                                                            Tout *__restrict__ out, size_t n,
                                                            int S) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4 *>(part + i);
  for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const f32x4 *>(part + (size_t)s * n + i);
#pragma unroll
  for (int e = 0; e < 4; ++e) out[i + e] = from_f32<Tout>(acc[e]);
}

int gemm_splitk_slices(int M, int N, int K, int elem_bytes) {
  const int BK = 128 / elem_bytes;
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  const int ksteps = (K + BK - 1) / BK;
  int S = 512 / tiles;
  if (S > ksteps / 2) S = ksteps / 2;
  if (S > 16) S = 16;
  return S < 1 ? 1 : S;
}

template <typename Tin, typename Tout>
hipError_t launch_gemm_nt(const Tin *A, const Tin *B, Tout *C, int M, int N, int K, int lda,
                          int ldb, int ldc, hipStream_t stream, float *splitk_ws,
                          size_t splitk_floats) {
  if (M <= 64 && splitk_ws) {
    // skinny product (a decode step): 64 x 64 tiles and a split contraction so
    // the weight stream is spread over enough workgroups
    constexpr int BM = 64, BN = 64, BK = 128 / (int)sizeof(Tin);
    const int S = gemm_splitk_slices(M, N, K, (int)sizeof(Tin));
    const int ksteps = (K + BK - 1) / BK;
    const int kchunk = (ksteps + S - 1) / S * BK;
    const int Sused = (K + kchunk - 1) / kchunk;
    if ((size_t)Sused * M * ldc <= splitk_floats && ldc == N && (N % 4) == 0) {
      const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
      hipLaunchKernelGGL((gemm_nt_kernel<Tin, float, BM, BN>), dim3(grid, Sused), dim3(256), 0,
                         stream, A, B, splitk_ws, M, N, K, lda, ldb, ldc, kchunk);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const size_t n = (size_t)M * N;
      hipLaunchKernelGGL((splitk_reduce_kernel<Tout>), dim3((unsigned)((n / 4 + 255) / 256)),
                         dim3(256), 0, stream, splitk_ws, C, n, Sused);
      return hipGetLastError();
    }
  }
  constexpr int BM = 128, BN = 128;
  int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if constexpr (sizeof(Tin) == 2) {
    // whole 32-element K tiles, and operands small enough that every byte
    // offset (out-of-range ones included) fits the 32-bit buffer range check
    const size_t lim = (1ull << 32) - 2 * (size_t)K;
    if (K % 32 == 0 && (size_t)M * lda * 2 < lim && (size_t)N * ldb * 2 < lim) {
      // one 256 x 192 tile per CU when that covers the product in a single
      // round; 128 x 256 tiles for wide products with a long contraction (the
      // backward's dx = dz W_qkv at K = 1536: 12% faster than 128 x 128 there,
      // slower at K = 512 and no faster at K = 1024); else 128 x 128 tiles (two
      // workgroups per CU)
      const double ab = 2.0 * M * K, bb = 2.0 * N * K;
      const int g256 = ((M + 255) / 256) * ((N + 191) / 192);
      if (g256 >= 224 && g256 <= 256) {
        const int xs = xcd_split((M + 255) / 256, (N + 191) / 192, ab, bb);
        hipLaunchKernelGGL((gemm_nt_dma_kernel<Tout, 256, 192, 32, 5, 1>), dim3(g256), dim3(256), 0,
                           stream, A, B, C, M, N, K, lda, ldb, ldc, K, xs);
      } else if (N % 256 == 0 && N >= 2048 && K >= 1536 && M >= 4096) {
        const int g = ((M + 127) / 128) * (N / 256);
        const int xs = xcd_split((M + 127) / 128, N / 256, ab, bb);
        hipLaunchKernelGGL((gemm_nt_dma_kernel<Tout, 128, 256, 32, 5, 1>), dim3(g), dim3(256), 0,
                           stream, A, B, C, M, N, K, lda, ldb, ldc, K, xs);
      } else {
        const int xs = xcd_split((M + BM - 1) / BM, (N + BN - 1) / BN, ab, bb);
        hipLaunchKernelGGL((gemm_nt_dma_kernel<Tout, 128, 128, 32, 5, 2>), dim3(grid), dim3(256), 0,
                           stream, A, B, C, M, N, K, lda, ldb, ldc, K, xs);
      }
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_nt_kernel<Tin, Tout, BM, BN>), dim3(grid, 1), dim3(256), 0, stream, A,
                     B, C, M, N, K, lda, ldb, ldc, K);
  return hipGetLastError();
}

// The split-contraction product without its reduction: for M <= 64 and room
// for the slices, the S fp32 partial products [S][M][N] go to splitk_ws and
// S is returned; otherwise the product goes to C (fp32, ldc = N) and 0 is
// returned.  A consumer sums the slices in order s = 0 .. S-1 (the order of
// splitk_reduce_kernel).
int gemm_nt_partial_slices(int M, int N, int K, int elem_bytes, size_t splitk_floats) {
  if (M > 64 || (N % 4) != 0) return 0;
  const int BK = 128 / elem_bytes;
  const int S = gemm_splitk_slices(M, N, K, elem_bytes);
  const int ksteps = (K + BK - 1) / BK;
  const int kchunk = (ksteps + S - 1) / S * BK;
  const int Sused = (K + kchunk - 1) / kchunk;
  return (size_t)Sused * M * N <= splitk_floats ? Sused : 0;
}

template <typename Tin>
hipError_t launch_gemm_nt_partials(const Tin *A, const Tin *B, float *C, int M, int N, int K,
                                   int lda, int ldb, float *splitk_ws, size_t splitk_floats,
                                   int *slices, hipStream_t stream) {
  *slices = splitk_ws ? gemm_nt_partial_slices(M, N, K, (int)sizeof(Tin), splitk_floats) : 0;
  if (*slices == 0) return launch_gemm_nt<Tin, float>(A, B, C, M, N, K, lda, ldb, N, stream);
  constexpr int BM = 64, BN = 64, BK = 128 / (int)sizeof(Tin);
  const int S = gemm_splitk_slices(M, N, K, (int)sizeof(Tin));
  const int ksteps = (K + BK - 1) / BK;
  const int kchunk = (ksteps + S - 1) / S * BK;
  const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_nt_kernel<Tin, float, BM, BN>), dim3(grid, *slices), dim3(256), 0,
                     stream, A, B, splitk_ws, M, N, K, lda, ldb, N, kchunk);
  return hipGetLastError();
}

template hipError_t launch_gemm_nt_partials<bf16>(const bf16 *, const bf16 *, float *, int, int,
                                                  int, int, int, float *, size_t, int *,
                                                  hipStream_t);
template hipError_t launch_gemm_nt_partials<float>(const float *, const float *, float *, int, int,
                                                   int, int, int, float *, size_t, int *,
                                                   hipStream_t);

// Contraction slices for a product with few output tiles and a long K (the
// weight gradients): enough 128 x 128 tiles x slices for one round of two
// workgroups per CU (more slices only add fp32 partial traffic), slices of
// at least 1024 elements.
int gemm_long_k_slices(int M, int N, int K) {
  // 128 x 128 tiles, S slices of the contraction: each CU runs
  // ceil(tiles * S / 256) workgroups of K / S steps (two at a time).  Take the
  // S that minimises that product, the smaller S on a tie (less to reduce).
  const long long tiles = (long long)((M + 127) / 128) * ((N + 127) / 128);
  int maxs = K / 1024;
  if (maxs > 16) maxs = 16;
  int best = 1;
  long long best_cost = -1;
  for (int S = 1; S <= maxs; ++S) {
    const long long chunk = ((K + S - 1) / S + 31) / 32 * 32;
    const long long cost = (tiles * S + 255) / 256 * chunk;
    if (best_cost < 0 || cost < best_cost) {
      best = S;
      best_cost = cost;
    }
  }
  return best;
}

template <typename Tin>
hipError_t launch_gemm_nt_long_k(const Tin *A, const Tin *B, float *C, int M, int N, int K, int lda,
                                 int ldb, float *ws, size_t ws_floats, hipStream_t stream) {
  const int S = gemm_long_k_slices(M, N, K);
  if constexpr (sizeof(Tin) == 2) {
    const size_t lim = (1ull << 32) - 2 * (size_t)K;
    int kchunk = (K + S - 1) / S;
    kchunk = (kchunk + 31) / 32 * 32;
    const int Sused = (K + kchunk - 1) / kchunk;
    if (S > 1 && K % 32 == 0 && (size_t)M * lda * 2 < lim && (size_t)N * ldb * 2 < lim &&
        (size_t)Sused * M * N <= ws_floats && (size_t)M * N % 4 == 0) {
      const int grid = ((M + 127) / 128) * ((N + 127) / 128);
      hipLaunchKernelGGL((gemm_nt_dma_kernel<float, 128, 128, 32, 5, 2>), dim3(grid, Sused),
                         dim3(256), 0, stream, A, B, ws, M, N, K, lda, ldb, N, kchunk, 0);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const size_t n = (size_t)M * N;
      hipLaunchKernelGGL((splitk_reduce_kernel<float>), dim3((unsigned)((n / 4 + 255) / 256)),
                         dim3(256), 0, stream, ws, C, n, Sused);
      return hipGetLastError();
    }
  }
  return launch_gemm_nt<Tin, float>(A, B, C, M, N, K, lda, ldb, N, stream);
}

hipError_t launch_gemm_tn_long_k(const bf16 *A, const bf16 *B, float *C, int M, int N, int K,
                                 int lda, int ldb, float *ws, size_t ws_floats,
                                 hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const bool fits = M > 0 && N > 0 && K > 0 && M % BM == 0 && N % BN == 0 && lda % 8 == 0 &&
                    ldb % 8 == 0 && lda >= M && ldb >= N &&
                    reinterpret_cast<uintptr_t>(A) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(B) % 16 == 0 &&
                    (size_t)(K + 64) * lda * 2 < (1ull << 31) &&
                    (size_t)(K + 64) * ldb * 2 < (1ull << 31);
  if (!fits) return hipErrorNotSupported;
  const int S = gemm_long_k_slices(M, N, K);
  int kchunk = ((K + S - 1) / S + 31) / 32 * 32;
  int Sused = (K + kchunk - 1) / kchunk;
  if (Sused > 1 && (!ws || (size_t)Sused * M * N > ws_floats)) {
    Sused = 1;
    kchunk = K;
  }
  const int grid = (M / BM) * (N / BN);
  hipLaunchKernelGGL((gemm_tn_dma_kernel<BM, BN, 5, 2>), dim3(grid, Sused), dim3(256), 0, stream, A,
                     B, Sused > 1 ? ws : C, M, N, K, lda, ldb, N, kchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || Sused == 1) return e;
  const size_t n = (size_t)M * N;
  hipLaunchKernelGGL((splitk_reduce_kernel<float>), dim3((unsigned)((n / 4 + 255) / 256)), dim3(256),
                     0, stream, ws, C, n, Sused);
  return hipGetLastError();
}

template hipError_t launch_gemm_nt<bf16, float>(const bf16 *, const bf16 *, float *, int, int, int,
                                                int, int, int, hipStream_t, float *, size_t);
template hipError_t launch_gemm_nt<bf16, f16>(const bf16 *, const bf16 *, f16 *, int, int, int,
                                              int, int, int, hipStream_t, float *, size_t);
template hipError_t launch_gemm_nt<bf16, bf16>(const bf16 *, const bf16 *, bf16 *, int, int, int,
                                               int, int, int, hipStream_t, float *, size_t);
template hipError_t launch_gemm_nt<float, float>(const float *, const float *, float *, int, int,
                                                 int, int, int, int, hipStream_t, float *, size_t);

template hipError_t launch_gemm_nt_long_k<bf16>(const bf16 *, const bf16 *, float *, int, int, int,
                                                int, int, float *, size_t, hipStream_t);
template hipError_t launch_gemm_nt_long_k<float>(const float *, const float *, float *, int, int,
                                                 int, int, int, float *, size_t, hipStream_t);

}  // namespace cca
