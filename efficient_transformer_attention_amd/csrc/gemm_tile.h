// The DMA-fed MFMA main loop of one C tile of A * B^T (bf16 operands, fp32
// accumulators), shared by the GEMM kernels and the fused down-projection +
// mixing kernel (gfx950).
//   K tile = 32 elements: LDS rows of 64 bytes (4 chunks of 16 bytes), chunk
//   swizzle f(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1) (no bank conflicts for 8-
//   or 16-lane phases).  A DMA instruction fills 1 KiB = 16 rows; lane l
//   writes LDS bytes [16 l, 16 l + 16) of it, so each lane fetches the global
//   chunk that the swizzle places there.  Rows past M / N read as zero (buffer
//   range check).
#pragma once

#include "cca_device.h"

namespace cca {

__device__ __forceinline__ int swz4(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }
// 128-byte rows (8 chunks): f(r) = (r & 7) ^ ((r >> 3) & 1)
template <int CPR> __device__ __forceinline__ int swz_rows(int row) {
  if constexpr (CPR == 4) return swz4(row);
  else return (row & 7) ^ ((row >> 3) & 1);
}

// acc[TM][TN] (TM = BM / 64, TN = BN / 64; the 4 waves split the tile 2 x 2)
// = rows m0 .. m0 + BM of A times the B rows brow(0) .. brow(BN - 1) (an index
// >= N reads as zero), over the contraction range [kbeg, kbeg + klen), klen
// a multiple of BK.  smem: STAGES * (BM + BN) * 2 * BK bytes of LDS.
template <int BM, int BN, int BK, int STAGES, typename BRow>
__device__ __forceinline__ void dma_gemm_tile(const bf16 *__restrict__ A,
                                              const bf16 *__restrict__ Bm, int M, int N, int lda,
                                              int ldb, int m0, BRow brow, int kbeg, int klen,
                                              unsigned char *smem,
                                              f32x16 (&acc)[BM / 64][BN / 64]) {
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
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hl = lane >> 5;
  const unsigned a_bytes = (unsigned)((size_t)M * lda * 2), b_bytes = (unsigned)((size_t)N * ldb * 2);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)A, 0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)Bm, 0, b_bytes, 0x00020000);

  // DMA instruction u of wave w moves 1 KiB chunk u*4 + w of a stage: the
  // first A_INS/4 instructions of every wave load A, the rest B.  Per lane:
  // the byte offset of its chunk in K tile 0, or the operand's size for rows
  // past M / N, which the buffer range check turns into zeros.
  unsigned doff[PER_WAVE];
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    constexpr int AU = A_INS / 4;
    const bool isA = u < AU;
    const int row = ((isA ? u : u - AU) * 4 + wave) * (1024 / ROWB) + lane / CPR;
    const int chunk = (lane % CPR) ^ swz_rows<CPR>(row);
    const int grow = isA ? m0 + row : brow(row);
    doff[u] = grow < (isA ? M : N) ? (unsigned)(((size_t)grow * (isA ? lda : ldb) + chunk * 8) * 2)
                                   : (isA ? a_bytes : b_bytes);
  }
  const int nk = klen / BK;
  // SPREAD (tiles with at least 3 MFMAs per DMA instruction of a wave): the
  // refill DMAs and the next tile's fragment reads are placed among the
  // MFMAs instead of in a burst after the barrier.  Keeping them in the
  // MFMAs' basic block means issuing every refill, so tiles at or past nk go
  // out as reads past the operand (zeros, no memory access) into a slot that
  // is never read again, and every wave always has STAGES - 2 stages ahead.
  constexpr int NMMA = KK * TM * TN;
  constexpr bool SPREAD = NMMA >= 3 * PER_WAVE;
  auto issue = [&](int kt, int slot) {
    unsigned char *base = smem + slot * STAGE + wave * 1024;
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const bool isA = u < A_INS / 4;
      unsigned char *dst = isA ? base + u * 4096 : base + A_INS * 1024 + (u - A_INS / 4) * 4096;
      if constexpr (SPREAD) {
        const unsigned off = kt < nk ? doff[u] + (unsigned)((kbeg + kt * BK) * 2) : (isA ? a_bytes : b_bytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? ra : rb, as_lds(dst), 16, (int)off, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? ra : rb, as_lds(dst), 16, (int)doff[u],
                                                 (kbeg + kt * BK) * 2, 0, 0);
      }
    }
  };

  // per-lane LDS byte offsets of the MFMA fragments inside one stage
  int aoff[KK][TM], boff[KK][TN];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int chunk = 2 * kk + hl;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WM + i * 32 + l32;
      aoff[kk][i] = row * ROWB + ((chunk ^ swz_rows<CPR>(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WN + j * 32 + l32;
      boff[kk][j] = BM * ROWB + row * ROWB + ((chunk ^ swz_rows<CPR>(row)) << 4);
    }
  }
  auto load = [&](int slot, Frag (&fa)[KK][TM], Frag (&fb)[KK][TN]) {
    const unsigned char *sbase = smem + slot * STAGE;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[kk][i] = *reinterpret_cast<const Frag *>(sbase + aoff[kk][i]);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[kk][j] = *reinterpret_cast<const Frag *>(sbase + boff[kk][j]);
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
  // wait until at most n of this wave's DMA stages are still in flight
  auto wait_stages = [&](int n) {
    if constexpr (STAGES >= 5) {
      if (n >= 2) { wait_vmcnt<2 * PER_WAVE>(); return; }
    }
    if constexpr (STAGES >= 4) {
      if (n >= 1) { wait_vmcnt<PER_WAVE>(); return; }
    }
    wait_vmcnt<0>();
  };

  // iteration kt < nk - 1: tile kt + 1 is read into registers while tile kt
  // (already in registers) is multiplied; tiles up to kt + STAGES - 2 fly
  auto iter = [&](int kt, Frag (&ca)[KK][TM], Frag (&cb)[KK][TN], Frag (&na)[KK][TM],
                  Frag (&nb)[KK][TN]) {
    // tile kt + 1 landed: of the tiles issued so far, those after it may fly
    wait_stages(SPREAD ? STAGES - 3 : min(nk, kt + STAGES - 1) - (kt + 2));
    // every wave's DMA of tile kt + 1 has landed, and every read of the slot
    // refilled below (tile kt - 1, read during iteration kt - 2) is done
    lds_barrier();
    if (SPREAD || kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
    load((kt + 1) % STAGES, na, nb);
    mma(ca, cb);
    if constexpr (SPREAD) {
      // two fragment reads per MFMA, then one DMA per two MFMAs, then the rest
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      }
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM: the DMA
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMMA - 3 * PER_WAVE, 0);
    }
  };

#pragma unroll
  for (int s0 = 0; s0 < STAGES - 1; ++s0)
    if (SPREAD || s0 < nk) issue(s0, s0);
  wait_stages(SPREAD ? STAGES - 2 : min(nk, STAGES - 1) - 1);
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
  // the zero-fill DMAs of the tail land before the caller reuses LDS
  if constexpr (SPREAD) wait_vmcnt<0>();
}

}  // namespace cca
