// Device-side building blocks shared by the libcca kernels (gfx950 only).
//
// MFMA conventions used throughout (32x32 output tiles, wave64):
//   A operand (M x K): lane l supplies row (l % 32), k-slots (l / 32) * KS .. + KS-1
//   B operand (K x N): lane l supplies column (l % 32), the same k-slots
//   C / accumulator:   lane l holds C[8*j + 4*(l/32) + i][l % 32] in acc[4*j + i]
// KS = 8 for the 16-bit types (v_mfma_f32_32x32x16_{bf16,f16}) and 1 for fp32
// (v_mfma_f32_32x32x2_f32).  Only the pairing of A's and B's k-slots matters
// for a product, so any bijection between k-slots and the contraction index
// is valid as long as A and B use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cca {

typedef __bf16 bf16;
typedef _Float16 f16;

typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ float to_f32(T v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return (T)v; }

// ---------------------------------------------------------------------------
// MFMA traits: one 32x32 tile, contraction chunk of 2*KS per instruction
// ---------------------------------------------------------------------------
template <typename T> struct Mfma32;

template <> struct Mfma32<bf16> {
  static constexpr int KS = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma32<f16> {
  static constexpr int KS = 8;
  typedef f16x8 frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma32<float> {
  static constexpr int KS = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Load KS consecutive elements (one fragment) from LDS or global memory.
template <typename T>
__device__ __forceinline__ typename Mfma32<T>::frag load_frag(const T *p) {
  return *reinterpret_cast<const typename Mfma32<T>::frag *>(p);
}

// Pack KS fp32 values into a fragment of type T.
template <typename T>
__device__ __forceinline__ typename Mfma32<T>::frag pack_frag(const float *v) {
  typename Mfma32<T>::frag f;
  if constexpr (Mfma32<T>::KS == 1) {
    f = (T)v[0];
  } else {
#pragma unroll
    for (int s = 0; s < Mfma32<T>::KS; ++s) f[s] = (T)v[s];
  }
  return f;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------------------
// 16-byte vector memory helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Inside each group of 16
// lanes, lane 4j + q gives the address of 4 consecutive 16-bit elements,
// which a caller points at row j, columns 4q .. 4q + 3 of a 4 x 16 block;
// lane i then receives column i of rows 0 .. 3 (element i % 4 of the fetches
// of lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4).
typedef short tr_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) tr_v4i16 lds_v4i16;
__device__ __forceinline__ tr_v4i16 lds_read_tr16(const unsigned char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16 *)((__attribute__((address_space(3))) void *)(const_cast<unsigned char *>(p))));
}
// an 8-element 16-bit MFMA operand from two transpose reads: slots 0..3 from
// rows k0 .. k0 + 3 (address lo), slots 4..7 from the rows at address hi
template <typename Frag>
__device__ __forceinline__ Frag tr_frag(const unsigned char *lo, const unsigned char *hi) {
  const tr_v4i16 a = lds_read_tr16(lo), b = lds_read_tr16(hi);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(Frag, v);
}

// 16-byte load marked non-temporal (streamed data read once: the KV cache)
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }
// Four consecutive elements as fp32 (16 bytes of fp32, or 8 bytes of a 16-bit type).
template <typename T> __device__ __forceinline__ f32x4 ld4f(const T *p);
template <> __device__ __forceinline__ f32x4 ld4f<float>(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}
template <> __device__ __forceinline__ f32x4 ld4f<f16>(const f16 *p) {
  const f16x4 v = *reinterpret_cast<const f16x4 *>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <> __device__ __forceinline__ f32x4 ld4f<bf16>(const bf16 *p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void st8(void *p, u32x2 v) { *reinterpret_cast<u32x2 *>(p) = v; }

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

// XOR swizzle of 16-byte chunks inside an LDS row, for lanes that read the
// same logical chunk of consecutive rows.  With 128-byte rows the pattern
// f(r) = (r & 7) ^ ((r >> 3) & 1) keeps every 8 consecutive rows on distinct
// chunks (conflict-free for 32 banks, 8 lanes per phase) and every 16
// consecutive rows on distinct (row parity, chunk) pairs (conflict-free for
// 64 banks, 16 lanes per phase).  `row_chunks` is the number of 16-byte
// chunks per row (a power of two).
__host__ __device__ __forceinline__ int swz_key(int row, int row_chunks) {
  return row_chunks >= 8 ? ((row & 7) ^ ((row >> 3) & 1)) : (row & (row_chunks - 1));
}
__device__ __forceinline__ int swz(int row, int byte_in_row, int row_chunks) {
  const int phys = (byte_in_row >> 4) ^ swz_key(row, row_chunks);
  return (phys << 4) | (byte_in_row & 15);
}

// ---------------------------------------------------------------------------
// DPP lane exchanges inside rows of 16 lanes (no LDS traffic)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Value of the lane one below inside its row of 16 (0 for the row's lane 0).
__device__ __forceinline__ float dpp_shr1(float v) { return dpp_f<0x111>(v); }
// Value of the lane one above inside its row of 16 (0 for the row's lane 15).
__device__ __forceinline__ float dpp_shl1(float v) { return dpp_f<0x101>(v); }
// Sum over aligned groups of W lanes (W in 1, 2, 4, 8, 16), every lane gets it.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if constexpr (W >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// Bits 2 and 3 of a token index exchanged: the key order inside the
// transposed value tile, so that the 8 keys one lane feeds to the P*V MFMA
// (keys 4h..4h+3 and 8+4h..8+4h+3 of a 16-key chunk) are contiguous.
__host__ __device__ __forceinline__ int vt_perm(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

// Index of the calling wave inside its workgroup, as a wave-uniform (scalar)
// value: values derived from it stay in SGPRs, branches on them stay scalar,
// and an LDS-DMA destination built from it needs no per-lane loop for M0.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// An LDS address as the LDS-DMA builtins take it.  Inside kernel templates,
// arguments of those builtins whose types depend on template parameters (an
// LDS array of dependent size, an element of a dependent-size array) make the
// host pass reject the call without a diagnostic and drop the kernel's launch
// stub; pass the LDS pointer through as_lds and offsets as plain int.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void *as_lds(void *p) { return (lds_void *)p; }

// Wait until at most N vector-memory operations of this wave are in flight
// (vmcnt(N)); expcnt and lgkmcnt are left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  // vmcnt is split over bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8)
  // are set to their maxima
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS-DMA pipelines: waits for this wave's own LDS
// operations, then s_barrier, without the vmcnt(0) that __syncthreads adds
// (which would also wait for the tiles still in flight).  Callers wait for
// the DMA tiles they need with wait_vmcnt first.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Physical XCD-aware block remap: the hardware deals consecutive workgroup
// ids round-robin to the 8 XCDs; remapping so that each XCD receives a
// contiguous run of logical blocks keeps blocks that share operands in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int nx = 8;
  int per = nblocks / nx;               // full rounds
  int rem = nblocks - per * nx;
  int xcd = bid % nx, slot = bid / nx;
  // XCDs 0..rem-1 own per+1 logical blocks, the rest own per.
  int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + slot;
}

// cos and sin of the RoPE angle pos * theta (theta = base^(-2i/d), evaluated
// on the host in double precision); the angle is formed and reduced mod 2*pi
// in double precision, so large positions keep fp32-accurate rotations.
__device__ __forceinline__ float2 rope_cs_theta(int pos, double theta, float base) {
  if (base == 0.f) return make_float2(1.f, 0.f);
  const double phi = (double)pos * theta;
  const double TWO_PI_HI = 6.283185307179586;        // nearest double to 2*pi
  const double TWO_PI_LO = 2.4492935982947064e-16;   // 2*pi - TWO_PI_HI
  const double n = rint(phi * (1.0 / TWO_PI_HI));
  double r = fma(-n, TWO_PI_HI, phi);
  r = fma(-n, TWO_PI_LO, r);
  // |r| <= pi after the double-precision reduction: the hardware sin/cos
  // (v_sin_f32 / v_cos_f32) are accurate to a few ulp there
  const float rf = (float)r;
  return make_float2(__cosf(rf), __sinf(rf));
}

}  // namespace cca
