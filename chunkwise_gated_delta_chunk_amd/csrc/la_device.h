// Internal device helpers for the gfx950 kernels (not part of the C ABI).
//
// MFMA conventions used throughout (16x16 output tiles, wave64):
//   A fragment: lane l holds A[m0 + l%16][k0 + (l/16)*KPL + i], i < KPL
//   B fragment: lane l holds B[k0 + (l/16)*KPL + i][n0 + l%16], i < KPL
//   C/D tile:   lane l holds C[m0 + (l/16)*4 + i][n0 + l%16],   i < 4
// Any permutation of k shared by A and B gives the same product, so the
// fragment loads only need both operands to use the same k order.  Both
// operands are therefore stored "k-contiguous": A as [m][k], B as [n][k].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kBT = 64;       // chunk length (tokens)
constexpr int kThreads = 256; // 4 waves per workgroup

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // raw 16-byte piece

struct bf16 { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Operand traits: bf16 inputs run on fp16 MFMA (bf16 values are exact in fp16
// inside its normal range), fp32 inputs on fp32 MFMA.
template <typename In> struct Op;
template <> struct Op<bf16> {
  using T = _Float16;
  using Frag = half8;
  static constexpr int KPL = 8;      // k elements per lane per MFMA
  static constexpr int PAD = 8;      // LDS row padding (16 bytes)
  __device__ static __forceinline__ f32x4 mfma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float load(const bf16 *p) { return bf16_to_f32(p->bits); }
};
template <> struct Op<float> {
  using T = float;
  using Frag = float;
  static constexpr int KPL = 1;
  static constexpr int PAD = 4;
  __device__ static __forceinline__ f32x4 mfma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float load(const float *p) { return *p; }
};

// Fragment of 16 rows starting at m0, KPL k-values starting at k0 + (lane/16)*KPL,
// from a k-contiguous LDS matrix with row stride `ld` (elements).
template <typename O>
__device__ __forceinline__ typename O::Frag frag_lds(const typename O::T *base, int ld, int m0,
                                                     int k0, int lane) {
  const typename O::T *p = base + (m0 + (lane & 15)) * ld + k0 + (lane >> 4) * O::KPL;
  return *reinterpret_cast<const typename O::Frag *>(p);
}

// Same from global memory (16-byte aligned rows for fp16; 4-byte for fp32).
template <typename O>
__device__ __forceinline__ typename O::Frag frag_glb(const typename O::T *__restrict__ base, int ld,
                                                     int m0, int k0, int lane) {
  const typename O::T *p = base + (size_t)(m0 + (lane & 15)) * ld + k0 + (lane >> 4) * O::KPL;
  return *reinterpret_cast<const typename O::Frag *>(p);
}

// "Chained" k order.  In k-step s, lane group g = lane/16, element i, the
// logical k index is
//   fp16 (KPL = 8): 32s + 4g + (i & 3) + 16 (i >> 2)
//   fp32 (KPL = 1): 16 (s / 4) + 4g + (s % 4)
// With this order the B fragment of a product that contracts over the rows
// of a column of 16x16 accumulator tiles (acc[t] = rows 16t..16t+15) is made
// of the accumulator registers themselves, so a result feeds the next product
// with no LDS round trip:
//   fp16: B = (acc[2s][0..3], acc[2s+1][0..3]);   fp32: B = acc[s/4][s%4].
// A operands are stored row-major with their k index at position kpos(k)
// (fp16: permuted inside each 32-element block; fp32: unpermuted), so an A
// fragment is one contiguous read.
template <typename O>
__device__ __host__ __forceinline__ constexpr int kpos(int k) {
  if constexpr (O::KPL == 1) {
    return k;
  } else {
    return (k & ~31) + 8 * ((k & 15) >> 2) + (k & 3) + 4 * ((k & 31) >> 4);
  }
}

// logical k stored at position p (inverse of kpos)
template <typename O>
__device__ __host__ __forceinline__ constexpr int kidx(int p) {
  if constexpr (O::KPL == 1) {
    return p;
  } else {
    const int i = p & 7, g = (p & 31) >> 3;
    return (p & ~31) + 4 * g + (i & 3) + 16 * (i >> 2);
  }
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Raw buffer resource over `bytes` bytes from `base` (gfx9 descriptor word 3).
// Buffer accesses at a lane offset >= bytes read zero / are dropped by the
// hardware range check, which covers the VGPR offset and the immediate offset
// only -- never put a data-dependent part of an offset in soffset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes < 0 ? 0 : bytes,
                                           0x00020000);
}

// A fragment of rows m0..m0+15, k-step s, from a row-major matrix whose k
// index is stored at kpos(k) (row stride ld elements)
template <typename O>
__device__ __forceinline__ typename O::Frag a_frag(const typename O::T *base, int ld, int m0,
                                                   int s, int lane) {
  const int lr = lane & 15, g = lane >> 4;
  if constexpr (O::KPL == 1) {
    return base[(m0 + lr) * ld + 16 * (s >> 2) + 4 * g + (s & 3)];
  } else {
    return *reinterpret_cast<const typename O::Frag *>(base + (m0 + lr) * ld + 32 * s + 8 * g);
  }
}

// B fragment of k-step s from a column of accumulator tiles (see kpos)
template <typename O>
__device__ __forceinline__ typename O::Frag b_frag(const f32x4 *acc, int s) {
  if constexpr (O::KPL == 1) {
    return acc[s >> 2][s & 3];
  } else {
    typename O::Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = (typename O::T)acc[2 * s][e];
      f[4 + e] = (typename O::T)acc[2 * s + 1][e];
    }
    return f;
  }
}

// Transposed A fragment (fp16 only): the operand M^T of a product that
// contracts over the rows of a row-major LDS matrix M whose columns are in
// chained order (kpos), for output rows m0..m0+15 of M^T (= columns of M) and
// k-step s over the rows of M.  Built from two ds_read_b64_tr_b16, which in
// each 16-lane group hand lane j element e of the 4-element row read by lane
// 4e + j/4, entry j%4: lane j therefore reads row 32s + 4g + j/4 (+16 for the
// upper half) at the four columns m0 + 4(j%4) .. +3, contiguous in kpos order.
__device__ __forceinline__ half8 a_frag_tr(const _Float16 *base, int ld, int m0, int s, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int j = lane & 15, g = lane >> 4;
  const int row = 32 * s + 4 * g + (j >> 2);
  const int pos = (m0 & ~31) + 8 * (j & 3) + 4 * ((m0 & 31) >> 4);
  const _Float16 *p0 = base + row * ld + pos;
  const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p0));
  const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p0 + 16 * ld));
  // whole-vector casts: a bit cast of a single vector element is lowered as
  // element 0 by this compiler
  return __builtin_shufflevector(__builtin_bit_cast(half4, lo), __builtin_bit_cast(half4, hi), 0,
                                 1, 2, 3, 4, 5, 6, 7);
}

// number of k-steps over K logical indices
template <typename O>
constexpr int ksteps(int K) { return K / (4 * O::KPL); }

// k-steps of a chunk-row contraction that reach row tile R of a lower
// triangular operand (all rows <= 16R + 15)
template <typename O>
__device__ __forceinline__ constexpr int ksteps_lower(int R) {
  if constexpr (O::KPL == 1) return 4 * (R + 1);
  else return R / 2 + 1;
}
// wave index as a scalar (uniform across the wave), so wave-dependent offsets
// and branches stay on the scalar unit
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Inclusive prefix sum over the 64 lanes of a wave (lane r holds x_r).  Both
// kernels that need the chunk-local cumulative gate call this same routine,
// so they see bit-identical values.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace la
