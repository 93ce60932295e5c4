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

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

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
