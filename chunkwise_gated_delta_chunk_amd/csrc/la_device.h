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

#include <type_traits>
#include <utility>

namespace la {

constexpr int kBT = 64;       // chunk length (tokens)
constexpr int kThreads = 256; // 4 waves per workgroup

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // raw 16-byte piece

struct bf16 { uint16_t bits; };
struct f16 { uint16_t bits; };  // fp16 input element

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ _Float16 f16_from_bits(uint32_t b) {
  return __builtin_bit_cast(_Float16, static_cast<uint16_t>(b));
}

// 16-bit input element (bf16 or fp16 bits) -> fp32
template <typename In> __device__ __forceinline__ float in16_to_f32(uint32_t b);
template <> __device__ __forceinline__ float in16_to_f32<bf16>(uint32_t b) {
  return bf16_to_f32(static_cast<uint16_t>(b));
}
template <> __device__ __forceinline__ float in16_to_f32<f16>(uint32_t b) {
  return static_cast<float>(f16_from_bits(b));
}

// cu_seqlens[i] of an int32 or int64 array (values checked to fit in int by
// the metadata kernel before any forward kernel uses them)
__device__ __forceinline__ int cu_at(const void *cu, int cu64, int i) {
  return cu64 ? static_cast<int>(static_cast<const int64_t *>(cu)[i])
              : static_cast<const int32_t *>(cu)[i];
}

// One 16-byte piece of input elements (8 bf16 / fp16 or 4 fp32) -> fp32.
template <typename In>
__device__ __forceinline__ void unpack16(const uint32_t (&r)[4], float *v) {
  if constexpr (sizeof(In) == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(r[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = in16_to_f32<In>(r[e] & 0xffffu);
      v[2 * e + 1] = in16_to_f32<In>(r[e] >> 16);
    }
  }
}

// Operand traits: bf16 and fp16 inputs run on fp16 MFMA (bf16 values are
// exact in fp16 inside its normal range), fp32 inputs on fp32 MFMA.
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
template <> struct Op<f16> : Op<bf16> {
  __device__ static __forceinline__ float load(const f16 *p) { return (float)f16_from_bits(p->bits); }
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

// ------------------------------------------------------------ tile images
// Operand tiles live in LDS as rows of 16-byte pieces with the piece index of
// each row XOR-swizzled, so that a tile can be copied into LDS verbatim (one
// lane per 16 bytes, as the direct global-to-LDS loads write it) and still be
// read without bank conflicts:
//   - 16 consecutive rows reading the same logical piece (an A fragment) hit
//     16 distinct pieces, i.e. all 64 banks once;
//   - 4 consecutive rows reading 4 consecutive pieces of a 32-element block
//     (the transposed reads of the state update, one per 16-lane group) hit
//     16 distinct pieces.
// P = pieces per row (16: 256-byte rows, 8: 128-byte rows; narrower rows
// need no swizzle for these patterns).
template <int P>
__device__ __host__ __forceinline__ constexpr int swz(int row) {
  if constexpr (P == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else if constexpr (P == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else return 0;
}
// byte offset of logical piece `piece` of row `row`
template <int P>
__device__ __host__ __forceinline__ constexpr int tile_off(int row, int piece) {
  return row * (16 * P) + ((piece ^ swz<P>(row)) << 4);
}

// The per-(chunk slot, head) image the map writes to the workspace and the
// reduce copies into LDS, element type e = 2 (fp16 operands) or 4 (fp32):
//   K   [64][d_k]  K (GDN) or K*exp(G) (KDA), key index in chained order
//   Q   [64][d_k]  likewise Q
//   KT  [d_k][64]  (KDA: (K*exp(G_C - G))^T; fp32 GDN: K^T), chunk rows chained;
//                  absent for fp16 GDN, whose reduce reads K^T from K
//   TN  [64][64]   T = A^-1 diag(beta) without its diagonal, columns chained
//   MM  [64][64]   masked decayed Q K^T, columns chained
//   VEC [192 + d_k] fp32: exp(G_r) | exp(G_C - G_r) | beta_r | state decay
//                  of each key row, padded to a multiple of 1 KiB
// every matrix swizzled as above; every region a multiple of 1 KiB.
struct ImageLayout {
  int K, Q, KT, TN, MM, VEC, BYTES, PK, PT;
};
__device__ __host__ constexpr ImageLayout image_layout(bool kda, int e, int dk) {
  const bool has_kt = kda || e == 4;
  ImageLayout L{};
  L.PK = dk * e / 16;
  L.PT = 64 * e / 16;
  L.K = 0;
  L.Q = L.K + 64 * dk * e;
  L.KT = L.Q + 64 * dk * e;
  L.TN = L.KT + (has_kt ? dk * 64 * e : 0);
  L.MM = L.TN + 64 * 64 * e;
  L.VEC = L.MM + 64 * 64 * e;
  L.BYTES = L.VEC + ((192 + dk) * 4 + 1023) / 1024 * 1024;
  return L;
}

// What of a cell's image the map stores in the workspace.  When the reduce
// stages K and Q itself from the raw q, k rows (raw: GDN with 16-bit inputs
// and 32-column slices) the stored image is the part from TN on (TN, MM,
// VEC); otherwise it is the whole image.  image_skip is the byte offset of
// the stored part inside the image layout, image_hbm_bytes its size per cell.
__device__ __host__ constexpr int image_skip(bool kda, int e, int dk, bool raw) {
  return raw ? image_layout(kda, e, dk).TN : 0;
}
__device__ __host__ constexpr int image_hbm_bytes(bool kda, int e, int dk, bool raw) {
  return image_layout(kda, e, dk).BYTES - image_skip(kda, e, dk, raw);
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;
// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x40u;
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// A generic pointer into LDS holds the LDS byte offset in its low 32 bits
// (the LDS aperture is 4 GiB aligned); taking it from there, rather than by an
// address-space cast, needs no null check.  Only for pointers into LDS.
__device__ __forceinline__ lds_ptr_t to_lds(void *p) {
  return (lds_ptr_t)(uintptr_t)(uint32_t)(uintptr_t)p;
}

// Direct global-to-LDS copy of 16 bytes per lane: lane l's bytes at buffer
// offset voff (+ soff, not range checked) land at lds + 16 l; lanes out of the
// resource's range write zeros.  `lds` must be the same for the whole wave.
// The builtin is emitted in the device pass only: in the host pass it would
// keep a kernel template from getting its launch stub.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, void *lds, int voff,
                                              int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, to_lds(lds), 16, voff, soff, 0, 0);
#endif
}

// s_waitcnt immediate waiting until at most n vector memory operations of
// this wave are outstanding (expcnt and lgkmcnt not waited for)
__device__ __host__ constexpr int vmcnt_imm(int n) {
  return (((n >> 4) & 3) << 14) | 0x0F70 | (n & 15);
}

// A fragment (rows m0..m0+15, k-step s) from a swizzled image tile with P
// pieces per row, k index in chained order
template <typename O, int P>
__device__ __forceinline__ typename O::Frag a_frag_img(const char *tile, int m0, int s, int lane) {
  const int lr = lane & 15, g = lane >> 4;
  const int row = m0 + lr;
  if constexpr (O::KPL == 1) {
    // fp32: k = 16 (s / 4) + 4 g + (s % 4): piece 4 (s / 4) + g, word s % 4
    return *reinterpret_cast<const float *>(tile + tile_off<P>(row, 4 * (s >> 2) + g) + 4 * (s & 3));
  } else {
    return *reinterpret_cast<const typename O::Frag *>(tile + tile_off<P>(row, 4 * s + g));
  }
}

// Transposed A fragment (fp16 only): the operand M^T of a product that
// contracts over the rows of an image tile M (P pieces per row) whose columns
// are in chained order (kpos), for output rows m0..m0+15 of M^T (= columns of
// M) and k-step s over the rows of M.  Built from two ds_read_b64_tr_b16,
// which in each 16-lane group hand lane j element e of the 4-element row read
// by lane 4e + j/4, entry j%4: lane j therefore reads row 32s + 4g + j/4 (+16
// for the upper half) at the four columns m0 + 4(j%4) .. +3, contiguous in
// kpos order.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 ds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
template <int P>
__device__ __forceinline__ half8 a_frag_tr(const char *tile, int m0, int s, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const int row = 32 * s + 4 * g + (j >> 2);
  const int piece = (m0 >> 5) * 4 + (j & 3);
  const int sub = 8 * ((m0 >> 4) & 1);
  const auto lo = ds_read_tr16(tile + tile_off<P>(row, piece) + sub);
  const auto hi = ds_read_tr16(tile + tile_off<P>(row + 16, piece) + sub);
  // whole-vector casts: a bit cast of a single vector element is lowered as
  // element 0 by this compiler
  return __builtin_shufflevector(__builtin_bit_cast(half4, lo), __builtin_bit_cast(half4, hi), 0,
                                 1, 2, 3, 4, 5, 6, 7);
}

// The same transposed read as opaque inline assembly, for use while direct
// global-to-LDS loads are in flight: the compiler cannot tell which LDS bytes
// the builtin reads and would otherwise wait for every outstanding vector
// memory operation first.  Its result is only valid after wait_lds_tied.
__device__ __forceinline__ void ds_read_tr16_async(s16x4 &r, const char *p) {
  const uint32_t a = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char *)p);
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
}
// wait until at most N LDS operations are outstanding (LDS operations
// complete in order), tying the four registers to the wait so no use of
// them is scheduled above it
template <int N>
__device__ __forceinline__ void wait_lds_tied(s16x4 &a, s16x4 &b, s16x4 &c, s16x4 &d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}
template <int N, typename F>
__device__ __forceinline__ void wait_lds_tied8(F &a, F &b, F &c, F &d, F &e, F &f, F &g, F &h) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h)
               : "n"(N));
}
// 16-byte LDS read as opaque inline assembly (valid after a tied wait)
__device__ __forceinline__ void ds_read_b128_async(half8 &r, const char *p) {
  const uint32_t a = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char *)p);
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
}
// the same two reads at LDS byte address `a` + OFF (OFF an immediate < 64 KiB)
template <int OFF>
__device__ __forceinline__ void ds_read_b128_at(half8 &r, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "DS immediate offset");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_read_b128_at(f32x4 &r, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "DS immediate offset");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_read_b32_at(float &r, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "DS immediate offset");
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(OFF));
}
// waits as wait_lds_tied, for other register counts and types
template <int N, typename F>
__device__ __forceinline__ void wait_lds_tied4(F &a, F &b, F &c, F &d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}
template <int N, typename F>
__device__ __forceinline__ void wait_lds_tied1(F &a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N, typename F>
__device__ __forceinline__ void wait_lds_tied2(F &a, F &b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int OFF>
__device__ __forceinline__ void ds_read_tr16_at(s16x4 &r, uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "DS immediate offset");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "n"(OFF));
}
// Workgroup barrier without the release fence of __syncthreads: a wave's
// pending global stores are not waited for.  The caller orders LDS itself:
// its own LDS reads must have been waited for, and direct-to-LDS loads that
// others read after the barrier must have completed (vmcnt) in the issuing
// wave.  The memory clobber keeps the compiler's memory accesses in place.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

// compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
__device__ __forceinline__ half8 join_half8(s16x4 lo, s16x4 hi) {
  return __builtin_shufflevector(__builtin_bit_cast(half4, lo), __builtin_bit_cast(half4, hi), 0, 1,
                                 2, 3, 4, 5, 6, 7);
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
