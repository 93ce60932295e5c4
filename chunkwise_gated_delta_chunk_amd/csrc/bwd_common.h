// Helpers shared by the chunk backward kernels (chunk_bwd.hip for GDN,
// chunk_bwd_kda.hip for KDA); internal, device only.
#pragma once

#include "la_device.h"
#include "kernels.h"

namespace la {
namespace bwd {

constexpr int kL = 68;  // row stride of the [64][64] LDS matrices (floats)

// bf16 MFMA helpers for the kernels of bf16 inputs
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_bf(bf16x8_t a, bf16x8_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fragment lane (g, j) <- X[row][k0 + 8g .. k0 + 8g + 7] (row picked by the caller)
__device__ __forceinline__ bf16x8_t frag_row(const __bf16 *X, int ld, int row, int k0) {
  return *reinterpret_cast<const bf16x8_t *>(X + row * ld + k0 + 8 * (lane_id() >> 4));
}

// fragment lane (g, j) <- X[k0 + 8g + e][n0 + j], e = 0..7: column n0 + j of
// the row-major X read down eight rows.  Each 16-lane group reads rows
// k0 + 8g .. +3 (then +4 .. +7) as sixteen 4-element pieces; the transposing
// read hands lane j element e of the piece read by lane 4e + j/4, entry j%4,
// so lane t addresses row k0 + 8g + t/4 at columns n0 + 4(t%4).
__device__ __forceinline__ bf16x8_t frag_col(const __bf16 *X, int ld, int k0, int n0) {
  const int l = lane_id(), g = l >> 4, t = l & 15;
  const __bf16 *a = X + (k0 + 8 * g + (t >> 2)) * ld + n0 + 4 * (t & 3);
  const s16x4 lo = ds_read_tr16(reinterpret_cast<const char *>(a));
  const s16x4 hi = ds_read_tr16(reinterpret_cast<const char *>(a + 4 * ld));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void splitb(float x, __bf16 &hi, __bf16 &lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// four consecutive values -> their bf16 hi / lo halves (8-byte stores)
__device__ __forceinline__ void split4(__bf16 *hi, __bf16 *lo, const f32x4 &v) {
  bf16x4_t a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = (__bf16)v[e];
    b[e] = (__bf16)(v[e] - (float)a[e]);
  }
  *reinterpret_cast<bf16x4_t *>(hi) = a;
  *reinterpret_cast<bf16x4_t *>(lo) = b;
}

// acc += A B over one 32-wide k-step, A and B both split
__device__ __forceinline__ f32x4 mfma3(bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl, f32x4 c) {
  c = mfma_bf(ah, bh, c);
  c = mfma_bf(ah, bl, c);
  return mfma_bf(al, bh, c);
}



// barrier after this wave's own LDS operations have completed; outstanding
// global loads and stores are not waited for
__device__ __forceinline__ void sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Products of 16x16 tiles on fp32 MFMA: A(m, k) at a[m * ams + k * aks],
// B(k, n) at b[k * bks + n * bns]; results in the MFMA layout (lane l: rows
// 4 (l / 16) + i, column l % 16).

// N tiles sharing one A: acc[j] += A B_j with B_j at b + j * bt.  The N
// accumulations are independent, so their MFMAs interleave, and each A value
// is read once for all N.
// K is a compile-time length: the loop unrolls fully, so the LDS reads of
// all k-steps can be issued ahead of the MFMAs that use them.
template <int N, int K>
__device__ __forceinline__ void mmN(f32x4 (&acc)[N], const float *a, int ams, int aks,
                                    const float *b, int bks, int bns, int bt) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const float *pa = a + r * ams + g * aks;
  const float *pb = b + g * bks + r * bns;
#pragma unroll
  for (int k = 0; k < K; k += 4) {
    const float av = pa[k * aks];
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = mfma4(av, pb[j * bt + k * bks], acc[j]);
  }
}

// one tile with the k range split over two accumulators (two interleaved
// chains), summed at the end
template <int K>
__device__ __forceinline__ f32x4 mm2k(const float *a, int ams, int aks, const float *b, int bks,
                                      int bns) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const float *pa = a + r * ams + g * aks;
  const float *pb = b + g * bks + r * bns;
  f32x4 c0 = zero4(), c1 = zero4();
#pragma unroll
  for (int k = 0; k < K; k += 8) {
    c0 = mfma4(pa[k * aks], pb[k * bks], c0);
    c1 = mfma4(pa[(k + 4) * aks], pb[(k + 4) * bks], c1);
  }
  return c0 + c1;
}

// the chunk of slot jj: first row, valid rows; false for a sentinel slot
struct Chunk { int n, r0, C; };
__device__ __forceinline__ bool chunk_of(const BwdParams &p, int slot, Chunk &c) {
  const int n = p.chunk_indices[2 * slot];
  if (n < 0) return false;
  const int i_t = p.chunk_indices[2 * slot + 1];
  const int bos = cu_at(p.cu_seqlens, p.cu64, n);
  const int eos = cu_at(p.cu_seqlens, p.cu64, n + 1);
  c.n = n;
  c.r0 = bos + i_t * kBT;
  c.C = min(kBT, eos - c.r0);
  return true;
}

// The loaders move 16-byte pieces, all of a thread's loads issued before its
// LDS stores, so a chunk's operands arrive in about one memory round trip.

// rows r < C of a [T][H][D] input, head h, columns c0 .. c0 + W, into LDS
// rows of stride ld (fp32, 16-byte aligned rows); rows >= C are zero
template <typename In, int D, int W = D, int R = kBT>
__device__ __forceinline__ void load_rows(float *dst, int ld, const void *src, int r0, int C, int H,
                                          int h, int c0 = 0) {
  constexpr int VEC = 16 / (int)sizeof(In);
  constexpr int PR = W / VEC;                 // pieces per row
  constexpr int NP = R * PR;                  // pieces
  constexpr int IT = (NP + 255) / 256;
  uint32_t raw[IT][4];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pc = threadIdx.x + 256 * it, r = pc / PR, c = (pc % PR) * VEC;
    const u32x4 v = (pc < NP && r < C)
        ? *reinterpret_cast<const u32x4 *>(static_cast<const char *>(src) +
                                           (((size_t)(r0 + r) * H + h) * D + c0 + c) * sizeof(In))
        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[it][e] = v[e];
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pc = threadIdx.x + 256 * it, r = pc / PR, c = (pc % PR) * VEC;
    if (pc < NP) {
      float f[VEC];
      unpack16<In>(raw[it], f);
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q)
        *reinterpret_cast<f32x4 *>(dst + r * ld + c + 4 * q) =
            f32x4{f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]};
    }
  }
}

// an [R][W] fp32 block at src (row stride sld floats) into LDS (stride ld)
template <int R, int W>
__device__ __forceinline__ void load_block(float *dst, int ld, const float *src, size_t sld) {
  constexpr int PR = W / 4, NP = R * PR, IT = (NP + 255) / 256;
  f32x4 v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pc = threadIdx.x + 256 * it;
    v[it] = pc < NP ? *reinterpret_cast<const f32x4 *>(src + (pc / PR) * sld + (pc % PR) * 4)
                    : zero4();
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pc = threadIdx.x + 256 * it;
    if (pc < NP) *reinterpret_cast<f32x4 *>(dst + (pc / PR) * ld + (pc % PR) * 4) = v[it];
  }
}

__device__ __forceinline__ void load_mat64(float *dst, const float *src) {
  load_block<64, 64>(dst, kL, src, 64);
}

// The sequence of rank `rank` by decreasing chunk count (ties by index), so
// that the reverse passes start the longest sequences first when their
// workgroups outnumber the CUs; -1 past the non-empty ones.  Up to 64
// sequences each wave ranks them itself (lane m holding sequence m); beyond
// that the natural order is kept.
__device__ __forceinline__ int seq_by_rank(const int32_t *co, int N_max, int rank) {
  if (N_max > 64) return rank;
  const int m = lane_id();
  int len = -1;
  if (m < N_max) len = co[m + 1] - co[m];
  if (rank >= __popcll(__ballot(len > 0))) return -1;
  int r = 0;
  for (int i = 0; i < N_max; ++i) {
    const int li = __builtin_amdgcn_readlane(len, i);
    r += (li > len) | ((li == len) & (i < m));
  }
  return __builtin_ctzll(__ballot(r == rank));
}

// X = (I + diag(beta) S)^-1 for the strict-lower S ([64][64], stride kL),
// rows and columns >= C zero, into sX (stride kL); the whole workgroup
// (4 waves) calls it between barriers.  The four 16x16 diagonal blocks by
// forward substitution (wave 0, one lane per column), then the blocks below
// the diagonal as X_ij = -X_ii sum_{k=j}^{i-1} L_ik X_kj on fp32 MFMA, one
// block per wave and diagonal distance; the sum waits in the upper block
// (j, i) of sX, which X never uses.  With `zeroed` the caller has already
// cleared sX (zero_mat64) before a barrier.
// sX = 0, four consecutive entries per thread and step (256 threads)
__device__ __forceinline__ void zero_mat64(float *sX) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = 4 * threadIdx.x + 1024 * it;
    *reinterpret_cast<f32x4 *>(sX + (idx >> 6) * kL + (idx & 63)) = zero4();
  }
}
__device__ __forceinline__ void unit_lower_inverse(const float *sS, const float *sB, float *sX,
                                                   int C, bool zeroed = false) {
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  if (!zeroed) {
    zero_mat64(sX);
    __syncthreads();
  }
  if (w == 0) {
    const int blk = l >> 4, c = l & 15;
    float xd[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = 16 * blk + r;
      float acc = r == c ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc -= sB[rr] * sS[rr * kL + 16 * blk + s] * xd[s];
      xd[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sX[(16 * blk + r) * kL + 16 * blk + c] = xd[r];
  }
  __syncthreads();
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    const int j = w, i = w + dist;
    if (i < 4) {
      f32x4 y = zero4();
      for (int kb = j; kb < i; ++kb)
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int row = 16 * i + lr;
          const float a = sB[row] * sS[row * kL + 16 * kb + k0 + lg];
          const float b = sX[(16 * kb + k0 + lg) * kL + 16 * j + lr];
          y = mfma4(a, b, y);
        }
      float *Y = sX + (16 * j) * kL + 16 * i;  // upper block (j, i)
#pragma unroll
      for (int e = 0; e < 4; ++e) Y[(lg * 4 + e) * kL + lr] = y[e];
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      f32x4 x = zero4();
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4)
        x = mfma4(sX[(16 * i + lr) * kL + 16 * i + k0 + lg], Y[(k0 + lg) * kL + lr], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(16 * i + lg * 4 + e) * kL + 16 * j + lr] = -x[e];
    }
    __syncthreads();
  }
  // clear the scratch blocks and the rows / columns past the chunk, four
  // consecutive entries per thread and step
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = 4 * tid + 1024 * it, r = idx >> 6, c = idx & 63;
    f32x4 *px = reinterpret_cast<f32x4 *>(sX + r * kL + c);
    f32x4 v = *px;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e > r || r >= C || c + e >= C) v[e] = 0.f;
    *px = v;
  }
  __syncthreads();
}

}  // namespace bwd
}  // namespace la
