// Work decoding shared by the reduce kernels (internal): which sequence,
// head, chunk range and state columns a reduce workgroup handles, one pass
// per sequence or segmented (sequence-parallel).
#pragma once

#include "kernels.h"
#include "la_device.h"

namespace la {

// ---- copy-wave helpers of the reduce kernels
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Keeps the vector memory operations issued before it ahead of those issued
// after it: the copy waves' vmcnt waits count operations in issue order, so
// neither the compiler nor its scheduler may interleave the groups.
__device__ __forceinline__ void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
template <int OFF>
__device__ __forceinline__ void ds_write_b128_at(uint32_t a, const u32x4 &v) {
  static_assert(OFF >= 0 && OFF < 65536, "DS immediate offset");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(a), "v"(v), "n"(OFF) : "memory");
}
__device__ __forceinline__ void ds_write_b128(uint32_t a, const u32x4 &v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// two bf16 / fp16 input values in one word -> two fp16 (nearest even)
template <typename In>
__device__ __forceinline__ uint32_t to_f16x2(uint32_t w) {
  if constexpr (std::is_same<In, f16>::value) {
    return w;
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 r = {(_Float16)__uint_as_float(w << 16), (_Float16)__uint_as_float(w & 0xffff0000u)};
    return __builtin_bit_cast(uint32_t, r);
  }
}

// What one workgroup does: chunk slots [j0, j1) of sequence n, head h, state
// columns col0 .. col0 + W - 1; the state starts from init ([d_k][d_v] fp32,
// this (sequence or segment, head)), the identity (init_id) or zero, and ends
// in fin (fp32) and / or pimg (fp16 hi and lo images, see the segment passes
// below).  vzero: V reads as zero.
struct Work {
  int n, h, j0, j1, t0, eos, col0;
  bool vzero, init_id;
  const float *init;
  float *fin;
  _Float16 *pimg;
};

// Which work a workgroup has: 0 none, 1 with output, 2 without (the Delta and
// P roles of the segmented first pass).
//
// One workgroup per sequence (seg == 0): units (sequence, head) go out
// longest sequence first, so that when there are more workgroups than CUs
// the ones on the critical path start in the first round: unit u takes the
// sequence of rank u / H by decreasing chunk count (ties by index).  Up to
// 64 sequences every wave ranks them by itself, lane m holding sequence m,
// with no LDS and no barrier; empty sequences rank last, so their units
// leave at once.  Beyond 64 sequences the natural order is kept.
//
// Segmented (seg = L > 0, N_max <= 64): sequence n's chunks form
// ceil(chunks / L) segments of L chunks, numbered after those of sequences
// m < n.  The state entering segment s + 1 is an affine function of the one
// entering s, H_{s+1} = P_s H_s + D_s, with P_s the segment's transition
// (the state it leaves from the identity with V = 0) and D_s the state it
// leaves from zero.  Pass 1: segment 0 runs with output from the initial
// state and leaves its state in hin of segment 1 (or in ht); middle segments
// compute D_s (d_v slices) and P_s (d_k slices, fp16 hi / lo images).  The
// combine kernel then walks H_{s+1} = P_s H_s + D_s.  Pass 2: segments s >= 1
// run with output from hin, the last one leaving ht.
template <int DK, int W>
__device__ __forceinline__ int decode_work(const ReduceParams &p, Work &wk) {
  const int b = blockIdx.x;
  const int xcd = b & 7, kk = b >> 3;
  const int H = p.H;
  const int SS = p.pass == 1 ? p.S + p.SP : p.S;  // slices per unit
  const int slice = kk % SS, unit = (kk / SS) * 8 + xcd;
  const int m = lane_id();
  const size_t mat = (size_t)DK * DK;
  wk.vzero = false;
  wk.init_id = false;
  wk.init = nullptr;
  wk.fin = nullptr;
  wk.pimg = nullptr;
  wk.col0 = slice * W;
  if (p.seg == 0) {
    if (unit >= p.N_max * H) return 0;
    const int rank = unit / H;
    wk.h = unit % H;
    int n = rank;
    if (p.N_max <= 64) {
      int len = -1;
      if (m < p.N_max) len = p.chunk_offsets[m + 1] - p.chunk_offsets[m];
      if (rank >= __popcll(__ballot(len > 0))) return 0;
      int r = 0;
      for (int i = 0; i < p.N_max; ++i) {
        const int li = __builtin_amdgcn_readlane(len, i);
        r += (li > len) | ((li == len) & (i < m));
      }
      n = __builtin_ctzll(__ballot(r == rank));
    }
    wk.n = n;
    wk.j0 = p.chunk_offsets[n];
    wk.j1 = p.chunk_offsets[n + 1];
    if (wk.j0 == wk.j1) return 0;  // empty sequence (or invalid cu_seqlens): no writes
    wk.t0 = cu_at(p.cu_seqlens, p.cu64, n);
    wk.eos = cu_at(p.cu_seqlens, p.cu64, n + 1);
    const size_t sb = ((size_t)n * H + wk.h) * mat;
    if (p.h0) wk.init = p.h0 + sb;
    if (p.ht) wk.fin = p.ht + sb;
    return p.o ? 1 : 2;  // without o: states only
  }
  if (unit >= p.NS_max * H) return 0;
  const int sig = unit / H;
  wk.h = unit % H;
  // the segment slot's sequence: lane i holds sequence i's segment count
  int ns = 0;
  if (m < p.N_max) ns = (p.chunk_offsets[m + 1] - p.chunk_offsets[m] + p.seg - 1) / p.seg;
  int n = -1, s = 0, nseg = 0, acc = 0;
  for (int i = 0; i < p.N_max; ++i) {
    const int ni = __builtin_amdgcn_readlane(ns, i);
    if (sig < acc + ni) {
      n = i;
      s = sig - acc;
      nseg = ni;
      break;
    }
    acc += ni;
  }
  if (n < 0) return 0;
  wk.n = n;
  wk.j0 = p.chunk_offsets[n] + s * p.seg;
  wk.j1 = min(wk.j0 + p.seg, p.chunk_offsets[n + 1]);
  wk.t0 = cu_at(p.cu_seqlens, p.cu64, n) + s * p.seg * kBT;
  wk.eos = cu_at(p.cu_seqlens, p.cu64, n + 1);
  const size_t here = ((size_t)sig * H + wk.h) * mat, next = here + (size_t)H * mat;
  const size_t sb = ((size_t)n * H + wk.h) * mat;
  if (p.pass == 1) {
    if (s == 0) {
      if (slice >= p.S) return 0;
      if (p.h0) wk.init = p.h0 + sb;
      if (nseg > 1) wk.fin = p.hin + next;
      else if (p.ht) wk.fin = p.ht + sb;
      return 1;
    }
    if (s == nseg - 1) return 0;
    if (slice < p.S) {
      wk.fin = p.dlt + here;
    } else {
      wk.col0 = (slice - p.S) * W;
      wk.vzero = true;
      wk.init_id = true;
      wk.pimg = p.pimg + 2 * here;
    }
    return 2;
  }
  if (s == 0 || slice >= p.S) return 0;
  wk.init = p.hin + here;
  if (s == nseg - 1 && p.ht) wk.fin = p.ht + sb;
  return 1;
}

}  // namespace la
