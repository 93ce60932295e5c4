// Device-side chunk metadata: cu_seqlens -> chunk_offsets, chunk_indices.
//
// FLA graph-capture RFC ("[RFC] Add Graph Capture Support for FLA Prefill and
// Training Paths on Ascend NPUs"), sections "Fixed-capacity execution" and
// "Device-side metadata": the chunk layout of the current cu_seqlens is built
// on the device into fixed-shape buffers, with no host round-trip, no
// data-dependent grid and the sentinel {-1, 0} in unused slots.  One
// workgroup: a validity check, a prefix sum of per-sequence chunk counts held
// in LDS, then one binary search per slot (up to 64 sequences: a single wave
// does the check and the scan with lane shuffles).  cu_seqlens may be int32 or int64;
// it is checked in its own width, so an int64 layout that passes the checks
// has every offset in [0, T_max] and the forward kernels read it as int.
#include "la_device.h"
#include "../../include/linattn.h"

namespace la {

constexpr int kMetaThreads = 1024;

template <typename Idx>
__global__ __launch_bounds__(kMetaThreads) void chunk_meta_kernel(
    const Idx *__restrict__ cu, int N_max, int T_max, int BT, int NT_max,
    int32_t *__restrict__ ci, int32_t *__restrict__ co, int32_t *__restrict__ status) {
  __shared__ int s_flags;
  __shared__ int s_part[kMetaThreads];
  __shared__ int s_off[LA_MAX_N + 1];
  const int tid = threadIdx.x;
  if (tid == 0) s_flags = 0;
  __syncthreads();

  int f = 0;
  for (int n = tid; n < N_max; n += kMetaThreads)
    if (cu[n + 1] < cu[n]) f |= LA_META_NOT_MONOTONE;
  if (tid == 0) {
    if (cu[0] != 0) f |= LA_META_BAD_START;
    if (cu[N_max] > (Idx)T_max) f |= LA_META_OVER_CAPACITY;
  }
  if (f) atomicOr(&s_flags, f);
  __syncthreads();

  // per-thread contiguous range of sequences; chunk counts are >= 0 once valid
  const int per = (N_max + kMetaThreads - 1) / kMetaThreads;
  const int n0 = tid * per;
  const int n1 = min(N_max, n0 + per);
  int local = 0;
  if (s_flags == 0)
    for (int n = n0; n < n1; ++n) local += ((int)(cu[n + 1] - cu[n]) + BT - 1) / BT;
  s_part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kMetaThreads; off <<= 1) {  // inclusive scan
    const int add = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += add;
    __syncthreads();
  }
  // the bound NT_max = ceil(T_max/BT) + N_max - 1 cannot be exceeded by a valid
  // cu_seqlens; treat an excess like an over-capacity input all the same
  if (tid == 0 && s_flags == 0 && s_part[kMetaThreads - 1] > NT_max)
    s_flags = LA_META_OVER_CAPACITY;
  __syncthreads();
  const int flags = s_flags;

  if (flags) {
    for (int j = tid; j < NT_max; j += kMetaThreads) {
      ci[2 * j] = -1;
      ci[2 * j + 1] = 0;
    }
    for (int n = tid; n <= N_max; n += kMetaThreads) co[n] = 0;
    if (status && tid == 0) *status = flags;
    return;
  }

  int run = s_part[tid] - local;
  for (int n = n0; n < n1; ++n) {
    s_off[n] = run;
    run += ((int)(cu[n + 1] - cu[n]) + BT - 1) / BT;
  }
  if (tid == 0) s_off[N_max] = s_part[kMetaThreads - 1];
  __syncthreads();
  for (int n = tid; n <= N_max; n += kMetaThreads) co[n] = s_off[n];
  const int total = s_off[N_max];
  for (int j = tid; j < NT_max; j += kMetaThreads) {
    int i_n = -1, i_t = 0;
    if (j < total) {
      // the sequence owning slot j: the last n with s_off[n] <= j
      int lo = 0, hi = N_max - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= j) lo = mid; else hi = mid - 1;
      }
      i_n = lo;
      i_t = j - s_off[lo];
    }
    ci[2 * j] = i_n;
    ci[2 * j + 1] = i_t;
  }
  if (status && tid == 0) *status = 0;
}

// N_max <= 64: one wave checks the offsets and scans the chunk counts with
// lane shuffles (lane n holding sequence n), one barrier, then the
// workgroup's four waves fill the slots
template <typename Idx>
__global__ __launch_bounds__(256) void chunk_meta_small_kernel(
    const Idx *__restrict__ cu, int N_max, int T_max, int BT, int NT_max,
    int32_t *__restrict__ ci, int32_t *__restrict__ co, int32_t *__restrict__ status) {
  __shared__ int s_off[65];
  __shared__ int s_flags;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int n = tid;
    const bool live = n < N_max;
    const Idx a = live ? cu[n] : Idx(0), b = live ? cu[n + 1] : Idx(0);
    int f = 0;
    if (__ballot(live && b < a)) f |= LA_META_NOT_MONOTONE;
    if (cu[0] != 0) f |= LA_META_BAD_START;
    if (cu[N_max] > (Idx)T_max) f |= LA_META_OVER_CAPACITY;
    int cnt = (live && !f) ? ((int)(b - a) + BT - 1) / BT : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(cnt, off, 64);
      if (n >= off) cnt += y;
    }
    const int total = __shfl(cnt, 63, 64);
    if (!f && total > NT_max) f = LA_META_OVER_CAPACITY;
    if (n == 0) {
      s_off[0] = 0;
      s_flags = f;
    }
    s_off[n + 1] = cnt;
  }
  __syncthreads();
  const int flags = s_flags;
  if (flags) {
    for (int j = tid; j < NT_max; j += 256) {
      ci[2 * j] = -1;
      ci[2 * j + 1] = 0;
    }
    for (int n = tid; n <= N_max; n += 256) co[n] = 0;
    if (status && tid == 0) *status = flags;
    return;
  }
  for (int n = tid; n <= N_max; n += 256) co[n] = s_off[n];
  const int total = s_off[N_max];
  for (int j = tid; j < NT_max; j += 256) {
    int i_n = -1, i_t = 0;
    if (j < total) {
      int lo = 0, hi = N_max - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= j) lo = mid; else hi = mid - 1;
      }
      i_n = lo;
      i_t = j - s_off[lo];
    }
    ci[2 * j] = i_n;
    ci[2 * j + 1] = i_t;
  }
  if (status && tid == 0) *status = 0;
}

hipError_t launch_chunk_meta(const void *cu, int cu64, int N_max, int T_max, int BT, int NT_max,
                             int32_t *ci, int32_t *co, int32_t *status, hipStream_t stream) {
  if (N_max <= 64) {
    if (cu64)
      hipLaunchKernelGGL(chunk_meta_small_kernel<int64_t>, dim3(1), dim3(256), 0, stream,
                         static_cast<const int64_t *>(cu), N_max, T_max, BT, NT_max, ci, co, status);
    else
      hipLaunchKernelGGL(chunk_meta_small_kernel<int32_t>, dim3(1), dim3(256), 0, stream,
                         static_cast<const int32_t *>(cu), N_max, T_max, BT, NT_max, ci, co, status);
    return hipGetLastError();
  }
  if (cu64)
    hipLaunchKernelGGL(chunk_meta_kernel<int64_t>, dim3(1), dim3(kMetaThreads), 0, stream,
                       static_cast<const int64_t *>(cu), N_max, T_max, BT, NT_max, ci, co, status);
  else
    hipLaunchKernelGGL(chunk_meta_kernel<int32_t>, dim3(1), dim3(kMetaThreads), 0, stream,
                       static_cast<const int32_t *>(cu), N_max, T_max, BT, NT_max, ci, co, status);
  return hipGetLastError();
}

}  // namespace la
