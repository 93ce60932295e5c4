// Segment combine of the sequence-parallel reduce (see decode_work in
// chunk_reduce.hip): along each sequence's segments,
//   H_{s+1} = P_s H_s + D_s        s = 1 .. nseg - 2,
// starting from H_1, which the first pass left in hin of segment 1, and
// leaving every H_{s+1} in hin of segment s + 1 for the second pass.  P_s is
// the segment's transition ([d_k][d_k]), D_s the state it leaves from zero.
//
// One workgroup per (sequence, head, 32 state columns): two compute waves of
// 16 columns and one wave that copies P_{s+1} into the other half of a
// double buffer while P_s is used.  The product runs on fp16 MFMA with both
// factors split into high and low halves (x = hi + lo, hi = fp16(x),
// lo = fp16(x - hi)): hi*hi + hi*lo + lo*hi carries about 21 significant
// bits, against the 11 of a plain fp16 product, so the walk adds no error
// of its own beyond fp32 rounding.  The first pass stores P_s as the two fp16
// images (rows of 16-byte pieces, chained columns, swizzled) an A fragment
// read expects; the state is the B operand straight from its accumulators.
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

template <int DK>
__global__ __launch_bounds__(192) void chunk_combine_kernel(CombineParams p) {
  using O = Op<bf16>;
  constexpr int NW = 2, W = 16 * NW;         // compute waves, state columns
  constexpr int SB = DK / W;                 // workgroups per (sequence, head)
  constexpr int NHT = DK / 16, NKD = DK / 32;
  constexpr int PP = DK * 2 / 16;            // 16-byte pieces per fp16 row
  constexpr int IMGB = DK * DK * 2;          // bytes of one fp16 image
  constexpr int STAGE = 2 * IMGB;            // hi and lo images
  static_assert(STAGE % 1024 == 0, "1 KiB copy pieces");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int b = blockIdx.x;
  const int xcd = b & 7, kk = b >> 3;
  const int slice = kk % SB, unit = (kk / SB) * 8 + xcd;
  const int H = p.H;
  if (unit >= p.N_max * H) return;
  const int n = unit / H, h = unit % H;
  // segment counts of the sequences, lane i holding sequence i
  const int lane = lane_id(), w = wave_id();
  int ns = 0;
  if (lane < p.N_max) ns = (p.chunk_offsets[lane + 1] - p.chunk_offsets[lane] + p.seg - 1) / p.seg;
  const int nseg = __builtin_amdgcn_readlane(ns, n);
  if (nseg < 3) return;  // H_1 is all the second pass needs
  int sig0 = 0;          // first segment slot of sequence n
  for (int i = 0; i < n; ++i) sig0 += __builtin_amdgcn_readlane(ns, i);

  const size_t mat = (size_t)DK * DK;
  auto here = [&](int s) { return ((size_t)(sig0 + s) * H + h) * mat; };

  if (w == NW) {
    // copier: P_s into buffer (s - 1) & 1, one segment ahead
    auto copy = [&](int s) {
      const auto r = buffer_rsrc(p.pimg + 2 * here(s), STAGE);
      char *dst = smem + ((s - 1) & 1) * STAGE;
#pragma unroll
      for (int q = 0; q < STAGE / 1024; ++q) copy16_to_lds(r, dst + q * 1024, lane * 16, q * 1024);
    };
    copy(1);
    for (int s = 1; s <= nseg - 2; ++s) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();  // P_s has landed; the buffer of P_{s-1} is free
      if (s + 1 <= nseg - 2) copy(s + 1);
    }
    return;
  }

  const int lr = lane & 15, lg = lane >> 4;
  const int cw = slice * W + 16 * w;
  f32x4 hs[NHT];
#pragma unroll
  for (int t = 0; t < NHT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) hs[t][e] = p.hin[here(1) + (size_t)(16 * t + 4 * lg + e) * DK + cw + lr];
  const uint32_t base = lds_addr(smem);
  for (int s = 1; s <= nseg - 2; ++s) {
    f32x4 acc[NHT];
    const float *d = p.dlt + here(s);
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = d[(size_t)(16 * t + 4 * lg + e) * DK + cw + lr];
    // high and low halves of the state as B operands
    half8 bh[NKD], bl[NKD];
#pragma unroll
    for (int ks = 0; ks < NKD; ++ks) {
      bh[ks] = b_frag<O>(hs, ks);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bl[ks][e] = (_Float16)(hs[2 * ks][e] - (float)bh[ks][e]);
        bl[ks][4 + e] = (_Float16)(hs[2 * ks + 1][e] - (float)bh[ks][4 + e]);
      }
    }
    __syncthreads();  // P_s is in buffer (s - 1) & 1
    const char *tile = smem + ((s - 1) & 1) * STAGE;
    (void)base;
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int ks = 0; ks < NKD; ++ks) {
        const int off = tile_off<PP>(16 * t + lr, 4 * ks + lg);
        const half8 ah = *reinterpret_cast<const half8 *>(tile + off);
        const half8 al = *reinterpret_cast<const half8 *>(tile + IMGB + off);
        acc[t] = O::mfma(ah, bh[ks], acc[t]);
        acc[t] = O::mfma(ah, bl[ks], acc[t]);
        acc[t] = O::mfma(al, bh[ks], acc[t]);
      }
    float *dst = p.hin + here(s + 1);
#pragma unroll
    for (int t = 0; t < NHT; ++t) {
      hs[t] = acc[t];
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(size_t)(16 * t + 4 * lg + e) * DK + cw + lr] = acc[t][e];
    }
  }
}

}  // namespace

hipError_t launch_chunk_combine(const CombineParams &p, int dk, hipStream_t st) {
  const int units = p.N_max * p.H;
  if (dk == 128) {
    const int grid = ((units + 7) / 8) * 8 * (128 / 32);
    hipLaunchKernelGGL(chunk_combine_kernel<128>, dim3(grid), dim3(192), 0, st, p);
  } else if (dk == 64) {
    const int grid = ((units + 7) / 8) * 8 * (64 / 32);
    hipLaunchKernelGGL(chunk_combine_kernel<64>, dim3(grid), dim3(192), 0, st, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace la
