// One recurrent (decode) step: one new token per sequence, the state updated
// in place.  Per sequence n and head h, with alpha = exp(g) (GDN: one value;
// KDA: one per key channel) and the state H = S^T ([d_k][d_v] fp32):
//   H <- diag(alpha) H                       decay
//   p  = H^T k,  u = beta (v - p)             what the state predicts for k
//   H <- H + k u^T                            delta-rule write
//   o  = scale H^T q                          read-out with the new state
// the token-level recurrence itself (the step after prefill; the FLA graph
// RFC keeps this decode path out of its graph phase, section "Principles").
//
// It streams the state: 2 d_k d_v 4 bytes per (sequence, head) against
// about 6 d_k d_v flops, so it is bound by HBM.  One workgroup of 256
// threads per (sequence, head): thread t holds 4 consecutive columns of
// d_k / RG consecutive rows (RG row groups of d_v / 4 threads), so each wave
// reads and writes whole 512-byte row spans with 16-byte accesses.  The two
// column sums p and o are reduced across the row groups through LDS.  All
// arithmetic is fp32; q, k, v may be bf16 or fp16.
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

template <typename In>
__device__ __forceinline__ float ld(const In *p, size_t i) {
  return Op<In>::load(p + i);
}

template <bool KDA, typename In, int DK>
__global__ __launch_bounds__(256) void recurrent_kernel(RecurrentParams p) {
  constexpr int DV = DK;
  constexpr int QD = DV / 4;      // column quads
  constexpr int RG = 256 / QD;    // row groups
  constexpr int RPG = DK / RG;    // rows per group
  static_assert(QD * RG == 256 && RPG * RG == DK, "thread layout");
  __shared__ f32x4 sred[RG][QD];

  const int unit = blockIdx.x;  // n * H + h
  const int t = threadIdx.x;
  const int cq = t % QD, rg = t / QD;
  const int c0 = 4 * cq, r0 = rg * RPG;
  // grouped value heads share q and k: value head h reads q, k head h / (H / Hqk)
  const int n = unit / p.H, hqk = (unit % p.H) / (p.H / p.Hqk);
  const size_t uqk = (size_t)n * p.Hqk + hqk;
  const In *q = static_cast<const In *>(p.q) + uqk * DK;
  const In *k = static_cast<const In *>(p.k) + uqk * DK;
  const In *v = static_cast<const In *>(p.v) + (size_t)unit * DV;
  const size_t sb = (size_t)unit * DK * DV;

  float kr[RPG], qr[RPG], ar[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    kr[i] = ld(k, r0 + i);
    qr[i] = ld(q, r0 + i);
    ar[i] = __expf(KDA ? p.g[(size_t)unit * DK + r0 + i] : p.g[unit]);
  }
  f32x4 hs[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i)
    hs[i] = p.h0 ? *reinterpret_cast<const f32x4 *>(p.h0 + sb + (size_t)(r0 + i) * DV + c0) : zero4();
  // decay, then this group's share of p = H^T k
  f32x4 pp = zero4();
#pragma unroll
  for (int i = 0; i < RPG; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hs[i][e] *= ar[i];
      pp[e] += hs[i][e] * kr[i];
    }
  sred[rg][cq] = pp;
  __syncthreads();
  f32x4 pt = zero4();
#pragma unroll
  for (int g2 = 0; g2 < RG; ++g2)
#pragma unroll
    for (int e = 0; e < 4; ++e) pt[e] += sred[g2][cq][e];
  const float b = p.beta[unit];
  f32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = b * (ld(v, c0 + e) - pt[e]);
  // write, store the new state, and this group's share of o = H^T q
  f32x4 oo = zero4();
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hs[i][e] += kr[i] * u[e];
      oo[e] += hs[i][e] * qr[i];
    }
    if (p.ht) *reinterpret_cast<f32x4 *>(p.ht + sb + (size_t)(r0 + i) * DV + c0) = hs[i];
  }
  __syncthreads();  // every thread has read the p shares
  sred[rg][cq] = oo;
  __syncthreads();
  if (rg == 0) {
    f32x4 ot = zero4();
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2)
#pragma unroll
      for (int e = 0; e < 4; ++e) ot[e] += sred[g2][cq][e];
#pragma unroll
    for (int e = 0; e < 4; ++e) ot[e] *= p.scale;
    if (p.o_bf16) {
      uint2 b;
      b.x = f32_to_bf16_rne(ot[0]) | (f32_to_bf16_rne(ot[1]) << 16);
      b.y = f32_to_bf16_rne(ot[2]) | (f32_to_bf16_rne(ot[3]) << 16);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.o) + (size_t)unit * DV + c0) = b;
    } else {
      *reinterpret_cast<f32x4 *>(static_cast<float *>(p.o) + (size_t)unit * DV + c0) = ot;
    }
  }
}

template <bool KDA, typename In>
hipError_t launch_rec_t(const RecurrentParams &p, int dk, hipStream_t st) {
  const dim3 grid(p.units), block(256);
  if (dk == 128) hipLaunchKernelGGL((recurrent_kernel<KDA, In, 128>), grid, block, 0, st, p);
  else if (dk == 64) hipLaunchKernelGGL((recurrent_kernel<KDA, In, 64>), grid, block, 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent(const RecurrentParams &p, bool kda, int dt, int dk, hipStream_t st) {
  if (dt == LA_BF16) return kda ? launch_rec_t<true, bf16>(p, dk, st) : launch_rec_t<false, bf16>(p, dk, st);
  if (dt == LA_F16) return kda ? launch_rec_t<true, f16>(p, dk, st) : launch_rec_t<false, f16>(p, dk, st);
  if (dt != LA_F32) return hipErrorInvalidValue;
  return kda ? launch_rec_t<true, float>(p, dk, st) : launch_rec_t<false, float>(p, dk, st);
}

}  // namespace la
