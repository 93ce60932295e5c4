// Varlen causal short convolution forward on the shared chunk metadata.
//
// The layer path of the FLA graph-capture RFC runs a short convolution
// between the projections and the chunk attention, on the same fixed-capacity
// chunk_indices (sections "Proposed API" and "Step 3: GDN and
// short-convolution graph support"); the edge-NPU paper reports the reuse of
// that metadata ("Empowering Hybrid Attention Models on NPUs", section 7).
// Per channel c, with kernel width W and the sequence's inputs x_t:
//   y_t[c] = act(b[c] + sum_i w[c][i] x_{t-W+1+i}[c]) + r_t[c]
// where inputs before the sequence come from its initial state (the last W-1
// inputs before it; zero without one), act is the identity or SiLU, r the
// optional residual.  The final state is the W-1 inputs ending at the
// sequence's last token.
//
// It streams x in and y out (2 bytes per element each way for 16-bit data
// against 2W + 4 flops), so it is bound by HBM.  One workgroup per (chunk
// slot, 512 or 256 channels), slots along x: each wave takes 8 of the
// chunk's rows (BT / 8 waves), each lane 16 bytes of channels (8 for 16-bit
// data, 4 for fp32), so a wave moves whole 1 KiB row spans with 16-byte
// accesses.  A lane issues all its row loads before it computes, and keeps the
// W-1 previous inputs in registers; the residual is a compile-time option, so
// without one no registers wait for it.  Sentinel slots exit at once.
//
// States: only wave 0 of a sequence's first chunk reads h0[n] (the other
// waves and chunks start at least 8 rows in, past the W-1 <= 3 history rows),
// and the same wave writes ht[n] after it, lane by lane on disjoint channels,
// so ht may be h0 (in-place state update).
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

constexpr int kConvRows = 8;  // rows per wave

template <typename In>
__device__ __forceinline__ void unpack(const u32x4 &r, float *v) {
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

template <typename In>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (std::is_same<In, bf16>::value) {
    return f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
  } else {
    const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)a);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)b);
    return lo | (hi << 16);
  }
}

template <typename In>
__device__ __forceinline__ u32x4 pack(const float *v) {
  u32x4 r;
  if constexpr (sizeof(In) == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __float_as_uint(v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = pack2<In>(v[2 * e], v[2 * e + 1]);
  }
  return r;
}

template <typename In, int W, bool SILU, bool RES>
__global__ __launch_bounds__(512) void short_conv_kernel(ConvParams p) {
  constexpr int VEC = 16 / (int)sizeof(In);  // channels per lane
  constexpr int CPW = 64 * VEC;              // channels per workgroup
  const int slot = blockIdx.x;
  const int n = p.chunk_indices[2 * slot];
  if (n < 0) return;  // sentinel slot
  const int i_t = p.chunk_indices[2 * slot + 1];
  const int c0 = blockIdx.y * CPW + lane_id() * VEC;
  if (c0 >= p.D) return;
  const int bos = cu_at(p.cu_seqlens, p.cu64, n);
  const int eos = cu_at(p.cu_seqlens, p.cu64, n + 1);
  const int w = threadIdx.x >> 6;
  const int t0 = bos + i_t * p.BT + w * kConvRows;
  const int nr = min(kConvRows, eos - t0);  // rows of this wave (<= 0: none)
  const size_t D = (size_t)p.D;
  const u32x4 *xr = reinterpret_cast<const u32x4 *>(p.x);
  const u32x4 *rr = reinterpret_cast<const u32x4 *>(p.res);
  const u32x4 *h0 = reinterpret_cast<const u32x4 *>(p.h0);
  u32x4 *yr = reinterpret_cast<u32x4 *>(p.y);
  u32x4 *ht = reinterpret_cast<u32x4 *>(p.ht);
  auto at = [&](size_t row) { return (row * D + c0) / VEC; };  // 16-byte piece index
  const bool state_wave = i_t == 0 && w == 0;

  if (nr > 0) {
    // all of this lane's input rows first, then the W-1 rows before them
    u32x4 raw[kConvRows], res[RES ? kConvRows : 1];
#pragma unroll
    for (int r = 0; r < kConvRows; ++r)
      if (r < nr) raw[r] = xr[at(t0 + r)];
    if constexpr (RES) {
#pragma unroll
      for (int r = 0; r < kConvRows; ++r)
        if (r < nr) res[r] = rr[at(t0 + r)];
    }
    float hist[W > 1 ? W - 1 : 1][VEC];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
      const int pos = t0 - (W - 1) + i;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (pos >= bos) v = xr[at(pos)];
      else if (h0) v = h0[at((size_t)n * (W - 1) + (W - 1) + (pos - bos))];
      unpack<In>(v, hist[i]);
    }
    // the lane's VEC x W weights and VEC biases, 16-byte aligned runs
    float wt[VEC][W], bias[VEC];
    {
      float flat[VEC * W];
      const f32x4 *wp = reinterpret_cast<const f32x4 *>(p.w + (size_t)c0 * W);
#pragma unroll
      for (int q = 0; q < VEC * W / 4; ++q) {
        const f32x4 v = wp[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) flat[4 * q + e] = v[e];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int i = 0; i < W; ++i) wt[e][i] = flat[e * W + i];
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        const f32x4 v = p.b ? reinterpret_cast<const f32x4 *>(p.b + c0)[q] : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[4 * q + e] = v[e];
      }
    }
#pragma unroll
    for (int r = 0; r < kConvRows; ++r) {
      if (r < nr) {  // (a guard, not a break: the arrays stay in registers)
      float cur[VEC], out[VEC];
      unpack<In>(raw[r], cur);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float z = bias[e];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) z += wt[e][i] * hist[i][e];
        z += wt[e][W - 1] * cur[e];
        // SiLU: z sigmoid(z), the reciprocal to about 1 ulp
        if constexpr (SILU) z = z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
        out[e] = z;
      }
      if constexpr (RES) {
        float rv[VEC];
        unpack<In>(res[r], rv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) out[e] += rv[e];
      }
      yr[at(t0 + r)] = pack<In>(out);
#pragma unroll
      for (int i = 0; i + 1 < W - 1; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) hist[i][e] = hist[i + 1][e];
      if constexpr (W > 1) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) hist[W - 2][e] = cur[e];
      }
      }
    }
  }

  // final state of sequence n: the W-1 inputs ending at its last token,
  // reaching into h0 when the sequence is shorter (raw copies, no rounding)
  if (W > 1 && state_wave && ht) {
    u32x4 fin[W > 1 ? W - 1 : 1];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) {
      const int pos = eos - (W - 1) + i;
      fin[i] = u32x4{0u, 0u, 0u, 0u};
      if (pos >= bos) fin[i] = xr[at(pos)];
      else if (h0) fin[i] = h0[at((size_t)n * (W - 1) + (W - 1) + (pos - bos))];
    }
#pragma unroll
    for (int i = 0; i < W - 1; ++i) ht[at((size_t)n * (W - 1) + i)] = fin[i];
  }
}

template <typename In, int W>
hipError_t launch_conv_w(const ConvParams &p, int NT, bool silu, hipStream_t st) {
  constexpr int CPW = 64 * (16 / (int)sizeof(In));
  const dim3 grid(NT, (p.D + CPW - 1) / CPW), block(64 * p.BT / kConvRows);
  const bool res = p.res != nullptr;
  if (silu && res) hipLaunchKernelGGL((short_conv_kernel<In, W, true, true>), grid, block, 0, st, p);
  else if (silu) hipLaunchKernelGGL((short_conv_kernel<In, W, true, false>), grid, block, 0, st, p);
  else if (res) hipLaunchKernelGGL((short_conv_kernel<In, W, false, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((short_conv_kernel<In, W, false, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_conv_t(const ConvParams &p, int NT, int W, bool silu, hipStream_t st) {
  switch (W) {
    case 1: return launch_conv_w<In, 1>(p, NT, silu, st);
    case 2: return launch_conv_w<In, 2>(p, NT, silu, st);
    case 3: return launch_conv_w<In, 3>(p, NT, silu, st);
    case 4: return launch_conv_w<In, 4>(p, NT, silu, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_short_conv(const ConvParams &p, int dt, int NT, int W, bool silu,
                             hipStream_t st) {
  if (p.BT != 32 && p.BT != 64) return hipErrorInvalidValue;
  if (dt == LA_BF16) return launch_conv_t<bf16>(p, NT, W, silu, st);
  if (dt == LA_F16) return launch_conv_t<f16>(p, NT, W, silu, st);
  if (dt == LA_F32) return launch_conv_t<float>(p, NT, W, silu, st);
  return hipErrorInvalidValue;
}

}  // namespace la
