// Chunk-parallel map stage: one workgroup per (chunk slot, head).
//
// For the chunk's C <= 64 rows (GDN, scalar gate per row):
//   G_r  = sum_{s<=r} g_s                                  (gate / chunk cumsum)
//   A    = I + strict_lower(beta_r (K K^T)_rs exp(G_r - G_s))
//   M    = lower_incl((Q K^T)_rs exp(G_r - G_s))
//   T    = A^-1 diag(beta)
// and writes T with its diagonal removed (the diagonal is beta, which the
// reduce applies exactly in fp32) and M to the workspace, fp16 for bf16 inputs
// (fp32 for fp32 inputs).  These are the state-independent "forward intra"
// pieces of the GDN pipeline in the FLA graph-capture RFC ("[RFC] Add Graph
// Capture Support for FLA Prefill and Training Paths on Ascend NPUs", section
// "Step 3"), and the shared-input products K K^T, Q K^T grouped ahead of the
// inversion as "Empowering Hybrid Attention Models on NPUs" (section 5)
// suggests, with A^-1 kept apart from W = A^-1 K: the reduce applies T to
// (V - K H) instead of materialising W.
//
// Sentinel slots exit before any pointer arithmetic (RFC, section
// "Fixed-capacity execution").  Rows >= C of K, Q, beta and g read as zero, so
// the tail's rows and columns of T and M are zero.
//
// KDA (a gate vector per row): the decay sits inside the contraction,
// (K K^T)_rs -> sum_i k_ri k_si exp(G_ri - G_si).  Off-diagonal 16-row blocks
// (R > S) factor it through the first row b of block R,
// k_ri exp(G_ri - G_bi) * k_si exp(G_bi - G_si), both factors <= 1 when g <= 0;
// the four diagonal 16x16 blocks are summed elementwise in fp32.
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

// (R, S) 16x16 tile pairs of the lower block triangle of a 64x64 matrix
__constant__ int8_t kTileR[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kTileS[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <bool KDA, typename In, int DK>
__global__ __launch_bounds__(kThreads) void chunk_map_kernel(MapParams p) {
  using O = Op<In>;
  using T = typename O::T;
  constexpr int LDK = DK + O::PAD;   // K / Q row stride (elements)
  constexpr int LDL = kBT + 4;       // fp32 64x64 stride
  constexpr int KSTEP = 4 * O::KPL;  // k per MFMA

  __shared__ __attribute__((aligned(16))) T sK[kBT * LDK];
  __shared__ __attribute__((aligned(16))) T sQ[kBT * LDK];
  __shared__ float sL[kBT * LDL];     // strict lower part of A
  __shared__ float sX[kBT * LDL];     // A^-1
  __shared__ float sY[3 * 256];       // block products during the inverse
  __shared__ float sB[kBT];
  __shared__ float sg[kBT];
  // KDA: per-channel cumulative gate and the decayed operands of one block row
  __shared__ float sG[KDA ? kBT * DK : 1];
  __shared__ __attribute__((aligned(16))) T sKr[KDA ? 16 * LDK : 1];  // rows of block R (K)
  __shared__ __attribute__((aligned(16))) T sQr[KDA ? 16 * LDK : 1];  // rows of block R (Q)
  __shared__ __attribute__((aligned(16))) T sKs[KDA ? 48 * LDK : 1];  // rows 0..16R-1 (K)

  const int slot = blockIdx.x;
  const int h = blockIdx.y;
  const int i_n = p.chunk_indices[2 * slot];
  if (i_n < 0) return;  // sentinel: nothing to do, nothing written
  const int i_t = p.chunk_indices[2 * slot + 1];
  const int bos = p.cu_seqlens[i_n];
  const int eos = p.cu_seqlens[i_n + 1];
  const int r0 = bos + i_t * kBT;
  const int C = min(kBT, eos - r0);
  const int H = p.H;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();

  // ---- stage K, Q (rows >= C zero), beta, g
  {
    constexpr int VEC = 16 / sizeof(In);  // 16-byte global loads
    constexpr int PER_ROW = DK / VEC;
    const In *q = static_cast<const In *>(p.q);
    const In *k = static_cast<const In *>(p.k);
    for (int idx = tid; idx < kBT * PER_ROW; idx += kThreads) {
      const int r = idx / PER_ROW, c = (idx % PER_ROW) * VEC;
      T kv[VEC], qv[VEC];
      if (r < C) {
        const size_t off = ((size_t)(r0 + r) * H + h) * DK + c;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          kv[e] = (T)O::load(k + off + e);
          qv[e] = (T)O::load(q + off + e);
        }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) kv[e] = qv[e] = (T)0.f;
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        sK[r * LDK + c + e] = kv[e];
        sQ[r * LDK + c + e] = qv[e];
      }
    }
    if (tid < kBT) {
      const bool ok = tid < C;
      sB[tid] = ok ? p.beta[(size_t)(r0 + tid) * H + h] : 0.f;
      if (!KDA) sg[tid] = ok ? p.g[(size_t)(r0 + tid) * H + h] : 0.f;
    }
    if constexpr (KDA) {
      // per-channel inclusive cumsum down the rows (sequential per channel)
      for (int c = tid; c < DK; c += kThreads) {
        float run = 0.f;
        for (int r = 0; r < kBT; ++r) {
          if (r < C) run += p.g[((size_t)(r0 + r) * H + h) * DK + c];
          sG[r * DK + c] = run;
        }
      }
    }
  }
  __syncthreads();

  // ---- masked products A (strict lower, fp32 in LDS) and M (to workspace)
  T *Mws = static_cast<T *>(p.M_raw) + ((size_t)slot * H + h) * (kBT * kBT);
  T *Tws = static_cast<T *>(p.Tn_raw) + ((size_t)slot * H + h) * (kBT * kBT);

  if constexpr (!KDA) {
    const float G = wave_inclusive_scan(sg[lane]);  // lane r holds G_r
    // 10 lower tiles of K K^T then 10 of Q K^T: 5 per wave, wave w takes w + 4i
    f32x4 a5[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int t = w + 4 * i;
      const int pr = t % 10;
      const int R = kTileR[pr], S = kTileS[pr];
      const T *src = t < 10 ? sK : sQ;
      f32x4 c = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += KSTEP) {
        c = O::mfma(frag_lds<O>(src, LDK, 16 * R, k0, lane), frag_lds<O>(sK, LDK, 16 * S, k0, lane),
                    c);
      }
      a5[i] = c;
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int t = w + 4 * i;
      const int pr = t % 10;
      const int R = kTileR[pr], S = kTileS[pr];
      const int s = 16 * S + (lane & 15);
      const float Gs = __shfl(G, s, 64);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + (lane >> 4) * 4 + e;
        const float Gr = __shfl(G, r, 64);
        if (t < 10) {
          sL[r * LDL + s] = s < r ? sB[r] * a5[i][e] * __expf(Gr - Gs) : 0.f;
        } else {
          Mws[r * kBT + s] = (T)(s <= r ? a5[i][e] * __expf(Gr - Gs) : 0.f);
        }
      }
    }
  } else {
    // KDA off-diagonal blocks: for block row R, reference row b = 16R
    for (int R = 1; R < 4; ++R) {
      const int b = 16 * R;
      // r-side rows of block R and s-side rows 0..b-1, decayed through row b
      for (int idx = tid; idx < (16 + b) * DK; idx += kThreads) {
        const int r = idx / DK, c = idx % DK;
        const float Gb = sG[b * DK + c];
        if (r < 16) {
          const int rr = b + r;
          const float f = __expf(sG[rr * DK + c] - Gb);
          sKr[r * LDK + c] = (T)((float)sK[rr * LDK + c] * f);
          sQr[r * LDK + c] = (T)((float)sQ[rr * LDK + c] * f);
        } else {
          const int ss = r - 16;
          const float f = __expf(Gb - sG[ss * DK + c]);
          sKs[ss * LDK + c] = (T)((float)sK[ss * LDK + c] * f);
        }
      }
      __syncthreads();
      // tiles (R, S) for S < R: A part and M part -> 2R tiles over 4 waves
      for (int t = w; t < 2 * R; t += 4) {
        const int S = t % R;
        const bool isM = t >= R;
        const T *src = isM ? sQr : sKr;
        f32x4 c = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KSTEP)
          c = O::mfma(frag_lds<O>(src, LDK, 0, k0, lane), frag_lds<O>(sKs, LDK, 16 * S, k0, lane),
                      c);
        const int s = 16 * S + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = b + (lane >> 4) * 4 + e;
          if (isM) Mws[r * kBT + s] = (T)c[e];
          else sL[r * LDL + s] = sB[r] * c[e];
        }
      }
      __syncthreads();
    }
    // diagonal blocks, elementwise in fp32: 4 blocks x 16 x 16 (r, s) pairs
    for (int idx = tid; idx < 4 * 256; idx += kThreads) {
      const int blk = idx >> 8, r = 16 * blk + ((idx >> 4) & 15), s = 16 * blk + (idx & 15);
      float a = 0.f, m = 0.f;
      if (s <= r) {
        for (int c = 0; c < DK; ++c) {
          const float e = __expf(sG[r * DK + c] - sG[s * DK + c]);
          const float ks = (float)sK[s * LDK + c];
          a += (float)sK[r * LDK + c] * ks * e;
          m += (float)sQ[r * LDK + c] * ks * e;
        }
      }
      sL[r * LDL + s] = s < r ? sB[r] * a : 0.f;
      Mws[r * kBT + s] = (T)m;
    }
  }
  // upper block triangle of M is zero (the reduce reads whole k-steps)
  for (int idx = tid; idx < 6 * 256; idx += kThreads) {
    const int u = idx >> 8;  // (R, S) with S > R
    const int R = u < 3 ? 0 : (u < 5 ? 1 : 2);
    const int S = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
    Mws[(16 * R + ((idx >> 4) & 15)) * kBT + 16 * S + (idx & 15)] = (T)0.f;
  }
  __syncthreads();

  // ---- X = (I + L)^-1 by blocks: diagonal 16x16 blocks by forward
  // substitution (one lane per column), then block rows below the diagonal.
  if (w == 0) {
    const int blk = lane >> 4, c = lane & 15;
    const float *Lb = sL + (16 * blk) * LDL + 16 * blk;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc -= Lb[r * LDL + s] * x[s];
      x[r] = acc;
    }
    float *Xb = sX + (16 * blk) * LDL + 16 * blk;
#pragma unroll
    for (int r = 0; r < 16; ++r) Xb[r * LDL + c] = x[r];
  }
  __syncthreads();
  // X_ij = -X_ii * sum_{s in [16j, 16i)} L[16i + r][s] X[s][16j + c], by i - j
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    const int nblk = 4 - dist;  // pairs (j + dist, j), j = 0..nblk-1
    for (int idx = tid; idx < nblk * 256; idx += kThreads) {
      const int j = idx >> 8, i = j + dist, r = (idx >> 4) & 15, c = idx & 15;
      float acc = 0.f;
      for (int s = 16 * j; s < 16 * i; ++s) acc += sL[(16 * i + r) * LDL + s] * sX[s * LDL + 16 * j + c];
      sY[idx] = acc;
    }
    __syncthreads();
    for (int idx = tid; idx < nblk * 256; idx += kThreads) {
      const int j = idx >> 8, i = j + dist, r = (idx >> 4) & 15, c = idx & 15;
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) acc += sX[(16 * i + r) * LDL + 16 * i + s] * sY[j * 256 + s * 16 + c];
      sX[(16 * i + r) * LDL + 16 * j + c] = -acc;
    }
    __syncthreads();
  }
  // ---- T = X diag(beta), strict lower part only
  for (int idx = tid; idx < kBT * kBT; idx += kThreads) {
    const int r = idx >> 6, s = idx & 63;
    Tws[idx] = (T)(s < r ? sX[r * LDL + s] * sB[s] : 0.f);
  }
}

}  // namespace

template <bool KDA, typename In, int DK>
static hipError_t launch_map_t(const MapParams &p, hipStream_t st) {
  hipLaunchKernelGGL((chunk_map_kernel<KDA, In, DK>), dim3(p.NT_max, p.H), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_chunk_map(const MapParams &p, bool kda, bool bf16_in, int dk, hipStream_t st) {
  if (bf16_in) {
    if (dk == 128) return kda ? launch_map_t<true, bf16, 128>(p, st) : launch_map_t<false, bf16, 128>(p, st);
    return kda ? launch_map_t<true, bf16, 64>(p, st) : launch_map_t<false, bf16, 64>(p, st);
  }
  // fp32 inputs: d = 64 only (the fp32 d = 128 KDA tiles exceed the 160 KiB LDS)
  if (dk != 64) return hipErrorInvalidValue;
  return kda ? launch_map_t<true, float, 64>(p, st) : launch_map_t<false, float, 64>(p, st);
}

}  // namespace la
