// Chunk-parallel map stage: one workgroup per (chunk slot, head).
//
// For the chunk's C <= 64 rows (GDN, scalar gate per row):
//   G_r  = sum_{s<=r} g_s                                  (gate / chunk cumsum)
//   A    = I + strict_lower(beta_r (K K^T)_rs exp(G_r - G_s))
//   M    = lower_incl((Q K^T)_rs exp(G_r - G_s))
//   T    = A^-1 diag(beta)
// These are the state-independent "forward intra" pieces of the GDN pipeline
// in the FLA graph-capture RFC ("[RFC] Add Graph Capture Support for FLA
// Prefill and Training Paths on Ascend NPUs", section "Step 3"), with the
// shared-input products K K^T, Q K^T grouped ahead of the inversion as
// "Empowering Hybrid Attention Models on NPUs" (section 5) suggests, and
// A^-1 kept apart from W = A^-1 K: the reduce applies T to (V - K H) instead
// of materialising W.
//
// Written to the workspace for the reduce, per (slot, head), as one image
// (image_layout in la_device.h: swizzled 16-byte pieces, ready to be copied
// into LDS verbatim):
//   K, Q  in the operand element type, key index in chained order (not for
//         GDN with RAW set, 16-bit inputs reduced in 32-column slices: that
//         reduce stages them itself from the raw rows, and the stored image
//         starts at Tn)
//   Tn  = T with its diagonal (beta) removed -- the reduce applies beta in fp32
//   M
//   vec = [exp(G_r) | exp(G_C - G_r) | beta_r | per-key-row state decay]
// The element type is fp16 for bf16 inputs (bf16 values are exact in fp16
// inside its normal range) and fp32 for fp32 inputs; matrices have their
// columns in the reduce's chained k order (kpos), ready to be MFMA A
// operands.  fp32 GDN also writes K^T (chunk rows chained); fp16 GDN does not
// need it, its reduce reads K^T from K with transposing LDS reads.
//
// A^-1 is formed by 16x16 blocks: the four diagonal blocks by forward
// substitution (one lane per column), then block row i of column block j as
// X_ij = -X_ii sum_{k=j}^{i-1} L_ik X_kj on fp32 MFMA, one block per wave.
//
// Sentinel slots exit before any pointer arithmetic (RFC, section
// "Fixed-capacity execution").  Rows >= C of K, Q, beta and g read as zero, so
// the tail's rows and columns of T and M are zero.
//
// KDA (a gate vector per row): the decay sits inside the contraction,
// (K K^T)_rs -> sum_i k_ri k_si exp(G_ri - G_si).  Off-diagonal 16-row blocks
// (R > S) factor it through the first row b of block R,
// k_ri exp(G_ri - G_bi) * k_si exp(G_bi - G_si), both factors <= 1 when g <= 0,
// formed in registers as MFMA operands.  The four diagonal 16x16 blocks factor
// through their own first row in fp32 (one factor grows, so a block whose
// decay exceeds e^60 in some channel is summed elementwise).  The KDA map
// writes the decayed operands in place of K and Q, K*exp(G) and Q*exp(G), and
// (K*exp(G_C - G))^T (chunk rows in chained order), and exp(G_C) as the state
// decay, so the reduce does no gate work.
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

// ---- the chunk layout built in the map's own prologue (up to 64 sequences)
// The FLA graph-capture RFC ("[RFC] Add Graph Capture Support for FLA Prefill
// and Training Paths on Ascend NPUs", "Device-side metadata") builds
// chunk_offsets and chunk_indices on the device from cu_seqlens.  When the
// caller asks the forward for that layout, every wave of the map derives it
// by itself, with the checks and results of build_chunk_meta at BT = 64, so
// the step needs no launch of its own for it: lane m holds the chunk slots of
// sequences 0..m (lanes >= N_max: all of them), and a layout that fails a
// check has no slots.
struct WaveLayout {
  int end;    // per lane, see above
  int total;  // slots in use: 0 for an invalid layout
  int flags;  // build_chunk_meta's status bits
};
template <typename Idx>
__device__ __forceinline__ WaveLayout wave_layout_t(const Idx *cu, int N_max, int T_max, int NT_max) {
  const int m = lane_id();
  const bool live = m < N_max;
  const Idx a = live ? cu[m] : Idx(0), b = live ? cu[m + 1] : Idx(0);
  int f = 0;
  if (__ballot(live && b < a)) f |= LA_META_NOT_MONOTONE;
  if (cu[0] != 0) f |= LA_META_BAD_START;
  if (cu[N_max] > (Idx)T_max) f |= LA_META_OVER_CAPACITY;
  int cnt = (live && !f) ? ((int)(b - a) + kBT - 1) / kBT : 0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(cnt, off, 64);
    if (m >= off) cnt += y;
  }
  const int total = __shfl(cnt, 63, 64);
  if (!f && total > NT_max) f = LA_META_OVER_CAPACITY;
  WaveLayout L;
  L.flags = f;
  L.total = f ? 0 : total;
  L.end = f ? 0 : cnt;
  return L;
}
__device__ __forceinline__ WaveLayout wave_layout(const MapParams &p) {
  return p.cu64 ? wave_layout_t(static_cast<const int64_t *>(p.cu_seqlens), p.N_max, p.T_max, p.NT_max)
                : wave_layout_t(static_cast<const int32_t *>(p.cu_seqlens), p.N_max, p.T_max, p.NT_max);
}
// slot j (the same in every lane) -> sequence and chunk (i_n = -1: sentinel),
// from this lane's `end` (lane 63's is the slot total)
__device__ __forceinline__ void layout_slot(int end, int j, int &i_n, int &i_t) {
  i_n = -1;
  i_t = 0;
  if (j >= __builtin_amdgcn_readlane(end, 63)) return;
  const int n = __popcll(__ballot(end <= j));
  i_n = n;
  i_t = j - (n > 0 ? __builtin_amdgcn_readlane(end, n - 1) : 0);
}
// Slots j = first + stride * t (t = 0, 1, ...: lane t of this wave's passes)
// -> chunk_indices, and with `head` also chunk_offsets and the status word.
// Every slot below NT_max is written by exactly one (wave, lane) of the grid.
// The whole wave runs every shuffle (the loop bounds are wave-uniform).
__device__ __forceinline__ void layout_store(const MapParams &p, const WaveLayout &L, int first,
                                             int stride, bool head) {
  const int m = lane_id();
  for (int base = first; base < p.NT_max; base += 64 * stride) {
    const int j = base + m * stride;
    // the owning sequence: how many sequences end at or before slot j
    int n = 0;
    for (int i = 0; i < p.N_max; ++i) n += __builtin_amdgcn_readlane(L.end, i) <= j;
    const int start = __shfl(L.end, (n - 1) & 63, 64);
    const bool in = j < L.total;
    if (j < p.NT_max) {
      p.meta_ci[2 * j] = in ? n : -1;
      p.meta_ci[2 * j + 1] = in ? j - (n > 0 ? start : 0) : 0;
    }
  }
  if (head) {
    // chunk_offsets[n] = slots of the sequences before n (all 0 when invalid)
    const int prev = __shfl_up(L.end, 1, 64);
    if (m <= p.N_max) p.meta_co[m] = m == 0 ? 0 : prev;
    if (m == 0 && p.N_max == 64) p.meta_co[64] = L.total;
    if (p.meta_status && m == 0) *p.meta_status = L.flags;
  }
}

// (R, S) of the p-th 16x16 tile of the lower block triangle of a 64x64 matrix,
// p = 0..9 in row order: R = 0,1,1,2,2,2,3,3,3,3 and S = 0,0,1,0,1,2,0,1,2,3,
// packed two bits per entry
__device__ __forceinline__ int tile_r(int p) { return (0xFFA94 >> (2 * p)) & 3; }
__device__ __forceinline__ int tile_s(int p) { return (0xE4910 >> (2 * p)) & 3; }

using F32 = Op<float>;

template <bool KDA, typename In, int DK, bool RAW>
__global__ __launch_bounds__(kThreads) void chunk_map_kernel(MapParams p) {
  using O = Op<In>;
  using T = typename O::T;
  constexpr int LDK = DK + O::PAD;   // K / Q row stride (elements)
  constexpr int LDL = kBT + 4;       // fp32 64x64 stride
  constexpr int KSTEP = 4 * O::KPL;  // k per MFMA
  constexpr int KQ_BYTES = 2 * kBT * LDK * (int)sizeof(T);
  constexpr int LX_BYTES = 2 * kBT * LDL * (int)sizeof(float);
  // K and Q are dead once the products are formed, and A / A^-1 take their
  // bytes (KDA: every wave holds its tiles of A and M in registers until all
  // waves are done reading K and Q)
  constexpr int AREA = KQ_BYTES > LX_BYTES ? KQ_BYTES : LX_BYTES;
  __shared__ __attribute__((aligned(16))) char sArea[AREA];
  __shared__ __attribute__((aligned(16))) float sY[4][16 * 17];  // per-wave 16x16 scratch
  __shared__ __attribute__((aligned(16))) float sB[kBT];
  __shared__ __attribute__((aligned(16))) float sg[kBT];
  // KDA: per-channel cumulative gate (rows padded so that 16 rows at one
  // channel hit distinct banks)
  constexpr int GS = DK + 4;
  __shared__ float sG[KDA ? kBT * GS : 1];
  constexpr int LDM = kBT + O::PAD;  // M, natural column order, before the write-out
  T *sK = reinterpret_cast<T *>(sArea);
  T *sQ = sK + kBT * LDK;
  float *sL = reinterpret_cast<float *>(sArea);
  float *sX = sL + kBT * LDL;
  // M waits for its write-out in the bytes of X, which the inverse fills
  // only after it
  T *sMt = reinterpret_cast<T *>(sX);
  static_assert(kBT * LDM * sizeof(T) <= kBT * LDL * sizeof(float), "M inside X");

  // heads vary fastest: the workgroups of one slot run together and share
  // the L2 lines of its token rows (q, k rows of adjacent heads, g, beta)
  const int h = blockIdx.x % p.H;
  const int slot = blockIdx.x / p.H;
  int i_n, i_t;
  if (p.fuse_meta) {
    // the layout from cu_seqlens; the head-0 workgroup of each slot stores it
    const WaveLayout L = wave_layout(p);
    if (h == 0 && wave_id() == 0) layout_store(p, L, slot, p.NT_max, slot == 0);
    layout_slot(L.end, slot, i_n, i_t);
  } else {
    i_n = p.chunk_indices[2 * slot];
    i_t = i_n < 0 ? 0 : p.chunk_indices[2 * slot + 1];
  }
  if (i_n < 0) return;  // sentinel: nothing to do, nothing written
  const int bos = cu_at(p.cu_seqlens, p.cu64, i_n);
  const int eos = cu_at(p.cu_seqlens, p.cu64, i_n + 1);
  const int r0 = bos + i_t * kBT;
  const int C = min(kBT, eos - r0);
  const int H = p.H;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int E = (int)sizeof(T);
  constexpr ImageLayout I = image_layout(KDA, E, DK);
  constexpr int PK = DK * E / 16, PT = kBT * E / 16;  // 16-byte pieces per row
  constexpr int CH = 16 / E;                          // elements per piece
  const size_t unit = (size_t)slot * H + h;
  // the stored part of the image starts at I.TN for 16-bit GDN (the reduce
  // stages K and Q from the raw rows): region offsets are relative to img
  constexpr int SKIP = image_skip(KDA, E, DK, RAW);
  char *img = static_cast<char *>(p.img) + unit * (size_t)image_hbm_bytes(KDA, E, DK, RAW) - SKIP;
  float *vec = reinterpret_cast<float *>(img + I.VEC);
  // 16 bytes of v[0..CH) -> piece `piece` of row `row` of an image tile
  auto put = [&](int region, int P, int row, int piece, const T *v) {
    const int off = P == 16 ? tile_off<16>(row, piece) : P == 8 ? tile_off<8>(row, piece)
                                                                 : row * 16 * P + 16 * piece;
    *reinterpret_cast<u32x4 *>(img + region + off) = *reinterpret_cast<const u32x4 *>(v);
  };

  // ---- stage K, Q (rows >= C zero), beta, g.  All global loads are issued
  // first (masked, raw bytes) and converted afterwards, so they overlap.
  // bf16: a unit is row r, 32-element block b, half g2: input pieces
  // 4b + g2 and 4b + 2 + g2 (8 elements each), which hold exactly the chained
  // pieces 4b + 2 g2 (their low halves) and 4b + 2 g2 + 1 (their high halves).
  // fp32: a unit is one 4-element piece (the chained order is the natural one).
  {
    constexpr int VEC = 16 / sizeof(In);              // elements per 16-byte load
    constexpr int UPR = VEC == 8 ? DK / 16 : DK / 4;  // units per row
    constexpr int NU = kBT * UPR / kThreads;
    constexpr int NP = VEC == 8 ? 2 : 1;              // input pieces per unit
    static_assert(kBT * UPR % kThreads == 0, "staging split");
    const In *q = static_cast<const In *>(p.q);
    const In *k = static_cast<const In *>(p.k);
    const int hqk = h / (H / p.Hqk);  // grouped value heads share q and k
    u32x4 kraw[NU][NP], qraw[NU][NP];
#pragma unroll
    for (int it = 0; it < NU; ++it) {
      const int u = tid + it * kThreads;
      const int r = u / UPR, pi = u % UPR;
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int piece = VEC == 8 ? 4 * (pi >> 1) + (pi & 1) + 2 * j : pi;
        kraw[it][j] = u32x4{0, 0, 0, 0};
        qraw[it][j] = u32x4{0, 0, 0, 0};
        if (r < C) {
          const size_t off = ((size_t)(r0 + r) * p.Hqk + hqk) * DK + piece * VEC;
          kraw[it][j] = *reinterpret_cast<const u32x4 *>(k + off);
          qraw[it][j] = *reinterpret_cast<const u32x4 *>(q + off);
        }
      }
    }
    float bval = 0.f, gval = 0.f;
    if (tid < C) {
      bval = p.beta[(size_t)(r0 + tid) * H + h];
      if (!KDA) gval = p.g[(size_t)(r0 + tid) * H + h];
    }
    constexpr int GIT = KDA ? kBT * DK / 4 / kThreads : 1;  // float4 gate loads per thread
    float4 graw[GIT];
    if constexpr (KDA) {
#pragma unroll
      for (int it = 0; it < GIT; ++it) {
        const int idx = tid + it * kThreads;
        const int r = idx / (DK / 4), c = (idx % (DK / 4)) * 4;
        graw[it] = float4{0.f, 0.f, 0.f, 0.f};
        if (r < C) graw[it] = *reinterpret_cast<const float4 *>(p.g + ((size_t)(r0 + r) * H + h) * DK + c);
      }
    }
#pragma unroll
    for (int it = 0; it < NU; ++it) {
      const int u = tid + it * kThreads;
      const int r = u / UPR, pi = u % UPR;
      T kv[NP][VEC], qv[NP][VEC];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        if constexpr (VEC == 8 && std::is_same<In, f16>::value) {  // fp16: the bits as they are
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[j][2 * e] = f16_from_bits(kraw[it][j][e]);
            kv[j][2 * e + 1] = f16_from_bits(kraw[it][j][e] >> 16);
            qv[j][2 * e] = f16_from_bits(qraw[it][j][e]);
            qv[j][2 * e + 1] = f16_from_bits(qraw[it][j][e] >> 16);
          }
        } else if constexpr (VEC == 8) {  // bf16 -> fp16
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[j][2 * e] = (T)__uint_as_float(kraw[it][j][e] << 16);
            kv[j][2 * e + 1] = (T)__uint_as_float(kraw[it][j][e] & 0xffff0000u);
            qv[j][2 * e] = (T)__uint_as_float(qraw[it][j][e] << 16);
            qv[j][2 * e + 1] = (T)__uint_as_float(qraw[it][j][e] & 0xffff0000u);
          }
        } else {  // fp32
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[j][e] = (T)__uint_as_float(kraw[it][j][e]);
            qv[j][e] = (T)__uint_as_float(qraw[it][j][e]);
          }
        }
        const int piece = VEC == 8 ? 4 * (pi >> 1) + (pi & 1) + 2 * j : pi;
        *reinterpret_cast<u32x4 *>(sK + r * LDK + piece * VEC) = *reinterpret_cast<const u32x4 *>(kv[j]);
        *reinterpret_cast<u32x4 *>(sQ + r * LDK + piece * VEC) = *reinterpret_cast<const u32x4 *>(qv[j]);
      }
      if constexpr (!KDA && SKIP == 0) {  // the reduce's K and Q operands, chained order
        if constexpr (VEC == 8) {
          const int cp = 4 * (pi >> 1) + 2 * (pi & 1);
          T lo[8], hi[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = kv[0][e];
            lo[4 + e] = kv[1][e];
            hi[e] = kv[0][4 + e];
            hi[4 + e] = kv[1][4 + e];
          }
          put(I.K, PK, r, cp, lo);
          put(I.K, PK, r, cp + 1, hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = qv[0][e];
            lo[4 + e] = qv[1][e];
            hi[e] = qv[0][4 + e];
            hi[4 + e] = qv[1][4 + e];
          }
          put(I.Q, PK, r, cp, lo);
          put(I.Q, PK, r, cp + 1, hi);
        } else {
          put(I.K, PK, r, pi, kv[0]);
          put(I.Q, PK, r, pi, qv[0]);
        }
      }
    }
    if (tid < kBT) {
      sB[tid] = bval;
      sg[tid] = gval;
    }
    if constexpr (KDA) {
#pragma unroll
      for (int it = 0; it < GIT; ++it) {
        const int idx = tid + it * kThreads;
        *reinterpret_cast<float4 *>(sG + (idx / (DK / 4)) * GS + (idx % (DK / 4)) * 4) = graw[it];
      }
    }
  }
  __syncthreads();
  if constexpr (!KDA && O::KPL == 1) {
    // fp32 GDN: K^T for the reduce's state update (chunk rows chained = natural)
    for (int idx = tid; idx < DK * PT; idx += kThreads) {
      const int c = idx / PT, pc = idx % PT;
      T v[CH];
#pragma unroll
      for (int e = 0; e < CH; ++e) v[e] = sK[kidx<O>(pc * CH + e) * LDK + c];
      put(I.KT, PT, c, pc, v);
    }
  }

  // M tile (R, S) from an accumulator -> sMt (natural order; the write-out
  // below zeroes the upper triangle)
  auto store_m = [&](int R, int S, const f32x4 &c) {
    const int s = 16 * S + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) sMt[(16 * R + lg * 4 + e) * LDM + s] = (T)c[e];
  };

  if constexpr (!KDA) {
    // ---- masked products: A (strict lower, fp32 -> sL) and M (-> workspace)
    const float G = wave_inclusive_scan(sg[lane]);  // lane r holds G_r
    // 10 lower tiles of K K^T then 10 of Q K^T: 5 per wave, wave w takes w + 4i
    f32x4 a5[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int t = w + 4 * i;
      const int pr = t % 10;
      const int R = tile_r(pr), S = tile_s(pr);
      const T *src = t < 10 ? sK : sQ;
      f32x4 c = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += KSTEP)
        c = O::mfma(frag_lds<O>(src, LDK, 16 * R, k0, lane), frag_lds<O>(sK, LDK, 16 * S, k0, lane),
                    c);
      a5[i] = c;
    }
    __syncthreads();  // K / Q are dead: their bytes now hold A and A^-1
    const float GC = __shfl(G, kBT - 1, 64);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int t = w + 4 * i;
      const int pr = t % 10;
      const int R = tile_r(pr), S = tile_s(pr);
      const int s = 16 * S + lr;
      const float Gs = __shfl(G, s, 64);
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + lg * 4 + e;
        v[e] = a5[i][e] * __expf(__shfl(G, r, 64) - Gs);
      }
      if (t < 10) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + lg * 4 + e;
          sL[r * LDL + s] = s < r ? sB[r] * v[e] : 0.f;
        }
      } else {
        store_m(R, S, v);
      }
    }
    if (w == 0) {
      vec[lane] = __expf(G);
      vec[64 + lane] = __expf(GC - G);
      vec[128 + lane] = sB[lane];
      const float gC = __expf(GC);
      for (int d = lane; d < DK; d += 64) vec[192 + d] = gC;
    }
  } else {
    // per-channel inclusive cumsum: SEG row segments per channel, then the
    // totals of earlier segments are added
    {
      constexpr int SEG = kThreads / DK, RPS = kBT / SEG;
      const int c = tid % DK, sgi = tid / DK;
      float run = 0.f;
      for (int r = sgi * RPS; r < (sgi + 1) * RPS; ++r) {
        run += sG[r * GS + c];
        sG[r * GS + c] = run;
      }
      __syncthreads();
      float off = 0.f;
      for (int s2 = 0; s2 < sgi; ++s2) off += sG[((s2 + 1) * RPS - 1) * GS + c];
      __syncthreads();
      if (sgi > 0)
        for (int r = sgi * RPS; r < (sgi + 1) * RPS; ++r) sG[r * GS + c] += off;
      __syncthreads();
    }
    // decayed operands for the reduce, in chained order
    {
      for (int idx = tid; idx < kBT * PK; idx += kThreads) {
        const int r = idx / PK, pc = idx % PK;
        T kv[CH], qv[CH];
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          const int c = kidx<O>(pc * CH + e);
          const float f = __expf(sG[r * GS + c]);
          kv[e] = (T)((float)sK[r * LDK + c] * f);
          qv[e] = (T)((float)sQ[r * LDK + c] * f);
        }
        put(I.K, PK, r, pc, kv);
        put(I.Q, PK, r, pc, qv);
      }
      for (int idx = tid; idx < DK * PT; idx += kThreads) {
        const int c = idx / PT, pc = idx % PT;
        const float GC = sG[(kBT - 1) * GS + c];
        T v[CH];
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          const int r = kidx<O>(pc * CH + e);
          v[e] = (T)((float)sK[r * LDK + c] * __expf(GC - sG[r * GS + c]));
        }
        put(I.KT, PT, c, pc, v);
      }
      if (tid < kBT) {
        vec[tid] = 1.f;
        vec[64 + tid] = 1.f;
        vec[128 + tid] = sB[tid];
      }
      for (int d = tid; d < DK; d += kThreads) vec[192 + d] = __expf(sG[(kBT - 1) * GS + d]);
    }
    // off-diagonal 16x16 tiles (R, S), S < R, wave w taking tiles w and
    // w + 4 of (1,0) (2,0) (2,1) (3,0) (3,1) (3,2): the decay of pair (r, s)
    // factors through row b = 16R per channel,
    //   k_rc e^{G_rc - G_bc} * k_sc e^{G_bc - G_sc},
    // both factors <= 1 when g <= 0.  Each lane forms its row's KPL channels
    // of both factors in registers (lane row r = b + lr for the A operands,
    // s = 16S + lr for the B operand) and feeds them to the MFMAs.
    f32x4 oca[2], ocm[2];  // this wave's off-diagonal tiles, written after the barrier
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int t = w + 4 * ti;
      if (t >= 6) break;
      const int R = t < 1 ? 1 : t < 3 ? 2 : 3, S = t - R * (R - 1) / 2;
      const int b = 16 * R, r = b + lr, s = 16 * S + lr;
      f32x4 ca = zero4(), cm = zero4();
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += KSTEP) {
        const int c = k0 + lg * O::KPL;
        float fk[O::KPL], fq[O::KPL], hs[O::KPL];
#pragma unroll
        for (int e = 0; e < O::KPL; ++e) {
          const float gb = sG[b * GS + c + e];
          const float er = __expf(sG[r * GS + c + e] - gb);
          const float es = __expf(gb - sG[s * GS + c + e]);
          fk[e] = (float)sK[r * LDK + c + e] * er;
          fq[e] = (float)sQ[r * LDK + c + e] * er;
          hs[e] = (float)sK[s * LDK + c + e] * es;
        }
        typename O::Frag af, qf, hf;
        if constexpr (O::KPL == 1) {
          af = fk[0];
          qf = fq[0];
          hf = hs[0];
        } else {
#pragma unroll
          for (int e = 0; e < O::KPL; ++e) {
            af[e] = (T)fk[e];
            qf[e] = (T)fq[e];
            hf[e] = (T)hs[e];
          }
        }
        ca = O::mfma(af, hf, ca);
        cm = O::mfma(qf, hf, cm);
      }
      oca[ti] = ca;
      ocm[ti] = cm;
    }
    // diagonal blocks: wave w takes block w (rows b .. b+15).  The decay of
    // pair (r, s) factors through row b per channel,
    //   k_rc e^{G_rc - G_bc} * k_sc e^{G_bc - G_sc},
    // so both products are fp32 MFMAs (k = channel; lane row r supplies the
    // A value of row r and the B value of column r).  The second factor grows
    // with the block's decay: a block where some |G_rc - G_bc| exceeds 60 is
    // summed elementwise instead, so no factor leaves the fp32 range.
    f32x4 dca = zero4(), dcm = zero4();  // this wave's diagonal block
    float ea[4], em[4];                   // or its elementwise sums
    bool diag_mfma;
    {
      const int b = 16 * w, r = b + lr;
      f32x4 ca = zero4(), cm = zero4();
      float span = 0.f;
#pragma unroll 4
      for (int c0 = 0; c0 < DK; c0 += 4) {
        const int c = c0 + lg;
        const float d = sG[r * GS + c] - sG[b * GS + c];
        span = fmaxf(span, fabsf(d));
        const float e1 = __expf(d), e2 = __expf(-d);
        const float kr = (float)sK[r * LDK + c], qr = (float)sQ[r * LDK + c];
        const float hs = kr * e2;
        ca = F32::mfma(kr * e1, hs, ca);
        cm = F32::mfma(qr * e1, hs, cm);
      }
      diag_mfma = __ballot(span > 60.f) == 0;
      if (diag_mfma) {
        dca = ca;
        dcm = cm;
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int idx = lane + 64 * q4;
          const int rr = b + (idx >> 4), ss = b + (idx & 15);
          float a = 0.f, m = 0.f;
          if (ss <= rr) {
            for (int c = 0; c < DK; ++c) {
              const float e = __expf(sG[rr * GS + c] - sG[ss * GS + c]);
              const float ks = (float)sK[ss * LDK + c];
              a += (float)sK[rr * LDK + c] * ks * e;
              m += (float)sQ[rr * LDK + c] * ks * e;
            }
          }
          ea[q4] = a;
          em[q4] = m;
        }
      }
    }
    __syncthreads();  // K and Q are dead: A and M take their bytes
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
      const int t = w + 4 * ti;
      if (t >= 6) break;
      const int R = t < 1 ? 1 : t < 3 ? 2 : 3, S = t - R * (R - 1) / 2;
      const int b = 16 * R, s = 16 * S + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = b + lg * 4 + e;
        sL[rr * LDL + s] = sB[rr] * oca[ti][e];
      }
      store_m(R, S, ocm[ti]);
    }
    {
      const int b = 16 * w, s = b + lr;
      if (diag_mfma) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = b + lg * 4 + e;
          sL[rr * LDL + s] = s < rr ? sB[rr] * dca[e] : 0.f;
          sMt[rr * LDM + s] = s <= rr ? (T)dcm[e] : (T)0.f;
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int idx = lane + 64 * q4;
          const int rr = b + (idx >> 4), ss = b + (idx & 15);
          sL[rr * LDL + ss] = ss < rr ? sB[rr] * ea[q4] : 0.f;
          sMt[rr * LDM + ss] = (T)em[q4];
        }
      }
    }
  }
  __syncthreads();
  // ---- X = (I + L)^-1: diagonal blocks by forward substitution, lane =
  // column; wave 0 solves them into registers while the M write-out runs
  float xd[16];
  if (w == 0) {
    const int blk = lane >> 4, c = lane & 15;
    const float *Lb = sL + (16 * blk) * LDL + 16 * blk;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float lrow[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v = *reinterpret_cast<const float4 *>(Lb + r * LDL + 4 * q4);
        lrow[4 * q4] = v.x;
        lrow[4 * q4 + 1] = v.y;
        lrow[4 * q4 + 2] = v.z;
        lrow[4 * q4 + 3] = v.w;
      }
      float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) acc -= lrow[s] * xd[s];
      xd[r] = acc;
    }
  }
  // M -> image, chained columns, upper triangle zero (the reduce reads whole
  // k-steps)
  for (int idx = tid; idx < kBT * PT; idx += kThreads) {
    const int r = idx / PT, pc = idx % PT;
    T v[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int s = kidx<O>(pc * CH + e);
      v[e] = s <= r ? sMt[r * LDM + s] : (T)0.f;
    }
    put(I.MM, PT, r, pc, v);
  }
  __syncthreads();  // M is written out: X may take its bytes
  if (w == 0) {
    const int blk = lane >> 4, c = lane & 15;
    float *Xb = sX + (16 * blk) * LDL + 16 * blk;
#pragma unroll
    for (int r = 0; r < 16; ++r) Xb[r * LDL + c] = xd[r];
  }
  __syncthreads();
  // block rows below the diagonal: X_ij = -X_ii sum_{k=j}^{i-1} L_ik X_kj, by i - j
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    const int j = w, i = w + dist;
    if (i < 4) {
      f32x4 y = zero4();
      for (int kb = j; kb < i; ++kb) {
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const float a = sL[(16 * i + lr) * LDL + 16 * kb + k0 + lg];
          const float bb = sX[(16 * kb + k0 + lg) * LDL + 16 * j + lr];
          y = F32::mfma(a, bb, y);
        }
      }
      float *Y = sY[w];
#pragma unroll
      for (int e = 0; e < 4; ++e) Y[(lg * 4 + e) * 17 + lr] = y[e];
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      f32x4 x = zero4();
#pragma unroll
      for (int k0 = 0; k0 < 16; k0 += 4) {
        const float a = sX[(16 * i + lr) * LDL + 16 * i + k0 + lg];
        const float bb = Y[(k0 + lg) * 17 + lr];
        x = F32::mfma(a, bb, x);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sX[(16 * i + lg * 4 + e) * LDL + 16 * j + lr] = -x[e];
    }
    __syncthreads();
  }
  // ---- Tn = X diag(beta), strict lower part, chained columns
  for (int idx = tid; idx < kBT * PT; idx += kThreads) {
    const int r = idx / PT, pc = idx % PT;
    T v[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int s = kidx<O>(pc * CH + e);
      v[e] = (T)(s < r ? sX[r * LDL + s] * sB[s] : 0.f);
    }
    put(I.TN, PT, r, pc, v);
  }
}

// ---------------------------------------------------------------------------
// 16-bit GDN (bf16 / fp16 inputs on fp16 MFMA): a persistent kernel, one
// workgroup per resident slot, walking cells (chunk slot, head).  Workgroups
// are dispatched to the 8 XCDs round-robin (b on XCD b % 8), and XCD x takes
// the slots s = x (mod 8) with all their heads: the g / beta lines of a
// slot's rows (every head of a token shares one) are then fetched into one
// XCD's L2 only.  The workgroups of an XCD walk its cells with a stride of
// their count.  The raw q / k rows of a workgroup's next cell are loaded into
// registers while it computes the current one, so the HBM reads of one cell
// overlap the products, the inverse and the stores of the previous.
//
// Every tile (R, S) of K K^T and Q K^T is one accumulator formed with
// A = K row tile S and B = K / Q row tile R: lane l holds row 16 R + l%16 at
// columns 16 S + 4 (l/16) .. +3, so M and Tn leave as 8-byte row pieces in
// the image's chained column order.  Products over the natural key order
// (both operands read alike).  Wave roles, per cell:
//   products:  w0 the diagonal tiles of K K^T, w1 its six lower tiles,
//              w2 the diagonal tiles of Q K^T and tile (1, 0), w3 the rest;
//   masks:     w0 L's diagonal blocks (fp32, column-major) and their inverse
//              X_ii by forward substitution, one lane per column; w1 L's rows
//              16..63 as fp16 hi / lo operands and the zero tiles; w2, w3 M
//              and the row vectors;
//   levels:    X_ij = -X_ii sum_{k=j}^{i-1} L_ik X_kj on fp16 hi / lo MFMAs
//              (about fp32 accuracy): w0 block column 0, w1 block columns 1
//              and 2; w2 Tn's diagonal tiles.
template <typename In, int DK, bool RAW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void chunk_map16_kernel(MapParams p) {
  using O = Op<In>;
  using T = typename O::T;
  static_assert(O::KPL == 8, "16-bit inputs");
  constexpr int LDK = DK + O::PAD;  // K / Q row stride (elements)
  constexpr int KSTEP = 32;
  constexpr int NKS = DK / KSTEP;
  constexpr int KQ_BYTES = 2 * kBT * LDK * 2;
  // inverse scratch over the K / Q bytes: L's diagonal blocks column-major
  // (fp32), L's rows 16..63 fp16 hi and lo (chained columns, swizzled), X_ii
  // row-major and column-major (fp32).  The 16x16 fp32 blocks sit BS bytes
  // apart (1 KiB + 64): the four blocks' accesses of one instruction fall on
  // different LDS banks.
  constexpr int BS = 1024 + 64;
  constexpr int LT = 0, LH = 4 * BS, LL = LH + 48 * 128, XR = LL + 48 * 128, XT = XR + 4 * BS;
  constexpr int AREA = KQ_BYTES > XT + 4 * BS ? KQ_BYTES : XT + 4 * BS;
  __shared__ __attribute__((aligned(16))) char sArea[AREA];
  __shared__ __attribute__((aligned(16))) float sGw[4][kBT];  // G, one copy per wave
  __shared__ __attribute__((aligned(16))) float sB[kBT];
  __shared__ __attribute__((aligned(16))) float sg[kBT];
  T *sK = reinterpret_cast<T *>(sArea);
  T *sQ = sK + kBT * LDK;
  char *sc = sArea;
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));

  const int H = p.H;
  const int w = wave_id();
  constexpr ImageLayout I = image_layout(false, 2, DK);
  constexpr int PK = DK * 2 / 16;
  constexpr int SKIP = image_skip(false, 2, DK, RAW);
  constexpr int HBM = image_hbm_bytes(false, 2, DK, RAW);
  float *Gw = sGw[w];

  // staging unit of a thread: row r, 32-element block b, half g2: input
  // pieces 4b + g2 and 4b + 2 + g2 (8 elements each), which hold exactly the
  // chained pieces 4b + 2 g2 (their low halves) and 4b + 2 g2 + 1 (their high
  // halves)
  constexpr int UPR = DK / 16;
  constexpr int NU = kBT * UPR / kThreads;
  static_assert(kBT * UPR % kThreads == 0, "staging split");
  const In *qsrc = static_cast<const In *>(p.q);
  const In *ksrc = static_cast<const In *>(p.k);
  const int G = H / p.Hqk;  // grouped value heads share q and k
  u32x4 kraw[NU][2], qraw[NU][2];
  float bval, gval;
  // the cell's chunk: first row, valid rows (0: sentinel)
  // the chunk layout, when this kernel builds it: each wave derives it and
  // keeps its lanes' slot ends in a row of sEnd of its own (read back by
  // the same wave only, so no barrier), wave 0 of workgroup b stores slots
  // b, b + grid, ...
  __shared__ int sEnd[kThreads / 64][64];
  if (p.fuse_meta) {
    const WaveLayout L = wave_layout(p);
    if (w == 0) layout_store(p, L, blockIdx.x, gridDim.x, blockIdx.x == 0);
    sEnd[w][lane_id()] = L.end;
  }
  auto cell_rows = [&](int cell, int &r0, int &C) {
    const int slot = cell / H;
    int i_n, i_t;
    if (p.fuse_meta) {
      layout_slot(sEnd[w][lane_id()], slot, i_n, i_t);
    } else {
      i_n = p.chunk_indices[2 * slot];
      i_t = i_n < 0 ? 0 : p.chunk_indices[2 * slot + 1];
    }
    C = 0;
    r0 = 0;
    if (i_n < 0) return;
    const int bos = cu_at(p.cu_seqlens, p.cu64, i_n);
    const int eos = cu_at(p.cu_seqlens, p.cu64, i_n + 1);
    r0 = bos + i_t * kBT;
    C = min(kBT, eos - r0);
  };
  auto load = [&](int tid, int cell, int r0, int C) {
    const int h = cell % H, hqk = h / G;
#pragma unroll
    for (int it = 0; it < NU; ++it) {
      const int u = tid + it * kThreads;
      const int r = u / UPR, pi = u % UPR;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int piece = 4 * (pi >> 1) + (pi & 1) + 2 * j;
        kraw[it][j] = u32x4{0, 0, 0, 0};
        qraw[it][j] = u32x4{0, 0, 0, 0};
        if (r < C) {
          const size_t off = ((size_t)(r0 + r) * p.Hqk + hqk) * DK + piece * 8;
          kraw[it][j] = *reinterpret_cast<const u32x4 *>(ksrc + off);
          qraw[it][j] = *reinterpret_cast<const u32x4 *>(qsrc + off);
        }
      }
    }
    bval = 0.f;
    gval = 0.f;
    if (tid < C) {
      bval = p.beta[(size_t)(r0 + tid) * H + h];
      gval = p.g[(size_t)(r0 + tid) * H + h];
    }
  };
  auto cvt = [](uint32_t x) -> T {  // one 16-bit input value in the low half
    if constexpr (std::is_same<In, f16>::value) return f16_from_bits(x);
    else return (T)__uint_as_float(x << 16);
  };

  // this workgroup's k-th cell: index jw + k * per of its XCD's cells, -1
  // past the last slot (the grid is a multiple of 8)
  const int xcd = blockIdx.x & 7, per = gridDim.x >> 3, jw = blockIdx.x >> 3;
  auto cell_at = [&](int k) {
    const int i = jw + k * per, slot = xcd + 8 * (i / H);
    return slot < p.NT_max ? slot * H + i % H : -1;
  };
  int kc = 0;
  int cell = cell_at(0);
  if (cell < 0) return;
  int r0, C;
  cell_rows(cell, r0, C);
  if (C <= 0) return;  // sentinel: this and every later cell (slots fill in order)
  load((int)threadIdx.x, cell, r0, C);

  auto oR = [](int i) { return i < 1 ? 1 : i < 3 ? 2 : 3; };          // lower tile i:
  auto oS = [](int i) { return i < 1 ? 0 : i < 3 ? i - 1 : i - 3; };  // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
  auto t8 = [](int r, int pc, int half) { return tile_off<8>(r, pc) + 8 * half; };
  auto put4 = [](char *dst, const f32x4 &v) {
    *reinterpret_cast<h4 *>(dst) = h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  };
  auto lo16 = [](float v) { return (_Float16)(v - (float)(_Float16)v); };

  for (;;) {
    // lane-derived offsets are formed anew in every pass, not kept live
    // across the loop
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    const int lr = lane & 15, lg = lane >> 4, tid = 64 * w + lane;
    const int h = cell % H;
    char *img = static_cast<char *>(p.img) + (size_t)cell * HBM - SKIP;
    float *vec = reinterpret_cast<float *>(img + I.VEC);

    // ---- stage K, Q (fp16, natural order; rows >= C zero), beta, g
#pragma unroll
    for (int it = 0; it < NU; ++it) {
      const int u = tid + it * kThreads;
      const int r = u / UPR, pi = u % UPR;
      T kv[2][8], qv[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[j][2 * e] = cvt(kraw[it][j][e]);
          kv[j][2 * e + 1] = cvt(kraw[it][j][e] >> 16);
          qv[j][2 * e] = cvt(qraw[it][j][e]);
          qv[j][2 * e + 1] = cvt(qraw[it][j][e] >> 16);
        }
        const int piece = 4 * (pi >> 1) + (pi & 1) + 2 * j;
        *reinterpret_cast<u32x4 *>(sK + r * LDK + piece * 8) = *reinterpret_cast<const u32x4 *>(kv[j]);
        *reinterpret_cast<u32x4 *>(sQ + r * LDK + piece * 8) = *reinterpret_cast<const u32x4 *>(qv[j]);
      }
      if constexpr (!RAW) {  // the reduce's K and Q operands, chained order
        const int cp = 4 * (pi >> 1) + 2 * (pi & 1);
        T lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = kv[0][e];
          lo[4 + e] = kv[1][e];
          hi[e] = kv[0][4 + e];
          hi[4 + e] = kv[1][4 + e];
        }
        *reinterpret_cast<u32x4 *>(img + I.K + tile_off<PK>(r, cp)) = *reinterpret_cast<const u32x4 *>(lo);
        *reinterpret_cast<u32x4 *>(img + I.K + tile_off<PK>(r, cp + 1)) = *reinterpret_cast<const u32x4 *>(hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = qv[0][e];
          lo[4 + e] = qv[1][e];
          hi[e] = qv[0][4 + e];
          hi[4 + e] = qv[1][4 + e];
        }
        *reinterpret_cast<u32x4 *>(img + I.Q + tile_off<PK>(r, cp)) = *reinterpret_cast<const u32x4 *>(lo);
        *reinterpret_cast<u32x4 *>(img + I.Q + tile_off<PK>(r, cp + 1)) = *reinterpret_cast<const u32x4 *>(hi);
      }
    }
    if (tid < kBT) {
      sB[tid] = bval;
      sg[tid] = gval;
    }
    // the next cell's rows (issued once the current ones are consumed)
    const int next = cell_at(kc + 1);
    int nr0 = 0, nC = 0;
    if (next >= 0) cell_rows(next, nr0, nC);
    __syncthreads();  // S1: K, Q, beta, g in LDS

    const float Gl = wave_inclusive_scan(sg[lane]);  // lane r holds G_r
    Gw[lane] = Gl;
    f32x4 a[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) a[i] = zero4();
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if (w < 2) {
        typename O::Frag kf[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) kf[R] = frag_lds<O>(sK, LDK, 16 * R, KSTEP * s, lane);
        if (w == 0) {
#pragma unroll
          for (int R = 0; R < 4; ++R) a[R] = O::mfma(kf[R], kf[R], a[R]);
        } else {
#pragma unroll
          for (int i = 0; i < 6; ++i) a[i] = O::mfma(kf[oS(i)], kf[oR(i)], a[i]);
        }
      } else if (w == 2) {
        typename O::Frag kf[4], qf[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          kf[R] = frag_lds<O>(sK, LDK, 16 * R, KSTEP * s, lane);
          qf[R] = frag_lds<O>(sQ, LDK, 16 * R, KSTEP * s, lane);
        }
#pragma unroll
        for (int R = 0; R < 4; ++R) a[R] = O::mfma(kf[R], qf[R], a[R]);
        a[4] = O::mfma(kf[0], qf[1], a[4]);
      } else {
        typename O::Frag kf[3], qf[2];
#pragma unroll
        for (int R = 0; R < 3; ++R) kf[R] = frag_lds<O>(sK, LDK, 16 * R, KSTEP * s, lane);
#pragma unroll
        for (int R = 0; R < 2; ++R) qf[R] = frag_lds<O>(sQ, LDK, 16 * (R + 2), KSTEP * s, lane);
#pragma unroll
        for (int i = 1; i < 6; ++i) a[i - 1] = O::mfma(kf[oS(i)], qf[oR(i) - 2], a[i - 1]);
      }
    }
    __syncthreads();  // S2: K and Q are dead, the inverse's scratch takes their bytes
    if (nC > 0) load(tid, next, nr0, nC);

    if (w == 0) {
      // L's diagonal blocks, column-major: the product is symmetric, so lane
      // (row lr, columns 4 lg + e) also holds row 4 lg + e at column lr:
      //   L_rs = beta_r (K K^T)_rs exp(G_r - G_s), s < r
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const float gs = Gw[16 * R + lr];
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(Gw + 16 * R + 4 * lg);
        const f32x4 br = *reinterpret_cast<const f32x4 *>(sB + 16 * R + 4 * lg);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = 4 * lg + e > lr ? br[e] * a[R][e] * __expf(gr[e] - gs) : 0.f;
        *reinterpret_cast<f32x4 *>(sc + LT + R * BS + lr * 64 + lg * 16) = v;
      }
      // X_ii = (I + L_ii)^-1, column c = l%16 of block l/16, in column order:
      // once x_s is final, x_r -= L_rs x_s for every r > s.  Column s of L
      // is read three steps ahead of its use.
      const int blk = lane >> 4, c = lane & 15;
      const char *Lb = sc + LT + blk * BS;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = r == c ? 1.f : 0.f;
      f32x4 lc[15][4];
      auto ldcol = [&](int s) {
#pragma unroll
        for (int q4 = (s + 1) >> 2; q4 < 4; ++q4) lc[s][q4] = *reinterpret_cast<const f32x4 *>(Lb + s * 64 + 16 * q4);
      };
      ldcol(0);
      ldcol(1);
      ldcol(2);
#pragma unroll
      for (int s = 0; s < 15; ++s) {
        if (s + 3 < 15) ldcol(s + 3);
        const float xs = x[s];
#pragma unroll
        for (int q4 = (s + 1) >> 2; q4 < 4; ++q4)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * q4 + e > s) x[4 * q4 + e] = fmaf(-lc[s][q4][e], xs, x[4 * q4 + e]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) *reinterpret_cast<float *>(sc + XR + blk * BS + r * 64 + c * 4) = x[r];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4 *>(sc + XT + blk * BS + c * 64 + 16 * q4) =
            f32x4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
    } else if (w == 1) {
      // L's rows 16..63 as fp16 hi / lo A operands of the levels; the
      // diagonal tiles 1 and 3, read there against zero operands, zero
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int R = oR(i), S = oS(i), r = 16 * R + lr;
        const float grr = Gw[r], brr = sB[r];
        const f32x4 gs = *reinterpret_cast<const f32x4 *>(Gw + 16 * S + 4 * lg);
        h4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = a[i][e] * brr * __expf(grr - gs[e]);
          hi[e] = (_Float16)v;
          lo[e] = lo16(v);
        }
        const int o = t8(r - 16, 4 * (S >> 1) + lg, S & 1);
        *reinterpret_cast<h4 *>(sc + LH + o) = hi;
        *reinterpret_cast<h4 *>(sc + LL + o) = lo;
      }
#pragma unroll
      for (int R = 1; R < 4; R += 2) {
        const int o = t8(16 * R - 16 + lr, 4 * (R >> 1) + lg, R & 1);
        *reinterpret_cast<h4 *>(sc + LH + o) = h4{0, 0, 0, 0};
        *reinterpret_cast<h4 *>(sc + LL + o) = h4{0, 0, 0, 0};
      }
      // the tiles above the diagonal that the reduce reads (the upper halves
      // of the 32-column k-steps of block rows 0 and 2): zero.  Tiles (0,2),
      // (0,3), (1,2) and (1,3) are read by no one and not written.
#pragma unroll
      for (int R = 0; R < 4; R += 2) {
        const int o = t8(16 * R + lr, 4 * (R >> 1) + lg, 1);
        put4(img + I.MM + o, zero4());
        put4(img + I.TN + o, zero4());
      }
    } else if (w == 2) {
      // M_rs = (Q K^T)_rs exp(G_r - G_s), s <= r: the diagonal tiles, (1, 0)
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int R = i < 4 ? i : 1, S = i < 4 ? i : 0, r = 16 * R + lr;
        const float grr = Gw[r];
        const f32x4 gs = *reinterpret_cast<const f32x4 *>(Gw + 16 * S + 4 * lg);
        f32x4 mv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float m = a[i][e] * __expf(grr - gs[e]);
          mv[e] = i == 4 || 4 * lg + e <= lr ? m : 0.f;
        }
        put4(img + I.MM + t8(r, 4 * (S >> 1) + lg, S & 1), mv);
      }
    } else {
      // M's tiles (2,0) (2,1) (3,0) (3,1) (3,2); the row vectors
#pragma unroll
      for (int i = 1; i < 6; ++i) {
        const int R = oR(i), S = oS(i), r = 16 * R + lr;
        const float grr = Gw[r];
        const f32x4 gs = *reinterpret_cast<const f32x4 *>(Gw + 16 * S + 4 * lg);
        f32x4 mv;
#pragma unroll
        for (int e = 0; e < 4; ++e) mv[e] = a[i - 1][e] * __expf(grr - gs[e]);
        put4(img + I.MM + t8(r, 4 * (S >> 1) + lg, S & 1), mv);
      }
      const float GC = Gw[kBT - 1];
      vec[lane] = __expf(Gl);
      vec[64 + lane] = __expf(GC - Gl);
      vec[128 + lane] = sB[lane];
      const float gC = __expf(GC);
      for (int d = lane; d < DK; d += 64) vec[192 + d] = gC;
    }
    __syncthreads();  // S3: L's hi / lo rows and the diagonal blocks of X are in LDS
    if (w < 2) {
      // The B operands X_kj stay in accumulators (chained k order, b_frag's
      // layout); Tn_ij = X_ij diag(beta_j) is transposed for its row-wise
      // store by one MFMA against an identity operand.
      const f32x4 z = zero4();
      auto bsplit = [&](const f32x4 &t0, const f32x4 &t1, half8 &bh, half8 &bl) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bh[e] = (_Float16)t0[e];
          bl[e] = lo16(t0[e]);
          bh[4 + e] = (_Float16)t1[e];
          bl[4 + e] = lo16(t1[e]);
        }
      };
      auto mfma3 = [&](const half8 &ah, const half8 &al, const half8 &bh, const half8 &bl, f32x4 c) {
        c = O::mfma(ah, bh, c);
        c = O::mfma(ah, bl, c);
        return O::mfma(al, bh, c);
      };
      auto close = [&](int i, const f32x4 &y) {  // -X_ii Y
        const f32x4 xv = *reinterpret_cast<const f32x4 *>(sc + XR + i * BS + lr * 64 + lg * 16);
        half8 ah, al, bh, bl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ah[e] = (_Float16)xv[e];
          al[e] = lo16(xv[e]);
          ah[4 + e] = (_Float16)0.f;
          al[4 + e] = (_Float16)0.f;
        }
        bsplit(y, z, bh, bl);
        const f32x4 r = mfma3(ah, al, bh, bl, z);
        return f32x4{-r[0], -r[1], -r[2], -r[3]};
      };
      auto lev = [&](int i, int s, const f32x4 &t0, const f32x4 &t1, const f32x4 &y) {  // y + L_i,[2s,2s+1] [t0; t1]
        const int o = tile_off<8>(16 * i - 16 + lr, 4 * s + lg);
        const half8 ah = *reinterpret_cast<const half8 *>(sc + LH + o);
        const half8 al = *reinterpret_cast<const half8 *>(sc + LL + o);
        half8 bh, bl;
        bsplit(t0, t1, bh, bl);
        return mfma3(ah, al, bh, bl, y);
      };
      auto xcol = [&](int j) {  // X_jj as an accumulator tile
        return *reinterpret_cast<const f32x4 *>(sc + XT + j * BS + lr * 64 + lg * 16);
      };
      auto put_tn = [&](int i, int j, const f32x4 &x) {
        const float bj = sB[16 * j + lr];
        half8 ident, av;  // B = [I; 0]: lane l supplies rows 4 (l/16) .. +3 of column l%16
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ident[e] = (_Float16)(4 * lg + e == lr ? 1.f : 0.f);
          ident[4 + e] = (_Float16)0.f;
          av[e] = (_Float16)(x[e] * bj);
          av[4 + e] = (_Float16)0.f;
        }
        put4(img + I.TN + t8(16 * i + lr, 4 * (j >> 1) + lg, j & 1), O::mfma(av, ident, z));
      };
      if (w == 0) {
        const f32x4 x00 = xcol(0);
        const f32x4 x10 = close(1, lev(1, 0, x00, z, z));
        const f32x4 x20 = close(2, lev(2, 0, x00, x10, z));
        const f32x4 x30 = close(3, lev(3, 1, x20, z, lev(3, 0, x00, x10, z)));
        put_tn(1, 0, x10);
        put_tn(2, 0, x20);
        put_tn(3, 0, x30);
      } else {
        const f32x4 x11 = xcol(1), x22 = xcol(2);
        const f32x4 x21 = close(2, lev(2, 0, z, x11, z));
        const f32x4 x31 = close(3, lev(3, 1, x21, z, lev(3, 0, z, x11, z)));
        const f32x4 x32 = close(3, lev(3, 1, x22, z, z));
        put_tn(2, 1, x21);
        put_tn(3, 1, x31);
        put_tn(3, 2, x32);
      }
    } else if (w == 2) {
      // Tn's diagonal tiles: X_RR diag(beta), strict lower
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const f32x4 xr = *reinterpret_cast<const f32x4 *>(sc + XR + R * BS + lr * 64 + lg * 16);
        const f32x4 bs = *reinterpret_cast<const f32x4 *>(sB + 16 * R + 4 * lg);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = 4 * lg + e < lr ? xr[e] * bs[e] : 0.f;
        put4(img + I.TN + t8(16 * R + lr, 4 * (R >> 1) + lg, R & 1), v);
      }
    }
    if (nC <= 0) break;  // no next cell, or a sentinel (slots fill in order)
    cell = next;
    ++kc;
    __syncthreads();  // S4: the scratch is free for the next cell's K and Q
  }
}

}  // namespace

template <bool KDA, typename In, int DK, bool RAW>
static hipError_t launch_map_t(const MapParams &p, hipStream_t st) {
  hipLaunchKernelGGL((chunk_map_kernel<KDA, In, DK, RAW>), dim3(p.H * p.NT_max), dim3(kThreads), 0, st,
                     p);
  return hipGetLastError();
}

// the 16-bit GDN kernel's grid: as many workgroups as the device holds at
// once (CUs x resident workgroups per CU, found once per device), capped by
// the cells
template <typename In, int DK, bool RAW>
static hipError_t launch_map16(const MapParams &p, hipStream_t st) {
  static int slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  int res = dev < 64 ? slots[dev] : 0;
  if (res == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, chunk_map16_kernel<In, DK, RAW>, kThreads, 0) !=
            hipSuccess)
      return hipErrorInvalidValue;
    res = cus * per > 0 ? cus * per : 1;
    if (dev < 64) slots[dev] = res;
  }
  // a multiple of 8 (the kernel's XCD order); workgroups past the cells exit
  const int cells = p.H * p.NT_max;
  const int grid = ((cells < res ? cells : res) + 7) / 8 * 8;
  hipLaunchKernelGGL((chunk_map16_kernel<In, DK, RAW>), dim3(grid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <typename In, int DK>
static hipError_t launch_map_d(const MapParams &p, bool kda, hipStream_t st) {
  if (kda) return launch_map_t<true, In, DK, false>(p, st);
  return p.raw_kq ? launch_map16<In, DK, true>(p, st) : launch_map16<In, DK, false>(p, st);
}

template <typename In>
static hipError_t launch_map_16(const MapParams &p, bool kda, int dk, hipStream_t st) {
  if (dk == 128) return launch_map_d<In, 128>(p, kda, st);
  if (dk == 64) return launch_map_d<In, 64>(p, kda, st);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_map(const MapParams &p, bool kda, int dt, int dk, hipStream_t st) {
  if (dt == LA_BF16) return launch_map_16<bf16>(p, kda, dk, st);
  if (dt == LA_F16) return launch_map_16<f16>(p, kda, dk, st);
  // fp32 inputs: d = 64 only (the fp32 d = 128 KDA tiles exceed the 160 KiB LDS)
  if (dt != LA_F32 || dk != 64) return hipErrorInvalidValue;
  return kda ? launch_map_t<true, float, 64, false>(p, st) : launch_map_t<false, float, 64, false>(p, st);
}

}  // namespace la
