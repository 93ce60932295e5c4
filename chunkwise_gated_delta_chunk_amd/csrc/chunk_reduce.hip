// Sequential reduce + output stage: one workgroup per (sequence, head, d_v
// slice), walking the sequence's chunks in order with its slice of the state
// H = S^T ([d_k][W] fp32) held in registers and updated in place.
//
// Per chunk (GDN; rows r of the chunk, gamma_r = exp(G_r), C = last row):
//   X   = V - diag(gamma) (K H)                        state-corrected values
//   U   = diag(beta) X + Tn X                          Tn = T - diag(beta)
//   O   = scale * (diag(gamma) (Q H) + M U)            forward o
//   H  <- gamma_C H + K^T (diag(gamma_C / gamma) U)    forward h
// K H and Q H share the state operand and are issued together (the grouped
// "K S, Q S" products of "Empowering Hybrid Attention Models on NPUs",
// section 5).  The state is read, the chunk output formed, then the state
// overwritten -- the chunk-first in-place order of the same paper (section 5,
// Figure 10).  Columns of U, O and H depend only on the same columns of V and
// H, so d_v is split into slices with no cross-slice reduction (the
// column-wise split of section 4).
//
// KDA: the map stage has already folded the per-channel decay into the
// operands (K*exp(G), Q*exp(G), (K*exp(G_C - G))^T, exp(G_C)), so the row
// factors are 1 and the state decays by diag(exp(G_C)).
//
// Work split: each wave owns 16 state columns for all chunk rows, so the
// chain H -> K H -> X -> U -> H of one column tile never leaves the wave.
// With the chained k order (see la_device.h) an accumulator tile is itself the
// B operand of the next product, so H, X and U stay in registers; only the
// shared, state-independent operands of a chunk (K, Q, K^T, Tn, M, V and the
// row vectors) are staged in LDS.  They are loaded one chunk ahead through
// buffer resources (loop-invariant lane offsets; rows past the chunk's end
// read as zero by the hardware range check) and written to the other half of
// a double buffer, so one workgroup barrier per chunk suffices and no global
// load is waited for on the chain.
//
// Blocks are numbered so that the slices of one (sequence, head) land on the
// same XCD (workgroup IDs are dealt round-robin over the 8 XCDs) and share
// its L2 for the K, Q and map-stage reads.  Zero-length sequences and padding
// units exit before touching memory, so they write nothing.
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

// byte layout of one buffer of the shared per-chunk operands
template <bool KDA, typename O, typename In, int DK, int W>
struct Stage {
  using T = typename O::T;
  // GDN with fp16 operands reads K^T straight from K with transposing LDS
  // reads; KDA stages its own (K*exp(G_C - G))^T and the fp32 path a copy
  static constexpr bool HAS_KT = KDA || O::KPL == 1;
  static constexpr int LDK = DK + O::PAD;  // K, Q rows: [64][LDK], d_k chained
  static constexpr int LDT = kBT + O::PAD; // K^T rows [DK][LDT], Tn / M rows [64][LDT]
  static constexpr int VECN = 192 + DK;
  static constexpr int K = 0;
  static constexpr int Q = K + kBT * LDK * (int)sizeof(T);
  static constexpr int KT = Q + kBT * LDK * (int)sizeof(T);
  static constexpr int TN = KT + (HAS_KT ? DK * LDT * (int)sizeof(T) : 0);
  static constexpr int MM = TN + kBT * LDT * (int)sizeof(T);
  static constexpr int VEC = MM + kBT * LDT * (int)sizeof(T);
  static constexpr int V = VEC + VECN * 4;                     // V slice [64][W], raw
  static constexpr int BYTES = V + kBT * W * (int)sizeof(In);
  static constexpr int NBUF = 2 * BYTES <= 160 * 1024 ? 2 : 1;
};

template <bool KDA, typename In, int DK, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_reduce_kernel(ReduceParams p) {
  using O = Op<In>;
  using T = typename O::T;
  constexpr int NT = 64 * NW;            // threads
  constexpr int W = 16 * NW;             // state columns per workgroup
  using L = Stage<KDA, O, In, DK, W>;
  constexpr int DV = DK;                 // d_v == d_k
  constexpr int NKD = ksteps<O>(DK);     // k-steps over d_k
  constexpr int NKR = ksteps<O>(kBT);    // k-steps over chunk rows
  constexpr int NHT = DK / 16;           // state row tiles per wave
  constexpr int NBUF = L::NBUF;
  // staging work per thread, in 16-byte pieces
  constexpr int ELEM = KDA ? (int)sizeof(T) : (int)sizeof(In);  // bytes per staged K / Q element
  constexpr int IN_ROW = DK * ELEM / 16;                  // 16-byte pieces per K row
  constexpr int NKQ = kBT * IN_ROW / NT;                  // K (and Q) pieces per thread
  constexpr int NKT = KDA ? DK * kBT * (int)sizeof(T) / 16 / NT : 0;
  constexpr int NTM = kBT * kBT * (int)sizeof(T) / 16 / NT;
  constexpr int NVEC = L::VECN * 4 / 16;                  // vector pieces (< NT)
  constexpr int PV = W * (int)sizeof(In) / 16;            // V pieces per row
  constexpr int NVP = kBT * PV / NT;                      // V pieces per thread
  static_assert(kBT * IN_ROW % NT == 0 && kBT * kBT * (int)sizeof(T) % (16 * NT) == 0, "split");
  static_assert(kBT * PV % NT == 0 && NVEC <= NT, "split");

  __shared__ __attribute__((aligned(16))) char smem[NBUF * L::BYTES];

  // ---- block -> (unit, slice), XCD-aware
  const int b = blockIdx.x;
  const int xcd = b & 7, kk = b >> 3;
  const int slice = kk % p.S, unit = (kk / p.S) * 8 + xcd;
  const int H = p.H;
  if (unit >= p.N_max * H) return;
  const int n = unit / H, h = unit % H;
  const int j0 = p.chunk_offsets[n], j1 = p.chunk_offsets[n + 1];
  if (j0 == j1) return;  // empty sequence (or invalid cu_seqlens): no writes
  const int bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int cw = slice * W + 16 * w;                 // this wave's first state column
  const int rs_qk = H * DK * (int)sizeof(In);        // token stride of q, k (bytes)
  const int rs_v = H * DV * (int)sizeof(In);         // token stride of v (bytes)
  const int rs_o = H * DV * 4;                       // token stride of o (bytes)

  // loop-invariant lane offsets of the staging pieces
  int off_kq[NKQ], off_v[NVP];
#pragma unroll
  for (int i = 0; i < NKQ; ++i) {
    const int c = tid + i * NT;
    off_kq[i] = KDA ? c * 16 : (c / IN_ROW) * rs_qk + (c % IN_ROW) * 16;
  }
#pragma unroll
  for (int i = 0; i < NVP; ++i) {
    const int c = tid + i * NT;
    off_v[i] = (c / PV) * rs_v + (c % PV) * 16;
  }
  int off_o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) off_o[e] = (lg * 4 + e) * rs_o + (cw + lr) * 4;

  // ---------------------------------------------------------------- staging
  struct Raw {
    u32x4 k[NKQ], q[NKQ], kt[NKT > 0 ? NKT : 1], tn[NTM], mm[NTM], vec, v[NVP];
  };
  auto stage_load = [&](Raw &R, int jj) {
    const int r0 = bos + (jj - j0) * kBT;
    const int C = min(kBT, eos - r0);
    const size_t cell = (size_t)jj * H + h;
    const size_t tok = (size_t)r0 * H + h;  // (first row, head) element index
    if constexpr (KDA) {
      const auto rk = buffer_rsrc(static_cast<const T *>(p.Kd_raw) + cell * (kBT * DK), kBT * DK * sizeof(T));
      const auto rq = buffer_rsrc(static_cast<const T *>(p.Qd_raw) + cell * (kBT * DK), kBT * DK * sizeof(T));
      const auto rt = buffer_rsrc(static_cast<const T *>(p.Kbt_raw) + cell * (kBT * DK), kBT * DK * sizeof(T));
#pragma unroll
      for (int i = 0; i < NKQ; ++i) {
        R.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_kq[i], 0, 0);
        R.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, off_kq[i], 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NKT; ++i)
        R.kt[i] = __builtin_amdgcn_raw_buffer_load_b128(rt, (tid + i * NT) * 16, 0, 0);
    } else {
      const auto rk = buffer_rsrc(static_cast<const In *>(p.k) + tok * DK, C * rs_qk);
      const auto rq = buffer_rsrc(static_cast<const In *>(p.q) + tok * DK, C * rs_qk);
#pragma unroll
      for (int i = 0; i < NKQ; ++i) {
        R.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off_kq[i], 0, 0);
        R.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, off_kq[i], 0, 0);
      }
    }
    const auto rtn = buffer_rsrc(static_cast<const T *>(p.Tn_raw) + cell * (kBT * kBT), kBT * kBT * sizeof(T));
    const auto rmm = buffer_rsrc(static_cast<const T *>(p.M_raw) + cell * (kBT * kBT), kBT * kBT * sizeof(T));
#pragma unroll
    for (int i = 0; i < NTM; ++i) {
      R.tn[i] = __builtin_amdgcn_raw_buffer_load_b128(rtn, (tid + i * NT) * 16, 0, 0);
      R.mm[i] = __builtin_amdgcn_raw_buffer_load_b128(rmm, (tid + i * NT) * 16, 0, 0);
    }
    const auto rvec = buffer_rsrc(p.vec + cell * L::VECN, L::VECN * 4);
    R.vec = __builtin_amdgcn_raw_buffer_load_b128(rvec, min(tid, NVEC - 1) * 16, 0, 0);
    const auto rv = buffer_rsrc(static_cast<const In *>(p.v) + tok * DV + slice * W, C * rs_v);
#pragma unroll
    for (int i = 0; i < NVP; ++i) R.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off_v[i], 0, 0);
  };
  auto stage_store = [&](char *buf, const Raw &R) {
    T *sK = reinterpret_cast<T *>(buf + L::K);
    T *sQ = reinterpret_cast<T *>(buf + L::Q);
    T *sKt = reinterpret_cast<T *>(buf + L::KT);
#pragma unroll
    for (int i = 0; i < NKQ; ++i) {
      const int c = tid + i * NT;
      if constexpr (KDA) {
        constexpr int E = 16 / sizeof(T);
        const int r = c / IN_ROW, col = (c % IN_ROW) * E;
        *reinterpret_cast<u32x4 *>(sK + r * L::LDK + col) = R.k[i];
        *reinterpret_cast<u32x4 *>(sQ + r * L::LDK + col) = R.q[i];
      } else if constexpr (sizeof(In) == 2) {
        // 8 bf16 of row r, d_k col..col+7 -> fp16 at chained positions
        const int r = c / IN_ROW, col = (c % IN_ROW) * 8;
        T kv[8], qv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[2 * e] = (T)__uint_as_float(R.k[i][e] << 16);
          kv[2 * e + 1] = (T)__uint_as_float(R.k[i][e] & 0xffff0000u);
          qv[2 * e] = (T)__uint_as_float(R.q[i][e] << 16);
          qv[2 * e + 1] = (T)__uint_as_float(R.q[i][e] & 0xffff0000u);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int pos = kpos<O>(col + 4 * hh);
          *reinterpret_cast<uint2 *>(sK + r * L::LDK + pos) = *reinterpret_cast<const uint2 *>(kv + 4 * hh);
          *reinterpret_cast<uint2 *>(sQ + r * L::LDK + pos) = *reinterpret_cast<const uint2 *>(qv + 4 * hh);
        }
        (void)sKt;  // K^T comes from transposing reads of K
      } else {
        // 4 fp32 of row r, d_k col..col+3 (unpermuted order)
        const int r = c / IN_ROW, col = (c % IN_ROW) * 4;
        *reinterpret_cast<u32x4 *>(sK + r * L::LDK + col) = R.k[i];
        *reinterpret_cast<u32x4 *>(sQ + r * L::LDK + col) = R.q[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) sKt[(col + e) * L::LDT + r] = __uint_as_float(R.k[i][e]);
      }
    }
    if constexpr (KDA) {
      constexpr int E = 16 / sizeof(T);
#pragma unroll
      for (int i = 0; i < NKT; ++i) {
        const int c = tid + i * NT;
        const int d = c / (kBT / E), col = (c % (kBT / E)) * E;
        *reinterpret_cast<u32x4 *>(sKt + d * L::LDT + col) = R.kt[i];
      }
    }
    {
      constexpr int E = 16 / sizeof(T);
      T *sTn = reinterpret_cast<T *>(buf + L::TN);
      T *sMm = reinterpret_cast<T *>(buf + L::MM);
#pragma unroll
      for (int i = 0; i < NTM; ++i) {
        const int c = tid + i * NT;
        const int r = c / (kBT / E), col = (c % (kBT / E)) * E;
        *reinterpret_cast<u32x4 *>(sTn + r * L::LDT + col) = R.tn[i];
        *reinterpret_cast<u32x4 *>(sMm + r * L::LDT + col) = R.mm[i];
      }
    }
    if (tid < NVEC) reinterpret_cast<u32x4 *>(buf + L::VEC)[tid] = R.vec;
#pragma unroll
    for (int i = 0; i < NVP; ++i)
      reinterpret_cast<u32x4 *>(buf + L::V)[tid + i * NT] = R.v[i];
  };

  // ---------------------------------------------------------- the state
  f32x4 hacc[NHT];
  const size_t sbase = ((size_t)n * H + h) * DK * DV;
#pragma unroll
  for (int t = 0; t < NHT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      hacc[t][e] = p.h0 ? p.h0[sbase + (size_t)(16 * t + lg * 4 + e) * DV + cw + lr] : 0.f;

  // ---------------------------------------------------------- one chunk
  auto compute = [&](const char *buf, int jj) {
    const int r0 = bos + (jj - j0) * kBT;
    const int C = min(kBT, eos - r0);
    const T *sK = reinterpret_cast<const T *>(buf + L::K);
    const T *sQ = reinterpret_cast<const T *>(buf + L::Q);
    const T *sKt = reinterpret_cast<const T *>(buf + L::KT);
    const T *sTn = reinterpret_cast<const T *>(buf + L::TN);
    const T *sMm = reinterpret_cast<const T *>(buf + L::MM);
    const float *sv = reinterpret_cast<const float *>(buf + L::VEC);
    const In *sV = reinterpret_cast<const In *>(buf + L::V);

    // K H and Q H, the state as B operand straight from its accumulators
    typename O::Frag hb[NKD];
#pragma unroll
    for (int s = 0; s < NKD; ++s) hb[s] = b_frag<O>(hacc, s);
    f32x4 yk[4], yq[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      yk[R] = zero4();
      yq[R] = zero4();
    }
#pragma unroll
    for (int s = 0; s < NKD; ++s)
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        yk[R] = O::mfma(a_frag<O>(sK, L::LDK, 16 * R, s, lane), hb[s], yk[R]);
        yq[R] = O::mfma(a_frag<O>(sQ, L::LDK, 16 * R, s, lane), hb[s], yq[R]);
      }
    // X = V - gamma (K H); V rows past the chunk's end were staged as zero
    f32x4 gam[4], x[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const int r4 = 16 * R + lg * 4;
      gam[R] = *reinterpret_cast<const f32x4 *>(sv + r4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[R][e] = O::load(sV + (r4 + e) * W + 16 * w + lr) - gam[R][e] * yk[R][e];
    }
    // U = beta X + Tn X
    typename O::Frag xb[NKR];
#pragma unroll
    for (int s = 0; s < NKR; ++s) xb[s] = b_frag<O>(x, s);
    f32x4 u[4], ub4[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const f32x4 bet = *reinterpret_cast<const f32x4 *>(sv + 128 + 16 * R + lg * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[R][e] = bet[e] * x[R][e];
#pragma unroll
      for (int s = 0; s < ksteps_lower<O>(R); ++s)
        u[R] = O::mfma(a_frag<O>(sTn, L::LDT, 16 * R, s, lane), xb[s], u[R]);
      if constexpr (!KDA) {
        const f32x4 fac = *reinterpret_cast<const f32x4 *>(sv + 64 + 16 * R + lg * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) ub4[R][e] = fac[e] * u[R][e];
      }
    }
    typename O::Frag ufr[NKR], ubf[NKR];
#pragma unroll
    for (int s = 0; s < NKR; ++s) {
      ufr[s] = b_frag<O>(u, s);
      if constexpr (KDA) ubf[s] = ufr[s];
      else ubf[s] = b_frag<O>(ub4, s);
    }
    // O = scale (gamma (Q H) + M U); rows past the chunk's end are dropped by
    // the range check of the per-tile output resource
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      f32x4 oa;
#pragma unroll
      for (int e = 0; e < 4; ++e) oa[e] = gam[R][e] * yq[R][e];
#pragma unroll
      for (int s = 0; s < ksteps_lower<O>(R); ++s)
        oa = O::mfma(a_frag<O>(sMm, L::LDT, 16 * R, s, lane), ufr[s], oa);
      const auto ro = buffer_rsrc(p.o + ((size_t)(r0 + 16 * R) * H + h) * DV, (C - 16 * R) * rs_o);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p.scale * oa[e]), ro, off_o[e], 0, 0);
    }
    // H <- decay H + Kbar^T Ubar
#pragma unroll
    for (int t = 0; t < NHT; ++t) {
      const f32x4 dec = *reinterpret_cast<const f32x4 *>(sv + 192 + 16 * t + lg * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[t][e] *= dec[e];
#pragma unroll
      for (int s = 0; s < NKR; ++s) {
        typename O::Frag a;
        if constexpr (L::HAS_KT) a = a_frag<O>(sKt, L::LDT, 16 * t, s, lane);
        else a = a_frag_tr(sK, L::LDK, 16 * t, s, lane);
        hacc[t] = O::mfma(a, ubf[s], hacc[t]);
      }
    }
  };

  // ---------------------------------------------------------- chunk loop
  Raw raw;
  stage_load(raw, j0);
  stage_store(smem, raw);
  __syncthreads();
  for (int jj = j0; jj < j1; ++jj) {
    const bool more = jj + 1 < j1;
    char *cur = smem + (NBUF == 2 ? ((jj - j0) & 1) * L::BYTES : 0);
    if (more) stage_load(raw, jj + 1);
    compute(cur, jj);
    // keep the next chunk's LDS stores (and so the wait on its loads) after
    // this chunk's arithmetic: hoisting them would put a full global-memory
    // latency in front of every chunk
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NBUF == 2) {
      if (more) stage_store(smem + (((jj - j0) & 1) ^ 1) * L::BYTES, raw);
      __syncthreads();
    } else {
      __syncthreads();
      if (more) stage_store(smem, raw);
      __syncthreads();
    }
  }

  // ---- final state slice
  if (p.ht) {
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.ht[sbase + (size_t)(16 * t + lg * 4 + e) * DV + cw + lr] = hacc[t][e];
  }
}

}  // namespace

template <bool KDA, typename In, int DK, int NW>
static hipError_t launch_reduce_t(const ReduceParams &p, hipStream_t st) {
  const int units = p.N_max * p.H;
  const int grid = ((units + 7) / 8) * 8 * p.S;
  hipLaunchKernelGGL((chunk_reduce_kernel<KDA, In, DK, NW>), dim3(grid), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

template <bool KDA, typename In, int DK>
static hipError_t launch_reduce_w(const ReduceParams &p, int W, hipStream_t st) {
  switch (W) {
    case 32: return launch_reduce_t<KDA, In, DK, 2>(p, st);
    case 64: return launch_reduce_t<KDA, In, DK, 4>(p, st);
    case 128:
      if constexpr (DK >= 128) return launch_reduce_t<KDA, In, DK, 8>(p, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chunk_reduce(const ReduceParams &p, bool kda, bool bf16_in, int dk, int W,
                               hipStream_t st) {
  if (bf16_in) {
    if (dk == 128)
      return kda ? launch_reduce_w<true, bf16, 128>(p, W, st) : launch_reduce_w<false, bf16, 128>(p, W, st);
    return kda ? launch_reduce_w<true, bf16, 64>(p, W, st) : launch_reduce_w<false, bf16, 64>(p, W, st);
  }
  if (dk != 64) return hipErrorInvalidValue;
  return kda ? launch_reduce_w<true, float, 64>(p, W, st) : launch_reduce_w<false, float, 64>(p, W, st);
}

}  // namespace la
