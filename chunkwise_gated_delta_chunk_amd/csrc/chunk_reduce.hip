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
// H, so d_v is split into S slices of W columns with no cross-slice reduction
// (the column-wise split of section 4).
//
// KDA: the gate is a vector over d_k; the decay is folded into the operands
// instead of row factors: K -> K * exp(G), Q -> Q * exp(G) and
// K^T -> (K * exp(G_C - G))^T, and H decays by diag(exp(G_C)).
//
// Blocks are numbered so that the S slices of one (sequence, head) land on the
// same XCD (workgroup IDs are dealt round-robin over the 8 XCDs) and share
// its L2 for the K, Q and map-stage reads.  Zero-length sequences and padding
// units exit before touching memory, so they write nothing.
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

template <bool KDA, typename In, int DK, int W>
__global__ __launch_bounds__(kThreads) void chunk_reduce_kernel(ReduceParams p) {
  using O = Op<In>;
  using T = typename O::T;
  constexpr int DV_ALL = DK;             // d_v == d_k
  constexpr int LDK = DK + O::PAD;       // [row][dk] stride
  constexpr int LDT = kBT + O::PAD;      // [x][row] stride
  constexpr int KSTEP = 4 * O::KPL;
  constexpr int NCT = W / 16;            // column tiles of the slice
  constexpr int NRT = DK / 64;           // d_k row tiles per wave
  static_assert(W % 16 == 0 && W <= DK, "slice width");

  __shared__ __attribute__((aligned(16))) T sK[kBT * LDK];   // K (KDA: K*exp(G))
  __shared__ __attribute__((aligned(16))) T sQ[kBT * LDK];   // Q (KDA: Q*exp(G))
  __shared__ __attribute__((aligned(16))) T sKt[DK * LDT];   // K^T (KDA: (K*exp(G_C-G))^T)
  __shared__ __attribute__((aligned(16))) T sHt[W * LDK];    // H^T slice, B operand
  __shared__ __attribute__((aligned(16))) T sXt[W * LDT];    // X^T
  __shared__ __attribute__((aligned(16))) T sUt[W * LDT];    // U^T
  __shared__ __attribute__((aligned(16))) T sUb[KDA ? 1 : W * LDT];  // (gamma_C/gamma U)^T
  __shared__ float sg[kBT], sb[kBT];
  __shared__ float sG[KDA ? kBT * DK : 1];                   // KDA cumulative gate

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
  const int c0 = slice * W;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const In *gq = static_cast<const In *>(p.q);
  const In *gk = static_cast<const In *>(p.k);
  const In *gv = static_cast<const In *>(p.v);
  const T *Tn_all = static_cast<const T *>(p.Tn_raw);
  const T *M_all = static_cast<const T *>(p.M_raw);

  // ---- initial state slice -> registers (accumulator layout)
  f32x4 hacc[NRT][NCT];
  const size_t sbase = ((size_t)n * H + h) * DK * DV_ALL;
#pragma unroll
  for (int t = 0; t < NRT; ++t)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dk = 16 * (w * NRT + t) + (lane >> 4) * 4 + e;
        const int col = c0 + 16 * ct + (lane & 15);
        hacc[t][ct][e] = p.h0 ? p.h0[sbase + (size_t)dk * DV_ALL + col] : 0.f;
      }

  auto write_Ht = [&]() {
#pragma unroll
    for (int t = 0; t < NRT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        T *dst = sHt + (16 * ct + (lane & 15)) * LDK + 16 * (w * NRT + t) + (lane >> 4) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = (T)hacc[t][ct][e];
      }
  };
  write_Ht();

  for (int jj = j0; jj < j1; ++jj) {
    const int r0 = bos + (jj - j0) * kBT;
    const int C = min(kBT, eos - r0);
    const T *Tn = Tn_all + ((size_t)jj * H + h) * (kBT * kBT);
    const T *Mm = M_all + ((size_t)jj * H + h) * (kBT * kBT);

    __syncthreads();  // previous chunk's readers of sK/sQ/sKt/sUt/sUb are done
    if (tid < kBT) {
      const bool ok = tid < C;
      sb[tid] = ok ? p.beta[(size_t)(r0 + tid) * H + h] : 0.f;
      if (!KDA) sg[tid] = ok ? p.g[(size_t)(r0 + tid) * H + h] : 0.f;
    }
    if constexpr (KDA) {
      // cumulative gate per channel: SEG segments of rows per channel, scanned
      // sequentially, then offset by the totals of earlier segments
      constexpr int SEG = kThreads / DK, RPS = kBT / SEG;
      const int c = tid % DK, sgi = tid / DK;
      float run = 0.f;
      for (int r = sgi * RPS; r < (sgi + 1) * RPS; ++r) {
        if (r < C) run += p.g[((size_t)(r0 + r) * H + h) * DK + c];
        sG[r * DK + c] = run;
      }
      __syncthreads();
      float off = 0.f;
      for (int s2 = 0; s2 < sgi; ++s2) off += sG[((s2 + 1) * RPS - 1) * DK + c];
      __syncthreads();
      if (sgi > 0)
        for (int r = sgi * RPS; r < (sgi + 1) * RPS; ++r) sG[r * DK + c] += off;
      __syncthreads();
    }
    // stage K, Q (row-major) and K^T; one 16-byte vector per (row, 8-col block)
    {
      constexpr int VEC = 16 / sizeof(In);
      constexpr int NB = DK / VEC;
      for (int idx = tid; idx < kBT * NB; idx += kThreads) {
        const int r = idx & 63, cb = (idx >> 6) * VEC;
        float kf[VEC], qf[VEC];
        if (r < C) {
          const size_t off = ((size_t)(r0 + r) * H + h) * DK + cb;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            kf[e] = O::load(gk + off + e);
            qf[e] = O::load(gq + off + e);
          }
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) kf[e] = qf[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float kd = kf[e], qd = qf[e], kb = kf[e];
          if constexpr (KDA) {
            const float Gr = sG[r * DK + cb + e];
            const float Gc = sG[(kBT - 1) * DK + cb + e];
            const float f = __expf(Gr);
            kd *= f;
            qd *= f;
            kb *= __expf(Gc - Gr);
          }
          sK[r * LDK + cb + e] = (T)kd;
          sQ[r * LDK + cb + e] = (T)qd;
          sKt[(cb + e) * LDT + r] = (T)kb;
        }
      }
    }
    __syncthreads();

    // row factors of this lane's 4 rows in tile w
    float gam[4], fac[4], bet[4];
    float gammaC = 1.f;
    if constexpr (!KDA) {
      const float G = wave_inclusive_scan(sg[lane]);
      const float GC = __shfl(G, kBT - 1, 64);
      gammaC = __expf(GC);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float Gr = __shfl(G, 16 * w + (lane >> 4) * 4 + e, 64);
        gam[e] = __expf(Gr);
        fac[e] = __expf(GC - Gr);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) gam[e] = fac[e] = 1.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) bet[e] = sb[16 * w + (lane >> 4) * 4 + e];

    // ---- K H and Q H for row tile w (shared state operand)
    f32x4 yk[NCT], yq[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) yk[ct] = yq[ct] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += KSTEP) {
      const auto ak = frag_lds<O>(sK, LDK, 16 * w, k0, lane);
      const auto aq = frag_lds<O>(sQ, LDK, 16 * w, k0, lane);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const auto bh = frag_lds<O>(sHt, LDK, 16 * ct, k0, lane);
        yk[ct] = O::mfma(ak, bh, yk[ct]);
        yq[ct] = O::mfma(aq, bh, yq[ct]);
      }
    }
    // ---- X = V - gamma * (K H); X^T -> LDS
    f32x4 x[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int col = c0 + 16 * ct + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + (lane >> 4) * 4 + e;
        const float vv = r < C ? O::load(gv + ((size_t)(r0 + r) * H + h) * DV_ALL + col) : 0.f;
        x[ct][e] = vv - gam[e] * yk[ct][e];
      }
      T *dst = sXt + (16 * ct + (lane & 15)) * LDT + 16 * w + (lane >> 4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = (T)x[ct][e];
    }
    __syncthreads();

    // ---- U = beta X + Tn X (Tn strictly lower: k < 16w + 16 suffices)
    f32x4 u[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) u[ct][e] = bet[e] * x[ct][e];
    for (int k0 = 0; k0 < 16 * w + 16; k0 += KSTEP) {
      const auto at = frag_glb<O>(Tn, kBT, 16 * w, k0, lane);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        u[ct] = O::mfma(at, frag_lds<O>(sXt, LDT, 16 * ct, k0, lane), u[ct]);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      T *du = sUt + (16 * ct + (lane & 15)) * LDT + 16 * w + (lane >> 4) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) du[e] = (T)u[ct][e];
      if constexpr (!KDA) {
        T *db = sUb + (16 * ct + (lane & 15)) * LDT + 16 * w + (lane >> 4) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) db[e] = (T)(fac[e] * u[ct][e]);
      }
    }
    __syncthreads();

    // ---- O = scale * (gamma (Q H) + M U), rows < C written
    {
      f32x4 oa[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) oa[ct][e] = gam[e] * yq[ct][e];
      for (int k0 = 0; k0 < 16 * w + 16; k0 += KSTEP) {
        const auto am = frag_glb<O>(Mm, kBT, 16 * w, k0, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          oa[ct] = O::mfma(am, frag_lds<O>(sUt, LDT, 16 * ct, k0, lane), oa[ct]);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int col = c0 + 16 * ct + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * w + (lane >> 4) * 4 + e;
          if (r < C) p.o[((size_t)(r0 + r) * H + h) * DV_ALL + col] = p.scale * oa[ct][e];
        }
      }
    }

    // ---- H <- decay H + K^T Ubar   (this wave's d_k row tiles)
    const T *ub = KDA ? sUt : sUb;
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      float dec[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (KDA) dec[e] = __expf(sG[(kBT - 1) * DK + 16 * (w * NRT + t) + (lane >> 4) * 4 + e]);
        else dec[e] = gammaC;
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[t][ct][e] *= dec[e];
#pragma unroll
      for (int k0 = 0; k0 < kBT; k0 += KSTEP) {
        const auto a = frag_lds<O>(sKt, LDT, 16 * (w * NRT + t), k0, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          hacc[t][ct] = O::mfma(a, frag_lds<O>(ub, LDT, 16 * ct, k0, lane), hacc[t][ct]);
      }
    }
    write_Ht();  // sHt is no longer read in this chunk (all K H / Q H done)
  }

  // ---- final state slice
  if (p.ht) {
#pragma unroll
    for (int t = 0; t < NRT; ++t)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dk = 16 * (w * NRT + t) + (lane >> 4) * 4 + e;
          const int col = c0 + 16 * ct + (lane & 15);
          p.ht[sbase + (size_t)dk * DV_ALL + col] = hacc[t][ct][e];
        }
  }
}

}  // namespace

template <bool KDA, typename In, int DK, int W>
static hipError_t launch_reduce_t(const ReduceParams &p, hipStream_t st) {
  const int units = p.N_max * p.H;
  const int grid = ((units + 7) / 8) * 8 * p.S;
  hipLaunchKernelGGL((chunk_reduce_kernel<KDA, In, DK, W>), dim3(grid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <bool KDA, typename In, int DK>
static hipError_t launch_reduce_w(const ReduceParams &p, int W, hipStream_t st) {
  switch (W) {
    case 16: return launch_reduce_t<KDA, In, DK, 16>(p, st);
    case 32: return launch_reduce_t<KDA, In, DK, 32>(p, st);
    case 64: return launch_reduce_t<KDA, In, DK, 64>(p, st);
    case 128:
      if constexpr (DK >= 128) return launch_reduce_t<KDA, In, DK, 128>(p, st);
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
