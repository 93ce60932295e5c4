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
// overwritten -- the chunk-first in-place order of the same paper (section 5).
// Columns of U, O and H depend only on the same columns of V and H, so d_v is
// split into slices with no cross-slice reduction (the column-wise split of
// section 4).
//
// KDA: the map stage has already folded the per-channel decay into the
// operands (K*exp(G), Q*exp(G), (K*exp(G_C - G))^T, exp(G_C)), so the row
// factors are 1 and the state decays by diag(exp(G_C)).
//
// Work split: each wave owns CT 16-column state tiles for all chunk rows, so
// the chain H -> K H -> X -> U -> H of its columns never leaves the wave, and
// every A-operand fragment read from LDS feeds CT MFMAs (CT = 1 by default:
// with two tiles the register pressure costs more than the saved LDS reads).  With
// the chained k order (see la_device.h) an accumulator tile is itself the B
// operand of the next product, so H, X and U stay in registers.  Only the
// shared, state-independent operands of a chunk are in LDS: the map stage's
// image of the chunk (K, Q, [K^T], Tn, M, row vectors) and the V slice.  Both
// are copied one chunk ahead by direct global-to-LDS loads (no registers, no
// LDS store instructions) into the other half of a double buffer: one
// barrier per chunk, and the copy of chunk j + 1 overlaps the arithmetic of
// chunk j.  V rows past the chunk's end read as zero through the buffer range
// check, and output rows past it are dropped the same way.
//
// Blocks are numbered so that the slices of one (sequence, head) land on the
// same XCD (workgroup IDs are dealt round-robin over the 8 XCDs) and share
// its L2 for the image reads.  Zero-length sequences and padding units exit
// before touching memory, so they write nothing.
#include "la_device.h"
#include "kernels.h"

namespace la {

namespace {

template <bool KDA, typename In, int DK, int NW, int CT>
__global__ __launch_bounds__(64 * NW) void chunk_reduce_kernel(ReduceParams p) {
  using O = Op<In>;
  constexpr int E = (int)sizeof(typename O::T);
  constexpr ImageLayout I = image_layout(KDA, E, DK);
  constexpr bool HAS_KT = KDA || O::KPL == 1;
  constexpr int PK = DK * E / 16, PT = kBT * E / 16;
  constexpr int W = 16 * CT * NW;            // state columns per workgroup (CT tiles per wave)
  constexpr int DV = DK;                     // d_v == d_k
  constexpr int NKD = ksteps<O>(DK);         // k-steps over d_k
  constexpr int NKR = ksteps<O>(kBT);        // k-steps over chunk rows
  constexpr int NHT = DK / 16;               // state row tiles
  constexpr int PV = W * (int)sizeof(In) / 16;   // 16-byte pieces per V row
  constexpr int V_BYTES = kBT * W * (int)sizeof(In);
  constexpr int STAGE = I.BYTES + V_BYTES;
  constexpr int NBUF = 2 * STAGE <= 160 * 1024 ? 2 : 1;
  constexpr int NIMG = I.BYTES / 1024, NVL = V_BYTES / 1024;
  constexpr int STORES = 4 * CT * 4;         // o stores per wave per chunk
  static_assert(I.BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "1 KiB staging pieces");
  static_assert(STORES < 64, "vmcnt range");

  __shared__ __attribute__((aligned(16))) char smem[NBUF * STAGE];

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
  const int lane = lane_id(), w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  const int cw = slice * W + 16 * CT * w;            // this wave's first state column
  const int rs_v = H * DV * (int)sizeof(In);         // token stride of v (bytes)
  const int rs_o = H * DV * 4;                       // token stride of o (bytes)
  const char *img_all = static_cast<const char *>(p.img);

  // ---------------------------------------------------------------- staging
  // V piece q of the LDS tile (row q / PV, stored piece q % PV) comes from the
  // global row's logical piece (stored ^ swizzle)
  auto v_voff = [&](int q) {
    const int row = q / PV, phys = q % PV;
    return row * rs_v + ((phys ^ swz<PV>(row)) << 4);
  };
  auto issue = [&](char *buf, int jj) {
    const int r0 = bos + (jj - j0) * kBT;
    const int C = min(kBT, eos - r0);
    const auto ri = buffer_rsrc(img_all + ((size_t)jj * H + h) * I.BYTES, I.BYTES);
    for (int q = w; q < NIMG; q += NW)
      copy16_to_lds(ri, buf + q * 1024, lane * 16, q * 1024);
    const auto rv = buffer_rsrc(static_cast<const In *>(p.v) + ((size_t)r0 * H + h) * DV + slice * W,
                                C * rs_v);
    for (int q = w; q < NVL; q += NW)
      copy16_to_lds(rv, buf + I.BYTES + q * 1024, v_voff(q * 64 + lane), 0);
  };

  // ---------------------------------------------------------- the state
  f32x4 hacc[CT][NHT];
  const size_t sbase = ((size_t)n * H + h) * DK * DV;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hacc[ct][t][e] =
            p.h0 ? p.h0[sbase + (size_t)(16 * t + lg * 4 + e) * DV + cw + 16 * ct + lr] : 0.f;

  int off_o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) off_o[e] = (lg * 4 + e) * rs_o + (cw + lr) * 4;

  // V values of rows 16R + 4 lg + e, column 16 CT w + 16 ct + lr of the block's tile
  auto load_v = [&](const char *tV, int R, int ct) {
    f32x4 v;
    if constexpr (sizeof(In) == 2) {
      // transposed read: lane i of a 16-lane group reads row 16R + 4 lg + i/4,
      // columns c0 + 4 (i % 4) .. +3, and receives column c0 + i of 4 rows
      const int row = 16 * R + 4 * lg + (lr >> 2);
      const int col = 16 * CT * w + 16 * ct + 4 * (lr & 3);
      const s16x4 raw = ds_read_tr16(tV + tile_off<PV>(row, col >> 3) + 2 * (col & 7));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __uint_as_float((uint32_t)(uint16_t)raw[e] << 16);
    } else {
      const int col = 16 * CT * w + 16 * ct + lr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * R + 4 * lg + e;
        v[e] = *reinterpret_cast<const float *>(tV + tile_off<PV>(row, col >> 2) + 4 * (col & 3));
      }
    }
    return v;
  };

  // ---------------------------------------------------------- one chunk
  // The next chunk's copy (into `next`, if not null) is issued after the last
  // LDS read that uses the transposing builtin (the V reads of X)
  auto compute = [&](const char *buf, int jj, char *next) {
    const int r0 = bos + (jj - j0) * kBT;
    const int C = min(kBT, eos - r0);
    const char *tK = buf + I.K;
    const char *tQ = buf + I.Q;
    const char *tKT = buf + I.KT;
    const char *tTN = buf + I.TN;
    const char *tMM = buf + I.MM;
    const float *sv = reinterpret_cast<const float *>(buf + I.VEC);
    const char *tV = buf + I.BYTES;

    // K H and Q H, the state as B operand straight from its accumulators
    typename O::Frag hb[CT][NKD];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NKD; ++s) hb[ct][s] = b_frag<O>(hacc[ct], s);
    f32x4 yk[CT][4], yq[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        yk[ct][R] = zero4();
        yq[ct][R] = zero4();
      }
#pragma unroll
    for (int s = 0; s < NKD; ++s)
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const auto ak = a_frag_img<O, PK>(tK, 16 * R, s, lane);
        const auto aq = a_frag_img<O, PK>(tQ, 16 * R, s, lane);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          yk[ct][R] = O::mfma(ak, hb[ct][s], yk[ct][R]);
          yq[ct][R] = O::mfma(aq, hb[ct][s], yq[ct][R]);
        }
      }
    // X = V - gamma (K H); V rows past the chunk's end were staged as zero
    f32x4 gam[4], x[CT][4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      gam[R] = *reinterpret_cast<const f32x4 *>(sv + 16 * R + lg * 4);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const f32x4 v = load_v(tV, R, ct);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[ct][R][e] = v[e] - gam[R][e] * yk[ct][R][e];
      }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (next) issue(next, jj + 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // U = beta X + Tn X
    typename O::Frag xb[CT][NKR];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NKR; ++s) xb[ct][s] = b_frag<O>(x[ct], s);
    f32x4 u[CT][4], ub[CT][4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      const f32x4 bet = *reinterpret_cast<const f32x4 *>(sv + 128 + 16 * R + lg * 4);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) u[ct][R][e] = bet[e] * x[ct][R][e];
#pragma unroll
      for (int s = 0; s < ksteps_lower<O>(R); ++s) {
        const auto at = a_frag_img<O, PT>(tTN, 16 * R, s, lane);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) u[ct][R] = O::mfma(at, xb[ct][s], u[ct][R]);
      }
      if constexpr (!KDA) {
        const f32x4 fac = *reinterpret_cast<const f32x4 *>(sv + 64 + 16 * R + lg * 4);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) ub[ct][R][e] = fac[e] * u[ct][R][e];
      }
    }
    typename O::Frag ufr[CT][NKR], ubf[CT][NKR];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int s = 0; s < NKR; ++s) {
        ufr[ct][s] = b_frag<O>(u[ct], s);
        if constexpr (KDA) ubf[ct][s] = ufr[ct][s];
        else ubf[ct][s] = b_frag<O>(ub[ct], s);
      }
    // O = scale (gamma (Q H) + M U); rows past the chunk's end are dropped by
    // the range check of the per-tile output resource
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      f32x4 oa[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) oa[ct][e] = gam[R][e] * yq[ct][R][e];
#pragma unroll
      for (int s = 0; s < ksteps_lower<O>(R); ++s) {
        const auto am = a_frag_img<O, PT>(tMM, 16 * R, s, lane);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) oa[ct] = O::mfma(am, ufr[ct][s], oa[ct]);
      }
      const auto ro = buffer_rsrc(p.o + ((size_t)(r0 + 16 * R) * H + h) * DV, (C - 16 * R) * rs_o);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p.scale * oa[ct][e]), ro,
                                                off_o[e] + 64 * ct, 0, 0);
    }
    // H <- decay H + Kbar^T Ubar
    if constexpr (HAS_KT) {
#pragma unroll
      for (int t = 0; t < NHT; ++t) {
        const f32x4 dec = *reinterpret_cast<const f32x4 *>(sv + 192 + 16 * t + lg * 4);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) hacc[ct][t][e] *= dec[e];
#pragma unroll
        for (int s = 0; s < NKR; ++s) {
          const auto a = a_frag_img<O, PT>(tKT, 16 * t, s, lane);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) hacc[ct][t] = O::mfma(a, ubf[ct][s], hacc[ct][t]);
        }
      }
    } else {
      // K^T straight from K by transposed reads (fp16 GDN, NKR = 2 k-steps):
      // tile t needs reads (s, half) = (0,lo) (0,hi) (1,lo) (1,hi); those of
      // tile t + 1 are issued before tile t's wait
      static_assert(NKR == 2, "two k-steps over the chunk rows");
      const int j = lr;
      const int roff = 4 * lg + (j >> 2);
      auto issue_t = [&](int t, s16x4 (&r)[4]) {
        const int piece = (t >> 1) * 4 + (j & 3);
        const int sub = 8 * (t & 1);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ds_read_tr16_async(r[q], tK + tile_off<PK>(32 * (q >> 1) + 16 * (q & 1) + roff, piece) + sub);
      };
      const float gdec = sv[192];
      s16x4 cur[4], nxt[4];
      issue_t(0, cur);
#pragma unroll
      for (int t = 0; t < NHT; ++t) {
        if (t + 1 < NHT) {
          issue_t(t + 1, nxt);
          wait_lds_tied<4>(cur[0], cur[1], cur[2], cur[3]);
        } else {
          wait_lds_tied<0>(cur[0], cur[1], cur[2], cur[3]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) hacc[ct][t][e] *= gdec;
#pragma unroll
        for (int s = 0; s < NKR; ++s) {
          const half8 a = join_half8(cur[2 * s], cur[2 * s + 1]);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) hacc[ct][t] = O::mfma(a, ubf[ct][s], hacc[ct][t]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
      }
    }
  };

  // ---------------------------------------------------------- chunk loop
  // Every vector memory operation of a wave inside the loop is one of its
  // staging loads or one of its STORES output stores per chunk, and they
  // complete in issue order: at the top of chunk jj the operations issued
  // after chunk jj's loads are the previous chunk's stores.
  issue(smem, j0);
  for (int jj = j0; jj < j1; ++jj) {
    char *cur = smem + (NBUF == 2 ? ((jj - j0) & 1) * STAGE : 0);
    if (NBUF == 2 && jj != j0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(STORES));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();  // every wave's copy of chunk jj has landed
    if constexpr (NBUF == 2) {
      // the copy of chunk jj + 1 is issued inside compute, before this chunk's
      // stores (see the count above)
      compute(cur, jj, jj + 1 < j1 ? smem + (((jj - j0) & 1) ^ 1) * STAGE : nullptr);
    } else {
      compute(cur, jj, nullptr);
      __syncthreads();  // every wave is done reading the buffer
      if (jj + 1 < j1) issue(smem, jj + 1);
    }
  }

  // ---- final state slice
  if (p.ht) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.ht[sbase + (size_t)(16 * t + lg * 4 + e) * DV + cw + 16 * ct + lr] = hacc[ct][t][e];
  }
}

}  // namespace

// 16-column state tiles per wave (1: four waves per 64 columns; 2: two)
#ifndef LA_REDUCE_CT
#define LA_REDUCE_CT 1
#endif

template <bool KDA, typename In, int DK, int NW>
static hipError_t launch_reduce_t(const ReduceParams &p, hipStream_t st) {
  constexpr int CT = LA_REDUCE_CT;
  const int units = p.N_max * p.H;
  const int grid = ((units + 7) / 8) * 8 * p.S;
  hipLaunchKernelGGL((chunk_reduce_kernel<KDA, In, DK, NW, CT>), dim3(grid), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

template <bool KDA, typename In, int DK>
static hipError_t launch_reduce_w(const ReduceParams &p, int W, hipStream_t st) {
  constexpr int CT = LA_REDUCE_CT;
  switch (W) {
    case 32: return launch_reduce_t<KDA, In, DK, 2 / CT>(p, st);
    case 64: return launch_reduce_t<KDA, In, DK, 4 / CT>(p, st);
    case 128:
      if constexpr (DK >= 128) return launch_reduce_t<KDA, In, DK, 8 / CT>(p, st);
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
