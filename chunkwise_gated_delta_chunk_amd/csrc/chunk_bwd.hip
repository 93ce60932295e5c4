// GDN chunk backward: gradients of L = <o, do> + <ht, dht> for q, k, v, the
// log-decay g, beta and the initial state (the backward half of the FLA
// graph-capture RFC's scope, sections "Scope" and "Step 3"), chunk by chunk
// in the chunkwise form of "Empowering Hybrid Attention Models on NPUs"
// (section 2.1).  Per chunk of C rows, with G the chunk-local cumulative
// gate, gam_r = exp(G_r), fac_r = exp(G_{C-1} - G_r), gam_C = exp(G_{C-1}),
// E_rs = exp(G_r - G_s), S = strict_lower(K K^T * E), A = I + diag(beta) S,
// T = A^-1 diag(beta) and M = lower_incl(Q K^T * E), the forward is
//   X = V - gam*(K H),  U = T X,  O = scale (gam*(Q H) + M U),
//   H' = gam_C H + K^T (fac*U)
// and its adjoint, given dO (dOb = scale dO) and dH' (the gradient of the
// state leaving the chunk):
//   dU = M^T dOb + fac*(K dH'),   dX = T^T dU,   dV = dX
//   dH = gam_C dH' + Q^T (gam*dOb) - K^T (gam*dX)          (state entering)
//   dQ = gam*(dOb H^T) + (dM*E) K,      dM = dOb U^T
//   dK = -gam*(dX H^T) + fac*(U dH'^T) + (dM*E)^T Q + F K + F^T K
//   dT = dU X^T -> dA^-1 = dT diag(beta), dA = -A^-T dA^-1 A^-T,
//   dbeta_s += sum_r dT_rs A^-1_rs,  dbeta_r += sum_s dA_rs S_rs,
//   F = beta_r dA_rs E_rs (strict lower), and the gate terms below,
// with dg the reverse cumulative sum of dG inside the chunk.
//
// Four launches after the forward recompute (map + reduce storing every
// chunk's entering state H): prep (per chunk slot and head: A^-1, M, S and the
// gate vectors, fp32; A^-1 by 16x16 blocks), dh (per sequence, head and 32 state columns, chunks in
// reverse: the dH recurrence, storing dH' of every chunk and dh0), part (per
// slot and head: dV and the d_v-contracted products dOb H^T, dX H^T,
// U dH'^T, dM, dT and <dH', H>) and final (per slot and head: the chunk-local
// algebra to dq, dk, dg, dbeta).  Arithmetic is fp32 on 16x16x4 MFMA.
#include "bwd_common.h"

namespace la {

namespace {

using namespace bwd;

// ------------------------------------------------------------------ prep
template <typename In, int DK>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int LK = DK + 4;
  __shared__ __attribute__((aligned(16))) float sK[kBT * LK], sQ[kBT * LK], sS[64 * kL], sX[64 * kL];
  __shared__ __attribute__((aligned(16))) float sG[64], sB[64];
  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  Chunk ch;
  if (!chunk_of(p, slot, ch)) return;
  const int C = ch.C;
  load_rows<In, DK>(sK, LK, p.k, ch.r0, C, p.Hqk, h / (H / p.Hqk));
  load_rows<In, DK>(sQ, LK, p.q, ch.r0, C, p.Hqk, h / (H / p.Hqk));
  const int tid = threadIdx.x;
  if (tid < 64) {
    const float gr = tid < C ? p.g[(size_t)(ch.r0 + tid) * H + h] : 0.f;
    sG[tid] = wave_inclusive_scan(gr);  // rows >= C repeat G_{C-1}
    sB[tid] = tid < C ? p.beta[(size_t)(ch.r0 + tid) * H + h] : 0.f;
  }
  __syncthreads();
  float *img = p.prep + (size_t)blockIdx.x * kPrepFloats;
  const int w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  // S = strict_lower(K K^T * E), M = lower_incl(Q K^T * E): wave w, rows 16w
  f32x4 aS[4] = {zero4(), zero4(), zero4(), zero4()};
  f32x4 aM[4] = {zero4(), zero4(), zero4(), zero4()};
  mmN<4, DK>(aS, sK + 16 * w * LK, LK, 1, sK, 1, LK, 16 * LK);
  mmN<4, DK>(aM, sQ + 16 * w * LK, LK, 1, sK, 1, LK, 16 * LK);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const f32x4 as = aS[s4], am = aM[s4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * lg + i, s = 16 * s4 + lr;
      const float e = (r < C && s <= r) ? __expf(sG[r] - sG[s]) : 0.f;
      const float Sv = s < r ? as[i] * e : 0.f;
      const float Mv = am[i] * e;
      sS[r * kL + s] = Sv;
      img[kPrepS + r * 64 + s] = Sv;
      img[kPrepM + r * 64 + s] = Mv;
    }
  }
  __syncthreads();
  // A^-1 = (I + diag(beta) S)^-1, by 16x16 blocks
  unit_lower_inverse(sS, sB, sX, C);
  for (int idx = tid; idx < 64 * 64; idx += 256) img[kPrepA + idx] = sX[(idx >> 6) * kL + (idx & 63)];
  if (tid < 64) {
    const float Gc = sG[C - 1];
    img[kPrepG + tid] = sG[tid];
    img[kPrepGam + tid] = tid < C ? __expf(sG[tid]) : 0.f;
    img[kPrepFac + tid] = tid < C ? __expf(Gc - sG[tid]) : 0.f;
    img[kPrepBeta + tid] = sB[tid];
  }
}

// -------------------------------------------------------------------- dh
// per (sequence, head, 32 columns), chunks in reverse; the state gradient
// slice [d_k][32] lives in LDS
template <typename In, int DK>
__global__ __launch_bounds__(256) void bwd_dh_kernel(BwdParams p) {
  constexpr int LK = DK + 4, LC = 36, DV = DK;
  constexpr int SV = DV / 32;
  __shared__ __attribute__((aligned(16))) float sK[kBT * LK], sQ[kBT * LK], sA[64 * kL], sM[64 * kL];
  __shared__ __attribute__((aligned(16))) float sO[64 * LC], sGO[64 * LC], sU[64 * LC], sY[64 * LC], sD[DK * LC];
  __shared__ __attribute__((aligned(16))) float sGam[64], sFac[64], sBeta[64];
  const int H = p.H;
  const int sv = blockIdx.x % SV, unit = blockIdx.x / SV;
  if (unit >= p.N_max * H) return;
  const int n = seq_by_rank(p.chunk_offsets, p.N_max, unit / H), h = unit % H;
  if (n < 0) return;
  const int j0 = p.chunk_offsets[n], j1 = p.chunk_offsets[n + 1];
  if (j0 == j1) return;
  const int bos = cu_at(p.cu_seqlens, p.cu64, n), eos = cu_at(p.cu_seqlens, p.cu64, n + 1);
  const int c0 = sv * 32;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  const size_t mat = (size_t)DK * DV;
  const size_t sb = ((size_t)n * H + h) * mat;
  if (p.dht) {
    load_block<DK, 32>(sD, LC, p.dht + sb + c0, DV);
  } else {
    for (int idx = tid; idx < DK * 32; idx += 256) sD[(idx / 32) * LC + idx % 32] = 0.f;
  }
  for (int jj = j1 - 1; jj >= j0; --jj) {
    __syncthreads();
    const int r0 = bos + (jj - j0) * kBT, C = min(kBT, eos - r0);
    load_rows<In, DK>(sK, LK, p.k, r0, C, p.Hqk, h / (H / p.Hqk));
    load_rows<In, DK>(sQ, LK, p.q, r0, C, p.Hqk, h / (H / p.Hqk));
    const float *img = p.prep + ((size_t)jj * H + h) * kPrepFloats;
    load_mat64(sA, img + kPrepA);
    load_mat64(sM, img + kPrepM);
    if (tid < 64) {
      sGam[tid] = img[kPrepGam + tid];
      sFac[tid] = img[kPrepFac + tid];
      sBeta[tid] = img[kPrepBeta + tid];
    }
    load_rows<float, DV, 32>(sO, LC, p.dout, r0, C, H, h, c0);
    // the gradient leaving this chunk, for the part kernel
    float *dst = p.dhs + ((size_t)jj * H + h) * mat + c0;
#pragma unroll
    for (int it = 0; it < DK * 8 / 256; ++it) {
      const int pc = tid + 256 * it, i = pc / 8, c = (pc % 8) * 4;
      *reinterpret_cast<f32x4 *>(dst + (size_t)i * DV + c) =
          *reinterpret_cast<const f32x4 *>(sD + i * LC + c);
    }
    __syncthreads();
    for (int idx = tid; idx < 64 * 32; idx += 256) {
      const int r = idx / 32, c = idx % 32;
      const float v = p.scale * sO[r * LC + c];
      sO[r * LC + c] = v;
      sGO[r * LC + c] = sGam[r] * v;
    }
    __syncthreads();
    // dU = M^T dOb + fac * (K dH'), rows 16w
    {
      f32x4 kd[2] = {zero4(), zero4()}, du[2] = {zero4(), zero4()};
      mmN<2, DK>(kd, sK + 16 * w * LK, LK, 1, sD, LC, 1, 16);
      mmN<2, 64>(du, sM + 16 * w, 1, kL, sO, LC, 1, 16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + 4 * lg + i;
          sU[r * LC + 16 * nt + lr] = du[nt][i] + sFac[r] * kd[nt][i];
        }
    }
    __syncthreads();
    // dX = beta * (A^-T dU); Y = gam * dX
    {
      f32x4 dx[2] = {zero4(), zero4()};
      mmN<2, 64>(dx, sA + 16 * w, 1, kL, sU, LC, 1, 16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + 4 * lg + i;
          sY[r * LC + 16 * nt + lr] = sGam[r] * sBeta[r] * dx[nt][i];
        }
    }
    __syncthreads();
    // dH = gam_C dH' + Q^T (gam dOb) - K^T Y
    const float gamC = sGam[C - 1];
    for (int t = w; t < DK / 16; t += 4) {
      f32x4 acc[2], ky[2] = {zero4(), zero4()};
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nt][i] = gamC * sD[(16 * t + 4 * lg + i) * LC + 16 * nt + lr];
      mmN<2, 64>(acc, sQ + 16 * t, 1, LK, sGO, LC, 1, 16);
      mmN<2, 64>(ky, sK + 16 * t, 1, LK, sY, LC, 1, 16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sD[(16 * t + 4 * lg + i) * LC + 16 * nt + lr] = acc[nt][i] - ky[nt][i];
    }
  }
  __syncthreads();
  if (p.dh0)
    for (int idx = tid; idx < DK * 32; idx += 256) {
      const int i = idx / 32, c = idx % 32;
      p.dh0[sb + (size_t)i * DV + c0 + c] = sD[i * LC + c];
    }
}

// ------------------------------------------------------------------ part
// per (slot, head): dV and the d_v-contracted products, over 16-column blocks
template <typename In, int DK>
__global__ __launch_bounds__(256) void bwd_part_kernel(BwdParams p) {
  constexpr int LK = DK + 4, LB = 20, DV = DK, NT = DK / 16;
  __shared__ __attribute__((aligned(16))) float sK[kBT * LK], sA[64 * kL], sM[64 * kL];
  __shared__ __attribute__((aligned(16))) float sHD[2 * DK * LB];  // H block, then dH' block
  float *sH = sHD, *sDH = sHD + DK * LB;
  __shared__ __attribute__((aligned(16))) float sV[64 * LB], sO[64 * LB], sX[64 * LB], sBX[64 * LB], sU[64 * LB],
      sDU[64 * LB], sDX[64 * LB];
  __shared__ __attribute__((aligned(16))) float sGam[64], sFac[64], sBeta[64], sRed[256];
  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  Chunk ch;
  if (!chunk_of(p, slot, ch)) return;
  const int C = ch.C, r0 = ch.r0;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  load_rows<In, DK>(sK, LK, p.k, r0, C, p.Hqk, h / (H / p.Hqk));
  const float *img = p.prep + (size_t)blockIdx.x * kPrepFloats;
  load_mat64(sA, img + kPrepA);
  load_mat64(sM, img + kPrepM);
  if (tid < 64) {
    sGam[tid] = img[kPrepGam + tid];
    sFac[tid] = img[kPrepFac + tid];
    sBeta[tid] = img[kPrepBeta + tid];
  }
  const size_t mat = (size_t)DK * DV;
  const float *Hs = p.hs + (size_t)blockIdx.x * mat;
  const float *Ds = p.dhs + (size_t)blockIdx.x * mat;
  f32x4 P1[NT], P2[NT], P3[NT], dM[4], dT[4];
#pragma unroll
  for (int t = 0; t < NT; ++t) P1[t] = P2[t] = P3[t] = zero4();
#pragma unroll
  for (int t = 0; t < 4; ++t) dM[t] = dT[t] = zero4();
  float shd = 0.f;
  for (int cb = 0; cb < DV / 16; ++cb) {
    __syncthreads();
    load_block<DK, 16>(sH, LB, Hs + 16 * cb, DV);
    load_block<DK, 16>(sDH, LB, Ds + 16 * cb, DV);
    load_rows<In, DV, 16>(sV, LB, p.v, r0, C, H, h, 16 * cb);
    load_rows<float, DV, 16>(sO, LB, p.dout, r0, C, H, h, 16 * cb);
    __syncthreads();
    for (int idx = tid; idx < DK * 16; idx += 256) {
      const int i = idx / 16, c = idx % 16;
      shd += sH[i * LB + c] * sDH[i * LB + c];
    }
    for (int idx = tid; idx < 64 * 16; idx += 256) sO[(idx / 16) * LB + idx % 16] *= p.scale;
    __syncthreads();
    {
      f32x4 khd[2] = {zero4(), zero4()};  // K H and K dH'
      mmN<2, DK>(khd, sK + 16 * w * LK, LK, 1, sHD, LB, 1, DK * LB);
      const f32x4 kh = khd[0], kd = khd[1];
      const f32x4 mo = mm2k<64>(sM + 16 * w, 1, kL, sO, LB, 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i;
        const float x = sV[r * LB + lr] - sGam[r] * kh[i];
        sX[r * LB + lr] = x;
        sBX[r * LB + lr] = sBeta[r] * x;
        sDU[r * LB + lr] = mo[i] + sFac[r] * kd[i];
      }
    }
    __syncthreads();
    {
      const f32x4 u = mm2k<64>(sA + 16 * w * kL, kL, 1, sBX, LB, 1);
      const f32x4 dx = mm2k<64>(sA + 16 * w, 1, kL, sDU, LB, 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i;
        sU[r * LB + lr] = u[i];
        const float d = sBeta[r] * dx[i];
        sDX[r * LB + lr] = d;
        if (r < C) p.dv[((size_t)(r0 + r) * H + h) * DV + 16 * cb + lr] = d;
      }
    }
    __syncthreads();
    mmN<NT, 16>(P1, sO + 16 * w * LB, LB, 1, sH, 1, LB, 16 * LB);
    mmN<NT, 16>(P2, sDX + 16 * w * LB, LB, 1, sH, 1, LB, 16 * LB);
    mmN<NT, 16>(P3, sU + 16 * w * LB, LB, 1, sDH, 1, LB, 16 * LB);
    mmN<4, 16>(dM, sO + 16 * w * LB, LB, 1, sU, 1, LB, 16 * LB);
    mmN<4, 16>(dT, sDU + 16 * w * LB, LB, 1, sX, 1, LB, 16 * LB);
  }
  float *gw = p.part + (size_t)blockIdx.x * part_floats(DK);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * lg + i, c = 16 * t + lr;
      gw[kPartP1 + r * DK + c] = P1[t][i];
      gw[part_p2(DK) + r * DK + c] = P2[t][i];
      gw[part_p3(DK) + r * DK + c] = P3[t][i];
    }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * lg + i, c = 16 * t + lr;
      gw[part_dm(DK) + r * 64 + c] = dM[t][i];
      gw[part_dt(DK) + r * 64 + c] = dT[t][i];
    }
  sRed[tid] = shd;
  __syncthreads();
  if (tid == 0) {
    float s = 0.f;
    for (int i = 0; i < 256; ++i) s += sRed[i];
    gw[part_sh(DK)] = s;
  }
}

// ----------------------------------------------------------------- final
template <typename In, int DK>
__global__ __launch_bounds__(256) void bwd_final_kernel(BwdParams p) {
  constexpr int LK = DK + 4, NT = DK / 16;
  // phase A: A^-1, M, S, dM, dT and a product scratch; phase B: K, Q over the
  // first four of them, dM*E and F kept
  constexpr int MAT = 64 * kL;
  constexpr int KQ = 2 * kBT * LK;
  static_assert(KQ <= 4 * MAT, "K and Q fit over the phase-A matrices");
  __shared__ __attribute__((aligned(16))) float smem[6 * MAT];
  __shared__ __attribute__((aligned(16))) float sG[64], sGam[64], sFac[64], sBeta[64];
  __shared__ __attribute__((aligned(16))) float zr[64], zc[64], yr[64], yc[64], bt[64], ba[64], dG[64], t3s[64];
  float *sA = smem, *sM = smem + MAT, *sS = smem + 2 * MAT, *sTmp = smem + 3 * MAT;
  float *sDM = smem + 4 * MAT, *sDT = smem + 5 * MAT;
  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  Chunk ch;
  if (!chunk_of(p, slot, ch)) return;
  const int C = ch.C, r0 = ch.r0;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  const float *img = p.prep + (size_t)blockIdx.x * kPrepFloats;
  const float *gw = p.part + (size_t)blockIdx.x * part_floats(DK);
  load_mat64(sA, img + kPrepA);
  load_mat64(sM, img + kPrepM);
  load_mat64(sS, img + kPrepS);
  load_mat64(sDM, gw + part_dm(DK));
  load_mat64(sDT, gw + part_dt(DK));
  if (tid < 64) {
    sG[tid] = img[kPrepG + tid];
    sGam[tid] = img[kPrepGam + tid];
    sFac[tid] = img[kPrepFac + tid];
    sBeta[tid] = img[kPrepBeta + tid];
  }
  __syncthreads();
  // Z = dM * M (gates), dT * A^-1 (beta), then dM <- dM * E, dT <- dA^-1
  for (int idx = tid; idx < 4096; idx += 256) {
    const int r = idx >> 6, s = idx & 63, o = r * kL + s;
    const bool lo = s <= r && r < C;
    const float dm = sDM[o], dt = sDT[o];
    sTmp[o] = lo ? dt * sA[o] : 0.f;
    sM[o] = lo ? dm * sM[o] : 0.f;
    sDM[o] = lo ? dm * __expf(sG[r] - sG[s]) : 0.f;
    sDT[o] = lo ? dt * sBeta[s] : 0.f;
  }
  __syncthreads();
  if (tid < 64) {
    float a = 0.f, b = 0.f, c = 0.f;
    for (int s = 0; s < 64; ++s) a += sM[tid * kL + s];
    for (int r = 0; r < 64; ++r) {
      b += sM[r * kL + tid];
      c += sTmp[r * kL + tid];
    }
    zr[tid] = a;
    zc[tid] = b;
    bt[tid] = c;
  }
  __syncthreads();
  // tmp = dA^-1 A^-T
  {
    f32x4 t[4] = {zero4(), zero4(), zero4(), zero4()};
    mmN<4, 64>(t, sDT + 16 * w * kL, kL, 1, sA, 1, kL, 16 * kL);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int i = 0; i < 4; ++i) sTmp[(16 * w + 4 * lg + i) * kL + 16 * s4 + lr] = t[s4][i];
  }
  __syncthreads();
  // dA = -A^-T tmp; strict lower part: W = dA S (beta), Y = beta dA S (gates),
  // F = beta dA E (keys)
  f32x4 tA[4] = {zero4(), zero4(), zero4(), zero4()};
  mmN<4, 64>(tA, sA + 16 * w, 1, kL, sTmp, kL, 1, 16);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const f32x4 t = tA[s4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * lg + i, s = 16 * s4 + lr, o = r * kL + s;
      const bool sl = s < r && r < C;
      const float dA = -t[i];
      const float Sv = sS[o];
      sM[o] = sl ? dA * Sv : 0.f;
      sS[o] = sl ? sBeta[r] * dA * Sv : 0.f;
      sDT[o] = sl ? sBeta[r] * dA * __expf(sG[r] - sG[s]) : 0.f;
    }
  }
  __syncthreads();
  if (tid < 64) {
    float a = 0.f, b = 0.f, c = 0.f;
    for (int s = 0; s < 64; ++s) {
      a += sM[tid * kL + s];
      b += sS[tid * kL + s];
    }
    for (int r = 0; r < 64; ++r) c += sS[r * kL + tid];
    ba[tid] = a;
    yr[tid] = b;
    yc[tid] = c;
  }
  __syncthreads();
  // phase B: K and Q over the first four matrices
  float *sK = smem, *sQ = smem + kBT * LK;
  load_rows<In, DK>(sK, LK, p.k, r0, C, p.Hqk, h / (H / p.Hqk));
  load_rows<In, DK>(sQ, LK, p.q, r0, C, p.Hqk, h / (H / p.Hqk));
  __syncthreads();
  const float *P1 = gw + kPartP1, *P2 = gw + part_p2(DK), *P3 = gw + part_p3(DK);
  // dQ = gam P1 + (dM E) K;  dK = -gam P2 + fac P3 + (dM E)^T Q + F K + F^T K,
  // and the gate dot products <q_r, P1_r>, <k_r, P2_r>, <k_r, P3_r> from the
  // same P reads: per lane over its columns, then over the 16 lanes of a row
  f32x4 dq[NT], dk[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) dq[t] = dk[t] = zero4();
  mmN<NT, 64>(dq, sDM + 16 * w * kL, kL, 1, sK, LK, 1, 16);
  mmN<NT, 64>(dk, sDM + 16 * w, 1, kL, sQ, LK, 1, 16);
  mmN<NT, 64>(dk, sDT + 16 * w * kL, kL, 1, sK, LK, 1, 16);
  mmN<NT, 64>(dk, sDT + 16 * w, 1, kL, sK, LK, 1, 16);
  float q1[4] = {0.f, 0.f, 0.f, 0.f}, k2[4] = {0.f, 0.f, 0.f, 0.f}, k3[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * lg + i, c = 16 * t + lr;
      const float p1 = P1[r * DK + c], p2 = P2[r * DK + c], p3 = P3[r * DK + c];
      q1[i] += sQ[r * LK + c] * p1;
      k2[i] += sK[r * LK + c] * p2;
      k3[i] += sK[r * LK + c] * p3;
      if (r < C) {
        const size_t o = ((size_t)(r0 + r) * H + h) * DK + c;
        p.dq[o] = sGam[r] * p1 + dq[t][i];
        p.dk[o] = -sGam[r] * p2 + sFac[r] * p3 + dk[t][i];
      }
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      q1[i] += __shfl_xor(q1[i], m, 64);
      k2[i] += __shfl_xor(k2[i], m, 64);
      k3[i] += __shfl_xor(k3[i], m, 64);
    }
  if (lr == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * lg + i;
      const float t3 = sFac[r] * k3[i];
      dG[r] = r < C ? sGam[r] * (q1[i] - k2[i]) - t3 + zr[r] - zc[r] + yr[r] - yc[r] : 0.f;
      t3s[r] = r < C ? t3 : 0.f;
    }
  __syncthreads();
  if (tid == 0) {
    float dGc = 0.f;
    for (int r = 0; r < C; ++r) dGc += t3s[r];
    dGc += sGam[C - 1] * gw[part_sh(DK)];
    dG[C - 1] += dGc;
    // dg_t = sum_{r >= t} dG_r
    float acc = 0.f;
    for (int r = C - 1; r >= 0; --r) {
      acc += dG[r];
      dG[r] = acc;
    }
  }
  __syncthreads();
  if (tid < C) {
    const size_t o = (size_t)(r0 + tid) * H + h;
    p.dg[o] = dG[tid];
    p.dbeta[o] = bt[tid] + ba[tid];
  }
}

template <typename In, int DK>
hipError_t launch_all(const BwdParams &p, hipStream_t st) {
  const int cells = p.NT * p.H;
  hipLaunchKernelGGL((bwd_prep_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((bwd_dh_kernel<In, DK>), dim3(p.N_max * p.H * (DK / 32)), dim3(256), 0, st, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((bwd_part_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((bwd_final_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_dk(const BwdParams &p, int dk, hipStream_t st) {
  if (dk == 128) return launch_all<In, 128>(p, st);
  if (dk == 64) return launch_all<In, 64>(p, st);
  return hipErrorInvalidValue;
}

// out [T][Hqk][d] = sum over the G = H / Hqk value heads of each group of
// full [T][H][d], four floats per thread, rows of real tokens only (none when
// the metadata marks cu_seqlens invalid)
__global__ __launch_bounds__(256) void group_sum_kernel(const float *full, float *out, int T_max,
                                                        int H, int Hqk, int d, const void *cu,
                                                        int cu64, int N_max, const int32_t *co) {
  const int total = co[N_max] > 0 ? cu_at(cu, cu64, N_max) : 0;
  const size_t q4 = (size_t)d / 4, n4 = (size_t)T_max * Hqk * q4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n4) return;
  const int t = (int)(idx / ((size_t)Hqk * q4));
  if (t >= total) return;
  const int hq = (int)(idx / q4 % Hqk), c = (int)(idx % q4) * 4;
  const int G = H / Hqk;
  f32x4 acc = zero4();
  for (int j = 0; j < G; ++j)
    acc += *reinterpret_cast<const f32x4 *>(full + ((size_t)t * H + hq * G + j) * d + c);
  *reinterpret_cast<f32x4 *>(out + ((size_t)t * Hqk + hq) * d + c) = acc;
}

}  // namespace

hipError_t launch_group_sum(const float *full, float *out, int T_max, int H, int Hqk, int d,
                            const void *cu, int cu64, int N_max, const int32_t *co,
                            hipStream_t st) {
  const size_t n4 = (size_t)T_max * Hqk * (d / 4);
  hipLaunchKernelGGL(group_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, full,
                     out, T_max, H, Hqk, d, cu, cu64, N_max, co);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd(const BwdParams &p, int dt, int dk, hipStream_t st) {
  if (dt == LA_BF16) return launch_dk<bf16>(p, dk, st);
  if (dt == LA_F16) return launch_dk<f16>(p, dk, st);
  if (dt == LA_F32) return dk == 64 ? launch_all<float, 64>(p, st) : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

}  // namespace la
