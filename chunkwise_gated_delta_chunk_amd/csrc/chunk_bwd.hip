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
// Launches after the forward recompute (map + reduce storing every chunk's
// entering state H): prep (per chunk slot and head: A^-1, M, S and the gate
// vectors, fp32; A^-1 by 16x16 blocks), dh (per sequence, head and 32 state
// columns, chunks in reverse: the dH recurrence, storing dH' of every chunk
// and dh0), then per slot and head the d_v-contracted products (dV, dOb H^T,
// dX H^T, U dH'^T, dM, dT, <dH', H>) and the chunk-local algebra to dq, dk,
// dg, dbeta.  fp16 and fp32 inputs run part and final as two kernels in fp32
// on 16x16x4 MFMA; bf16 inputs run dh and one fused part + final kernel on
// bf16 MFMA with operands split into bf16 high and low halves.
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

// The same for bf16 inputs: K and Q stay bf16 in LDS (exact) and S, M run
// on bf16 MFMA with fp32 accumulation, one product per k-step.  Persistent:
// a workgroup walks cells with a stride of the grid (two per CU), and the
// next cell's K, Q, g and beta rows are loaded into registers as soon as
// the current ones are staged, so their latency passes under this cell's
// products and inverse.
template <int DK>
__global__ __launch_bounds__(256, 2) void bwd_prep_bf16_kernel(BwdParams p) {
  constexpr int LDK = DK + 16, KP = 64 * DK / 8 / 256;
  __shared__ __attribute__((aligned(16))) __bf16 sK[64 * LDK], sQ[64 * LDK];
  __shared__ __attribute__((aligned(16))) float sS[64 * kL], sX[64 * kL];
  __shared__ __attribute__((aligned(16))) float sG[64], sB[64];
  const int H = p.H, ncell = p.NT * H;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  u32x4 kv[KP], qv[KP];
  float gv = 0.f, bv = 0.f;
  auto load = [&](int cell, const Chunk &c) {
    const int h = cell % H, hq = h / (H / p.Hqk);
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int pc = tid + 256 * it, r = pc / (DK / 8), cc = (pc % (DK / 8)) * 8;
      kv[it] = qv[it] = u32x4{0u, 0u, 0u, 0u};
      if (r < c.C) {
        const size_t off = ((size_t)(c.r0 + r) * p.Hqk + hq) * DK + cc;
        kv[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.k) + off);
        qv[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.q) + off);
      }
    }
    if (tid < 64) {
      gv = tid < c.C ? p.g[(size_t)(c.r0 + tid) * H + h] : 0.f;
      bv = tid < c.C ? p.beta[(size_t)(c.r0 + tid) * H + h] : 0.f;
    }
  };
  int cell = blockIdx.x;
  Chunk ch;
  // sentinel slots come last: the first one ends the walk
  if (cell >= ncell || !chunk_of(p, cell / H, ch)) return;
  load(cell, ch);
  for (;;) {
    const int h = cell % H, C = ch.C;
    zero_mat64(sX);  // the inverse's scratch
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int pc = tid + 256 * it, r = pc / (DK / 8), c = (pc % (DK / 8)) * 8;
      *reinterpret_cast<u32x4 *>(sK + r * LDK + c) = kv[it];
      *reinterpret_cast<u32x4 *>(sQ + r * LDK + c) = qv[it];
    }
    if (tid < 64) {
      sG[tid] = wave_inclusive_scan(gv);  // rows >= C repeat G_{C-1}
      sB[tid] = bv;
    }
    __syncthreads();
    const int next = cell + gridDim.x;
    Chunk nch;
    const bool more = next < ncell && chunk_of(p, next / H, nch);
    if (more) load(next, nch);
    float *img = p.prep + (size_t)cell * kPrepFloats;
    __bf16 *imh = reinterpret_cast<__bf16 *>(img + kPrepH);
    // S = strict_lower(K K^T * E), M = lower_incl(Q K^T * E): wave w, rows
    // 16w, formed transposed (operands swapped) so that lane (g, n) holds row
    // 16 w + n at the columns 16 s4 + 4 g .. +3: S goes to LDS and M's bf16
    // halves to the image in 16- and 8-byte pieces
    f32x4 aS[4] = {zero4(), zero4(), zero4(), zero4()};
    f32x4 aM[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const bf16x8_t ak = frag_row(sK, LDK, 16 * w + lr, 32 * s), aq = frag_row(sQ, LDK, 16 * w + lr, 32 * s);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const bf16x8_t b = frag_row(sK, LDK, 16 * s4 + lr, 32 * s);
        aS[s4] = mfma_bf(b, ak, aS[s4]);
        aM[s4] = mfma_bf(b, aq, aM[s4]);
      }
    }
    {
      const int r = 16 * w + lr;
      const float gr = sG[r];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int s0 = 16 * s4 + 4 * lg;
        const f32x4 gs = *reinterpret_cast<const f32x4 *>(sG + s0);
        f32x4 sv;
        bf16x4_t mh, ml;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = s0 + i;
          const float e = (r < C && s <= r) ? __expf(gr - gs[i]) : 0.f;
          sv[i] = s < r ? aS[s4][i] * e : 0.f;
          const float mv = aM[s4][i] * e;  // (no fp32 S, M: see the fused kernel)
          mh[i] = (__bf16)mv;
          ml[i] = (__bf16)(mv - (float)mh[i]);
        }
        *reinterpret_cast<f32x4 *>(sS + r * kL + s0) = sv;
        *reinterpret_cast<bf16x4_t *>(imh + r * 64 + s0) = mh;
        *reinterpret_cast<bf16x4_t *>(imh + 4096 + r * 64 + s0) = ml;
      }
    }
    __syncthreads();
    // A^-1 = (I + diag(beta) S)^-1, by 16x16 blocks; stored with its
    // A^-1 diag(beta) halves, four consecutive entries per thread
    unit_lower_inverse(sS, sB, sX, C, true);  // sX cleared at the start
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int idx = 4 * tid + 1024 * it, r = idx >> 6, c = idx & 63;
      const f32x4 a = *reinterpret_cast<const f32x4 *>(sX + r * kL + c);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(sB + c);
      bf16x4_t ah, al;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = a[e] * b[e];
        ah[e] = (__bf16)x;
        al[e] = (__bf16)(x - (float)ah[e]);
      }
      *reinterpret_cast<f32x4 *>(img + kPrepA + idx) = a;
      *reinterpret_cast<bf16x4_t *>(imh + 8192 + idx) = ah;
      *reinterpret_cast<bf16x4_t *>(imh + 12288 + idx) = al;
    }
    if (tid < 64) {
      const float Gc = sG[C - 1];
      img[kPrepG + tid] = sG[tid];
      img[kPrepGam + tid] = tid < C ? __expf(sG[tid]) : 0.f;
      img[kPrepFac + tid] = tid < C ? __expf(Gc - sG[tid]) : 0.f;
      img[kPrepBeta + tid] = sB[tid];
    }
    if (!more) break;
    __syncthreads();  // this cell's LDS reads are done before the next staging
    cell = next;
    ch = nch;
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

// ----------------------------------------------------------- dh, bf16 MFMA
// The reverse pass for bf16 inputs on v_mfma_f32_16x16x32_bf16.  K and Q are
// exact in bf16; every other operand is split x = hi + lo (hi = bf16(x), lo =
// bf16(x - hi), about 17 significant bits together, with fp32's exponent
// range, so the scale of dO does not matter).  A product with K or Q takes
// the other side's two halves (2 MFMAs); a product of two split operands
// takes hi*hi + hi*lo + lo*hi (3).
//
// Every LDS array is row-major.  An operand whose contraction index runs
// down the rows (K^T, Q^T, dH', dOb, dU, Y) is read with ds_read_b64_tr_b16,
// so nothing is scattered transposed into LDS.  The next chunk's inputs are
// fetched into registers while the current chunk computes; barriers are
// plain s_barrier after this wave's LDS operations, so those loads stay in
// flight across them.
template <int DK>
__global__ __launch_bounds__(512) void bwd_dh_bf16_kernel(BwdParams p) {
  constexpr int DV = DK, SV = DV / 32, LDK = DK + 16, LT = 72, LO = 48, LC = 36, NKS = DK / 32;
  constexpr int KP = 64 * DK / 8 / 512;  // 16-byte K (and Q) pieces per thread
  __shared__ __attribute__((aligned(16))) __bf16 sK[64 * LDK], sQ[64 * LDK];
  // M and A~ = A^-1 diag(beta), both halves; M^T and A~^T are read transposed
  __shared__ __attribute__((aligned(16))) __bf16 sMh[64 * LT], sMl[64 * LT], sAh[64 * LT],
      sAl[64 * LT];
  // dOb halves; Y's halves take their place once dU is formed
  __shared__ __attribute__((aligned(16))) __bf16 sOh[64 * LO], sOl[64 * LO];
  __shared__ __attribute__((aligned(16))) __bf16 sGOh[64 * LO], sGOl[64 * LO], sUh[64 * LO],
      sUl[64 * LO];
  __shared__ __attribute__((aligned(16))) __bf16 sDh[DK * LO], sDl[DK * LO];
  __shared__ __attribute__((aligned(16))) float sD[DK * LC];
  __shared__ __attribute__((aligned(16))) float sGam[64], sFac[64];
  __bf16 *const sYh = sOh, *const sYl = sOl;
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
  // the dU and dX tiles: rows 16rt, columns 16ct; the dH tiles: column
  // tile ht, row tiles (w >> 1) + 4k
  const int rt = w & 3, ct = w >> 2, ht = w & 1;
  const int Hqk = p.Hqk, hq = h / (H / Hqk);
  const size_t mat = (size_t)DK * DV;
  const size_t sb = ((size_t)n * H + h) * mat;

  // one chunk's inputs in registers
  u32x4 rk[KP], rq[KP], rimg[4];
  f32x4 rdo;
  float rgo, rvec = 0.f;
  auto fetch = [&](int jj) {
    const int r0 = bos + (jj - j0) * kBT, C = min(kBT, eos - r0);
    const float *img = p.prep + ((size_t)jj * H + h) * kPrepFloats;
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int pc = tid + 512 * it, r = pc / (DK / 8), c = (pc % (DK / 8)) * 8;
      const size_t off = ((size_t)(r0 + r) * Hqk + hq) * DK + c;
      rk[it] = rq[it] = u32x4{0u, 0u, 0u, 0u};
      if (r < C) {
        rk[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.k) + off);
        rq[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.q) + off);
      }
    }
    const u32x4 *imh = reinterpret_cast<const u32x4 *>(img + kPrepH);
#pragma unroll
    for (int it = 0; it < 4; ++it) rimg[it] = imh[tid + 512 * it];
    {
      const int r = tid / 8, c = (tid % 8) * 4;
      rdo = r < C ? *reinterpret_cast<const f32x4 *>(p.dout + ((size_t)(r0 + r) * H + h) * DV + c0 + c)
                  : zero4();
      rgo = img[kPrepGam + r];
    }
    if (tid < 128) rvec = img[kPrepGam + tid];  // gam, fac: consecutive in the image
  };
  static_assert(kPrepFac == kPrepGam + 64, "gate vectors");

  // the state gradient: fp32 [DK][32] and its halves
  for (int idx = tid; idx < DK * 32; idx += 512) {
    const int i = idx / 32, c = idx % 32;
    const float v = p.dht ? p.dht[sb + (size_t)i * DV + c0 + c] : 0.f;
    sD[i * LC + c] = v;
    splitb(v, sDh[i * LO + c], sDl[i * LO + c]);
  }
  fetch(j1 - 1);
  for (int jj = j1 - 1; jj >= j0; --jj) {
    sync_lds();
    const int r0 = bos + (jj - j0) * kBT, C = min(kBT, eos - r0);
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int pc = tid + 512 * it, r = pc / (DK / 8), c = (pc % (DK / 8)) * 8;
      *reinterpret_cast<u32x4 *>(sK + r * LDK + c) = rk[it];
      *reinterpret_cast<u32x4 *>(sQ + r * LDK + c) = rq[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int pc = tid + 512 * it, a = pc >> 9, r = (pc & 511) / 8, c = (pc % 8) * 8;
      __bf16 *dst = a == 0 ? sMh : a == 1 ? sMl : a == 2 ? sAh : sAl;
      *reinterpret_cast<u32x4 *>(dst + r * LT + c) = rimg[it];
    }
    {
      const int r = tid / 8, c = (tid % 8) * 4;
      bf16x4_t oh, ol, gh, gl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = p.scale * rdo[e];
        const float gv = rgo * v;
        oh[e] = (__bf16)v;
        ol[e] = (__bf16)(v - (float)oh[e]);
        gh[e] = (__bf16)gv;
        gl[e] = (__bf16)(gv - (float)gh[e]);
      }
      *reinterpret_cast<bf16x4_t *>(sOh + r * LO + c) = oh;
      *reinterpret_cast<bf16x4_t *>(sOl + r * LO + c) = ol;
      *reinterpret_cast<bf16x4_t *>(sGOh + r * LO + c) = gh;
      *reinterpret_cast<bf16x4_t *>(sGOl + r * LO + c) = gl;
    }
    if (tid < 64) sGam[tid] = rvec;
    else if (tid < 128) sFac[tid - 64] = rvec;
    // the gradient leaving this chunk, for the next kernel
    float *dst = p.dhs + ((size_t)jj * H + h) * mat + c0;
#pragma unroll
    for (int it = 0; it < DK * 8 / 512; ++it) {
      const int pc = tid + 512 * it, i = pc / 8, c = (pc % 8) * 4;
      *reinterpret_cast<f32x4 *>(dst + (size_t)i * DV + c) =
          *reinterpret_cast<const f32x4 *>(sD + i * LC + c);
    }
    if (jj > j0) fetch(jj - 1);
    sync_lds();
    // Every tile below is formed transposed (operands swapped): lane (g, n)
    // holds row 16 x + n of its tile at the columns 16 y + 4 g .. +3, so
    // results go to LDS in 16- and 8-byte pieces.
    const int ur = 16 * rt + lr, uo = ur * LO + 16 * ct + 4 * lg;
    // dU = M^T dOb + fac * (K dH'): one tile per wave
    {
      f32x4 kd = zero4(), du = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8_t a = frag_row(sK, LDK, 16 * rt + lr, 32 * s);
        kd = mfma_bf(frag_col(sDh, LO, 32 * s, 16 * ct), a, kd);
        kd = mfma_bf(frag_col(sDl, LO, 32 * s, 16 * ct), a, kd);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
        du = mfma3(frag_col(sOh, LO, 32 * s, 16 * ct), frag_col(sOl, LO, 32 * s, 16 * ct),
                   frag_col(sMh, LT, 32 * s, 16 * rt), frag_col(sMl, LT, 32 * s, 16 * rt), du);
      const float f = sFac[ur];
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] += f * kd[i];
      split4(sUh + uo, sUl + uo, du);
    }
    sync_lds();
    // dX = beta * (A^-T dU) = A~^T dU; Y = gam * dX (over dOb, read by now)
    {
      f32x4 dx = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s)
        dx = mfma3(frag_col(sUh, LO, 32 * s, 16 * ct), frag_col(sUl, LO, 32 * s, 16 * ct),
                   frag_col(sAh, LT, 32 * s, 16 * rt), frag_col(sAl, LT, 32 * s, 16 * rt), dx);
      const float gm = sGam[ur];
#pragma unroll
      for (int i = 0; i < 4; ++i) dx[i] *= gm;
      split4(sYh + uo, sYl + uo, dx);
    }
    sync_lds();
    // dH = gam_C dH' + Q^T (gam dOb) - K^T Y
    {
      const float gamC = sGam[C - 1];
      bf16x8_t bgh[2], bgl[2], byh[2], byl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bgh[s] = frag_col(sGOh, LO, 32 * s, 16 * ht);
        bgl[s] = frag_col(sGOl, LO, 32 * s, 16 * ht);
        byh[s] = frag_col(sYh, LO, 32 * s, 16 * ht);
        byl[s] = frag_col(sYl, LO, 32 * s, 16 * ht);
      }
#pragma unroll
      for (int tt = 0; tt < DK / 64; ++tt) {
        const int t = (w >> 1) + 4 * tt;
        const int row = 16 * t + lr, c0 = 16 * ht + 4 * lg;
        f32x4 acc = *reinterpret_cast<const f32x4 *>(sD + row * LC + c0), ky = zero4();
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= gamC;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8_t aq = frag_col(sQ, LDK, 32 * s, 16 * t);
          const bf16x8_t ak = frag_col(sK, LDK, 32 * s, 16 * t);
          acc = mfma_bf(bgh[s], aq, acc);
          acc = mfma_bf(bgl[s], aq, acc);
          ky = mfma_bf(byh[s], ak, ky);
          ky = mfma_bf(byl[s], ak, ky);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] -= ky[i];
        *reinterpret_cast<f32x4 *>(sD + row * LC + c0) = acc;
        split4(sDh + row * LO + c0, sDl + row * LO + c0, acc);
      }
    }
  }
  sync_lds();
  if (p.dh0)
    for (int idx = tid; idx < DK * 32; idx += 512) {
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

// ------------------------------------------------------ reductions
__device__ __forceinline__ float sum16(float x) {  // over the 16 lanes of a row group
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// ------------------------------------------------------- part + final, bf16
// One kernel per (slot, head) for bf16 inputs: the partial products of the
// part stage stay in registers and the chunk-local algebra of the final
// stage follows in the same block, so nothing of either goes through HBM.
// Phase 1 is the 32-column loop (X, dU, U, dX = dV, and P1 = dOb H^T,
// P2 = dX H^T, P3 = U dH'^T, dM = dOb U^T, dT = dU X^T accumulated); phase 2
// reuses the loop's LDS for A^-1, tmp = dT' A^-T, F^T and dM*E.  Wave w
// owns row tile w throughout, so the P tiles it accumulates are the dq/dk
// tiles it writes.
// Eight waves, two per SIMD, so that one wave's LDS and MFMA latencies hide
// behind the other's work (with 256 registers per wave and nothing spilled:
// a spill reload would wait for every load in flight).  Wave w takes row
// tile rt = w % 4 and column half hc = w / 4 of every per-wave product: the
// X / dU / U / dX tile of column half hc, the P1..P3 (and dq / dk) column
// tiles of half hc, and the dM, dT (Z, dA, tmp) column tiles 2 hc, 2 hc + 1.
// Row sums of the two halves meet in a [6][2][64] table; column sums stay
// per row tile.
template <int DK>
__global__ __launch_bounds__(512) void bwd_cell8_bf16_kernel(BwdParams p) {
  constexpr int DV = DK, LDK = DK + 16, LT = 72, NB = 32, LB = NB + 8, NBLK = DV / NB, NKS = DK / 32;
  constexpr int KP = 64 * DK / 8 / 512;  // 16-byte K (or Q) pieces per thread
  constexpr int HP = DK * NB / 4 / 512;  // float4 pieces of an H (or dH') block per thread
  constexpr int PT = DK / 16;            // column tiles of P1..P3, dq and dk
  constexpr int PW = PT / 2;             // ... per wave
  constexpr int MT = 64 * LT;            // one [64][LT] array
  static_assert(KP >= 1 && HP >= 1, "piece split");
  // pool: [K][phase 1: M, A~ halves | H, dH' halves | 64-row block arrays]
  //       [K][phase 2: A^-1 (then Q), tmp, dT'^T (then F^T), dM*E, halves]
  constexpr int P1SZ = 4 * MT + 4 * DK * LB + 11 * 64 * LB, P2SZ = 8 * MT;
  static_assert(P2SZ <= P1SZ && 64 * LDK <= 2 * MT, "phase-2 arrays fit");
  __shared__ __attribute__((aligned(16))) __bf16 pool[64 * LDK + P1SZ];
  __shared__ __attribute__((aligned(16))) float sGam[64], sFac[64], sG[64], sBeta[64];
  __shared__ __attribute__((aligned(16))) float rowp[6][2][64], colt[3][4][64], sh8[8];
  __bf16 *const sK = pool, *const ph = pool + 64 * LDK;
  __bf16 *const sMh = ph, *const sMl = ph + MT, *const sAh = ph + 2 * MT, *const sAl = ph + 3 * MT;
  __bf16 *const sHh = ph + 4 * MT, *const sHl = sHh + DK * LB, *const sDh = sHl + DK * LB,
                *const sDl = sDh + DK * LB;
  __bf16 *const b64 = sDl + DK * LB;  // the 64-row block arrays
  __bf16 *const sOh = b64, *const sOl = b64 + 64 * LB, *const sXh = b64 + 2 * 64 * LB,
                *const sXl = b64 + 3 * 64 * LB, *const sGh = b64 + 4 * 64 * LB, *const sGl = b64 + 5 * 64 * LB,
                *const sUh = b64 + 6 * 64 * LB, *const sUl = b64 + 7 * 64 * LB, *const sEh = b64 + 8 * 64 * LB,
                *const sEl = b64 + 9 * 64 * LB, *const sV = b64 + 10 * 64 * LB;
  __bf16 *const qA1h = ph, *const qA1l = ph + MT, *const qTh = ph + 2 * MT, *const qTl = ph + 3 * MT;
  __bf16 *const qFh = ph + 4 * MT, *const qFl = ph + 5 * MT, *const qEh = ph + 6 * MT, *const qEl = ph + 7 * MT;
  __bf16 *const sQ = ph;  // over A^-1 once it is read

  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  Chunk ch;
  if (!chunk_of(p, slot, ch)) return;
  const int C = ch.C, r0 = ch.r0;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  const int rt = w & 3, hc = w >> 2;  // row tile, column half
  const int Hqk = p.Hqk, hq = h / (H / Hqk);
  const float *img = p.prep + (size_t)blockIdx.x * kPrepFloats;
  const size_t mat = (size_t)DK * DV;
  const float *Hs = p.hs + (size_t)blockIdx.x * mat;
  const float *Ds = p.dhs + (size_t)blockIdx.x * mat;
  static_assert(kPrepFac == kPrepGam + 64, "gate vectors");

  // ---- the cell's K, M and A~ halves, gam and fac
  {
    u32x4 rk[KP], rimg[4];
    float rvec = 0.f;
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int pc = tid + 512 * it, r = pc / (DK / 8), c = (pc % (DK / 8)) * 8;
      rk[it] = u32x4{0u, 0u, 0u, 0u};
      if (r < C)
        rk[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.k) +
                                                   ((size_t)(r0 + r) * Hqk + hq) * DK + c);
    }
    const u32x4 *imh = reinterpret_cast<const u32x4 *>(img + kPrepH);
#pragma unroll
    for (int it = 0; it < 4; ++it) rimg[it] = imh[tid + 512 * it];
    if (tid < 128) rvec = img[kPrepGam + tid];
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int pc = tid + 512 * it, r = pc / (DK / 8), c = (pc % (DK / 8)) * 8;
      *reinterpret_cast<u32x4 *>(sK + r * LDK + c) = rk[it];
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = tid / 8, c = (tid % 8) * 8;  // array it, row r, 8 columns
      *reinterpret_cast<u32x4 *>(ph + it * MT + r * LT + c) = rimg[it];
    }
    if (tid < 64) sGam[tid] = rvec;
    else if (tid < 128) sFac[tid - 64] = rvec;
  }

  // ---- phase 1
  f32x4 rh[HP], rd[HP], ro;
  u32x4 rv = u32x4{0u, 0u, 0u, 0u};
  auto fetch = [&](int cb) {
    const int cc = NB * cb;
#pragma unroll
    for (int it = 0; it < HP; ++it) {
      const int pc = tid + 512 * it, i = pc / (NB / 4), c = (pc % (NB / 4)) * 4;
      rh[it] = *reinterpret_cast<const f32x4 *>(Hs + (size_t)i * DV + cc + c);
      rd[it] = *reinterpret_cast<const f32x4 *>(Ds + (size_t)i * DV + cc + c);
    }
    {
      const int r = tid / (NB / 4), c = (tid % (NB / 4)) * 4;
      ro = r < C ? *reinterpret_cast<const f32x4 *>(p.dout + ((size_t)(r0 + r) * H + h) * DV + cc + c)
                 : zero4();
    }
    if (tid < 64 * NB / 8) {
      const int r = tid / (NB / 8), c = (tid % (NB / 8)) * 8;
      rv = r < C ? *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.v) +
                                                     ((size_t)(r0 + r) * H + h) * DV + cc + c)
                 : u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x4 P1[PW], P2[PW], P3[PW], dM[2], dT[2];
#pragma unroll
  for (int t = 0; t < PW; ++t) P1[t] = P2[t] = P3[t] = zero4();
#pragma unroll
  for (int t = 0; t < 2; ++t) dM[t] = dT[t] = zero4();
  float shd = 0.f;
  fetch(0);
  for (int cb = 0; cb < NBLK; ++cb) {
    sync_lds();
#pragma unroll
    for (int it = 0; it < HP; ++it) {
      const int pc = tid + 512 * it, i = pc / (NB / 4), c = (pc % (NB / 4)) * 4;
      split4(sHh + i * LB + c, sHl + i * LB + c, rh[it]);
      split4(sDh + i * LB + c, sDl + i * LB + c, rd[it]);
#pragma unroll
      for (int e = 0; e < 4; ++e) shd += rh[it][e] * rd[it][e];
    }
    {
      const int r = tid / (NB / 4), c = (tid % (NB / 4)) * 4;
      split4(sOh + r * LB + c, sOl + r * LB + c, ro * p.scale);
    }
    if (tid < 64 * NB / 8) {
      const int r = tid / (NB / 8), c = (tid % (NB / 8)) * 8;
      *reinterpret_cast<u32x4 *>(sV + r * LB + c) = rv;
    }
    if (cb + 1 < NBLK) fetch(cb + 1);
    sync_lds();
    // Transposed products (operands swapped): lane (g, n) holds row
    // xr = 16 rt + n at the columns 16 hc + 4 g .. +3 of this block.
    const int xr = 16 * rt + lr, xo = xr * LB + 16 * hc + 4 * lg;
    // X = V - gam*(K H), dU = M^T dOb + fac*(K dH'): rows 16 rt, column half hc
    {
      f32x4 kh = zero4(), kd = zero4(), mo = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8_t a = frag_row(sK, LDK, xr, 32 * s);
        kh = mfma_bf(frag_col(sHh, LB, 32 * s, 16 * hc), a, kh);
        kh = mfma_bf(frag_col(sHl, LB, 32 * s, 16 * hc), a, kh);
        kd = mfma_bf(frag_col(sDh, LB, 32 * s, 16 * hc), a, kd);
        kd = mfma_bf(frag_col(sDl, LB, 32 * s, 16 * hc), a, kd);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
        mo = mfma3(frag_col(sOh, LB, 32 * s, 16 * hc), frag_col(sOl, LB, 32 * s, 16 * hc),
                   frag_col(sMh, LT, 32 * s, 16 * rt), frag_col(sMl, LT, 32 * s, 16 * rt), mo);
      const float gx = sGam[xr], fx = sFac[xr];
      const bf16x4_t v4 = *reinterpret_cast<const bf16x4_t *>(sV + xo);
      f32x4 x, y;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = (float)v4[i] - gx * kh[i];
        y[i] = mo[i] + fx * kd[i];
      }
      split4(sXh + xo, sXl + xo, x);
      split4(sGh + xo, sGl + xo, y);
    }
    sync_lds();
    // U = A~ X, dX = A~^T dU (= dV)
    {
      f32x4 u = zero4(), dx = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u = mfma3(frag_col(sXh, LB, 32 * s, 16 * hc), frag_col(sXl, LB, 32 * s, 16 * hc),
                  frag_row(sAh, LT, xr, 32 * s), frag_row(sAl, LT, xr, 32 * s), u);
        dx = mfma3(frag_col(sGh, LB, 32 * s, 16 * hc), frag_col(sGl, LB, 32 * s, 16 * hc),
                   frag_col(sAh, LT, 32 * s, 16 * rt), frag_col(sAl, LT, 32 * s, 16 * rt), dx);
      }
      split4(sUh + xo, sUl + xo, u);
      split4(sEh + xo, sEl + xo, dx);
      if (xr < C)
        *reinterpret_cast<f32x4 *>(p.dv + ((size_t)(r0 + xr) * H + h) * DV + NB * cb + 16 * hc + 4 * lg) = dx;
    }
    sync_lds();
    // contracted over this block's columns
    {
      const bf16x8_t oh = frag_row(sOh, LB, xr, 0), ol = frag_row(sOl, LB, xr, 0);
      const bf16x8_t eh = frag_row(sEh, LB, xr, 0), el = frag_row(sEl, LB, xr, 0);
      const bf16x8_t uh = frag_row(sUh, LB, xr, 0), ul = frag_row(sUl, LB, xr, 0);
      const bf16x8_t gh = frag_row(sGh, LB, xr, 0), gl = frag_row(sGl, LB, xr, 0);
#pragma unroll
      for (int tp = 0; tp < PW; ++tp) {
        const int br = 16 * (PW * hc + tp) + lr;
        const bf16x8_t hh = frag_row(sHh, LB, br, 0), hl = frag_row(sHl, LB, br, 0);
        // transposed: lane (g, n) holds row 16 rt + n at the columns
        // 16 t + 4 g .. +3, as the dq / dk stores want them
        P1[tp] = mfma3(hh, hl, oh, ol, P1[tp]);
        P2[tp] = mfma3(hh, hl, eh, el, P2[tp]);
        P3[tp] = mfma3(frag_row(sDh, LB, br, 0), frag_row(sDl, LB, br, 0), uh, ul, P3[tp]);
      }
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int br = 16 * (2 * hc + tq) + lr;
        dM[tq] = mfma3(oh, ol, frag_row(sUh, LB, br, 0), frag_row(sUl, LB, br, 0), dM[tq]);
        dT[tq] = mfma3(gh, gl, frag_row(sXh, LB, br, 0), frag_row(sXl, LB, br, 0), dT[tq]);
      }
    }
  }

  // ---- phase 2
  // M at this lane's dM tile positions from its halves, still in LDS
  float fa[8], fam[2][4], fmm[2][4], fvec = 0.f;
  u32x4 rq[KP];
#pragma unroll
  for (int tq = 0; tq < 2; ++tq)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (16 * rt + 4 * lg + i) * LT + 16 * (2 * hc + tq) + lr;
      fmm[tq][i] = (float)sMh[o] + (float)sMl[o];
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) fa[e] = img[kPrepA + tid + 512 * e];
#pragma unroll
  for (int tq = 0; tq < 2; ++tq)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fam[tq][i] = img[kPrepA + (16 * rt + 4 * lg + i) * 64 + 16 * (2 * hc + tq) + lr];
#pragma unroll
  for (int it = 0; it < KP; ++it) {
    const int pc = tid + 512 * it, r = pc / (DK / 8), c = (pc % (DK / 8)) * 8;
    rq[it] = u32x4{0u, 0u, 0u, 0u};
    if (r < C)
      rq[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.q) +
                                                 ((size_t)(r0 + r) * Hqk + hq) * DK + c);
  }
  if (tid < 64) fvec = img[kPrepG + tid];
  else if (tid < 128) fvec = img[kPrepBeta + tid - 64];
  shd = wave_sum(shd);
  if (l == 0) sh8[w] = shd;
  sync_lds();  // every phase-1 LDS read is done
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = (tid + 512 * e) >> 6;  // row; the column is the lane
    splitb(fa[e], qA1h[r * LT + l], qA1l[r * LT + l]);
  }
  if (tid < 64) sG[tid] = fvec;
  else if (tid < 128) sBeta[tid - 64] = fvec;
  sync_lds();
  // Z = dM * M (gates), dT * A^-1 (beta); dT' = dT diag(beta), dM * E, split,
  // over the lower triangle of real rows, both stored transposed
  {
    float zr[4] = {0.f, 0.f, 0.f, 0.f};
    const int q0 = 16 * rt + 4 * lg;
    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sG + q0);
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int s = 16 * (2 * hc + tq) + lr, o = s * LT + q0;
      const float bs = sBeta[s], gs = sG[s];
      float zc = 0.f, bt = 0.f;
      f32x4 fv, ev;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = q0 + i;
        const bool lo = s <= r && r < C;
        const float z = lo ? dM[tq][i] * fmm[tq][i] : 0.f;
        zr[i] += z;
        zc += z;
        bt += lo ? dT[tq][i] * fam[tq][i] : 0.f;
        fv[i] = lo ? dT[tq][i] * bs : 0.f;
        ev[i] = lo ? dM[tq][i] * __expf(g4[i] - gs) : 0.f;
      }
      split4(qFh + o, qFl + o, fv);
      split4(qEh + o, qEl + o, ev);
      zc += __shfl_xor(zc, 16, 64);
      zc += __shfl_xor(zc, 32, 64);
      bt += __shfl_xor(bt, 16, 64);
      bt += __shfl_xor(bt, 32, 64);
      if (lg == 0) {
        colt[0][rt][s] = bt;
        colt[1][rt][s] = zc;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = sum16(zr[i]);
      if (lr == 0) rowp[0][hc][q0 + i] = v;
    }
  }
  sync_lds();
  // tmp = dT' A^-T
  {
    f32x4 t2[2] = {zero4(), zero4()};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8_t ah = frag_col(qFh, LT, 32 * s, 16 * rt), al = frag_col(qFl, LT, 32 * s, 16 * rt);
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int t = 2 * hc + tq;
        t2[tq] = mfma3(ah, al, frag_row(qA1h, LT, 16 * t + lr, 32 * s), frag_row(qA1l, LT, 16 * t + lr, 32 * s),
                       t2[tq]);
      }
    }
#pragma unroll
    for (int tq = 0; tq < 2; ++tq)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (16 * rt + 4 * lg + i) * LT + 16 * (2 * hc + tq) + lr;
        splitb(t2[tq][i], qTh[o], qTl[o]);
      }
  }
  sync_lds();
  // dA = -A^-T tmp; strict lower part: W = dA S (beta), Y = beta dA S
  // (gates), F = beta dA E (keys), stored as F^T over dT'^T.  S = K K^T * E
  // is recomputed here: K is exact in bf16 and still in LDS.
  {
    f32x4 kk[2] = {zero4(), zero4()};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8_t a = frag_row(sK, LDK, 16 * rt + lr, 32 * s);
#pragma unroll
      for (int tq = 0; tq < 2; ++tq)
        kk[tq] = mfma_bf(a, frag_row(sK, LDK, 16 * (2 * hc + tq) + lr, 32 * s), kk[tq]);
    }
    f32x4 t3[2] = {zero4(), zero4()};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8_t ah = frag_col(qA1h, LT, 32 * s, 16 * rt), al = frag_col(qA1l, LT, 32 * s, 16 * rt);
#pragma unroll
      for (int tq = 0; tq < 2; ++tq) {
        const int t = 2 * hc + tq;
        t3[tq] = mfma3(ah, al, frag_col(qTh, LT, 32 * s, 16 * t), frag_col(qTl, LT, 32 * s, 16 * t), t3[tq]);
      }
    }
    float wr[4] = {0.f, 0.f, 0.f, 0.f}, yr[4] = {0.f, 0.f, 0.f, 0.f};
    const int q0 = 16 * rt + 4 * lg;
    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sG + q0);
    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(sBeta + q0);
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      const int s = 16 * (2 * hc + tq) + lr;
      const float gs = sG[s];
      float yc = 0.f;
      f32x4 fv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = q0 + i;
        const bool sl = s < r && r < C;
        const float dA = -t3[tq][i];
        const float ex = __expf(g4[i] - gs);
        const float Wv = sl ? dA * kk[tq][i] * ex : 0.f;
        const float Yv = b4[i] * Wv;
        fv[i] = sl ? b4[i] * dA * ex : 0.f;
        wr[i] += Wv;
        yr[i] += Yv;
        yc += Yv;
      }
      split4(qFh + s * LT + q0, qFl + s * LT + q0, fv);
      yc += __shfl_xor(yc, 16, 64);
      yc += __shfl_xor(yc, 32, 64);
      if (lg == 0) colt[2][rt][s] = yc;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = sum16(wr[i]), b = sum16(yr[i]);
      if (lr == 0) {
        rowp[1][hc][q0 + i] = a;
        rowp[2][hc][q0 + i] = b;
      }
    }
  }
  sync_lds();
  // Q over A^-1
#pragma unroll
  for (int it = 0; it < KP; ++it) {
    const int pc = tid + 512 * it, r = pc / (DK / 8), c = (pc % (DK / 8)) * 8;
    *reinterpret_cast<u32x4 *>(sQ + r * LDK + c) = rq[it];
  }
  sync_lds();
  // dQ = gam P1 + (dM E) K;  dK = -gam P2 + fac P3 + (dM E)^T Q + F K + F^T K,
  // and the gate dots <q_r, P1_r>, <k_r, P2_r>, <k_r, P3_r>, over this
  // wave's column half
  {
    bf16x8_t aE[2][2], aET[2][2], aF[2][2], aFT[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      aE[s][0] = frag_col(qEh, LT, 32 * s, 16 * rt);  // E is stored transposed
      aE[s][1] = frag_col(qEl, LT, 32 * s, 16 * rt);
      aET[s][0] = frag_row(qEh, LT, 16 * rt + lr, 32 * s);
      aET[s][1] = frag_row(qEl, LT, 16 * rt + lr, 32 * s);
      aF[s][0] = frag_col(qFh, LT, 32 * s, 16 * rt);  // F^T is stored
      aF[s][1] = frag_col(qFl, LT, 32 * s, 16 * rt);
      aFT[s][0] = frag_row(qFh, LT, 16 * rt + lr, 32 * s);
      aFT[s][1] = frag_row(qFl, LT, 16 * rt + lr, 32 * s);
    }
    const int rr = 16 * rt + lr;
    const float gr = sGam[rr], fr = sFac[rr];
    float q1 = 0.f, k2 = 0.f, k3 = 0.f;
#pragma unroll
    for (int tp = 0; tp < PW; ++tp) {
      const int t = PW * hc + tp;
      f32x4 dq = zero4(), dk = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8_t bk = frag_col(sK, LDK, 32 * s, 16 * t), bq = frag_col(sQ, LDK, 32 * s, 16 * t);
        dq = mfma_bf(bk, aE[s][0], dq);
        dq = mfma_bf(bk, aE[s][1], dq);
        dk = mfma_bf(bq, aET[s][0], dk);
        dk = mfma_bf(bq, aET[s][1], dk);
        dk = mfma_bf(bk, aF[s][0], dk);
        dk = mfma_bf(bk, aF[s][1], dk);
        dk = mfma_bf(bk, aFT[s][0], dk);
        dk = mfma_bf(bk, aFT[s][1], dk);
      }
      const int c0 = 16 * t + 4 * lg;
      const bf16x4_t q4 = *reinterpret_cast<const bf16x4_t *>(sQ + rr * LDK + c0);
      const bf16x4_t k4 = *reinterpret_cast<const bf16x4_t *>(sK + rr * LDK + c0);
      f32x4 oq, ok;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q1 += (float)q4[i] * P1[tp][i];
        k2 += (float)k4[i] * P2[tp][i];
        k3 += (float)k4[i] * P3[tp][i];
        oq[i] = gr * P1[tp][i] + dq[i];
        ok[i] = -gr * P2[tp][i] + fr * P3[tp][i] + dk[i];
      }
      if (rr < C) {
        const size_t o = ((size_t)(r0 + rr) * H + h) * DK + c0;
        *reinterpret_cast<f32x4 *>(p.dq + o) = oq;
        *reinterpret_cast<f32x4 *>(p.dk + o) = ok;
      }
    }
#pragma unroll
    for (int m = 16; m < 64; m <<= 1) {
      q1 += __shfl_xor(q1, m, 64);
      k2 += __shfl_xor(k2, m, 64);
      k3 += __shfl_xor(k3, m, 64);
    }
    if (lg == 0) {
      rowp[3][hc][rr] = q1;
      rowp[4][hc][rr] = k2;
      rowp[5][hc][rr] = k3;
    }
  }
  sync_lds();
  if (w == 0) {
    // dG_r = gam_r (<q_r,P1_r> - <k_r,P2_r>) - fac_r <k_r,P3_r> + row and
    // column sums of Z and Y; dG_{C-1} also takes sum_r fac_r <k_r, P3_r> and
    // gam_{C-1} <dH', H>; dg_t = sum_{r >= t} dG_r; dbeta = the two beta sums
    const int r = l;
    float rs[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) rs[k] = rowp[k][0][r] + rowp[k][1][r];
    float cl[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) cl[k] = colt[k][0][r] + colt[k][1][r] + colt[k][2][r] + colt[k][3][r];
    const float t3 = r < C ? sFac[r] * rs[5] : 0.f;
    const float dGr = r < C ? sGam[r] * (rs[3] - rs[4]) - t3 + rs[0] - cl[1] + rs[2] - cl[2] : 0.f;
    float shs = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) shs += sh8[k];
    const float extra = wave_sum(t3) + sGam[C - 1] * shs;
    const float x = dGr + (r == C - 1 ? extra : 0.f);
    const float incl = wave_inclusive_scan(x);
    const float suffix = __shfl(incl, 63, 64) - incl + x;
    if (r < C) {
      const size_t o = (size_t)(r0 + r) * H + h;
      p.dg[o] = suffix;
      p.dbeta[o] = cl[0] + rs[1];
    }
  }
}

// the persistent bf16 prep's grid: the workgroups the device holds at once
// (found once per device), capped by the cells
template <int DK>
int prep_grid(int cells) {
  static int slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return cells;
  int res = dev < 64 ? slots[dev] : 0;
  if (res == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, bwd_prep_bf16_kernel<DK>, 256, 0) != hipSuccess ||
        cus * per <= 0)
      return cells;
    res = cus * per;
    if (dev < 64) slots[dev] = res;
  }
  return cells < res ? cells : res;
}

template <typename In, int DK>
hipError_t launch_all(const BwdParams &p, int stage, hipStream_t st) {
  const int cells = p.NT * p.H;
  if (stage == 1) {  // prep: needs no forward recompute
    if constexpr (std::is_same_v<In, bf16>)
      hipLaunchKernelGGL((bwd_prep_bf16_kernel<DK>), dim3(prep_grid<DK>(cells)), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_prep_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  if (stage == 2) {  // the reverse pass: needs prep only
    if constexpr (std::is_same_v<In, bf16>)
      hipLaunchKernelGGL((bwd_dh_bf16_kernel<DK>), dim3(p.N_max * p.H * (DK / 32)), dim3(512), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dh_kernel<In, DK>), dim3(p.N_max * p.H * (DK / 32)), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  // the per-chunk stage: needs the recomputed states and the reverse pass
  if constexpr (std::is_same_v<In, bf16>) {
    hipLaunchKernelGGL((bwd_cell8_bf16_kernel<DK>), dim3(cells), dim3(512), 0, st, p);
  } else {
    hipLaunchKernelGGL((bwd_part_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((bwd_final_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

template <typename In>
hipError_t launch_dk(const BwdParams &p, int dk, int stage, hipStream_t st) {
  if (dk == 128) return launch_all<In, 128>(p, stage, st);
  if (dk == 64) return launch_all<In, 64>(p, stage, st);
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

hipError_t launch_chunk_bwd(const BwdParams &p, int dt, int dk, int stage, hipStream_t st) {
  if (dt == LA_BF16) return launch_dk<bf16>(p, dk, stage, st);
  if (dt == LA_F16) return launch_dk<f16>(p, dk, stage, st);
  if (dt == LA_F32) return dk == 64 ? launch_all<float, 64>(p, stage, st) : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

}  // namespace la
