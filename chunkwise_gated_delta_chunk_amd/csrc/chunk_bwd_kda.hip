// KDA chunk backward: as chunk_bwd.hip for GDN, with the gate a vector over
// the key channels.  Per chunk, with G [C][d_k] the chunk-local cumulative
// gate, gam = exp(G), Kt = K*gam, Qt = Q*gam, Kh = K*exp(G_C - G) (G_C the
// last row), E_rsi = exp(G_ri - G_si), S_rs = sum_i k_ri k_si E_rsi (s < r),
// M_rs = sum_i q_ri k_si E_rsi (s <= r), A = I + diag(beta) S, T = A^-1 diag(beta),
// the forward ("Empowering Hybrid Attention Models on NPUs", section 2.1, in
// the chunk form) is
//   X = V - Kt H,  U = T X,  O = scale (Qt H + M U),  H' = diag(exp(G_C)) H + Kh^T U
// and its adjoint, with dOb = scale dO and dH' the gradient leaving the chunk:
//   dU = M^T dOb + Kh dH',  dX = T^T dU = dV,
//   dH = diag(exp(G_C)) dH' + Qt^T dOb - Kt^T dX
//   P1 = dOb H^T, P2 = dX H^T, P3 = U dH'^T, dM = dOb U^T, dT = dU X^T
//   dS = beta_r dA_rs (strict lower), dA from dT as for GDN
//   F1_xi = sum_s dM_xs k_si E_xsi   F2_xi = sum_r dM_rx q_ri E_rxi
//   F3_xi = sum_s dS_xs k_si E_xsi   F4_xi = sum_r dS_rx k_ri E_rxi
//   dq = gam P1 + F1
//   dk = -gam P2 + exp(G_C - G) P3 + F2 + F3 + F4
//   dG = gam q P1 - gam k P2 - Kh P3 + q F1 - k F2 + k F3 - k F4,
//        plus, on the last row, sum_r Kh P3 and exp(G_C) <dH', H> per channel
// and dg the reverse cumulative sum of dG over the chunk's rows, per channel.
// S, M (prep) and the E-weighted sums (final) go by 16-row blocks: inside a
// diagonal block as direct loops (exp(G_r - G_s) <= 1 for s <= r); across
// blocks R > S' the decay factorises through the last row b of S',
// exp(G_r - G_s) = exp(G_r - G_b) exp(G_b - G_s), both factors at most one
// for a decay (g <= 0), and those tiles run on fp32 MFMA.  The reverse pass
// runs for bf16 inputs on bf16 MFMA with split operands (as for GDN), for
// fp16 and fp32 inputs on fp32 MFMA; prep, part and final on fp32 MFMA.
#include "bwd_common.h"

namespace la {

namespace {

using namespace bwd;

// rows r < C of a [T][H][D] input times exp(G_r) (FAC = 0) or exp(G_C - G_r)
// (FAC = 1), G from the prep cell ([64][D] fp32)
template <typename In, int D, int FAC>
__device__ __forceinline__ void load_decayed(float *dst, int ld, const void *src, const float *G,
                                             int r0, int C, int H, int h) {
  constexpr int VEC = 16 / (int)sizeof(In);
  constexpr int PR = D / VEC, NP = kBT * PR, IT = (NP + 255) / 256;
  uint32_t raw[IT][4];
  f32x4 gv[IT][VEC / 4], gc[IT][VEC / 4];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pc = threadIdx.x + 256 * it, r = pc / PR, c = (pc % PR) * VEC;
    const bool ok = pc < NP && r < C;
    const u32x4 v = ok ? *reinterpret_cast<const u32x4 *>(static_cast<const char *>(src) +
                                                          (((size_t)(r0 + r) * H + h) * D + c) *
                                                              sizeof(In))
                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) raw[it][e] = v[e];
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      gv[it][q] = ok ? *reinterpret_cast<const f32x4 *>(G + r * D + c + 4 * q) : zero4();
      gc[it][q] = (ok && FAC) ? *reinterpret_cast<const f32x4 *>(G + (C - 1) * D + c + 4 * q)
                              : zero4();
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int pc = threadIdx.x + 256 * it, r = pc / PR, c = (pc % PR) * VEC;
    if (pc < NP) {
      float f[VEC];
      unpack16<In>(raw[it], f);
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = f[4 * q + e] * __expf(FAC ? gc[it][q][e] - gv[it][q][e] : gv[it][q][e]);
        *reinterpret_cast<f32x4 *>(dst + r * ld + c + 4 * q) = o;
      }
    }
  }
}

// ------------------------------------------------------------------ prep
template <typename In, int DK>
__global__ __launch_bounds__(256) void kda_prep_kernel(BwdParams p) {
  constexpr int LK = DK + 4;
  __shared__ __attribute__((aligned(16))) float sK[kBT * LK], sQ[kBT * LK], sG[kBT * LK];
  __shared__ __attribute__((aligned(16))) float sS[64 * kL], sX[64 * kL];
  __shared__ __attribute__((aligned(16))) float sB[64];
  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  Chunk ch;
  if (!chunk_of(p, slot, ch)) return;
  const int C = ch.C, tid = threadIdx.x;
  load_rows<In, DK>(sK, LK, p.k, ch.r0, C, p.Hqk, h / (H / p.Hqk));
  load_rows<In, DK>(sQ, LK, p.q, ch.r0, C, p.Hqk, h / (H / p.Hqk));
  // raw gates [C][DK], then the per-channel cumulative sum down the rows
  load_rows<float, DK>(sG, LK, p.g, ch.r0, C, H, h);
  if (tid < 64) sB[tid] = tid < C ? p.beta[(size_t)(ch.r0 + tid) * H + h] : 0.f;
  __syncthreads();
  if (tid < DK) {
    float acc = 0.f;
    for (int r = 0; r < 64; ++r) {
      acc += sG[r * LK + tid];  // rows >= C hold 0: they repeat G_{C-1}
      sG[r * LK + tid] = acc;
    }
  }
  __syncthreads();
  float *img = p.prep + (size_t)blockIdx.x * kda_prep_floats(DK);
  // S and M by 16-row blocks, the decay inside the channel sum.  Within a
  // diagonal block, pair by pair (e^{G_r - G_s} <= 1 for s <= r).  A block
  // pair R > S' factorises through the last row b of S':
  // e^{G_r - G_s} = e^{G_r - G_b} e^{G_b - G_s}, both factors <= 1, so the
  // tile is a plain product of decayed rows on fp32 MFMA.
  __bf16 *imh = reinterpret_cast<__bf16 *>(img + kda_halves(DK));
  auto put = [&](int r, int s, float as, float am) {
    const float Sv = s < r ? as : 0.f;
    sS[r * kL + s] = Sv;
    img[kPrepS + r * 64 + s] = Sv;
    img[kPrepM + r * 64 + s] = am;
    if constexpr (std::is_same_v<In, bf16>) {
      const __bf16 mh = (__bf16)am;
      imh[r * 64 + s] = mh;
      imh[4096 + r * 64 + s] = (__bf16)(am - (float)mh);
    }
  };
  // zero everything above the diagonal blocks, four entries per item
  for (int it = tid; it < 64 * 16; it += 256) {
    const int r = it >> 4, c0 = (it & 15) * 4;
    if ((c0 >> 4) > (r >> 4)) {
      *reinterpret_cast<f32x4 *>(sS + r * kL + c0) = zero4();
      *reinterpret_cast<f32x4 *>(img + kPrepS + r * 64 + c0) = zero4();
      *reinterpret_cast<f32x4 *>(img + kPrepM + r * 64 + c0) = zero4();
      if constexpr (std::is_same_v<In, bf16>) {
        const bf16x4_t z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
        *reinterpret_cast<bf16x4_t *>(imh + r * 64 + c0) = z;
        *reinterpret_cast<bf16x4_t *>(imh + 4096 + r * 64 + c0) = z;
      }
    }
  }
  {
    const int w = tid >> 6, l = lane_id(), j = l & 15, g = l >> 4;
    // The diagonal block of wave w, factored through its first row b:
    // e^{G_r - G_s} = e^{G_r - G_b} e^{G_b - G_s}, the first factor <= 1 and
    // the second >= 1, exact in fp32 while G_b - G_s <= 60 in every channel
    // (G decreases down the rows, so the block's last row bounds it).
    // Otherwise the block is summed pair by pair.
    const int b = 16 * w, ra = b + j;  // this lane's A row and B column
    bool fits = true;
    for (int i = l; i < DK; i += 64) fits &= sG[b * LK + i] - sG[(b + 15) * LK + i] <= 60.f;
    if (__ballot(!fits) == 0) {
      f32x4 aS = zero4(), aM = zero4();
#pragma unroll 4
      for (int i0 = 0; i0 < DK; i0 += 4) {
        const int i = i0 + g;
        const float gb = sG[b * LK + i], gr = sG[ra * LK + i];
        const float kr = sK[ra * LK + i];
        const float bk = kr * __expf(gb - gr), er = __expf(gr - gb);
        aS = mfma4(kr * er, bk, aS);
        aM = mfma4(sQ[ra * LK + i] * er, bk, aM);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = b + 4 * g + ii, s = b + j;
        const bool ok = r < C && s <= r;
        put(r, s, ok ? aS[ii] : 0.f, ok ? aM[ii] : 0.f);
      }
    } else {
      for (int pr = l; pr < 256; pr += 64) {
        const int r = b + (pr >> 4), s = b + (pr & 15);
        float as = 0.f, am = 0.f;
        if (r < C && s <= r) {
#pragma unroll 8
          for (int i = 0; i < DK; ++i) {
            const float e = __expf(sG[r * LK + i] - sG[s * LK + i]) * sK[s * LK + i];
            as += sK[r * LK + i] * e;
            am += sQ[r * LK + i] * e;
          }
        }
        put(r, s, as, am);
      }
    }
  }
  {
    const int w = tid >> 6, l = lane_id(), j = l & 15, g = l >> 4;
    for (int t = w; t < 6; t += 4) {  // (R, S'): (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
      const int R = t < 1 ? 1 : t < 3 ? 2 : 3, Sb = t - R * (R - 1) / 2, b = 16 * Sb + 15;
      const int ra = 16 * R + j, sa = 16 * Sb + j;  // this lane's A row and B column
      f32x4 aS = zero4(), aM = zero4();
#pragma unroll 4
      for (int i0 = 0; i0 < DK; i0 += 4) {
        const int i = i0 + g;
        const float gb = sG[b * LK + i];
        const float er = __expf(sG[ra * LK + i] - gb), es = __expf(gb - sG[sa * LK + i]);
        const float bk = sK[sa * LK + i] * es;
        aS = mfma4(sK[ra * LK + i] * er, bk, aS);
        aM = mfma4(sQ[ra * LK + i] * er, bk, aM);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * R + 4 * g + ii, s = 16 * Sb + j;
        const bool ok = r < C;
        put(r, s, ok ? aS[ii] : 0.f, ok ? aM[ii] : 0.f);
      }
    }
  }
  __syncthreads();
  unit_lower_inverse(sS, sB, sX, C);
  for (int idx = tid; idx < 4096; idx += 256) {
    const float a = sX[(idx >> 6) * kL + (idx & 63)];
    img[kPrepA + idx] = a;
    if constexpr (std::is_same_v<In, bf16>) {
      const float at = a * sB[idx & 63];  // A^-1 diag(beta)
      const __bf16 ah = (__bf16)at;
      imh[8192 + idx] = ah;
      imh[12288 + idx] = (__bf16)(at - (float)ah);
    }
  }
  if (tid < 64) img[kKdaBeta + tid] = sB[tid];
  for (int idx = tid; idx < 64 * DK; idx += 256) img[kKdaG + idx] = sG[(idx / DK) * LK + idx % DK];
}

// -------------------------------------------------------------------- dh
// The next chunk's raw K and Q rows, gates, A^-1 and M images and dO slice
// are fetched into registers while the current chunk computes; the decays
// are applied as the rows go to LDS, and Kt waits in registers until the dH
// step needs it (in place of Kh), so no global read sits inside a chunk.
// Barriers are plain s_barrier after the wave's own LDS operations, so the
// fetch stays in flight across them.
template <typename In, int DK>
__global__ __launch_bounds__(256) void kda_dh_kernel(BwdParams p) {
  constexpr int LK = DK + 4, LC = 36, DV = DK, SV = DV / 32;
  constexpr int VEC = 16 / (int)sizeof(In), PR = DK / VEC, IT = 64 * PR / 256;
  static_assert(256 % PR == 0 && (64 * PR) % 256 == 0, "piece layout");
  __shared__ __attribute__((aligned(16))) float sK[kBT * LK], sQ[kBT * LK], sA[64 * kL],
      sM[64 * kL];
  __shared__ __attribute__((aligned(16))) float sO[64 * LC], sU[64 * LC], sY[64 * LC], sD[DK * LC];
  __shared__ __attribute__((aligned(16))) float sGC[DK], sBeta[64];
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
  const int Hqk = p.Hqk, hq = h / (H / Hqk);
  const size_t mat = (size_t)DK * DV;
  const size_t sb = ((size_t)n * H + h) * mat;
  const int pcol = (tid % PR) * VEC;  // this thread's column in every K/Q piece

  // one chunk's inputs in registers
  u32x4 rk[IT], rq[IT];
  f32x4 rg[IT][VEC / 4], rgc[VEC / 4], ra[4], rm[4], ro[2];
  float rbeta = 0.f, rgcv = 0.f;
  auto fetch = [&](int jj) {
    const int r0 = bos + (jj - j0) * kBT, C = min(kBT, eos - r0);
    const float *img = p.prep + ((size_t)jj * H + h) * kda_prep_floats(DK);
    const float *G = img + kKdaG;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (tid + 256 * it) / PR;
      rk[it] = rq[it] = u32x4{0u, 0u, 0u, 0u};
      if (r < C) {
        const size_t off = (((size_t)(r0 + r) * Hqk + hq) * DK + pcol) * sizeof(In);
        rk[it] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.k) + off);
        rq[it] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.q) + off);
      }
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q) rg[it][q] = *reinterpret_cast<const f32x4 *>(G + r * DK + pcol + 4 * q);
    }
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) rgc[q] = *reinterpret_cast<const f32x4 *>(G + (C - 1) * DK + pcol + 4 * q);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q;
      ra[q] = *reinterpret_cast<const f32x4 *>(img + kPrepA + 4 * idx);
      rm[q] = *reinterpret_cast<const f32x4 *>(img + kPrepM + 4 * idx);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int pc = tid + 256 * q, r = pc / 8, c = (pc % 8) * 4;
      ro[q] = r < C ? *reinterpret_cast<const f32x4 *>(p.dout + ((size_t)(r0 + r) * H + h) * DV + c0 + c)
                    : zero4();
    }
    if (tid < 64) rbeta = img[kKdaBeta + tid];
    if (tid < DK) rgcv = G[(C - 1) * DK + tid];
  };

  if (p.dht) {
    load_block<DK, 32>(sD, LC, p.dht + sb + c0, DV);
  } else {
    for (int idx = tid; idx < DK * 32; idx += 256) sD[(idx / 32) * LC + idx % 32] = 0.f;
  }
  fetch(j1 - 1);
  float kt[IT][VEC];
  for (int jj = j1 - 1; jj >= j0; --jj) {
    sync_lds();
    // Kh = K exp(G_C - G) and Qt = Q exp(G) to LDS; Kt = K exp(G) kept
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (tid + 256 * it) / PR;
      uint32_t kw[4], qw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw[e] = rk[it][e];
        qw[e] = rq[it][e];
      }
      float kf[VEC], qf[VEC];
      unpack16<In>(kw, kf);
      unpack16<In>(qw, qf);
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        f32x4 kh, qt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gv = rg[it][q][e], eg = __expf(gv);
          kh[e] = kf[4 * q + e] * __expf(rgc[q][e] - gv);
          qt[e] = qf[4 * q + e] * eg;
          kt[it][4 * q + e] = kf[4 * q + e] * eg;
        }
        *reinterpret_cast<f32x4 *>(sK + r * LK + pcol + 4 * q) = kh;
        *reinterpret_cast<f32x4 *>(sQ + r * LK + pcol + 4 * q) = qt;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, r = idx / 16, c = (idx % 16) * 4;
      *reinterpret_cast<f32x4 *>(sA + r * kL + c) = ra[q];
      *reinterpret_cast<f32x4 *>(sM + r * kL + c) = rm[q];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int pc = tid + 256 * q, r = pc / 8, c = (pc % 8) * 4;
      *reinterpret_cast<f32x4 *>(sO + r * LC + c) = ro[q] * p.scale;
    }
    if (tid < 64) sBeta[tid] = rbeta;
    if (tid < DK) sGC[tid] = __expf(rgcv);
    float *dst = p.dhs + ((size_t)jj * H + h) * mat + c0;
#pragma unroll
    for (int it = 0; it < DK * 8 / 256; ++it) {
      const int pc = tid + 256 * it, i = pc / 8, c = (pc % 8) * 4;
      *reinterpret_cast<f32x4 *>(dst + (size_t)i * DV + c) =
          *reinterpret_cast<const f32x4 *>(sD + i * LC + c);
    }
    if (jj > j0) fetch(jj - 1);
    sync_lds();
    {  // dU = M^T dOb + Kh dH'
      f32x4 kd[2] = {zero4(), zero4()};
      mmN<2, DK>(kd, sK + 16 * w * LK, LK, 1, sD, LC, 1, 16);
      mmN<2, 64>(kd, sM + 16 * w, 1, kL, sO, LC, 1, 16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sU[(16 * w + 4 * lg + i) * LC + 16 * nt + lr] = kd[nt][i];
    }
    sync_lds();
    {  // dX = beta (A^-T dU)
      f32x4 dx[2] = {zero4(), zero4()};
      mmN<2, 64>(dx, sA + 16 * w, 1, kL, sU, LC, 1, 16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + 4 * lg + i;
          sY[r * LC + 16 * nt + lr] = sBeta[r] * dx[nt][i];
        }
    }
    sync_lds();
    // Kt over Kh
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = (tid + 256 * it) / PR;
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q)
        *reinterpret_cast<f32x4 *>(sK + r * LK + pcol + 4 * q) =
            f32x4{kt[it][4 * q], kt[it][4 * q + 1], kt[it][4 * q + 2], kt[it][4 * q + 3]};
    }
    sync_lds();
    // dH = exp(G_C) dH' + Qt^T dOb - Kt^T dX
    for (int t = w; t < DK / 16; t += 4) {
      f32x4 acc[2], ky[2] = {zero4(), zero4()};
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * t + 4 * lg + i;
          acc[nt][i] = sGC[row] * sD[row * LC + 16 * nt + lr];
        }
      mmN<2, 64>(acc, sQ + 16 * t, 1, LK, sO, LC, 1, 16);
      mmN<2, 64>(ky, sK + 16 * t, 1, LK, sY, LC, 1, 16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sD[(16 * t + 4 * lg + i) * LC + 16 * nt + lr] = acc[nt][i] - ky[nt][i];
    }
  }
  sync_lds();
  if (p.dh0)
    for (int idx = tid; idx < DK * 32; idx += 256) {
      const int i = idx / 32, c = idx % 32;
      p.dh0[sb + (size_t)i * DV + c0 + c] = sD[i * LC + c];
    }
}

// ---------------------------------------------------------- dh, bf16 MFMA
// The reverse pass for bf16 inputs on bf16 MFMA with split operands, as for
// GDN.  The decayed rows Kh = K exp(G_C - G), Kt = K exp(G), Qt = Q exp(G)
// are not exact in bf16, so they are split too (three MFMAs per product).
// Kh and the M, A~ halves occupy LDS for dU and dX; Kt and Qt wait in
// registers and take their places for the dH step.  The next chunk's raw
// rows, gates, image halves and dO slice are fetched into registers while
// the current chunk computes.
template <int DK>
__global__ __launch_bounds__(512) void kda_dh_bf16_kernel(BwdParams p) {
  constexpr int DV = DK, SV = DV / 32, LDK = DK + 16, LT = 72, LO = 48, LC = 36, NKS = DK / 32;
  constexpr int KP = 64 * DK / 8 / 512;  // 8-element K (and Q) pieces per thread
  constexpr int R1 = 2 * 64 * LDK, R2 = 4 * 64 * LT;
  static_assert(2 * 64 * LDK <= R2, "Qt halves fit over the M and A~ halves");
  __shared__ __attribute__((aligned(16))) __bf16 r1[R1], r2[R2];
  __shared__ __attribute__((aligned(16))) __bf16 sOh[64 * LO], sOl[64 * LO], sUh[64 * LO], sUl[64 * LO],
      sXh[64 * LO], sXl[64 * LO];
  __shared__ __attribute__((aligned(16))) __bf16 sDh[DK * LO], sDl[DK * LO];
  __shared__ __attribute__((aligned(16))) float sD[DK * LC], sGC[DK];
  __bf16 *const sKh = r1, *const sKl = r1 + 64 * LDK;          // Kh, then Kt
  __bf16 *const sMh = r2, *const sMl = r2 + 64 * LT, *const sAh = r2 + 2 * 64 * LT,
                *const sAl = r2 + 3 * 64 * LT;
  __bf16 *const sQh = r2, *const sQl = r2 + 64 * LDK;          // Qt, after dX
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
  const int pcol = (tid % (DK / 8)) * 8;  // this thread's column in every K/Q piece

  u32x4 rk[KP], rq[KP], rimg[4];
  f32x4 rg[KP][2], rgc[2], ro;
  float rgcv = 0.f;
  auto fetch = [&](int jj) {
    const int r0 = bos + (jj - j0) * kBT, C = min(kBT, eos - r0);
    const float *img = p.prep + ((size_t)jj * H + h) * kda_prep_floats(DK);
    const float *G = img + kKdaG;
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int r = (tid + 512 * it) / (DK / 8);
      rk[it] = rq[it] = u32x4{0u, 0u, 0u, 0u};
      if (r < C) {
        const size_t off = ((size_t)(r0 + r) * Hqk + hq) * DK + pcol;
        rk[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.k) + off);
        rq[it] = *reinterpret_cast<const u32x4 *>(static_cast<const bf16 *>(p.q) + off);
      }
      rg[it][0] = *reinterpret_cast<const f32x4 *>(G + r * DK + pcol);
      rg[it][1] = *reinterpret_cast<const f32x4 *>(G + r * DK + pcol + 4);
    }
    rgc[0] = *reinterpret_cast<const f32x4 *>(G + (C - 1) * DK + pcol);
    rgc[1] = *reinterpret_cast<const f32x4 *>(G + (C - 1) * DK + pcol + 4);
    const u32x4 *imh = reinterpret_cast<const u32x4 *>(img + kda_halves(DK));
#pragma unroll
    for (int it = 0; it < 4; ++it) rimg[it] = imh[tid + 512 * it];
    {
      const int r = tid / 8, c = (tid % 8) * 4;
      ro = r < C ? *reinterpret_cast<const f32x4 *>(p.dout + ((size_t)(r0 + r) * H + h) * DV + c0 + c)
                 : zero4();
    }
    if (tid < DK) rgcv = G[(C - 1) * DK + tid];
  };
  auto put4 = [](__bf16 *hi, __bf16 *lo, f32x4 v) {
    bf16x4_t a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = (__bf16)v[e];
      b[e] = (__bf16)(v[e] - (float)a[e]);
    }
    *reinterpret_cast<bf16x4_t *>(hi) = a;
    *reinterpret_cast<bf16x4_t *>(lo) = b;
  };

  for (int idx = tid; idx < DK * 32; idx += 512) {
    const int i = idx / 32, c = idx % 32;
    const float v = p.dht ? p.dht[sb + (size_t)i * DV + c0 + c] : 0.f;
    sD[i * LC + c] = v;
    splitb(v, sDh[i * LO + c], sDl[i * LO + c]);
  }
  fetch(j1 - 1);
  bf16x8_t kth[KP], ktl[KP], qth[KP], qtl[KP];  // Kt and Qt halves until the dH step
  for (int jj = j1 - 1; jj >= j0; --jj) {
    sync_lds();
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int r = (tid + 512 * it) / (DK / 8);
      uint32_t kw[4], qw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kw[e] = rk[it][e];
        qw[e] = rq[it][e];
      }
      float kf[8], qf[8];
      unpack16<bf16>(kw, kf);
      unpack16<bf16>(qw, qf);
      bf16x8_t khh, khl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = rg[it][e >> 2][e & 3], eg = __expf(gv);
        const float kh = kf[e] * __expf(rgc[e >> 2][e & 3] - gv), kt = kf[e] * eg, qt = qf[e] * eg;
        khh[e] = (__bf16)kh;
        khl[e] = (__bf16)(kh - (float)khh[e]);
        kth[it][e] = (__bf16)kt;
        ktl[it][e] = (__bf16)(kt - (float)kth[it][e]);
        qth[it][e] = (__bf16)qt;
        qtl[it][e] = (__bf16)(qt - (float)qth[it][e]);
      }
      *reinterpret_cast<bf16x8_t *>(sKh + r * LDK + pcol) = khh;
      *reinterpret_cast<bf16x8_t *>(sKl + r * LDK + pcol) = khl;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int pc = tid + 512 * it, a = pc >> 9, r = (pc & 511) / 8, c = (pc % 8) * 8;
      *reinterpret_cast<u32x4 *>(r2 + a * 64 * LT + r * LT + c) = rimg[it];
    }
    {
      const int r = tid / 8, c = (tid % 8) * 4;
      put4(sOh + r * LO + c, sOl + r * LO + c, ro * p.scale);
    }
    if (tid < DK) sGC[tid] = __expf(rgcv);
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
    const int uo = (16 * rt + lr) * LO + 16 * ct + 4 * lg;
    // dU = M^T dOb + Kh dH': one tile per wave
    {
      f32x4 du = zero4();
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        du = mfma3(frag_col(sDh, LO, 32 * s, 16 * ct), frag_col(sDl, LO, 32 * s, 16 * ct),
                   frag_row(sKh, LDK, 16 * rt + lr, 32 * s), frag_row(sKl, LDK, 16 * rt + lr, 32 * s), du);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        du = mfma3(frag_col(sOh, LO, 32 * s, 16 * ct), frag_col(sOl, LO, 32 * s, 16 * ct),
                   frag_col(sMh, LT, 32 * s, 16 * rt), frag_col(sMl, LT, 32 * s, 16 * rt), du);
      split4(sUh + uo, sUl + uo, du);
    }
    sync_lds();
    // dX = A~^T dU
    {
      f32x4 dx = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s)
        dx = mfma3(frag_col(sUh, LO, 32 * s, 16 * ct), frag_col(sUl, LO, 32 * s, 16 * ct),
                   frag_col(sAh, LT, 32 * s, 16 * rt), frag_col(sAl, LT, 32 * s, 16 * rt), dx);
      split4(sXh + uo, sXl + uo, dx);
    }
    sync_lds();
    // Kt over Kh, Qt over the M and A~ halves
#pragma unroll
    for (int it = 0; it < KP; ++it) {
      const int r = (tid + 512 * it) / (DK / 8);
      *reinterpret_cast<bf16x8_t *>(sKh + r * LDK + pcol) = kth[it];
      *reinterpret_cast<bf16x8_t *>(sKl + r * LDK + pcol) = ktl[it];
      *reinterpret_cast<bf16x8_t *>(sQh + r * LDK + pcol) = qth[it];
      *reinterpret_cast<bf16x8_t *>(sQl + r * LDK + pcol) = qtl[it];
    }
    sync_lds();
    // dH = exp(G_C) dH' + Qt^T dOb - Kt^T dX
    {
      bf16x8_t boh[2], bol[2], bxh[2], bxl[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        boh[s] = frag_col(sOh, LO, 32 * s, 16 * ht);
        bol[s] = frag_col(sOl, LO, 32 * s, 16 * ht);
        bxh[s] = frag_col(sXh, LO, 32 * s, 16 * ht);
        bxl[s] = frag_col(sXl, LO, 32 * s, 16 * ht);
      }
#pragma unroll
      for (int tt = 0; tt < DK / 64; ++tt) {
        const int t = (w >> 1) + 4 * tt;
        const int row = 16 * t + lr, c0 = 16 * ht + 4 * lg;
        f32x4 acc = *reinterpret_cast<const f32x4 *>(sD + row * LC + c0), ky = zero4();
        const float gc = sGC[row];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= gc;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          acc = mfma3(boh[s], bol[s], frag_col(sQh, LDK, 32 * s, 16 * t), frag_col(sQl, LDK, 32 * s, 16 * t), acc);
          ky = mfma3(bxh[s], bxl[s], frag_col(sKh, LDK, 32 * s, 16 * t), frag_col(sKl, LDK, 32 * s, 16 * t), ky);
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
template <typename In, int DK>
__global__ __launch_bounds__(256) void kda_part_kernel(BwdParams p) {
  constexpr int LK = DK + 4, LB = 20, DV = DK, NT = DK / 16;
  __shared__ __attribute__((aligned(16))) float sKt[kBT * LK], sKh[kBT * LK], sA[64 * kL],
      sM[64 * kL];
  __shared__ __attribute__((aligned(16))) float sHD[2 * DK * LB];
  __shared__ __attribute__((aligned(16))) float sV[64 * LB], sO[64 * LB], sX[64 * LB],
      sBX[64 * LB], sU[64 * LB], sDU[64 * LB], sDX[64 * LB];
  __shared__ __attribute__((aligned(16))) float sBeta[64];
  float *sH = sHD, *sDH = sHD + DK * LB;
  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  Chunk ch;
  if (!chunk_of(p, slot, ch)) return;
  const int C = ch.C, r0 = ch.r0;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  const float *img = p.prep + (size_t)blockIdx.x * kda_prep_floats(DK);
  load_decayed<In, DK, 0>(sKt, LK, p.k, img + kKdaG, r0, C, p.Hqk, h / (H / p.Hqk));
  load_decayed<In, DK, 1>(sKh, LK, p.k, img + kKdaG, r0, C, p.Hqk, h / (H / p.Hqk));
  load_mat64(sA, img + kPrepA);
  load_mat64(sM, img + kPrepM);
  if (tid < 64) sBeta[tid] = img[kKdaBeta + tid];
  const size_t mat = (size_t)DK * DV;
  const float *Hs = p.hs + (size_t)blockIdx.x * mat;
  const float *Ds = p.dhs + (size_t)blockIdx.x * mat;
  f32x4 P1[NT], P2[NT], P3[NT], dM[4], dT[4];
#pragma unroll
  for (int t = 0; t < NT; ++t) P1[t] = P2[t] = P3[t] = zero4();
#pragma unroll
  for (int t = 0; t < 4; ++t) dM[t] = dT[t] = zero4();
  float shv = 0.f;  // <dH'_i, H_i> of row i = tid (tid < DK)
  // the next 16-column block's H, dH', dO and V are fetched into registers
  // while the current one computes; the loop's barriers wait only for LDS
  constexpr int HPc = DK * 4 / 256, VECV = 16 / (int)sizeof(In), VPR = 16 / VECV, VNP = 64 * VPR;
  f32x4 rh[HPc], rd[HPc], rdo;
  u32x4 rvv = u32x4{0u, 0u, 0u, 0u};
  auto fetch = [&](int cb) {
#pragma unroll
    for (int it = 0; it < HPc; ++it) {
      const int pc = tid + 256 * it, i = pc / 4, c = (pc % 4) * 4;
      rh[it] = *reinterpret_cast<const f32x4 *>(Hs + (size_t)i * DV + 16 * cb + c);
      rd[it] = *reinterpret_cast<const f32x4 *>(Ds + (size_t)i * DV + 16 * cb + c);
    }
    {
      const int r = tid / 4, c = (tid % 4) * 4;
      rdo = r < C ? *reinterpret_cast<const f32x4 *>(p.dout + ((size_t)(r0 + r) * H + h) * DV + 16 * cb + c)
                  : zero4();
    }
    if (tid < VNP) {
      const int r = tid / VPR, c = (tid % VPR) * VECV;
      rvv = r < C ? *reinterpret_cast<const u32x4 *>(static_cast<const char *>(p.v) +
                                                      (((size_t)(r0 + r) * H + h) * DV + 16 * cb + c) * sizeof(In))
                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  fetch(0);
  for (int cb = 0; cb < DV / 16; ++cb) {
    sync_lds();
#pragma unroll
    for (int it = 0; it < HPc; ++it) {
      const int pc = tid + 256 * it, i = pc / 4, c = (pc % 4) * 4;
      *reinterpret_cast<f32x4 *>(sH + i * LB + c) = rh[it];
      *reinterpret_cast<f32x4 *>(sDH + i * LB + c) = rd[it];
    }
    {
      const int r = tid / 4, c = (tid % 4) * 4;
      *reinterpret_cast<f32x4 *>(sO + r * LB + c) = rdo * p.scale;
    }
    if (tid < VNP) {
      const int r = tid / VPR, c = (tid % VPR) * VECV;
      uint32_t vw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vw[e] = rvv[e];
      float f[VECV];
      unpack16<In>(vw, f);
#pragma unroll
      for (int q = 0; q < VECV / 4; ++q)
        *reinterpret_cast<f32x4 *>(sV + r * LB + c + 4 * q) = f32x4{f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]};
    }
    if (cb + 1 < DV / 16) fetch(cb + 1);
    sync_lds();
    if (tid < DK)
      for (int c = 0; c < 16; ++c) shv += sH[tid * LB + c] * sDH[tid * LB + c];
    {
      f32x4 kh[1] = {zero4()}, kd[1] = {zero4()};
      mmN<1, DK>(kh, sKt + 16 * w * LK, LK, 1, sH, LB, 1, 0);
      mmN<1, DK>(kd, sKh + 16 * w * LK, LK, 1, sDH, LB, 1, 0);
      const f32x4 mo = mm2k<64>(sM + 16 * w, 1, kL, sO, LB, 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i;
        const float x = sV[r * LB + lr] - kh[0][i];
        sX[r * LB + lr] = x;
        sBX[r * LB + lr] = sBeta[r] * x;
        sDU[r * LB + lr] = mo[i] + kd[0][i];
      }
    }
    sync_lds();
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
    sync_lds();
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
  if (tid < DK) gw[part_sh(DK) + tid] = shv;
}

// ----------------------------------------------------------------- final
template <typename In, int DK>
__global__ __launch_bounds__(256) void kda_final_kernel(BwdParams p) {
  constexpr int LK = DK + 4;
  constexpr int MAT = 64 * kL;
  // phase A over the first part: A^-1, S, dM, dT, a product scratch; phase B:
  // K, Q, G ([64][LK] each) with dM (masked) and dS kept after them
  constexpr int KQG = 3 * kBT * LK;
  constexpr int AREA = KQG > 4 * MAT ? KQG : 4 * MAT;
  __shared__ __attribute__((aligned(16))) float smem[AREA + 2 * MAT];
  __shared__ __attribute__((aligned(16))) float sBeta[64], bt[64], ba[64], sEx[256], sTot[256];
  __shared__ int sFit[4];  // row block X's in-block decays run on MFMA (see below)
  float *sK = smem, *sQ = smem + kBT * LK, *sG = smem + 2 * kBT * LK;
  float *sDM = smem + AREA, *sDS = smem + AREA + MAT;
  float *sA = smem, *sS = smem + MAT, *sTmp = smem + 2 * MAT, *sDAi = smem + 3 * MAT;
  const int H = p.H;
  const int slot = blockIdx.x / H, h = blockIdx.x % H;
  Chunk ch;
  if (!chunk_of(p, slot, ch)) return;
  const int C = ch.C, r0 = ch.r0;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), lr = l & 15, lg = l >> 4;
  const float *img = p.prep + (size_t)blockIdx.x * kda_prep_floats(DK);
  const float *gw = p.part + (size_t)blockIdx.x * part_floats(DK);
  const float *P1 = gw + kPartP1, *P2 = gw + part_p2(DK), *P3 = gw + part_p3(DK);
  // this thread's P1..P3 entries for the first two steps of the (row,
  // channel) pass, fetched now so that their latency passes under phase A;
  // the pass then fetches two steps ahead
  constexpr int NPR = 64 * DK / 256;
  float pa[3], pb[3];
  pa[0] = P1[tid], pa[1] = P2[tid], pa[2] = P3[tid];
  pb[0] = P1[tid + 256], pb[1] = P2[tid + 256], pb[2] = P3[tid + 256];
  load_mat64(sA, img + kPrepA);
  load_mat64(sS, img + kPrepS);
  load_mat64(sDM, gw + part_dm(DK));
  load_mat64(sDS, gw + part_dt(DK));  // dT for now
  if (tid < 64) sBeta[tid] = img[kKdaBeta + tid];
  __syncthreads();
  for (int idx = tid; idx < 4096; idx += 256) {
    const int r = idx >> 6, s = idx & 63, o = r * kL + s;
    const bool lo = s <= r && r < C;
    const float dt = sDS[o];
    sTmp[o] = lo ? dt * sA[o] : 0.f;
    sDAi[o] = lo ? dt * sBeta[s] : 0.f;
    sDM[o] = lo ? sDM[o] : 0.f;
  }
  __syncthreads();
  if (tid < 64) {
    float c = 0.f;
    for (int r = 0; r < 64; ++r) c += sTmp[r * kL + tid];
    bt[tid] = c;
  }
  __syncthreads();
  {
    f32x4 t[4] = {zero4(), zero4(), zero4(), zero4()};
    mmN<4, 64>(t, sDAi + 16 * w * kL, kL, 1, sA, 1, kL, 16 * kL);
    __syncthreads();  // every wave is done reading sTmp's column sums above
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int i = 0; i < 4; ++i) sTmp[(16 * w + 4 * lg + i) * kL + 16 * s4 + lr] = t[s4][i];
  }
  __syncthreads();
  {
    f32x4 tA[4] = {zero4(), zero4(), zero4(), zero4()};
    mmN<4, 64>(tA, sA + 16 * w, 1, kL, sTmp, kL, 1, 16);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * lg + i, s = 16 * s4 + lr, o = r * kL + s;
        const bool sl = s < r && r < C;
        const float dA = -tA[s4][i];
        sDAi[o] = sl ? dA * sS[o] : 0.f;          // for dbeta (row sums)
        sDS[o] = sl ? sBeta[r] * dA : 0.f;         // dS
      }
  }
  __syncthreads();
  if (tid < 64) {
    float a = 0.f;
    for (int s = 0; s < 64; ++s) a += sDAi[tid * kL + s];
    ba[tid] = a;
  }
  __syncthreads();
  // phase B: K, Q, G over the phase-A matrices
  load_rows<In, DK>(sK, LK, p.k, r0, C, p.Hqk, h / (H / p.Hqk));
  load_rows<In, DK>(sQ, LK, p.q, r0, C, p.Hqk, h / (H / p.Hqk));
  load_block<64, DK>(sG, LK, img + kKdaG, DK);
  __syncthreads();
  // Row block X's terms inside the block factor through its first row b0
  // (e^{G_x - G_s} = e^{G_x - G_b0} e^{G_b0 - G_s}, one factor <= 1, the other
  // >= 1) and run on MFMA with the cross-block terms, when G_b0 - G_s <= 60
  // in every channel (G decreases down the rows, so the block's last row
  // bounds it); otherwise the (row, channel) pass sums them pair by pair.
  {
    bool fits = true;
    for (int i = l; i < DK; i += 64) fits &= sG[16 * w * LK + i] - sG[(16 * w + 15) * LK + i] <= 60.f;
    const bool all = __ballot(!fits) == 0;
    if (l == 0) sFit[w] = all;
  }
  __syncthreads();
  if (tid < C) {
    const size_t o = (size_t)(r0 + tid) * H + h;
    p.dbeta[o] = bt[tid] + ba[tid];
  }
  const float *shv = gw + part_sh(DK);
  // (row, channel) pairs over all threads, a wave's lanes on consecutive
  // channels of one row: the E-weighted sums, dq, dk and each row's dG
#pragma unroll 1
  for (int k = 0; k < NPR; ++k) {
    const int pr = tid + 256 * k, x = pr / DK, i = pr % DK;
    const float p1 = pa[0], p2 = pa[1], p3 = pa[2];
    pa[0] = pb[0], pa[1] = pb[1], pa[2] = pb[2];
    if (k + 2 < NPR) {
      const int q = pr + 512;
      pb[0] = P1[q], pb[1] = P2[q], pb[2] = P3[q];
    }
    if (x >= C) continue;
    const float Gx = sG[x * LK + i], qx = sQ[x * LK + i], kx = sK[x * LK + i];
    const float GCi = sG[(C - 1) * LK + i];
    float f1 = 0.f, f2 = 0.f, f3 = 0.f, f4 = 0.f;
    // the terms inside x's 16-row block, unless they run on MFMA below (the
    // other blocks follow on MFMA)
    const bool mf = sFit[x >> 4] != 0;
    const int xb = x & ~15, xs = mf ? xb - 1 : x, xe = mf ? xb : min(C, xb + 16);
#pragma unroll 4
    for (int s = xb; s <= xs; ++s) {  // E_xs = exp(G_x - G_s), s <= x
      const float e = __expf(Gx - sG[s * LK + i]) * sK[s * LK + i];
      f1 += sDM[x * kL + s] * e;
      f3 += sDS[x * kL + s] * e;
    }
#pragma unroll 4
    for (int r = x; r < xe; ++r) {  // E_rx = exp(G_r - G_x), r >= x
      const float e = __expf(sG[r * LK + i] - Gx);
      f2 += sDM[r * kL + x] * sQ[r * LK + i] * e;
      f4 += sDS[r * kL + x] * sK[r * LK + i] * e;
    }
    const float gam = __expf(Gx), kh = __expf(GCi - Gx);
    const size_t o = ((size_t)(r0 + x) * H + h) * DK + i;
    p.dq[o] = gam * p1 + f1;
    p.dk[o] = -gam * p2 + kh * p3 + f2 + f3 + f4;
    p.dg[o] = gam * qx * p1 - gam * kx * p2 - kh * kx * p3 + qx * f1 - kx * f2 + kx * f3 - kx * f4;
  }
  __syncthreads();  // every row's dq, dk and dG is in memory
  // The E-weighted sums across 16-row blocks, added to dq, dk and dG.  Wave w
  // owns row block X = w.  For a block S < X the decay factorises through
  // the last row b of S: F1/F3 += exp(G_x - G_b) (dM|dS)[X,S] Kb_S with
  // Kb_S = K_S exp(G_b - G_S); for blocks R > X through the last row b' of
  // X: F2 + F4 += exp(G_b' - G_x) (dM[R,X]^T Qb_R + dS[R,X]^T Kb_R) with
  // Qb_R, Kb_R = (Q_R, K_R) exp(G_R - G_b').  Every factor is at most one.
  {
    const int X = w, j = l & 15, g = l >> 4;
    f32x4 F1[DK / 16], F3[DK / 16], F24[DK / 16];
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) F1[t] = F3[t] = F24[t] = zero4();
    for (int Sb = 0; Sb < X; ++Sb) {
      const int b = 16 * Sb + 15;
#pragma unroll
      for (int t = 0; t < DK / 16; ++t) {
        const int i = 16 * t + j;
        f32x4 z1 = zero4(), z3 = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int s = 16 * Sb + k0 + g;  // B row (k) of this lane
          const float bv = sK[s * LK + i] * __expf(sG[b * LK + i] - sG[s * LK + i]);
          const int am = 16 * X + j, ak = 16 * Sb + k0 + g;  // A (m, k) of this lane
          z1 = mfma4(sDM[am * kL + ak], bv, z1);
          z3 = mfma4(sDS[am * kL + ak], bv, z3);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float sc = __expf(sG[(16 * X + 4 * g + ii) * LK + i] - sG[b * LK + i]);
          F1[t][ii] += sc * z1[ii];
          F3[t][ii] += sc * z3[ii];
        }
      }
    }
    // the block's own terms on MFMA (rows and columns inside block X):
    // F1/F3 += exp(G_x - G_b0) (dM|dS)[X,X] Kb0_X with Kb0 = K exp(G_b0 - G);
    // F24d = exp(G_b0 - G_x) (dM[X,X]^T Qc + dS[X,X]^T Kc) with
    // Qc, Kc = (Q, K) exp(G - G_b0)
    f32x4 F24d[DK / 16];
    const bool mfx = sFit[X] != 0;
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) F24d[t] = zero4();
    if (mfx) {
      const int b0 = 16 * X, am = b0 + j;
#pragma unroll
      for (int t = 0; t < DK / 16; ++t) {
        const int i = 16 * t + j;
        const float gb = sG[b0 * LK + i];
        f32x4 z1 = zero4(), z3 = zero4(), zd = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int s = b0 + k0 + g;  // k index of this lane (a row of block X)
          const float gs = sG[s * LK + i], ks = sK[s * LK + i];
          const float bv = ks * __expf(gb - gs), e = __expf(gs - gb);
          z1 = mfma4(sDM[am * kL + s], bv, z1);
          z3 = mfma4(sDS[am * kL + s], bv, z3);
          zd = mfma4(sDM[s * kL + am], sQ[s * LK + i] * e, zd);
          zd = mfma4(sDS[s * kL + am], ks * e, zd);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float gx = sG[(b0 + 4 * g + ii) * LK + i];
          const float sc = __expf(gx - gb);
          F1[t][ii] += sc * z1[ii];
          F3[t][ii] += sc * z3[ii];
          F24d[t][ii] = __expf(gb - gx) * zd[ii];
        }
      }
    }
    const int bx = 16 * X + 15;
    for (int Rb = X + 1; Rb < 4; ++Rb) {
#pragma unroll
      for (int t = 0; t < DK / 16; ++t) {
        const int i = 16 * t + j;
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) {
          const int r = 16 * Rb + k0 + g;
          const float e = __expf(sG[r * LK + i] - sG[bx * LK + i]);
          const int am = 16 * X + j;
          F24[t] = mfma4(sDM[r * kL + am], sQ[r * LK + i] * e, F24[t]);
          F24[t] = mfma4(sDS[r * kL + am], sK[r * LK + i] * e, F24[t]);
        }
      }
    }
    // every value is read before any is written: the three outputs may
    // alias as far as the compiler knows, so interleaved read-modify-writes
    // would each wait for the previous one.  The complete dG goes to LDS
    // (over dM and dS, read by now) for the scan below.
    f32x4 oq[DK / 16], ok[DK / 16], og[DK / 16];
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int x = 16 * X + 4 * g + ii;
        oq[t][ii] = ok[t][ii] = og[t][ii] = 0.f;
        if (x < C) {
          const size_t o = ((size_t)(r0 + x) * H + h) * DK + 16 * t + j;
          oq[t][ii] = p.dq[o];
          ok[t][ii] = p.dk[o];
          og[t][ii] = p.dg[o];
        }
      }
    __syncthreads();  // every wave is done reading dM and dS
    float *dGs = sDM;  // [64][DK], over dM and dS
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) {
      const int i = 16 * t + j;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int x = 16 * X + 4 * g + ii;
        if (x >= C) continue;
        const float f24 =
            (X < 3 ? __expf(sG[bx * LK + i] - sG[x * LK + i]) * F24[t][ii] : 0.f) + F24d[t][ii];
        const float f1 = F1[t][ii], f3 = F3[t][ii];
        const float qx = sQ[x * LK + i], kx = sK[x * LK + i];
        const size_t o = ((size_t)(r0 + x) * H + h) * DK + i;
        p.dq[o] = oq[t][ii] + f1;
        p.dk[o] = ok[t][ii] + f3 + f24;
        dGs[x * DK + i] = og[t][ii] + qx * f1 + kx * (f3 - f24);
      }
    }
  }
  static_assert(64 * DK <= 2 * MAT, "dG fits over dM and dS");
  __syncthreads();  // every row's dG is complete
  // per channel: the last-row terms (sum_r Kh P3 and exp(G_C) <dH', H>)
  // belong to G_{C-1}, which every row's cumulative sum includes; then dg is
  // the reverse cumulative sum down the rows.  NQ threads per channel take
  // RP rows each; their partial sums meet in a small table.
  {
    constexpr int NQ = 256 / DK, RP = 64 / NQ;
    const float *dGs = sDM;
    const int i = tid % DK, part = tid / DK, x0 = part * RP;
    const float GCi = sG[(C - 1) * LK + i];
    float ex = part == 0 ? __expf(GCi) * shv[i] : 0.f;
    float loc[RP], tot = 0.f;
#pragma unroll
    for (int e = RP - 1; e >= 0; --e) {
      const int x = x0 + e;
      float v = 0.f;
      if (x < C) {
        v = dGs[x * DK + i];
        ex += __expf(GCi - sG[x * LK + i]) * sK[x * LK + i] * P3[x * DK + i];
      }
      tot += v;
      loc[e] = tot;  // sum of this part's rows x .. x0 + RP - 1
    }
    sEx[tid] = ex;
    sTot[tid] = tot;
    __syncthreads();
    float exT = 0.f, above = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      exT += sEx[q * DK + i];
      if (q > part) above += sTot[q * DK + i];
    }
#pragma unroll
    for (int e = 0; e < RP; ++e) {
      const int x = x0 + e;
      if (x < C) p.dg[((size_t)(r0 + x) * H + h) * DK + i] = loc[e] + above + exT;
    }
  }
}

template <typename In, int DK>
hipError_t launch_all(const BwdParams &p, int stage, hipStream_t st) {
  const int cells = p.NT * p.H;
  if (stage == 1) {  // prep: needs no forward recompute
    hipLaunchKernelGGL((kda_prep_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  if (stage == 2) {  // the reverse pass: needs prep only
    if constexpr (std::is_same_v<In, bf16>)
      hipLaunchKernelGGL((kda_dh_bf16_kernel<DK>), dim3(p.N_max * p.H * (DK / 32)), dim3(512), 0, st, p);
    else
      hipLaunchKernelGGL((kda_dh_kernel<In, DK>), dim3(p.N_max * p.H * (DK / 32)), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((kda_part_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((kda_final_kernel<In, DK>), dim3(cells), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_dk(const BwdParams &p, int dk, int stage, hipStream_t st) {
  if (dk == 128) return launch_all<In, 128>(p, stage, st);
  if (dk == 64) return launch_all<In, 64>(p, stage, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_bwd_kda(const BwdParams &p, int dt, int dk, int stage, hipStream_t st) {
  if (dt == LA_BF16) return launch_dk<bf16>(p, dk, stage, st);
  if (dt == LA_F16) return launch_dk<f16>(p, dk, stage, st);
  if (dt == LA_F32) return dk == 64 ? launch_all<float, 64>(p, stage, st) : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

}  // namespace la
