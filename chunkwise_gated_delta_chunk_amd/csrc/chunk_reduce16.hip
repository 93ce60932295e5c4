// Sequential reduce + output stage for 16-bit inputs (bf16 / fp16 values on
// fp16 MFMA): one workgroup per (sequence, head, slice of W = 32 NCW state
// columns), walking the sequence's chunks in order with its slice of the
// state H = S^T ([d_k][W] fp32) held in registers and updated in place.
//
// Per chunk (GDN; rows r of the chunk, gamma_r = exp(G_r), C = last row):
//   X   = V - diag(gamma) (K H)                        state-corrected values
//   U   = diag(beta) X + Tn X                          Tn = T - diag(beta)
//   O   = scale * (diag(gamma) (Q H) + M U)            forward o
//   H  <- gamma_C H + K^T (diag(gamma_C / gamma) U)    forward h
// KDA takes K*exp(G), Q*exp(G), (K*exp(G_C - G))^T and exp(G_C) per key row
// from the map's image, so its row factors are 1.  Columns of U, O and H
// depend only on the same columns of V and H, so d_v splits into slices with
// no cross-slice reduction (the column-wise split of "Empowering Hybrid
// Attention Models on NPUs", section 4); the state is read, the output
// formed, then the state overwritten in place (same paper, section 5).
//
// Wave roles.  Only H -> K H -> X -> U -> H is serial from chunk to chunk;
// the output products Q H and M U hang off it.  So the work splits by role:
//  - chain waves (NCW): each owns 32 state columns (two 16-column MFMA
//    tiles that share every A-operand read) and runs K H, X, U and the
//    update.  It hands the fp16 B operands of H (at the chunk start) and of
//    U (mid-chunk) to its output wave through LDS;
//  - output waves (NCW): the same 32 columns' Q H, then M U and the stores
//    of o, while the chain wave runs the update;
//  - two copy waves: stage the next chunk into the other half of a double
//    buffer.  GDN's K and Q are read as raw 16-bit rows of q and k and
//    converted to fp16 in the chained k order here (the map does not store
//    them); V, Tn, M, the row vectors and KDA's decayed operands arrive by
//    direct global-to-LDS loads.  Raw rows are loaded two chunks ahead into
//    registers, so their latency hides behind a whole chunk.
// Two barriers per chunk: B0 opens the chunk (its stage and the H operands
// are in LDS), B1 publishes U.
//
// Operand scale: the fp16 operands carrying state-side values (H, X, U) are
// formed from those values times a power of two cs per wave, chosen from
// the initial state and the first chunk's V; the recurrence is linear in
// (V, H), so o and every stored state are divided by cs again (exact).
//
// Blocks are numbered so the slices of one (sequence, head) land on the same
// XCD (workgroup IDs are dealt round-robin over the 8 XCDs) and share its L2;
// zero-length sequences and padding units exit before touching memory.
#include "la_device.h"
#include "kernels.h"
#include "reduce_work.h"

namespace la {

namespace {

using O16 = Op<bf16>;  // fp16 MFMA operand traits (bf16 and fp16 inputs alike)

template <bool KDA, int DK, int NCW, int CT>
struct R16 {
  static constexpr ImageLayout I = image_layout(KDA, 2, DK);  // stage layout from K on
  static constexpr int SKIP = image_skip(KDA, 2, DK, !KDA);   // GDN: staged from raw q, k rows
  static constexpr int HBM = image_hbm_bytes(KDA, 2, DK, !KDA);  // DMA'd from the workspace
  static constexpr int W = 16 * CT * NCW;                     // state columns
  static constexpr int PV = W * 2 / 16;                       // 16-byte V pieces per row
  static constexpr int V_BYTES = kBT * W * 2;
  static constexpr int IMG = V_BYTES;                         // image part of a stage
  static constexpr int STAGE = V_BYTES + I.BYTES;
  static constexpr int NKD = DK / 32;                         // k-steps over d_k
  static constexpr int NHT = DK / 16;                         // state row tiles
  static constexpr int PK = DK * 2 / 16, PT = kBT * 2 / 16;   // pieces per K / Tn row
  static constexpr int HB = NKD * CT * 1024;                  // H operands of a chain wave
  static constexpr int UB = 2 * CT * 1024;                    // U operands of a chain wave
  static constexpr int XCH = 2 * STAGE;                       // exchange area
  static constexpr int XW = HB + UB + 16;                     // per chain wave: HB, UB, 1/cs
  static constexpr int LDS = XCH + NCW * XW;
  static constexpr int THREADS = 64 * (2 * NCW + 2);
  static constexpr int NVL = V_BYTES / 1024, NIM = HBM / 1024;
  static constexpr int NU = DK / 16;  // raw K or Q conversion units per copy lane
  static_assert(I.BYTES % 1024 == 0 && HBM % 1024 == 0 && V_BYTES % 1024 == 0, "1 KiB pieces");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(IMG + I.TN + 3 * 256 * PT + 16 <= 65536, "immediate offsets");
};

// Tn / M fragment i = (row tile, k-step) (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__device__ __host__ constexpr int fR(int i) { return i < 2 ? i : (i + 2) / 2; }
__device__ __host__ constexpr int fS(int i) { return i < 2 ? 0 : (i & 1); }

__device__ __forceinline__ half8 as_half8(const u32x4 &v) { return __builtin_bit_cast(half8, v); }
__device__ __forceinline__ u32x4 as_u32x4(const half8 &v) { return __builtin_bit_cast(u32x4, v); }

template <bool KDA, typename In, int DK, int NCW, int CT, bool OUT>
__device__ __forceinline__ void reduce16_body(const ReduceParams &p, const Work &wk, char *smem) {
  using SH = R16<KDA, DK, NCW, CT>;
  using O = O16;
  constexpr ImageLayout I = SH::I;
  constexpr int PV = SH::PV, IMG = SH::IMG, STAGE = SH::STAGE;
  constexpr int NKD = SH::NKD, NHT = SH::NHT, PK = SH::PK, PT = SH::PT;
  constexpr int DV = DK;
  constexpr int DMM = I.MM - I.TN;
  const int H = p.H, h = wk.h, j0 = wk.j0, j1 = wk.j1, eos = wk.eos;
  const int lane = lane_id(), w = wave_id();
  const int lr = lane & 15, lg = lane >> 4;
  // waves 0 .. NCW-1 chain, NCW, NCW+1 copy, then NCW output waves: the
  // waves of a workgroup are dealt over the 4 SIMDs in order, so the chain
  // waves do not share a SIMD with the copy waves' conversion work
  const bool chain = w < NCW, outw = w >= NCW + 2;
  const int cpw = chain || outw ? -1 : w - NCW;  // copy wave index (0, 1) or -1
  const int ci = chain ? w : outw ? w - NCW - 2 : 0;  // chain / output pair index
  const int cw0 = wk.col0 + 16 * CT * ci;        // first state column of the pair
  const uint32_t base = lds_addr(smem);
  const uint32_t xch = base + SH::XCH + ci * SH::XW;  // HB, UB, then 1 / cs
  char *spare = smem + SH::XCH + ci * SH::XW + SH::HB + SH::UB;
  const int rs_v = H * DV * (int)sizeof(In);  // token stride of v (bytes)
  const int osz = p.o_bf16 ? 2 : 4;
  const int rs_o = H * DV * osz;
  auto chunk_barrier = [&]() { barrier_lds(); };

  // ============================================================ copy waves
  if (cpw >= 0) {
    const char *img_c = static_cast<const char *>(p.img) + ((size_t)j0 * H + h) * SH::HBM;
    const size_t img_step = (size_t)H * SH::HBM;
    const In *v_c = static_cast<const In *>(p.v) + ((size_t)wk.t0 * H + h) * DV + (wk.vzero ? 0 : wk.col0);
    const size_t v_step = (size_t)kBT * H * DV;
    int voff[SH::NVL];
#pragma unroll
    for (int q = 0; q < SH::NVL; ++q) {
      const int e = q * 64 + lane;
      const int row = e / PV, phys = e % PV;
      voff[q] = row * rs_v + ((phys ^ swz<PV>(row)) << 4);
    }
    // direct loads of chunk jj's V and image into buffer buf (this copy
    // wave's share: every other 1 KiB piece); beyond the last chunk they run
    // over an empty range (zeros, no memory traffic) so the counts stay fixed
    auto dma = [&](int buf, int jj) {
      const bool live = jj < j1;
      const int r0 = wk.t0 + (jj - j0) * kBT;
      const int C = live ? min(kBT, eos - r0) : 0;
      const auto ri = buffer_rsrc(img_c + (size_t)(jj - j0) * img_step, live ? SH::HBM : 0);
      const auto rv = buffer_rsrc(v_c + (size_t)(jj - j0) * v_step, wk.vzero ? 0 : C * rs_v);
      char *dst = smem + buf * STAGE;
#pragma unroll
      for (int q = 0; q < SH::NVL; ++q)
        if ((q & 1) == cpw) copy16_to_lds(rv, dst + q * 1024, voff[q], 0);
#pragma unroll
      for (int q = 0; q < SH::NIM; ++q) {
        const int at = SH::SKIP + q * 1024;  // stage offset of this piece
        const bool unused = !OUT && ((at >= I.Q && at < I.Q + kBT * DK * 2) ||
                                     (at >= I.MM && at < I.MM + kBT * kBT * 2));
        if ((q & 1) == cpw && !unused) copy16_to_lds(ri, dst + IMG + at, lane * 16, q * 1024);
      }
    };
    // the direct loads this wave issues per chunk (compile-time count)
    constexpr int NDMA = [] {
      int n = 0;
      for (int q = 0; q < SH::NVL; ++q) n += (q & 1) == 0;
      return n;
    }();
    constexpr int NDMA1 = SH::NVL - NDMA;
    constexpr int NIMG0 = [] {
      int n = 0;
      for (int q = 0; q < SH::NIM; ++q) {
        const int at = SH::SKIP + q * 1024;
        const bool unused = !OUT && ((at >= SH::I.Q && at < SH::I.Q + kBT * DK * 2) ||
                                     (at >= SH::I.MM && at < SH::I.MM + kBT * kBT * 2));
        n += (q & 1) == 0 && !unused;
      }
      return n;
    }();
    constexpr int NIMG1 = [] {
      int n = 0;
      for (int q = 0; q < SH::NIM; ++q) {
        const int at = SH::SKIP + q * 1024;
        const bool unused = !OUT && ((at >= SH::I.Q && at < SH::I.Q + kBT * DK * 2) ||
                                     (at >= SH::I.MM && at < SH::I.MM + kBT * kBT * 2));
        n += (q & 1) == 1 && !unused;
      }
      return n;
    }();

    if constexpr (!KDA) {
      // GDN: copy wave 0 stages K, copy wave 1 stages Q (when there is
      // output) from the raw rows, converted to fp16 in the chained k order.
      // Unit i of a lane: row r, 32-element block b, half g2: input pieces
      // 4b + g2 and 4b + 2 + g2 hold the chained pieces 4b + 2 g2 (their low
      // halves) and 4b + 2 g2 + 1 (their high halves).
      constexpr int NU = SH::NU, UPR = DK / 16;  // units per lane, per row
      const bool active = cpw == 0 || OUT;
      const In *src = static_cast<const In *>(cpw == 0 ? p.k_raw : p.q_raw);
      const int Hqk = p.Hqk, hqk = h / (H / Hqk);
      const int rs_q = Hqk * DK * (int)sizeof(In);  // token stride of q, k (bytes)
      const In *src_c = src + ((size_t)wk.t0 * Hqk + hqk) * DK;
      const size_t src_step = (size_t)kBT * Hqk * DK;
      int roff0[NU], roff1[NU];
      uint32_t loff[NU];
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        const int u = lane + 64 * i;
        const int r = u / UPR, b = (u % UPR) >> 1, g2 = u & 1;
        roff0[i] = r * rs_q + (4 * b + g2) * 16;
        roff1[i] = r * rs_q + (4 * b + 2 + g2) * 16;
        loff[i] = (uint32_t)(IMG + (cpw == 0 ? I.K : I.Q) + tile_off<PK>(r, 4 * b + 2 * g2));
      }
      u32x4 raw[2][NU][2];
      auto load_raw = [&](auto rc, int jj) {
        constexpr int RB = decltype(rc)::value;
        const bool live = active && jj < j1;
        const int r0 = wk.t0 + (jj - j0) * kBT;
        const int C = live ? min(kBT, eos - r0) : 0;
        const auto rr = buffer_rsrc(src_c + (size_t)(jj - j0) * src_step, C * rs_q);
#pragma unroll
        for (int i = 0; i < NU; ++i) {
          raw[RB][i][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, roff0[i], 0, 0));
          raw[RB][i][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, roff1[i], 0, 0));
        }
      };
      // units [I0, I1) of the raw rows in register set RB -> buffer buf
      auto put_raw = [&](auto rc, int buf, auto i0c, auto i1c) {
        constexpr int RB = decltype(rc)::value;
        constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
        if (!active) return;
        const uint32_t b0 = base + buf * STAGE;
#pragma unroll
        for (int i = I0; i < I1; ++i) {
          const u32x4 &a = raw[RB][i][0], &c = raw[RB][i][1];
          const u32x4 lo = {to_f16x2<In>(a[0]), to_f16x2<In>(a[1]), to_f16x2<In>(c[0]), to_f16x2<In>(c[1])};
          const u32x4 hi = {to_f16x2<In>(a[2]), to_f16x2<In>(a[3]), to_f16x2<In>(c[2]), to_f16x2<In>(c[3])};
          ds_write_b128(b0 + loff[i], lo);
          ds_write_b128(b0 + (loff[i] ^ 16u), hi);
        }
      };
      constexpr int NR = 2 * NU;  // raw loads per chunk
      // vmcnt waits need compile-time counts: one path per copy wave
      auto run = [&](auto cpc) {
        constexpr int CP = decltype(cpc)::value;
        constexpr int ND = CP == 0 ? NDMA + NIMG0 : NDMA1 + NIMG1;
        // prologue, in the steady state's issue order: the first chunk's raw
        // rows, its direct loads, the second chunk's raw rows; then the
        // first chunk's K / Q into buffer 0
        load_raw(std::integral_constant<int, 0>{}, j0);
        issue_fence();
        dma(0, j0);
        issue_fence();
        load_raw(std::integral_constant<int, 1>{}, j0 + 1);
        issue_fence();
        wait_vm<ND + NR>();  // raw rows of j0
        put_raw(std::integral_constant<int, 0>{}, 0, std::integral_constant<int, 0>{},
                std::integral_constant<int, NU>{});
        wait_vm<NR>();       // direct loads of j0 (only j0 + 1's raw rows may be outstanding)
        wait_lgkm<0>();
        chunk_barrier();     // P
        auto step = [&](auto bc, int jj) {
          constexpr int B = decltype(bc)::value;  // buffer and register set of chunk jj
          chunk_barrier();                         // B0 of chunk jj
          issue_fence();
          dma(1 - B, jj + 1);
          issue_fence();
          load_raw(std::integral_constant<int, B>{}, jj + 2);
          issue_fence();
          // the conversion only has to land before B0 of chunk jj + 1: a
          // quarter of it runs before B1 (where its LDS writes meet the K H,
          // X and U reads), the rest after
          wait_vm<ND + NR>();                      // raw rows of jj + 1
          put_raw(std::integral_constant<int, 1 - B>{}, 1 - B, std::integral_constant<int, 0>{},
                  std::integral_constant<int, NU / 4>{});
          chunk_barrier();                         // B1 of chunk jj
          put_raw(std::integral_constant<int, 1 - B>{}, 1 - B, std::integral_constant<int, NU / 4>{},
                  std::integral_constant<int, NU>{});
          wait_vm<NR>();                           // direct loads of jj + 1
          wait_lgkm<0>();
        };
        for (int jj = j0;;) {
          step(std::integral_constant<int, 0>{}, jj);
          if (++jj == j1) break;
          step(std::integral_constant<int, 1>{}, jj);
          if (++jj == j1) break;
        }
        wait_vm<0>();
      };
      if (cpw == 0) run(std::integral_constant<int, 0>{});
      else run(std::integral_constant<int, 1>{});
    } else {
      auto run = [&](auto cpc) {
        constexpr int CP = decltype(cpc)::value;
        constexpr int ND = CP == 0 ? NDMA + NIMG0 : NDMA1 + NIMG1;
        (void)ND;
        dma(0, j0);
        issue_fence();
        wait_vm<0>();
        chunk_barrier();  // P
        auto step = [&](auto bc, int jj) {
          constexpr int B = decltype(bc)::value;
          chunk_barrier();  // B0
          issue_fence();
          dma(1 - B, jj + 1);
          issue_fence();
          chunk_barrier();  // B1
          wait_vm<0>();
        };
        for (int jj = j0;;) {
          step(std::integral_constant<int, 0>{}, jj);
          if (++jj == j1) break;
          step(std::integral_constant<int, 1>{}, jj);
          if (++jj == j1) break;
        }
      };
      if (cpw == 0) run(std::integral_constant<int, 0>{});
      else run(std::integral_constant<int, 1>{});
    }
    return;
  }

  // ====================================================== compute waves
  // per-lane LDS byte addresses, one set per buffer; immediates add the rest
  uint32_t aK[2][NKD];      // A fragment of K (row tile 0, k-step s); Q at + I.Q - I.K
  uint32_t aT[2][NHT / 2];  // GDN: transposed K^T reads, tile pair u
  uint32_t aKT[2][2];       // KDA: A fragment of K^T (row tile 0, k-step s)
  uint32_t aV[2][CT];       // transposed V reads, column tile c
  uint32_t aP[2][2];        // Tn fragments (row tile 0, k-step s); M at + DMM
  uint32_t aS[2];           // row vectors, rows 4 lg .. 4 lg + 3
#pragma unroll
  for (int bf = 0; bf < 2; ++bf) {
    const uint32_t b0 = base + bf * STAGE;
#pragma unroll
    for (int s = 0; s < NKD; ++s) aK[bf][s] = b0 + tile_off<PK>(lr, 4 * s + lg);
    const int row = 4 * lg + (lr >> 2);
#pragma unroll
    for (int u = 0; u < NHT / 2; ++u) aT[bf][u] = b0 + tile_off<PK>(row, 4 * u + (lr & 3));
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      aKT[bf][s] = b0 + tile_off<PT>(lr, 4 * s + lg);
      aP[bf][s] = b0 + IMG + I.TN + tile_off<PT>(lr, 4 * s + lg);
    }
    aS[bf] = b0 + IMG + I.VEC + 16 * lg;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      // lane i of a 16-lane group reads row 4 lg + i / 4 at columns
      // col + 4 (i % 4) .. +3 and receives column col + i of 4 rows
      const int col = 16 * CT * ci + 16 * c + 4 * (lr & 3);
      aV[bf][c] = b0 + tile_off<PV>(row, col >> 3) + 2 * (col & 7);
    }
  }
  const uint32_t aHB = xch + 16 * lane;                // + (CT s + c) KiB
  const uint32_t aUB = xch + SH::HB + 16 * lane;       // + (CT s + c) KiB

  // ------------------------------------------------------------ output waves
  if (outw) {
    // the chain wave's 1 / cs: in the exchange area from the first B0 on
    float osc = p.scale;
    chunk_barrier();  // P
    // The output tile is formed transposed, O^T = (Q H)^T diag(gamma) +
    // U^T M^T: the H and U operands the chain wave hands over serve as A
    // fragments of H^T and U^T as they are, and the Q and M fragments
    // (row = token, k = key / chunk column in chained order) as B fragments
    // of Q^T and M^T.  Lane (g, n) of tile (c, R) then holds output row
    // 16 R + n at the four columns 16 c + 4 g .. +3: 16 contiguous bytes of
    // one row, stored straight from the accumulators (no LDS round trip);
    // one store per tile covers 16 rows x 64 bytes.
    const int off_st = lr * rs_o + (cw0 + 4 * lg) * osz;
    char *o_c = static_cast<char *>(p.o) + ((size_t)wk.t0 * H + h) * DV * osz;
    const size_t o_step = (size_t)kBT * H * DV * osz;
    // chunk jj's O^T tiles -> o (C valid rows)
    auto store_o = [&](const f32x4 (*ot)[4], int jj, int C) {
      char *o_r = o_c + (size_t)(jj - j0) * o_step;
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const auto ro = buffer_rsrc(o_r + (size_t)16 * R * rs_o, (C - 16 * R) * rs_o);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          if (p.o_bf16) {
            const uint32_t w0 = f32_to_bf16_rne(ot[c][R][0]) | (f32_to_bf16_rne(ot[c][R][1]) << 16);
            const uint32_t w1 = f32_to_bf16_rne(ot[c][R][2]) | (f32_to_bf16_rne(ot[c][R][3]) << 16);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, ro, off_st + 16 * c * osz, 0, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ot[c][R]), ro,
                                                   off_st + 16 * c * osz, 0, 0);
          }
        }
      }
    };
    // A chunk's O rows are stored during the next chunk, once that chunk's
    // first LDS reads are issued: the stores then queue behind the copy
    // waves' loads while this wave waits for its operands anyway, instead of
    // holding up the barrier that opens the next chunk.
    f32x4 opend[CT][4];
    int jpend = j0, cpend = 0;  // cpend > 0: the O rows of chunk jpend are pending
    // gamma of this lane's token in row tile R: exp(G) at 16 R + lane % 16
    const uint32_t aG = IMG + I.VEC + 4 * lr;  // + buffer base
    auto ochunk = [&](auto bc, int jj) {
      constexpr int B = decltype(bc)::value;
      chunk_barrier();  // B0
      if (OUT && jj == j0) osc = p.scale * *reinterpret_cast<const volatile float *>(spare);
      if constexpr (!OUT) {
        chunk_barrier();  // B1
        return;
      } else {
        const int r0 = wk.t0 + (jj - j0) * kBT;
        const int C = min(kBT, eos - r0);
        half8 hb[CT][NKD];
        static_for<NKD>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          static_for<CT>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            ds_read_b128_at<(CT * s + c) * 1024>(hb[c][s], aHB);
          });
        });
        half8 fq[NKD][4];
        auto read_q = [&](auto sc) {
          constexpr int s = decltype(sc)::value;
          static_for<4>([&](auto rc) {
            constexpr int R = decltype(rc)::value;
            ds_read_b128_at<IMG + I.Q + R * 256 * PK>(fq[s][R], aK[B][s]);
          });
        };
        read_q(std::integral_constant<int, 0>{});
        if constexpr (NKD > 1) read_q(std::integral_constant<int, 1>{});
        if (cpend > 0) store_o(opend, jpend, cpend);
        f32x4 yq[CT][4];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int R = 0; R < 4; ++R) yq[c][R] = zero4();
        float gam[4];
        half8 fm[6];
        static_for<NKD>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          // outstanding after k-step s's Q reads: those of k-step s + 1
          constexpr int LATER = s + 1 < NKD ? 4 : 0;
          wait_lds_tied4<LATER>(fq[s][0], fq[s][1], fq[s][2], fq[s][3]);
          if constexpr (s == 0) {
            // the H operands were issued before the Q reads
            if constexpr (CT == 2 && NKD == 4) {
              wait_lds_tied8<LATER>(hb[0][0], hb[0][1], hb[0][2], hb[0][3], hb[1][0], hb[1][1],
                                    hb[1][2], hb[1][3]);
            } else if constexpr (CT == 2 || NKD == 4) {
              wait_lds_tied4<LATER>(hb[0][0], hb[0][1], hb[CT - 1][NKD - 2], hb[CT - 1][NKD - 1]);
            } else {
              wait_lds_tied2<LATER>(hb[0][0], hb[0][1]);
            }
          }
          if constexpr (s + 2 < NKD) read_q(std::integral_constant<int, s + 2>{});
          if constexpr (s == NKD - 1) {
            static_for<4>([&](auto rc) {
              constexpr int R = decltype(rc)::value;
              ds_read_b32_at<64 * R>(gam[R], base + B * STAGE + aG);
            });
            static_for<6>([&](auto ic) {
              constexpr int i = decltype(ic)::value;
              ds_read_b128_at<DMM + fR(i) * 256 * PT>(fm[i], aP[B][fS(i)]);
            });
          }
#pragma unroll
          for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int c = 0; c < CT; ++c) yq[c][R] = O::mfma(hb[c][s], fq[s][R], yq[c][R]);
        });
        wait_lds_tied4<6>(gam[0], gam[1], gam[2], gam[3]);
        chunk_barrier();  // B1: U of this chunk is in the exchange area
        half8 ub[CT][2];
        static_for<2>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          static_for<CT>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            ds_read_b128_at<(CT * s + c) * 1024>(ub[c][s], aUB);
          });
        });
        f32x4 oa[CT][4];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int e = 0; e < 4; ++e) oa[c][R][e] = gam[R] * yq[c][R][e];
        wait_lds_tied2<4>(fm[0], fm[1]);
        wait_lds_tied4<4>(fm[2], fm[3], fm[4], fm[5]);
        if constexpr (CT == 2) wait_lds_tied4<0>(ub[0][0], ub[1][0], ub[0][1], ub[1][1]);
        else wait_lds_tied2<0>(ub[0][0], ub[0][1]);
        static_for<6>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
#pragma unroll
          for (int c = 0; c < CT; ++c) oa[c][fR(i)] = O::mfma(ub[c][fS(i)], fm[i], oa[c][fR(i)]);
        });
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int e = 0; e < 4; ++e) opend[c][R][e] = osc * oa[c][R][e];
        jpend = jj;
        cpend = C;
      }
    };
    for (int jj = j0;;) {
      ochunk(std::integral_constant<int, 0>{}, jj);
      if (++jj == j1) break;
      ochunk(std::integral_constant<int, 1>{}, jj);
      if (++jj == j1) break;
    }
    if (cpend > 0) store_o(opend, jpend, cpend);
    return;
  }

  // ------------------------------------------------------------- chain waves
  (void)chain;
  f32x4 hacc[CT][NHT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int colc = cw0 + 16 * c + lr;
    if (wk.init) {
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[c][t][e] = wk.init[(size_t)(16 * t + lg * 4 + e) * DV + colc];
    } else {
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[c][t][e] = wk.init_id && 16 * t + lg * 4 + e == colc ? 1.f : 0.f;
    }
  }
  float cs = 1.f, ics = 1.f;
  chunk_barrier();  // P: the first chunk's stage has landed in buffer 0
  {
    s16x4 v0[CT][4];
    static_for<4>([&](auto rc) {
      constexpr int R = decltype(rc)::value;
#pragma unroll
      for (int c = 0; c < CT; ++c) ds_read_tr16_at<R * 256 * PV>(v0[c][R], aV[0][c]);
    });
#pragma unroll
    for (int c = 0; c < CT; ++c) wait_lds_tied<0>(v0[c][0], v0[c][1], v0[c][2], v0[c][3]);
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(in16_to_f32<In>((uint16_t)v0[c][R][e])));
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(hacc[c][t][e]));
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (m > 0.f && m <= 3.0e38f) {
      int ex;
      (void)frexpf(m, &ex);  // m in [2^(ex-1), 2^ex): m cs in [4, 8)
      const int k = min(max(3 - ex, -100), 100);
      cs = ldexpf(1.f, k);
      ics = ldexpf(1.f, -k);
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int t = 0; t < NHT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) hacc[c][t][e] *= cs;
    }
  }
  // the output wave's divisor: 1 / cs in the exchange area's last word
  if constexpr (OUT) {
    if (lane == 0) *reinterpret_cast<volatile float *>(spare) = ics;
  }
  half8 hb[CT][NKD];
  // the B operands of k-step s of H (state row tiles 2s, 2s + 1), kept for
  // this wave's next K H and handed to the output wave
  auto put_hb_step = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
#pragma unroll
    for (int c = 0; c < CT; ++c) hb[c][s] = b_frag<O>(hacc[c], s);
    if constexpr (OUT) {
      static_for<CT>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        ds_write_b128_at<(CT * s + c) * 1024>(aHB, as_u32x4(hb[c][s]));
      });
    }
  };
  auto put_hb = [&]() { static_for<NKD>([&](auto sc) { put_hb_step(sc); }); };
  put_hb();
  wait_lgkm<0>();

  constexpr bool GDN = !KDA;
  auto cchunk = [&](auto bc, int jj) {
    constexpr int B = decltype(bc)::value;
    chunk_barrier();  // B0: this chunk's stage and H operands are in LDS
    if (p.hsave) {    // the state entering chunk jj (backward recompute)
      float *hs = p.hsave + ((size_t)jj * H + h) * DK * DV;
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int t = 0; t < NHT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            hs[(size_t)(16 * t + lg * 4 + e) * DV + cw0 + 16 * c + lr] = hacc[c][t][e] * ics;
    }
    // ---- K H, the state operand from registers; K fragments two k-steps ahead
    half8 fk[NKD][4];
    auto read_k = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      static_for<4>([&](auto rc) {
        constexpr int R = decltype(rc)::value;
        ds_read_b128_at<IMG + I.K + R * 256 * PK>(fk[s][R], aK[B][s]);
      });
    };
    read_k(std::integral_constant<int, 0>{});
    if constexpr (NKD > 1) read_k(std::integral_constant<int, 1>{});
    f32x4 yk[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int R = 0; R < 4; ++R) yk[c][R] = zero4();
    s16x4 vr[CT][4];
    f32x4 gam[4];
    static_for<NKD>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      constexpr int LATER = s + 1 < NKD ? 4 : 0;
      wait_lds_tied4<LATER>(fk[s][0], fk[s][1], fk[s][2], fk[s][3]);
      if constexpr (s + 2 < NKD) read_k(std::integral_constant<int, s + 2>{});
      if constexpr (s == NKD - 1) {
        // V and gamma, behind the last K reads
        static_for<4>([&](auto rc) {
          constexpr int R = decltype(rc)::value;
#pragma unroll
          for (int c = 0; c < CT; ++c) ds_read_tr16_at<R * 256 * PV>(vr[c][R], aV[B][c]);
        });
        if constexpr (GDN)
          static_for<4>([&](auto rc) {
            constexpr int R = decltype(rc)::value;
            ds_read_b128_at<64 * R>(gam[R], aS[B]);
          });
      }
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int c = 0; c < CT; ++c) yk[c][R] = O::mfma(fk[s][R], hb[c][s], yk[c][R]);
    });
    // ---- X = cs V - gamma (K H)
    if constexpr (GDN) wait_lds_tied4<0>(gam[0], gam[1], gam[2], gam[3]);
#pragma unroll
    for (int c = 0; c < CT; ++c) wait_lds_tied<0>(vr[c][0], vr[c][1], vr[c][2], vr[c][3]);
    // Tn, beta, the update factors and the state decay while X forms
    half8 ft[6];
    f32x4 bet[4], fac[4], dcv;
    f32x4 dec[KDA ? NHT : 1];  // KDA: the state decay of each key row
    static_for<6>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      ds_read_b128_at<fR(i) * 256 * PT>(ft[i], aP[B][fS(i)]);
    });
    static_for<4>([&](auto rc) {
      constexpr int R = decltype(rc)::value;
      ds_read_b128_at<512 + 64 * R>(bet[R], aS[B]);
      if constexpr (GDN) ds_read_b128_at<256 + 64 * R>(fac[R], aS[B]);
    });
    if constexpr (GDN) ds_read_b128_at<768>(dcv, aS[B]);
    if constexpr (KDA)
      static_for<NHT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        ds_read_b128_at<768 + 64 * t>(dec[t], aS[B]);
      });
    constexpr int AFTER_TN0 = GDN ? 9 : 4 + NHT;
    constexpr int AFTER_TN = AFTER_TN0 < 15 ? AFTER_TN0 : 15;
    f32x4 x[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = in16_to_f32<In>((uint16_t)vr[c][R][e]);
          x[c][R][e] = GDN ? fmaf(v, cs, -gam[R][e] * yk[c][R][e]) : fmaf(v, cs, -yk[c][R][e]);
        }
    half8 xb[CT][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < CT; ++c) xb[c][s] = b_frag<O>(x[c], s);
    // ---- U = beta X + Tn X
    wait_lds_tied2<AFTER_TN>(ft[0], ft[1]);
    wait_lds_tied4<AFTER_TN>(ft[2], ft[3], ft[4], ft[5]);
    f32x4 u[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int R = 0; R < 4; ++R) u[c][R] = zero4();
    static_for<6>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int c = 0; c < CT; ++c) u[c][fR(i)] = O::mfma(ft[i], xb[c][fS(i)], u[c][fR(i)]);
    });
    wait_lds_tied4<0>(bet[0], bet[1], bet[2], bet[3]);
    if constexpr (KDA) {
      if constexpr (NHT == 8) {
        wait_lds_tied8<0>(dec[0], dec[1], dec[2], dec[3], dec[4], dec[5], dec[6], dec[7]);
      } else {
        wait_lds_tied4<0>(dec[0], dec[1], dec[2], dec[3]);
      }
    }
    float gdec = 1.f;
    if constexpr (GDN) {
      wait_lds_tied4<0>(fac[0], fac[1], fac[2], fac[3]);
      wait_lds_tied1<0>(dcv);
      gdec = dcv[0];
    }
    half8 ufr[CT][2], ubf[CT][2];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      f32x4 ub[4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[c][R][e] += bet[R][e] * x[c][R][e];
        if constexpr (GDN)
#pragma unroll
          for (int e = 0; e < 4; ++e) ub[R][e] = fac[R][e] * u[c][R][e];
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        ufr[c][s] = b_frag<O>(u[c], s);
        if constexpr (GDN) ubf[c][s] = b_frag<O>(ub, s);
        else ubf[c][s] = ufr[c][s];
      }
    }
    // ---- U to the output wave; the first K^T reads of the update
    if constexpr (OUT) {
      static_for<2>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        static_for<CT>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          ds_write_b128_at<(CT * s + c) * 1024>(aUB, as_u32x4(ufr[c][s]));
        });
      });
    }
    // GDN: K^T of state row tile t, k-step s as two transposed reads
    // (half q of k-step s: rows 32 s + 16 q ..) from the row-major K tile
    s16x4 tr[GDN ? NHT : 1][4];
    half8 fkt[KDA ? NHT : 1][2];
    auto read_kt = [&](auto tc) {
      constexpr int t = decltype(tc)::value;
      if constexpr (GDN) {
        static_for<4>([&](auto qc) {
          constexpr int q = decltype(qc)::value;  // (k-step, half) = (q / 2, q % 2)
          constexpr int OFF = IMG + I.K + (32 * (q >> 1) + 16 * (q & 1)) * 16 * PK + 8 * (t & 1);
          ds_read_tr16_at<OFF>(tr[t][q], aT[B][t >> 1]);
        });
      } else {
        ds_read_b128_at<IMG + I.KT + t * 256 * PT>(fkt[t][0], aKT[B][0]);
        ds_read_b128_at<IMG + I.KT + t * 256 * PT>(fkt[t][1], aKT[B][1]);
      }
    };
    constexpr int RPT = GDN ? 4 : 2;                      // reads per state row tile
    // tiles read before B1: none.  B1 then comes as soon as U is out, which
    // starts the output waves' M U and the copy waves' conversion earlier;
    // the transposed reads' latency moves to the chain's own update
    constexpr int PRE = 0;
    static_for<PRE>([&](auto tc) { read_kt(tc); });
    // the exchange writes must land before B1
    wait_lgkm<PRE * RPT>();
    chunk_barrier();  // B1
    static_for<NHT - PRE>([&](auto tc) { read_kt(std::integral_constant<int, PRE + decltype(tc)::value>{}); });
    // ---- H <- decay H + Kbar^T Ubar
    static_for<NHT>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      // outstanding after tile t's reads: the later tiles'
      constexpr int LATER0 = RPT * (NHT - 1 - t);
      constexpr int LATER = LATER0 < 15 ? LATER0 : 15;
      if constexpr (GDN) {
        wait_lds_tied<LATER>(tr[t][0], tr[t][1], tr[t][2], tr[t][3]);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
          for (int e = 0; e < 4; ++e) hacc[c][t][e] *= gdec;
#pragma unroll
          for (int s = 0; s < 2; ++s)
            hacc[c][t] = O::mfma(join_half8(tr[t][2 * s], tr[t][2 * s + 1]), ubf[c][s], hacc[c][t]);
        }
      } else {
        wait_lds_tied2<LATER>(fkt[t][0], fkt[t][1]);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
#pragma unroll
          for (int e = 0; e < 4; ++e) hacc[c][t][e] *= dec[t][e];
#pragma unroll
          for (int s = 0; s < 2; ++s) hacc[c][t] = O::mfma(fkt[t][s], ubf[c][s], hacc[c][t]);
        }
      }
      // the H operands of a pair of row tiles go out while the next pair's
      // products run (the pair before the one just issued is complete)
      if constexpr (t % 2 == 1 && t >= 3) put_hb_step(std::integral_constant<int, (t - 3) / 2>{});
    });
    put_hb_step(std::integral_constant<int, NKD - 1>{});
    wait_lgkm<0>();
  };
  for (int jj = j0;;) {
    cchunk(std::integral_constant<int, 0>{}, jj);
    if (++jj == j1) break;
    cchunk(std::integral_constant<int, 1>{}, jj);
    if (++jj == j1) break;
  }

  // ---- final state slice: fp32, or the fp16 hi / lo images of a segment's
  // transition (element (r, c) where an A fragment of a [d_k][d_k] operand
  // with chained columns expects it: row r, column kpos(c))
  if (wk.fin) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wk.fin[(size_t)(16 * t + lg * 4 + e) * DV + cw0 + 16 * c + lr] = hacc[c][t][e] * ics;
  }
  if (wk.pimg) {
    constexpr int PP = DK * 2 / 16;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int kc = kpos<O>(cw0 + 16 * c + lr);
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * t + lg * 4 + e;
          const int off = (tile_off<PP>(r, kc >> 3) >> 1) + (kc & 7);
          const float hv = hacc[c][t][e] * ics;
          const _Float16 hi = (_Float16)hv;
          wk.pimg[off] = hi;
          wk.pimg[DK * DK + off] = (_Float16)(hv - (float)hi);
        }
    }
  }
}

template <bool KDA, typename In, int DK, int NCW, int CT>
__global__ __launch_bounds__(64 * (2 * NCW + 2)) void chunk_reduce16_kernel(ReduceParams p) {
  using SH = R16<KDA, DK, NCW, CT>;
  __shared__ __attribute__((aligned(16))) char smem[SH::LDS];
  Work wk;
  const int role = decode_work<DK, SH::W>(p, wk);
  if (role == 1) reduce16_body<KDA, In, DK, NCW, CT, true>(p, wk, smem);
  else if (role == 2) reduce16_body<KDA, In, DK, NCW, CT, false>(p, wk, smem);
}

}  // namespace

template <bool KDA, typename In, int DK, int NCW, int CT>
static hipError_t launch_r16(const ReduceParams &p, hipStream_t st) {
  using SH = R16<KDA, DK, NCW, CT>;
  const int units = (p.seg ? p.NS_max : p.N_max) * p.H;
  const int grid = ((units + 7) / 8) * 8 * (p.pass == 1 ? p.S + p.SP : p.S);
  hipLaunchKernelGGL((chunk_reduce16_kernel<KDA, In, DK, NCW, CT>), dim3(grid), dim3(SH::THREADS), 0, st, p);
  return hipGetLastError();
}

template <bool KDA, typename In, int DK>
static hipError_t launch_r16_w(const ReduceParams &p, int W, hipStream_t st) {
  // 32 columns: two chain waves and two output waves of one 16-column tile
  if (W == 32) return launch_r16<KDA, In, DK, 2, 1>(p, st);
  return hipErrorInvalidValue;
}

template <typename In>
static hipError_t launch_r16_t(const ReduceParams &p, bool kda, int dk, int W, hipStream_t st) {
  if (dk == 128)
    return kda ? launch_r16_w<true, In, 128>(p, W, st) : launch_r16_w<false, In, 128>(p, W, st);
  if (dk == 64)
    return kda ? launch_r16_w<true, In, 64>(p, W, st) : launch_r16_w<false, In, 64>(p, W, st);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_reduce16(const ReduceParams &p, bool kda, int dt, int dk, int W,
                                 hipStream_t st) {
  if (dt == LA_BF16) return launch_r16_t<bf16>(p, kda, dk, W, st);
  if (dt == LA_F16) return launch_r16_t<f16>(p, kda, dk, W, st);
  return hipErrorInvalidValue;
}

}  // namespace la
