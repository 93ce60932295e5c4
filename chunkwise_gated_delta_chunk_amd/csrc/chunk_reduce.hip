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
// Work split: each wave owns 16 state columns for all chunk rows, so the
// chain H -> K H -> X -> U -> H of its columns never leaves the wave.  With
// the chained k order (see la_device.h) an accumulator tile is itself the B
// operand of the next product, so H, X and U stay in registers.  Only the
// shared, state-independent operands of a chunk are in LDS: the V slice and
// the map stage's image of the chunk (K, Q, [K^T], Tn, M, row vectors).  Both
// are copied one chunk ahead by direct global-to-LDS loads (no registers, no
// LDS store instructions) into the other half of a double buffer, by one
// extra wave per workgroup that does nothing else: one barrier per chunk,
// the copy of chunk j + 1 overlaps the arithmetic of chunk j, and the
// compute waves never block on issuing vector memory loads.  V rows past the
// chunk's end read as zero through the buffer range check, and output rows
// past it are dropped the same way.
//
// Instruction overhead is kept off the per-chunk path: every hot LDS address
// is a per-lane pattern computed once plus an immediate offset (the chunk
// loop is unrolled over the two buffers so the buffer is a constant), the
// copy's per-lane offsets are computed once, and the memory resources
// advance by pointer bumps.  The fp16 reads of K and Q fragments, of V and of
// the transposed K^T fragments are opaque inline-assembly reads issued well
// ahead of their MFMAs with waits tied to their registers: the compiler's own
// schedule keeps only one or two LDS reads in flight, and it waits for every
// outstanding vector memory operation before a builtin transposed read.
//
// Blocks are numbered so that the slices of one (sequence, head) land on the
// same XCD (workgroup IDs are dealt round-robin over the 8 XCDs) and share
// its L2 for the image reads.  Zero-length sequences and padding units exit
// before touching memory, so they write nothing.
#include "la_device.h"
#include "kernels.h"
#include "reduce_work.h"

namespace la {

namespace {

// Geometry shared by the kernel (LDS size) and its body.
template <bool KDA, typename In, int DK, int NW, bool RAW>
struct ReduceShape {
  using O = Op<In>;
  static constexpr int E = (int)sizeof(typename O::T);
  static constexpr ImageLayout I = image_layout(KDA, E, DK);
  // RAW (GDN, 16-bit): the image in the workspace starts at Tn; K and Q are
  // staged from the raw rows of k and q by the copy waves (a second one for Q)
  static constexpr int SKIP = image_skip(KDA, E, DK, RAW);
  static constexpr int HBM = image_hbm_bytes(KDA, E, DK, RAW);
  static constexpr int THREADS = 64 * (NW + 1 + (RAW ? 1 : 0));
  static constexpr int W = 16 * NW;                       // state columns per workgroup
  static constexpr int V_BYTES = kBT * W * (int)sizeof(In);
  // stage buffer: the V tile first (its reads and those of K and Q stay
  // under the 64 KiB immediate offset), then the image
  static constexpr int IMG = V_BYTES;
  static constexpr int STAGE = V_BYTES + I.BYTES;
  static constexpr int NBUF = 2 * STAGE <= 160 * 1024 ? 2 : 1;
};

template <bool KDA, typename In, int DK, int NW, bool OUT, bool RAW>
__device__ __forceinline__ void reduce_body(const ReduceParams &p, const Work &wk, char *smem) {
  using O = Op<In>;
  using SH = ReduceShape<KDA, In, DK, NW, RAW>;
  constexpr int E = SH::E;
  constexpr ImageLayout I = SH::I;
  constexpr bool HAS_KT = KDA || O::KPL == 1;
  constexpr bool F16 = O::KPL == 8;
  constexpr int PK = DK * E / 16, PT = kBT * E / 16;
  constexpr int W = SH::W;                   // state columns per workgroup
  constexpr int DV = DK;                     // d_v == d_k
  constexpr int NKD = ksteps<O>(DK);         // k-steps over d_k
  constexpr int NKR = ksteps<O>(kBT);        // k-steps over chunk rows
  constexpr int NHT = DK / 16;               // state row tiles
  constexpr int PV = W * (int)sizeof(In) / 16;   // 16-byte pieces per V row
  constexpr int V_BYTES = SH::V_BYTES;
  constexpr int IMG = SH::IMG;
  constexpr int STAGE = SH::STAGE;
  constexpr int NBUF = SH::NBUF;
  constexpr int NVL = V_BYTES / 1024, NIMG = SH::HBM / 1024;
  static_assert(I.BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "1 KiB staging pieces");
  static_assert(!RAW || (F16 && !KDA && NBUF == 2), "raw K / Q staging: 16-bit GDN, two buffers");
  static_assert(!F16 || IMG + I.Q + 3 * 256 * PK + 16 <= 65536, "immediate offsets");

  const int H = p.H;
  const int n = wk.n, h = wk.h, j0 = wk.j0, j1 = wk.j1, eos = wk.eos;
  (void)n;
  const int lane = lane_id(), w = wave_id();
  const bool copier = w >= NW;  // the extra wave(s) only stage operands
  const int lr = lane & 15, lg = lane >> 4;
  const int cw = wk.col0 + 16 * w;                   // this wave's first state column
  const int rs_v = H * DV * (int)sizeof(In);         // token stride of v (bytes)
  const int osz = p.o_bf16 ? 2 : 4;                  // o element bytes
  const int rs_o = H * DV * osz;                     // token stride of o (bytes)

  // ---------------------------------------------------------------- staging
  // One extra wave per workgroup does all the staging: piece q (1 KiB) of a
  // stage is V piece q for q < NVL, then image piece q - NVL.  A CU's vector
  // memory path takes tens of cycles per piece, and a wave that issues loads
  // blocks until they are accepted; the compute waves issue none.  A V
  // piece's per-lane source offset (row and swizzled column piece within the
  // chunk) does not depend on the chunk.
  int voff[NVL];
#pragma unroll
  for (int q = 0; q < NVL; ++q) {
    const int e = q * 64 + lane;  // 16-byte V piece index
    const int row = e / PV, phys = e % PV;
    voff[q] = row * rs_v + ((phys ^ swz<PV>(row)) << 4);
  }
  const char *img_c = static_cast<const char *>(p.img) + ((size_t)j0 * H + h) * SH::HBM;
  const size_t img_step = (size_t)H * SH::HBM;
  const In *v_c = static_cast<const In *>(p.v) + ((size_t)wk.t0 * H + h) * DV + (wk.vzero ? 0 : wk.col0);
  const size_t v_step = (size_t)kBT * H * DV;
  // copy of the chunk whose image starts at img and whose C V rows start at vrow
  // (no output: the Q and M pieces of the image are not needed; a zero V
  // has an empty range, so its loads write zeros)
  auto copy_chunk = [&](int buf, const char *img, const In *vrow, int C) {
    const auto ri = buffer_rsrc(img, C > 0 ? SH::HBM : 0);
    const auto rv = buffer_rsrc(vrow, wk.vzero ? 0 : C * rs_v);
    char *dst = smem + buf * STAGE;
#pragma unroll
    for (int q = 0; q < NVL; ++q) copy16_to_lds(rv, dst + q * 1024, voff[q], 0);
#pragma unroll
    for (int q = 0; q < NIMG; ++q) {
      const int at = SH::SKIP + q * 1024;  // stage offset of the piece
      const bool unused = !OUT && ((at >= I.Q && at < I.Q + kBT * DK * E) ||
                                   (at >= I.MM && at < I.MM + kBT * kBT * E));
      if (!unused) copy16_to_lds(ri, dst + IMG + at, lane * 16, q * 1024);
    }
  };
  // the direct loads copy_chunk issues (compile-time count)
  constexpr int NDMA = [] {
    int n = NVL;
    for (int q = 0; q < NIMG; ++q) {
      const int at = SH::SKIP + q * 1024;
      n += !(!OUT && ((at >= SH::I.Q && at < SH::I.Q + kBT * DK * SH::E) ||
                      (at >= SH::I.MM && at < SH::I.MM + kBT * kBT * SH::E)));
    }
    return n;
  }();

  // ---------------------------------------------------------- LDS patterns
  // per-lane byte addresses, one set per buffer; immediates add the rest
  uint32_t aK[NBUF][F16 ? NKD : 1];      // A fragment, row tile 0, k-step s (K; Q at +I.Q - I.K)
  uint32_t aT[NBUF][F16 ? NHT / 2 : 1];  // transposed K^T reads, tile pair t / 2
  uint32_t aV[NBUF];                     // transposed V reads, row tile 0
  uint32_t aP[NBUF][2];                  // Tn fragments, row tile 0, k-step s (M at +I.MM - I.TN)
  uint32_t aS[NBUF];                     // row vectors, rows 4 lg .. 4 lg + 3
  const uint32_t base = lds_addr(smem);
#pragma unroll
  for (int bf = 0; bf < NBUF; ++bf) {
    const uint32_t b0 = base + bf * STAGE;
    if constexpr (F16) {
#pragma unroll
      for (int s = 0; s < NKD; ++s) aK[bf][s] = b0 + tile_off<PK>(lr, 4 * s + lg);
      const int row = 4 * lg + (lr >> 2);
#pragma unroll
      for (int u = 0; u < NHT / 2; ++u) aT[bf][u] = b0 + tile_off<PK>(row, 4 * u + (lr & 3));
#pragma unroll
      for (int s = 0; s < 2; ++s) aP[bf][s] = b0 + IMG + I.TN + tile_off<PT>(lr, 4 * s + lg);
      aS[bf] = b0 + IMG + I.VEC + 16 * lg;
    }
    if constexpr (sizeof(In) == 2) {
      // lane i of a 16-lane group reads row 4 lg + i / 4 at columns
      // 16 w + 4 (i % 4) .. +3 and receives column 16 w + i of 4 rows
      const int row = 4 * lg + (lr >> 2);
      const int col = 16 * w + 4 * (lr & 3);
      aV[bf] = b0 + tile_off<PV>(row, col >> 3) + 2 * (col & 7);
    } else {
      aV[bf] = b0;
    }
  }

  // ---------------------------------------------------------- the state
  f32x4 hacc[NHT];
  if (wk.init && !copier) {
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[t][e] = wk.init[(size_t)(16 * t + lg * 4 + e) * DV + cw + lr];
  } else {
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) hacc[t][e] = wk.init_id && 16 * t + lg * 4 + e == cw + lr ? 1.f : 0.f;
  }

  // ---- operand scale (16-bit inputs).  The fp16 MFMA operands that carry
  // state-side values (H, X, U) are formed from those values times a power
  // of two cs, one per wave: the recurrence is linear in (V, H), so the wave
  // runs on cs V and cs H exactly and divides o and the states it stores by
  // cs.  cs maps the largest |value| of the wave's columns of the initial
  // state and of the first chunk's V into [4, 8) (1 if both are zero), which
  // keeps those operands inside fp16's normal range whatever the input scale.
  float cs = 1.f, ics = 1.f;
  float osc = p.scale;  // o = p.scale * (cs-scaled result) / cs

  int off_o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) off_o[e] = (lg * 4 + e) * rs_o + (cw + lr) * osz;
  char *o_c = static_cast<char *>(p.o) + ((size_t)wk.t0 * H + h) * DV * osz;
  const size_t o_step = (size_t)kBT * H * DV * osz;
  // 16-bit inputs form the output tile transposed (O^T, see below): lane
  // (g, n) of row tile R holds row 16 R + n at this wave's columns 4 g ..
  // 4 g + 3, stored as one 16-byte (fp32) or 8-byte (bf16) piece
  const int off_ot = lr * rs_o + (cw + 4 * lg) * osz;
  auto store_ot = [&](int R, int C, const f32x4 &oa) {
    const auto ro = buffer_rsrc(o_c + (size_t)16 * R * rs_o, (C - 16 * R) * rs_o);
    if (p.o_bf16) {
      const uint32_t w0 = f32_to_bf16_rne(osc * oa[0]) | (f32_to_bf16_rne(osc * oa[1]) << 16);
      const uint32_t w1 = f32_to_bf16_rne(osc * oa[2]) | (f32_to_bf16_rne(osc * oa[3]) << 16);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, ro, off_ot, 0, 0);
    } else {
      const f32x4 v = {osc * oa[0], osc * oa[1], osc * oa[2], osc * oa[3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, off_ot, 0, 0);
    }
  };
  (void)store_ot;
  // 4 output rows of a row tile: fp32, or bf16 rounded to nearest even
  auto store_o = [&](int R, int C, const f32x4 &oa) {
    const auto ro = buffer_rsrc(o_c + (size_t)16 * R * rs_o, (C - 16 * R) * rs_o);
    if (p.o_bf16) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(osc * oa[e]), ro,
                                              off_o[e], 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(osc * oa[e]), ro, off_o[e], 0, 0);
    }
  };

  // ---------------------------------------------------------- one chunk
  // buffer BUF holds chunk jj; the copy of the next chunk, if any, goes to
  // the other buffer and is issued after the V reads
  // The copier and the compute waves run separate loops with the same
  // barriers.  At the barrier opening chunk jj the copier's loads of chunk
  // jj have landed and every compute wave is done with chunk jj - 1, whose
  // buffer (two buffers) the copier then refills with chunk jj + 1.  Every
  // LDS read of a compute wave is waited for inside its chunk, so that
  // barrier needs no fence, and the compute waves' output stores stay in
  // flight across it.
  auto chunk_barrier = [&]() {
    if constexpr (NBUF == 2) barrier_lds();
    else __syncthreads();
  };
  auto copy_step = [&](int jj) {
    const int r0 = wk.t0 + (jj - j0) * kBT;
    const bool more = jj + 1 < j1;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    chunk_barrier();
    if (NBUF == 2 && more) copy_chunk(1 - ((jj - j0) & 1), img_c + img_step, v_c + v_step, min(kBT, eos - r0 - kBT));
    if constexpr (NBUF == 1) {
      __syncthreads();  // the compute waves are done with the buffer
      if (more) copy_chunk(0, img_c + img_step, v_c + v_step, min(kBT, eos - r0 - kBT));
    }
    img_c += img_step;
    v_c += v_step;
  };
  auto chunk = [&](auto bufc, int jj) {
    constexpr int BUF = decltype(bufc)::value;
    const int r0 = wk.t0 + (jj - j0) * kBT;
    const int C = min(kBT, eos - r0);
    chunk_barrier();
    if (p.hsave) {  // the state entering chunk jj (backward recompute)
      float *hs = p.hsave + ((size_t)jj * H + h) * DK * DV;
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) hs[(size_t)(16 * t + lg * 4 + e) * DV + cw + lr] = hacc[t][e] * ics;
    }
    const char *buf = smem + BUF * STAGE;
    const char *tV = buf;
    const char *tK = buf + IMG + I.K;
    const char *tQ = buf + IMG + I.Q;
    const char *tKT = buf + IMG + I.KT;
    const char *tTN = buf + IMG + I.TN;
    const char *tMM = buf + IMG + I.MM;
    const float *sv = reinterpret_cast<const float *>(buf + IMG + I.VEC);

    // ---- K H and Q H, the state as B operand straight from its accumulators
    typename O::Frag hb[NKD];
#pragma unroll
    for (int s = 0; s < NKD; ++s) hb[s] = b_frag<O>(hacc, s);
    f32x4 yk[4], yq[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      yk[R] = zero4();
      yq[R] = zero4();
    }
    if constexpr (F16) {
      // the 8 fragments of k-step s are read two k-steps ahead
      half8 fr[NKD][8];
      auto read_step = [&](auto sc) {
        constexpr int s = decltype(sc)::value;
        static_for<4>([&](auto rc) {
          constexpr int R = decltype(rc)::value;
          ds_read_b128_at<IMG + I.K + R * 256 * PK>(fr[s][2 * R], aK[BUF][s]);
          if constexpr (OUT) ds_read_b128_at<IMG + I.Q + R * 256 * PK>(fr[s][2 * R + 1], aK[BUF][s]);
        });
      };
      read_step(std::integral_constant<int, 0>{});
      if constexpr (NKD > 1) read_step(std::integral_constant<int, 1>{});
      static_for<NKD>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        auto &f = fr[s];
        if constexpr (OUT) {
          if constexpr (s + 1 < NKD) wait_lds_tied8<8>(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
          else wait_lds_tied8<0>(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
        } else {
          if constexpr (s + 1 < NKD) wait_lds_tied4<4>(f[0], f[2], f[4], f[6]);
          else wait_lds_tied4<0>(f[0], f[2], f[4], f[6]);
        }
        if constexpr (s + 2 < NKD) read_step(std::integral_constant<int, s + 2>{});
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          yk[R] = O::mfma(f[2 * R], hb[s], yk[R]);
          // (Q H)^T: the state fragment as A, the Q fragment as B
          if constexpr (OUT) yq[R] = O::mfma(hb[s], f[2 * R + 1], yq[R]);
        }
      });
    } else {
#pragma unroll
      for (int s = 0; s < NKD; ++s)
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          yk[R] = O::mfma(a_frag_img<O, PK>(tK, 16 * R, s, lane), hb[s], yk[R]);
          if constexpr (OUT) yq[R] = O::mfma(a_frag_img<O, PK>(tQ, 16 * R, s, lane), hb[s], yq[R]);
        }
    }

    // ---- X = V - gamma (K H); U = beta X + Tn X; O = scale (gamma (Q H) + M U).
    // V rows past the chunk's end were staged as zero; output rows past it
    // are dropped by the range check of the per-tile output resource.
    f32x4 gam[4], x[4];
    typename O::Frag ufr[NKR], ubf[NKR];
    s16x4 tr[F16 && !HAS_KT ? NHT : 1][4];
    float gdec = 0.f;
    if constexpr (F16) {
      // Every LDS read of these phases is issued ahead of its first use as
      // inline assembly and waited for with its registers tied (LDS
      // operations complete in order): V, gamma and the six Tn fragments;
      // beta, the update factors and the state decay while X forms; the six
      // M fragments while U's products run; the K^T reads of the update in
      // two halves around the output.  Fragment i of Tn and M is
      // (row tile, k-step) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
      constexpr auto fR = [](int i) { return i < 2 ? i : (i + 2) / 2; };
      constexpr auto fS = [](int i) { return i < 2 ? 0 : (i & 1); };
      constexpr int DMM = I.MM - I.TN;
      s16x4 vr[4];
      half8 ft[6], fm[6];
      f32x4 bet[4], fac[4], dcv;
      static_for<4>([&](auto rc) {
        constexpr int R = decltype(rc)::value;
        ds_read_tr16_at<R * 256 * PV>(vr[R], aV[BUF]);
      });
      static_for<4>([&](auto rc) {
        constexpr int R = decltype(rc)::value;
        ds_read_b128_at<64 * R>(gam[R], aS[BUF]);
      });
      static_for<6>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        ds_read_b128_at<fR(i) * 256 * PT>(ft[i], aP[BUF][fS(i)]);
      });
      wait_lds_tied<6>(vr[0], vr[1], vr[2], vr[3]);
      wait_lds_tied4<6>(gam[0], gam[1], gam[2], gam[3]);
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[R][e] = fmaf(in16_to_f32<In>((uint16_t)vr[R][e]), cs, -gam[R][e] * yk[R][e]);
      static_for<4>([&](auto rc) {
        constexpr int R = decltype(rc)::value;
        ds_read_b128_at<512 + 64 * R>(bet[R], aS[BUF]);
        if constexpr (!KDA) ds_read_b128_at<256 + 64 * R>(fac[R], aS[BUF]);
      });
      if constexpr (!HAS_KT) ds_read_b128_at<768>(dcv, aS[BUF]);
      constexpr int AFTER_TN = (KDA ? 4 : 8) + (HAS_KT ? 0 : 1);
      typename O::Frag xb[NKR];
#pragma unroll
      for (int s = 0; s < NKR; ++s) xb[s] = b_frag<O>(x, s);
      wait_lds_tied2<AFTER_TN>(ft[0], ft[1]);
      wait_lds_tied4<AFTER_TN>(ft[2], ft[3], ft[4], ft[5]);
      f32x4 u[4], ub[4];
#pragma unroll
      for (int R = 0; R < 4; ++R) u[R] = zero4();
      static_for<6>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        u[fR(i)] = O::mfma(ft[i], xb[fS(i)], u[fR(i)]);
      });
      constexpr int NM = OUT ? 6 : 0;  // M fragments in flight
      if constexpr (OUT)
        static_for<6>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          ds_read_b128_at<DMM + fR(i) * 256 * PT>(fm[i], aP[BUF][fS(i)]);
        });
      wait_lds_tied4<NM>(bet[0], bet[1], bet[2], bet[3]);
      if constexpr (!KDA) wait_lds_tied4<NM>(fac[0], fac[1], fac[2], fac[3]);
      if constexpr (!HAS_KT) {
        wait_lds_tied1<NM>(dcv);
        gdec = dcv[0];
      }
#pragma unroll
      for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[R][e] += bet[R][e] * x[R][e];
        if constexpr (!KDA)
#pragma unroll
          for (int e = 0; e < 4; ++e) ub[R][e] = fac[R][e] * u[R][e];
      }
#pragma unroll
      for (int s = 0; s < NKR; ++s) {
        ufr[s] = b_frag<O>(u, s);
        if constexpr (KDA) ubf[s] = ufr[s];
        else ubf[s] = b_frag<O>(ub, s);
      }
      if constexpr (OUT) {
        wait_lds_tied2<0>(fm[0], fm[1]);
        wait_lds_tied4<0>(fm[2], fm[3], fm[4], fm[5]);
      }
      // the transposed K^T reads of the update (GDN), first half
      auto read_kt = [&](auto t0c) {
        constexpr int T0 = decltype(t0c)::value;
        static_for<NHT / 2>([&](auto tc) {
          constexpr int t = T0 + decltype(tc)::value;
          static_for<4>([&](auto qc) {
            constexpr int q = decltype(qc)::value;  // (k-step, half) = (q / 2, q % 2)
            constexpr int OFF = IMG + I.K + (32 * (q >> 1) + 16 * (q & 1)) * 16 * PK + 8 * (t & 1);
            ds_read_tr16_at<OFF>(tr[t][q], aT[BUF][t >> 1]);
          });
        });
      };
      if constexpr (!HAS_KT) {
        static_assert(NKR == 2, "two k-steps over the chunk rows");
        read_kt(std::integral_constant<int, 0>{});
      }
      if constexpr (OUT) {
        // O^T = (Q H)^T diag(gamma) + U^T M^T: U's B fragments serve as A
        // fragments of U^T and M's A fragments as B fragments of M^T.  Lane
        // (g, n) scales by the gamma of its row 16 R + n, which lane 16 (n /
        // 4) + n % 4 holds as element n % 4 of gam[R].
        const int gsrc = 16 * (lr >> 2) + (lr & 3);
        f32x4 oa[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const float pub = (lr & 2) ? ((lr & 1) ? gam[R][3] : gam[R][2]) : ((lr & 1) ? gam[R][1] : gam[R][0]);
          const float gt = __shfl(pub, gsrc, 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) oa[R][e] = gt * yq[R][e];
        }
        static_for<6>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          oa[fR(i)] = O::mfma(ufr[fS(i)], fm[i], oa[fR(i)]);
        });
        if constexpr (!HAS_KT) read_kt(std::integral_constant<int, NHT / 2>{});
#pragma unroll
        for (int R = 0; R < 4; ++R) store_ot(R, C, oa[R]);
      } else {
        if constexpr (!HAS_KT) read_kt(std::integral_constant<int, NHT / 2>{});
      }
    } else {
      const int col = 16 * w + lr;
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        gam[R] = *reinterpret_cast<const f32x4 *>(sv + 16 * R + lg * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * R + 4 * lg + e;
          const float v = *reinterpret_cast<const float *>(tV + tile_off<PV>(row, col >> 2) + 4 * (col & 3));
          x[R][e] = v - gam[R][e] * yk[R][e];
        }
      }
      typename O::Frag xb[NKR];
#pragma unroll
      for (int s = 0; s < NKR; ++s) xb[s] = b_frag<O>(x, s);
      f32x4 u[4], ub[4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        const f32x4 bet = *reinterpret_cast<const f32x4 *>(sv + 128 + 16 * R + lg * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[R][e] = bet[e] * x[R][e];
#pragma unroll
        for (int s = 0; s < ksteps_lower<O>(R); ++s)
          u[R] = O::mfma(a_frag_img<O, PT>(tTN, 16 * R, s, lane), xb[s], u[R]);
        if constexpr (!KDA) {
          const f32x4 fac = *reinterpret_cast<const f32x4 *>(sv + 64 + 16 * R + lg * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) ub[R][e] = fac[e] * u[R][e];
        }
      }
#pragma unroll
      for (int s = 0; s < NKR; ++s) {
        ufr[s] = b_frag<O>(u, s);
        if constexpr (KDA) ubf[s] = ufr[s];
        else ubf[s] = b_frag<O>(ub, s);
      }
#pragma unroll
      for (int R = 0; R < 4 && OUT; ++R) {
        f32x4 oa;
#pragma unroll
        for (int e = 0; e < 4; ++e) oa[e] = gam[R][e] * yq[R][e];
#pragma unroll
        for (int s = 0; s < ksteps_lower<O>(R); ++s)
          oa = O::mfma(a_frag_img<O, PT>(tMM, 16 * R, s, lane), ufr[s], oa);
        store_o(R, C, oa);
      }
    }

    // ---- H <- decay H + Kbar^T Ubar
    if constexpr (HAS_KT) {
#pragma unroll
      for (int t = 0; t < NHT; ++t) {
        const f32x4 dec = *reinterpret_cast<const f32x4 *>(sv + 192 + 16 * t + lg * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[t][e] *= dec[e];
#pragma unroll
        for (int s = 0; s < NKR; ++s)
          hacc[t] = O::mfma(a_frag_img<O, PT>(tKT, 16 * t, s, lane), ubf[s], hacc[t]);
      }
    } else {
      static_for<NHT>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        // outstanding after tile t's reads: those of the later tiles
        constexpr int LATER = 4 * (NHT - 1 - t) < 15 ? 4 * (NHT - 1 - t) : 15;
        wait_lds_tied<LATER>(tr[t][0], tr[t][1], tr[t][2], tr[t][3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[t][e] *= gdec;
#pragma unroll
        for (int s = 0; s < NKR; ++s)
          hacc[t] = O::mfma(join_half8(tr[t][2 * s], tr[t][2 * s + 1]), ubf[s], hacc[t]);
      });
    }

    // ---- single buffer: the copier refills it once every wave is done
    if constexpr (NBUF == 1) __syncthreads();
    o_c += o_step;
  };

  // ---------------------------------------------------------- chunk loop
  if constexpr (RAW) {
    if (copier) {
      // Two copy waves.  Wave NW stages V and the image (from Tn on) by
      // direct loads and K from the raw rows of k; wave NW + 1 stages Q from
      // the raw rows of q (when there is output).  Raw rows are loaded two
      // chunks ahead into registers and converted to fp16 in the chained k
      // order one chunk ahead, into the buffer the compute waves will read
      // next.  Unit i of a lane: row r, 32-element block b, half g2: input
      // pieces 4b + g2 and 4b + 2 + g2 hold the chained pieces 4b + 2 g2
      // (their low halves) and 4b + 2 g2 + 1 (their high halves).  Loads past
      // the sequence run over empty ranges (zeros, no memory traffic), so the
      // counts the vmcnt waits rely on stay fixed.
      const int cpw = w - NW;
      const bool active = cpw == 0 || OUT;
      constexpr int NU = DK / 16, UPR = DK / 16;  // units per lane, per row
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
      auto chunk_rows = [&](int jj) { return jj < j1 ? min(kBT, eos - (wk.t0 + (jj - j0) * kBT)) : 0; };
      auto load_raw = [&](auto rc, int jj) {
        constexpr int RB = decltype(rc)::value;
        const int C = active ? chunk_rows(jj) : 0;
        const auto rr = buffer_rsrc(src_c + (size_t)(jj - j0) * src_step, C * rs_q);
#pragma unroll
        for (int i = 0; i < NU; ++i) {
          raw[RB][i][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, roff0[i], 0, 0));
          raw[RB][i][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, roff1[i], 0, 0));
        }
      };
      auto put_raw = [&](auto rc, int buf) {
        constexpr int RB = decltype(rc)::value;
        if (!active) return;
        const uint32_t b0 = base + buf * STAGE;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
          const u32x4 &a = raw[RB][i][0], &c = raw[RB][i][1];
          const u32x4 lo = {to_f16x2<In>(a[0]), to_f16x2<In>(a[1]), to_f16x2<In>(c[0]), to_f16x2<In>(c[1])};
          const u32x4 hi = {to_f16x2<In>(a[2]), to_f16x2<In>(a[3]), to_f16x2<In>(c[2]), to_f16x2<In>(c[3])};
          ds_write_b128(b0 + loff[i], lo);
          ds_write_b128(b0 + (loff[i] ^ 16u), hi);
        }
      };
      // direct loads of chunk jj into buffer buf (wave NW only)
      auto dma = [&](int buf, int jj) {
        if (cpw != 0) return;
        copy_chunk(buf, img_c + (size_t)(jj - j0) * img_step, v_c + (size_t)(jj - j0) * v_step,
                   chunk_rows(jj));
      };
      constexpr int NR = 2 * NU;  // raw loads per chunk
      auto run = [&](auto cpc) {
        constexpr int CP = decltype(cpc)::value;
        constexpr int ND = CP == 0 ? NDMA : 0;
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
        put_raw(std::integral_constant<int, 0>{}, 0);
        wait_vm<NR>();       // direct loads of j0
        wait_lgkm<0>();
        chunk_barrier();     // the first chunk's stage has landed in buffer 0
        // chunk jj: buffer and register set B hold it; the next chunk goes
        // to the other buffer once every compute wave is done with it
        auto step = [&](auto bc, int jj) {
          constexpr int B = decltype(bc)::value;
          chunk_barrier();  // opens chunk jj: chunk jj - 1's buffer is free
          issue_fence();
          dma(1 - B, jj + 1);
          issue_fence();
          load_raw(std::integral_constant<int, B>{}, jj + 2);
          issue_fence();
          wait_vm<ND + NR>();  // raw rows of jj + 1
          put_raw(std::integral_constant<int, 1 - B>{}, 1 - B);
          wait_vm<NR>();       // direct loads of jj + 1
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
      return;
    }
  }
  if (copier) {
    copy_chunk(0, img_c, v_c, min(kBT, eos - wk.t0));
    if constexpr (F16) {  // the compute waves read the first chunk's V for cs
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      chunk_barrier();
    }
    for (int jj = j0; jj < j1; ++jj) copy_step(jj);
    return;
  }
  if constexpr (F16) {
    chunk_barrier();  // the first chunk's stage has landed in buffer 0
    s16x4 v0[4];
    static_for<4>([&](auto rc) {
      constexpr int R = decltype(rc)::value;
      ds_read_tr16_at<R * 256 * PV>(v0[R], aV[0]);
    });
    wait_lds_tied<0>(v0[0], v0[1], v0[2], v0[3]);
    float m = 0.f;
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(in16_to_f32<In>((uint16_t)v0[R][e])));
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(hacc[t][e]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (m > 0.f && m <= 3.0e38f) {
      int ex;
      (void)frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
      const int k = min(max(3 - ex, -100), 100);
      cs = ldexpf(1.f, k);
      ics = ldexpf(1.f, -k);
      osc = p.scale * ics;
#pragma unroll
      for (int t = 0; t < NHT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) hacc[t][e] *= cs;
    }
  }
  // two chunks per trip, one per buffer; leaving through the breaks keeps a
  // single path into the loop header, so the state accumulators keep their
  // registers from trip to trip
  for (int jj = j0;;) {
    chunk(std::integral_constant<int, 0>{}, jj);
    if (++jj == j1) break;
    chunk(std::integral_constant<int, NBUF == 2 ? 1 : 0>{}, jj);
    if (++jj == j1) break;
  }

  // ---- final state slice: fp32, or the fp16 hi / lo images of a segment's
  // transition (element (r, c) at the place an A fragment of a [d_k][d_k]
  // operand with chained columns expects it: row r, column kpos(c))
  if (wk.fin) {
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) wk.fin[(size_t)(16 * t + lg * 4 + e) * DV + cw + lr] = hacc[t][e] * ics;
  }
  if (wk.pimg) {
    constexpr int PP = DK * 2 / 16;  // 16-byte pieces per fp16 row
    const int kc = kpos<Op<bf16>>(cw + lr);
#pragma unroll
    for (int t = 0; t < NHT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * t + lg * 4 + e;
        const int off = (tile_off<PP>(r, kc >> 3) >> 1) + (kc & 7);
        const float hv = hacc[t][e] * ics;
        const _Float16 hi = (_Float16)hv;
        wk.pimg[off] = hi;
        wk.pimg[DK * DK + off] = (_Float16)(hv - (float)hi);
      }
  }
}

template <bool KDA, typename In, int DK, int NW, bool RAW>
__global__ __launch_bounds__(64 * (NW + 1 + (RAW ? 1 : 0))) void chunk_reduce_kernel(ReduceParams p) {
  using SH = ReduceShape<KDA, In, DK, NW, RAW>;
  __shared__ __attribute__((aligned(16))) char smem[SH::NBUF * SH::STAGE];
  Work wk;
  const int role = decode_work<DK, SH::W>(p, wk);
  if (role == 1) reduce_body<KDA, In, DK, NW, true, RAW>(p, wk, smem);
  else if (role == 2) reduce_body<KDA, In, DK, NW, false, RAW>(p, wk, smem);
}

}  // namespace

template <bool KDA, typename In, int DK, int NW, bool RAW = false>
static hipError_t launch_reduce_t(const ReduceParams &p, hipStream_t st) {
  using SH = ReduceShape<KDA, In, DK, NW, RAW>;
  const int units = (p.seg ? p.NS_max : p.N_max) * p.H;
  const int grid = ((units + 7) / 8) * 8 * (p.pass == 1 ? p.S + p.SP : p.S);
  hipLaunchKernelGGL((chunk_reduce_kernel<KDA, In, DK, NW, RAW>), dim3(grid), dim3(SH::THREADS), 0, st,
                     p);
  return hipGetLastError();
}

template <bool KDA, typename In, int DK>
static hipError_t launch_reduce_w(const ReduceParams &p, int W, hipStream_t st) {
  // raw K / Q staging: 16-bit GDN at 64 columns
  if (p.raw_kq) {
    if constexpr (!KDA && sizeof(In) == 2) {
      if (W == 64) return launch_reduce_t<KDA, In, DK, 4, true>(p, st);
    }
    return hipErrorInvalidValue;
  }
  switch (W) {
    case 32: return launch_reduce_t<KDA, In, DK, 2>(p, st);
    case 64: return launch_reduce_t<KDA, In, DK, 4>(p, st);
    case 128:
      if constexpr (DK >= 128) return launch_reduce_t<KDA, In, DK, 8>(p, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename In>
static hipError_t launch_reduce_16(const ReduceParams &p, bool kda, int dk, int W, hipStream_t st) {
  if (dk == 128)
    return kda ? launch_reduce_w<true, In, 128>(p, W, st) : launch_reduce_w<false, In, 128>(p, W, st);
  if (dk == 64)
    return kda ? launch_reduce_w<true, In, 64>(p, W, st) : launch_reduce_w<false, In, 64>(p, W, st);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_reduce(const ReduceParams &p, bool kda, int dt, int dk, int W,
                               hipStream_t st) {
  if (dt == LA_BF16) return launch_reduce_16<bf16>(p, kda, dk, W, st);
  if (dt == LA_F16) return launch_reduce_16<f16>(p, kda, dk, W, st);
  if (dt != LA_F32 || dk != 64) return hipErrorInvalidValue;
  return kda ? launch_reduce_w<true, float, 64>(p, W, st) : launch_reduce_w<false, float, 64>(p, W, st);
}

}  // namespace la
