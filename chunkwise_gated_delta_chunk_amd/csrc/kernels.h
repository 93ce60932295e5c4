// Launch parameters and host launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_device.h"
#include "../../include/linattn.h"

namespace la {

// The map stage writes one image per (chunk slot, head) to the workspace
// (layout: image_layout in la_device.h), the reduce copies it into LDS.
struct MapParams {
  const void *q, *k;
  const float *g, *beta;
  const void *cu_seqlens;  // int32, or int64 with cu64
  const int32_t *chunk_indices;
  int cu64;
  int H, NT_max;
  int Hqk;  // q, k heads: value head h reads q, k head h / (H / Hqk)
  int raw_kq;  // GDN, 16-bit: the reduce stages K and Q itself (no K, Q stored)
  void *img;
  // fuse_meta (N_max <= 64): the kernel derives the chunk layout from
  // cu_seqlens itself (chunk_indices unread) and stores it as build_chunk_meta
  // does at BT = 64: meta_ci [NT_max][2], meta_co [N_max+1], meta_status
  // (optional)
  int fuse_meta, N_max, T_max;
  int32_t *meta_ci, *meta_co, *meta_status;
};

struct ReduceParams {
  const void *v;
  // 16-bit GDN: the raw q, k rows ([T][Hqk][d_k]), staged by the reduce itself
  // (always at 32 columns; at 64 columns when raw_kq is set)
  const void *q_raw, *k_raw;
  int Hqk;
  int raw_kq;
  const void *cu_seqlens;  // int32, or int64 with cu64
  const int32_t *chunk_offsets;
  int cu64;
  const float *h0;
  void *o;       // fp32, or bf16 with o_bf16
  float *ht;
  const void *img;
  int H, N_max, S;  // S = d_v slices per (sequence, head)
  float scale;
  int o_bf16;
  // sequence-parallel reduce (chunk_reduce.hip): seg = chunks per segment
  // (0: one workgroup walks a whole sequence), pass 1 or 2, SP = d_k slices
  // of the transitions, NS_max segment slots; per (segment slot, head):
  // hin, dlt [d_k][d_v] fp32 and pimg 2 x [d_k][d_k] fp16
  int seg, pass, SP, NS_max;
  float *hin, *dlt;
  _Float16 *pimg;
  // one-pass reduce only: when set, the state at the start of every chunk is
  // stored to hsave[slot][h] ([d_k][d_v] fp32, the backward's recompute);
  // o may then be NULL (no output)
  float *hsave;
};

// Segment combine: H_{s+1} = P_s H_s + D_s along each sequence's segments.
struct CombineParams {
  const int32_t *chunk_offsets;
  int H, N_max, seg;
  float *hin;
  const float *dlt;
  const _Float16 *pimg;
};

// One recurrent step per (sequence, head) unit (recurrent.hip).
struct RecurrentParams {
  const void *q, *k, *v;
  const float *g, *beta, *h0;
  void *o;       // fp32, or bf16 with o_bf16
  float *ht;
  int units;     // N * H
  int H, Hqk;    // value heads, q / k heads
  float scale;
  int o_bf16;
};

// Varlen causal short convolution (short_conv.hip): x, res, y and the states
// in the input dtype; w [D][W], b [D] fp32; states [N_max][W-1][D].
struct ConvParams {
  const void *x, *res, *h0;
  const float *w, *b;
  const void *cu_seqlens;  // int32, or int64 with cu64
  const int32_t *chunk_indices;
  int cu64, D, BT;
  void *y, *ht;
};

// Chunk backward (chunk_bwd.hip).  prep: per (slot, head) cell, kPrepFloats
// fp32: A^-1, M, S ([64][64] each), then G, exp(G), exp(G_C - G), beta (64
// each).  part: per cell, part_floats(d) fp32: dOb H^T, dX H^T, U dH'^T
// ([64][d] each), dM, dT ([64][64] each), <dH', H>.  hs / dhs: per cell the
// state entering / the state gradient leaving the chunk, [d][d] fp32.
constexpr int kPrepA = 0, kPrepM = 4096, kPrepS = 8192, kPrepG = 12288, kPrepGam = 12352,
              kPrepFac = 12416, kPrepBeta = 12480;
// then, for bf16 inputs, bf16 high and low halves of M and of
// A^-1 diag(beta), row-major [64][64] each, in the order M hi, M lo,
// A^-1 diag(beta) hi, lo, from float offset kPrepH
constexpr int kPrepH = 12544, kPrepFloats = kPrepH + 4 * 4096 / 2;
constexpr int kPartP1 = 0;
__host__ __device__ constexpr int part_p2(int d) { return 64 * d; }
__host__ __device__ constexpr int part_p3(int d) { return 128 * d; }
__host__ __device__ constexpr int part_dm(int d) { return 192 * d; }
__host__ __device__ constexpr int part_dt(int d) { return 192 * d + 4096; }
__host__ __device__ constexpr int part_sh(int d) { return 192 * d + 8192; }
// (KDA: the <dH', H> term is a vector over the d_k rows, at part_sh)
__host__ __device__ constexpr int part_floats(int d) { return 192 * d + 8192 + 256; }
// KDA prep cell: A^-1, M, S ([64][64] each), beta (64), the per-channel
// cumulative gate G ([64][d]), then for bf16 inputs bf16 high and low halves
// of M and of A^-1 diag(beta), row-major [64][64] each (M hi, M lo, hi, lo)
constexpr int kKdaBeta = 12288, kKdaG = 12352;
__host__ __device__ constexpr int kda_halves(int d) { return kKdaG + 64 * d; }
__host__ __device__ constexpr int kda_prep_floats(int d) { return kda_halves(d) + 4 * 4096 / 2; }

struct BwdParams {
  const void *q, *k, *v;
  const float *g, *beta;
  const void *cu_seqlens;  // int32, or int64 with cu64
  const int32_t *chunk_indices, *chunk_offsets;
  const float *dout, *dht;
  float *dq, *dk, *dv, *dg, *dbeta, *dh0;
  float *prep, *part, *hs, *dhs;
  int cu64, H, N_max, NT;
  int Hqk;  // q, k heads: value head h reads (and its dq, dk belong to) head h / (H / Hqk)
  float scale;
};

// cu: int32 cu_seqlens, or int64 with cu64
hipError_t launch_chunk_meta(const void *cu, int cu64, int N_max, int T_max, int BT, int NT_max,
                             int32_t *ci, int32_t *co, int32_t *status, hipStream_t stream);
// dt: la_dtype code of q, k, v (LA_BF16, LA_F32, LA_F16)
hipError_t launch_chunk_map(const MapParams &p, bool kda, int dt, int dk, hipStream_t st);
// W = d_v / S columns per workgroup (16 per compute wave); full images
hipError_t launch_chunk_reduce(const ReduceParams &p, bool kda, int dt, int dk, int W,
                               hipStream_t st);
// 16-bit inputs (bf16, fp16), W = 32 columns per workgroup; GDN stages K and
// Q from the raw rows (the map's images start at TN)
hipError_t launch_chunk_reduce16(const ReduceParams &p, bool kda, int dt, int dk, int W,
                                 hipStream_t st);
hipError_t launch_chunk_combine(const CombineParams &p, int dk, hipStream_t st);
hipError_t launch_recurrent(const RecurrentParams &p, bool kda, int dt, int dk, hipStream_t st);
// stage 1: prep; stage 2: the reverse pass (both need only q, k, g, beta,
// dout and dht); stage 3: the per-chunk kernels, after stage 2 and the
// forward recompute
hipError_t launch_chunk_bwd(const BwdParams &p, int dt, int dk, int stage, hipStream_t st);
hipError_t launch_chunk_bwd_kda(const BwdParams &p, int dt, int dk, int stage, hipStream_t st);
// grouped value heads: out[t][hq] = sum of full[t][h] over the value heads h
// of group hq, rows of real tokens only
hipError_t launch_group_sum(const float *full, float *out, int T_max, int H, int Hqk, int d,
                            const void *cu, int cu64, int N_max, const int32_t *co,
                            hipStream_t st);
// NT chunk slots, W in 1..4
hipError_t launch_short_conv(const ConvParams &p, int dt, int NT, int W, bool silu,
                             hipStream_t st);

}  // namespace la
