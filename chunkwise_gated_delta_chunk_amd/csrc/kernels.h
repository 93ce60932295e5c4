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
  void *img;
};

struct ReduceParams {
  const void *v;
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

// cu: int32 cu_seqlens, or int64 with cu64
hipError_t launch_chunk_meta(const void *cu, int cu64, int N_max, int T_max, int BT, int NT_max,
                             int32_t *ci, int32_t *co, int32_t *status, hipStream_t stream);
// dt: la_dtype code of q, k, v (LA_BF16, LA_F32, LA_F16)
hipError_t launch_chunk_map(const MapParams &p, bool kda, int dt, int dk, hipStream_t st);
// W = d_v / S columns per workgroup: 32 per wave
hipError_t launch_chunk_reduce(const ReduceParams &p, bool kda, int dt, int dk, int W,
                               hipStream_t st);
hipError_t launch_chunk_combine(const CombineParams &p, int dk, hipStream_t st);
hipError_t launch_recurrent(const RecurrentParams &p, bool kda, int dt, int dk, hipStream_t st);
// NT chunk slots, W in 1..4
hipError_t launch_short_conv(const ConvParams &p, int dt, int NT, int W, bool silu,
                             hipStream_t st);

}  // namespace la
