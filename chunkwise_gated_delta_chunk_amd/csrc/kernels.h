// Launch parameters and host launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_device.h"

namespace la {

// Map-stage results in the workspace, per (chunk slot, head), element type T
// (fp16 for bf16 inputs, fp32 for fp32 inputs):
//   Tn, M  [64][64]  columns in chained k order (kpos)
//   vec    [192 + d_k] fp32: exp(G_r) | exp(G_C - G_r) | beta_r | state decay
// and for KDA
//   Kd, Qd [64][d_k]  K*exp(G), Q*exp(G), key index in chained order
//   Kbt    [d_k][64]  (K*exp(G_C - G))^T, chunk rows in chained order
struct MapParams {
  const void *q, *k;
  const float *g, *beta;
  const int32_t *cu_seqlens, *chunk_indices;
  int H, NT_max;
  void *Tn_raw, *M_raw;
  float *vec;
  void *Kd_raw, *Qd_raw, *Kbt_raw;
};

struct ReduceParams {
  const void *q, *k, *v;
  const int32_t *cu_seqlens, *chunk_offsets;
  const float *h0;
  float *o, *ht;
  const void *Tn_raw, *M_raw;
  const float *vec;
  const void *Kd_raw, *Qd_raw, *Kbt_raw;
  int H, N_max, S;  // S = d_v slices per (sequence, head)
  float scale;
};

hipError_t launch_chunk_meta(const int32_t *cu, int N_max, int T_max, int BT, int NT_max,
                             int32_t *ci, int32_t *co, int32_t *status, hipStream_t stream);
hipError_t launch_chunk_map(const MapParams &p, bool kda, bool bf16_in, int dk, hipStream_t st);
// W = d_v / S columns per workgroup: 16 per wave
hipError_t launch_chunk_reduce(const ReduceParams &p, bool kda, bool bf16_in, int dk, int W,
                               hipStream_t st);

}  // namespace la
