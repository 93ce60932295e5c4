// Launch parameters and host launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_device.h"

namespace la {

// Workspace element type of the map results: fp16 for bf16 inputs, fp32 for
// fp32 inputs.  Kernels reinterpret the void pointers accordingly.
struct MapParams {
  const void *q, *k;
  const float *g, *beta;
  const int32_t *cu_seqlens, *chunk_indices;
  int H, NT_max;
  void *Tn_raw, *M_raw;
};

struct ReduceParams {
  const void *q, *k, *v;
  const float *g, *beta;
  const int32_t *cu_seqlens, *chunk_offsets;
  const float *h0;
  float *o, *ht;
  const void *Tn_raw, *M_raw;
  int H, N_max, S;  // S = d_v slices per (sequence, head)
  float scale;
};

hipError_t launch_chunk_meta(const int32_t *cu, int N_max, int T_max, int BT, int NT_max,
                             int32_t *ci, int32_t *co, int32_t *status, hipStream_t stream);
hipError_t launch_chunk_map(const MapParams &p, bool kda, bool bf16_in, int dk, hipStream_t st);
hipError_t launch_chunk_reduce(const ReduceParams &p, bool kda, bool bf16_in, int dk, int W,
                               hipStream_t st);

}  // namespace la
