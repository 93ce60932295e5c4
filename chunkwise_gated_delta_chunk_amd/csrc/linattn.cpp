// Host side of the C ABI declared in include/linattn.h: argument checks (all
// before anything is enqueued), workspace sizing, split choice and launches.
// No allocation, no synchronisation, no state kept between calls.
#include "../../include/linattn.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr int kBTSupported = 64;
// rows per chunk of the chunk kernels; a caller's BT = 32 layout is rebuilt on
// the device at this size (see meta_bytes)
constexpr int kBTk = 64;
constexpr int kCUs = 256;  // compute units of one MI355X

bool known_dtype(int dt) { return dt == LA_BF16 || dt == LA_F16 || dt == LA_F32; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// shape checks shared by the workspace query and the forward calls
int check_shape(const la_chunk_fwd_args *a) {
  if (a->T_max < 1 || a->N_max < 1 || a->H < 1) return LA_ERR_SHAPE;
  if (a->T_max > 0x7fffffff - 2 * kBTSupported) return LA_ERR_SHAPE;
  if (!known_dtype(a->qkv_dtype)) return LA_ERR_DTYPE;
  if (a->o_bf16 != 0 && a->o_bf16 != 1) return LA_ERR_DTYPE;
  if (a->cu_seqlens_i64 != 0 && a->cu_seqlens_i64 != 1) return LA_ERR_DTYPE;
  if (a->H_qk < 0 || (a->H_qk > 0 && a->H % a->H_qk != 0)) return LA_ERR_SHAPE;
  if (a->BT != 32 && a->BT != 64) return LA_ERR_UNSUPPORTED;
  if (a->d_k != a->d_v) return LA_ERR_UNSUPPORTED;
  if (a->qkv_dtype != LA_F32 && a->d_k != 64 && a->d_k != 128) return LA_ERR_UNSUPPORTED;
  if (a->qkv_dtype == LA_F32 && a->d_k != 64) return LA_ERR_UNSUPPORTED;
  // dv_split: 0 (auto) or a power of two leaving 32, 64 or 128 columns
  const int s = a->dv_split;
  if (s != 0 && s != 1 && s != 2 && s != 4) return LA_ERR_UNSUPPORTED;
  if (s != 0 && a->d_v / s < 32) return LA_ERR_UNSUPPORTED;
  // seg_len: -1 (off), 0 (auto) or chunks per segment, 16-bit and N_max <= 64
  if (a->seg_len < -1) return LA_ERR_UNSUPPORTED;
  if (a->seg_len > 0 && (a->qkv_dtype == LA_F32 || a->N_max > 64)) return LA_ERR_UNSUPPORTED;
  // every (token, head) index and (slot, head) workspace index stays in size_t
  const int64_t nt = la_nt_max(a->T_max, a->N_max, kBTk);
  if (nt < 1 || nt > 0x7fffffff) return LA_ERR_SHAPE;
  if ((int64_t)a->N_max * a->H > 0x7fffffff / 8) return LA_ERR_SHAPE;
  if (nt * a->H > 0x7fffffff) return LA_ERR_SHAPE;  // one map workgroup per cell
  // byte offsets inside one chunk of v / o (64 token rows) stay in int
  if ((int64_t)a->H * a->d_v * 4 * 64 > 0x7fffffff) return LA_ERR_SHAPE;
  return LA_OK;
}

int split_for(const la_chunk_fwd_args *a) {
  if (a->dv_split) return a->dv_split;
  // 64 state columns per workgroup; when that leaves at most one workgroup
  // per CU, 32 columns, which run a chunk faster: the sequences' serial
  // chains then bound the time, not the total work
  const int s = a->d_v / 64 > 0 ? a->d_v / 64 : 1;
  if ((int64_t)a->N_max * a->H * s <= kCUs && a->d_v / (2 * s) >= 32) return 2 * s;
  return s;
}

// 16-bit inputs in 32-column slices run the dedicated 16-bit reduce, which
// for GDN stages K and Q from the raw q, k rows (the map then stores no K, Q)
bool reduce16(const la_chunk_fwd_args *a, int S) {
  return a->qkv_dtype != LA_F32 && a->d_v / S == 32;
}

hipError_t launch_reduce(const la::ReduceParams &rp, const la_chunk_fwd_args *a, bool kda,
                         hipStream_t st) {
  const int W = a->d_v / rp.S;
  if (reduce16(a, rp.S)) return la::launch_chunk_reduce16(rp, kda, a->qkv_dtype, a->d_k, W, st);
  return la::launch_chunk_reduce(rp, kda, a->qkv_dtype, a->d_k, W, st);
}

size_t elem_bytes(const la_chunk_fwd_args *a) { return a->qkv_dtype == LA_F32 ? 4 : 2; }

// Chunks per segment of the sequence-parallel reduce, 0 for one workgroup
// per sequence.  Automatic when the (sequence, head) units cannot fill half
// the CUs even at 64 columns per workgroup: about the length that spreads
// the capacity's chunks of all units over the CUs once, at least 8, and only
// where the longest possible sequence then has at least 3 segments.
int seg_for(const la_chunk_fwd_args *a) {
  if (a->seg_len < 0 || a->qkv_dtype == LA_F32 || a->N_max > 64) return 0;
  if (a->seg_len > 0) return a->seg_len;
  const int64_t s2 = a->d_v / 64 > 0 ? a->d_v / 64 : 1;
  if ((int64_t)a->N_max * a->H * s2 > kCUs / 2) return 0;
  const int64_t nt = la_nt_max(a->T_max, a->N_max, kBTk);
  int64_t L = (nt * a->H * s2 + kCUs - 1) / kCUs;
  if (L < 8) L = 8;
  const int64_t longest = (a->T_max + kBTk - 1) / kBTk;
  if (longest < 3 * L) return 0;
  return (int)L;
}

// d_v slices of the segmented passes unless dv_split is given: 32 columns
// (a faster chunk) while the first pass then has at most two workgroups per
// CU (d_v / 32 output or D slices and d_k / 32 P slices per segment and
// head), else 64 (the passes are throughput-bound)
int seg_split(const la_chunk_fwd_args *a) {
  if (a->dv_split) return a->dv_split;
  const int L = seg_for(a);
  if (L > 0) {
    const int64_t nt = la_nt_max(a->T_max, a->N_max, kBTk);
    const int64_t narrow = (nt + L - 1) / L * a->H * (a->d_v / 32 + a->d_k / 32);
    if (narrow <= 2 * kCUs) return a->d_v / 32;
  }
  return a->d_v / 64 > 0 ? a->d_v / 64 : 1;
}

// the d_v slices of the forward's reduce
int fwd_split(const la_chunk_fwd_args *a) { return seg_for(a) ? seg_split(a) : split_for(a); }

// whether the map stores no K, Q: GDN with 16-bit inputs in 32- or 64-column
// slices, whose reduces stage them from the raw q, k rows (128-column slices
// read them from the image)
bool raw_kq(const la_chunk_fwd_args *a, bool kda) {
  if (kda || a->qkv_dtype == LA_F32) return false;
  const int W = a->d_v / fwd_split(a);
  return W == 32 || W == 64;
}

// segment slots: ceil(T_max / (BT L)) + N_max - 1
int64_t ns_max(const la_chunk_fwd_args *a, int L) {
  return ((int64_t)a->T_max + (int64_t)kBTk * L - 1) / ((int64_t)kBTk * L) + a->N_max - 1;
}

// Workspace: one map-stage image per (chunk slot, head), image_layout bytes
// each; with segments, then hin, dlt ([d_k][d_v] fp32) and the transition
// images (2 x [d_k][d_k] fp16) per (segment slot, head)
size_t ws_img_bytes(const la_chunk_fwd_args *a, bool kda) {
  const size_t cells = (size_t)la_nt_max(a->T_max, a->N_max, kBTk) * a->H;
  return cells * (size_t)la::image_hbm_bytes(kda, (int)elem_bytes(a), a->d_k, raw_kq(a, kda));
}
size_t ws_seg_bytes(const la_chunk_fwd_args *a) {
  const int L = seg_for(a);
  if (L == 0) return 0;
  return 3 * (size_t)ns_max(a, L) * a->H * a->d_k * a->d_v * sizeof(float);
}
// BT = 32: the 64-row chunk layout the kernels run on, rebuilt from
// cu_seqlens into the workspace (chunk_indices, chunk_offsets, status)
size_t meta_bytes(const la_chunk_fwd_args *a) {
  if (a->BT == kBTk) return 0;
  const size_t nt = (size_t)la_nt_max(a->T_max, a->N_max, kBTk);
  return (2 * nt + a->N_max + 2) * sizeof(int32_t);
}
size_t ws_bytes(const la_chunk_fwd_args *a, bool kda) {
  return ws_img_bytes(a, kda) + ws_seg_bytes(a) + meta_bytes(a);
}

// the chunk layout the kernels read: the caller's (BT = 64), or one built
// now at the workspace's end (BT = 32)
// With meta_indices set the layout goes to the caller's meta_* arrays: built
// in the map's prologue up to 64 sequences (fuse), otherwise by the metadata
// kernel before a map stage.
struct Meta { const int32_t *ci, *co; bool fuse; };
hipError_t kernel_meta(const la_chunk_fwd_args *a, char *meta_base, hipStream_t st, Meta &m,
                       bool map_stage = true) {
  m.ci = a->chunk_indices;
  m.co = a->chunk_offsets;
  m.fuse = false;
  if (a->meta_indices) {
    m.ci = a->meta_indices;
    m.co = a->meta_offsets;
    m.fuse = a->N_max <= 64;
    if (m.fuse || !map_stage) return hipSuccess;
    const int nt = (int)la_nt_max(a->T_max, a->N_max, kBTk);
    return la::launch_chunk_meta(a->cu_seqlens, a->cu_seqlens_i64, a->N_max, a->T_max, kBTk, nt,
                                 a->meta_indices, a->meta_offsets, a->meta_status, st);
  }
  if (a->BT == kBTk) return hipSuccess;
  const int nt = (int)la_nt_max(a->T_max, a->N_max, kBTk);
  int32_t *ci = reinterpret_cast<int32_t *>(meta_base);
  int32_t *co = ci + 2 * (size_t)nt;
  int32_t *stat = co + a->N_max + 1;
  m.ci = ci;
  m.co = co;
  return la::launch_chunk_meta(a->cu_seqlens, a->cu_seqlens_i64, a->N_max, a->T_max, kBTk, nt, ci,
                               co, stat, st);
}

int forward(const la_chunk_fwd_args *a, bool kda, int stages, void *stream) {
  if (!a) return LA_ERR_NULL;
  if (stages < 1 || stages > 3) return LA_ERR_UNSUPPORTED;
  const int sc = check_shape(a);
  if (sc != LA_OK) return sc;
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->cu_seqlens || !a->o) return LA_ERR_NULL;
  if (a->meta_indices) {
    if (!a->meta_offsets) return LA_ERR_NULL;
    if (a->BT != kBTk) return LA_ERR_UNSUPPORTED;
  } else if (!a->chunk_indices || !a->chunk_offsets) {
    return LA_ERR_NULL;
  }
  if (!a->workspace) return LA_ERR_WORKSPACE;
  if (a->workspace_bytes < ws_bytes(a, kda)) return LA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(a->workspace) % 256 != 0) return LA_ERR_WORKSPACE;
  if (a->h0 && a->ht && a->h0 != a->ht) {
    const size_t sb = (size_t)a->N_max * a->H * a->d_k * a->d_v * sizeof(float);
    if (overlaps(a->h0, sb, a->ht, sb)) return LA_ERR_ALIAS;
  }
  // 16-byte vector loads of q, k and v rows
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->k) |
                        reinterpret_cast<uintptr_t>(a->v) | reinterpret_cast<uintptr_t>(a->o);
  if (mis % 16 != 0) return LA_ERR_SHAPE;

  const int dt = a->qkv_dtype;
  char *ws = static_cast<char *>(a->workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  Meta meta;
  if (kernel_meta(a, ws + ws_img_bytes(a, kda) + ws_seg_bytes(a), st, meta,
                  (stages & LA_STAGE_MAP) != 0) != hipSuccess)
    return LA_ERR_HIP;
  if (stages & LA_STAGE_MAP) {
    la::MapParams mp{};
    mp.q = a->q;
    mp.k = a->k;
    mp.g = a->g;
    mp.beta = a->beta;
    mp.cu_seqlens = a->cu_seqlens;
    mp.cu64 = a->cu_seqlens_i64;
    mp.chunk_indices = meta.ci;
    mp.H = a->H;
    mp.Hqk = a->H_qk ? a->H_qk : a->H;
    mp.NT_max = (int)la_nt_max(a->T_max, a->N_max, kBTk);
    mp.raw_kq = raw_kq(a, kda);
    mp.img = ws;
    mp.fuse_meta = meta.fuse;
    mp.N_max = a->N_max;
    mp.T_max = a->T_max;
    mp.meta_ci = a->meta_indices;
    mp.meta_co = a->meta_offsets;
    mp.meta_status = a->meta_status;
    if (la::launch_chunk_map(mp, kda, dt, a->d_k, st) != hipSuccess) return LA_ERR_HIP;
  }
  if (stages & LA_STAGE_REDUCE) {
    la::ReduceParams rp{};
    rp.v = a->v;
    rp.q_raw = a->q;
    rp.k_raw = a->k;
    rp.Hqk = a->H_qk ? a->H_qk : a->H;
    rp.raw_kq = raw_kq(a, kda);
    rp.cu_seqlens = a->cu_seqlens;
    rp.cu64 = a->cu_seqlens_i64;
    rp.chunk_offsets = meta.co;
    rp.h0 = a->h0;
    rp.o = a->o;
    rp.ht = a->ht;
    rp.img = ws;
    rp.H = a->H;
    rp.N_max = a->N_max;
    rp.S = fwd_split(a);
    rp.scale = a->scale;
    rp.o_bf16 = a->o_bf16;
    const int L = seg_for(a);
    if (L == 0) {
      if (launch_reduce(rp, a, kda, st) != hipSuccess) return LA_ERR_HIP;
    } else {
      rp.SP = a->d_k / (a->d_v / rp.S);
      rp.seg = L;
      rp.NS_max = (int)ns_max(a, L);
      const size_t mat = (size_t)rp.NS_max * a->H * a->d_k * a->d_v;
      rp.hin = reinterpret_cast<float *>(ws + ws_img_bytes(a, kda));
      rp.dlt = rp.hin + mat;
      rp.pimg = reinterpret_cast<_Float16 *>(rp.dlt + mat);
      rp.pass = 1;
      if (launch_reduce(rp, a, kda, st) != hipSuccess) return LA_ERR_HIP;
      la::CombineParams cp{};
      cp.chunk_offsets = meta.co;
      cp.H = a->H;
      cp.N_max = a->N_max;
      cp.seg = L;
      cp.hin = rp.hin;
      cp.dlt = rp.dlt;
      cp.pimg = rp.pimg;
      if (la::launch_chunk_combine(cp, a->d_k, st) != hipSuccess) return LA_ERR_HIP;
      rp.pass = 2;
      if (launch_reduce(rp, a, kda, st) != hipSuccess) return LA_ERR_HIP;
    }
  }
  return LA_OK;
}

}  // namespace

extern "C" {

int64_t la_nt_max(int64_t T_max, int64_t N_max, int32_t BT) {
  if (T_max < 1 || N_max < 1 || BT < 1) return -1;
  return (T_max + BT - 1) / BT + N_max - 1;
}

static int chunk_meta(const void *cu_seqlens, int cu64, int32_t N_max, int32_t T_max, int32_t BT,
                      int32_t *chunk_indices, int32_t *chunk_offsets, int32_t *status,
                      void *stream) {
  if (!cu_seqlens || !chunk_indices || !chunk_offsets) return LA_ERR_NULL;
  if (N_max < 1 || N_max > LA_MAX_N || T_max < 1 || T_max > 0x7fffffff - 2 * kBTSupported)
    return LA_ERR_SHAPE;
  if (BT != 32 && BT != 64) return LA_ERR_UNSUPPORTED;
  const int64_t nt = la_nt_max(T_max, N_max, BT);
  if (nt > 0x7fffffff / 2) return LA_ERR_SHAPE;
  if (la::launch_chunk_meta(cu_seqlens, cu64, N_max, T_max, BT, (int)nt, chunk_indices,
                            chunk_offsets, status, static_cast<hipStream_t>(stream)) != hipSuccess)
    return LA_ERR_HIP;
  return LA_OK;
}

int build_chunk_meta(const int32_t *cu_seqlens, int32_t N_max, int32_t T_max, int32_t BT,
                     int32_t *chunk_indices, int32_t *chunk_offsets, int32_t *status,
                     void *stream) {
  return chunk_meta(cu_seqlens, 0, N_max, T_max, BT, chunk_indices, chunk_offsets, status, stream);
}

int build_chunk_meta_i64(const int64_t *cu_seqlens, int32_t N_max, int32_t T_max, int32_t BT,
                         int32_t *chunk_indices, int32_t *chunk_offsets, int32_t *status,
                         void *stream) {
  return chunk_meta(cu_seqlens, 1, N_max, T_max, BT, chunk_indices, chunk_offsets, status, stream);
}

size_t la_chunk_fwd_workspace_bytes(const la_chunk_fwd_args *a, int is_kda) {
  if (!a || check_shape(a) != LA_OK) return 0;
  return ws_bytes(a, is_kda != 0);
}

int gdn_chunk_fwd(const la_chunk_fwd_args *a, void *stream) {
  return forward(a, false, LA_STAGE_MAP | LA_STAGE_REDUCE, stream);
}

int kda_chunk_fwd(const la_chunk_fwd_args *a, void *stream) {
  return forward(a, true, LA_STAGE_MAP | LA_STAGE_REDUCE, stream);
}

int la_chunk_fwd_stages(const la_chunk_fwd_args *a, int is_kda, int stages, void *stream) {
  return forward(a, is_kda != 0, stages, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free forward: the workspace is this static device array, one
// copy per GPU the library runs on (held until the process ends).  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
namespace {
static __device__ __align__(256) char scratch[LA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// the current device's scratch address, nullptr if it cannot be found
void *scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int la_chunk_fwd_static(const la_chunk_fwd_args *a, int is_kda, void *stream) {
  if (!a) return LA_ERR_NULL;
  const int sc = check_shape(a);
  if (sc != LA_OK) return sc;
  // the largest workspace the array holds: larger shapes are rejected before
  // anything is looked up or enqueued
  if (ws_bytes(a, is_kda != 0) > LA_STATIC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
  void *ws = scratch_ptr();
  if (!ws) return LA_ERR_HIP;
  la_chunk_fwd_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = LA_STATIC_SCRATCH_BYTES;
  return forward(&b, is_kda != 0, LA_STAGE_MAP | LA_STAGE_REDUCE, stream);
}

int32_t la_chunk_fwd_dv_split(const la_chunk_fwd_args *a) {
  if (!a || check_shape(a) != LA_OK) return 0;
  return fwd_split(a);
}

int32_t la_chunk_fwd_seg_len(const la_chunk_fwd_args *a) {
  if (!a || check_shape(a) != LA_OK) return -1;
  return seg_for(a);
}

static int recurrent(const la_recurrent_args *a, bool kda, void *stream) {
  if (!a) return LA_ERR_NULL;
  if (a->N < 1 || a->H < 1) return LA_ERR_SHAPE;
  if ((int64_t)a->N * a->H > 0x7fffffff) return LA_ERR_SHAPE;
  if (!known_dtype(a->qkv_dtype)) return LA_ERR_DTYPE;
  if (a->o_bf16 != 0 && a->o_bf16 != 1) return LA_ERR_DTYPE;
  if (a->H_qk < 0 || (a->H_qk > 0 && a->H % a->H_qk != 0)) return LA_ERR_SHAPE;
  if (a->d_k != a->d_v || (a->d_k != 64 && a->d_k != 128)) return LA_ERR_UNSUPPORTED;
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o) return LA_ERR_NULL;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->k) |
                        reinterpret_cast<uintptr_t>(a->v) | reinterpret_cast<uintptr_t>(a->o) |
                        reinterpret_cast<uintptr_t>(a->h0) | reinterpret_cast<uintptr_t>(a->ht);
  if (mis % 16 != 0) return LA_ERR_SHAPE;
  if (a->h0 && a->ht && a->h0 != a->ht) {
    const size_t sb = (size_t)a->N * a->H * a->d_k * a->d_v * sizeof(float);
    if (overlaps(a->h0, sb, a->ht, sb)) return LA_ERR_ALIAS;
  }
  la::RecurrentParams rp{};
  rp.q = a->q;
  rp.k = a->k;
  rp.v = a->v;
  rp.g = a->g;
  rp.beta = a->beta;
  rp.h0 = a->h0;
  rp.o = a->o;
  rp.ht = a->ht;
  rp.units = a->N * a->H;
  rp.H = a->H;
  rp.Hqk = a->H_qk ? a->H_qk : a->H;
  rp.scale = a->scale;
  rp.o_bf16 = a->o_bf16;
  if (la::launch_recurrent(rp, kda, a->qkv_dtype, a->d_k, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return LA_ERR_HIP;
  return LA_OK;
}

int gdn_recurrent_fwd(const la_recurrent_args *a, void *stream) { return recurrent(a, false, stream); }

int kda_recurrent_fwd(const la_recurrent_args *a, void *stream) { return recurrent(a, true, stream); }

int la_short_conv_fwd(const la_short_conv_args *a, void *stream) {
  if (!a) return LA_ERR_NULL;
  if (!a->x || !a->weight || !a->cu_seqlens || !a->chunk_indices || !a->y) return LA_ERR_NULL;
  if (!known_dtype(a->x_dtype)) return LA_ERR_DTYPE;
  if (a->activation != LA_ACT_NONE && a->activation != LA_ACT_SILU) return LA_ERR_DTYPE;
  if (a->cu_seqlens_i64 != 0 && a->cu_seqlens_i64 != 1) return LA_ERR_DTYPE;
  if (a->W < 1 || a->W > 4) return LA_ERR_UNSUPPORTED;
  if (a->BT != 32 && a->BT != 64) return LA_ERR_UNSUPPORTED;
  if (a->T_max < 1 || a->N_max < 1 || a->D < 1) return LA_ERR_SHAPE;
  if (a->T_max > 0x7fffffff - 2 * kBTSupported) return LA_ERR_SHAPE;
  const int esz = a->x_dtype == LA_F32 ? 4 : 2;
  if (a->D % (16 / esz) != 0) return LA_ERR_SHAPE;
  const int64_t nt = la_nt_max(a->T_max, a->N_max, a->BT);
  if (nt < 1 || nt > 0x7fffffff) return LA_ERR_SHAPE;
  // element indices of x / y and of the states stay in size_t; the grid's y
  // dimension (channel blocks of 64 x 16 bytes) stays within 65535
  if ((int64_t)a->D * esz / 1024 >= 65535) return LA_ERR_SHAPE;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a->x) | reinterpret_cast<uintptr_t>(a->y) |
                        reinterpret_cast<uintptr_t>(a->residual) |
                        reinterpret_cast<uintptr_t>(a->h0) | reinterpret_cast<uintptr_t>(a->ht) |
                        reinterpret_cast<uintptr_t>(a->weight) |
                        reinterpret_cast<uintptr_t>(a->bias);
  if (mis % 16 != 0) return LA_ERR_SHAPE;
  const size_t xb = (size_t)a->T_max * a->D * esz;
  if (overlaps(a->x, xb, a->y, xb)) return LA_ERR_ALIAS;
  if (a->residual && a->residual != a->y && overlaps(a->residual, xb, a->y, xb)) return LA_ERR_ALIAS;
  if (a->W > 1 && a->h0 && a->ht && a->h0 != a->ht) {
    const size_t sb = (size_t)a->N_max * (a->W - 1) * a->D * esz;
    if (overlaps(a->h0, sb, a->ht, sb)) return LA_ERR_ALIAS;
  }
  la::ConvParams cp{};
  cp.x = a->x;
  cp.res = a->residual;
  cp.h0 = a->W > 1 ? a->h0 : nullptr;
  cp.w = a->weight;
  cp.b = a->bias;
  cp.cu_seqlens = a->cu_seqlens;
  cp.chunk_indices = a->chunk_indices;
  cp.cu64 = a->cu_seqlens_i64;
  cp.D = a->D;
  cp.BT = a->BT;
  cp.y = a->y;
  cp.ht = a->W > 1 ? a->ht : nullptr;
  if (la::launch_short_conv(cp, a->x_dtype, (int)nt, a->W, a->activation == LA_ACT_SILU,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
    return LA_ERR_HIP;
  return LA_OK;
}

static la_chunk_fwd_args fwd_view(const la_chunk_bwd_args *a) {
  la_chunk_fwd_args f{};
  f.T_max = a->T_max;
  f.N_max = a->N_max;
  f.H = a->H;
  f.d_k = a->d_k;
  f.d_v = a->d_v;
  f.BT = a->BT;
  f.qkv_dtype = a->qkv_dtype;
  f.seg_len = -1;  // the recompute stores per-chunk states: one pass
  // 16-bit inputs: 32-column slices (the dedicated 16-bit reduce, which stores
  // the per-chunk states)
  f.dv_split = a->qkv_dtype != LA_F32 ? a->d_v / 32 : 0;
  f.cu_seqlens_i64 = a->cu_seqlens_i64;
  f.H_qk = a->H_qk;
  f.scale = a->scale;
  return f;
}

// backward workspace: [forward images][hs][dhs][prep][part], each 256-aligned
struct BwdLayout { size_t img, hs, dhs, prep, part, meta, gva, total; };
static BwdLayout bwd_layout(const la_chunk_bwd_args *a, bool kda) {
  const la_chunk_fwd_args f = fwd_view(a);
  const size_t cells = (size_t)la_nt_max(a->T_max, a->N_max, kBTk) * a->H;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  BwdLayout L{};
  L.img = 0;
  L.hs = up(ws_img_bytes(&f, kda));
  L.dhs = L.hs + up(cells * a->d_k * a->d_v * sizeof(float));
  L.prep = L.dhs + up(cells * a->d_k * a->d_v * sizeof(float));
  L.part = L.prep + up(cells * (kda ? la::kda_prep_floats(a->d_k) : la::kPrepFloats) * sizeof(float));
  L.meta = L.part + up(cells * la::part_floats(a->d_k) * sizeof(float));
  L.gva = L.meta + up(meta_bytes(&f));
  const bool grouped = a->H_qk > 0 && a->H_qk != a->H;
  L.total = L.gva + (grouped ? 2 * up((size_t)a->T_max * a->H * a->d_k * sizeof(float)) : 0);
  return L;
}

static int check_bwd(const la_chunk_bwd_args *a) {
  const la_chunk_fwd_args f = fwd_view(a);
  const int sc = check_shape(&f);
  if (sc != LA_OK) return sc;
  return LA_OK;
}

size_t la_chunk_bwd_workspace_bytes(const la_chunk_bwd_args *a, int is_kda) {
  if (!a || check_bwd(a) != LA_OK) return 0;
  return bwd_layout(a, is_kda != 0).total;
}

// The backward's reverse pass needs only the inputs and the prep.  When the
// caller hands over a second stream and two events (la_chunk_bwd_args
// aux_stream, fork_event, join_event), the reverse pass is forked onto that
// stream while `stream` recomputes the forward, and joined back before the
// per-chunk stage; otherwise everything runs in order on `stream`.  The
// library creates no stream or event and keeps no state between calls.
static int chunk_bwd(const la_chunk_bwd_args *a, bool kda, void *stream) {
  if (!a) return LA_ERR_NULL;
  const int sc = check_bwd(a);
  if (sc != LA_OK) return sc;
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->cu_seqlens || !a->chunk_indices ||
      !a->chunk_offsets || !a->dout || !a->dq || !a->dk || !a->dv || !a->dg || !a->dbeta)
    return LA_ERR_NULL;
  const int aux = (a->aux_stream != nullptr) + (a->fork_event != nullptr) +
                  (a->join_event != nullptr);
  if (aux != 0 && aux != 3) return LA_ERR_NULL;
  if (!a->workspace) return LA_ERR_WORKSPACE;
  const BwdLayout L = bwd_layout(a, kda);
  if (a->workspace_bytes < L.total) return LA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(a->workspace) % 256 != 0) return LA_ERR_WORKSPACE;
  // 16-byte vector loads of q, k, v and dout rows, 16-byte stores of dq, dk, dv
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->k) |
                        reinterpret_cast<uintptr_t>(a->v) | reinterpret_cast<uintptr_t>(a->dout) |
                        reinterpret_cast<uintptr_t>(a->dq) | reinterpret_cast<uintptr_t>(a->dk) |
                        reinterpret_cast<uintptr_t>(a->dv);
  if (mis % 16 != 0) return LA_ERR_SHAPE;
  char *ws = static_cast<char *>(a->workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // forward recompute: map images, then the reduce storing every chunk's
  // entering state (no output, no final state)
  la_chunk_fwd_args f = fwd_view(a);
  f.cu_seqlens = a->cu_seqlens;
  f.chunk_indices = a->chunk_indices;
  f.chunk_offsets = a->chunk_offsets;
  Meta meta;
  if (kernel_meta(&f, ws + L.meta, st, meta) != hipSuccess) return LA_ERR_HIP;
  const int NT = (int)la_nt_max(a->T_max, a->N_max, kBTk);
  la::BwdParams bp{};
  bp.q = a->q;
  bp.k = a->k;
  bp.v = a->v;
  bp.g = a->g;
  bp.beta = a->beta;
  bp.cu_seqlens = a->cu_seqlens;
  bp.cu64 = a->cu_seqlens_i64;
  bp.chunk_indices = meta.ci;
  bp.chunk_offsets = meta.co;
  bp.dout = a->dout;
  bp.dht = a->dht;
  const int Hqk = a->H_qk ? a->H_qk : a->H;
  const bool grouped = Hqk != a->H;
  const size_t full = (size_t)a->T_max * a->H * a->d_k * sizeof(float);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  float *dq_full = reinterpret_cast<float *>(ws + L.gva);
  float *dk_full = reinterpret_cast<float *>(ws + L.gva + up(full));
  bp.dq = grouped ? dq_full : a->dq;
  bp.dk = grouped ? dk_full : a->dk;
  bp.Hqk = Hqk;
  bp.dv = a->dv;
  bp.dg = a->dg;
  bp.dbeta = a->dbeta;
  bp.dh0 = a->dh0;
  bp.hs = reinterpret_cast<float *>(ws + L.hs);
  bp.dhs = reinterpret_cast<float *>(ws + L.dhs);
  bp.prep = reinterpret_cast<float *>(ws + L.prep);
  bp.part = reinterpret_cast<float *>(ws + L.part);
  bp.H = a->H;
  bp.N_max = a->N_max;
  bp.NT = NT;
  bp.scale = a->scale;
  const auto stage = [&](int k, hipStream_t sk) {
    return kda ? la::launch_chunk_bwd_kda(bp, a->qkv_dtype, a->d_k, k, sk)
               : la::launch_chunk_bwd(bp, a->qkv_dtype, a->d_k, k, sk);
  };
  // prep first (the reverse pass needs it), then the reverse pass on the
  // caller's second stream (if given) while this stream recomputes the
  // forward
  if (stage(1, st) != hipSuccess) return LA_ERR_HIP;
  hipStream_t s1 = st;
  hipEvent_t fork = static_cast<hipEvent_t>(a->fork_event);
  hipEvent_t join = static_cast<hipEvent_t>(a->join_event);
  if (aux) {
    s1 = static_cast<hipStream_t>(a->aux_stream);
    if (hipEventRecord(fork, st) != hipSuccess || hipStreamWaitEvent(s1, fork, 0) != hipSuccess)
      return LA_ERR_HIP;
  }
  bool ok = stage(2, s1) == hipSuccess;
  if (ok) {
    la::MapParams mp{};
    mp.q = a->q;
    mp.k = a->k;
    mp.g = a->g;
    mp.beta = a->beta;
    mp.cu_seqlens = a->cu_seqlens;
    mp.cu64 = a->cu_seqlens_i64;
    mp.chunk_indices = meta.ci;
    mp.H = a->H;
    mp.Hqk = a->H_qk ? a->H_qk : a->H;
    mp.NT_max = NT;
    mp.raw_kq = raw_kq(&f, kda);
    mp.img = ws;
    ok = la::launch_chunk_map(mp, kda, a->qkv_dtype, a->d_k, st) == hipSuccess;
  }
  if (ok) {
    la::ReduceParams rp{};
    rp.v = a->v;
    rp.cu_seqlens = a->cu_seqlens;
    rp.cu64 = a->cu_seqlens_i64;
    rp.chunk_offsets = meta.co;
    rp.h0 = a->h0;
    rp.o = nullptr;
    rp.ht = nullptr;
    rp.img = ws;
    rp.H = a->H;
    rp.N_max = a->N_max;
    rp.q_raw = a->q;
    rp.k_raw = a->k;
    rp.Hqk = a->H_qk ? a->H_qk : a->H;
    rp.raw_kq = raw_kq(&f, kda);
    rp.S = split_for(&f);
    rp.scale = a->scale;
    rp.hsave = reinterpret_cast<float *>(ws + L.hs);
    ok = launch_reduce(rp, &f, kda, st) == hipSuccess;
  }
  // the join is recorded even after a failed launch, so a capture of
  // `stream` never holds an unjoined fork
  if (aux && (hipEventRecord(join, s1) != hipSuccess || hipStreamWaitEvent(st, join, 0) != hipSuccess))
    ok = false;
  if (!ok) return LA_ERR_HIP;
  if (stage(3, st) != hipSuccess) return LA_ERR_HIP;
  if (grouped) {
    if (la::launch_group_sum(dq_full, a->dq, a->T_max, a->H, Hqk, a->d_k, a->cu_seqlens,
                             a->cu_seqlens_i64, a->N_max, meta.co, st) != hipSuccess ||
        la::launch_group_sum(dk_full, a->dk, a->T_max, a->H, Hqk, a->d_k, a->cu_seqlens,
                             a->cu_seqlens_i64, a->N_max, meta.co, st) != hipSuccess)
      return LA_ERR_HIP;
  }
  return LA_OK;
}

int gdn_chunk_bwd(const la_chunk_bwd_args *a, void *stream) { return chunk_bwd(a, false, stream); }

int kda_chunk_bwd(const la_chunk_bwd_args *a, void *stream) { return chunk_bwd(a, true, stream); }

const char *la_status_string(int status) {
  switch (status) {
    case LA_OK: return "ok";
    case LA_ERR_NULL: return "a required pointer is NULL";
    case LA_ERR_SHAPE: return "shape out of range or misaligned input";
    case LA_ERR_DTYPE: return "unsupported dtype";
    case LA_ERR_UNSUPPORTED: return "unsupported BT, head dim or dv_split";
    case LA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case LA_ERR_ALIAS: return "ht partially overlaps h0";
    case LA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
