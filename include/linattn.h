/*
 * linattn.h -- C ABI of the MI355X (gfx950) varlen chunkwise gated-delta-rule
 * prefill forward (GDN: scalar per-head decay; KDA: per-key-channel decay).
 *
 * The operation.  For each sequence n of a varlen batch and each head h, the
 * per-head recurrent state ("Empowering Hybrid Attention Models on NPUs",
 * section 2.1) evolves token by token as
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,        alpha_t = exp(g_t),
 * where g_t is a log-decay: one value per (token, head) for GDN, one per
 * (token, head, key channel) for KDA.  The library stores the state
 * transposed, H = S^T, as a d_k x d_v fp32 block.  It is evaluated chunkwise
 * with BT-token chunks as Map-Reduce-Map (same paper, section 2.1): a
 * chunk-parallel map (gate cumsum, masked K K^T / Q K^T, triangular inverse)
 * and a sequential reduce over each sequence's chunks that carries the state
 * and forms the outputs -- the pipeline "gate / chunk cumsum -> forward intra
 * -> recompute_w_u -> forward h -> forward o" of the FLA graph-capture RFC
 * ("[RFC] Add Graph Capture Support for FLA Prefill and Training Paths on
 * Ascend NPUs", section "Step 3").
 *
 * Fixed-capacity execution (same RFC, sections "Fixed-capacity execution",
 * "Device-side metadata", "Static buffer contract", "API proposal").  A bucket
 * is (T_max, N_max, BT) with NT_max = ceil(T_max/BT) + N_max - 1 chunk slots.
 * cu_seqlens has the fixed shape [N_max+1]; build_chunk_meta turns it into
 * chunk_indices [NT_max][2] (unused slots hold the sentinel {-1, 0}) and
 * chunk_offsets [N_max+1] on the device, and every kernel grid is sized from
 * (T_max, N_max, H) only, so one capture of the calls in a hipGraph replays
 * any layout written into the same cu_seqlens buffer.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, caches nothing, creates no stream or graph and never
 *    synchronises; calls are asynchronous on `stream` (a hipStream_t; NULL is
 *    the null stream) and may be captured into a hipGraph.
 *  - Arguments that can be checked on the host are checked before anything is
 *    enqueued; a failed check returns a negative la_status and enqueues
 *    nothing.  There is no fallback path.
 *  - Layouts are row-major, token-major varlen packing (batch 1):
 *    q, k [T_max][H][d_k]; v, o [T_max][H][d_v]; g [T_max][H] (GDN) or
 *    [T_max][H][d_k] (KDA); beta [T_max][H]; h0, ht [N_max][H][d_k][d_v].
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_NULL = -1,        /* a required pointer is NULL                      */
    LA_ERR_SHAPE = -2,       /* T_max, N_max or H out of range                  */
    LA_ERR_DTYPE = -3,       /* unknown or unsupported dtype code               */
    LA_ERR_UNSUPPORTED = -4, /* BT, d_k/d_v combination not built               */
    LA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required         */
    LA_ERR_ALIAS = -6,       /* ht overlaps h0 without being identical          */
    LA_ERR_HIP = -7          /* a HIP launch failed (hipGetLastError)           */
} la_status;

typedef enum { LA_BF16 = 0, LA_F32 = 1, LA_F16 = 2 } la_dtype;

/* Device status bits written by build_chunk_meta (0 = valid cu_seqlens). */
#define LA_META_BAD_START 1     /* cu_seqlens[0] != 0                           */
#define LA_META_NOT_MONOTONE 2  /* cu_seqlens[n+1] < cu_seqlens[n] for some n   */
#define LA_META_OVER_CAPACITY 4 /* cu_seqlens[N_max] > T_max                    */

/* Largest N_max build_chunk_meta accepts (its offsets scan lives in LDS). */
#define LA_MAX_N 8192

/* Chunk capacity of a bucket: ceil(T_max/BT) + N_max - 1, or -1 if any
 * argument is < 1 (FLA RFC, section "Fixed-capacity execution"). */
int64_t la_nt_max(int64_t T_max, int64_t N_max, int32_t BT);

/*
 * Device-side metadata (FLA RFC, sections "Fixed-capacity execution" and
 * "Device-side metadata").  Reads cu_seqlens[N_max+1] (int32; int64 for
 * build_chunk_meta_i64) on the device and writes
 *   chunk_offsets[n]    = sum_{m<n} ceil((cu[m+1]-cu[m]) / BT)   (int32, N_max+1)
 *   chunk_indices[j]    = {n, i_t} for j = chunk_offsets[n] + i_t,
 *                         {-1, 0}  for j >= chunk_offsets[N_max] (int32, NT_max x 2)
 *   *status             = OR of LA_META_* bits (int32; status may be NULL).
 * Slots are sequence-major then chunk-minor; zero-length sequences own none.
 * If cu_seqlens is invalid (status != 0) every slot is the sentinel and every
 * offset is 0, so the forward calls then write nothing.  The int64 variant
 * checks the offsets as int64 (a valid layout has all of them in
 * [0, T_max]).  BT may be 32 or 64 (the RFC's two chunk sizes; the chunk
 * kernels run 64-row chunks).  One launch of one workgroup; capturable.
 * Host errors: LA_ERR_NULL (cu_seqlens, chunk_indices or chunk_offsets NULL),
 * LA_ERR_SHAPE (N_max < 1, N_max > LA_MAX_N, T_max < 1),
 * LA_ERR_UNSUPPORTED (BT not 32 or 64), LA_ERR_HIP.
 */
int build_chunk_meta(const int32_t *cu_seqlens, int32_t N_max, int32_t T_max,
                     int32_t BT, int32_t *chunk_indices,
                     int32_t *chunk_offsets, int32_t *status, void *stream);
int build_chunk_meta_i64(const int64_t *cu_seqlens, int32_t N_max, int32_t T_max,
                         int32_t BT, int32_t *chunk_indices,
                         int32_t *chunk_offsets, int32_t *status, void *stream);

/* Arguments of the forward calls.  Sizes describe the bucket (capacity); the
 * actual layout comes from cu_seqlens on the device. */
typedef struct {
    int32_t T_max, N_max, H;   /* bucket capacity and head count (>= 1)          */
    int32_t d_k, d_v;          /* head dims: d_k == d_v; 64 or 128 (bf16, fp16), */
                               /* 64 (fp32 inputs)                               */
    int32_t BT;                /* chunk size of the caller's metadata: 32 or 64  */
                               /* (the kernels run 64-row chunks; for 32 the    */
                               /* call builds that layout from cu_seqlens in    */
                               /* its workspace and does not read chunk_indices */
                               /* or chunk_offsets)                             */
    int32_t qkv_dtype;         /* LA_BF16, LA_F16 or LA_F32: dtype of q, k, v    */
    int32_t dv_split;          /* state column slices per (seq, head): 0 = auto, */
                               /* else 1, 2 or 4 with d_v / dv_split >= 32.      */
                               /* auto: d_v / 64 slices, twice that when         */
                               /* N_max * H * (d_v / 64) <= 256 (the CU count)   */
    int32_t seg_len;           /* sequence-parallel reduce: chunks per segment;  */
                               /* -1 = off, 0 = auto, > 0 needs 16-bit inputs    */
                               /* and N_max <= 64 (see la_chunk_fwd_seg_len)     */
    int32_t H_qk;              /* q, k heads: 0 = H; else H % H_qk == 0 and      */
                               /* value head h reads q, k head h / (H / H_qk)    */
                               /* (grouped value heads share keys and queries)   */
    int32_t o_bf16;            /* 0: o fp32; 1: o bf16, rounded to nearest even  */
    int32_t cu_seqlens_i64;    /* 0: cu_seqlens int32; 1: int64                  */
    float scale;               /* o = scale * S q                                */
    const void *q, *k, *v;     /* [T_max][H_qk][d_k] / [T_max][H][d_v], qkv_dtype */
    const float *g;            /* log-decay: GDN [T_max][H]; KDA [T_max][H][d_k] */
    const float *beta;         /* [T_max][H]                                     */
    const void *cu_seqlens;    /* [N_max+1], int32 or int64 (cu_seqlens_i64)     */
    const int32_t *chunk_indices; /* [NT_max][2], from build_chunk_meta          */
    const int32_t *chunk_offsets; /* [N_max+1], from build_chunk_meta            */
    const float *h0;           /* [N_max][H][d_k][d_v] or NULL (zero state)      */
    void *o;                   /* [T_max][H][d_v] fp32 (bf16 with o_bf16)        */
    float *ht;                 /* [N_max][H][d_k][d_v] or NULL; may equal h0     */
    void *workspace;           /* >= la_chunk_fwd_workspace_bytes(...) bytes,    */
    size_t workspace_bytes;    /* 256-byte aligned                               */
    /* Chunk layout built by the call itself (optional; BT must be 64).  With   */
    /* meta_indices != NULL the call does not read chunk_indices and          */
    /* chunk_offsets (they may be NULL): it derives the layout of cu_seqlens  */
    /* on the device and writes meta_indices [NT_max][2], meta_offsets        */
    /* [N_max+1] and, if not NULL, meta_status [1], with the values           */
    /* build_chunk_meta (BT = 64) writes for the same arguments.  Up to 64    */
    /* sequences the map kernel does this in its prologue (no launch of its   */
    /* own); beyond, the call runs build_chunk_meta's kernel first.  A        */
    /* LA_STAGE_REDUCE-only call reads meta_offsets as its earlier            */
    /* LA_STAGE_MAP call left them.  Later calls on the same layout may pass  */
    /* the written arrays as chunk_indices / chunk_offsets.                   */
    int32_t *meta_indices, *meta_offsets, *meta_status;
} la_chunk_fwd_args;

/*
 * Workspace the forward needs for this shape (only T_max, N_max, H, d_k, d_v,
 * BT, qkv_dtype, dv_split and seg_len are read); 0 if the shape is invalid.
 * It holds the map stage's results for the reduce: one image per
 * (chunk slot, head) cell, NT_max * H cells in slot-major order, each a
 * multiple of 1 KiB.  With e = 2 (bf16, fp16 inputs: fp16 values) or 4 (fp32
 * inputs), a cell holds in order
 *   K, Q  [BT][d_k]  the chunk's keys and queries (KDA: K*exp(G), Q*exp(G));
 *                    absent for GDN with 16-bit inputs in 32- or 64-column
 *                    slices, whose reduce reads the rows of k and q itself
 *   KT    [d_k][BT]  KDA: (K*exp(G_C - G))^T; fp32 inputs: K^T; absent for
 *                    GDN with 16-bit inputs
 *   Tn    [BT][BT]   T = A^-1 diag(beta) with its diagonal removed
 *   M     [BT][BT]   masked decayed Q K^T (lower triangle incl. diagonal)
 *                    Above the diagonal of Tn and M the reduce reads only the
 *                    16x16 tiles (0,1) and (2,3), which are written as zeros;
 *                    with GDN and 16-bit inputs the other upper tiles are
 *                    not written, otherwise they are zeros too
 *   vec   [192 + d_k] fp32: exp(G_r), exp(G_C - G_r), beta_r (BT each), then
 *                    the state decay of each key row; padded to 1 KiB
 * where G is the chunk-local cumulative gate and G_C its last row.  Matrices
 * are rows of 16-byte pieces whose piece index is XOR-swizzled per row; for
 * e = 2 the column index inside every 32-column block is stored permuted
 * (the MFMA operand order of the reduce).  When the reduce runs segmented
 * (la_chunk_fwd_seg_len), the images are followed by hin and dlt
 * ([d_k][d_v] fp32) and the transition images (2 x [d_k][d_k] fp16), each
 * [NS_max][H], NS_max = ceil(T_max / (BT * seg_len)) + N_max - 1.  Content
 * between calls is unspecified.
 */
size_t la_chunk_fwd_workspace_bytes(const la_chunk_fwd_args *shape, int is_kda);

/*
 * GDN / KDA chunk forward.  For every non-empty sequence n and head h:
 * o rows cu[n]..cu[n+1]-1 of head h and ht[n][h] (if ht != NULL) are written;
 * o rows >= cu[N_max], sentinel slots and zero-length sequences are never
 * written.  h0 == NULL means a zero initial state.  ht may be the same
 * pointer as h0 (in-place state update); a partial overlap is LA_ERR_ALIAS.
 * Matrix products run on MFMA: bf16 and fp16 inputs in fp16 operands with fp32
 * accumulation (inputs and intermediates must stay within fp16 range,
 * |x| < 65504; g <= 0 is assumed for KDA), fp32 inputs in fp32 operands.
 * The reduce of 16-bit inputs scales each wave's v, h0 and state operands
 * by one power of two taken from its first chunk's v and its h0 (the
 * recurrence is linear in them, so o and ht are unchanged up to rounding):
 * v and h0 of any magnitude from about 2^-24 to 2^16 keep fp16 precision.
 * The metadata must come from build_chunk_meta on the same cu_seqlens, T_max,
 * N_max and BT, unless the call builds it itself (meta_indices set).
 * Host errors: LA_ERR_NULL (also: meta_indices without meta_offsets),
 * LA_ERR_SHAPE, LA_ERR_DTYPE, LA_ERR_UNSUPPORTED (also: meta_indices with
 * BT != 64), LA_ERR_WORKSPACE, LA_ERR_ALIAS, LA_ERR_HIP.
 */
int gdn_chunk_fwd(const la_chunk_fwd_args *a, void *stream);
int kda_chunk_fwd(const la_chunk_fwd_args *a, void *stream);

/*
 * The forward split into its two launches, for callers that time or overlap
 * them: stages = LA_STAGE_MAP runs the chunk-parallel map into the workspace,
 * LA_STAGE_REDUCE runs the sequential reduce + output from it, and
 * LA_STAGE_MAP | LA_STAGE_REDUCE equals gdn_chunk_fwd / kda_chunk_fwd.
 * A reduce must follow a map of the same arguments on the same workspace.
 */
#define LA_STAGE_MAP 1
#define LA_STAGE_REDUCE 2
int la_chunk_fwd_stages(const la_chunk_fwd_args *a, int is_kda, int stages,
                        void *stream);

/*
 * For callers that cannot allocate -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: gdn_chunk_fwd (is_kda = 0)
 * or kda_chunk_fwd (is_kda = 1) with the library's own static device array of
 * LA_STATIC_SCRATCH_BYTES bytes as the workspace; a->workspace and
 * a->workspace_bytes are ignored, every other argument and result is as for
 * those calls (same kernels, bit-identical outputs).  A shape whose workspace
 * (la_chunk_fwd_workspace_bytes) exceeds LA_STATIC_SCRATCH_BYTES returns
 * LA_ERR_WORKSPACE before anything is enqueued.  The array exists once per
 * GPU the library runs on and is held until the process ends; the call
 * allocates nothing (its first call on a device looks up that device's copy,
 * with the device current).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU -- on two streams, from two threads, or as
 * graphs replayed concurrently -- race and give wrong results; calls ordered
 * on one stream do not.  Nothing in the array needs to start at zero.
 * Host errors: as gdn_chunk_fwd, and LA_ERR_HIP if the array's device
 * address cannot be found.
 */
#define LA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int la_chunk_fwd_static(const la_chunk_fwd_args *a, int is_kda, void *stream);

/* The dv_split the forward uses for these arguments (after "auto").  Run
 * segmented, auto takes 32-column slices while the first pass has at most
 * 512 workgroups with them (2 per CU), else 64-column slices. */
int32_t la_chunk_fwd_dv_split(const la_chunk_fwd_args *a);

/*
 * Chunks per segment the forward's reduce uses (after "auto"), 0 when one
 * workgroup walks each whole sequence, -1 for an invalid shape.  Segmented,
 * each sequence's chunks are cut into segments of seg_len chunks and the
 * reduce runs in three launches: the first segments (with output) together
 * with each later segment's transition P and zero-state result D (the state
 * entering segment s+1 is P_s H_s + D_s: the recurrence is affine in the
 * state), a serial combine of those along each sequence, then the later
 * segments with output from their entering state.  Auto (seg_len = 0)
 * segments only 16-bit inputs with N_max <= 64 whose (sequence, head) units
 * cannot fill half of the 256 CUs at 64 state columns per workgroup, with
 * about ceil(NT_max * H * (d_v / 64) / 256) chunks per segment (at least 8),
 * and only when a sequence of T_max tokens would have 3 segments or more.
 */
int32_t la_chunk_fwd_seg_len(const la_chunk_fwd_args *a);

/* Arguments of one recurrent (decode) step: one token per sequence. */
typedef struct {
    int32_t N, H;              /* sequences (one token each) and heads (>= 1)    */
    int32_t d_k, d_v;          /* d_k == d_v: 64 or 128                          */
    int32_t qkv_dtype;         /* LA_BF16, LA_F16 or LA_F32: dtype of q, k, v    */
    int32_t H_qk;              /* q, k heads: 0 = H; else H % H_qk == 0          */
    int32_t o_bf16;            /* 0: o fp32; 1: o bf16 (nearest even)            */
    float scale;               /* o = scale * S q                                */
    const void *q, *k;         /* [N][H_qk][d_k], qkv_dtype                      */
    const void *v;             /* [N][H][d_v], qkv_dtype                         */
    const float *g;            /* log-decay: GDN [N][H]; KDA [N][H][d_k]         */
    const float *beta;         /* [N][H]                                         */
    const float *h0;           /* [N][H][d_k][d_v] or NULL (zero state)          */
    void *o;                   /* [N][H][d_v] fp32 (bf16 with o_bf16)            */
    float *ht;                 /* [N][H][d_k][d_v] or NULL; may equal h0         */
} la_recurrent_args;

/*
 * One step of the recurrence per sequence n and head h (the token-level
 * form the chunk forward computes in bulk): with alpha = exp(g),
 *   H = diag(alpha) h0[n][h];  u = beta (v - H^T k);  H += k u^T;
 *   ht[n][h] = H;  o[n][h] = scale H^T q
 * (H = S^T, [d_k][d_v] fp32; alpha one value per (n, h) for GDN, one per key
 * channel for KDA).  ht == h0 updates the state in place; a partial overlap
 * is LA_ERR_ALIAS.  Arithmetic is fp32 throughout.  One launch, no
 * workspace, capturable.
 * Host errors: LA_ERR_NULL (q, k, v, g, beta or o NULL), LA_ERR_SHAPE (N or
 * H < 1, N * H beyond 2^31 - 1, H_qk < 0 or not dividing H, or q, k, v, h0,
 * ht, o not 16-byte aligned), LA_ERR_DTYPE (qkv_dtype unknown, o_bf16 not 0 / 1),
 * LA_ERR_UNSUPPORTED (d_k != d_v or not 64 / 128), LA_ERR_ALIAS, LA_ERR_HIP.
 */
int gdn_recurrent_fwd(const la_recurrent_args *a, void *stream);
int kda_recurrent_fwd(const la_recurrent_args *a, void *stream);

/* Arguments of the GDN / KDA chunk backward: the forward's inputs and
 * metadata, the output gradient, and the gradient outputs. */
typedef struct {
    int32_t T_max, N_max, H;   /* as la_chunk_fwd_args                           */
    int32_t d_k, d_v;          /* d_k == d_v: 64 or 128 (16-bit), 64 (fp32)      */
    int32_t BT;                /* 32 or 64, as la_chunk_fwd_args                 */
    int32_t qkv_dtype;         /* LA_BF16, LA_F16 or LA_F32                      */
    int32_t cu_seqlens_i64;    /* 0: cu_seqlens int32; 1: int64                  */
    int32_t H_qk;              /* q, k heads as la_chunk_fwd_args (0 = H)        */
    float scale;               /* the forward's scale                            */
    const void *q, *k, *v;     /* [T_max][H_qk][d_k] / [T_max][H][d_v], qkv_dtype */
    const float *g;            /* log-decay: GDN [T_max][H]; KDA [T_max][H][d_k] */
    const float *beta;         /* [T_max][H]                                     */
    const void *cu_seqlens;    /* [N_max+1]                                      */
    const int32_t *chunk_indices, *chunk_offsets; /* from build_chunk_meta      */
    const float *h0;           /* [N_max][H][d_k][d_v] or NULL (zero state)      */
    const float *dout;         /* gradient of o: [T_max][H][d_v] fp32            */
    const float *dht;          /* gradient of ht: [N_max][H][d_k][d_v] or NULL   */
    float *dq, *dk;            /* [T_max][H_qk][d_k] fp32 (summed over a group's */
                               /* value heads)                                   */
    float *dv;                 /* [T_max][H][d_v] fp32                           */
    float *dg;                 /* like g, fp32                                   */
    float *dbeta;              /* [T_max][H] fp32                                */
    float *dh0;                /* [N_max][H][d_k][d_v] fp32 or NULL              */
    void *workspace;           /* >= la_chunk_bwd_workspace_bytes(...) bytes,    */
    size_t workspace_bytes;    /* 256-byte aligned                               */
    void *aux_stream;          /* optional second stream (hipStream_t) of the   */
                               /* caller for the reverse pass, with two of the  */
                               /* caller's events (hipEvent_t) to fork it from  */
    void *fork_event;          /* `stream` and join it back; all three NULL     */
    void *join_event;          /* (everything on `stream`) or all three set     */
} la_chunk_bwd_args;

/* Workspace of gdn_chunk_bwd / kda_chunk_bwd for this shape (T_max, N_max,
 * H, d_k, d_v, BT, qkv_dtype read); 0 if the shape is invalid.  It holds the
 * forward recompute's map images, the state entering and the state gradient
 * leaving every chunk ([d_k][d_v] fp32 per chunk slot and head), per-cell
 * prep images (fp32 A^-1, M, S and gate vectors, KDA also the per-channel
 * cumulative gate, and bf16 high/low halves of M and A^-1 diag(beta)),
 * per-cell partial products, with BT = 32 the 64-row chunk layout, and with
 * grouped value heads the per-value-head dq, dk ([T_max][H][d_k] fp32 each). */
size_t la_chunk_bwd_workspace_bytes(const la_chunk_bwd_args *shape, int is_kda);

/*
 * GDN / KDA chunk backward: the gradients of L = sum(o * dout) + sum(ht * dht)
 * of gdn_chunk_fwd / kda_chunk_fwd with the same inputs, for q, k, v, g, beta
 * and h0 (FLA RFC,
 * sections "Scope" and "Step 3": the backward of the chunk path).  It
 * runs a chunk-parallel prep (A^-1, M, S, gates), then a reverse pass over
 * each sequence's chunks for the state gradient (writing dh0) while the
 * forward's per-chunk states are recomputed (map, then the reduce storing the
 * state entering each chunk), then chunk-parallel passes for dv and the
 * d_v-contracted products and for dq, dk, dg, dbeta (one fused kernel for
 * bf16 inputs).  bf16 inputs run on bf16 MFMA with operands split into bf16
 * high and low halves (about 17 significant bits, fp32 exponent range); fp16
 * and fp32 inputs on fp32 MFMA; accumulation is fp32.  Rows outside every
 * sequence, sentinel slots and dh0 of zero-length sequences are not written.
 * With grouped value heads each value head's dq, dk go to the workspace and
 * one more launch sums every group into dq, dk.
 * Streams: everything is ordered after the work already queued on `stream`,
 * and work queued on `stream` afterwards sees every output.  With
 * aux_stream, fork_event and join_event all NULL every launch goes to
 * `stream`, in order.  With all three set (the caller's own stream and
 * events, on the current device), the reverse pass runs on aux_stream,
 * forked after the prep (fork_event recorded on `stream`, waited for by
 * aux_stream) and joined back before the per-chunk stage (join_event
 * recorded on aux_stream, waited for by `stream`) while `stream` recomputes
 * the forward; capturing `stream` into a HIP graph captures both branches.
 * The join is recorded even when a launch fails.  The caller must not use
 * aux_stream or the two events for anything else until the call's work on
 * `stream` has completed (two concurrent calls need their own triples).  As
 * every call, it creates no stream or event and allocates nothing (all
 * scratch is the caller's workspace).
 * Host errors: LA_ERR_NULL (also: only some of aux_stream, fork_event,
 * join_event set), LA_ERR_SHAPE (also: q, k, v, dout, dq, dk or dv not
 * 16-byte aligned), LA_ERR_DTYPE, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE,
 * LA_ERR_HIP.
 */
int gdn_chunk_bwd(const la_chunk_bwd_args *a, void *stream);
int kda_chunk_bwd(const la_chunk_bwd_args *a, void *stream);

/* Activation of the short convolution. */
#define LA_ACT_NONE 0
#define LA_ACT_SILU 1

/* Arguments of the varlen causal short convolution. */
typedef struct {
    int32_t T_max, N_max;      /* bucket capacity (>= 1)                         */
    int32_t D;                 /* channels: a multiple of 8 (16-bit x) or 4      */
    int32_t W;                 /* kernel width, 1 .. 4                           */
    int32_t BT;                /* chunk size chunk_indices was built with: 32/64 */
    int32_t x_dtype;           /* LA_BF16, LA_F16 or LA_F32: x, residual, y,     */
                               /* h0 and ht                                      */
    int32_t activation;        /* LA_ACT_NONE or LA_ACT_SILU                     */
    int32_t cu_seqlens_i64;    /* 0: cu_seqlens int32; 1: int64                  */
    const void *x;             /* [T_max][D]                                     */
    const float *weight;       /* [D][W] fp32                                    */
    const float *bias;         /* [D] fp32 or NULL                               */
    const void *residual;      /* [T_max][D] or NULL; may be y itself            */
    const void *cu_seqlens;    /* [N_max+1], int32 or int64                      */
    const int32_t *chunk_indices; /* [NT_max][2], build_chunk_meta with this BT  */
    const void *h0;            /* [N_max][W-1][D] or NULL (zero history)         */
    void *y;                   /* [T_max][D]; must not overlap x                 */
    void *ht;                  /* [N_max][W-1][D] or NULL; may equal h0          */
} la_short_conv_args;

/*
 * Varlen causal short convolution forward, the layer step before the chunk
 * attention, run on the same chunk metadata (FLA RFC, sections "Proposed API"
 * and "Step 3: GDN and short-convolution graph support"; the reuse of that
 * metadata: "Empowering Hybrid Attention Models on NPUs", section 7).  Per
 * sequence n, channel c and token t of the sequence (inputs x_p, p < 0, are
 * row W-1+p of h0[n], zero when h0 is NULL):
 *   y_t[c] = act(bias[c] + sum_{i<W} weight[c][i] x_{t-W+1+i}[c]) + residual_t[c]
 * with act the identity or SiLU (z sigmoid(z)), computed in fp32 and rounded
 * to x_dtype (nearest even).  ht[n] = the W-1 inputs ending at the sequence's
 * last token (reaching into h0[n] for sequences shorter than W-1), copied
 * bit for bit; ht may equal h0.  Rows of y outside every sequence, sentinel
 * slots and ht of zero-length sequences are not written.  chunk_indices must
 * come from build_chunk_meta on the same cu_seqlens, T_max, N_max and BT.
 * One launch, no workspace, capturable.  x, residual, y, h0, ht, weight and
 * bias must be 16-byte aligned.
 * Host errors: LA_ERR_NULL (x, weight, cu_seqlens, chunk_indices or y NULL),
 * LA_ERR_SHAPE (T_max, N_max or D < 1, D not a multiple of the channels of a
 * 16-byte piece, sizes beyond the index range, misaligned pointers),
 * LA_ERR_DTYPE (x_dtype, activation or cu_seqlens_i64 unknown),
 * LA_ERR_UNSUPPORTED (W not 1 .. 4, BT not 32 or 64), LA_ERR_ALIAS (y
 * overlapping x or partly overlapping residual, ht partly overlapping h0),
 * LA_ERR_HIP.
 */
int la_short_conv_fwd(const la_short_conv_args *a, void *stream);

/* Static text for a la_status value. */
const char *la_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
