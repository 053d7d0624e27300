/*
 * tri_attn.h -- C ABI of the MI355X (gfx950) TriangleMix prefill-attention
 * library (libtriattn.so).
 *
 * What is computed.  One attention layer of a long-context prefill, as the
 * TriangleMix pages describe it (blog post "TriangleMix", sections "介绍" and
 * "速度"; 36kr interview with Yang Yuqing, technical-motivation paragraphs):
 * shallow layers keep dense causal attention, deep layers use the static
 * "triangle" pattern, which keeps the streaming region (the leading sink keys
 * plus a sliding window along the diagonal) and the final "Last Q-K" rows, and
 * skips the middle Q-K region, so its cost grows as O(N) instead of O(N^2).
 *
 * For batch b, query head h, query row i (g = h / (heads_q / heads_kv)):
 *   K_i   = { j <= i : j < sink  or  i - j < window  or  i >= N - last_q }
 *           (triangle), or { j <= i } (causal);
 *   z_ij  = softmax_scale * <q[b,h,i,:], k[b,g,j,:]>
 *   o[b,h,i,:] = sum_{j in K_i} softmax_j(z_i.) * v[b,g,j,:]
 *   lse[b,h,i] = ln sum_{j in K_i} exp(z_ij)        (natural log)
 *
 * Conventions.
 *   - Every call returns TRI_OK (0) or a negative tri_status; nothing throws
 *     across the ABI.  On error, tri_attn_last_error() returns a message.
 *   - All argument validation happens before any HIP runtime call, so every
 *     error path can be exercised on a machine without a GPU.
 *   - The library never allocates, frees or copies device memory and keeps no
 *     global state other than the per-thread error message and the scratch
 *     array of tri_dyn_plan_noalloc (one per GPU, in the code object).  The
 *     caller owns every other buffer, host or device.
 *   - Device calls enqueue on the caller's stream and return; results are
 *     bit-deterministic for identical inputs (fixed traversal order, no
 *     atomics).  Device faults surface at the caller's next synchronisation.
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TRI_OK = 0,
  TRI_ERR_INVALID = -1,     /* malformed argument (null, negative, inconsistent) */
  TRI_ERR_CAPACITY = -2,    /* output arrays too small; *nnz_out holds the need   */
  TRI_ERR_UNSUPPORTED = -3, /* valid but not implemented (head_dim, tile size)   */
  TRI_ERR_HIP = -4          /* the HIP runtime reported an error at launch        */
} tri_status;

typedef enum { TRI_MASK_TRIANGLE = 0, TRI_MASK_CAUSAL = 1 } tri_mask_kind;
typedef enum { TRI_DTYPE_BF16 = 0, TRI_DTYPE_F32 = 1 } tri_dtype;
enum { TRI_TILE_FULL = 0, TRI_TILE_PARTIAL = 1 };

/* Tile shape the GPU kernel walks (query rows x key columns per tile). */
enum { TRI_KERNEL_BLOCK_Q = 128, TRI_KERNEL_BLOCK_K = 64 };

/* Static mask of one layer.  sink, window and last_q are token counts; values
 * larger than seqlen are legal and mean "the whole range".  window >= 1, so
 * the diagonal is always kept and no row is ever empty. */
typedef struct {
  int64_t seqlen;   /* N >= 0 (N == 0: nothing to do)                        */
  int32_t block_q;  /* planner: any >= 1; prefill: TRI_KERNEL_BLOCK_Q        */
  int32_t block_k;  /* planner: any >= 1; prefill: TRI_KERNEL_BLOCK_K        */
  int32_t kind;     /* tri_mask_kind                                         */
  int32_t reserved; /* must be 0                                             */
  int64_t sink;     /* >= 0: keys j < sink are kept by every row             */
  int64_t window;   /* >= 1: keys with i - j < window are kept               */
  int64_t last_q;   /* >= 0: rows i >= N - last_q keep every key j <= i      */
} tri_mask_params;

/*
 * tri_attn_plan -- host-only tile planner (pure, deterministic, no HIP call).
 *
 * Lists, for every query tile t (rows [t*block_q, min(N,(t+1)*block_q))), the
 * key tiles kt (columns [kt*block_k, (kt+1)*block_k)) that hold at least one
 * kept (row, column) pair, in ascending kt, as CSR:
 *   row_ptr[t] .. row_ptr[t+1]-1 index k_tile[] and flags[];
 *   flags[e] = TRI_TILE_FULL when every valid row of the query tile keeps every
 *   column of the key tile (columns >= N never count as kept), else
 *   TRI_TILE_PARTIAL.
 * The kernel computes kept tiles only, masking inside PARTIAL ones; this is the
 * index-driven tile skipping the FlashPrefill page (section 2.3) contrasts with
 * branch-per-block skipping.
 *
 * Sizing call: row_ptr, k_tile and flags all NULL -> writes *n_qtiles_out and
 * *nnz_out only.  Fill call: all three non-NULL; row_ptr has n_qtiles + 1
 * entries, k_tile and flags have `capacity` entries.  If capacity < nnz the call
 * writes *n_qtiles_out and *nnz_out and returns TRI_ERR_CAPACITY.
 * n_qtiles_out and nnz_out must be non-NULL.
 */
int tri_attn_plan(const tri_mask_params* mp, int32_t* row_ptr, int32_t* k_tile,
                  uint8_t* flags, int64_t capacity, int32_t* n_qtiles_out,
                  int64_t* nnz_out);

/*
 * tri_attn_check_plan -- host only: checks a host copy of a tile plan before
 * its device copy is handed to a prefill call (the kernel walks the arrays
 * as given).  The plan is CSR over n_rows list rows (a multiple of n_qtiles);
 * row r lists key tiles of query tile r % n_qtiles.  With heads > 0, row r
 * follows head (r / n_qtiles) % heads's sink[] and window[] (the layout of
 * tri_attn_plan_heads); with heads = 0 (sink, window may be NULL) every row
 * follows *mp.  Checked: row_ptr[0] = 0, row_ptr non-decreasing up to
 * row_ptr[n_rows] = nnz; within a row, key tiles strictly ascending and
 * inside the row's causal range; each listed tile holds a kept pair of the
 * mask (TriangleMix blog "介绍"; 36kr interview, technical motivation); its
 * flag equals the tile_flag definition of tri_attn_plan.  A list of some of
 * the kept tiles passes (a dynamic selection under kind = TRI_MASK_CAUSAL).
 * Returns TRI_OK, or TRI_ERR_INVALID with the first bad entry named in
 * tri_attn_last_error().  Reads row_ptr[0 .. n_rows], k_tile[0 .. nnz),
 * flags[0 .. nnz); writes nothing.
 */
int tri_attn_check_plan(const tri_mask_params* mp, int32_t heads, const int64_t* sink,
                        const int64_t* window, const int32_t* row_ptr, int64_t n_rows,
                        const int32_t* k_tile, const uint8_t* flags, int64_t nnz);

/* Device tensors of one layer.  Strides are in elements, for the (batch, head,
 * token) axes; the channel axis is contiguous.  q, k, v are bf16, 16-byte
 * aligned, with token strides that are multiples of 8 elements; the N token
 * rows of one (batch, KV head) of k and of v must span fewer than 2^31 bytes.
 * o is bf16 (8-byte aligned, token stride a multiple of 4) or f32 (16-byte aligned,
 * token stride a multiple of 4).  lse (f32) may be NULL. */
typedef struct {
  const void* q;       /* [B, Hq,  N, d] */
  const void* k;       /* [B, Hkv, N, d] */
  const void* v;       /* [B, Hkv, N, d] */
  void* o;             /* [B, Hq,  N, d] in o_dtype */
  float* lse;          /* [B, Hq,  N] natural-log log-sum-exp, or NULL */
  int32_t batch;       /* >= 1 */
  int32_t heads_q;     /* >= 1, multiple of heads_kv */
  int32_t heads_kv;    /* >= 1; query head h reads KV head h / (heads_q/heads_kv) */
  int32_t head_dim;    /* 64 or 128 */
  int64_t seqlen;      /* N; must equal mp->seqlen in tri_attn_prefill */
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int64_t lse_stride[2];
  float softmax_scale; /* finite, > 0 (1/sqrt(head_dim) for standard attention) */
  int32_t o_dtype;     /* tri_dtype */
} tri_attn_tensors;

/*
 * tri_attn_prefill -- triangle (or any planned) layer on the GPU.
 *
 * d_row_ptr, d_k_tile, d_flags are device copies of tri_attn_plan's output for
 * the same *mp (block_q = TRI_KERNEL_BLOCK_Q, block_k = TRI_KERNEL_BLOCK_K); the
 * caller owns them and keeps them alive until the work completes.  `stream` is
 * a hipStream_t (NULL = the null stream).  Returns after enqueueing.
 */
int tri_attn_prefill(const tri_attn_tensors* t, const tri_mask_params* mp,
                     const int32_t* d_row_ptr, const int32_t* d_k_tile,
                     const uint8_t* d_flags, void* stream);

/*
 * dense_causal_prefill -- dense (shallow) layer: the same kernel walking the
 * full causal tile list, enumerated in the kernel (equal to tri_attn_plan with
 * kind = TRI_MASK_CAUSAL and the kernel tile shape).
 */
int dense_causal_prefill(const tri_attn_tensors* t, void* stream);

/*
 * Dynamic block-sparse lists for the dense (shallow) layers.
 *
 * The TriangleMix pages leave the shallow layers dense and note that a
 * dynamic sparse method can be used there on top of the static triangle
 * layers.  The FlashPrefill page gives such a method: evenly spread query
 * rows act as probes (section 2.1), each key block is represented by the
 * mean of its keys (2.1), a key block is kept when its score reaches alpha
 * times the largest score of its query block, with no sort (2.2), and the
 * kept blocks are walked through an index list (2.3).  Here the blocks are
 * the kernel tiles (TRI_KERNEL_BLOCK_Q query rows x TRI_KERNEL_BLOCK_K keys):
 *   - probes of query tile t: rows t*128 + 8p, p = 0..15, that are < N;
 *   - kbar_kt: the mean of the keys of tile kt (keys < N), rounded to bf16;
 *   - probe i sees the tiles kt with 64*kt <= i; its attention over them is
 *     softmax_kt(softmax_scale * <q_i, kbar_kt>);
 *   - score(t, kt): that attention averaged over the tile's probes;
 *   - kt (0 <= 64*kt <= last row of t) is kept when score >= alpha * max
 *     score, and always when it crosses the causal diagonal of the query
 *     tile (64*kt + 63 > 128*t), so no row is ever empty.
 * The result is a CSR list per (batch, query head): row r = (b*heads_q + h)
 * * nq + t (nq = ceil(N/128)) spans d_k_tile[row_ptr[r] .. row_ptr[r+1]),
 * ascending, with causal flags (TRI_TILE_FULL iff every key of the tile is
 * <= the tile's first row).
 */
enum { TRI_DYN_PROBES = 16 };

typedef struct {
  float alpha;      /* keep threshold factor, 0 <= alpha <= 1 (0 keeps every causal tile) */
  int32_t n_probe;  /* probe rows per query tile; must be TRI_DYN_PROBES */
} tri_dyn_params;

/*
 * tri_dyn_plan_sizes -- host only.  For the layer described by *t (its q and
 * k are what tri_dyn_plan reads; every field is validated as for the prefill
 * calls), writes the device workspace size in bytes, the number of list rows
 * (batch * heads_q * nq; row_ptr needs one more entry) and the largest
 * possible number of list entries (every causal tile kept), which is the
 * capacity tri_dyn_plan requires for d_k_tile and d_flags.
 * Workspace layout (byte offsets from its start): bf16 pooled keys
 * [batch, heads_kv, ceil(N/64), head_dim] at 0; the rest is scratch.
 */
int tri_dyn_plan_sizes(const tri_attn_tensors* t, int64_t* workspace_bytes, int64_t* n_rows,
                       int64_t* max_nnz);

/*
 * tri_dyn_plan -- enqueue the selection on `stream` and return.  The caller
 * owns the 256-byte-aligned device workspace (>= workspace_bytes of
 * tri_dyn_plan_sizes) and the device outputs d_row_ptr [n_rows + 1],
 * d_k_tile and d_flags [capacity >= max_nnz].  No host synchronisation: the
 * list length is d_row_ptr[n_rows] on the device.
 */
int tri_dyn_plan(const tri_attn_tensors* t, const tri_dyn_params* dp, void* d_workspace,
                 int64_t workspace_bytes, int32_t* d_row_ptr, int32_t* d_k_tile, uint8_t* d_flags,
                 int64_t capacity, void* stream);

/*
 * tri_dyn_plan_noalloc -- tri_dyn_plan for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is a library-owned device
 * array of TRI_DYN_SCRATCH_BYTES per GPU (each GPU the library runs on holds
 * it until the process ends); the call allocates nothing and the caller
 * passes only the outputs (as for tri_dyn_plan).  The array of the current
 * device is used (`stream` must belong to it).  A layer whose workspace
 * (tri_dyn_plan_sizes) exceeds TRI_DYN_SCRATCH_BYTES is rejected with
 * TRI_ERR_CAPACITY before any HIP call (64 MiB covers e.g. 32 query / 8 KV
 * heads, d = 128, up to N = 337920 at batch 1).  Every call on one GPU
 * shares that GPU's array and leaves its contents behind (nothing in it
 * needs to start at zero): calls that overlap on one GPU -- on two streams,
 * or from two threads -- race and must be serialised by the caller.
 */
enum { TRI_DYN_SCRATCH_BYTES = 64 << 20 };
int tri_dyn_plan_noalloc(const tri_attn_tensors* t, const tri_dyn_params* dp, int32_t* d_row_ptr,
                         int32_t* d_k_tile, uint8_t* d_flags, int64_t capacity, void* stream);

/*
 * tri_attn_prefill_lists -- the attention kernel walking per-(batch, head)
 * tile lists in the format above (e.g. tri_dyn_plan's output), with the
 * causal mask inside the listed tiles: row i keeps the keys of its query
 * tile's listed key tiles that are <= i.  The lists must be ascending, hold
 * only tiles kt with 64*kt <= the tile's last row, and include the tiles
 * crossing the diagonal, flagged as above.
 */
int tri_attn_prefill_lists(const tri_attn_tensors* t, const int32_t* d_row_ptr,
                           const int32_t* d_k_tile, const uint8_t* d_flags, void* stream);

/*
 * Per-head boundaries of the triangle mask.  The TriAttention page encodes
 * each attention head's computation region with two diagonal-distance
 * boundaries, so that the policy's storage does not grow with the context.
 * In the TriangleMix pattern the two per-head quantities are the sink length
 * and the window (the diagonal distance below which keys are kept): head h
 * keeps, for row i, the keys j <= i with j < sink[h], i - j < window[h], or
 * i >= N - last_q (last_q stays one value for the layer).
 *
 * tri_attn_plan_heads -- host only, like tri_attn_plan; mp gives seqlen,
 * tile shape, kind (must be TRI_MASK_TRIANGLE) and last_q (its sink and
 * window are not used).  sink[heads], window[heads] (>= 0, >= 1; int32
 * range).  Lists are CSR over rows h * n_qtiles + t (row_ptr has
 * heads * n_qtiles + 1 entries), each list as tri_attn_plan would give for
 * that head's (sink, window).  Sizing and capacity as in tri_attn_plan.
 */
int tri_attn_plan_heads(const tri_mask_params* mp, int32_t heads, const int64_t* sink,
                        const int64_t* window, int32_t* row_ptr, int32_t* k_tile, uint8_t* flags,
                        int64_t capacity, int32_t* n_qtiles_out, int64_t* nnz_out);

/*
 * tri_attn_prefill_heads -- a triangle layer with per-head boundaries: the
 * device copy of tri_attn_plan_heads's output for heads = t->heads_q (shared
 * by every batch entry) and device int32 arrays d_head_sink, d_head_window
 * [heads_q] holding the same boundaries (values past N mean "everything").
 */
int tri_attn_prefill_heads(const tri_attn_tensors* t, const tri_mask_params* mp,
                           const int32_t* d_head_sink, const int32_t* d_head_window,
                           const int32_t* d_row_ptr, const int32_t* d_k_tile,
                           const uint8_t* d_flags, void* stream);

/*
 * Precision tiers.  The TriAttention page scores query-key tiles at two
 * precisions, chosen per head by diagonal-distance boundaries, and combines
 * both groups in one normalised output.  Here the lower tier is fp8 (e4m3)
 * on MI355X's fp8 matrix cores, for the scores only (P and V stay bf16): a
 * kept key tile kt of query tile t is LOW when 128*t - (64*kt + 63) >=
 * low_dist[h] (every query-key distance in the tile reaches the boundary).
 * A LOW tile's score is softmax_scale * s_q * s_k * <q8, k8>, with
 *   s_q = amax |q row| / 448,           q8 = e4m3(q * (448 / amax_q)),
 *   s_k = amax |K of the key tile| / 448, k8 = e4m3(k * (448 / amax_k)),
 * rounded to nearest even after clamping to +-448 (all-zero blocks: scale 0).
 * The page assigns a precision per query-key tile, so one K scale covers the
 * TRI_KERNEL_BLOCK_K keys of a key tile.
 *
 * tri_attn_quantize_k_sizes -- bytes of the fp8 K (batch*heads_kv*N*head_dim)
 * and number of scales (batch*heads_kv*ceil(N/64)).
 * tri_attn_quantize_k -- enqueue the fp8 copy of t->k: d_k8 (16-byte
 * aligned) holds, for each (batch, KV head), N rows of head_dim bytes in the
 * kernel's operand order (byte 64s + 32h + j of a row is channel
 * 64s + 16(j/8) + 8h + j%8); d_scale [batch, heads_kv, ceil(N/64)] f32.
 *
 * The page's two lower tiers are 4-bit and 8-bit: a second per-head boundary
 * selects fp4 (e2m1, on the same matrix cores at twice the fp8 rate) for
 * the farthest tiles.  The farthest tier wins: a tile is fp4 when
 * 128*t - (64*kt + 63) >= fp4_dist[h], else fp8 when >= low_dist[h], else
 * bf16.  fp4 scores use s_q = amax |q row| / 6, s_k = amax / 6 of the key
 * tile, codes e2m1(clamp(x * 6 / amax, -6, 6)) rounded to nearest, ties to
 * the even code.
 *
 * tri_attn_quantize_k4_sizes / tri_attn_quantize_k4 -- the fp4 copy of t->k:
 * d_k4 (16-byte aligned) holds, per (batch, KV head), N rows of head_dim / 2
 * bytes; 16-byte block 2s + h of a row holds the 32 elements e of k-step s,
 * lane half h (channel 64s + 16(e/8) + 8h + e%8, as in the fp8 copy) at
 * nibble e of the block; d_scale [batch, heads_kv, ceil(N/64)] f32.
 * tri_attn_prefill_tiered -- tri_attn_prefill with the LOW tiles scored from
 * d_k8 / d_scale (the output of tri_attn_quantize_k for the same K) and the
 * device int32 boundaries d_head_low_dist [heads_q], and, when
 * d_head_fp4_dist, d_k4 and d_scale4 are given (all three, or all NULL for
 * no fp4 tier), the farthest tiles from the fp4 copy; Q is quantized in the
 * kernel.  Boundaries larger than N give the plain triangle layer.
 */
int tri_attn_quantize_k_sizes(const tri_attn_tensors* t, int64_t* k8_bytes, int64_t* n_scales);
int tri_attn_quantize_k(const tri_attn_tensors* t, void* d_k8, float* d_scale, void* stream);
int tri_attn_quantize_k4_sizes(const tri_attn_tensors* t, int64_t* k4_bytes, int64_t* n_scales);
int tri_attn_quantize_k4(const tri_attn_tensors* t, void* d_k4, float* d_scale, void* stream);
int tri_attn_prefill_tiered(const tri_attn_tensors* t, const tri_mask_params* mp,
                            const int32_t* d_head_low_dist, const void* d_k8, const float* d_scale,
                            const int32_t* d_head_fp4_dist, const void* d_k4, const float* d_scale4,
                            const int32_t* d_row_ptr, const int32_t* d_k_tile,
                            const uint8_t* d_flags, void* stream);

/*
 * Split of the last-Q rows.  Query tiles holding last-Q rows keep every key
 * tile (2048 at N = 131072 against ~38 for a band tile), and one workgroup
 * walking such a list sets the layer's critical path when the band is short.
 * The split launch walks each of those lists in chunks of chunk_tiles key
 * tiles on separate workgroups, each leaving an unnormalised partial output
 * and its row statistics in a caller-provided workspace, then merges the
 * chunks by the usual rescaling of partial softmax sums.  The layer computed
 * is the triangle layer of tri_attn_prefill (TriangleMix pages: sink, window
 * and last-Q regions), or of tri_attn_prefill_heads when per-head boundaries
 * are given; only the summation order of the split rows differs.
 *
 * tri_attn_split_workspace_size -- device bytes the split launch needs for
 * (t, mp, chunk_tiles): 0 when mp has no last-Q rows (last_q = 0).
 * mp->kind must be TRI_MASK_TRIANGLE; chunk_tiles >= 1.
 * tri_attn_prefill_split -- enqueue the split layer on the plan arrays of
 * tri_attn_plan (d_head_sink = d_head_window = NULL) or of
 * tri_attn_plan_heads (device int32 [heads_q] boundaries, as for
 * tri_attn_prefill_heads).  d_workspace: device, 256-byte aligned, at least
 * the size above (TRI_ERR_CAPACITY otherwise); its contents need no
 * initialisation and are overwritten.  Two launches (attention, then merge)
 * on `stream`; calls that share a workspace must not overlap.
 */
int tri_attn_split_workspace_size(const tri_attn_tensors* t, const tri_mask_params* mp,
                                  int32_t chunk_tiles, int64_t* bytes);
int tri_attn_prefill_split(const tri_attn_tensors* t, const tri_mask_params* mp,
                           const int32_t* d_head_sink, const int32_t* d_head_window,
                           const int32_t* d_row_ptr, const int32_t* d_k_tile,
                           const uint8_t* d_flags, int32_t chunk_tiles, void* d_workspace,
                           int64_t workspace_bytes, void* stream);

/* Message for the last non-OK return on this thread ("" if none). */
const char* tri_attn_last_error(void);

/* ABI version of this header (incremented on incompatible change). */
int tri_attn_abi_version(void);

/*
 * tri_attn_work_item -- host-only view of the kernel's block schedule, for
 * testing that the launch covers every (batch, head, query tile) exactly once.
 * For launch block index `bid` of a launch over (batch, heads_q, heads_kv,
 * seqlen, kind, last_q), writes the work item it computes (or -1 in all three
 * when that block has none) and the grid size to *grid_out.
 */
int tri_attn_work_item(int32_t batch, int32_t heads_q, int32_t heads_kv,
                       int64_t seqlen, int32_t kind, int64_t last_q, int64_t bid,
                       int32_t* b_out, int32_t* h_out, int32_t* qtile_out,
                       int64_t* grid_out);

/*
 * tri_attn_split_work_item -- the same view for a split triangle launch:
 * also writes the chunk (or -1 for a whole row) the block computes.
 */
int tri_attn_split_work_item(int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t seqlen,
                             int64_t last_q, int32_t chunk_tiles, int64_t bid, int32_t* b_out,
                             int32_t* h_out, int32_t* qtile_out, int32_t* chunk_out,
                             int64_t* grid_out);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_H */
