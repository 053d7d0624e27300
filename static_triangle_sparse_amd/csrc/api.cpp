// C ABI of libtriattn: argument validation, error reporting and dispatch to
// the gfx950 kernel.  Every check runs before the first HIP runtime call, so
// each error path can be driven from a host without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "tri_attn.h"
#include "tri_attn_internal.h"

namespace triattn {

namespace {
thread_local char g_error[512] = "";
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

namespace {

constexpr int64_t kMaxSeqlen = int64_t(1) << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_strides(const char* name, const int64_t* s, int n) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0) return fail(TRI_ERR_INVALID, "%s stride %d is negative", name, i);
  return TRI_OK;
}

int validate_tensors(const tri_attn_tensors* t) {
  if (!t) return fail(TRI_ERR_INVALID, "tensor descriptor pointer is NULL");
  if (!t->q || !t->k || !t->v || !t->o)
    return fail(TRI_ERR_INVALID, "q, k, v and o must be non-NULL device pointers");
  if (t->batch < 1 || t->heads_q < 1 || t->heads_kv < 1)
    return fail(TRI_ERR_INVALID, "batch, heads_q and heads_kv must be >= 1");
  if (t->heads_q % t->heads_kv != 0)
    return fail(TRI_ERR_INVALID, "heads_q (%d) must be a multiple of heads_kv (%d)", t->heads_q,
                t->heads_kv);
  if (t->head_dim != 64 && t->head_dim != 128)
    return fail(TRI_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", t->head_dim);
  if (t->seqlen < 0) return fail(TRI_ERR_INVALID, "seqlen must be >= 0");
  if (t->seqlen >= kMaxSeqlen) return fail(TRI_ERR_UNSUPPORTED, "seqlen must be < 2^30");
  if (t->o_dtype != TRI_DTYPE_BF16 && t->o_dtype != TRI_DTYPE_F32)
    return fail(TRI_ERR_INVALID, "o_dtype must be TRI_DTYPE_BF16 or TRI_DTYPE_F32");
  if (!(t->softmax_scale > 0.0f) || !isfinite(t->softmax_scale))
    return fail(TRI_ERR_INVALID, "softmax_scale must be finite and > 0");
  int st;
  if ((st = check_strides("q", t->q_stride, 3)) != TRI_OK) return st;
  if ((st = check_strides("k", t->k_stride, 3)) != TRI_OK) return st;
  if ((st = check_strides("v", t->v_stride, 3)) != TRI_OK) return st;
  if ((st = check_strides("o", t->o_stride, 3)) != TRI_OK) return st;
  if (t->lse && (st = check_strides("lse", t->lse_stride, 2)) != TRI_OK) return st;
  if (!aligned(t->q, 16) || !aligned(t->k, 16) || !aligned(t->v, 16))
    return fail(TRI_ERR_INVALID, "q, k and v must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (t->q_stride[i] % 8 || t->k_stride[i] % 8 || t->v_stride[i] % 8)
      return fail(TRI_ERR_INVALID, "q/k/v strides must be multiples of 8 elements (16 bytes)");
    if (t->o_stride[i] % 4)
      return fail(TRI_ERR_INVALID, "o strides must be multiples of 4 elements");
  }
  // the kernel addresses the keys of one (batch, KV head) through 32-bit
  // buffer descriptors: N token rows of K (and of V) must span < 2^31 bytes
  if (t->seqlen * t->k_stride[2] * 2 >= (int64_t(1) << 31) ||
      t->seqlen * t->v_stride[2] * 2 >= (int64_t(1) << 31))
    return fail(TRI_ERR_UNSUPPORTED, "seqlen x k/v token stride must be < 2^31 bytes");
  if (!aligned(t->o, t->o_dtype == TRI_DTYPE_BF16 ? 8 : 16))
    return fail(TRI_ERR_INVALID, "o must be %d-byte aligned", t->o_dtype == TRI_DTYPE_BF16 ? 8 : 16);
  if (t->lse && !aligned(t->lse, 4)) return fail(TRI_ERR_INVALID, "lse must be 4-byte aligned");
  const int64_t nq = (t->seqlen + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  const int64_t blocks = static_cast<int64_t>(t->batch) * t->heads_q * (nq + kNumXcd);
  if (blocks >= INT32_MAX) return fail(TRI_ERR_UNSUPPORTED, "launch grid exceeds 2^31-1 blocks");
  return TRI_OK;
}

AttnLaunch make_launch(const tri_attn_tensors* t, bool causal, int64_t sink, int64_t window,
                       int64_t last_q) {
  AttnLaunch a{};
  a.q = t->q;
  a.k = t->k;
  a.v = t->v;
  a.o = t->o;
  a.lse = t->lse;
  memcpy(a.q_stride, t->q_stride, sizeof(a.q_stride));
  memcpy(a.k_stride, t->k_stride, sizeof(a.k_stride));
  memcpy(a.v_stride, t->v_stride, sizeof(a.v_stride));
  memcpy(a.o_stride, t->o_stride, sizeof(a.o_stride));
  if (t->lse) memcpy(a.lse_stride, t->lse_stride, sizeof(a.lse_stride));
  a.head_dim = t->head_dim;
  a.o_bf16 = t->o_dtype == TRI_DTYPE_BF16 ? 1 : 0;
  a.causal = causal ? 1 : 0;
  const int64_t N = t->seqlen;
  a.seqlen = static_cast<int32_t>(N);
  // Values past N mean "everything": j < N, i - j <= N - 1 and i >= 0 always.
  a.sink = static_cast<int32_t>(std::min(sink, N));
  a.window = static_cast<int32_t>(std::max<int64_t>(1, std::min(window, N)));
  a.last_q = static_cast<int32_t>(std::min(last_q, N));
  a.scale = t->softmax_scale;
  a.sched = make_schedule(t->batch, t->heads_q, t->heads_kv, N, TRI_KERNEL_BLOCK_Q, causal,
                          causal ? N : a.last_q);
  return a;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Largest list of a dense layer: every causal key tile of every query tile.
int64_t causal_tiles(int64_t N) {
  const int64_t nq = (N + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  int64_t n = 0;
  for (int64_t t = 0; t < nq; ++t)
    n += (std::min(N, (t + 1) * TRI_KERNEL_BLOCK_Q) - 1) / TRI_KERNEL_BLOCK_K + 1;
  return n;
}

// Heavy tiles and chunks of a split launch of a triangle plan.
void split_shape(int64_t N, int64_t last_q, int32_t chunk_tiles, int32_t* n_heavy, int32_t* n_split) {
  const Schedule s = make_schedule(1, 1, 1, N, TRI_KERNEL_BLOCK_Q, false, std::min(last_q, N));
  const int64_t nkt = (N + TRI_KERNEL_BLOCK_K - 1) / TRI_KERNEL_BLOCK_K;
  *n_heavy = s.n_heavy;
  *n_split = s.n_heavy > 0 ? static_cast<int32_t>((nkt + chunk_tiles - 1) / chunk_tiles) : 1;
}

}  // namespace

SplitWorkspace split_workspace(int64_t batch, int64_t heads_q, int64_t head_dim, int64_t n_heavy,
                               int64_t n_split) {
  SplitWorkspace w{};
  w.n_items = n_split > 1 ? batch * heads_q * n_heavy * n_split : 0;
  w.stats = 0;
  w.o = align256(w.n_items * 3 * TRI_KERNEL_BLOCK_Q * 4);
  w.total = w.o + align256(w.n_items * TRI_KERNEL_BLOCK_Q * head_dim * 4);
  return w;
}

DynWorkspace dyn_workspace(int64_t batch, int64_t heads_q, int64_t heads_kv, int64_t head_dim,
                           int64_t seqlen) {
  const int64_t nq = (seqlen + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  const int64_t nkt = (seqlen + TRI_KERNEL_BLOCK_K - 1) / TRI_KERNEL_BLOCK_K;
  const int64_t words = (nkt + 31) / 32;
  DynWorkspace w{};
  w.pooled = 0;
  w.bitmap = align256(batch * heads_kv * nkt * head_dim * 2);
  w.counts = w.bitmap + align256(batch * heads_q * nq * words * 4);
  w.total = w.counts + align256(batch * heads_q * nq * 4);
  return w;
}

}  // namespace triattn

using namespace triattn;

extern "C" const char* tri_attn_last_error(void) { return g_error; }

extern "C" int tri_attn_abi_version(void) { return 4; }

extern "C" int tri_attn_prefill(const tri_attn_tensors* t, const tri_mask_params* mp,
                                const int32_t* d_row_ptr, const int32_t* d_k_tile,
                                const uint8_t* d_flags, void* stream) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if ((st = validate_tensors(t)) != TRI_OK) return st;
  if (mp->block_q != TRI_KERNEL_BLOCK_Q || mp->block_k != TRI_KERNEL_BLOCK_K)
    return fail(TRI_ERR_UNSUPPORTED, "the kernel walks %dx%d tiles; plan has %dx%d",
                TRI_KERNEL_BLOCK_Q, TRI_KERNEL_BLOCK_K, mp->block_q, mp->block_k);
  if (mp->seqlen != t->seqlen)
    return fail(TRI_ERR_INVALID, "mask seqlen %lld differs from tensor seqlen %lld",
                static_cast<long long>(mp->seqlen), static_cast<long long>(t->seqlen));
  if (!d_row_ptr || !d_k_tile || !d_flags)
    return fail(TRI_ERR_INVALID, "plan arrays (row_ptr, k_tile, flags) must be non-NULL");
  if (!aligned(d_row_ptr, 4) || !aligned(d_k_tile, 4))
    return fail(TRI_ERR_INVALID, "row_ptr and k_tile must be 4-byte aligned");
  if (t->seqlen == 0) return TRI_OK;
  AttnLaunch a = make_launch(t, mp->kind == TRI_MASK_CAUSAL, mp->sink, mp->window, mp->last_q);
  a.causal = 0;  // walk the caller's list even for a causal plan
  a.row_ptr = d_row_ptr;
  a.k_tile = d_k_tile;
  a.flags = d_flags;
  if (mp->kind == TRI_MASK_CAUSAL) {
    // a causal plan masks like the causal kernel: make the triangle predicate
    // keep every j <= i
    a.last_q = a.seqlen;
  }
  return launch_attn_fwd(a, stream);
}

extern "C" int dense_causal_prefill(const tri_attn_tensors* t, void* stream) {
  clear_error();
  int st = validate_tensors(t);
  if (st != TRI_OK) return st;
  if (t->seqlen == 0) return TRI_OK;
  AttnLaunch a = make_launch(t, true, 0, 1, t->seqlen);
  return launch_attn_fwd(a, stream);
}

extern "C" int tri_attn_work_item(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                  int64_t seqlen, int32_t kind, int64_t last_q, int64_t bid,
                                  int32_t* b_out, int32_t* h_out, int32_t* qtile_out,
                                  int64_t* grid_out) {
  clear_error();
  if (!b_out || !h_out || !qtile_out || !grid_out)
    return fail(TRI_ERR_INVALID, "output pointers must be non-NULL");
  if (batch < 1 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv)
    return fail(TRI_ERR_INVALID, "bad head counts");
  if (seqlen < 1 || seqlen >= kMaxSeqlen) return fail(TRI_ERR_INVALID, "bad seqlen");
  if (kind != TRI_MASK_TRIANGLE && kind != TRI_MASK_CAUSAL)
    return fail(TRI_ERR_INVALID, "bad kind");
  if (last_q < 0) return fail(TRI_ERR_INVALID, "last_q must be >= 0");
  const bool causal = kind == TRI_MASK_CAUSAL;
  const Schedule s = make_schedule(batch, heads_q, heads_kv, seqlen, TRI_KERNEL_BLOCK_Q, causal,
                                   causal ? seqlen : std::min(last_q, seqlen));
  const WorkItem w = schedule_item(s, bid);
  *b_out = w.b;
  *h_out = w.h;
  *qtile_out = w.t;
  *grid_out = s.grid;
  return TRI_OK;
}

extern "C" int tri_dyn_plan_sizes(const tri_attn_tensors* t, int64_t* workspace_bytes,
                                  int64_t* n_rows, int64_t* max_nnz) {
  clear_error();
  int st = validate_tensors(t);
  if (st != TRI_OK) return st;
  if (!workspace_bytes || !n_rows || !max_nnz)
    return fail(TRI_ERR_INVALID, "output pointers must be non-NULL");
  const int64_t nq = (t->seqlen + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  *workspace_bytes = dyn_workspace(t->batch, t->heads_q, t->heads_kv, t->head_dim, t->seqlen).total;
  *n_rows = static_cast<int64_t>(t->batch) * t->heads_q * nq;
  *max_nnz = static_cast<int64_t>(t->batch) * t->heads_q * causal_tiles(t->seqlen);
  return TRI_OK;
}

namespace {

// Validation of a dynamic plan's arguments except the workspace; fills the
// launch description (workspace pointers left unset).
int dyn_prepare(const tri_attn_tensors* t, const tri_dyn_params* dp, int32_t* d_row_ptr, int32_t* d_k_tile,
                uint8_t* d_flags, int64_t capacity, DynLaunch* a, DynWorkspace* ws) {
  int st = validate_tensors(t);
  if (st != TRI_OK) return st;
  if (!dp) return fail(TRI_ERR_INVALID, "dynamic-plan parameters pointer is NULL");
  if (!(dp->alpha >= 0.0f && dp->alpha <= 1.0f))
    return fail(TRI_ERR_INVALID, "alpha must be in [0, 1]");
  if (dp->n_probe != TRI_DYN_PROBES)
    return fail(TRI_ERR_UNSUPPORTED, "n_probe must be %d", TRI_DYN_PROBES);
  const int64_t N = t->seqlen;
  const int64_t nq = (N + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  const int64_t nkt = (N + TRI_KERNEL_BLOCK_K - 1) / TRI_KERNEL_BLOCK_K;
  const int64_t rows = static_cast<int64_t>(t->batch) * t->heads_q * nq;
  const int64_t need = static_cast<int64_t>(t->batch) * t->heads_q * causal_tiles(N);
  *ws = dyn_workspace(t->batch, t->heads_q, t->heads_kv, t->head_dim, N);
  if (need >= INT32_MAX || rows >= INT32_MAX)
    return fail(TRI_ERR_UNSUPPORTED, "list sizes exceed 2^31-1 entries");
  if (!d_row_ptr || !d_k_tile || !d_flags)
    return fail(TRI_ERR_INVALID, "output pointers must be non-NULL");
  if (!aligned(d_row_ptr, 4) || !aligned(d_k_tile, 4))
    return fail(TRI_ERR_INVALID, "row_ptr and k_tile must be 4-byte aligned");
  if (capacity < need)
    return fail(TRI_ERR_CAPACITY, "list capacity %lld, %lld needed", static_cast<long long>(capacity),
                static_cast<long long>(need));
  *a = DynLaunch{};
  a->q = t->q;
  a->k = t->k;
  memcpy(a->q_stride, t->q_stride, sizeof(a->q_stride));
  memcpy(a->k_stride, t->k_stride, sizeof(a->k_stride));
  a->batch = t->batch;
  a->heads_q = t->heads_q;
  a->heads_kv = t->heads_kv;
  a->head_dim = t->head_dim;
  a->seqlen = static_cast<int32_t>(N);
  a->nq = static_cast<int32_t>(nq);
  a->nkt = static_cast<int32_t>(nkt);
  a->words = static_cast<int32_t>((nkt + 31) / 32);
  a->n_rows = rows;
  a->n_pool_tiles = static_cast<int64_t>(t->batch) * t->heads_kv * nkt;
  a->scale = t->softmax_scale;
  a->alpha = dp->alpha;
  a->row_ptr = d_row_ptr;
  a->k_tile = d_k_tile;
  a->flags = d_flags;
  return TRI_OK;
}

void dyn_set_workspace(DynLaunch* a, const DynWorkspace& ws, void* base) {
  char* w = static_cast<char*>(base);
  a->pooled = w + ws.pooled;
  a->bitmap = reinterpret_cast<uint32_t*>(w + ws.bitmap);
  a->counts = reinterpret_cast<int32_t*>(w + ws.counts);
}

}  // namespace

extern "C" int tri_dyn_plan(const tri_attn_tensors* t, const tri_dyn_params* dp, void* d_workspace,
                            int64_t workspace_bytes, int32_t* d_row_ptr, int32_t* d_k_tile,
                            uint8_t* d_flags, int64_t capacity, void* stream) {
  clear_error();
  DynLaunch a;
  DynWorkspace ws;
  int st = dyn_prepare(t, dp, d_row_ptr, d_k_tile, d_flags, capacity, &a, &ws);
  if (st != TRI_OK) return st;
  if (!d_workspace) return fail(TRI_ERR_INVALID, "workspace pointer must be non-NULL");
  if (!aligned(d_workspace, 256)) return fail(TRI_ERR_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < ws.total)
    return fail(TRI_ERR_CAPACITY, "workspace of %lld bytes, %lld needed",
                static_cast<long long>(workspace_bytes), static_cast<long long>(ws.total));
  if (t->seqlen == 0) return TRI_OK;
  dyn_set_workspace(&a, ws, d_workspace);
  return launch_dyn_plan(a, stream);
}

extern "C" int tri_dyn_plan_noalloc(const tri_attn_tensors* t, const tri_dyn_params* dp, int32_t* d_row_ptr,
                                    int32_t* d_k_tile, uint8_t* d_flags, int64_t capacity, void* stream) {
  clear_error();
  DynLaunch a;
  DynWorkspace ws;
  int st = dyn_prepare(t, dp, d_row_ptr, d_k_tile, d_flags, capacity, &a, &ws);
  if (st != TRI_OK) return st;
  if (ws.total > TRI_DYN_SCRATCH_BYTES)
    return fail(TRI_ERR_CAPACITY,
                "the layer needs %lld bytes of workspace; the library-owned scratch holds %lld "
                "(use tri_dyn_plan with a caller workspace)",
                static_cast<long long>(ws.total), static_cast<long long>(TRI_DYN_SCRATCH_BYTES));
  if (t->seqlen == 0) return TRI_OK;
  void* base = nullptr;
  if ((st = dyn_scratch(&base)) != TRI_OK) return st;
  dyn_set_workspace(&a, ws, base);
  return launch_dyn_plan(a, stream);
}

extern "C" int tri_attn_prefill_lists(const tri_attn_tensors* t, const int32_t* d_row_ptr,
                                      const int32_t* d_k_tile, const uint8_t* d_flags,
                                      void* stream) {
  clear_error();
  int st = validate_tensors(t);
  if (st != TRI_OK) return st;
  if (!d_row_ptr || !d_k_tile || !d_flags)
    return fail(TRI_ERR_INVALID, "list arrays (row_ptr, k_tile, flags) must be non-NULL");
  if (!aligned(d_row_ptr, 4) || !aligned(d_k_tile, 4))
    return fail(TRI_ERR_INVALID, "row_ptr and k_tile must be 4-byte aligned");
  const int64_t nq = (t->seqlen + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  if (static_cast<int64_t>(t->batch) * t->heads_q * nq >= INT32_MAX)
    return fail(TRI_ERR_UNSUPPORTED, "list rows exceed 2^31-1");
  if (t->seqlen == 0) return TRI_OK;
  // causal schedule (longest lists first) and causal mask inside the listed tiles
  AttnLaunch a = make_launch(t, true, 0, 1, t->seqlen);
  a.causal = 0;
  a.row_ptr = d_row_ptr;
  a.k_tile = d_k_tile;
  a.flags = d_flags;
  a.list_batch_rows = t->heads_q * nq;
  a.list_head_rows = static_cast<int32_t>(nq);
  return launch_attn_fwd(a, stream);
}

extern "C" int tri_attn_prefill_heads(const tri_attn_tensors* t, const tri_mask_params* mp,
                                      const int32_t* d_head_sink, const int32_t* d_head_window,
                                      const int32_t* d_row_ptr, const int32_t* d_k_tile,
                                      const uint8_t* d_flags, void* stream) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if ((st = validate_tensors(t)) != TRI_OK) return st;
  if (mp->kind != TRI_MASK_TRIANGLE)
    return fail(TRI_ERR_INVALID, "per-head boundaries apply to the triangle mask");
  if (mp->block_q != TRI_KERNEL_BLOCK_Q || mp->block_k != TRI_KERNEL_BLOCK_K)
    return fail(TRI_ERR_UNSUPPORTED, "the kernel walks %dx%d tiles; plan has %dx%d",
                TRI_KERNEL_BLOCK_Q, TRI_KERNEL_BLOCK_K, mp->block_q, mp->block_k);
  if (mp->seqlen != t->seqlen)
    return fail(TRI_ERR_INVALID, "mask seqlen %lld differs from tensor seqlen %lld",
                static_cast<long long>(mp->seqlen), static_cast<long long>(t->seqlen));
  if (!d_head_sink || !d_head_window || !d_row_ptr || !d_k_tile || !d_flags)
    return fail(TRI_ERR_INVALID, "per-head arrays and plan arrays must be non-NULL");
  if (!aligned(d_head_sink, 4) || !aligned(d_head_window, 4) || !aligned(d_row_ptr, 4) ||
      !aligned(d_k_tile, 4))
    return fail(TRI_ERR_INVALID, "int32 arrays must be 4-byte aligned");
  if (t->seqlen == 0) return TRI_OK;
  const int64_t nq = (t->seqlen + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  AttnLaunch a = make_launch(t, false, mp->sink, mp->window, mp->last_q);
  a.row_ptr = d_row_ptr;
  a.k_tile = d_k_tile;
  a.flags = d_flags;
  a.list_batch_rows = 0;
  a.list_head_rows = static_cast<int32_t>(nq);
  a.head_sink = d_head_sink;
  a.head_window = d_head_window;
  return launch_attn_fwd(a, stream);
}

extern "C" int tri_attn_split_workspace_size(const tri_attn_tensors* t, const tri_mask_params* mp,
                                             int32_t chunk_tiles, int64_t* bytes) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if ((st = validate_tensors(t)) != TRI_OK) return st;
  if (!bytes) return fail(TRI_ERR_INVALID, "bytes must be non-NULL");
  if (mp->kind != TRI_MASK_TRIANGLE) return fail(TRI_ERR_INVALID, "the split applies to the triangle mask");
  if (chunk_tiles < 1) return fail(TRI_ERR_INVALID, "chunk_tiles must be >= 1");
  if (mp->seqlen != t->seqlen)
    return fail(TRI_ERR_INVALID, "mask seqlen %lld differs from tensor seqlen %lld",
                static_cast<long long>(mp->seqlen), static_cast<long long>(t->seqlen));
  int32_t n_heavy = 0, n_split = 1;
  if (t->seqlen > 0) split_shape(t->seqlen, mp->last_q, chunk_tiles, &n_heavy, &n_split);
  *bytes = split_workspace(t->batch, t->heads_q, t->head_dim, n_heavy, n_split).total;
  return TRI_OK;
}

extern "C" int tri_attn_prefill_split(const tri_attn_tensors* t, const tri_mask_params* mp,
                                      const int32_t* d_head_sink, const int32_t* d_head_window,
                                      const int32_t* d_row_ptr, const int32_t* d_k_tile,
                                      const uint8_t* d_flags, int32_t chunk_tiles, void* d_workspace,
                                      int64_t workspace_bytes, void* stream) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if ((st = validate_tensors(t)) != TRI_OK) return st;
  if (mp->kind != TRI_MASK_TRIANGLE) return fail(TRI_ERR_INVALID, "the split applies to the triangle mask");
  if (mp->block_q != TRI_KERNEL_BLOCK_Q || mp->block_k != TRI_KERNEL_BLOCK_K)
    return fail(TRI_ERR_UNSUPPORTED, "the kernel walks %dx%d tiles; plan has %dx%d",
                TRI_KERNEL_BLOCK_Q, TRI_KERNEL_BLOCK_K, mp->block_q, mp->block_k);
  if (mp->seqlen != t->seqlen)
    return fail(TRI_ERR_INVALID, "mask seqlen %lld differs from tensor seqlen %lld",
                static_cast<long long>(mp->seqlen), static_cast<long long>(t->seqlen));
  if (chunk_tiles < 1) return fail(TRI_ERR_INVALID, "chunk_tiles must be >= 1");
  if ((d_head_sink == nullptr) != (d_head_window == nullptr))
    return fail(TRI_ERR_INVALID, "per-head sink and window go together (both NULL for one plan)");
  if (!d_row_ptr || !d_k_tile || !d_flags)
    return fail(TRI_ERR_INVALID, "plan arrays (row_ptr, k_tile, flags) must be non-NULL");
  if (!aligned(d_row_ptr, 4) || !aligned(d_k_tile, 4) || (d_head_sink && !aligned(d_head_sink, 4)) ||
      (d_head_window && !aligned(d_head_window, 4)))
    return fail(TRI_ERR_INVALID, "int32 arrays must be 4-byte aligned");
  if (t->seqlen == 0) return TRI_OK;
  int32_t n_heavy = 0, n_split = 1;
  split_shape(t->seqlen, mp->last_q, chunk_tiles, &n_heavy, &n_split);
  const SplitWorkspace ws = split_workspace(t->batch, t->heads_q, t->head_dim, n_heavy, n_split);
  if (ws.total > 0) {
    if (!d_workspace || !aligned(d_workspace, 256))
      return fail(TRI_ERR_INVALID, "workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < ws.total)
      return fail(TRI_ERR_CAPACITY, "workspace of %lld bytes, %lld needed",
                  static_cast<long long>(workspace_bytes), static_cast<long long>(ws.total));
  }
  const int64_t nq = (t->seqlen + TRI_KERNEL_BLOCK_Q - 1) / TRI_KERNEL_BLOCK_Q;
  AttnLaunch a = make_launch(t, false, mp->sink, mp->window, mp->last_q);
  a.sched = make_schedule(t->batch, t->heads_q, t->heads_kv, t->seqlen, TRI_KERNEL_BLOCK_Q, false, a.last_q,
                          n_split);
  a.row_ptr = d_row_ptr;
  a.k_tile = d_k_tile;
  a.flags = d_flags;
  if (d_head_sink) {
    a.list_batch_rows = 0;
    a.list_head_rows = static_cast<int32_t>(nq);
    a.head_sink = d_head_sink;
    a.head_window = d_head_window;
  }
  a.chunk_tiles = chunk_tiles;
  if (ws.total > 0) {
    a.split_stats = reinterpret_cast<float*>(static_cast<char*>(d_workspace) + ws.stats);
    a.split_o = reinterpret_cast<float*>(static_cast<char*>(d_workspace) + ws.o);
  }
  if ((st = launch_attn_fwd(a, stream)) != TRI_OK) return st;
  return launch_split_merge(a, stream);
}

extern "C" int tri_attn_split_work_item(int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t seqlen,
                                        int64_t last_q, int32_t chunk_tiles, int64_t bid, int32_t* b_out,
                                        int32_t* h_out, int32_t* qtile_out, int32_t* chunk_out,
                                        int64_t* grid_out) {
  clear_error();
  if (!b_out || !h_out || !qtile_out || !chunk_out || !grid_out)
    return fail(TRI_ERR_INVALID, "output pointers must be non-NULL");
  if (batch < 1 || heads_q < 1 || heads_kv < 1 || heads_q % heads_kv)
    return fail(TRI_ERR_INVALID, "bad head counts");
  if (seqlen < 1 || seqlen >= kMaxSeqlen) return fail(TRI_ERR_INVALID, "bad seqlen");
  if (last_q < 0) return fail(TRI_ERR_INVALID, "last_q must be >= 0");
  if (chunk_tiles < 1) return fail(TRI_ERR_INVALID, "chunk_tiles must be >= 1");
  int32_t n_heavy = 0, n_split = 1;
  split_shape(seqlen, last_q, chunk_tiles, &n_heavy, &n_split);
  const Schedule s = make_schedule(batch, heads_q, heads_kv, seqlen, TRI_KERNEL_BLOCK_Q, false,
                                   std::min(last_q, seqlen), n_split);
  const WorkItem w = schedule_item(s, bid);
  *b_out = w.b;
  *h_out = w.h;
  *qtile_out = w.t;
  *chunk_out = w.c;
  *grid_out = s.grid;
  return TRI_OK;
}

extern "C" int tri_attn_quantize_k_sizes(const tri_attn_tensors* t, int64_t* k8_bytes,
                                         int64_t* n_scales) {
  clear_error();
  int st = validate_tensors(t);
  if (st != TRI_OK) return st;
  if (!k8_bytes || !n_scales) return fail(TRI_ERR_INVALID, "output pointers must be non-NULL");
  *k8_bytes = static_cast<int64_t>(t->batch) * t->heads_kv * t->seqlen * t->head_dim;
  *n_scales = static_cast<int64_t>(t->batch) * t->heads_kv *
              ((t->seqlen + TRI_KERNEL_BLOCK_K - 1) / TRI_KERNEL_BLOCK_K);
  return TRI_OK;
}

namespace {
int quantize_k(const tri_attn_tensors* t, void* d_out, float* d_scale, void* stream, bool fp4) {
  clear_error();
  int st = validate_tensors(t);
  if (st != TRI_OK) return st;
  if (!d_out || !d_scale) return fail(TRI_ERR_INVALID, "the K copy and d_scale must be non-NULL");
  if (!aligned(d_out, 16) || !aligned(d_scale, 4))
    return fail(TRI_ERR_INVALID, "the K copy must be 16-byte and d_scale 4-byte aligned");
  if (t->seqlen == 0) return TRI_OK;
  QuantLaunch a{};
  a.fp4 = fp4 ? 1 : 0;
  a.k = t->k;
  memcpy(a.k_stride, t->k_stride, sizeof(a.k_stride));
  a.heads_kv = t->heads_kv;
  a.head_dim = t->head_dim;
  a.seqlen = static_cast<int32_t>(t->seqlen);
  a.n_blocks = static_cast<int64_t>(t->batch) * t->heads_kv *
               ((t->seqlen + TRI_KERNEL_BLOCK_K - 1) / TRI_KERNEL_BLOCK_K);
  a.k8 = d_out;
  a.scale = d_scale;
  return launch_quantize_k(a, stream);
}
}  // namespace

extern "C" int tri_attn_quantize_k(const tri_attn_tensors* t, void* d_k8, float* d_scale, void* stream) {
  return quantize_k(t, d_k8, d_scale, stream, false);
}

extern "C" int tri_attn_quantize_k4_sizes(const tri_attn_tensors* t, int64_t* k4_bytes, int64_t* n_scales) {
  clear_error();
  int st = validate_tensors(t);
  if (st != TRI_OK) return st;
  if (!k4_bytes || !n_scales) return fail(TRI_ERR_INVALID, "output pointers must be non-NULL");
  *k4_bytes = static_cast<int64_t>(t->batch) * t->heads_kv * t->seqlen * (t->head_dim / 2);
  *n_scales = static_cast<int64_t>(t->batch) * t->heads_kv *
              ((t->seqlen + TRI_KERNEL_BLOCK_K - 1) / TRI_KERNEL_BLOCK_K);
  return TRI_OK;
}

extern "C" int tri_attn_quantize_k4(const tri_attn_tensors* t, void* d_k4, float* d_scale, void* stream) {
  return quantize_k(t, d_k4, d_scale, stream, true);
}

extern "C" int tri_attn_prefill_tiered(const tri_attn_tensors* t, const tri_mask_params* mp,
                                       const int32_t* d_head_low_dist, const void* d_k8,
                                       const float* d_scale, const int32_t* d_head_fp4_dist,
                                       const void* d_k4, const float* d_scale4,
                                       const int32_t* d_row_ptr, const int32_t* d_k_tile,
                                       const uint8_t* d_flags, void* stream) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if ((st = validate_tensors(t)) != TRI_OK) return st;
  if (mp->kind != TRI_MASK_TRIANGLE)
    return fail(TRI_ERR_INVALID, "precision tiers apply to the triangle mask");
  if (mp->block_q != TRI_KERNEL_BLOCK_Q || mp->block_k != TRI_KERNEL_BLOCK_K)
    return fail(TRI_ERR_UNSUPPORTED, "the kernel walks %dx%d tiles; plan has %dx%d",
                TRI_KERNEL_BLOCK_Q, TRI_KERNEL_BLOCK_K, mp->block_q, mp->block_k);
  if (mp->seqlen != t->seqlen)
    return fail(TRI_ERR_INVALID, "mask seqlen %lld differs from tensor seqlen %lld",
                static_cast<long long>(mp->seqlen), static_cast<long long>(t->seqlen));
  if (!d_head_low_dist || !d_k8 || !d_scale || !d_row_ptr || !d_k_tile || !d_flags)
    return fail(TRI_ERR_INVALID, "boundary, fp8 K, scale and plan arrays must be non-NULL");
  if (!aligned(d_head_low_dist, 4) || !aligned(d_k8, 16) || !aligned(d_scale, 4) ||
      !aligned(d_row_ptr, 4) || !aligned(d_k_tile, 4))
    return fail(TRI_ERR_INVALID, "misaligned array (fp8 K: 16 bytes, int32/float: 4 bytes)");
  const int fp4_given = (d_head_fp4_dist != nullptr) + (d_k4 != nullptr) + (d_scale4 != nullptr);
  if (fp4_given != 0 && fp4_given != 3)
    return fail(TRI_ERR_INVALID, "the fp4 boundary, fp4 K and its scales go together (all NULL: no fp4 tier)");
  if (fp4_given && (!aligned(d_head_fp4_dist, 4) || !aligned(d_k4, 16) || !aligned(d_scale4, 4)))
    return fail(TRI_ERR_INVALID, "misaligned fp4 array (fp4 K: 16 bytes, int32/float: 4 bytes)");
  if (t->seqlen * t->head_dim >= (int64_t(1) << 31))
    return fail(TRI_ERR_UNSUPPORTED, "seqlen x head_dim must be < 2^31 bytes of fp8 K per head");
  if (t->seqlen == 0) return TRI_OK;
  AttnLaunch a = make_launch(t, false, mp->sink, mp->window, mp->last_q);
  a.row_ptr = d_row_ptr;
  a.k_tile = d_k_tile;
  a.flags = d_flags;
  a.k8 = d_k8;
  a.k8_scale = d_scale;
  a.head_low_dist = d_head_low_dist;
  a.k4 = d_k4;
  a.k4_scale = d_scale4;
  a.head_fp4_dist = d_head_fp4_dist;
  return launch_attn_fwd(a, stream);
}
