// Internal declarations shared by the host planner, the ABI layer and the
// gfx950 kernel launcher of libtriattn.  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "tri_attn.h"

namespace triattn {

// Per-thread error message (tri_attn_last_error); returns `code`.
int fail(int code, const char* fmt, ...)
#if defined(__GNUC__)
    __attribute__((format(printf, 2, 3)))
#endif
    ;
void clear_error();

int validate_mask(const tri_mask_params* mp);

// ---------------------------------------------------------------- schedule
//
// Maps a launch block index to the (batch, query head, query tile) it
// computes.  MI355X hands consecutive workgroups of a launch to its 8 XCDs in
// turn (block b runs on XCD b % 8) and each XCD has its own L2, so blocks that
// share K/V tiles (the query heads of one KV group, neighbouring query tiles)
// are placed on the same XCD:
//   * each (batch, KV head) group is cut into S interleaved streams of query
//     tiles (position p goes to stream p % S), with S chosen so the number of
//     streams is a multiple of 8; XCD x owns streams [x*spx, (x+1)*spx);
//   * inside an XCD, blocks run position-major, then stream, then the G query
//     heads of the group, so the blocks in flight on one XCD work on the same
//     K/V window;
//   * an XCD places its blocks on its 32 CUs in a fixed rotation, in order,
//     waiting for the chosen CU to have room (measured on MI355X).  With G a
//     divisor of 32, head slot j of every position would land on the same
//     CUs, and heads of unequal cost (per-head windows) would leave most CUs
//     idle behind the busiest ones; so the head given to slot j rotates by one
//     per 32-block cycle of the XCD (the cycle of the position's first slot,
//     keeping the heads of a position a permutation);
//   * positions are ordered heaviest first: for the triangle mask the query
//     tiles holding last-Q rows (which read every earlier key) come first in
//     descending order, then the rest ascending; for the causal mask the
//     tiles run in descending order;
//   * with a split (n_split > 1, triangle only), each heavy tile becomes
//     n_split chunk items, chunk c walking list entries [c C, (c + 1) C) of
//     the tile's row (C = chunk_tiles); the chunk items come first.
// Positions past the last item of a stream leave the block idle (t = -1).
struct Schedule {
  int32_t batch, heads_q, heads_kv, group;  // group = heads_q / heads_kv
  int32_t n_qtiles;                          // query tiles of 128 rows
  int32_t causal;                            // 1: causal order, 0: triangle order
  int32_t n_heavy;                           // triangle: tiles with last-Q rows
  int32_t n_split;                           // chunk items per heavy tile (1: no split)
  int32_t streams;                           // S: streams per KV group
  int32_t streams_per_xcd;                   // spx
  int32_t positions;                         // P = ceil(items per group / S)
  int64_t grid;                              // 8 * spx * P * group
};

constexpr int kNumXcd = 8;
constexpr int kCusPerXcd = 32;

constexpr int32_t gcd_i32(int32_t a, int32_t b) {
  while (b) {
    const int32_t r = a % b;
    a = b;
    b = r;
  }
  return a;
}

// block_q: rows per query tile; last_q: clamped to [0, N]; n_split: chunk
// items per heavy triangle tile (1: none).
constexpr Schedule make_schedule(int32_t batch, int32_t heads_q, int32_t heads_kv, int64_t N,
                                 int32_t block_q, bool causal, int64_t last_q, int32_t n_split = 1) {
  Schedule s{};
  s.batch = batch;
  s.heads_q = heads_q;
  s.heads_kv = heads_kv;
  s.group = heads_q / heads_kv;
  s.n_qtiles = static_cast<int32_t>((N + block_q - 1) / block_q);
  s.causal = causal ? 1 : 0;
  if (causal || last_q <= 0) {
    s.n_heavy = causal ? s.n_qtiles : 0;
  } else {
    const int64_t first_heavy = (N - last_q) / block_q;  // tile of row N - last_q
    s.n_heavy = static_cast<int32_t>(s.n_qtiles - first_heavy);
  }
  s.n_split = (!causal && s.n_heavy > 0 && n_split > 1) ? n_split : 1;
  const int32_t n_groups = batch * heads_kv;
  s.streams = kNumXcd / gcd_i32(n_groups, kNumXcd);
  s.streams_per_xcd = n_groups * s.streams / kNumXcd;
  const int64_t items = static_cast<int64_t>(s.n_heavy) * (s.n_split - 1) + s.n_qtiles;
  s.positions = static_cast<int32_t>((items + s.streams - 1) / s.streams);
  s.grid = static_cast<int64_t>(kNumXcd) * s.streams_per_xcd * s.positions * s.group;
  return s;
}

struct WorkItem {
  int32_t b, h, t;  // t = -1: idle block
  int32_t c;        // chunk of a split heavy tile, or -1 (the whole row)
};

constexpr WorkItem schedule_item(const Schedule& s, int64_t bid) {
  const int64_t x = bid % kNumXcd;
  const int64_t u = bid / kNumXcd;
  const int64_t per_pos = static_cast<int64_t>(s.streams_per_xcd) * s.group;
  const int64_t pi = u / per_pos;
  const int64_t rem = u % per_pos;
  const int64_t si = rem / s.group;
  const int64_t cycle = (pi * per_pos + si * s.group) / kCusPerXcd;
  const int32_t hh = static_cast<int32_t>((rem % s.group + cycle) % s.group);
  const int64_t stream = x * s.streams_per_xcd + si;
  const int32_t grp = static_cast<int32_t>(stream / s.streams);
  const int64_t p = pi * s.streams + stream % s.streams;
  WorkItem w{-1, -1, -1, -1};
  const int64_t n_chunk_items = static_cast<int64_t>(s.n_heavy) * s.n_split;
  if (bid < 0 || bid >= s.grid || p >= n_chunk_items - s.n_heavy + s.n_qtiles) return w;
  int32_t t = -1;
  if (s.causal) {
    t = s.n_qtiles - 1 - static_cast<int32_t>(p);
  } else if (s.n_split > 1 && p < n_chunk_items) {
    t = s.n_qtiles - 1 - static_cast<int32_t>(p / s.n_split);
    w.c = static_cast<int32_t>(p % s.n_split);
  } else if (s.n_split == 1 && p < s.n_heavy) {
    t = s.n_qtiles - 1 - static_cast<int32_t>(p);
  } else {
    t = static_cast<int32_t>(p - (s.n_split > 1 ? n_chunk_items : s.n_heavy));
  }
  w.b = grp / s.heads_kv;
  w.h = (grp % s.heads_kv) * s.group + hh;
  w.t = t;
  return w;
}

// ---------------------------------------------------------------- launch

struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], lse_stride[2];
  int32_t head_dim;
  int32_t o_bf16;  // 1: bf16 output, 0: f32 output
  int32_t causal;  // 1: in-kernel causal tile range, 0: explicit tile list
  int32_t seqlen;  // N (validated < 2^30)
  int32_t sink, window, last_q;  // clamped to [0, N] ([1, N] for window)
  float scale;                   // softmax scale
  const int32_t* row_ptr;
  const int32_t* k_tile;
  const uint8_t* flags;
  // list row of (batch b, head h, query tile t):
  //   b * list_batch_rows + h * list_head_rows + t
  // (0, 0): one list for every (batch, head); (0, nq): per-head lists shared
  // by the batch; (heads_q * nq, nq): per-(batch, head) lists
  int64_t list_batch_rows;
  int32_t list_head_rows;
  // per-head sink and window (device, [heads_q]), or NULL for the layer's
  const int32_t* head_sink;
  const int32_t* head_window;
  // precision tiers (device; NULL k8 = off): fp8 K [B, Hkv, N, d bytes] in
  // the fp8 operand channel order, its per-key-tile scales [B, Hkv,
  // ceil(N / 64)], and the per-head LOW boundary [heads_q]
  const void* k8;
  const float* k8_scale;
  const int32_t* head_low_dist;
  // fp4 tier (NULL k4 = off): fp4 K [B, Hkv, N, d / 2 bytes], its scales, and
  // the per-head fp4 boundary (tiles at or beyond it are scored in fp4)
  const void* k4;
  const float* k4_scale;
  const int32_t* head_fp4_dist;
  // split of heavy tiles (sched.n_split > 1): chunk items write unnormalised
  // partials, item = ((b * heads_q + h) * n_heavy + (n_qtiles - 1 - t)) *
  // n_split + c: O [item][128][d] f32 and (m, l, lb) [item][3][128] f32
  int32_t chunk_tiles;
  float* split_o;
  float* split_stats;
  Schedule sched;
};

// Enqueue the gfx950 kernel; returns TRI_OK or TRI_ERR_HIP.
int launch_attn_fwd(const AttnLaunch& a, void* stream);

// Workspace of a split launch (byte offsets, each 256-aligned): per-row
// statistics, then partial outputs.
struct SplitWorkspace {
  int64_t n_items;  // batch * heads_q * n_heavy * n_split
  int64_t stats, o, total;
};
SplitWorkspace split_workspace(int64_t batch, int64_t heads_q, int64_t head_dim, int64_t n_heavy,
                               int64_t n_split);

// Enqueue the merge of the chunk partials into O and LSE (one thread per
// (heavy tile row, 4 channels)); returns TRI_OK or TRI_ERR_HIP.
int launch_split_merge(const AttnLaunch& a, void* stream);

// ---------------------------------------------------------------- dynamic plan

struct DynLaunch {
  const void* q;  // bf16 [B, Hq, N, d]
  const void* k;  // bf16 [B, Hkv, N, d]
  int64_t q_stride[3], k_stride[3];
  int32_t batch, heads_q, heads_kv, head_dim, seqlen;
  int32_t nq, nkt;       // query tiles, key tiles
  int32_t words;         // keep-bitmap words per row: ceil(nkt / 32)
  int64_t n_rows;        // batch * heads_q * nq
  int64_t n_pool_tiles;  // batch * heads_kv * nkt
  float scale, alpha;
  void* pooled;       // workspace: bf16 [B, Hkv, nkt, d]
  uint32_t* bitmap;   // workspace: [n_rows, words]
  int32_t* counts;    // workspace: [n_rows]
  int32_t* row_ptr;   // out: [n_rows + 1]
  int32_t* k_tile;    // out
  uint8_t* flags;     // out
};

// Workspace layout of the dynamic plan (byte offsets, each 256-aligned).
struct DynWorkspace {
  int64_t pooled, bitmap, counts, total;
};
DynWorkspace dyn_workspace(int64_t batch, int64_t heads_q, int64_t heads_kv, int64_t head_dim,
                           int64_t seqlen);

// Enqueue the four launches of the dynamic plan; returns TRI_OK or TRI_ERR_HIP.
int launch_dyn_plan(const DynLaunch& a, void* stream);

// Device address of the current GPU's library-owned workspace of
// TRI_DYN_SCRATCH_BYTES (tri_dyn_plan_noalloc); TRI_OK or TRI_ERR_HIP.
int dyn_scratch(void** ptr);

// ---------------------------------------------------------------- precision tiers

struct QuantLaunch {
  const void* k;  // bf16 [B, Hkv, N, d]
  int64_t k_stride[3];
  int32_t heads_kv, head_dim, seqlen;
  int64_t n_blocks;  // batch * heads_kv * ceil(N / 64): one scale per key tile
  int32_t fp4;       // 0: fp8 copy (d bytes per row), 1: fp4 copy (d / 2 bytes per row)
  void* k8;          // out: fp8 [B, Hkv, N, d bytes] or fp4 [B, Hkv, N, d / 2 bytes]
  float* scale;      // out: [B, Hkv, ceil(N / 64)], one per key tile
};

// Enqueue the fp8 quantization of K; returns TRI_OK or TRI_ERR_HIP.
int launch_quantize_k(const QuantLaunch& a, void* stream);

}  // namespace triattn
