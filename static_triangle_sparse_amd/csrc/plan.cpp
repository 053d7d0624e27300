// Host tile planner of the TriangleMix static mask.
//
// The triangle pattern (TriangleMix blog, "介绍"; 36kr interview, technical
// motivation) keeps, for query row i of an N-token prefill, the keys j <= i
// with j < sink (leading sink keys), i - j < window (diagonal window) or
// i >= N - last_q (final-aggregation rows); the middle Q-K region is dropped.
// Because the pattern is static, its tile list is computed once per shape on
// the host and the kernel walks it directly (index-driven skipping, as the
// FlashPrefill page's section 2.3 describes for block-sparse prefill).
//
// For query tile t with rows [r0, r1] the kept key tiles follow from the
// union of the row sets over the tile:
//   * causal, or r1 is a last-Q row:  every key tile up to r1 / block_k;
//   * otherwise: sink keys [0, min(sink, r1 + 1)) and window keys
//     [max(0, r0 - window + 1), r1] (the windows of consecutive rows overlap,
//     so their union is one interval).
// A kept tile [c0, c1] is FULL when every row keeps every column:
//   c1 < N and c1 <= r0 (under the diagonal of the first row), and every
//   non-last row i keeps it, i.e. c1 < sink (inside the sink), or
//   i <= c0 + window - 1 (inside the window), or i <= sink + window - 1 (the
//   sink and window intervals of row i touch, so the row keeps all j <= i).
//   The last two conditions are hardest for the largest non-last row.
#include <stdint.h>
#include <string.h>

#include <algorithm>

#include "tri_attn.h"
#include "tri_attn_internal.h"

namespace triattn {

namespace {

struct TileRange {
  int64_t lo, hi;  // inclusive; empty if hi < lo
};

// Kept key-tile ranges of query tile t (at most two, ascending, disjoint).
int kept_ranges(const tri_mask_params& mp, int64_t t, TileRange out[2]) {
  const int64_t N = mp.seqlen;
  const int64_t r0 = t * mp.block_q;
  const int64_t r1 = std::min(N, r0 + mp.block_q) - 1;
  const int64_t bk = mp.block_k;
  if (mp.kind == TRI_MASK_CAUSAL || r1 >= N - mp.last_q) {
    out[0] = {0, r1 / bk};
    return 1;
  }
  const int64_t sink_end = std::min(mp.sink, r1 + 1);  // exclusive key bound
  const int64_t win_lo = std::max<int64_t>(0, r0 - mp.window + 1);
  TileRange w = {win_lo / bk, r1 / bk};
  if (sink_end <= 0) {
    out[0] = w;
    return 1;
  }
  TileRange s = {0, (sink_end - 1) / bk};
  if (s.hi + 1 >= w.lo) {  // touching or overlapping: one range
    out[0] = {0, std::max(s.hi, w.hi)};
    return 1;
  }
  out[0] = s;
  out[1] = w;
  return 2;
}

uint8_t tile_flag(const tri_mask_params& mp, int64_t t, int64_t kt) {
  const int64_t N = mp.seqlen;
  const int64_t r0 = t * mp.block_q;
  const int64_t r1 = std::min(N, r0 + mp.block_q) - 1;
  const int64_t c0 = kt * mp.block_k;
  const int64_t c1 = c0 + mp.block_k - 1;
  if (c1 >= N || c1 > r0) return TRI_TILE_PARTIAL;
  if (mp.kind == TRI_MASK_CAUSAL) return TRI_TILE_FULL;
  const int64_t last_start = N - mp.last_q;      // first last-Q row
  const int64_t i_max = std::min(r1, last_start - 1);  // largest non-last row
  if (i_max < r0) return TRI_TILE_FULL;          // every row is a last-Q row
  if (c1 < mp.sink) return TRI_TILE_FULL;
  if (i_max <= c0 + mp.window - 1) return TRI_TILE_FULL;
  if (i_max <= mp.sink + mp.window - 1) return TRI_TILE_FULL;
  return TRI_TILE_PARTIAL;
}

}  // namespace

int validate_mask(const tri_mask_params* mp) {
  if (!mp) return fail(TRI_ERR_INVALID, "mask params pointer is NULL");
  if (mp->seqlen < 0) return fail(TRI_ERR_INVALID, "seqlen must be >= 0");
  if (mp->block_q < 1 || mp->block_k < 1)
    return fail(TRI_ERR_INVALID, "block_q and block_k must be >= 1");
  if (mp->kind != TRI_MASK_TRIANGLE && mp->kind != TRI_MASK_CAUSAL)
    return fail(TRI_ERR_INVALID, "kind must be TRI_MASK_TRIANGLE or TRI_MASK_CAUSAL");
  if (mp->reserved != 0) return fail(TRI_ERR_INVALID, "reserved field must be 0");
  if (mp->sink < 0) return fail(TRI_ERR_INVALID, "sink must be >= 0");
  if (mp->window < 1)
    return fail(TRI_ERR_INVALID, "window must be >= 1 (an empty window can leave a row with no key)");
  if (mp->last_q < 0) return fail(TRI_ERR_INVALID, "last_q must be >= 0");
  // keep every tile index and row_ptr entry inside int32
  const int64_t nq = (mp->seqlen + mp->block_q - 1) / mp->block_q;
  const int64_t nk = (mp->seqlen + mp->block_k - 1) / mp->block_k;
  if (nq >= INT32_MAX || nk >= INT32_MAX)
    return fail(TRI_ERR_UNSUPPORTED, "too many tiles for int32 indices");
  return TRI_OK;
}

}  // namespace triattn

using namespace triattn;

extern "C" int tri_attn_plan(const tri_mask_params* mp, int32_t* row_ptr, int32_t* k_tile,
                             uint8_t* flags, int64_t capacity, int32_t* n_qtiles_out,
                             int64_t* nnz_out) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if (!n_qtiles_out || !nnz_out)
    return fail(TRI_ERR_INVALID, "n_qtiles_out and nnz_out must be non-NULL");
  const bool sizing = !row_ptr && !k_tile && !flags;
  if (!sizing && (!row_ptr || !k_tile || !flags))
    return fail(TRI_ERR_INVALID, "row_ptr, k_tile and flags must be all NULL (sizing) or all non-NULL");
  if (!sizing && capacity < 0) return fail(TRI_ERR_INVALID, "capacity must be >= 0");

  const int64_t nq = (mp->seqlen + mp->block_q - 1) / mp->block_q;
  int64_t nnz = 0;
  for (int64_t t = 0; t < nq; ++t) {
    TileRange r[2];
    const int n = kept_ranges(*mp, t, r);
    for (int e = 0; e < n; ++e) nnz += r[e].hi - r[e].lo + 1;
  }
  *n_qtiles_out = static_cast<int32_t>(nq);
  *nnz_out = nnz;
  if (nnz >= INT32_MAX) return fail(TRI_ERR_UNSUPPORTED, "plan has more than 2^31-1 entries");
  if (sizing) return TRI_OK;
  if (capacity < nnz)
    return fail(TRI_ERR_CAPACITY, "capacity %lld is smaller than the plan's %lld entries",
                static_cast<long long>(capacity), static_cast<long long>(nnz));

  int64_t e = 0;
  row_ptr[0] = 0;
  for (int64_t t = 0; t < nq; ++t) {
    TileRange r[2];
    const int n = kept_ranges(*mp, t, r);
    for (int x = 0; x < n; ++x) {
      for (int64_t kt = r[x].lo; kt <= r[x].hi; ++kt, ++e) {
        k_tile[e] = static_cast<int32_t>(kt);
        flags[e] = tile_flag(*mp, t, kt);
      }
    }
    row_ptr[t + 1] = static_cast<int32_t>(e);
  }
  return TRI_OK;
}

extern "C" int tri_attn_plan_heads(const tri_mask_params* mp, int32_t heads, const int64_t* sink,
                                   const int64_t* window, int32_t* row_ptr, int32_t* k_tile,
                                   uint8_t* flags, int64_t capacity, int32_t* n_qtiles_out,
                                   int64_t* nnz_out) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if (mp->kind != TRI_MASK_TRIANGLE)
    return fail(TRI_ERR_INVALID, "per-head boundaries apply to the triangle mask");
  if (heads < 1) return fail(TRI_ERR_INVALID, "heads must be >= 1");
  if (!sink || !window) return fail(TRI_ERR_INVALID, "sink and window arrays must be non-NULL");
  if (!n_qtiles_out || !nnz_out)
    return fail(TRI_ERR_INVALID, "n_qtiles_out and nnz_out must be non-NULL");
  const bool sizing = !row_ptr && !k_tile && !flags;
  if (!sizing && (!row_ptr || !k_tile || !flags))
    return fail(TRI_ERR_INVALID, "row_ptr, k_tile and flags must be all NULL (sizing) or all non-NULL");
  if (!sizing && capacity < 0) return fail(TRI_ERR_INVALID, "capacity must be >= 0");
  for (int32_t h = 0; h < heads; ++h) {
    if (sink[h] < 0) return fail(TRI_ERR_INVALID, "sink[%d] must be >= 0", h);
    if (window[h] < 1) return fail(TRI_ERR_INVALID, "window[%d] must be >= 1", h);
    if (sink[h] > INT32_MAX || window[h] > INT32_MAX)
      return fail(TRI_ERR_UNSUPPORTED, "sink[%d] and window[%d] must fit in int32", h, h);
  }
  const int64_t nq = (mp->seqlen + mp->block_q - 1) / mp->block_q;
  if (nq * heads >= INT32_MAX) return fail(TRI_ERR_UNSUPPORTED, "too many list rows for int32");
  int64_t nnz = 0;
  for (int32_t h = 0; h < heads; ++h) {
    tri_mask_params m = *mp;
    m.sink = sink[h];
    m.window = window[h];
    for (int64_t t = 0; t < nq; ++t) {
      TileRange r[2];
      const int n = kept_ranges(m, t, r);
      for (int e = 0; e < n; ++e) nnz += r[e].hi - r[e].lo + 1;
    }
  }
  *n_qtiles_out = static_cast<int32_t>(nq);
  *nnz_out = nnz;
  if (nnz >= INT32_MAX) return fail(TRI_ERR_UNSUPPORTED, "plan has more than 2^31-1 entries");
  if (sizing) return TRI_OK;
  if (capacity < nnz)
    return fail(TRI_ERR_CAPACITY, "capacity %lld is smaller than the plan's %lld entries",
                static_cast<long long>(capacity), static_cast<long long>(nnz));
  int64_t e = 0;
  row_ptr[0] = 0;
  for (int32_t h = 0; h < heads; ++h) {
    tri_mask_params m = *mp;
    m.sink = sink[h];
    m.window = window[h];
    for (int64_t t = 0; t < nq; ++t) {
      TileRange r[2];
      const int n = kept_ranges(m, t, r);
      for (int x = 0; x < n; ++x) {
        for (int64_t kt = r[x].lo; kt <= r[x].hi; ++kt, ++e) {
          k_tile[e] = static_cast<int32_t>(kt);
          flags[e] = tile_flag(m, t, kt);
        }
      }
      row_ptr[h * nq + t + 1] = static_cast<int32_t>(e);
    }
  }
  return TRI_OK;
}

// Check of a caller's host plan before its device copy reaches a prefill
// call: the kernel trusts the arrays it walks.  Row r of the plan lists the
// key tiles of query tile t = r % nq; with per-head boundaries (heads > 0),
// head (r / nq) % heads's sink and window define its mask.  Every entry must
// be a key tile of the row's causal range, in strictly ascending order, that
// holds a kept pair of the mask, flagged exactly as tri_attn_plan flags it.
// A plan that lists only some kept tiles (a dynamic selection) passes when
// each listed tile is valid; a complete static plan is what tri_attn_plan
// returns.
extern "C" int tri_attn_check_plan(const tri_mask_params* mp, int32_t heads, const int64_t* sink,
                                   const int64_t* window, const int32_t* row_ptr, int64_t n_rows,
                                   const int32_t* k_tile, const uint8_t* flags, int64_t nnz) {
  clear_error();
  int st = validate_mask(mp);
  if (st != TRI_OK) return st;
  if (heads < 0) return fail(TRI_ERR_INVALID, "heads must be >= 0 (0: one mask for every row)");
  if (heads > 0 && (!sink || !window))
    return fail(TRI_ERR_INVALID, "per-head plans need the sink and window arrays");
  if (heads > 0 && mp->kind != TRI_MASK_TRIANGLE)
    return fail(TRI_ERR_INVALID, "per-head boundaries apply to the triangle mask");
  for (int32_t h = 0; h < heads; ++h)
    if (sink[h] < 0 || window[h] < 1)
      return fail(TRI_ERR_INVALID, "head %d: sink must be >= 0 and window >= 1", h);
  if (!row_ptr || (nnz > 0 && (!k_tile || !flags)))
    return fail(TRI_ERR_INVALID, "row_ptr (and k_tile, flags when nnz > 0) must be non-NULL");
  const int64_t nq = (mp->seqlen + mp->block_q - 1) / mp->block_q;
  if (nnz < 0 || n_rows < 0) return fail(TRI_ERR_INVALID, "n_rows and nnz must be >= 0");
  if (nq == 0 ? n_rows != 0 : n_rows % nq != 0)
    return fail(TRI_ERR_INVALID, "n_rows %lld is not a multiple of the %lld query tiles",
                static_cast<long long>(n_rows), static_cast<long long>(nq));
  if (row_ptr[0] != 0) return fail(TRI_ERR_INVALID, "row_ptr[0] is %d, not 0", row_ptr[0]);
  if (row_ptr[n_rows] != nnz)
    return fail(TRI_ERR_INVALID, "row_ptr[%lld] is %d, not nnz = %lld", static_cast<long long>(n_rows),
                row_ptr[n_rows], static_cast<long long>(nnz));
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
    if (e1 < e0 || e1 > nnz)
      return fail(TRI_ERR_INVALID, "row_ptr is not non-decreasing within [0, nnz] at row %lld",
                  static_cast<long long>(r));
    const int64_t t = r % nq;
    tri_mask_params m = *mp;
    if (heads > 0) {
      const int64_t h = (r / nq) % heads;
      m.sink = sink[h];
      m.window = window[h];
    }
    const int64_t r1 = std::min(mp->seqlen, (t + 1) * mp->block_q) - 1;
    TileRange kept[2];
    const int n_kept = kept_ranges(m, t, kept);
    for (int64_t e = e0; e < e1; ++e) {
      const int64_t kt = k_tile[e];
      if (kt < 0 || kt > r1 / mp->block_k)
        return fail(TRI_ERR_INVALID, "row %lld entry %lld: key tile %lld is outside 0..%lld",
                    static_cast<long long>(r), static_cast<long long>(e), static_cast<long long>(kt),
                    static_cast<long long>(r1 / mp->block_k));
      if (e > e0 && kt <= k_tile[e - 1])
        return fail(TRI_ERR_INVALID, "row %lld entry %lld: key tiles are not strictly ascending",
                    static_cast<long long>(r), static_cast<long long>(e));
      bool is_kept = false;
      for (int x = 0; x < n_kept; ++x) is_kept = is_kept || (kt >= kept[x].lo && kt <= kept[x].hi);
      if (!is_kept)
        return fail(TRI_ERR_INVALID, "row %lld entry %lld: key tile %lld holds no kept pair",
                    static_cast<long long>(r), static_cast<long long>(e), static_cast<long long>(kt));
      if (flags[e] != tile_flag(m, t, kt))
        return fail(TRI_ERR_INVALID, "row %lld entry %lld: key tile %lld flagged %d, the mask gives %d",
                    static_cast<long long>(r), static_cast<long long>(e), static_cast<long long>(kt),
                    flags[e], tile_flag(m, t, kt));
    }
  }
  return TRI_OK;
}
