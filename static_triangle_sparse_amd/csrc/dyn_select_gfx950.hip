// Dynamic block-sparse tile selection for the dense (shallow) layers on
// gfx950: FlashPrefill page, section 2.1 (evenly spread probe queries scored
// against key blocks replaced by their mean key, score and pooling fused),
// section 2.2 (keep a key block when its score reaches alpha times the
// largest score of its query block; no sort, no cumulative sum) and section
// 2.3 (the kept blocks are handed to the attention kernel as an index list).
//
// Blocks are the attention kernel's tiles (128 query rows x 64 keys).  For
// each (batch, query head, query tile):
//   * probes: rows t*128 + 8p (p = 0..15) that are < N;
//   * probe i sees the key tiles kt with 64 kt <= i; z = scale <q_i, kbar_kt>
//     with kbar_kt the mean key of tile kt, stored in bf16;
//   * score(kt) = sum over probes of softmax_kt(z) (the mean over probes has
//     the same ordering, and only the ratio to the maximum matters);
//   * kt is kept when score >= alpha * max score, and always when it crosses
//     the causal diagonal of the query tile (64 kt + 63 > 128 t).
// Output: a CSR list over rows r = (b * Hq + h) * nq + t, ascending key
// tiles, causal FULL/PARTIAL flags -- the list format the attention kernel
// walks.
//
// Four launches: pool (mean keys), select (scores -> keep bitmap + count per
// row), scan (counts -> row pointers), emit (bitmap -> list).  The select
// computes each probe logit twice (softmax sums, then scores); the keep
// decisions read the scores back from LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tri_attn_internal.h"

namespace triattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBq = TRI_KERNEL_BLOCK_Q;
constexpr int kBk = TRI_KERNEL_BLOCK_K;
constexpr int kProbes = TRI_DYN_PROBES;
constexpr int kProbeStep = kBq / kProbes;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bfloat16 bits, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- pool
// One wave per key tile (4 per workgroup); lane l owns channels 2l, 2l + 1.
// The fp32 sum of the tile's bf16 keys is exact for inputs whose magnitudes
// span fewer than 2^16; the mean is formed in double and rounded once to
// float, then to bf16.
template <int D>
__global__ __launch_bounds__(256) void dyn_pool_kernel(const DynLaunch a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (tile >= a.n_pool_tiles || lane >= D / 2) return;
  const int kt = static_cast<int>(tile % a.nkt);
  const int64_t bg = tile / a.nkt;
  const int b = static_cast<int>(bg / a.heads_kv), g = static_cast<int>(bg % a.heads_kv);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_stride[0] + g * a.k_stride[1] +
                       static_cast<int64_t>(kt) * kBk * a.k_stride[2] + 2 * lane;
  const int n = min(kBk, a.seqlen - kt * kBk);
  float s0 = 0.0f, s1 = 0.0f;
  for (int j = 0; j < n; ++j) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(kp + j * a.k_stride[2]);
    s0 += bf16_to_f32(w & 0xFFFFu);
    s1 += bf16_to_f32(w >> 16);
  }
  const float m0 = static_cast<float>(static_cast<double>(s0) / n);
  const float m1 = static_cast<float>(static_cast<double>(s1) / n);
  reinterpret_cast<uint32_t*>(a.pooled)[(tile * D + 2 * lane) / 2] = f32_to_bf16(m0) | (f32_to_bf16(m1) << 16);
}

// ---------------------------------------------------------------- select
// One workgroup (4 waves) per (batch, query head, group of kQT = 4
// consecutive query tiles t0 .. t0 + 3); blocks run the heaviest group (the
// most candidate tiles) first, and consecutive blocks cycle through the KV
// heads.  Every pooled key a workgroup reads scores the probes of all four
// query tiles, so the keys cross the L2 once per 64 probes.  Scores come from
// v_mfma_f32_16x16x32_bf16 on mini-groups of 16 key tiles: block rb of the A
// operand holds the 16 probes of query tile t0 + rb (zero rows for a missing
// tile or a probe >= N), the B operand the pooled keys of the 16 tiles; lane
// l then holds tile kt0 + l % 16 and, in register r of block rb, probe
// 4 (l / 16) + r of that query tile.  Wave w takes the mini-groups w, w + 4,
// ..., two at a time from two key buffers, each reloaded for the mini-group
// two steps on right after its use.
//
// The softmax of probe p over the tiles it sees is taken against one
// reference per probe, its logit on key tile 0 (every probe sees tile 0):
//   pass 1: l_p = sum over tiles of exp2(c z - c ref_p), summed over the
//           lanes and waves directly (one reference per probe);
//   pass 2: score(t, kt) = sum over the probes p of t of
//           exp2(c z - c ref_p - log2 l_p), written to LDS, and its maximum;
//   keep:   bits from the LDS scores (score >= alpha * max, or the tile
//           crosses the diagonal), one 32-bit word per 32 tiles and query tile.
// Softmax does not depend on the reference point, so this is the softmax of
// the definition.  A logit more than 64 / c above its reference (exp2
// range) sends the workgroup through an exact-max pass first, which makes
// the per-probe maximum the reference.  Layers with more candidate tiles
// than the LDS score buffer holds recompute the scores for the keep bits.
constexpr int kQT = 4;                // query tiles per workgroup
constexpr int kLdsScoreTiles = 4096;  // 64 KiB of scores (four query tiles)
constexpr float kRefMargin = 64.0f;   // log2 units a logit may exceed its reference by
constexpr int kMg = 16;               // key tiles per mini-group
constexpr int kPr = 4 * kQT;          // probe registers per lane

template <int D>
struct Select {
  static constexpr int kSteps = D / 32;  // k-steps of 32 channels

  struct Ctx {
    bf16x8 q[kQT][kSteps];  // probe operand (A), block rb = query tile t0 + rb
    const uint16_t* kbar;   // pooled keys of the query's KV head
    int nc;                 // candidate key tiles (of the last tile of the group)
    int t0;                 // first query tile of the group
    int n_qt;               // query tiles of the group that exist
    int n;                  // N
    float c;                // scale * log2(e)
    int col, quad;          // lane % 16 (tile), lane / 16 (probe quad)
  };

  struct Keys {
    u32x4 w[kSteps];
  };

  // Keys of tiles kt0 + col; a tile past the candidates reads the last
  // candidate instead (its logits are masked to -inf), so that the loads
  // carry no branch and the walk's waits can count them exactly.
  static __device__ __forceinline__ Keys load(const Ctx& cx, int kt0) {
    Keys k;
    const int kt = min(kt0 + cx.col, cx.nc - 1);
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      k.w[s] = *reinterpret_cast<const u32x4*>(cx.kbar + static_cast<int64_t>(kt) * D + s * 32 + cx.quad * 8);
    return k;
  }

  // Pooled key of tile 0 in every column: each lane's registers then hold
  // its probes' logits on tile 0.
  static __device__ __forceinline__ Keys load_tile0(const Ctx& cx) {
    Keys k;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      k.w[s] = *reinterpret_cast<const u32x4*>(cx.kbar + s * 32 + cx.quad * 8);
    return k;
  }

  // raw logits <q_p, kbar> (scale not applied): z[4 rb + r]
  static __device__ __forceinline__ void raw(const Ctx& cx, const Keys& k, float (&z)[kPr]) {
#pragma unroll
    for (int rb = 0; rb < kQT; ++rb) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cx.q[rb][s], __builtin_bit_cast(bf16x8, k.w[s]), acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) z[4 * rb + r] = acc[r];
    }
  }

  // probe (0 .. 16 kQT - 1 over the group) and row of register x = 4 rb + r
  static __device__ __forceinline__ int probe_of(const Ctx& cx, int x) { return 16 * (x >> 2) + 4 * cx.quad + (x & 3); }
  static __device__ __forceinline__ int row_of(const Ctx& cx, int x) {
    return (cx.t0 + (x >> 2)) * kBq + (4 * cx.quad + (x & 3)) * kProbeStep;
  }
  // the probe of register x exists (its query tile exists, its row < N)
  static __device__ __forceinline__ bool probe_exists(const Ctx& cx, int x) {
    return (x >> 2) < cx.n_qt && row_of(cx, x) < cx.n;
  }

  // Raw logits z of a mini-group (the caller forms c z - c ref with one
  // fma), -inf where the probe does not exist or does not see the tile
  // (64 kt > its row) or the tile is past the candidates.  Only mini-groups
  // near the diagonal or the end need the test; elsewhere a probe that does
  // not exist (zero query) has z = 0 and weight 0 (its reference is -inf in
  // the score pass).
  static __device__ __forceinline__ void logits(const Ctx& cx, const Keys& k, int kt0, float (&z)[kPr]) {
    raw(cx, k, z);
    const bool clear = kt0 + kMg - 1 < cx.nc && (kt0 + kMg - 1) * kBk <= cx.t0 * kBq;
    if (!clear) {
      const int kt = kt0 + cx.col;
#pragma unroll
      for (int x = 0; x < kPr; ++x)
        z[x] = (probe_exists(cx, x) && kt < cx.nc && kt * kBk <= row_of(cx, x)) ? z[x] : -INFINITY;
    }
  }

  // Walk this wave's mini-groups (gi = wave, wave + 4, ...) two at a time,
  // each of two key buffers reloaded right after its use for the mini-group
  // two steps on.  Fixed buffers and unconditional loads: a rotation of
  // buffers compiles to register moves at the loop head and a conditional
  // load to a branch, and either makes the loop wait for every load in
  // flight instead of the one it needs.
  template <class F>
  static __device__ __forceinline__ void walk(const Ctx& cx, int wave, int n_mg, F&& f) {
    if (wave >= n_mg) return;
    Keys ka = load(cx, wave * kMg);
    Keys kb = load(cx, (wave + 4) * kMg);
    int gi = wave;
    for (; gi + 4 < n_mg; gi += 8) {
      float z[kPr];
      logits(cx, ka, gi * kMg, z);
      f(gi, z);
      __builtin_amdgcn_sched_barrier(0);
      ka = load(cx, (gi + 8) * kMg);
      __builtin_amdgcn_sched_barrier(0);
      float y[kPr];
      logits(cx, kb, (gi + 4) * kMg, y);
      f(gi + 4, y);
      __builtin_amdgcn_sched_barrier(0);
      kb = load(cx, (gi + 12) * kMg);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (gi < n_mg) {
      float z[kPr];
      logits(cx, ka, gi * kMg, z);
      f(gi, z);
    }
  }
};

// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48]: the sum over the four probe quads
// of a tile's column (v_permlane16_swap, then v_permlane32_swap)
__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
__global__ __launch_bounds__(256) void dyn_select_kernel(const DynLaunch a) {
  using S = Select<D>;
  extern __shared__ float score_lds[];  // [kQT][words * 32] when the scores fit
  __shared__ float red_l[4][16 * kQT];
  __shared__ float red_m[4][16 * kQT];
  __shared__ float red_max[4][kQT];
  __shared__ int red_cnt[4][kQT];

  const int groups = (a.nq + kQT - 1) / kQT;
  const int64_t n_bh = a.n_rows / a.nq;  // batch * heads_q
  const int u = groups - 1 - static_cast<int>(blockIdx.x / n_bh);
  // consecutive blocks cycle through the KV heads
  const int64_t i_bh = blockIdx.x % n_bh;
  const int G = a.heads_q / a.heads_kv;
  const int g = static_cast<int>(i_bh % a.heads_kv);
  const int64_t j_bh = i_bh / a.heads_kv;
  const int b = static_cast<int>(j_bh / G);
  const int h = g * G + static_cast<int>(j_bh % G);
  const int N = a.seqlen;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = kQT * u;

  typename S::Ctx cx;
  cx.col = lane & 15;
  cx.quad = lane >> 4;
  cx.t0 = t0;
  cx.n = N;
  cx.n_qt = min(kQT, a.nq - t0);
  cx.nc = (min(N, (t0 + cx.n_qt) * kBq) - 1) / kBk + 1;
  cx.c = a.scale * kLog2e;
  cx.kbar = static_cast<const uint16_t*>(a.pooled) + (static_cast<int64_t>(b) * a.heads_kv + g) * a.nkt * D;
  // A operand: lane l holds probe l % 16 of block rb, channels 32 s + 8 (l / 16) .. + 7
#pragma unroll
  for (int rb = 0; rb < kQT; ++rb) {
    const int qr = (t0 + rb) * kBq + cx.col * kProbeStep;
    const bool valid = rb < cx.n_qt && qr < N;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_stride[0] + h * a.q_stride[1] +
                         static_cast<int64_t>(valid ? qr : 0) * a.q_stride[2] + cx.quad * 8;
#pragma unroll
    for (int s = 0; s < S::kSteps; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (valid) w = *reinterpret_cast<const u32x4*>(qp + s * 32);
      cx.q[rb][s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const int n_mg = (cx.nc + kMg - 1) / kMg;
  const bool lds_scores = a.words * 32 <= kLdsScoreTiles;
  const int tiles_lds = a.words * 32;

  // references: each probe's logit on tile 0, as -c ref
  float nref[kPr];
  {
    float z0[kPr];
    S::raw(cx, S::load_tile0(cx), z0);
#pragma unroll
    for (int x = 0; x < kPr; ++x) nref[x] = -z0[x] * cx.c;
  }

  // pass 1: this lane's share of l_p, and the largest c z - c ref it met
  float l[kPr];
  float over = -INFINITY;
  auto sum_pass = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < kPr; ++x) l[x] = 0.0f;
    over = -INFINITY;
    S::walk(cx, wave, n_mg, [&](int, const float (&z)[kPr]) {
#pragma unroll
      for (int x = 0; x < kPr; ++x) {
        const float e = fmaf(z[x], cx.c, nref[x]);
        over = fmaxf(over, e);
        l[x] += __builtin_amdgcn_exp2f(e);
      }
    });
  };
  sum_pass();
  if (__syncthreads_or(over > kRefMargin)) {
    // a logit far above its reference: take each probe's exact maximum as
    // the reference instead, then sum again (every term <= 1)
    float mx[kPr];
#pragma unroll
    for (int x = 0; x < kPr; ++x) mx[x] = -INFINITY;
    S::walk(cx, wave, n_mg, [&](int, const float (&z)[kPr]) {
#pragma unroll
      for (int x = 0; x < kPr; ++x) mx[x] = fmaxf(mx[x], z[x] * cx.c);
    });
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int x = 0; x < kPr; ++x) mx[x] = fmaxf(mx[x], __shfl_xor(mx[x], off));
    if (cx.col == 0) {
#pragma unroll
      for (int x = 0; x < kPr; ++x) red_m[wave][S::probe_of(cx, x)] = mx[x];
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kPr; ++x) {
      const int p = S::probe_of(cx, x);
      const float m = fmaxf(fmaxf(red_m[0][p], red_m[1][p]), fmaxf(red_m[2][p], red_m[3][p]));
      nref[x] = m == -INFINITY ? 0.0f : -m;  // m is already in units of c z
    }
    sum_pass();
  }
  // l_p over the 16 lanes of each probe quad (same probes, other tiles), then
  // over the waves
#pragma unroll
  for (int off = 1; off < 16; off <<= 1)
#pragma unroll
    for (int x = 0; x < kPr; ++x) l[x] += __shfl_xor(l[x], off);
  if (cx.col == 0) {
#pragma unroll
    for (int x = 0; x < kPr; ++x) red_l[wave][S::probe_of(cx, x)] = l[x];
  }
  __syncthreads();
  // the normalisation 1 / l_p joins the exponent: exp2(c z - c ref - log2 l);
  // a probe that does not exist weighs nothing
#pragma unroll
  for (int x = 0; x < kPr; ++x) {
    const int p = S::probe_of(cx, x);
    const float ll = (red_l[0][p] + red_l[1][p]) + (red_l[2][p] + red_l[3][p]);
    nref[x] = (ll > 0.0f && S::probe_exists(cx, x)) ? nref[x] - __log2f(ll) : -INFINITY;
  }

  // score of this lane's tile for query tile t0 + rb, in every lane of the
  // tile's column
  auto score_rb = [&](const float (&z)[kPr], int rb) __attribute__((always_inline)) -> float {
    float p = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) p += __builtin_amdgcn_exp2f(fmaf(z[4 * rb + r], cx.c, nref[4 * rb + r]));
    return quad_sum(p);
  };

  // pass 2: scores (to LDS when they fit) and their maximum per query tile
  float smax[kQT];
#pragma unroll
  for (int rb = 0; rb < kQT; ++rb) smax[rb] = 0.0f;
  S::walk(cx, wave, n_mg, [&](int gi, const float (&z)[kPr]) {
    const int kt = gi * kMg + cx.col;
    float mine = 0.0f;
#pragma unroll
    for (int rb = 0; rb < kQT; ++rb) {
      const float sc = score_rb(z, rb);
      smax[rb] = fmaxf(smax[rb], sc);
      mine = cx.quad == rb ? sc : mine;
    }
    // quad q of the column stores query tile t0 + q's score (kQT = 4 quads)
    if (lds_scores) score_lds[cx.quad * tiles_lds + kt] = mine;
  });
#pragma unroll
  for (int off = 1; off < 16; off <<= 1)
#pragma unroll
    for (int rb = 0; rb < kQT; ++rb) smax[rb] = fmaxf(smax[rb], __shfl_xor(smax[rb], off));
  if (lane == 0) {
#pragma unroll
    for (int rb = 0; rb < kQT; ++rb) red_max[wave][rb] = smax[rb];
  }
  __syncthreads();

  // keep bits, one 32-bit word per 32 tiles, two query tiles per ballot:
  // lanes 0..31 decide tile t0 + 2 j's tiles, lanes 32..63 t0 + 2 j + 1's
  const int64_t row0 = (static_cast<int64_t>(b) * a.heads_q + h) * a.nq + t0;
  const int hi = lane >> 5, l32 = lane & 31;
  const int n_words = (cx.nc + 31) / 32;
  int count[kQT];
#pragma unroll
  for (int rb = 0; rb < kQT; ++rb) count[rb] = 0;
  if (lds_scores) __syncthreads();  // every score written
#pragma unroll
  for (int j = 0; j < kQT / 2; ++j) {
    const int rb = 2 * j + hi;  // this lane's query tile of the pair
    const int tq = t0 + rb;
    const int nc_q = rb < cx.n_qt ? (min(N, (tq + 1) * kBq) - 1) / kBk + 1 : 0;
    const float thr = a.alpha * fmaxf(fmaxf(red_max[0][rb], red_max[1][rb]), fmaxf(red_max[2][rb], red_max[3][rb]));
    const int nc_lo = 2 * j < cx.n_qt ? (min(N, (t0 + 2 * j + 1) * kBq) - 1) / kBk + 1 : 0;
    for (int wi = wave; wi < n_words; wi += 4) {
      float sc;
      if (lds_scores) {
        sc = score_lds[rb * tiles_lds + wi * 32 + l32];
      } else {
        // recompute: mini-groups 2 wi and 2 wi + 1 of word wi; this lane's
        // tile l32 lies in the one of parity l32 / 16
        float s2[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int gi = 2 * wi + half;
          float z[kPr];
          S::logits(cx, S::load(cx, gi * kMg), gi * kMg, z);
          float v = 0.0f;
#pragma unroll
          for (int q = 0; q < kQT; ++q) {
            const float s_q = score_rb(z, q);
            v = rb == q ? s_q : v;
          }
          s2[half] = v;
        }
        sc = (l32 >> 4) == 0 ? s2[0] : s2[1];
      }
      const int kt = wi * 32 + l32;
      const bool keep = kt < nc_q && (sc >= thr || kt * kBk + kBk - 1 > tq * kBq);
      const uint64_t m = __ballot(keep);
      const uint32_t w0 = static_cast<uint32_t>(m), w1 = static_cast<uint32_t>(m >> 32);
      if (lane == 0) {
        if (wi * 32 < nc_lo) a.bitmap[(row0 + 2 * j) * a.words + wi] = w0;
        if (2 * j + 1 < cx.n_qt) a.bitmap[(row0 + 2 * j + 1) * a.words + wi] = w1;
      }
      count[2 * j] += __builtin_popcount(w0);
      count[2 * j + 1] += __builtin_popcount(w1);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int rb = 0; rb < kQT; ++rb) red_cnt[wave][rb] = count[rb];
  }
  __syncthreads();
  if (threadIdx.x < kQT && static_cast<int>(threadIdx.x) < cx.n_qt) {
    const int rb = threadIdx.x;
    a.counts[row0 + rb] = red_cnt[0][rb] + red_cnt[1][rb] + red_cnt[2][rb] + red_cnt[3][rb];
  }
}

// ---------------------------------------------------------------- scan
// Exclusive prefix sum of the per-row counts into row pointers (one
// workgroup of 1024 threads, each summing a contiguous segment).
__global__ __launch_bounds__(1024) void dyn_scan_kernel(const DynLaunch a) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int64_t R = a.n_rows;
  const int64_t seg = (R + 1023) / 1024;
  const int64_t s0 = min(R, tid * seg), s1 = min(R, s0 + seg);
  int sum = 0;
  for (int64_t i = s0; i < s1; ++i) sum += a.counts[i];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;  // exclusive prefix of this segment
  for (int64_t i = s0; i < s1; ++i) {
    a.row_ptr[i] = run;
    run += a.counts[i];
  }
  if (tid == 1023) a.row_ptr[R] = part[1023];
}

// ---------------------------------------------------------------- emit
// One wave per row, 64 key tiles per step: lane l decides tile c0 + l from
// the row's keep bits, and the kept tiles of the step go to consecutive list
// positions (each lane's rank among the kept lanes below it).
__global__ __launch_bounds__(256) void dyn_emit_kernel(const DynLaunch a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (row >= a.n_rows) return;
  const int t = static_cast<int>(row % a.nq);
  const int nc = (min(a.seqlen, (t + 1) * kBq) - 1) / kBk + 1;
  const uint32_t* bits = a.bitmap + row * a.words;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int out = a.row_ptr[row];
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const int kt = c0 + lane;
    const bool keep = kt < nc && ((bits[kt >> 5] >> (kt & 31)) & 1u);
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int pos = out + __popcll(m & below);
      a.k_tile[pos] = kt;
      a.flags[pos] = kt * kBk + kBk - 1 > t * kBq ? TRI_TILE_PARTIAL : TRI_TILE_FULL;
    }
    out += __popcll(m);
  }
}

template <int D>
int launch_d(const DynLaunch& a, hipStream_t stream) {
  const int64_t pool_blocks = (a.n_pool_tiles + 3) / 4;
  hipLaunchKernelGGL(dyn_pool_kernel<D>, dim3(static_cast<unsigned>(pool_blocks)), dim3(256), 0, stream, a);
  const int64_t select_blocks = a.n_rows / a.nq * ((a.nq + kQT - 1) / kQT);
  // LDS for the scores of the query tiles of a group, when they fit
  const size_t score_bytes = a.words * 32 <= kLdsScoreTiles ? kQT * sizeof(float) * a.words * 32 : 0;
  hipLaunchKernelGGL(dyn_select_kernel<D>, dim3(static_cast<unsigned>(select_blocks)), dim3(256), score_bytes,
                     stream, a);
  hipLaunchKernelGGL(dyn_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  hipLaunchKernelGGL(dyn_emit_kernel, dim3(static_cast<unsigned>((a.n_rows + 3) / 4)), dim3(256), 0, stream,
                     a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(TRI_ERR_HIP, "dynamic plan launch failed: %s", hipGetErrorString(err));
  return TRI_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// Workspace of tri_dyn_plan_noalloc: one array per GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in; the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is handed to kernels.
static __device__ __align__(256) char scratch[TRI_DYN_SCRATCH_BYTES];

int dyn_scratch(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(TRI_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(TRI_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return fail(TRI_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(err));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TRI_OK;
}

int launch_dyn_plan(const DynLaunch& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.head_dim == 128) return launch_d<128>(a, s);
  if (a.head_dim == 64) return launch_d<64>(a, s);
  return fail(TRI_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

}  // namespace triattn
