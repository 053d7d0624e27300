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
// row), scan (counts -> row pointers), emit (bitmap -> list).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tri_attn_internal.h"

namespace triattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
// One workgroup (4 waves) per (batch, query head, pair of query tiles t0 =
// 2u, t1 = 2u + 1).  Scores come from v_mfma_f32_32x32x16_bf16 with the 32
// probes of the pair as the A rows (rows 0..15: t0, rows 16..31: t1; rows of
// a missing tile or a probe >= N are zero) and the pooled keys of 32 tiles as
// the B columns: lane l then holds tile kt0 + l % 32, and register r holds
// row 8 (r >> 2) + 4 (l >> 5) + (r & 3) -- registers 0..7 probes of t0,
// 8..15 probes of t1.  Wave w takes the 32-tile groups w, w + 4, ..., with the
// next group's pooled keys loaded while the current one is scored.  Three
// passes recompute the scores: per-probe softmax max and sum, the maximum
// tile score of each query tile, the keep bits (one 32-bit word per group
// and query tile).
template <int D>
struct Select {
  static constexpr int kSteps = D / 16;

  struct Ctx {
    bf16x8 q[kSteps];    // probe operand (A)
    int probe_row[16];   // row of register r's probe (INT32_MIN: none)
    const uint16_t* kbar;  // pooled keys of the query's KV head
    int nc;              // candidate key tiles (of the later tile of the pair)
    float c;             // scale * log2(e)
    int l32, hi;
  };

  struct Keys {
    u32x4 w[kSteps];
  };

  static __device__ __forceinline__ Keys load(const Ctx& cx, int kt0) {
    Keys k;
    const int kt = kt0 + cx.l32;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (kt < cx.nc)
        w = *reinterpret_cast<const u32x4*>(cx.kbar + static_cast<int64_t>(kt) * D + s * 16 + cx.hi * 8);
      k.w[s] = w;
    }
    return k;
  }

  // z (log2 units) of this lane's 16 probes against tile kt0 + l32; -inf where
  // the probe does not exist or does not see the tile
  static __device__ __forceinline__ void logits(const Ctx& cx, const Keys& k, int kt0, float (&z)[16]) {
    const int kt = kt0 + cx.l32;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cx.q[s], __builtin_bit_cast(bf16x8, k.w[s]), acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool sees = kt < cx.nc && kt * kBk <= cx.probe_row[r];
      z[r] = sees ? acc[r] * cx.c : -INFINITY;
    }
  }

  // Score of this lane's tile for the probes in registers r0 .. r0 + 7: sum
  // of exp2(z - m) / l.  Contraction is off so that every pass computes
  // bit-identical scores.
  static __device__ __forceinline__ float partial_score(const float (&z)[16], const float (&m)[16],
                                                        const float (&inv_l)[16], int r0) {
#pragma clang fp contract(off)
    float e[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
      e[r] = z[r0 + r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(z[r0 + r] - m[r0 + r]) * inv_l[r0 + r];
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }

  // Walk this wave's groups with the next group's keys in flight.
  template <class F>
  static __device__ __forceinline__ void walk(const Ctx& cx, int wave, int n_groups, F&& f) {
    if (wave >= n_groups) return;
    Keys cur = load(cx, wave * 32);
    for (int gi = wave; gi < n_groups; gi += 4) {
      Keys nxt;
      if (gi + 4 < n_groups) nxt = load(cx, (gi + 4) * 32);
      float z[16];
      logits(cx, cur, gi * 32, z);
      f(gi, z);
      cur = nxt;
    }
  }
};

// row of register r of lane half hi
__device__ __forceinline__ int reg_row(int r, int hi) { return 8 * ((r & 7) >> 2) + 4 * hi + (r & 3) + 16 * (r >> 3); }

template <int D>
__global__ __launch_bounds__(256) void dyn_select_kernel(const DynLaunch a) {
  using S = Select<D>;
  __shared__ float red[4][32][2];
  __shared__ float red_max[4][2];
  __shared__ int red_cnt[4][2];

  const int pairs = (a.nq + 1) / 2;
  const int u = static_cast<int>(blockIdx.x % pairs);
  const int64_t bh = blockIdx.x / pairs;
  const int h = static_cast<int>(bh % a.heads_q), b = static_cast<int>(bh / a.heads_q);
  const int g = h / (a.heads_q / a.heads_kv);
  const int N = a.seqlen;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = 2 * u;
  const bool has_t1 = t0 + 1 < a.nq;

  typename S::Ctx cx;
  cx.l32 = lane & 31;
  cx.hi = lane >> 5;
  const int nc0 = (min(N, (t0 + 1) * kBq) - 1) / kBk + 1;
  const int nc1 = has_t1 ? (min(N, (t0 + 2) * kBq) - 1) / kBk + 1 : 0;
  cx.nc = max(nc0, nc1);
  cx.c = a.scale * kLog2e;
  cx.kbar = static_cast<const uint16_t*>(a.pooled) + (static_cast<int64_t>(b) * a.heads_kv + g) * a.nkt * D;
  {
    // A operand: lane l holds probe row l % 32, channels 16 s + 8 hi .. + 7
    const int row = cx.l32;
    const int qr = (t0 + (row >> 4)) * kBq + (row & 15) * kProbeStep;
    const bool valid = (row < 16 || has_t1) && qr < N;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + b * a.q_stride[0] + h * a.q_stride[1] +
                         static_cast<int64_t>(valid ? qr : 0) * a.q_stride[2] + cx.hi * 8;
#pragma unroll
    for (int s = 0; s < S::kSteps; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (valid) w = *reinterpret_cast<const u32x4*>(qp + s * 16);
      cx.q[s] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pr = reg_row(r, cx.hi);
      const int rr = (t0 + (pr >> 4)) * kBq + (pr & 15) * kProbeStep;
      cx.probe_row[r] = ((pr < 16 || has_t1) && rr < N) ? rr : INT32_MIN;
    }
  }
  const int n_groups = (cx.nc + 31) / 32;

  // pass 1: per-probe max and sum of exp2(z - max) over the tiles it sees
  float m[16], l[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
  }
  S::walk(cx, wave, n_groups, [&](int, const float (&z)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (z[r] == -INFINITY) continue;
      const float mn = fmaxf(m[r], z[r]);
      l[r] = l[r] * __builtin_amdgcn_exp2f(m[r] - mn) + __builtin_amdgcn_exp2f(z[r] - mn);
      m[r] = mn;
    }
  });
  // combine over the 32 lanes of each half-wave (same probes, other tiles)
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float mo = __shfl_xor(m[r], off), lo = __shfl_xor(l[r], off);
      const float mn = fmaxf(m[r], mo);
      if (mn != -INFINITY) {
        l[r] = l[r] * __builtin_amdgcn_exp2f(m[r] - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
        m[r] = mn;
      }
    }
  }
  if (cx.l32 == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pr = reg_row(r, cx.hi);
      red[wave][pr][0] = m[r];
      red[wave][pr][1] = l[r];
    }
  }
  __syncthreads();
  float inv_l[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pr = reg_row(r, cx.hi);
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][pr][0]);
    float ll = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (red[w][pr][0] != -INFINITY) ll += red[w][pr][1] * __builtin_amdgcn_exp2f(red[w][pr][0] - mm);
    m[r] = mm;
    inv_l[r] = ll > 0.0f ? 1.0f / ll : 0.0f;
  }

  // pass 2: the largest tile score of each query tile
  float smax0 = 0.0f, smax1 = 0.0f;
  S::walk(cx, wave, n_groups, [&](int, const float (&z)[16]) {
    const float p0 = S::partial_score(z, m, inv_l, 0), p1 = S::partial_score(z, m, inv_l, 8);
    smax0 = fmaxf(smax0, p0 + __shfl_xor(p0, 32));
    smax1 = fmaxf(smax1, p1 + __shfl_xor(p1, 32));
  });
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    smax0 = fmaxf(smax0, __shfl_xor(smax0, off));
    smax1 = fmaxf(smax1, __shfl_xor(smax1, off));
  }
  if (lane == 0) {
    red_max[wave][0] = smax0;
    red_max[wave][1] = smax1;
  }
  __syncthreads();
  smax0 = fmaxf(fmaxf(red_max[0][0], red_max[1][0]), fmaxf(red_max[2][0], red_max[3][0]));
  smax1 = fmaxf(fmaxf(red_max[0][1], red_max[1][1]), fmaxf(red_max[2][1], red_max[3][1]));
  const float thr0 = a.alpha * smax0, thr1 = a.alpha * smax1;

  // pass 3: keep bits, one word per 32-tile group and query tile
  const int64_t row0 = (static_cast<int64_t>(b) * a.heads_q + h) * a.nq + t0;
  uint32_t* bits0 = a.bitmap + row0 * a.words;
  uint32_t* bits1 = bits0 + a.words;
  int count0 = 0, count1 = 0;
  S::walk(cx, wave, n_groups, [&](int gi, const float (&z)[16]) {
    const float p0 = S::partial_score(z, m, inv_l, 0), p1 = S::partial_score(z, m, inv_l, 8);
    const float sc0 = p0 + __shfl_xor(p0, 32), sc1 = p1 + __shfl_xor(p1, 32);
    const int kt = gi * 32 + cx.l32;
    const bool keep0 = kt < nc0 && (sc0 >= thr0 || kt * kBk + kBk - 1 > t0 * kBq);
    const bool keep1 = kt < nc1 && (sc1 >= thr1 || kt * kBk + kBk - 1 > (t0 + 1) * kBq);
    const uint32_t w0 = static_cast<uint32_t>(__ballot(keep0 && cx.hi == 0));
    const uint32_t w1 = static_cast<uint32_t>(__ballot(keep1 && cx.hi == 0));
    if (lane == 0) {
      if (gi * 32 < nc0) bits0[gi] = w0;
      if (has_t1) bits1[gi] = w1;
    }
    count0 += __builtin_popcount(w0);
    count1 += __builtin_popcount(w1);
  });
  if (lane == 0) {
    red_cnt[wave][0] = count0;
    red_cnt[wave][1] = count1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.counts[row0] = red_cnt[0][0] + red_cnt[1][0] + red_cnt[2][0] + red_cnt[3][0];
    if (has_t1) a.counts[row0 + 1] = red_cnt[0][1] + red_cnt[1][1] + red_cnt[2][1] + red_cnt[3][1];
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
// One wave per row: bitmap words -> ascending key tiles with causal flags.
__global__ __launch_bounds__(256) void dyn_emit_kernel(const DynLaunch a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (row >= a.n_rows) return;
  const int t = static_cast<int>(row % a.nq);
  const int nc = (min(a.seqlen, (t + 1) * kBq) - 1) / kBk + 1;
  const int n_words = (nc + 31) / 32;
  const uint32_t* bits = a.bitmap + row * a.words;
  int out = a.row_ptr[row];
  for (int w0 = 0; w0 < n_words; w0 += 64) {
    const int wi = w0 + lane;
    uint32_t word = wi < n_words ? bits[wi] : 0u;
    const int c = __builtin_popcount(word);
    int incl = c;  // inclusive scan of the popcounts over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    int pos = out + incl - c;
    while (word) {
      const int bit = __builtin_ctz(word);
      word &= word - 1;
      const int kt = wi * 32 + bit;
      a.k_tile[pos] = kt;
      a.flags[pos] = kt * kBk + kBk - 1 > t * kBq ? TRI_TILE_PARTIAL : TRI_TILE_FULL;
      ++pos;
    }
    out += __shfl(incl, 63);
  }
}

template <int D>
int launch_d(const DynLaunch& a, hipStream_t stream) {
  const int64_t pool_blocks = (a.n_pool_tiles + 3) / 4;
  hipLaunchKernelGGL(dyn_pool_kernel<D>, dim3(static_cast<unsigned>(pool_blocks)), dim3(256), 0, stream, a);
  const int64_t select_blocks = a.n_rows / a.nq * ((a.nq + 1) / 2);
  hipLaunchKernelGGL(dyn_select_kernel<D>, dim3(static_cast<unsigned>(select_blocks)), dim3(256), 0, stream, a);
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
