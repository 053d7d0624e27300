// Merge of split rows.  The last-Q query tiles of a triangle layer keep every
// key tile, so their lists are ~50x longer than a band tile's; a split launch
// walks each such list in chunks of C key tiles on separate workgroups.  Each
// chunk leaves, per row, its unnormalised output O_c = sum_j P_j v_j with
// P_j = exp2(c (s_j - m_c)) (m_c: the chunk's reference score, raw units),
// the fp32 sum l_c of its P and the sum lb_c of the bf16-rounded P the PV
// product used.  Softmax over the union of the chunks' keys is then
//   M = max_c m_c,  w_c = exp2(c (m_c - M)),
//   o = sum_c w_c O_c / sum_c w_c lb_c,  lse = scale M + ln(sum_c w_c l_c),
// the standard rescaling of partial softmax sums (the same identity the
// online softmax applies key block by key block).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri_attn_internal.h"

namespace triattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = TRI_KERNEL_BLOCK_Q;

// One thread per (heavy tile item, row, 4 channels).
template <int D, bool kOutBf16>
__global__ __launch_bounds__(256) void split_merge_kernel(const AttnLaunch a) {
  constexpr int kQuads = D / 4;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const Schedule& s = a.sched;
  const int64_t n_tiles = static_cast<int64_t>(s.batch) * s.heads_q * s.n_heavy;
  if (gid >= n_tiles * kRows * kQuads) return;
  const int quad = static_cast<int>(gid % kQuads);
  const int row = static_cast<int>((gid / kQuads) % kRows);
  const int64_t tile = gid / (static_cast<int64_t>(kQuads) * kRows);  // (b * Hq + h) * n_heavy + hi
  const int hi = static_cast<int>(tile % s.n_heavy);
  const int64_t bh = tile / s.n_heavy;
  const int h = static_cast<int>(bh % s.heads_q);
  const int b = static_cast<int>(bh / s.heads_q);
  const int t = s.n_qtiles - 1 - hi;
  const int qrow = t * kRows + row;
  if (qrow >= a.seqlen) return;

  const float c_log2 = a.scale * 1.4426950408889634f;
  const int64_t item0 = tile * s.n_split;
  float mx = -INFINITY;
  for (int c = 0; c < s.n_split; ++c) mx = fmaxf(mx, a.split_stats[(item0 + c) * 3 * kRows + row]);
  float sum_l = 0.0f, sum_lb = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = 0; c < s.n_split; ++c) {
    const float* sp = a.split_stats + (item0 + c) * 3 * kRows + row;
    const float m = sp[0];
    if (m == -INFINITY) continue;  // no key of this chunk kept for the row
    const float wgt = exp2f((m - mx) * c_log2);
    sum_l += wgt * sp[kRows];
    sum_lb += wgt * sp[2 * kRows];
    const f32x4 o = *reinterpret_cast<const f32x4*>(a.split_o + ((item0 + c) * kRows + row) * D + quad * 4);
    acc += wgt * o;
  }
  const float inv = 1.0f / sum_lb;
  const int64_t orow = b * a.o_stride[0] + h * a.o_stride[1] + static_cast<int64_t>(qrow) * a.o_stride[2];
  if constexpr (kOutBf16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = {static_cast<__bf16>(acc[0] * inv), static_cast<__bf16>(acc[1] * inv),
                      static_cast<__bf16>(acc[2] * inv), static_cast<__bf16>(acc[3] * inv)};
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(a.o) + orow + quad * 4) = v;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + quad * 4) = acc * inv;
  }
  if (a.lse && quad == 0) a.lse[b * a.lse_stride[0] + h * a.lse_stride[1] + qrow] = mx * a.scale + logf(sum_l);
}

template <int D>
int launch_d(const AttnLaunch& a, hipStream_t stream) {
  const int64_t threads = static_cast<int64_t>(a.sched.batch) * a.sched.heads_q * a.sched.n_heavy * kRows * (D / 4);
  const unsigned grid = static_cast<unsigned>((threads + 255) / 256);
  if (a.o_bf16)
    hipLaunchKernelGGL((split_merge_kernel<D, true>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((split_merge_kernel<D, false>), dim3(grid), dim3(256), 0, stream, a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(TRI_ERR_HIP, "merge launch failed: %s", hipGetErrorString(err));
  return TRI_OK;
}

}  // namespace

int launch_split_merge(const AttnLaunch& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.sched.n_split <= 1 || a.sched.n_heavy == 0) return TRI_OK;
  if (a.head_dim == 128) return launch_d<128>(a, s);
  if (a.head_dim == 64) return launch_d<64>(a, s);
  return fail(TRI_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

}  // namespace triattn
