// Precision tiers (TriAttention page: tiles grouped by per-head
// diagonal-distance boundaries and scored at different precisions, combined
// in one normalised output): the fp8 copy of K that the far (LOW) tiles of
// the tiered attention kernel read.
//
// For every (batch, KV head, 32-key half-tile): amax = max |k| over the 32
// keys (keys >= N excluded), scale = amax / 448, and each value becomes the
// e4m3 code of clamp(k * (448 / amax), -448, 448) (round to nearest even,
// v_cvt_pk_fp8_f32); an all-zero block has scale 0 and zero codes.  A row of
// D channels is stored as D bytes in the fp8 operand order of the attention
// kernel: byte p = 64 s + 32 h + j holds channel 64 s + 16 (j / 8) + 8 h +
// j % 8, so each lane of the fp8 MFMA reads 32 contiguous bytes.
//
// The fp4 (e2m1) copy for the farthest tiles uses the same blocks with
// scale = amax / 6 and codes e2m1(clamp(k * (6 / amax), -6, 6)) (round to
// nearest even, v_cvt_scalef32_pk_fp4_f32 at unit scale).  A row is D / 2
// bytes: 16-byte block b = 2 s + h holds the 32 elements e of k-step s, lane
// half h, element e (channel 64 s + 16 (e / 8) + 8 h + e % 8, as in the fp8
// copy) at nibble e of the block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri_attn_internal.h"

namespace triattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHalfKeys = TRI_KERNEL_BLOCK_K / 2;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One wave per (batch, KV head, half-tile), 4 per workgroup.  Lane l owns key
// l / 2 of the block and output bytes [(l % 2) D / 2, (l % 2 + 1) D / 2) of
// its row, in groups of 8 bytes = 8 consecutive channels.
template <int D>
__global__ __launch_bounds__(256) void quantize_k_kernel(const QuantLaunch a) {
  constexpr int kGroups = D / 16;  // 8-byte output groups per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (blk >= a.n_blocks) return;
  const int nh = (a.seqlen + kHalfKeys - 1) / kHalfKeys;
  const int hb = static_cast<int>(blk % nh);
  const int64_t bg = blk / nh;
  const int b = static_cast<int>(bg / a.heads_kv), g = static_cast<int>(bg % a.heads_kv);
  const int key = hb * kHalfKeys + (lane >> 1);
  const bool valid = key < a.seqlen;
  const int p0 = (lane & 1) * (D / 2);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_stride[0] + g * a.k_stride[1] +
                       static_cast<int64_t>(valid ? key : 0) * a.k_stride[2];
  u32x4 in[kGroups];
  float amax = 0.0f;
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int p = p0 + gi * 8;
    const int s = p >> 6, h = (p >> 5) & 1, j = p & 31;
    const int d0 = 64 * s + 16 * (j >> 3) + 8 * h;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (valid) w = *reinterpret_cast<const u32x4*>(kp + d0);
    in[gi] = w;
#pragma unroll
    for (int x = 0; x < 4; ++x) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[x])), fabsf(bf16_hi(w[x]))));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
  if (lane == 0) a.scale[blk] = amax / 448.0f;
  if (!valid) return;
  uint32_t* out = reinterpret_cast<uint32_t*>(static_cast<char*>(a.k8) + (bg * a.seqlen + key) * D + p0);
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    uint32_t o2[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t w0 = in[gi][2 * half], w1 = in[gi][2 * half + 1];
      const float v0 = fminf(fmaxf(bf16_lo(w0) * inv, -448.0f), 448.0f);
      const float v1 = fminf(fmaxf(bf16_hi(w0) * inv, -448.0f), 448.0f);
      const float v2 = fminf(fmaxf(bf16_lo(w1) * inv, -448.0f), 448.0f);
      const float v3 = fminf(fmaxf(bf16_hi(w1) * inv, -448.0f), 448.0f);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, word, true);
      o2[half] = static_cast<uint32_t>(word);
    }
    out[2 * gi] = o2[0];
    out[2 * gi + 1] = o2[1];
  }
}

// fp4 copy: one wave per (batch, KV head, half-tile).  Lane l owns key l / 2
// of the block and output bytes [(l % 2) D / 4, (l % 2 + 1) D / 4) of its
// row: D / 64 blocks of 16 bytes, each from 4 groups of 8 channels.
template <int D>
__global__ __launch_bounds__(256) void quantize_k4_kernel(const QuantLaunch a) {
  constexpr int kBlocks = D / 64;  // 16-byte output blocks per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (blk >= a.n_blocks) return;
  const int nh = (a.seqlen + kHalfKeys - 1) / kHalfKeys;
  const int hb = static_cast<int>(blk % nh);
  const int64_t bg = blk / nh;
  const int b = static_cast<int>(bg / a.heads_kv), g = static_cast<int>(bg % a.heads_kv);
  const int key = hb * kHalfKeys + (lane >> 1);
  const bool valid = key < a.seqlen;
  const int b0 = (lane & 1) * kBlocks;  // first output block of this lane
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_stride[0] + g * a.k_stride[1] +
                       static_cast<int64_t>(valid ? key : 0) * a.k_stride[2];
  u32x4 in[kBlocks][4];
  float amax = 0.0f;
#pragma unroll
  for (int bi = 0; bi < kBlocks; ++bi) {
    const int blkid = b0 + bi, st = blkid >> 1, h = blkid & 1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid) x = *reinterpret_cast<const u32x4*>(kp + 64 * st + 16 * w + 8 * h);
      in[bi][w] = x;
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(x[j])), fabsf(bf16_hi(x[j]))));
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float inv = amax > 0.0f ? 6.0f / amax : 0.0f;
  if (lane == 0) a.scale[blk] = amax / 6.0f;
  if (!valid) return;
  u32x4* out = reinterpret_cast<u32x4*>(static_cast<char*>(a.k8) + (bg * a.seqlen + key) * (D / 2)) + b0;
#pragma unroll
  for (int bi = 0; bi < kBlocks; ++bi) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = fminf(fmaxf(bf16_lo(in[bi][w][j]) * inv, -6.0f), 6.0f);
        v[2 * j + 1] = fminf(fmaxf(bf16_hi(in[bi][w][j]) * inv, -6.0f), 6.0f);
      }
      unsigned word = 0;
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[0], v[1], 1.0f, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[2], v[3], 1.0f, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[4], v[5], 1.0f, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[6], v[7], 1.0f, 3);
      o[w] = word;
    }
    out[bi] = o;
  }
}

}  // namespace

int launch_quantize_k(const QuantLaunch& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = static_cast<unsigned>((a.n_blocks + 3) / 4);
  if (a.fp4) {
    if (a.head_dim == 128)
      hipLaunchKernelGGL(quantize_k4_kernel<128>, dim3(grid), dim3(256), 0, s, a);
    else if (a.head_dim == 64)
      hipLaunchKernelGGL(quantize_k4_kernel<64>, dim3(grid), dim3(256), 0, s, a);
    else
      return fail(TRI_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
  } else if (a.head_dim == 128)
    hipLaunchKernelGGL(quantize_k_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL(quantize_k_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  else
    return fail(TRI_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(TRI_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(err));
  return TRI_OK;
}

}  // namespace triattn
