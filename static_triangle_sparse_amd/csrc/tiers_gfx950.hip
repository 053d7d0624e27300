// Precision tiers (TriAttention page: tiles grouped by per-head
// diagonal-distance boundaries and scored at different precisions, combined
// in one normalised output): the fp8 copy of K that the far (LOW) tiles of
// the tiered attention kernel read.
//
// For every (batch, KV head, key tile of 64 keys, the unit the page assigns a
// precision to): amax = max |k| over the tile's keys (keys >= N excluded),
// scale = amax / 448, and each value becomes the
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

constexpr int kTileKeys = TRI_KERNEL_BLOCK_K;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One wave per (batch, KV head, key tile), 4 per workgroup.  Lane l owns
// the 8-channel group m = l % (D / 8) of rows l / (D / 8) + (64 / (D / 8)) i:
// each load instruction reads whole 2D-byte rows (coalesced), and the 8
// channels of a group land on 8 consecutive bytes of the fp8 row (4 of the
// fp4 row), so every lane stores its own codes.
template <int D, bool kFp4>
__global__ __launch_bounds__(256) void quantize_kernel(const QuantLaunch a) {
  constexpr int kGroups = D / 8;                  // 8-channel groups per row
  constexpr int kRowsPerStep = 64 / kGroups;      // rows one load instruction covers
  constexpr int kSteps = kTileKeys / kRowsPerStep;
  constexpr float kMax = kFp4 ? 6.0f : 448.0f;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (blk >= a.n_blocks) return;
  const int nt = (a.seqlen + kTileKeys - 1) / kTileKeys;
  const int kt = static_cast<int>(blk % nt);
  const int64_t bg = blk / nt;
  const int b = static_cast<int>(bg / a.heads_kv), g = static_cast<int>(bg % a.heads_kv);
  const int m = lane % kGroups, r0 = lane / kGroups;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + b * a.k_stride[0] + g * a.k_stride[1] + 8 * m;
  u32x4 in[kSteps];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int key = kt * kTileKeys + r0 + kRowsPerStep * i;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < a.seqlen) w = *reinterpret_cast<const u32x4*>(kp + static_cast<int64_t>(key) * a.k_stride[2]);
    in[i] = w;
#pragma unroll
    for (int x = 0; x < 4; ++x) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[x])), fabsf(bf16_hi(w[x]))));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float inv = amax > 0.0f ? kMax / amax : 0.0f;
  if (lane == 0) a.scale[blk] = amax / kMax;
  // channels 8 m .. 8 m + 7 = k-step s = m / 8, lane half h = m % 2, elements
  // 8 ((m % 8) / 2) .. + 7 of that (step, half) in the operand order
  const int s = m / 8, h = m % 2, e0 = 8 * ((m % 8) / 2);
  const int out_off = kFp4 ? 16 * (2 * s + h) + e0 / 2 : 64 * s + 32 * h + e0;
  constexpr int kOutRow = kFp4 ? D / 2 : D;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int key = kt * kTileKeys + r0 + kRowsPerStep * i;
    if (key >= a.seqlen) continue;
    float v[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      v[2 * x] = fminf(fmaxf(bf16_lo(in[i][x]) * inv, -kMax), kMax);
      v[2 * x + 1] = fminf(fmaxf(bf16_hi(in[i][x]) * inv, -kMax), kMax);
    }
    char* row = static_cast<char*>(a.k8) + (bg * a.seqlen + key) * kOutRow + out_off;
    if constexpr (kFp4) {
      unsigned word = 0;
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[0], v[1], 1.0f, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[2], v[3], 1.0f, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[4], v[5], 1.0f, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[6], v[7], 1.0f, 3);
      *reinterpret_cast<uint32_t*>(row) = word;
    } else {
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 o = {static_cast<uint32_t>(w0), static_cast<uint32_t>(w1)};
      *reinterpret_cast<u32x2*>(row) = o;
    }
  }
}

}  // namespace

int launch_quantize_k(const QuantLaunch& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = static_cast<unsigned>((a.n_blocks + 3) / 4);
  if (a.head_dim != 128 && a.head_dim != 64) return fail(TRI_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
  if (a.fp4) {
    if (a.head_dim == 128)
      hipLaunchKernelGGL((quantize_kernel<128, true>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_kernel<64, true>), dim3(grid), dim3(256), 0, s, a);
  } else if (a.head_dim == 128) {
    hipLaunchKernelGGL((quantize_kernel<128, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((quantize_kernel<64, false>), dim3(grid), dim3(256), 0, s, a);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(TRI_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(err));
  return TRI_OK;
}

}  // namespace triattn
