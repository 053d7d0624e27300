// Flash-style prefill attention for MI355X (gfx950, CDNA4) walking a list of
// kept key tiles: the TriangleMix triangle layer (sink + diagonal window +
// last-Q rows, middle skipped; TriangleMix blog "介绍", 36kr interview
// technical motivation) and the dense causal layer use the same kernel.
//
// One workgroup = one (batch, query head, 128-row query tile); 4 waves, each
// owning 32 query rows.  Per kept 64-key tile:
//   1. K (row-major) and V (transposed to channel-major) are staged in LDS from
//      registers that were prefetched from HBM during the previous tile;
//   2. S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS, Q held in
//      registers for the whole loop).  Computing the transpose puts one query
//      per lane, so row statistics are per-lane scalars;
//   3. PARTIAL tiles apply the mask predicate per element, FULL tiles skip it;
//   4. online softmax in fp32 with exp2 (log2 e folded into the scale);
//   5. O^T += V^T . P^T on MFMA: the fp32 scores of step 2 are already laid out
//      as the B operand of this product once converted to bf16 (the key order
//      of that layout is mirrored by the column order of V^T in LDS), so P never
//      leaves registers.
// Output O = acc / l (bf16 round-to-nearest-even or f32) and the natural-log
// LSE = scale * m + ln l are written once per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tri_attn_internal.h"

namespace triattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockQ = TRI_KERNEL_BLOCK_Q;  // 128 query rows per workgroup
constexpr int kBlockK = TRI_KERNEL_BLOCK_K;  // 64 keys per tile
constexpr int kThreads = 256;                // 4 waves x 32 query rows
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Cfg {
  static constexpr int kKStride = D * 2 + 16;      // bytes per K row in LDS (padded)
  static constexpr int kVStride = kBlockK * 2 + 16;  // bytes per V^T row (one channel)
  static constexpr int kKBytes = kBlockK * kKStride;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kQSteps = D / 16;            // k-steps of S^T = K Q^T
  static constexpr int kOBlocks = D / 32;           // 32-channel blocks of O^T
  static constexpr int kKLoads = kBlockK * D / 8 / kThreads;  // 16-B K chunks / thread
  static constexpr int kVUnits = (kBlockK / 4) * (D / 8);     // 4 keys x 8 channels units
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Column (key position) of key quad `kq` (keys 4*kq..4*kq+3 of the tile) in
// the V^T rows.  In the S^T accumulator, lane half `hi` of a 32-key block
// holds keys {4*hi..4*hi+3, 8+4*hi..8+4*hi+3} (+16 for the next half block) in
// registers 0..7; the PV MFMA reads those registers as k-positions
// 8*hi..8*hi+7 of a 16-key step.  Storing key quads 1 and 2 of every 16-key
// group swapped makes V^T's columns follow that order.
__device__ __forceinline__ int vt_column(int kq) {
  const int grp = kq >> 2, q = kq & 3;
  return grp * 16 + ((q & 1) * 2 + (q >> 1)) * 4;
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

template <int D, bool kOutBf16, bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const AttnLaunch a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::kBufBytes];

  const WorkItem w = schedule_item(a.sched, blockIdx.x);
  if (w.t < 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int N = a.seqlen;
  const int G = a.sched.group;
  const int g = w.h / G;
  const int q0 = w.t * kBlockQ;
  const int qrow = q0 + wave * 32 + l32;

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + w.b * a.q_stride[0] + w.h * a.q_stride[1];
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + w.b * a.k_stride[0] + g * a.k_stride[1];
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + w.b * a.v_stride[0] + g * a.v_stride[1];
  const int64_t ks_n = a.k_stride[2];
  const int64_t vs_n = a.v_stride[2];

  // kept tiles of this query tile
  int e_begin, e_end;
  if (kCausal) {
    e_begin = 0;
    e_end = (min(N, q0 + kBlockQ) - 1) / kBlockK + 1;
  } else {
    e_begin = a.row_ptr[w.t];
    e_end = a.row_ptr[w.t + 1];
  }

  // Q^T operand: lane holds Q[qrow][16*s + 8*hi .. +7] for every k-step s.
  bf16x8 qreg[C::kQSteps];
  {
    const uint16_t* qp = qbase + static_cast<int64_t>(qrow) * a.q_stride[2] + hi * 8;
#pragma unroll
    for (int s = 0; s < C::kQSteps; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < N) x = *reinterpret_cast<const u32x4*>(qp + s * 16);
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Global -> register prefetch of one K/V tile.
  //   K: chunk c = r*256 + tid -> key c / (D/8), 8 channels at 8*(c % (D/8)).
  //   V: unit tid -> keys 4*(tid%16)..+3, channels 8*(tid/16)..+7.
  u32x4 kpre[C::kKLoads];
  u32x4 vpre[4];
  const int v_kq = tid & 15;
  const int v_dq = tid >> 4;
  const bool v_active = tid < C::kVUnits;
  auto gload = [&](int kt) {
    const int key0 = kt * kBlockK;
#pragma unroll
    for (int r = 0; r < C::kKLoads; ++r) {
      const int c = r * kThreads + tid;
      const int key = key0 + c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < N) x = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * ks_n + col);
      kpre[r] = x;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + v_kq * 4 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (v_active && key < N)
        x = *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(key) * vs_n + v_dq * 8);
      vpre[r] = x;
    }
  };
  auto tile_of = [&](int e) -> int { return kCausal ? e : a.k_tile[e]; };

  // mask constants (triangle predicate: j <= i, j < N and (j < sink or
  // i - j < window or i >= N - last_q))
  const int last_start = N - a.last_q;
  const float c_log2 = a.scale * kLog2e;

  f32x16 oacc[C::kOBlocks];
#pragma unroll
  for (int i = 0; i < C::kOBlocks; ++i)
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
  float m_i = -INFINITY;  // running max of raw scores q.k
  float l_i = 0.0f;       // this lane's partial sum (its 16 keys of each block)

  if (e_begin < e_end) gload(tile_of(e_begin));

  for (int e = e_begin; e < e_end; ++e) {
    char* buf = smem + ((e - e_begin) & 1) * C::kBufBytes;
    const int kt = tile_of(e);
    bool partial;
    if (kCausal) {
      const int c1 = kt * kBlockK + kBlockK - 1;
      partial = c1 > q0 || c1 >= N;
    } else {
      partial = a.flags[e] != TRI_TILE_FULL;
    }

    // stage the prefetched tile in LDS
#pragma unroll
    for (int r = 0; r < C::kKLoads; ++r) {
      const int c = r * kThreads + tid;
      *reinterpret_cast<u32x4*>(buf + (c / (D / 8)) * C::kKStride + (c % (D / 8)) * 16) = kpre[r];
    }
    if (v_active) {
      char* vt = buf + C::kKBytes + vt_column(v_kq) * 2;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const u32x2 lo = {pack_lo(vpre[0][wd], vpre[1][wd]), pack_lo(vpre[2][wd], vpre[3][wd])};
        const u32x2 hv = {pack_hi(vpre[0][wd], vpre[1][wd]), pack_hi(vpre[2][wd], vpre[3][wd])};
        *reinterpret_cast<u32x2*>(vt + (v_dq * 8 + 2 * wd) * C::kVStride) = lo;
        *reinterpret_cast<u32x2*>(vt + (v_dq * 8 + 2 * wd + 1) * C::kVStride) = hv;
      }
    }
    __syncthreads();
    if (e + 1 < e_end) gload(tile_of(e + 1));

    // S^T = K . Q^T : two 32-key blocks, lane = query, 16 keys per lane per block
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      const char* kp = buf + (kb * 32 + l32) * C::kKStride + hi * 16;
#pragma unroll
      for (int st = 0; st < C::kQSteps; ++st) {
        const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kp + st * 32);
        s[kb] = mfma32(kv, qreg[st], s[kb]);
      }
    }

    if (partial) {
      const int key0 = kt * kBlockK + hi * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = key0 + kb * 32 + (r >> 2) * 8 + (r & 3);
          bool ok = j <= qrow && j < N;
          if (!kCausal) ok = ok && (j < a.sink || qrow - j < a.window || qrow >= last_start);
          if (!ok) s[kb][r] = -INFINITY;
        }
    }

    // online softmax (lane-local row statistics; the other 32 keys of the
    // tile live in lane ^ 32)
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_i, mx);
    const float m_sub = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_i - m_sub) * c_log2);
    const float neg_mc = -m_sub * c_log2;
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, neg_mc));
        s[kb][r] = p;
        rs += p;
      }
    l_i = l_i * alpha + rs;
    m_i = m_new;
#pragma unroll
    for (int i = 0; i < C::kOBlocks; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;

    // P^T as bf16 B operands: 16-key step kc = registers 8*(kc&1)..+7 of block kc/2
    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int x = 0; x < 8; ++x) pb[kc][x] = static_cast<__bf16>(s[kc >> 1][(kc & 1) * 8 + x]);

    // O^T += V^T . P^T
#pragma unroll
    for (int ob = 0; ob < C::kOBlocks; ++ob) {
      const char* vp = buf + C::kKBytes + (ob * 32 + l32) * C::kVStride + hi * 16;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 vv = *reinterpret_cast<const bf16x8*>(vp + kc * 32);
        oacc[ob] = mfma32(vv, pb[kc], oacc[ob]);
      }
    }
  }

  // epilogue
  const float l_tot = l_i + __shfl_xor(l_i, 32);
  if (qrow < N) {
    const float inv = 1.0f / l_tot;
    const int64_t orow = w.b * a.o_stride[0] + w.h * a.o_stride[1] + static_cast<int64_t>(qrow) * a.o_stride[2];
#pragma unroll
    for (int ob = 0; ob < C::kOBlocks; ++ob)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = ob * 32 + r4 * 8 + hi * 4;
        f32x4 v4 = {oacc[ob][r4 * 4 + 0] * inv, oacc[ob][r4 * 4 + 1] * inv,
                    oacc[ob][r4 * 4 + 2] * inv, oacc[ob][r4 * 4 + 3] * inv};
        if (kOutBf16) {
          bf16x4 b4 = {static_cast<__bf16>(v4[0]), static_cast<__bf16>(v4[1]),
                       static_cast<__bf16>(v4[2]), static_cast<__bf16>(v4[3])};
          *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(a.o) + orow + d0) = b4;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d0) = v4;
        }
      }
    if (a.lse && hi == 0)
      a.lse[w.b * a.lse_stride[0] + w.h * a.lse_stride[1] + qrow] = m_i * a.scale + logf(l_tot);
  }
}

template <int D, bool kOutBf16, bool kCausal>
int launch_t(const AttnLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, kOutBf16, kCausal>), dim3(static_cast<unsigned>(a.sched.grid)),
                     dim3(kThreads), 0, stream, a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(TRI_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return TRI_OK;
}

template <int D>
int launch_d(const AttnLaunch& a, hipStream_t stream) {
  if (a.o_bf16) return a.causal ? launch_t<D, true, true>(a, stream) : launch_t<D, true, false>(a, stream);
  return a.causal ? launch_t<D, false, true>(a, stream) : launch_t<D, false, false>(a, stream);
}

}  // namespace

int launch_attn_fwd(const AttnLaunch& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.head_dim == 128) return launch_d<128>(a, s);
  if (a.head_dim == 64) return launch_d<64>(a, s);
  return fail(TRI_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

}  // namespace triattn
