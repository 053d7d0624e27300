// Flash-style prefill attention for MI355X (gfx950, CDNA4) walking a list of
// kept key tiles: the TriangleMix triangle layer (sink + diagonal window +
// last-Q rows, middle skipped; TriangleMix blog "介绍", 36kr interview
// technical motivation) and the dense causal layer use the same kernel.
//
// One workgroup = one (batch, query head, 128-row query tile); 4 waves, each
// owning 32 query rows.  A kept 64-key tile is processed as two 32-key
// halves, and the LDS stage holds one half (38 KiB for two stages), so three
// workgroups share a CU: three waves per SIMD keep the matrix cores fed while
// the others wait on LDS reads, dependent vector instructions or copies.
// Per 32-key half:
//   1. K and V are copied HBM -> LDS by the LDS-DMA path (each lane's 16
//      bytes land at LDS base + 16 * lane), double-buffered, one half ahead of
//      the compute and overlapped with it, without staging registers.
//      Rows are padded (K by 16 bytes, V by 64 bytes) so the MFMA operand
//      reads below hit distinct LDS banks while every read address is a
//      per-lane base plus a compile-time offset;
//   2. S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (K rows from LDS, Q held in
//      registers for the whole loop).  Computing the transpose puts one query
//      per lane, so row statistics are per-lane scalars;
//   3. PARTIAL tiles apply the mask predicate per element, FULL tiles skip it;
//      a half that no row of the wave keeps is skipped by that wave;
//   4. softmax in fp32 with exp2 (log2 e folded into the scale) against a
//      reference max that is fixed per row by the first block that keeps one
//      of its keys, so the O accumulators are never rescaled in the loop; a
//      row whose max later outgrows the reference by more than 2^64 in p
//      units sends the workgroup through a second pass with exact maxima;
//   5. O^T += V^T . P^T on MFMA: the fp32 scores of step 2 are already laid out
//      as the B operand of this product once converted to bf16, so P never
//      leaves registers; the A operand V^T is read from the row-major V tile
//      with the transposing LDS read ds_read_b64_tr_b16.
// Output O = acc / sum(bf16 P) (stored bf16 round-to-nearest-even or f32) and
// the natural-log LSE = scale * m + ln sum(P) are written once per row.
//
// Variants of the same walk:
//   * list rows per (batch, head) for per-head boundaries and dynamic lists;
//   * chunks of a split last-Q row, which leave unnormalised partials for
//     the merge kernel instead of O and LSE;
//   * precision tiers (TriAttention page): the far tiles of a list are a
//     prefix of it, scored from fp4 and/or fp8 copies of Q and K on the
//     scaled MFMA before the bf16 tiles; the tier count is a template value.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "tri_attn_internal.h"

namespace triattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))
// Read-only data read at uniform addresses inside the tile loop (the fp8 and
// fp4 K scales): through the constant address space such loads are scalar
// (s_load, counted on lgkmcnt).  As vector loads they were counted on vmcnt,
// in order with the LDS-DMA copies, and waiting for one waited for the copies
// of the next half in flight.
#define CONST_AS __attribute__((address_space(4)))
#define GLOBAL_AS __attribute__((address_space(1)))

constexpr int kBlockQ = TRI_KERNEL_BLOCK_Q;  // 128 query rows per workgroup
constexpr int kBlockK = TRI_KERNEL_BLOCK_K;  // 64 keys per tile
constexpr int kHalf = kBlockK / 2;           // keys per stage
constexpr int kThreads = 256;                // 4 waves x 32 query rows
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSumLimit = 0x1p64f;  // a row sum of P above this sends the workgroup to the exact-max passes
constexpr uint32_t kNegInfBits = 0xFF800000u;

template <int D>
struct Cfg {
  static constexpr int kRowBytes = D * 2;  // data bytes of one K or V row
  // K rows padded by 16 bytes: the 16 lanes of one S^T operand read (16
  // consecutive rows, one chunk) then start on distinct banks.
  static constexpr int kKStride = kRowBytes + 16;
  // V rows padded by 64 bytes: consecutive rows then start 64 bytes apart
  // modulo the 256-byte bank window, so the transposing read of a half-wave
  // (4 rows x 64 bytes) covers every bank once.
  static constexpr int kVStride = kRowBytes + 64;
  // a stage holds one 32-key half of a tile (K region rounded up to whole
  // 1 KiB copy blocks)
  static constexpr int kKBytes = (kHalf * kKStride + 1023) / 1024 * 1024;
  static constexpr int kVBytes = kHalf * kVStride;
  static constexpr int kKBlocks = kKBytes / 1024;  // 1 KiB DMA blocks
  static constexpr int kVBlocks = kVBytes / 1024;
  static constexpr int kKBlocksPerWave = (kKBlocks + kWaves - 1) / kWaves;
  static constexpr int kVBlocksPerWave = (kVBlocks + kWaves - 1) / kWaves;
  static constexpr int kStageBytes = kKBytes + kVBytes;
  // fp8 K of a far (LOW tier) half: 32 rows of D bytes, padded by 16 bytes
  // (one 16-byte bank step per row), in whole 1 KiB copy blocks
  static constexpr int kK8Stride = D + 16;
  static constexpr int kK8Blocks = (kHalf * kK8Stride + 1023) / 1024;
  static constexpr int kK8BlocksPerWave = (kK8Blocks + kWaves - 1) / kWaves;
  // fp4 K of a far half: 32 rows of D / 2 bytes, padded by 16 bytes
  static constexpr int kK4Stride = D / 2 + 16;
  static constexpr int kK4Blocks = (kHalf * kK4Stride + 1023) / 1024;
  static constexpr int kK4BlocksPerWave = (kK4Blocks + kWaves - 1) / kWaves;
  static constexpr int kQ8Steps = D / 64;  // k-steps of the fp8 S^T
  static constexpr int kQSteps = D / 16;   // k-steps of S^T = K Q^T
  static constexpr int kOBlocks = D / 32;  // 32-channel blocks of O^T
  static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "tiles fill whole DMA blocks");
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// value of x in lane l ^ 32 combined with x: returns {x[l & 31], x[(l & 31) + 32]}
__device__ __forceinline__ void pair_halves(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Max of finite or -inf scores.  Written as assembly: the compiler's fmaxf
// first quiets each operand (v_max_f32 x, x) because it cannot prove the
// MFMA results are not signalling NaNs.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Bits [0, x) set, for any x (none for x <= 0, all for x >= 32): the bit
// field mask of min(max(x, 0), 31) bits, or'ed with all ones when x > 31.
// Assembly, because the compiler rewrites the sign trick into a compare and
// a select.
__device__ __forceinline__ uint32_t low_bits(int x) {
  uint32_t r, t, u;
  asm("v_med3_i32 %1, %3, 0, 31\n\t"
      "v_bfm_b32 %1, %1, 0\n\t"
      "v_sub_u32 %2, 31, %3\n\t"
      "v_ashrrev_i32 %2, 31, %2\n\t"
      "v_or_b32 %0, %1, %2"
      : "=v"(r), "=&v"(t), "=&v"(u)
      : "v"(x));
  return r;
}

// Each score s becomes -inf where its bit of `drop` is set: a sign-extended
// one-bit field selects the -inf pattern bit by bit (two full-rate
// instructions instead of a compare and a select).
// Register r of a score block holds key offset 8 (r >> 2) + (r & 3) (+ 4 for
// the upper half-wave, removed by the caller's shift of `drop`).  One
// assembly block for all 16 registers: as separate statements the compiler
// put a wait state between every two of them.
__device__ __forceinline__ void drop_keys(float (&s)[16], uint32_t drop) {
  uint32_t u[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) u[r] = __float_as_uint(s[r]);
  uint32_t m;
  asm("v_bfe_i32 %16, %17, 0, 1\n\tv_bfi_b32 %0, %16, %18, %0\n\t"
      "v_bfe_i32 %16, %17, 1, 1\n\tv_bfi_b32 %1, %16, %18, %1\n\t"
      "v_bfe_i32 %16, %17, 2, 1\n\tv_bfi_b32 %2, %16, %18, %2\n\t"
      "v_bfe_i32 %16, %17, 3, 1\n\tv_bfi_b32 %3, %16, %18, %3\n\t"
      "v_bfe_i32 %16, %17, 8, 1\n\tv_bfi_b32 %4, %16, %18, %4\n\t"
      "v_bfe_i32 %16, %17, 9, 1\n\tv_bfi_b32 %5, %16, %18, %5\n\t"
      "v_bfe_i32 %16, %17, 10, 1\n\tv_bfi_b32 %6, %16, %18, %6\n\t"
      "v_bfe_i32 %16, %17, 11, 1\n\tv_bfi_b32 %7, %16, %18, %7\n\t"
      "v_bfe_i32 %16, %17, 16, 1\n\tv_bfi_b32 %8, %16, %18, %8\n\t"
      "v_bfe_i32 %16, %17, 17, 1\n\tv_bfi_b32 %9, %16, %18, %9\n\t"
      "v_bfe_i32 %16, %17, 18, 1\n\tv_bfi_b32 %10, %16, %18, %10\n\t"
      "v_bfe_i32 %16, %17, 19, 1\n\tv_bfi_b32 %11, %16, %18, %11\n\t"
      "v_bfe_i32 %16, %17, 24, 1\n\tv_bfi_b32 %12, %16, %18, %12\n\t"
      "v_bfe_i32 %16, %17, 25, 1\n\tv_bfi_b32 %13, %16, %18, %13\n\t"
      "v_bfe_i32 %16, %17, 26, 1\n\tv_bfi_b32 %14, %16, %18, %14\n\t"
      "v_bfe_i32 %16, %17, 27, 1\n\tv_bfi_b32 %15, %16, %18, %15\n\t"
      : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]), "+v"(u[4]), "+v"(u[5]), "+v"(u[6]), "+v"(u[7]),
        "+v"(u[8]), "+v"(u[9]), "+v"(u[10]), "+v"(u[11]), "+v"(u[12]), "+v"(u[13]), "+v"(u[14]), "+v"(u[15]),
        "=&v"(m)
      : "v"(drop), "s"(kNegInfBits));
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __uint_as_float(u[r]);
}

// An MFMA result may be read by a VALU instruction only some wait states
// after the MFMA issued (the matrix core writes it over its passes).  The
// compiler inserts them before its own instructions, but not before inline
// assembly, which it does not look into.  The score helpers below that read
// MFMA results in assembly (masking, row max) therefore first pass the block
// through this fence: 21 wait states, enough for the longest MFMA here (the
// 16-pass fp8 32x32x64); the "+v" operand orders every later read after it.
__device__ __forceinline__ void mfma_result_fence(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s));
}

__device__ __forceinline__ void wait_vmcnt0() {
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Raw buffer descriptor (no swizzle, stride 0) of `bytes` bytes at p; loads
// past the end return zeros.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
__device__ __forceinline__ u32x4 buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const u32x4 r = {static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xFFFFu, bytes, kRsrcWord3};
  return r;
}

// One LDS-DMA copy: every lane loads 16 bytes at `voffset` of the buffer and
// they land at lds + 16 * lane.  Written as inline assembly so that the
// compiler does not make every later LDS read wait for all copies in flight
// (it cannot tell the stages apart); the kernel waits for exactly the copies
// a step needs (wait_vmcnt) before the barrier that publishes them.  The
// instruction has no register results.  The compiler's hazard recognizer
// does not look inside inline assembly, so the wait states a buffer load needs
// are issued here: 5 after a VALU write of an SGPR it reads (the descriptor
// may come from v_readlane) and 1 after the write of M0.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t voffset, char LDS_AS* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(m0)
               : "memory");
}

// Tile row and 16-byte source chunk of the DMA chunk that lands at byte x of a
// tile stored with `stride`-byte padded rows.  Chunks that land on row padding
// re-read chunk 0 of their row (in bounds, never used).
template <int D>
__device__ __forceinline__ void dma_source(int x, int stride, int& row, int& chunk) {
  row = x / stride;
  chunk = (x - row * stride) / 16;
  if (chunk >= D / 8) chunk = 0;
}

// Quantized Q of the tiered kernel (empty otherwise).
// kTiers: 0 none, 1 fp8 + bf16, 2 fp4 + fp8 + bf16
template <int D, int kTiers>
struct TierState {};
template <int D>
struct TierState<D, 1> {
  i32x8 q8[Cfg<D>::kQ8Steps];  // fp8 e4m3 Q in the fp8 operand order
  float s_q;                   // its scale: row amax / 448
};
template <int D>
struct TierState<D, 2> : TierState<D, 1> {
  u32x4 q4[Cfg<D>::kQ8Steps];  // fp4 e2m1 Q in the fp4 operand order
  float s_q4;                  // its scale: row amax / 6
};
template <int D, int kTiers>
struct TierLane {};
template <int D>
struct TierLane<D, 1> {
  int k8_rd;
};
template <int D>
struct TierLane<D, 2> : TierLane<D, 1> {
  int k4_rd;
};

// Lane id, materialized afresh where it is used: the copy offsets of the fp8
// and fp4 K halves are recomputed at every copy from it rather than held in
// registers.  Held over the loop, they were spilled, and every reload from
// scratch waited (vmcnt, in order) for all copies in flight.  The volatile
// statement keeps the compiler from hoisting the computation out of the loop.
__device__ __forceinline__ int lane_id_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Global byte offset (within the half) of the 16-byte chunk that lands at
// byte x of an LDS half stored as 32 rows of `stride` bytes holding `row_bytes`
// bytes each; chunks on row padding re-read chunk 0 of their row.
template <int kStride, int kRowBytes>
__device__ __forceinline__ uint32_t padded_dma_offset(int x) {
  const int row = x / kStride;
  int chunk = (x - row * kStride) / 16;
  if (chunk >= kRowBytes / 16) chunk = 0;
  return static_cast<uint32_t>(min(row, kHalf - 1) * kRowBytes + chunk * 16);
}

template <int D, bool kOutBf16, bool kCausal, int kTiers>
struct Kernel {
  using C = Cfg<D>;

  struct State : TierState<D, kTiers> {
    bf16x8 q[C::kQSteps];
    f32x16 o[C::kOBlocks];
    float m;       // reference max of raw scores q.k (fixed once set, see compute_half)
    float neg_mc;  // -m c log2(e), or 0 while m is unset
    float mt;      // true running max of raw scores q.k (exact-max pass only)
    float l;   // this lane's partial row sum of fp32 P (its 16 keys of each 32-key block)
    float lb;  // the same sum over the bf16-rounded P
  };

  // Per-lane constants of one workgroup.
  struct Lane : TierLane<D, kTiers> {
    int hi;
    int k_rd;  // K operand read offset (stage-relative bytes)
    int v_rd;  // V^T transposing-read offset (relative to the V tile)
    uint32_t k_dma[C::kKBlocksPerWave];  // global byte offsets within a tile
    uint32_t v_dma[C::kVBlocksPerWave];
    int qrow;
    int hi_lim, sink_lim, win_lo;  // mask: j <= hi_lim and (j < sink_lim or j >= win_lo)
  };

  // The i-th DMA block of wave w is block i * waves + w of the tile; lane l of
  // it fills LDS bytes [16 l, 16 l + 16) of that block.  The copies go through
  // buffer descriptors that start at the tile and end at the sequence end:
  // rows past the end are outside the descriptor and land as zeros.
  static __device__ __forceinline__ void issue_dma(char LDS_AS* stage, const Lane& ln, int wave,
                                                   const u32x4& k_rsrc, const u32x4& v_rsrc) {
#pragma unroll
    for (int i = 0; i < C::kKBlocksPerWave; ++i) {
      const int blk = i * kWaves + wave;
      if (C::kKBlocks % kWaves == 0 || blk < C::kKBlocks)
        lds_dma16(k_rsrc, ln.k_dma[i], stage + blk * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::kVBlocksPerWave; ++i) {
      const int blk = i * kWaves + wave;
      if (C::kVBlocks % kWaves == 0 || blk < C::kVBlocks)
        lds_dma16(v_rsrc, ln.v_dma[i], stage + C::kKBytes + blk * 1024);
    }
  }

  // fp8 K of a LOW half (blocks of the K region) plus V, as issue_dma.
  static __device__ __forceinline__ void issue_dma_low(char LDS_AS* stage, const Lane& ln, int wave,
                                                       const u32x4& k8_rsrc, const u32x4& v_rsrc) {
    if constexpr (kTiers) {
      const int l16 = lane_id_fresh() * 16;
#pragma unroll
      for (int i = 0; i < C::kK8BlocksPerWave; ++i) {
        const int blk = i * kWaves + wave;
        if (C::kK8Blocks % kWaves == 0 || blk < C::kK8Blocks)
          lds_dma16(k8_rsrc, padded_dma_offset<C::kK8Stride, D>(blk * 1024 + l16), stage + blk * 1024);
      }
#pragma unroll
      for (int i = 0; i < C::kVBlocksPerWave; ++i) {
        const int blk = i * kWaves + wave;
        if (C::kVBlocks % kWaves == 0 || blk < C::kVBlocks)
          lds_dma16(v_rsrc, ln.v_dma[i], stage + C::kKBytes + blk * 1024);
      }
    }
  }

  // fp4 K of a far half (blocks of the K region) plus V, as issue_dma.
  static __device__ __forceinline__ void issue_dma_fp4(char LDS_AS* stage, const Lane& ln, int wave,
                                                       const u32x4& k4_rsrc, const u32x4& v_rsrc) {
    if constexpr (kTiers >= 2) {
      const int l16 = lane_id_fresh() * 16;
#pragma unroll
      for (int i = 0; i < C::kK4BlocksPerWave; ++i) {
        const int blk = i * kWaves + wave;
        if (C::kK4Blocks % kWaves == 0 || blk < C::kK4Blocks)
          lds_dma16(k4_rsrc, padded_dma_offset<C::kK4Stride, D / 2>(blk * 1024 + l16), stage + blk * 1024);
      }
#pragma unroll
      for (int i = 0; i < C::kVBlocksPerWave; ++i) {
        const int blk = i * kWaves + wave;
        if (C::kVBlocks % kWaves == 0 || blk < C::kVBlocks)
          lds_dma16(v_rsrc, ln.v_dma[i], stage + C::kKBytes + blk * 1024);
      }
    }
  }

  // S^T block of one 32-key half (kb): lane = query, 16 of the 32 keys per
  // lane; register r holds key key0 + 32 kb + 8 (r >> 2) + 4 hi + (r & 3).
  // Keys a PARTIAL tile drops are set to -inf.
  // In the tiered kernel a LOW half (low) is scored from fp8 K and Q with
  // v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales); its scores are left
  // in fp8 code units, s_q s_k times smaller than raw scores (the caller folds
  // that factor into its exponent and maxima).
  // A far half (fp4) is scored the same way from fp4 K and Q (format code 4
  // on both operands, 16 bytes per lane per 64-wide k-step).
  static __device__ __forceinline__ f32x16 scores(const char LDS_AS* stage, const Lane& ln, const State& st,
                                                  int kb, int key0, bool partial, uint32_t keep,
                                                  bool low = false, bool fp4 = false) {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    bool done = false;
    if constexpr (kTiers >= 2) {
      if (fp4) {
        const char LDS_AS* kp4 = stage + ln.k4_rd;
#pragma unroll
        for (int q = 0; q < C::kQ8Steps; ++q) {
          const u32x4 a0 = *reinterpret_cast<const LDS_AS u32x4*>(kp4 + q * 32);
          const i32x8 ka = {static_cast<int>(a0[0]), static_cast<int>(a0[1]), static_cast<int>(a0[2]),
                            static_cast<int>(a0[3]), 0, 0, 0, 0};
          const i32x8 qb = {static_cast<int>(st.q4[q][0]), static_cast<int>(st.q4[q][1]),
                            static_cast<int>(st.q4[q][2]), static_cast<int>(st.q4[q][3]), 0, 0, 0, 0};
          s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qb, s, 4, 4, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
        }
        done = true;
      }
    }
    if constexpr (kTiers >= 1) {
      if (low && !done) {
        const char LDS_AS* kp8 = stage + ln.k8_rd;
#pragma unroll
        for (int q = 0; q < C::kQ8Steps; ++q) {
          const u32x4 a0 = *reinterpret_cast<const LDS_AS u32x4*>(kp8 + q * 64);
          const u32x4 a1 = *reinterpret_cast<const LDS_AS u32x4*>(kp8 + q * 64 + 16);
          const i32x8 ka = {static_cast<int>(a0[0]), static_cast<int>(a0[1]), static_cast<int>(a0[2]),
                            static_cast<int>(a0[3]), static_cast<int>(a1[0]), static_cast<int>(a1[1]),
                            static_cast<int>(a1[2]), static_cast<int>(a1[3])};
          s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, st.q8[q], s, 0, 0, 0, 0x7F7F7F7F, 0,
                                                              0x7F7F7F7F);
        }
        done = true;
      }
    }
    if (!done) {
      // Four K operand reads run ahead of the dependent MFMA chain: four
      // reads first, then each MFMA followed by the next read.  Without the
      // schedule groups the allocator keeps only two in flight.
      const char LDS_AS* kp = stage + ln.k_rd;
      bf16x8 kv[C::kQSteps];
#pragma unroll
      for (int q = 0; q < C::kQSteps; ++q) kv[q] = *reinterpret_cast<const LDS_AS bf16x8*>(kp + q * 32);
#pragma unroll
      for (int q = 0; q < C::kQSteps; ++q) s = mfma32(kv[q], st.q[q], s);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
      for (int q = 0; q < C::kQSteps - 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // the last 4 MFMAs
    }
    if (partial) {
      mfma_result_fence(s);  // the masking below reads the MFMA result in assembly
      // bit o of `drop` is set when key 32 kb + o of the tile is masked for this lane's row
      const uint32_t drop = ~keep >> (ln.hi * 4);
      float sv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = s[r];
      drop_keys(sv, drop);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = sv[r];
    }
    return s;
  }

  // Bit o set when key base + o is kept for this lane's row (one 32-key half).
  static __device__ __forceinline__ uint32_t keep_bits(const Lane& ln, int base) {
    return low_bits(ln.hi_lim - base + 1) & (low_bits(ln.sink_lim - base) | ~low_bits(ln.win_lo - base));
  }

  // Row max over the 32 keys of a score block (16 here, 16 in lane ^ 32).
  // Reads the block in assembly: fenced first (the block may be fresh from
  // the MFMA).
  static __device__ __forceinline__ float row_max(f32x16& s) {
    mfma_result_fence(s);
    const float a0 = vmax3(s[0], s[1], s[2]), a1 = vmax3(s[3], s[4], s[5]);
    const float a2 = vmax3(s[6], s[7], s[8]), a3 = vmax3(s[9], s[10], s[11]);
    const float a4 = vmax3(s[12], s[13], s[14]);
    const float mx = vmax2(vmax3(a0, a1, a2), vmax3(a3, a4, s[15]));
    float h0, h1;
    pair_halves(mx, h0, h1);
    return vmax2(h0, h1);
  }

  // One 32-key half (kb) of a tile: S^T block, mask, softmax, PV.
  //
  // The reference max of a row is fixed by the first block that keeps a key
  // of it and never moves afterwards, so the O accumulators are never
  // rescaled and, once every row of the wave has its reference (need_ref
  // false), no max is taken at all.  P = exp2(s c - m c) can then exceed 1
  // when a later key outscores the reference; the caller checks the row
  // sums at the end and, if any exceeds kSumLimit (so some P may have lost
  // range), reruns the list with each row's exact max as the reference.
  // A LOW half's scores are sc times the fp8 code-unit scores (sc > 0).
  static __device__ __forceinline__ void compute_half(const char LDS_AS* stage, const Lane& ln,
                                                      State& st, int kb, int key0, bool partial,
                                                      float c_log2, bool& need_ref, bool low = false,
                                                      float sc = 1.0f, bool fp4 = false) {
    uint32_t keep = ~0u;
    if (partial) {
      keep = keep_bits(ln, key0 + kb * 32);
      if (__ballot(keep != 0) == 0) return;  // no row of the wave keeps a key of this half
    }
    f32x16 s = scores(stage, ln, st, kb, key0, partial, keep, low, fp4);
    const float c = low ? c_log2 * sc : c_log2;
    if (need_ref) {
      // a row with no kept key so far has O = 0 and l = 0: its reference may still move
      const float mx = low ? row_max(s) * sc : row_max(s);
      if (st.m == -INFINITY && mx != -INFINITY) {
        st.m = mx;
        st.neg_mc = -mx * c_log2;
      }
      need_ref = __ballot(st.m == -INFINITY) != 0;
    }
    // P = exp2(s c - m c) as packed bf16; 16-key step kc = registers 8 kc .. 8 kc + 7.
    // Two row sums: of the fp32 P for the LSE, and of the bf16 P the PV
    // product actually uses (v_dot2_f32_bf16) to normalise O, so that the
    // output weights sum to one exactly.  The fp32 sum is a pairwise tree;
    // the bf16 sum is one v_dot2 chain seeded with the running sum (no
    // separate partials to initialise and add).
    bf16x8 pb[2];
    float pf[16];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kc * 8 + x], c, st.neg_mc));
        pf[kc * 8 + x] = p;
        pb[kc][x] = static_cast<__bf16>(p);
      }
#pragma unroll
    for (int r = 0; r < 8; ++r) pf[r] += pf[r + 8];
#pragma unroll
    for (int r = 0; r < 4; ++r) pf[r] += pf[r + 4];
    st.l += (pf[0] + pf[2]) + (pf[1] + pf[3]);
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const bf16x2 pr = {pb[kc][2 * x], pb[kc][2 * x + 1]};
        st.lb = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, st.lb, false);
      }
    // Keep both sums here: left alone, the compiler sinks them past the PV
    // product into the next half, so the 16 fp32 P registers stay live
    // across it and the V reads below run one MFMA ahead instead of four.
    asm volatile("" : "+v"(st.l), "+v"(st.lb));

    // O^T += V^T . P^T ; V^T operand from two transposing reads per 16-key step
    // The PV product runs at raised wave priority: while one wave issues
    // its MFMAs, the other waves of the SIMD fill the gaps with their
    // softmax work instead of holding the MFMA-ready wave back.
    __builtin_amdgcn_s_setprio(1);
    const char LDS_AS* vp = stage + C::kKBytes + ln.v_rd;
    constexpr int kPv = 2 * C::kOBlocks;
    u32x4 vop[kPv];
#pragma unroll
    for (int i = 0; i < kPv; ++i) {
      const int kc = i / C::kOBlocks, ob = i % C::kOBlocks;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(vp + ob * 64 + (kc * 16) * C::kVStride));
      const i16x4 hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(vp + ob * 64 + (kc * 16 + 8) * C::kVStride));
      const u32x2 w0 = __builtin_bit_cast(u32x2, lo);
      const u32x2 w1 = __builtin_bit_cast(u32x2, hv);
      vop[i] = u32x4{w0[0], w0[1], w1[0], w1[1]};
    }
#pragma unroll
    for (int i = 0; i < kPv; ++i)
      st.o[i % C::kOBlocks] = mfma32(__builtin_bit_cast(bf16x8, vop[i]), pb[i / C::kOBlocks], st.o[i % C::kOBlocks]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // operands of the first two MFMAs
#pragma unroll
    for (int i = 0; i < kPv - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the operand of the MFMA two ahead
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_s_setprio(0);
  }

  // Exact-max pass over one 32-key half: scores and row max only.
  static __device__ __forceinline__ void max_half(const char LDS_AS* stage, const Lane& ln, State& st, int kb,
                                                  int key0, bool partial, bool low = false, float sc = 1.0f,
                                                  bool fp4 = false) {
    uint32_t keep = ~0u;
    if (partial) {
      keep = keep_bits(ln, key0 + kb * 32);
      if (__ballot(keep != 0) == 0) return;
    }
    f32x16 s = scores(stage, ln, st, kb, key0, partial, keep, low, fp4);
    const float mx = row_max(s);
    st.mt = fmaxf(st.mt, low ? mx * sc : mx);
  }
};

template <int D, bool kOutBf16, bool kCausal, int kTiers>
__global__ __launch_bounds__(kThreads, 3) void attn_fwd_kernel(const AttnLaunch a) {
  using K = Kernel<D, kOutBf16, kCausal, kTiers>;
  using C = Cfg<D>;
  // two K/V stages
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * C::kStageBytes];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;

  const WorkItem w = schedule_item(a.sched, blockIdx.x);
  if (w.t < 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the range is lost through readfirstlane; with it the copy loops below
  // drop the guards of the blocks every wave has
  __builtin_assume(wave >= 0 && wave < kWaves);
  const int N = a.seqlen;
  const int n_ktiles = (N + kBlockK - 1) / kBlockK;
  const int g = w.h / a.sched.group;
  const int q0 = w.t * kBlockQ;
  const int l32 = lane & 31;

  typename K::Lane ln;
  ln.hi = lane >> 5;
  ln.qrow = q0 + wave * 32 + l32;

  const int64_t ks_b = a.k_stride[2] * 2;  // token strides in bytes
  const int64_t vs_b = a.v_stride[2] * 2;
  const char* kbase = static_cast<const char*>(a.k) + (w.b * a.k_stride[0] + g * a.k_stride[1]) * 2;
  const char* vbase = static_cast<const char*>(a.v) + (w.b * a.v_stride[0] + g * a.v_stride[1]) * 2;

  // operand read offsets: K row l32, channels 8 hi .. 8 hi + 7 (+ 16 per k-step);
  // V^T transposing read: lane (G = lane / 16, k' = lane % 16 / 4, r = lane % 4)
  // points at key 4 (G / 2) + k' (+ 16 kc + 8 x), channels 16 (G % 2) + 4 r .. +3
  // (+ 32 ob).  Destination lane (G, 4 r + c) then receives channel
  // 16 (G % 2) + 4 r + c of keys 4 (G / 2) + 0..3: the layout of the PV operand.
  ln.k_rd = l32 * C::kKStride + ln.hi * 16;
  {
    const int G = lane >> 4, kq = (lane >> 2) & 3, r = lane & 3;
    ln.v_rd = ((G >> 1) * 4 + kq) * C::kVStride + (16 * (G & 1) + 4 * r) * 2;
  }
  // DMA sources of this lane (see issue_dma)
#pragma unroll
  for (int i = 0; i < C::kKBlocksPerWave; ++i) {
    int row, chunk;
    dma_source<D>((i * kWaves + wave) * 1024 + lane * 16, C::kKStride, row, chunk);
    ln.k_dma[i] = static_cast<uint32_t>(min(row, kHalf - 1) * ks_b) + chunk * 16;
  }
#pragma unroll
  for (int i = 0; i < C::kVBlocksPerWave; ++i) {
    int row, chunk;
    dma_source<D>((i * kWaves + wave) * 1024 + lane * 16, C::kVStride, row, chunk);
    ln.v_dma[i] = static_cast<uint32_t>(min(row, kHalf - 1) * vs_b) + chunk * 16;
  }

  // tiered kernel: fp8 K rows of D bytes per (batch, KV head); the LOW test
  // of key tile kt is q0 - (64 kt + 63) >= this head's boundary
  const char* k8base = nullptr;
  const CONST_AS float* k8scale = nullptr;
  int low_dist = 0;
  if constexpr (kTiers) {
    const int64_t bg = static_cast<int64_t>(w.b) * a.sched.heads_kv + g;
    k8base = static_cast<const char*>(a.k8) + bg * N * D;
    k8scale = reinterpret_cast<const CONST_AS float*>(reinterpret_cast<uintptr_t>(a.k8_scale)) + bg * n_ktiles;
    low_dist = a.head_low_dist[w.h];
    ln.k8_rd = l32 * C::kK8Stride + ln.hi * 32;
  }
  // fp4 tier (optional): rows of D / 2 bytes; a tile is fp4 when
  // q0 - (64 kt + 63) >= this head's fp4 boundary (the farthest tier wins)
  const char* k4base = nullptr;
  const CONST_AS float* k4scale = nullptr;
  int fp4_dist = INT_MAX;
  if constexpr (kTiers >= 2) {
    {
      const int64_t bg = static_cast<int64_t>(w.b) * a.sched.heads_kv + g;
      k4base = static_cast<const char*>(a.k4) + bg * N * (D / 2);
      k4scale = reinterpret_cast<const CONST_AS float*>(reinterpret_cast<uintptr_t>(a.k4_scale)) + bg * n_ktiles;
      fp4_dist = a.head_fp4_dist[w.h];
    }
    ln.k4_rd = l32 * C::kK4Stride + ln.hi * 16;
  }
  auto is_low = [&](int kt) __attribute__((always_inline)) -> bool { return kTiers && q0 - (kt * kBlockK + kBlockK - 1) >= low_dist; };
  auto is_fp4 = [&](int kt) __attribute__((always_inline)) -> bool { return kTiers >= 2 && q0 - (kt * kBlockK + kBlockK - 1) >= fp4_dist; };

  // mask bounds of this lane's row: j <= hi_lim and (j < sink_lim or j >= win_lo);
  // per-head boundaries, when given, replace the layer's sink and window
  int head_sink = a.sink, head_window = a.window;
  if (a.head_sink) {
    head_sink = min(max(a.head_sink[w.h], 0), N);
    head_window = max(1, min(a.head_window[w.h], N));
  }
  ln.hi_lim = min(ln.qrow, N - 1);
  if (kCausal || ln.qrow >= N - a.last_q) {
    ln.sink_lim = 0;
    ln.win_lo = 0;
  } else {
    ln.sink_lim = head_sink;
    ln.win_lo = ln.qrow - head_window + 1;
  }


  // kept tiles of this query tile
  int e_begin, e_end;
  if (kCausal) {
    e_begin = 0;
    e_end = (min(N, q0 + kBlockQ) - 1) / kBlockK + 1;
  } else {
    const int64_t r = w.b * a.list_batch_rows + static_cast<int64_t>(w.h) * a.list_head_rows + w.t;
    e_begin = a.row_ptr[r];
    e_end = a.row_ptr[r + 1];
    if (!kTiers && w.c >= 0) {
      // chunk c of a split row: entries [c C, (c + 1) C) of the list (possibly none)
      const int lo = e_begin + w.c * a.chunk_tiles;
      e_end = min(e_end, lo + a.chunk_tiles);
      e_begin = min(lo, e_end);
    }
  }
  // tile list in registers, 64 entries per batch (lane i holds entry e0 + i)
  int list_e0 = e_begin;
  int list_kt = 0, list_fl = 0;
  auto load_list = [&](int e0) __attribute__((always_inline)) {
    list_e0 = e0;
    if (!kCausal) {
      const int e = e0 + lane;
      list_kt = e < e_end ? a.k_tile[e] : 0;
      list_fl = e < e_end ? a.flags[e] : 0;
    }
  };
  auto tile_of = [&](int e) __attribute__((always_inline)) -> int {
    return kCausal ? e : __builtin_amdgcn_readlane(list_kt, e - list_e0);
  };
  auto partial_of = [&](int e, int kt) __attribute__((always_inline)) -> bool {
    if (kCausal) {
      const int c1 = kt * kBlockK + kBlockK - 1;
      return c1 > q0 || c1 >= N;
    }
    return __builtin_amdgcn_readlane(list_fl, e - list_e0) != TRI_TILE_FULL;
  };

  typename K::State st;
  auto load_q = [&]() __attribute__((always_inline)) {
    const int qr = ln.qrow;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + w.b * a.q_stride[0] + w.h * a.q_stride[1] +
                         static_cast<int64_t>(qr) * a.q_stride[2] + ln.hi * 8;
#pragma unroll
    for (int q = 0; q < C::kQSteps; ++q) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qr < N) x = *reinterpret_cast<const u32x4*>(qp + q * 16);
      st.q[q] = __builtin_bit_cast(bf16x8, x);
    }
  };
  // Tiered kernel: fp8 Q (from the bf16 Q just loaded) in the fp8 operand
  // order: step q8 takes the bf16 k-steps 4 q8 .. 4 q8 + 3 of this lane
  // (channels 16 s + 8 hi + 0..7), so the fp8 K rows are stored with the same
  // channel order; scale = amax / 448.
  // row amax of the bf16 Q just loaded (its two lane halves)
  auto q_amax = [&]() __attribute__((always_inline)) -> float {
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < C::kQSteps; ++q)
#pragma unroll
      for (int x = 0; x < 8; ++x) amax = fmaxf(amax, fabsf(static_cast<float>(st.q[q][x])));
    float p0, p1;
    pair_halves(amax, p0, p1);
    return fmaxf(p0, p1);
  };
  // fp4 Q (three-tier kernel): word s of step q holds the 8 channels of bf16
  // k-step 4 q + s, the element order of the fp4 K rows; scale = amax / 6
  auto make_q4 = [&]() __attribute__((always_inline)) {
    if constexpr (kTiers >= 2) {
      const float amax = q_amax();
      const float inv4 = amax > 0.0f ? 6.0f / amax : 0.0f;
      st.s_q4 = amax / 6.0f;
#pragma unroll
      for (int q4 = 0; q4 < C::kQ8Steps; ++q4)
#pragma unroll
        for (int qs = 0; qs < 4; ++qs) {
          float v[8];
#pragma unroll
          for (int x = 0; x < 8; ++x)
            v[x] = fminf(fmaxf(static_cast<float>(st.q[4 * q4 + qs][x]) * inv4, -6.0f), 6.0f);
          unsigned word = 0;
          word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[0], v[1], 1.0f, 0);
          word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[2], v[3], 1.0f, 1);
          word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[4], v[5], 1.0f, 2);
          word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[6], v[7], 1.0f, 3);
          st.q4[q4][qs] = word;
        }
    }
  };
  auto make_q8 = [&]() __attribute__((always_inline)) {
    if constexpr (kTiers >= 1) {
      const float amax = q_amax();
      const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
      st.s_q = amax / 448.0f;
#pragma unroll
      for (int q8 = 0; q8 < C::kQ8Steps; ++q8)
#pragma unroll
        for (int qs = 0; qs < 4; ++qs)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            float v[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
              v[x] = fminf(fmaxf(static_cast<float>(st.q[4 * q8 + qs][4 * half + x]) * inv, -448.0f), 448.0f);
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
            st.q8[q8][2 * qs + half] = word;
          }
    }
  };
  // the Q form of the first phase: fp4 Q in the three-tier kernel (fp8 Q is
  // made at the fp4 -> fp8 boundary), else fp8 Q
  auto first_q = [&]() __attribute__((always_inline)) {
    load_q();
    if constexpr (kTiers >= 2)
      make_q4();
    else
      make_q8();
  };
  first_q();
  st.m = -INFINITY;
  st.neg_mc = 0.0f;
  st.mt = -INFINITY;
  bool need_ref = true;

  const float c_log2 = a.scale * kLog2e;

  // copies of half kb of tile kt into a stage: bf16 K (tier 0), fp8 K (tier
  // 1) or fp4 K (tier 2), and V
  auto dma = [&](char LDS_AS* stage, int kt, int kb, int tier) __attribute__((always_inline)) {
    const int key0 = kt * kBlockK + kb * kHalf;
    // keys past the sequence end (the second half of a last tile can start
    // there) are outside the descriptor and land as zeros; so does a key tile
    // outside 0 .. nk - 1 (a malformed list): no byte outside K and V is read
    const int rows = static_cast<unsigned>(kt) < static_cast<unsigned>(n_ktiles) ? max(N - key0, 0) : 0;
    if (kTiers && tier == 2)
      K::issue_dma_fp4(stage, ln, wave, buffer_rsrc(k4base + static_cast<int64_t>(key0) * (D / 2),
                                                    static_cast<uint32_t>(rows * (D / 2))),
                       buffer_rsrc(vbase + key0 * vs_b, static_cast<uint32_t>(rows * vs_b)));
    else if (kTiers && tier == 1)
      K::issue_dma_low(stage, ln, wave, buffer_rsrc(k8base + static_cast<int64_t>(key0) * D,
                                                    static_cast<uint32_t>(rows * D)),
                       buffer_rsrc(vbase + key0 * vs_b, static_cast<uint32_t>(rows * vs_b)));
    else
      K::issue_dma(stage, ln, wave, buffer_rsrc(kbase + key0 * ks_b, static_cast<uint32_t>(rows * ks_b)),
                   buffer_rsrc(vbase + key0 * vs_b, static_cast<uint32_t>(rows * vs_b)));
  };

  // The LOW test is monotone in kt, so in an ascending list the LOW tiles
  // are the entries [e_begin, e_split); the tiered walk takes them first with
  // fp8 Q only, then reloads bf16 Q for the rest, so the two copies of Q are
  // never held together.
  // Likewise the fp4 tiles are a prefix [e_begin, e_split4) of it, and the
  // fp8 ones [e_split4, e_split) follow.
  int e_split = e_begin, e_split4 = e_begin;
  if constexpr (kTiers) {
    for (int e0 = e_begin; e0 < e_end; e0 += 64) {
      const int e = e0 + lane;
      const int kt = e < e_end ? a.k_tile[e] : 0;
      const uint64_t bits = __ballot(e < e_end && (is_low(kt) || is_fp4(kt)));
      const uint64_t bits4 = __ballot(e < e_end && is_fp4(kt));
      e_split += __popcll(bits);
      e_split4 += __popcll(bits4);
      if (~bits != 0) break;
    }
  }

  // tier of list entry e (2: fp4, 1: fp8, 0: bf16)
  auto tier_of = [&](int e) __attribute__((always_inline)) -> int { return e < e_split4 ? 2 : (e < e_split ? 1 : 0); };

  // Walks the kept tiles in 32-key halves: entries [e_begin, e_split4) with
  // fp4_half, [e_split4, e_split) with low_half, then at_split(), then
  // [e_split, e_end) with high_half; each half callback is called as
  // half(stage, key0, kb, partial).
  auto walk = [&](auto&& fp4_half, auto&& low_half, auto&& at_split, auto&& high_half) __attribute__((always_inline)) {
    load_list(e_begin);
    if (e_begin < e_end) dma(smem, tile_of(e_begin), 0, tier_of(e_begin));
    int cur = 0;  // byte offset of the stage holding the current half
    // tier: of the phase's halves; a prefetch takes min(tier, the next entry's)
    auto run = [&](int e_lo, int e_hi, int tier, auto&& half) __attribute__((always_inline)) {
      for (int e = e_lo; e < e_hi; ++e) {
        const int kt = tile_of(e);
        const bool partial = partial_of(e, kt);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          wait_vmcnt0();    // this wave's copies of this half have landed
          __syncthreads();  // ... and every wave's; all reads of the other stage are done
          if (kb == 0) {
            dma(smem + (cur ^ C::kStageBytes), kt, 1, tier);
          } else if (e + 1 < e_end) {
            if (e + 1 - list_e0 == 64) load_list(e + 1);
            dma(smem + (cur ^ C::kStageBytes), tile_of(e + 1), 0, min(tier, tier_of(e + 1)));
          }
          half(smem + cur, kt * kBlockK, kb, partial);
          cur ^= C::kStageBytes;
        }
      }
    };
    if constexpr (kTiers >= 2) {
      run(e_begin, e_split4, 2, fp4_half);
      load_q();  // fp4 -> fp8: fp8 Q from a fresh bf16 Q
      make_q8();
    }
    if constexpr (kTiers >= 1) {
      run(e_split4, e_split, 1, low_half);
      at_split();
    }
    run(e_split, e_end, 0, high_half);
    __syncthreads();  // all reads of the last stage are done before another walk refills it
  };
  // score scale of a LOW key tile starting at key0: s_q times the fp8 K scale
  // of that tile (kept positive so that 0 * -inf never arises: a zero scale
  // means all-zero codes, whose scores are 0 at any positive scale); the
  // index stays inside the ceil(N / 64) scales of the head
  auto tile_scale = [&](const CONST_AS float* sc, int key0) __attribute__((always_inline)) -> float {
    return sc[min(max(key0 / kBlockK, 0), n_ktiles - 1)];
  };
  auto low_sc = [&](int key0) __attribute__((always_inline)) -> float {
    if constexpr (kTiers) return fmaxf(st.s_q * tile_scale(k8scale, key0), 1.17549435e-38f);
    return 1.0f;
  };
  auto fp4_sc = [&](int key0) __attribute__((always_inline)) -> float {
    if constexpr (kTiers >= 2) return fmaxf(st.s_q4 * tile_scale(k4scale, key0), 1.17549435e-38f);
    return 1.0f;
  };
  auto attend_fp4 = [&](const char LDS_AS* stage, int key0, int kb, bool partial) __attribute__((always_inline)) {
    K::compute_half(stage, ln, st, kb, key0, partial, c_log2, need_ref, true, fp4_sc(key0), true);
  };
  auto attend_low = [&](const char LDS_AS* stage, int key0, int kb, bool partial) __attribute__((always_inline)) {
    K::compute_half(stage, ln, st, kb, key0, partial, c_log2, need_ref, true, low_sc(key0));
  };
  auto attend = [&](const char LDS_AS* stage, int key0, int kb, bool partial) __attribute__((always_inline)) {
    K::compute_half(stage, ln, st, kb, key0, partial, c_log2, need_ref);
  };
  auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::kOBlocks; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[i][r] = 0.0f;
    st.l = 0.0f;
    st.lb = 0.0f;
  };
  auto reload_q = [&]() __attribute__((always_inline)) {
    if constexpr (kTiers) load_q();
  };
  auto requant_q = [&]() __attribute__((always_inline)) {
    if constexpr (kTiers) first_q();
  };

  // Usual case: one walk with a fixed reference per row.  Every P of a row is
  // at most its row sum, so below kSumLimit nothing lost range; otherwise
  // walk again for the exact row maxima and once more with them as the
  // reference (then every P <= 1).
  clear();
  walk(attend_fp4, attend_low, reload_q, attend);
  if (__syncthreads_or(!(st.l <= kSumLimit))) {
    requant_q();
    walk([&](const char LDS_AS* stage, int key0, int kb, bool partial) __attribute__((always_inline)) {
           K::max_half(stage, ln, st, kb, key0, partial, true, fp4_sc(key0), true);
         },
         [&](const char LDS_AS* stage, int key0, int kb, bool partial) __attribute__((always_inline)) {
           K::max_half(stage, ln, st, kb, key0, partial, true, low_sc(key0));
         },
         reload_q,
         [&](const char LDS_AS* stage, int key0, int kb, bool partial) __attribute__((always_inline)) {
           K::max_half(stage, ln, st, kb, key0, partial);
         });
    st.m = st.mt;
    st.neg_mc = st.mt == -INFINITY ? 0.0f : -st.mt * c_log2;
    need_ref = false;
    clear();
    requant_q();
    walk(attend_fp4, attend_low, reload_q, attend);
  }

  // epilogue
  float l0, l1, b0, b1;
  pair_halves(st.l, l0, l1);
  pair_halves(st.lb, b0, b1);
  const float l_tot = l0 + l1;
  if (!kTiers && w.c >= 0) {
    // chunk of a split row (the tiered kernel is never split): unnormalised O and the row's (reference max, fp32
    // sum, bf16 sum), merged by the split merge kernel.  A row that kept no
    // key of this chunk leaves m = -inf, sums 0 and O 0.
    const int64_t item =
        ((static_cast<int64_t>(w.b) * a.sched.heads_q + w.h) * a.sched.n_heavy + (a.sched.n_qtiles - 1 - w.t)) *
            a.sched.n_split + w.c;
    const int row = wave * 32 + l32;
    float* op = a.split_o + (item * kBlockQ + row) * D;
#pragma unroll
    for (int ob = 0; ob < C::kOBlocks; ++ob)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = ob * 32 + r4 * 8 + ln.hi * 4;
        const f32x4 v4 = {st.o[ob][r4 * 4 + 0], st.o[ob][r4 * 4 + 1], st.o[ob][r4 * 4 + 2], st.o[ob][r4 * 4 + 3]};
        *reinterpret_cast<f32x4*>(op + d0) = v4;
      }
    if (ln.hi == 0) {
      float* sp = a.split_stats + item * 3 * kBlockQ + row;
      sp[0] = st.m;
      sp[kBlockQ] = l_tot;
      sp[2 * kBlockQ] = b0 + b1;
    }
    return;
  }
  if (ln.qrow < N) {
    const float inv = 1.0f / (b0 + b1);
    const int64_t orow =
        w.b * a.o_stride[0] + w.h * a.o_stride[1] + static_cast<int64_t>(ln.qrow) * a.o_stride[2];
#pragma unroll
    for (int ob = 0; ob < C::kOBlocks; ++ob)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = ob * 32 + r4 * 8 + ln.hi * 4;
        const f32x4 v4 = {st.o[ob][r4 * 4 + 0] * inv, st.o[ob][r4 * 4 + 1] * inv,
                          st.o[ob][r4 * 4 + 2] * inv, st.o[ob][r4 * 4 + 3] * inv};
        if (kOutBf16) {
          const bf16x4 b4 = {static_cast<__bf16>(v4[0]), static_cast<__bf16>(v4[1]),
                             static_cast<__bf16>(v4[2]), static_cast<__bf16>(v4[3])};
          *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(a.o) + orow + d0) = b4;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d0) = v4;
        }
      }
    if (a.lse && ln.hi == 0)
      a.lse[w.b * a.lse_stride[0] + w.h * a.lse_stride[1] + ln.qrow] = st.m * a.scale + logf(l_tot);
  }
}

template <int D, bool kOutBf16, bool kCausal, int kTiers = 0>
int launch_t(const AttnLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, kOutBf16, kCausal, kTiers>),
                     dim3(static_cast<unsigned>(a.sched.grid)), dim3(kThreads), 0, stream, a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(TRI_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return TRI_OK;
}

template <int D>
int launch_d(const AttnLaunch& a, hipStream_t stream) {
  if (a.k4) return a.o_bf16 ? launch_t<D, true, false, 2>(a, stream) : launch_t<D, false, false, 2>(a, stream);
  if (a.k8) return a.o_bf16 ? launch_t<D, true, false, 1>(a, stream) : launch_t<D, false, false, 1>(a, stream);
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
