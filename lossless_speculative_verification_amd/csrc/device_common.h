// Device helpers shared by the gfx950 kernels of the verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mv {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kRowBlockBytes = 256; // bytes of one row per K block of the packed GEMM layout
constexpr int kChunksPerRow = kRowBlockBytes / 16;  // 16-byte chunks per row per K block
constexpr int kPairUnits = 2 * 4 * kWave;           // 16-byte units per (pair, K block) = 8 KB
constexpr int kGemmWaves = 4;                       // waves per GEMM workgroup (one pair each)
// Streaming GEMM shape: row tiles (16 rows each) per work item and K blocks in flight
// per wavefront, for the expert GEMMs and the LM head.
#ifndef MV_GEMM_NMT
#define MV_GEMM_NMT 2
#endif
#ifndef MV_GEMM_D
#define MV_GEMM_D 2
#endif
#ifndef MV_GEMM_WAVES_PER_SIMD
#define MV_GEMM_WAVES_PER_SIMD 2
#endif
// Wavefronts per workgroup of the streaming expert GEMM. Each wavefront works alone, and a
// compute unit's share of the weight stream sets the kernel's time (one CU sustains only
// so many loads in flight). The gate/up launch has about two workgroups of four per CU;
// the down launch has fewer chunks per item, and one-wavefront workgroups let the
// dispatcher spread its wavefronts more evenly over the compute units.
constexpr int kStreamWavesUp = 4;
constexpr int kStreamWavesDown = 1;
constexpr int kGemmMB = 16 * MV_GEMM_NMT;           // rows per expert GEMM work item
constexpr int kLmRows = 128;                        // positions per LM-head row block
constexpr int kLmWaves = 8;                          // wavefronts per LM-head workgroup (one workgroup per CU)
constexpr int kSelfPlanMaxSlots = 4096;      // routed slots up to which the streaming gate/up plans itself
constexpr int kNormSplitMaxPositions = 4096;  // passes below this use the split norm/router kernel
constexpr int kTileM = 256;                         // rows per work item of the LDS-tiled expert GEMM
constexpr int kPlanChunk = 2048;                    // routed slots per workgroup of the large-pass plan
constexpr int kPlanSingleMaxChunks = 8;             // up to this many chunks one workgroup plans alone

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Calls f(std::integral_constant<int, i>{}) for i = 0..N-1: a loop whose index must be a
// compile-time constant (it selects a register array of a software pipeline).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Stage-ordered row layout of bf16 activation rows, read by the LDS-tiled expert GEMM:
// within each 256-byte block of a row, the 16-byte chunk c = 4*g + s (s = c % 4) is
// stored at chunk position 4*s + g, so the four chunks one MFMA step contracts (chunks
// 4*g + s, g = 0..3) are 64 contiguous bytes. Element index of element e of a row.
__device__ __forceinline__ int stage_ordered_elem(int e) {
  const int c = (e >> 3) & 15;
  return (e & ~127) | ((((c & 3) << 2) | (c >> 2)) << 3) | (e & 7);
}

// bf16 is carried as uint16_t bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bf16 bit pattern, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int per16 = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ float load(const float* p, int i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static constexpr int per16 = 8;
  __device__ static __forceinline__ float load(const uint16_t* p, int i) { return bf16_to_f32(p[i]); }
};

// Store a float32 value as the element type (bf16 rounding or plain float).
__device__ __forceinline__ void store_elem(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, size_t i, float v) { p[i] = (uint16_t)f32_to_bf16(v); }

// acc += A_chunk * B_chunk over one 16-byte chunk per lane.
// Lane l holds row (l % 16) of A and column (l % 16) of B; the four lane groups
// (l / 16) hold disjoint K slices, identically placed in A and B, so the sum covers
// every K element of the chunk exactly once whatever the K order inside the MFMA.
// The 16x16 result: lane l holds column (l % 16), rows 4*(l/16) + 0..3.
__device__ __forceinline__ void mma_chunk(f32x4_t& acc, uint4 a, uint4 b, uint16_t*) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_chunk(f32x4_t& acc, uint4 a, uint4 b, float*) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Streaming (read-once) 16-byte load: non-temporal, so the weight stream does not
// evict the small, re-used activation rows from the caches.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// SwiGLU of one gate/up pair, silu(g) * u with silu(g) = g / (1 + e^-g), from the
// hardware exponential and reciprocal (a few ulp of float32, far below the bf16 rounding
// the result gets; e^-g overflowing to infinity gives a reciprocal of exactly 0).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Top-1/top-2 record for the argmax reductions: value, lowest index, second value.
struct Top2 {
  float v1;
  int i1;
  float v2;
};

// Merge two records: the larger value wins, the lower index on equal values; the
// loser's best competes for second place. Commutative and associative. Written with
// selects only (no branch), so merges of independent records overlap.
__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  // (bitwise operators: a short-circuit form compiles to a branch)
  const bool b_wins = (b.v1 > a.v1) | ((b.v1 == a.v1) & (b.i1 < a.i1));
  const float w2 = b_wins ? b.v2 : a.v2, l1 = b_wins ? a.v1 : b.v1;
  return Top2{b_wins ? b.v1 : a.v1, b_wins ? b.i1 : a.i1, fmaxf(w2, l1)};
}

// Fold value v of column c into a running record whose columns all precede c: v takes
// first place only when strictly larger (so the lowest index wins on equal values), else
// competes for second place. A NaN value changes nothing.
__device__ __forceinline__ void top2_push(Top2& b, float v, int c) {
  const bool gt = v > b.v1, g2 = v > b.v2;
  b.v2 = gt ? b.v1 : (g2 ? v : b.v2);
  b.i1 = gt ? c : b.i1;
  b.v1 = gt ? v : b.v1;
}

// The value of lane l ^ mask. Masks 16 and 32 use the gfx950 row swaps (no LDS round trip):
// swapping a register with itself leaves, in each lane, either its own value or its
// partner's in one of the two results.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x, int mask) {
  if (mask == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  }
  if (mask == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
  return (uint32_t)__shfl_xor((int)x, mask, kWave);
}

__device__ __forceinline__ Top2 top2_shfl_xor(Top2 t, int mask) {
  Top2 o;
  o.v1 = __builtin_bit_cast(float, lane_xor_u32(__builtin_bit_cast(uint32_t, t.v1), mask));
  o.i1 = (int)lane_xor_u32((uint32_t)t.i1, mask);
  o.v2 = __builtin_bit_cast(float, lane_xor_u32(__builtin_bit_cast(uint32_t, t.v2), mask));
  return o;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Logical workgroup index of hardware workgroup h when the first n carry work.
// Workgroups are dealt to the 8 XCDs round-robin; here each XCD takes one contiguous
// range of logical indices instead, so logical neighbours (the row blocks of one expert,
// which stream the same weights) share one L2.
__device__ __forceinline__ int xcd_logical(int h, int n) {
  const int x = h & 7, j = h >> 3;
  int start = 0;
  for (int y = 0; y < x; ++y) start += (n - y + 7) >> 3;
  return start + j;
}

}  // namespace mv
