// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, cross-lane reductions, bf16 packing and the XCD-aware
// workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBlockSize = 16;  // paged KV block, in tokens

// 32x32 output tile, K = 16.  A: lane l holds row l%32, 8 contraction
// elements; B: lane l holds column l%32, the same 8 contraction elements.
// D: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16 output tile, K = 32.  D: lane l, register r holds row 4*(l/16) + r,
// column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane l ^ 32 (the other half of the wavefront).
__device__ __forceinline__ float xor32(float x) {
  int v = __float_as_int(x);
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  // lanes 0..31: r[1] holds lane l+32; lanes 32..63: r[0] holds lane l-32
  return __int_as_float((__lane_id() < 32) ? r[1] : r[0]);
}

// Value held by lane l ^ 16 (within each 32-lane half): ds_swizzle in
// bit-mask mode with and_mask 0x1f, xor_mask 0x10.
__device__ __forceinline__ float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// Round-to-nearest-even float -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f2bf_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f2bf_bits(lo) | (f2bf_bits(hi) << 16);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// bf16 value of a float after rounding, as a float (for sums that must see
// exactly the rounded weights).
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f2bf_bits(f) << 16); }

// Rotary embedding, shared by every kernel that rotates so that they all
// round identically.  cos and sin of the angle pos * theta: positions reach
// tens of thousands of radians, where a float angle is off by ~1e-3 rad, so
// the angle is formed and reduced modulo 2*pi in double precision (two-part
// 2*pi, Cody-Waite); sine and cosine of the reduced angle (|r| <= pi) are then
// taken in float, accurate to about one float ulp.
__device__ __forceinline__ void rope_cos_sin(int32_t pos, double theta, float& c, float& s) {
  constexpr double kTwoPiHi = 6.283185307179586;       // 2*pi rounded to double
  constexpr double kTwoPiLo = 2.4492935982947064e-16;  // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189535;
  const double ang = (double)pos * theta;
  const double k = rint(ang * kInvTwoPi);
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
  sincosf((float)r, &s, &c);
}
// Rotation of the pair (x1, x2) = (x[i], x[i + D/2]) by that angle, with an
// explicit order of roundings (no contraction left to the compiler).
__device__ __forceinline__ void rope_rotate(float x1, float x2, float c, float s, float& y1, float& y2) {
  y1 = fmaf(x1, c, -__fmul_rn(x2, s));
  y2 = fmaf(x2, c, __fmul_rn(x1, s));
}

// Partials that cross workgroups (and XCDs, whose L2 caches are not
// coherent with each other) inside one launch are written and read as
// device-scope relaxed atomics: they go to the device's coherence point
// instead of the XCD's L2, so no cache writeback or invalidation is needed.
// A workgroup's partial stores are complete (vmcnt 0) before it counts its
// arrival, and the merging workgroup reads them after the count.
__device__ __forceinline__ void store_coherent(float* p, float x, float y) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, f32x2{x, y}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 load_coherent(const float* p) {
  return __builtin_bit_cast(f32x2, __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}

// Arrival of one of `n` workgroups that share a merge: returns true (to
// every thread) in the last to arrive, which then restores the counter to
// its value before the launch (zero).  Every thread's partial stores must be
// complete (vmcnt 0) before the call; `flag` is one int of LDS that no wave
// still uses.
__device__ __forceinline__ bool arrive_last(int32_t* counter, int n, int* flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(counter, 1);
    const int last = prev == n - 1;
    if (last) atomicSub(counter, n);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// ---- debug builds (compiled with MI_ATTN_DEBUG=1)
// The kernels keep every access in bounds whatever the caller passes (block
// ids are clamped, bad slots and pairs skipped, lengths cut to what the
// launch covers).  A debug build also says that it happened: each kernel ORs
// a bit per kind of malformed input it met (ATTN_DEBUG_* in mi_attn.h) into
// a word of its translation unit, which attn_debug_flags reads back.  In a
// release build the checks compile to nothing.
#ifndef MI_ATTN_DEBUG
#define MI_ATTN_DEBUG 0
#endif
constexpr uint32_t kDebugBlockId = 1u;   // a block-table entry in use outside [0, num_blocks)
constexpr uint32_t kDebugSlot = 2u;      // a slot below -1 or at or past num_blocks * 16
constexpr uint32_t kDebugContext = 4u;   // a length below 0 or beyond what the table row / launch covers
constexpr uint32_t kDebugCopyPair = 8u;  // a copy pair with an id outside [0, num_blocks)
constexpr uint32_t kDebugSeqlens = 16u;  // cu_seqlens_q not rising from 0 to at most total_q

// DEBUG_ONLY(statement): the statement in debug builds, nothing at all in
// release builds (whose code is then exactly what it is without the checks).
#if MI_ATTN_DEBUG
#define DEBUG_ONLY(...) __VA_ARGS__
static __device__ uint32_t debug_word;

__device__ __forceinline__ void debug_report(bool bad, uint32_t bit) {
  if (bad) atomicOr(&debug_word, bit);
}
// Checks of per-sequence inputs, made by thread 0 of a workgroup: a length
// against the tokens the launch (or table row) covers, and a paged
// prefill's query offsets.
__device__ __forceinline__ void debug_check_length(int32_t len, int32_t bound) {
  debug_report(threadIdx.x == 0 && (len < 0 || len > bound), kDebugContext);
}
__device__ __forceinline__ void debug_check_seqlens(const int32_t* cu_seqlens_q, int b, int32_t total_q) {
  if (threadIdx.x == 0) {
    const int32_t c0 = cu_seqlens_q[b], c1 = cu_seqlens_q[b + 1];
    debug_report((b == 0 && c0 != 0) || c1 < c0 || c1 > total_q, kDebugSeqlens);
  }
}
// A slot of the paged cache: -1 (skip) or in [0, num_blocks * 16).
__device__ __forceinline__ void debug_check_slot(bool live, int32_t slot, int32_t num_blocks) {
  debug_report(live && (slot < -1 || slot >= num_blocks * kBlockSize), kDebugSlot);
}
#else
#define DEBUG_ONLY(...)
#endif

// Host side: OR this translation unit's word on the current device into
// *acc, and zero it when `clear` (synchronous; the caller has synchronised
// the device).  Release builds: nothing.
static inline hipError_t debug_take_word(uint32_t* acc, bool clear) {
#if MI_ATTN_DEBUG
  uint32_t w = 0;
  hipError_t e = hipMemcpyFromSymbol(&w, HIP_SYMBOL(debug_word), sizeof(w), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *acc |= w;
  if (clear && w != 0) {
    const uint32_t zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(debug_word), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
  }
  return e;
#else
  (void)acc;
  (void)clear;
  return hipSuccess;
#endif
}

// A block-table entry outside the pool is replaced by block 0 so that a
// corrupt table can never address memory outside the cache.  Callers pass
// only entries the kernel needs (debug builds report the others).
__device__ __forceinline__ int32_t safe_block(int32_t blk, int32_t num_blocks) {
  DEBUG_ONLY(debug_report(blk < 0 || blk >= num_blocks, kDebugBlockId));
  return (blk >= 0 && blk < num_blocks) ? blk : 0;
}

}  // namespace mi_attn
