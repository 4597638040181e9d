// Fused rotary embedding + paged KV-cache write.
//
// "Fast Attention Kernels and Operator Fusion", §Operator Fusion, lists
// "applying rotary position embeddings to queries and keys" and "updating the
// KV cache while transforming key and value tensors" as fusion targets: one
// pass reads q, k and v once, rotates q in place and writes the rotated key
// and the value into the token's paged slot.
//
// Rotation (half-split pairs): for i < D/2 the pair (x[i], x[i + D/2]) turns
// by angle pos * base^(-2i/D).  Positions reach tens of thousands of radians,
// where a float angle is off by ~1e-3 rad, so the angle is formed and reduced
// modulo 2*pi in double precision (two-part 2*pi, Cody-Waite); sine and cosine
// of the reduced angle (|r| <= pi) are then taken in float, accurate to about
// one float ulp.  The rotation itself is float arithmetic; bf16 outputs are
// rounded to nearest even.
//
// Workgroup = kTok tokens, 256 threads.  Each thread moves four channel pairs
// of one row (8-byte accesses for bf16).

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

constexpr int kTok = 8;

template <typename T>
struct Vec4;
template <>
struct Vec4<__bf16> {
  static __device__ __forceinline__ f32x4 load(const __bf16* p) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
  }
  static __device__ __forceinline__ void store(__bf16* p, f32x4 v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};
template <>
struct Vec4<float> {
  static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};

template <int D, typename T>
__global__ __launch_bounds__(256) void rope_write_kernel(const RopeWriteArgs a) {
  constexpr int H2 = D / 2;
  constexpr int CPR = H2 / 4;  // four-pair chunks per row
  __shared__ double theta[H2];
  __shared__ float cs[kTok][H2], sn[kTok][H2];
  __shared__ int32_t slot_sm[kTok];
  const int n0 = blockIdx.x * kTok;
  const int tid = threadIdx.x;
  const int ntok = min(kTok, a.num_tokens - n0);
  const bool rot = a.rope_base != 0.0;

  if (tid < kTok) {
    int32_t sl = tid < ntok ? a.slot_mapping[n0 + tid] : -1;
    if (sl >= a.num_blocks * kBlockSize) sl = -1;  // outside the pool: skipped
    slot_sm[tid] = sl;
  }
  if (rot) {
    for (int i = tid; i < H2; i += blockDim.x) theta[i] = pow(a.rope_base, -2.0 * (double)i / (double)D);
    __syncthreads();
    constexpr double kTwoPiHi = 6.283185307179586;        // 2*pi rounded to double
    constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2*pi - kTwoPiHi
    constexpr double kInvTwoPi = 0.15915494309189535;
    for (int e = tid; e < ntok * H2; e += blockDim.x) {
      const int t = e / H2, i = e % H2;
      const double ang = (double)a.positions[n0 + t] * theta[i];
      const double k = rint(ang * kInvTwoPi);
      const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
      float s, c;
      sincosf((float)r, &s, &c);
      cs[t][i] = c;
      sn[t][i] = s;
    }
  }
  __syncthreads();

  // q rows (rotated in place) and k rows (rotated into the cache)
  const int rows = a.hq + a.hkv;
  T* q = static_cast<T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  T* kc = static_cast<T*>(a.k_cache);
  for (int w = tid; w < ntok * rows * CPR; w += blockDim.x) {
    const int t = w / (rows * CPR);
    const int rr = (w / CPR) % rows;
    const int i0 = 4 * (w % CPR);
    const int n = n0 + t;
    const bool is_q = rr < a.hq;
    if (is_q && (q == nullptr || !rot)) continue;
    const int32_t sl = slot_sm[t];
    if (!is_q && sl < 0) continue;
    const T* src = is_q ? q + ((int64_t)n * a.hq + rr) * D : k + ((int64_t)n * a.hkv + (rr - a.hq)) * D;
    f32x4 x1 = Vec4<T>::load(src + i0);
    f32x4 x2 = Vec4<T>::load(src + i0 + H2);
    if (rot) {
      f32x4 y1, y2;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = cs[t][i0 + e], s = sn[t][i0 + e];
        y1[e] = x1[e] * c - x2[e] * s;
        y2[e] = x2[e] * c + x1[e] * s;
      }
      x1 = y1;
      x2 = y2;
    }
    T* dst;
    if (is_q) {
      dst = q + ((int64_t)n * a.hq + rr) * D;
    } else {
      const int64_t blk = sl / kBlockSize;
      dst = kc + ((blk * a.hkv + (rr - a.hq)) * kBlockSize + sl % kBlockSize) * D;
    }
    Vec4<T>::store(dst + i0, x1);
    Vec4<T>::store(dst + i0 + H2, x2);
  }

  // values, copied into the token-minor cache: [block][kv head][channel][16]
  const T* v = static_cast<const T*>(a.v);
  T* vc = static_cast<T*>(a.v_cache);
  for (int w = tid; w < ntok * a.hkv * (D / 4); w += blockDim.x) {
    const int t = w / (a.hkv * (D / 4));
    const int g = (w / (D / 4)) % a.hkv;
    const int d0 = 4 * (w % (D / 4));
    const int32_t sl = slot_sm[t];
    if (sl < 0) continue;
    const f32x4 x = Vec4<T>::load(v + ((int64_t)(n0 + t) * a.hkv + g) * D + d0);
    const int64_t blk = sl / kBlockSize;
    T* dst = vc + ((blk * a.hkv + g) * D + d0) * kBlockSize + sl % kBlockSize;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e * kBlockSize] = static_cast<T>(x[e]);
  }
}

}  // namespace

hipError_t launch_rope_write(const RopeWriteArgs& a, int head_dim, bool bf16, hipStream_t s) {
  dim3 grid((a.num_tokens + kTok - 1) / kTok), block(256);
  if (bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((rope_write_kernel<128, __bf16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((rope_write_kernel<64, __bf16>), grid, block, 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((rope_write_kernel<128, float>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((rope_write_kernel<64, float>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mi_attn
