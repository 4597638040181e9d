// Fused rotary embedding + paged KV-cache write.
//
// "Fast Attention Kernels and Operator Fusion", §Operator Fusion, lists
// "applying rotary position embeddings to queries and keys" and "updating the
// KV cache while transforming key and value tensors" as fusion targets: one
// pass reads q, k and v once, rotates q in place and writes the rotated key
// and the value into the token's paged slot.
//
// Rotation (half-split pairs): for i < D/2 the pair (x[i], x[i + D/2]) turns
// by angle pos * base^(-2i/D).  The angle, its sine and its cosine are
// computed in double precision once per (token, i) and shared by every head
// of the token: positions reach tens of thousands, where a float angle is off
// by ~1e-3 rad.  The rotation itself is float arithmetic; bf16 outputs are
// rounded to nearest even.
//
// Workgroup = one token, 256 threads.

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return static_cast<float>(*p); }
template <typename T>
__device__ __forceinline__ void st(T* p, float x) { *p = static_cast<T>(x); }

template <int D, typename T>
__global__ __launch_bounds__(256) void rope_write_kernel(const RopeWriteArgs a) {
  constexpr int H2 = D / 2;
  __shared__ float cs[H2], sn[H2];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const bool rot = a.rope_base != 0.0;
  const int32_t pos = a.positions[n];
  const int32_t slot = a.slot_mapping[n];

  if (rot) {
    for (int i = tid; i < H2; i += blockDim.x) {
      const double theta = pow(a.rope_base, -2.0 * (double)i / (double)D);
      double s, c;
      sincos((double)pos * theta, &s, &c);
      cs[i] = (float)c;
      sn[i] = (float)s;
    }
  }
  __syncthreads();

  if (a.q != nullptr && rot) {
    T* q = static_cast<T*>(a.q) + (int64_t)n * a.hq * D;
    for (int idx = tid; idx < a.hq * H2; idx += blockDim.x) {
      const int h = idx / H2, i = idx % H2;
      T* row = q + h * D;
      const float x1 = ld(row + i), x2 = ld(row + i + H2);
      st(row + i, x1 * cs[i] - x2 * sn[i]);
      st(row + i + H2, x2 * cs[i] + x1 * sn[i]);
    }
  }
  if (slot < 0 || slot >= a.num_blocks * kBlockSize) return;
  const int64_t blk = slot / kBlockSize;
  const int off = slot % kBlockSize;
  const T* k = static_cast<const T*>(a.k) + (int64_t)n * a.hkv * D;
  const T* v = static_cast<const T*>(a.v) + (int64_t)n * a.hkv * D;
  T* kc = static_cast<T*>(a.k_cache);
  T* vc = static_cast<T*>(a.v_cache);
  for (int idx = tid; idx < a.hkv * H2; idx += blockDim.x) {
    const int g = idx / H2, i = idx % H2;
    const T* row = k + g * D;
    T* dst = kc + ((blk * a.hkv + g) * kBlockSize + off) * D;
    if (rot) {
      const float x1 = ld(row + i), x2 = ld(row + i + H2);
      st(dst + i, x1 * cs[i] - x2 * sn[i]);
      st(dst + i + H2, x2 * cs[i] + x1 * sn[i]);
    } else {
      dst[i] = row[i];
      dst[i + H2] = row[i + H2];
    }
  }
  // value cache is token-minor: [block][kv head][channel][16]
  for (int idx = tid; idx < a.hkv * D; idx += blockDim.x) {
    const int g = idx / D, d = idx % D;
    vc[((blk * a.hkv + g) * D + d) * kBlockSize + off] = v[g * D + d];
  }
}

}  // namespace

hipError_t launch_rope_write(const RopeWriteArgs& a, int head_dim, bool bf16, hipStream_t s) {
  dim3 grid(a.num_tokens), block(256);
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
