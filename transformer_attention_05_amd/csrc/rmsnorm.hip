// Fused residual add + RMS normalisation.
//
// "Fast Attention Kernels and Operator Fusion", §Operator Fusion: adding the
// residual and applying RMSNorm is a fusion target; its example adds the
// residual to the input, divides each row by the root mean square of the sum
// (eps under the root) and scales by a weight vector; it has two outputs,
// the normalised rows and the new residual.  Fused, one pass reads every
// input once and writes both: HBM-bound.
//
// One wavefront per row (four rows per workgroup, no barriers): lane l holds
// the 8-element chunks l, l + 64, ... of the row in registers (CPL chunks at
// most), adds the residual in float32, stores the sum in the input dtype
// (the updated residual, rounded once), accumulates the squares of the
// stored values, and after a wavefront sum scales the same registers.
// Consecutive lanes touch consecutive 16-byte (bf16) or 32-byte (fp32)
// chunks, so every access is coalesced.

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

constexpr int kRowsPerWg = 4;

template <typename T>
struct Chunk8;
template <>
struct Chunk8<__bf16> {
  static __device__ __forceinline__ void load(const __bf16* p, float (&v)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf_lo(w[i]);
      v[2 * i + 1] = bf_hi(w[i]);
    }
  }
  static __device__ __forceinline__ void store(__bf16* p, const float (&v)[8]) {
    *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                         pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
  static __device__ __forceinline__ float round(float f) { return round_bf16(f); }
};
template <>
struct Chunk8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
  static __device__ __forceinline__ float round(float f) { return f; }
};

template <typename T, int CPL>
__global__ __launch_bounds__(64 * kRowsPerWg) void residual_rms_norm_kernel(const RmsNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + (threadIdx.x >> 6);
  if (row >= a.rows) return;  // whole wavefronts; the kernel has no barrier
  const int nch = a.hidden / 8;
  const T* x = static_cast<const T*>(a.x) + row * a.hidden;
  const T* r = static_cast<const T*>(a.residual) + row * a.hidden;
  const T* w = static_cast<const T*>(a.weight);
  T* y = static_cast<T*>(a.y) + row * a.hidden;
  T* h_out = static_cast<T*>(a.h_out) + row * a.hidden;

  float h[CPL][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      float xv[8], rv[8];
      Chunk8<T>::load(x + 8 * c, xv);
      Chunk8<T>::load(r + 8 * c, rv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[j][e] = Chunk8<T>::round(xv[e] + rv[e]);  // the updated residual as stored
        ss = fmaf(h[j][e], h[j][e], ss);
      }
      Chunk8<T>::store(h_out + 8 * c, h[j]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.f / sqrtf(ss / (float)a.hidden + a.eps);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c < nch) {
      float wv[8], out[8];
      Chunk8<T>::load(w + 8 * c, wv);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = h[j][e] * inv * wv[e];
      Chunk8<T>::store(y + 8 * c, out);
    }
  }
}

template <typename T>
void launch_t(const RmsNormArgs& a, hipStream_t st) {
  const dim3 grid((uint32_t)((a.rows + kRowsPerWg - 1) / kRowsPerWg)), block(64 * kRowsPerWg);
  const int cpl = (a.hidden / 8 + 63) / 64;
  if (cpl <= 1) hipLaunchKernelGGL((residual_rms_norm_kernel<T, 1>), grid, block, 0, st, a);
  else if (cpl <= 2) hipLaunchKernelGGL((residual_rms_norm_kernel<T, 2>), grid, block, 0, st, a);
  else if (cpl <= 4) hipLaunchKernelGGL((residual_rms_norm_kernel<T, 4>), grid, block, 0, st, a);
  else if (cpl <= 8) hipLaunchKernelGGL((residual_rms_norm_kernel<T, 8>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((residual_rms_norm_kernel<T, 16>), grid, block, 0, st, a);
}

}  // namespace

hipError_t launch_residual_rms_norm(const RmsNormArgs& a, bool bf16, hipStream_t st) {
  if (bf16) launch_t<__bf16>(a, st);
  else launch_t<float>(a, st);
  return hipGetLastError();
}

}  // namespace mi_attn
