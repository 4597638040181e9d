// Fused rotary embedding + paged KV-cache write.
//
// "Fast Attention Kernels and Operator Fusion", §Operator Fusion, counts the
// rotary embedding of queries and keys, and the KV-cache update made while
// keys and values are transformed, among the usual fusion targets: one pass
// reads q, k and v once, rotates q in place and writes the rotated key and
// the value into the token's paged slot.
//
// Rotation (half-split pairs): for i < D/2 the pair (x[i], x[i + D/2]) turns
// by angle pos * base^(-2i/D) (frequencies from the host, in double; the
// angle, its reduction and the rotation by rope_cos_sin and rope_rotate, the
// same code as the decode's fused write).  bf16 outputs are rounded to
// nearest even.
//
// Workgroup = kTok tokens, 512 threads.  A q or k item is four channel pairs
// of one row (8-byte accesses for bf16; consecutive lanes cover consecutive
// chunks of a row).  A value item is four channels of one token; the token
// index runs fastest, so the 16 lanes of a quarter-wave store 16 consecutive
// tokens' elements of one channel row of the token-minor value block: one
// contiguous 32-byte run when the tokens' slots are consecutive, instead of
// 16 isolated 2-byte stores.
//
// The kernel is a chain of memory round trips, and every workgroup of a
// launch is resident at once, so its time is the length of that chain.  It
// has two: the slots and positions, then all of a thread's q, k and v data
// (up to kItems q/k items per thread and pass), loaded while the angles are
// computed.  (The query rotates in place, so the compiler could not move a
// later item's load above an earlier item's store by itself.)

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

constexpr int kTok = 16;
constexpr int kThreads = 512;
constexpr int kItems = 8;   // q/k items held per thread and pass
constexpr int kVItems = 2;  // value items held per thread and pass

template <typename T>
struct Vec4;
// Four elements as loaded (raw: two bf16 pairs or four floats), widened to
// float for the arithmetic only when stored.
template <>
struct Vec4<__bf16> {
  typedef u32x2 raw;
  static __device__ __forceinline__ raw load(const __bf16* p) { return *reinterpret_cast<const u32x2*>(p); }
  static __device__ __forceinline__ f32x4 widen(raw w) {
    return f32x4{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
  }
  static __device__ __forceinline__ void store(__bf16* p, f32x4 v) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
};
template <>
struct Vec4<float> {
  typedef f32x4 raw;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ f32x4 widen(raw v) { return v; }
  static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};

template <int D, typename T>
__global__ __launch_bounds__(kThreads) void rope_write_kernel(const RopeWriteArgs a) {
  constexpr int H2 = D / 2;
  constexpr int CPR = H2 / 4;  // four-pair chunks per row
  __shared__ double theta[H2];
  __shared__ float cs[kTok][H2], sn[kTok][H2];
  __shared__ int32_t slot_sm[kTok], pos_sm[kTok];
  const int n0 = blockIdx.x * kTok;
  const int tid = threadIdx.x;
  const int ntok = min(kTok, a.num_tokens - n0);
  const bool rot = a.rope != 0;

  // round trip 1: slots, positions and frequencies, all in flight at once
  // (unconditional loads from clamped indexes: a load under a lane
  // condition becomes a branch the compiler waits behind)
  const int tt = min(tid, ntok - 1);
  int32_t sl = a.slot_mapping[n0 + tt];
  const int32_t ps = a.positions[n0 + tt];
  const double th = a.freqs.theta[tid & (H2 - 1)];
  if (tid < kTok) {
    if (tid >= ntok || sl >= a.num_blocks * kBlockSize) sl = -1;  // outside the pool: skipped
    slot_sm[tid] = sl;
    pos_sm[tid] = tid < ntok ? ps : 0;
  }
  if (rot && tid < H2) theta[tid] = th;
  __syncthreads();

  T* q = static_cast<T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  T* kc = static_cast<T*>(a.k_cache);
  const T* v = static_cast<const T*>(a.v);
  T* vc = static_cast<T*>(a.v_cache);
  const int rows = a.hq + a.hkv;
  const int total = ntok * rows * CPR;
  const int vtotal = a.hkv * (D / 4) * kTok;

  // one q/k item: source, destination (null: skipped) and rotation index
  struct Item {
    typename Vec4<T>::raw x1, x2;
    T* dst;
    int t, i0;
  };
  auto load_item = [&](int w, Item& it) {
    it.dst = nullptr;
    it.t = 0;
    it.i0 = 0;
    if (w >= total) return;
    const int t = w / (rows * CPR);
    const int rr = (w / CPR) % rows;
    const int i0 = 4 * (w % CPR);
    const int n = n0 + t;
    const bool is_q = rr < a.hq;
    if (is_q && (q == nullptr || !rot)) return;
    const int32_t sl = slot_sm[t];
    if (!is_q && sl < 0) return;
    const T* src = is_q ? q + ((int64_t)n * a.hq + rr) * D : k + ((int64_t)n * a.hkv + (rr - a.hq)) * D;
    it.x1 = Vec4<T>::load(src + i0);
    it.x2 = Vec4<T>::load(src + i0 + H2);
    if (is_q) {
      it.dst = q + ((int64_t)n * a.hq + rr) * D + i0;
    } else {
      const int64_t blk = sl / kBlockSize;
      it.dst = kc + ((blk * a.hkv + (rr - a.hq)) * kBlockSize + sl % kBlockSize) * D + i0;
    }
    it.t = t;
    it.i0 = i0;
  };
  auto store_item = [&](const Item& it) {
    if (it.dst == nullptr) return;
    const f32x4 x1 = Vec4<T>::widen(it.x1), x2 = Vec4<T>::widen(it.x2);
    f32x4 y1 = x1, y2 = x2;
    if (rot) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float r1, r2;
        rope_rotate(x1[e], x2[e], cs[it.t][it.i0 + e], sn[it.t][it.i0 + e], r1, r2);
        y1[e] = r1;
        y2[e] = r2;
      }
    }
    Vec4<T>::store(it.dst, y1);
    Vec4<T>::store(it.dst + H2, y2);
  };
  // one value item: four channels of one token
  struct VItem {
    typename Vec4<T>::raw x;
    T* dst;
  };
  auto load_vitem = [&](int w, VItem& it) {
    it.dst = nullptr;
    if (w >= vtotal) return;
    const int t = w % kTok;
    const int c = (w / kTok) % (D / 4);
    const int g = w / (kTok * (D / 4));
    if (t >= ntok) return;
    const int32_t sl = slot_sm[t];
    if (sl < 0) return;
    it.x = Vec4<T>::load(v + ((int64_t)(n0 + t) * a.hkv + g) * D + 4 * c);
    const int64_t blk = sl / kBlockSize;
    it.dst = vc + ((blk * a.hkv + g) * D + 4 * c) * kBlockSize + sl % kBlockSize;
  };
  auto store_vitem = [&](const VItem& it) {
    if (it.dst == nullptr) return;
    const f32x4 x = Vec4<T>::widen(it.x);
#pragma unroll
    for (int e = 0; e < 4; ++e) it.dst[e * kBlockSize] = static_cast<T>(x[e]);
  };

  // round trip 2: the first pass of data, in flight while the angles are formed
  Item items[kItems];
  VItem vitems[kVItems];
#pragma unroll
  for (int u = 0; u < kItems; ++u) load_item(tid + u * kThreads, items[u]);
#pragma unroll
  for (int u = 0; u < kVItems; ++u) load_vitem(tid + u * kThreads, vitems[u]);
  if (rot) {
    for (int e = tid; e < ntok * H2; e += kThreads) {
      const int t = e / H2, i = e % H2;
      rope_cos_sin(pos_sm[t], theta[i], cs[t][i], sn[t][i]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kItems; ++u) store_item(items[u]);
#pragma unroll
  for (int u = 0; u < kVItems; ++u) store_vitem(vitems[u]);

  // further passes (more heads than one pass holds)
  for (int w0 = tid + kItems * kThreads; w0 < total; w0 += kItems * kThreads) {
#pragma unroll
    for (int u = 0; u < kItems; ++u) load_item(w0 + u * kThreads, items[u]);
#pragma unroll
    for (int u = 0; u < kItems; ++u) store_item(items[u]);
  }
  for (int w0 = tid + kVItems * kThreads; w0 < vtotal; w0 += kVItems * kThreads) {
#pragma unroll
    for (int u = 0; u < kVItems; ++u) load_vitem(w0 + u * kThreads, vitems[u]);
#pragma unroll
    for (int u = 0; u < kVItems; ++u) store_vitem(vitems[u]);
  }
}

}  // namespace

hipError_t launch_rope_write(const RopeWriteArgs& a, int head_dim, bool bf16, hipStream_t s) {
  dim3 grid((a.num_tokens + kTok - 1) / kTok), block(kThreads);
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
