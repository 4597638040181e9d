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
// Workgroup = 512 threads over TOK tokens (16 at D 128, 32 at D 64).  A
// thread owns one (token, chunk) of the rotation: chunk c is the four pairs
// 4c .. 4c+3, i.e. channels 4c .. 4c+3 and 4c + D/2 .. +3 of a row, and the
// thread takes that chunk of every other query/key row of its token (two
// threads per chunk, rows of alternating parity).  The two threads of a
// chunk (neighbouring lanes) form two of its four (cos, sin) values each and
// swap them by a lane shuffle: no table in LDS, no barrier.  A value item is four channels of one
// token; the token index runs fastest, so the 16 lanes of a quarter-wave
// store 16 consecutive tokens' elements of one channel row of the
// token-minor value block (one contiguous 32-byte run when the slots are
// consecutive).
//
// Every workgroup of a launch is resident at once, so the kernel takes as
// long as one thread's chain of memory round trips.  There is one: the
// position, slot, frequencies and all of a thread's q, k and v data are
// loaded together (unconditional loads from clamped indexes), then the
// angles are formed, the rows rotated and everything stored.

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

constexpr int kThreads = 512;
constexpr int kRowsPerPass = 8;  // q/k rows held per thread and pass
constexpr int kVItems = 2;       // value items held per thread and pass

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
  static __device__ __forceinline__ void store_raw(__bf16* p, raw w) { *reinterpret_cast<u32x2*>(p) = w; }
};
template <>
struct Vec4<float> {
  typedef f32x4 raw;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ f32x4 widen(raw v) { return v; }
  static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
  static __device__ __forceinline__ void store_raw(float* p, raw v) { *reinterpret_cast<f32x4*>(p) = v; }
};

template <int D, typename T>
__global__ __launch_bounds__(kThreads) void rope_write_kernel(const RopeWriteArgs a) {
  constexpr int H2 = D / 2;
  constexpr int CPR = H2 / 4;         // four-pair chunks per row
  constexpr int TPT = 2 * CPR;        // threads per token
  constexpr int TOK = kThreads / TPT;  // tokens per workgroup
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * TOK;
  const int last = a.num_tokens - 1;
  const bool rot = a.rope != 0;

  // ---- the rotation part: token t, chunk c, row parity h
  const int t = tid / TPT;
  const int c = (tid / 2) % CPR;
  const int h = tid & 1;
  const int n = min(n0 + t, last);       // clamped: loads stay in range
  const bool live = n0 + t <= last;
  // rows 0 .. hq-1 are the query heads (rotated in place), hq .. hq+hkv-1
  // the key heads (rotated into the cache); without rotation or without q
  // only the keys are copied
  const int rlo = (a.q != nullptr && rot) ? 0 : a.hq;
  const int rows = a.hq + a.hkv;
  const int32_t pos = a.positions[n];
  int32_t slot = a.slot_mapping[n];
  // this thread forms the angles of pairs 4c + 2h and 4c + 2h + 1; the
  // other thread of the chunk (lane ^ 1) forms the other two
  const double th0 = a.freqs.theta[4 * c + 2 * h], th1 = a.freqs.theta[4 * c + 2 * h + 1];
  T* q = static_cast<T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  T* kc = static_cast<T*>(a.k_cache);
  const T* v = static_cast<const T*>(a.v);
  T* vc = static_cast<T*>(a.v_cache);

  // value items of this pass: token tv (fastest), kv head gv, channels 4 dv ..
  const int vtotal = TOK * a.hkv * (D / 4);
  auto v_item = [&](int w, int& tv, int& gv, int& dv) {
    tv = w % TOK;
    dv = (w / TOK) % (D / 4);
    gv = w / (TOK * (D / 4));
  };

  for (int r0 = rlo + h; r0 < rows || r0 == rlo + h; r0 += 2 * kRowsPerPass) {
    // loads of this pass: q/k chunks of up to kRowsPerPass rows (row index
    // clamped into range, the store decides), and, in the first pass, the
    // value items
    typename Vec4<T>::raw x1[kRowsPerPass], x2[kRowsPerPass];
#pragma unroll
    for (int u = 0; u < kRowsPerPass; ++u) {
      const int r = min(r0 + 2 * u, rows - 1);
      const T* src = r < a.hq ? q + ((int64_t)n * a.hq + r) * D : k + ((int64_t)n * a.hkv + (r - a.hq)) * D;
      x1[u] = Vec4<T>::load(src + 4 * c);
      x2[u] = Vec4<T>::load(src + 4 * c + H2);
    }
    const bool first = r0 == rlo + h;
    typename Vec4<T>::raw vx[kVItems];
    int32_t vslot[kVItems];
    if (first) {
#pragma unroll
      for (int u = 0; u < kVItems; ++u) {
        int tv, gv, dv;
        v_item(min(tid + u * kThreads, vtotal - 1), tv, gv, dv);
        const int nv = min(n0 + tv, last);
        vslot[u] = a.slot_mapping[nv];
        vx[u] = Vec4<T>::load(v + ((int64_t)nv * a.hkv + gv) * D + 4 * dv);
      }
    }
    // angles of the chunk's four pairs (formed while the data arrives): two
    // here, two from the neighbouring lane
    float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
    if (rot) {
      float c0, s0, c1, s1;
      rope_cos_sin(pos, th0, c0, s0);
      rope_cos_sin(pos, th1, c1, s1);
      const float d0 = __shfl_xor(c0, 1), e0 = __shfl_xor(s0, 1), d1 = __shfl_xor(c1, 1), e1 = __shfl_xor(s1, 1);
      // (selects, not an index by h: a lane-dependent index would move the
      // arrays to memory)
      cs[0] = h ? d0 : c0; sn[0] = h ? e0 : s0;
      cs[1] = h ? d1 : c1; sn[1] = h ? e1 : s1;
      cs[2] = h ? c0 : d0; sn[2] = h ? s0 : e0;
      cs[3] = h ? c1 : d1; sn[3] = h ? s1 : e1;
    }
    DEBUG_ONLY(debug_check_slot(first && live && c == 0 && h == 0, slot, a.num_blocks));
    if (slot >= a.num_blocks * kBlockSize) slot = -1;  // outside the pool: skipped
#pragma unroll
    for (int u = 0; u < kRowsPerPass; ++u) {
      const int r = r0 + 2 * u;
      if (!live || r >= rows) continue;
      T* dst;
      if (r < a.hq) {
        dst = q + ((int64_t)n * a.hq + r) * D + 4 * c;
      } else {
        if (slot < 0) continue;
        dst = kc + (((int64_t)(slot / kBlockSize) * a.hkv + (r - a.hq)) * kBlockSize + slot % kBlockSize) * D + 4 * c;
      }
      if (rot) {
        const f32x4 y1 = Vec4<T>::widen(x1[u]), y2 = Vec4<T>::widen(x2[u]);
        f32x4 z1, z2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float o1, o2;
          rope_rotate(y1[e], y2[e], cs[e], sn[e], o1, o2);
          z1[e] = o1;
          z2[e] = o2;
        }
        Vec4<T>::store(dst, z1);
        Vec4<T>::store(dst + H2, z2);
      } else {
        Vec4<T>::store_raw(dst, x1[u]);
        Vec4<T>::store_raw(dst + H2, x2[u]);
      }
    }
    if (first) {
#pragma unroll
      for (int u = 0; u < kVItems; ++u) {
        const int w = tid + u * kThreads;
        int tv, gv, dv;
        v_item(w, tv, gv, dv);
        const int32_t sl = vslot[u];
        if (w >= vtotal || n0 + tv > last || sl < 0 || sl >= a.num_blocks * kBlockSize) continue;
        const f32x4 x = Vec4<T>::widen(vx[u]);
        T* dst = vc + ((int64_t)(sl / kBlockSize) * a.hkv + gv) * D * kBlockSize + (4 * dv) * kBlockSize + sl % kBlockSize;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e * kBlockSize] = static_cast<T>(x[e]);
      }
      // further value passes (more kv heads than one pass holds)
      for (int w0 = tid + kVItems * kThreads; w0 < vtotal; w0 += kThreads) {
        int tv, gv, dv;
        v_item(w0, tv, gv, dv);
        const int nv = n0 + tv;
        if (nv > last) continue;
        const int32_t sl = a.slot_mapping[nv];
        if (sl < 0 || sl >= a.num_blocks * kBlockSize) continue;
        const f32x4 x = Vec4<T>::widen(Vec4<T>::load(v + ((int64_t)nv * a.hkv + gv) * D + 4 * dv));
        T* dst = vc + ((int64_t)(sl / kBlockSize) * a.hkv + gv) * D * kBlockSize + (4 * dv) * kBlockSize + sl % kBlockSize;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e * kBlockSize] = static_cast<T>(x[e]);
      }
    }
    if (r0 + 2 * kRowsPerPass >= rows) break;
  }
}

}  // namespace

hipError_t launch_rope_write(const RopeWriteArgs& a, int head_dim, bool bf16, hipStream_t s) {
  const int tok = kThreads / (head_dim / 4);  // tokens per workgroup (16 at D 128, 32 at D 64)
  dim3 grid((a.num_tokens + tok - 1) / tok), block(kThreads);
  if (bf16) {
    if (head_dim == 128) hipLaunchKernelGGL((rope_write_kernel<128, __bf16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((rope_write_kernel<64, __bf16>), grid, block, 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((rope_write_kernel<128, float>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((rope_write_kernel<64, float>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// debug builds: this file's report word (nothing in release builds)
hipError_t debug_take_rope_write(uint32_t* acc, bool clear) { return debug_take_word(acc, clear); }

}  // namespace mi_attn
