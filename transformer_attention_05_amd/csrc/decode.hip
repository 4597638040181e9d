// Paged decode for gfx950: one query token per sequence against its paged
// KV cache, split into partitions of the context that are merged in the same launch.
//
// "Fast Attention Kernels and Operator Fusion": a decode step brings only a
// query or two per request, so its cost is the read of the ever longer KV
// cache (§FlashAttention-Style Kernels); the kernel goes through the block
// table and never takes K[t+1] to follow K[t] in memory (§Paged Attention
// Kernels).  The
// partition statistics are the running max and sum of the online softmax,
// merged exactly by rescaling each partition with exp(m_p - max m).
//
// Partition kernel: one workgroup of 4 wavefronts per (partition, kv head
// [x 16-head slice], sequence), over a padded grid or a host-built list of
// the real (sequence, partition) items.  Each wavefront takes every fourth 16-token
// block of the partition and keeps two blocks' loads in flight while it
// consumes a third; the block-table entries of the partition come in with one
// lane-parallel load.  Per block:
//   * the K block (16 tokens x D, contiguous per kv head) goes straight into
//     the A operand of v_mfma_f32_16x16x32_bf16 (lane: token l%16, 8
//     channels); the B operand is Q^T of up to 16 query heads of the kv
//     group, so every K/V byte is read once for all heads of the group.  S^T
//     lands as lane = head, 4 consecutive tokens.
//   * value blocks are token-minor ([D][16]), so the A operand of
//     O^T += V^T P^T with v_mfma_f32_16x16x16_bf16 (lane: channel, the same
//     4 tokens) is one 8-byte load, and P passes from the S accumulator to
//     the B operand without any data movement.
// The wavefronts are combined through LDS.  A sequence with a single
// partition writes its output directly; otherwise the (m, l, O) partials go
// to the workspace, and the last workgroup of the sequence's kv slice to
// finish (an arrival counter in the workspace) merges them, so the decode is
// one launch.

#include <mutex>

#include "decode_body.h"

namespace mi_attn {

namespace {

using namespace dc;

// Padded grid (partition, kv slice, sequence): partitions past a sequence's
// context exit at once.
template <int D, bool FUSED>
__global__ __launch_bounds__(64 * DW) void decode_partition_kernel(const DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[decode_lds_bytes<D, DW>()];
  decode_body<D, DW, FUSED>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

template <int D, bool FUSED>
__global__ __launch_bounds__(64 * DW) void decode_planned_kernel(const DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[decode_lds_bytes<D, DW>()];
  planned_body<D, FUSED>(a, blockIdx.x, lds);
}


// ---------------------------------------------------------------------------
// fp32 decode (full-precision parity runs): the same partitions, workspace
// and in-launch merge as the bf16 kernel, on the VALU.  Workgroup = 256
// threads for one (partition, kv head x 16-head slice, sequence); thread
// (h, x) = (tid / 16, tid % 16) forms the score of head h against token x
// of each 16-token block and accumulates output channels x*D/16 .. +D/16-1
// of head h.  The weights of a block pass between the 16 threads of a head
// by lane shuffles.  K and V blocks are staged through LDS, the next
// block's loads in flight while the current one is consumed.  Partitions
// may be any multiple of 16 tokens.
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(const DecodeArgs a) {
  constexpr int DPT = D / 16;        // output channels per thread
  constexpr int KV4 = 16 * D / 4;    // float4 per K (or V) block of one kv head
  constexpr int LPT = KV4 / 256;     // float4 per thread and block, each of K and V
  __shared__ float qs[16][D];
  __shared__ float ks[16][D + 1];
  __shared__ float vs[D][17];
  __shared__ int flag;
  int p, yy, s;
  if (a.plan != nullptr) {
    const int Y = a.hkv * a.head_groups;
    yy = (int)(blockIdx.x % (uint32_t)Y);
    const int it = (int)(blockIdx.x / (uint32_t)Y);
    s = a.plan[2 * it];
    p = a.plan[2 * it + 1];
    if (s < 0 || s >= a.num_seqs || p < 0 || p >= a.max_parts) return;
  } else {
    p = blockIdx.x;
    yy = blockIdx.y;
    s = blockIdx.z;
  }
  const int kvh = yy / a.head_groups;
  const int hgi = yy % a.head_groups;
  const int head0 = kvh * a.group + hgi * 16;
  const int nh = min(16, a.group - hgi * 16);
  const int ctx = min(a.context_lens[s], min(a.max_parts * a.part_size, a.bt_stride * kBlockSize));
  DEBUG_ONLY(debug_check_length(a.context_lens[s], min(a.max_parts * a.part_size, a.bt_stride * kBlockSize)));
  const int nparts = (ctx + a.part_size - 1) / a.part_size;
  if (p >= nparts) return;  // uniform
  const int tok_begin = p * a.part_size;
  const int tok_end = min(ctx, tok_begin + a.part_size);
  const int tid = threadIdx.x;
  const int h = tid >> 4, x = tid & 15;
  const float* q = static_cast<const float*>(a.q);
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const int32_t* bt = a.block_table + (int64_t)s * a.bt_stride;
  for (int e = tid; e < 16 * D; e += 256) {
    const int hh = e / D, d = e % D;
    qs[hh][d] = hh < nh ? q[((int64_t)s * a.hq + head0 + hh) * D + d] : 0.f;
  }
  // this thread's share of a block: float4 e = tid + 256 i of the K block
  // (row e / (D/4)) and of the token-minor V block (channel e / 4, tokens
  // 4 (e % 4) .. +3)
  f32x4 kr[LPT], vr[LPT];
  auto load_block = [&](int blk) {
    const int32_t phys = safe_block(bt[blk], a.num_blocks);
    const int64_t base = ((int64_t)phys * a.hkv + kvh) * (kBlockSize * D);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = tid + 256 * i;
      kr[i] = *reinterpret_cast<const f32x4*>(kc + base + 4 * e);
      vr[i] = *reinterpret_cast<const f32x4*>(vc + base + 4 * e);
    }
  };
  const float c2 = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  float o[DPT];
#pragma unroll
  for (int j = 0; j < DPT; ++j) o[j] = 0.f;
  const int b0 = tok_begin >> 4, b1 = (tok_end + 15) >> 4;
  load_block(b0);
  for (int blk = b0; blk < b1; ++blk) {
    __syncthreads();  // the previous block is consumed
    const int t0 = blk * kBlockSize;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = tid + 256 * i;
      const int row = e / (D / 4), c4 = e % (D / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) ks[row][4 * c4 + j] = kr[i][j];
      const int d = e / 4, tq = 4 * (e % 4);
      // tokens past the partition hold other data or arbitrary bits (0 * NaN
      // is NaN): zero them
#pragma unroll
      for (int j = 0; j < 4; ++j) vs[d][tq + j] = t0 + tq + j < tok_end ? vr[i][j] : 0.f;
    }
    __syncthreads();
    if (blk + 1 < b1) load_block(blk + 1);
    // score of head h against token x (raw units), masked past the partition
    float sc = 0.f;
#pragma unroll 16
    for (int d = 0; d < D; ++d) sc = fmaf(qs[h][d], ks[x][d], sc);
    if (h >= nh || t0 + x >= tok_end) sc = -INFINITY;
    float tmax = sc;
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, m, 16));
    const float m_new = fmaxf(m_run, tmax);
    const float mu = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - mu) * c2);  // 0 while m_run is -inf
    const float pw = __builtin_amdgcn_exp2f((sc - mu) * c2);        // 0 for masked keys
    float psum = pw;
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) psum += __shfl_xor(psum, m, 16);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < DPT; ++j) o[j] *= alpha;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float pt = __shfl(pw, t, 16);
#pragma unroll
      for (int j = 0; j < DPT; ++j) o[j] = fmaf(pt, vs[x * DPT + j][t], o[j]);
    }
  }
  const int64_t row = (int64_t)s * a.hq + head0 + h;
  if (nparts == 1) {
    if (h < nh) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
      for (int j = 0; j < DPT; ++j) static_cast<float*>(a.o)[row * D + x * DPT + j] = o[j] * inv;
    }
    return;
  }
  if (h < nh) {
    const int64_t slot = row * a.max_parts + p;
#pragma unroll
    for (int j = 0; j < DPT; j += 2) store_coherent(a.ws_o + slot * D + x * DPT + j, o[j], o[j + 1]);
    if (x == 0) store_coherent(a.ws_ml + slot * 2, m_run, l_run);
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (!arrive_last(a.counters + (int64_t)s * (a.hkv * a.head_groups) + yy, nparts, &flag)) return;
  merge_partials<D, float>(a, s, head0, nh, nparts, tid, 256);
}

// ---------------------------------------------------------------------------
// Fixed decode scratch for attn_decode_paged_noalloc: the same workspace
// layout (arrival counters, partial outputs, (m, l) pairs) in a device array
// of the library's own, so that a call allocates nothing.  Each GPU holds
// its own copy at its own address, found once per device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) p[i] = uint4{0, 0, 0, 0};
}

}  // namespace

hipError_t decode_scratch(hipStream_t s, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    // the host-side name of the array is not a device address: take the
    // address this device gave it, and use only that from here on
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the arrival counters must start at zero (every completed call leaves
    // them zero again); a fill kernel rather than a memset, so that a first
    // call under graph capture records a plain kernel node
    hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(p),
                       kDecodeScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

template <int D, bool FUSED>
static void launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  if (a.plan != nullptr) {
    const dim3 gp((uint32_t)a.plan_items * (uint32_t)(a.hkv * a.head_groups));
    if (a.plan_items > 0) hipLaunchKernelGGL((decode_planned_kernel<D, FUSED>), gp, dim3(64 * DW), 0, st, a);
    return;
  }
  const dim3 grid(a.max_parts | 1, a.hkv * a.head_groups, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<D, FUSED>), grid, dim3(64 * DW), 0, st, a);
}

hipError_t launch_decode_f32(const DecodeArgs& a, int head_dim, hipStream_t st) {
  dim3 grid;
  if (a.plan != nullptr) {
    if (a.plan_items == 0) return hipSuccess;
    grid = dim3((uint32_t)a.plan_items * (uint32_t)(a.hkv * a.head_groups));
  } else {
    grid = dim3(a.max_parts, a.hkv * a.head_groups, a.num_seqs);
  }
  if (head_dim == 128) hipLaunchKernelGGL(decode_f32_kernel<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(decode_f32_kernel<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool fused, hipStream_t st) {
  if (head_dim == 128) {
    if (fused) launch_decode_t<128, true>(a, st);
    else launch_decode_t<128, false>(a, st);
  } else {
    if (fused) launch_decode_t<64, true>(a, st);
    else launch_decode_t<64, false>(a, st);
  }
  return hipGetLastError();
}

// debug builds: this file's report word (nothing in release builds)
hipError_t debug_take_decode(uint32_t* acc, bool clear) { return debug_take_word(acc, clear); }

}  // namespace mi_attn
