// Paged decode for gfx950: one query token per sequence against its paged
// KV cache, split into partitions of the context plus a merge pass.
//
// "Fast Attention Kernels and Operator Fusion": decode has one or a few new
// queries per request and is dominated by reading the growing KV cache
// (§FlashAttention-Style Kernels); the kernel follows the block table and
// cannot assume K[t+1] sits next to K[t] (§Paged Attention Kernels).  The
// partition statistics are the running max and sum of the online softmax,
// merged exactly by rescaling each partition with exp(m_p - max m).
//
// Partition kernel, workgroup = (partition, kv head [x 16-head slice], seq),
// 4 wavefronts.  Each wavefront takes pairs of 16-token blocks:
//   * K block (16 tokens x D, one contiguous 4 KiB run per kv head at D=128)
//     is loaded straight into the A operand of v_mfma_f32_16x16x32_bf16:
//     lane l reads token l%16, 8 channels.  The B operand is Q^T of up to 16
//     query heads of the kv group (GQA: every K/V byte is read once per kv
//     head, for all its query heads).  S^T lands as lane = head, 4 tokens.
//   * V blocks are stored token-minor ([D][16]), so the A operand of
//     O^T += V^T P^T (lane = channel, 4 consecutive tokens from each block of
//     the pair) is two 8-byte loads, and P goes from the S accumulator to the
//     B operand without leaving registers.
//   * the four wavefronts are combined through LDS; a sequence with a single
//     partition writes its output directly, otherwise (m, l, O) partials go
//     to the workspace for the merge kernel.

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

constexpr int DW = 4;  // wavefronts per workgroup

template <int D>
__global__ __launch_bounds__(DW * 64) void decode_partition_kernel(const DecodeArgs a) {
  const int p = blockIdx.x;
  const int s = blockIdx.z;
  // the grid and the block table bound what a malformed length can reach
  const int ctx = min(a.context_lens[s], min(a.max_parts * a.part_size, a.bt_stride * kBlockSize));
  const int nparts = (ctx + a.part_size - 1) / a.part_size;
  if (p >= nparts) return;

  const int kvh = blockIdx.y / a.head_groups;
  const int hgi = blockIdx.y % a.head_groups;
  const int head0 = kvh * a.group + hgi * 16;
  const int nh = min(16, a.group - hgi * 16);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;  // token (K operand) / head (Q operand, S and O columns)
  const int g4 = lane >> 4;   // 8-element contraction group

  const int tok_begin = p * a.part_size;
  const int tok_end = min(ctx, tok_begin + a.part_size);
  const int blk_begin = tok_begin >> 4;
  const int blk_end = (tok_end + 15) >> 4;
  const int32_t* bt = a.block_table + (int64_t)s * a.bt_stride;

  const __bf16* kc = static_cast<const __bf16*>(a.k_cache);
  const __bf16* vc = static_cast<const __bf16*>(a.v_cache);

  // Q^T: lane holds head `col`, channels 32c + 8*g4 .. +7
  bf16x8 qreg[D / 32];
  {
    const __bf16* qrow = static_cast<const __bf16*>(a.q) + ((int64_t)s * a.hq + head0 + col) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      qreg[c] = col < nh ? *reinterpret_cast<const bf16x8*>(qrow + 32 * c + 8 * g4) : bf16x8{};
  }

  const float c2 = a.scale_log2;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share of the row sum
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{};

  for (int blk = blk_begin + 2 * wave; blk < blk_end; blk += 2 * DW) {
    int32_t phys[2];
    bool valid[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      valid[i] = blk + i < blk_end;
      phys[i] = valid[i] ? bt[blk + i] : 0;
      if (phys[i] < 0 || phys[i] >= a.num_blocks) valid[i] = false;  // corrupt table: read zeros
    }
    // ---- loads
    bf16x8 kreg[2][D / 32];
    u32x2 vreg[2][D / 16];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const __bf16* kb = kc + (((int64_t)phys[i] * a.hkv + kvh) * kBlockSize + col) * D + 8 * g4;
      const __bf16* vb = vc + (((int64_t)phys[i] * a.hkv + kvh) * D + col) * kBlockSize + 4 * g4;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        kreg[i][c] = valid[i] ? *reinterpret_cast<const bf16x8*>(kb + 32 * c) : bf16x8{};
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        vreg[i][dt] = valid[i] ? *reinterpret_cast<const u32x2*>(vb + (int64_t)16 * dt * kBlockSize) : u32x2{0, 0};
    }
    // ---- S^T = K Q^T, one 16x16 tile per block
    f32x4 sacc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sacc[i] = f32x4{};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) sacc[i] = mfma16(kreg[i][c], qreg[c], sacc[i]);
    }
    // ---- mask tokens past the partition; zero their V (past the context the
    // cache holds arbitrary bits, and 0 * NaN would poison the sum)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t0 = (blk + i) * 16 + 4 * g4;
      if (t0 + 3 >= tok_end) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + r >= tok_end) sacc[i][r] = -INFINITY;
        const int nvalid = tok_end - t0;  // 4-token run of this lane
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          u32x2 w = vreg[i][dt];
          if (nvalid <= 0) w = u32x2{0, 0};
          else if (nvalid == 1) w = u32x2{w[0] & 0xffffu, 0};
          else if (nvalid == 2) w = u32x2{w[0], 0};
          else if (nvalid == 3) w = u32x2{w[0], w[1] & 0xffffu};
          vreg[i][dt] = w;
        }
      }
    }
    // ---- online softmax over the 32 tokens of the pair (per head = column)
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sacc[i][r]);
    tmax = fmaxf(tmax, xor16(tmax));
    tmax = fmaxf(tmax, xor32(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
    const float mc = m_use * c2;
    bf16x8 pb;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const __bf16 pv = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[i][r], c2, -mc)));
        pb[4 * i + r] = pv;
        lsum += static_cast<float>(pv);
      }
    l_run = fmaf(l_run, alpha, lsum);
    m_run = m_new;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x4 w = {vreg[0][dt][0], vreg[0][dt][1], vreg[1][dt][0], vreg[1][dt][1]};
      oacc[dt] = mfma16(__builtin_bit_cast(bf16x8, w), pb, oacc[dt] * alpha);
    }
  }

  // ---- combine the wavefronts
  __shared__ float sm_m[DW][16];
  __shared__ float sm_l[DW][16];
  __shared__ float sm_o[DW][D][17];
  float l_all = l_run + xor16(l_run);
  l_all += xor32(l_all);
  if (g4 == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_all;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wave][16 * dt + 4 * g4 + r][col] = oacc[dt][r];
  __syncthreads();

  const bool single = nparts == 1;
  for (int idx = tid; idx < nh * D; idx += DW * 64) {
    const int hl = idx / D, d = idx % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < DW; ++w) mx = fmaxf(mx, sm_m[w][hl]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      const float f = __builtin_amdgcn_exp2f((sm_m[w][hl] - mu) * c2);
      lsum = fmaf(f, sm_l[w][hl], lsum);
      osum = fmaf(f, sm_o[w][d][hl], osum);
    }
    const int64_t row = (int64_t)s * a.hq + head0 + hl;
    if (single) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      static_cast<__bf16*>(a.o)[row * D + d] = static_cast<__bf16>(osum * inv);
    } else {
      const int64_t slot = row * a.max_parts + p;
      a.ws_o[slot * D + d] = osum;
      if (d == 0) {
        a.ws_ml[slot * 2 + 0] = mx;
        a.ws_ml[slot * 2 + 1] = lsum;
      }
    }
  }
}

// Merge kernel: workgroup = (query head, seq); O = sum_p f_p O_p / sum_p f_p l_p
// with f_p = exp(m_p - max m).
template <int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(const DecodeArgs a) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int ctx = min(a.context_lens[s], min(a.max_parts * a.part_size, a.bt_stride * kBlockSize));
  const int nparts = (ctx + a.part_size - 1) / a.part_size;
  if (nparts <= 1) return;
  extern __shared__ float sm_w[];  // [max_parts]
  __shared__ float sm_red[128];
  __shared__ float sm_scalar[2];
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)s * a.hq + h;
  const float* ml = a.ws_ml + row * a.max_parts * 2;
  const float c2 = a.scale_log2;

  float mx = -INFINITY;
  for (int i = tid; i < nparts; i += 128) mx = fmaxf(mx, ml[2 * i]);
  sm_red[tid] = mx;
  __syncthreads();
  for (int w = 64; w > 0; w >>= 1) {
    if (tid < w) sm_red[tid] = fmaxf(sm_red[tid], sm_red[tid + w]);
    __syncthreads();
  }
  mx = sm_red[0];
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  __syncthreads();
  float lsum = 0.f;
  for (int i = tid; i < nparts; i += 128) {
    const float f = __builtin_amdgcn_exp2f((ml[2 * i] - mu) * c2);
    sm_w[i] = f;
    lsum = fmaf(f, ml[2 * i + 1], lsum);
  }
  sm_red[tid] = lsum;
  __syncthreads();
  for (int w = 64; w > 0; w >>= 1) {
    if (tid < w) sm_red[tid] += sm_red[tid + w];
    __syncthreads();
  }
  if (tid == 0) sm_scalar[0] = sm_red[0] > 0.f ? 1.f / sm_red[0] : 0.f;
  __syncthreads();
  const float inv = sm_scalar[0];
  const float* po = a.ws_o + row * a.max_parts * D;
  for (int d = tid; d < D; d += 128) {
    float acc = 0.f;
    for (int i = 0; i < nparts; ++i) acc = fmaf(sm_w[i], po[(int64_t)i * D + d], acc);
    static_cast<__bf16*>(a.o)[row * D + d] = static_cast<__bf16>(acc * inv);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, hipStream_t st) {
  dim3 grid1(a.max_parts, a.hkv * a.head_groups, a.num_seqs);
  dim3 grid2(a.hq, a.num_seqs);
  const size_t merge_smem = sizeof(float) * (size_t)a.max_parts;
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_partition_kernel<128>, grid1, dim3(DW * 64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.max_parts > 1) hipLaunchKernelGGL(decode_merge_kernel<128>, grid2, dim3(128), merge_smem, st, a);
  } else {
    hipLaunchKernelGGL(decode_partition_kernel<64>, grid1, dim3(DW * 64), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.max_parts > 1) hipLaunchKernelGGL(decode_merge_kernel<64>, grid2, dim3(128), merge_smem, st, a);
  }
  return hipGetLastError();
}

}  // namespace mi_attn
