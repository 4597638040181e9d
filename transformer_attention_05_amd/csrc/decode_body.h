// Device code of the bf16 paged decode workgroup: the block registers and
// loads, the partials' merge, decode_body (one workgroup of a partition) and
// planned_body (a workgroup of a planned launch); the method is described at
// the top of decode.hip.  Shared by decode.hip and mixed.hip, each compiling
// its own copy.
#pragma once

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {
namespace {
namespace dc {

typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr float kLazyTau = 8.f;  // keep the reference max until a score exceeds it by 2^8
constexpr int DW = 4;            // wavefronts per partition workgroup

__device__ __forceinline__ f32x4 mfma16k16(v4i16 a, v4i16 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int D>
struct BlockRegs {
  bf16x8 k[D / 32];  // K: token l%16, channels 32c + 8*(l/16) .. +7
  u32x2 v[D / 16];   // V^T: channel 16dt + l%16, tokens 4*(l/16) .. +3
};

template <int D>
__device__ __forceinline__ void load_block(BlockRegs<D>& r, const __bf16* kb, const __bf16* vb) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c) r.k[c] = *reinterpret_cast<const bf16x8*>(kb + 32 * c);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) r.v[dt] = *reinterpret_cast<const u32x2*>(vb + 16 * dt * kBlockSize);
}

// Merge of one sequence's partitions for the query heads head0 .. head0+nh-1:
// O = sum_p f_p O_p / sum_p f_p l_p with f_p = exp(m_p - max m), taken as one
// online pass over batches of MK partitions whose loads are all in flight at
// once (the merge is bound by load latency).  Thread = (head, four channels).
template <int D, typename TO = __bf16>
__device__ __forceinline__ void merge_partials(const DecodeArgs& a, int s, int head0, int nh, int nparts,
                                               int tid, int nthreads) {
  constexpr int CG = D / 4;  // four-channel groups per head
  constexpr int MK = 8;
  const float c2 = a.scale_log2;
  for (int t = tid; t < nh * CG; t += nthreads) {
    const int hl = t / CG, cg = t % CG;
    const int64_t row = (int64_t)s * a.hq + head0 + hl;
    const float* ml = a.ws_ml + row * a.max_parts * 2;
    const float* po = a.ws_o + row * a.max_parts * D + 4 * cg;
    float mx = -INFINITY, lsum = 0.f;
    f32x4 acc = f32x4{};
    for (int p0 = 0; p0 < nparts; p0 += MK) {
      f32x4 ov[MK];
      f32x2 mlv[MK];
#pragma unroll
      for (int k = 0; k < MK; ++k) {
        const int p = p0 + k;
        if (p < nparts) {
          const f32x2 lo = load_coherent(po + (int64_t)p * D), hi = load_coherent(po + (int64_t)p * D + 2);
          ov[k] = f32x4{lo[0], lo[1], hi[0], hi[1]};
          mlv[k] = load_coherent(ml + 2 * p);
        } else {
          ov[k] = f32x4{};
          mlv[k] = f32x2{-INFINITY, 0.f};
        }
      }
      float bm = mlv[0][0];
#pragma unroll
      for (int k = 1; k < MK; ++k) bm = fmaxf(bm, mlv[k][0]);
      const float mn = fmaxf(mx, bm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float f_old = __builtin_amdgcn_exp2f((mx - mu) * c2);  // 0 while mx is -inf
      lsum *= f_old;
      acc *= f_old;
#pragma unroll
      for (int k = 0; k < MK; ++k) {
        const float f = __builtin_amdgcn_exp2f((mlv[k][0] - mu) * c2);  // 0 past nparts (m = -inf)
        acc += f * ov[k];
        lsum = fmaf(f, mlv[k][1], lsum);
      }
      mx = mn;
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if constexpr (sizeof(TO) == 4) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + row * D + 4 * cg) = acc * inv;
    } else {
      *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + row * D + 4 * cg) =
          u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    }
  }
}

// Grid (partition, kv head x head slice, sequence), partitions fastest so a
// long context's partitions start together.  Workgroups are dealt to the 8
// XCDs round-robin in dispatch order; the partition dimension is padded to an
// odd size so that partition p lands on a different XCD for each sequence
// (with a multiple of 8, short contexts would load only a few XCDs).
template <int D, int DWT, bool FUSED>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, const int p, const int yy, const int s, char* lds) {
  const int kvh = yy / a.head_groups;
  const int hgi = yy % a.head_groups;
  const int head0 = kvh * a.group + hgi * 16;
  const int nh = min(16, a.group - hgi * 16);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // token (K operand) / head (Q operand, S and O columns) / channel (V operand)
  const int g4 = lane >> 4;

  // The partition's block-table entries (at most 64 blocks, one per lane)
  // and Q^T do not depend on the context length: they are loaded before it
  // arrives, so the length's round trip overlaps theirs.  Table entries are
  // read up to the partition's end or the row's, whichever comes first.
  const int tok_begin = p * a.part_size;
  const int blk_begin = tok_begin >> 4;
  const int32_t* bt = a.block_table + (int64_t)s * a.bt_stride;
  // (unconditional loads from clamped indexes, selected afterwards: a load
  // under a lane condition becomes a branch the compiler waits behind)
  const int tab_n = min(a.bt_stride - blk_begin, a.part_size >> 4);  // entries readable, <= 0 past the row
  const int tab_ld = bt[blk_begin + min(lane, max(tab_n - 1, 0)) - (tab_n > 0 ? 0 : blk_begin)];
  // Q^T: lane holds head `col`, channels 32c + 8*g4 .. +7
  bf16x8 qreg[D / 32];
  {
    const __bf16* qrow = static_cast<const __bf16*>(a.q) + ((int64_t)s * a.hq + head0 + (col < nh ? col : 0)) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) qreg[c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c + 8 * g4);
  }

  // the grid and the block table bound what a malformed length can reach
  const int ctx = min(a.context_lens[s], min(a.max_parts * a.part_size, a.bt_stride * kBlockSize));
  DEBUG_ONLY(debug_check_length(a.context_lens[s], min(a.max_parts * a.part_size, a.bt_stride * kBlockSize)));
  const int nparts = (ctx + a.part_size - 1) / a.part_size;
  // (a partition past the context leaves after the wait below: a branch
  // here would let the compiler sink the loads above behind the length)

  const int tok_end = min(ctx, tok_begin + a.part_size);
  const int blk_end = (tok_end + 15) >> 4;
  const __bf16* kc = static_cast<const __bf16*>(a.k_cache);
  const __bf16* vc = static_cast<const __bf16*>(a.v_cache);
  const int64_t k_lane = (int64_t)col * D + 8 * g4;          // within a K block of one kv head
  const int64_t v_lane = (int64_t)col * kBlockSize + 4 * g4;  // within a V^T block of one kv head
  // entries past the context: block 0 (the ring's prefetches past the end
  // then all read one block)
  const int tab = (blk_begin + lane < blk_end) ? tab_ld : 0;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    if (col >= nh) qreg[c] = bf16x8{};

  // Block pointers.  Blocks past the partition (prefetched, never consumed)
  // and table entries outside the pool read block 0, so every load is
  // unconditional and in bounds.
  auto block_ptrs = [&](int blk, const __bf16*& kb, const __bf16*& vb) {
    const int idx = min(blk - blk_begin, 63);
    const int32_t phys = safe_block(__builtin_amdgcn_readlane(tab, idx), a.num_blocks);
    const int64_t base = ((int64_t)phys * a.hkv + kvh) * (kBlockSize * D);
    kb = kc + base + k_lane;
    vb = vc + base + v_lane;
  };

  // fused RoPE: this lane's cos and sin for pair index `lane` (D/2 pairs)
  float rc = 1.f, rs = 0.f;
  if constexpr (FUSED) {
    if (a.rope) rope_cos_sin(a.positions[s], a.freqs.theta[lane & (D / 2 - 1)], rc, rs);
  }

  // the table and Q^T must be in registers before the block pipeline starts:
  // waiting here keeps the loop's waits to the blocks themselves
  __builtin_amdgcn_s_waitcnt(0);
  if (p >= nparts) return;

  if constexpr (FUSED) {
    // rotate Q^T: the pair (channel i, i + D/2) sits in qreg[c][e] and
    // qreg[c + D/64][e] of the same lane, i = 32c + 8*g4 + e
    if (a.rope) {
#pragma unroll
      for (int c = 0; c < D / 64; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int src = 32 * c + 8 * g4 + e;
          const float cc = __shfl(rc, src), ss = __shfl(rs, src);
          float y1, y2;
          rope_rotate((float)qreg[c][e], (float)qreg[c + D / 64][e], cc, ss, y1, y2);
          qreg[c][e] = static_cast<__bf16>(y1);
          qreg[c + D / 64][e] = static_cast<__bf16>(y2);
        }
    }
    // The new token (position ctx - 1, in the last partition): the
    // workgroups of that partition write its rotated key and its value into
    // the slot before they read the partition's blocks; the other
    // partitions never read that block.  Wave 0, lane i: pair (i, i + D/2).
    const int32_t slot = a.slot_mapping[s];
    DEBUG_ONLY(debug_check_slot(p == nparts - 1 && tid == 0, slot, a.num_blocks));
    if (p == nparts - 1 && slot >= 0 && slot < a.num_blocks * kBlockSize) {
      if (wave == 0 && lane < D / 2) {
        const int64_t src = ((int64_t)s * a.hkv + kvh) * D;
        const float x1 = (float)static_cast<const __bf16*>(a.k_new)[src + lane];
        const float x2 = (float)static_cast<const __bf16*>(a.k_new)[src + lane + D / 2];
        const __bf16 v1 = static_cast<const __bf16*>(a.v_new)[src + lane];
        const __bf16 v2 = static_cast<const __bf16*>(a.v_new)[src + lane + D / 2];
        float y1 = x1, y2 = x2;
        if (a.rope) rope_rotate(x1, x2, rc, rs, y1, y2);
        const int64_t base = ((int64_t)(slot / kBlockSize) * a.hkv + kvh) * (kBlockSize * D);
        const int off = slot % kBlockSize;
        __bf16* kd = static_cast<__bf16*>(const_cast<void*>(a.k_cache)) + base + off * D;
        __bf16* vd = static_cast<__bf16*>(const_cast<void*>(a.v_cache)) + base + off;
        kd[lane] = static_cast<__bf16>(y1);
        kd[lane + D / 2] = static_cast<__bf16>(y2);
        vd[lane * kBlockSize] = v1;
        vd[(lane + D / 2) * kBlockSize] = v2;
        __builtin_amdgcn_s_waitcnt(0);  // the stores have reached the cache hierarchy
      }
      __syncthreads();
    }
    if (a.q_rot_out != nullptr && p == 0 && col < nh) {
      __bf16* qo = static_cast<__bf16*>(a.q_rot_out) + ((int64_t)s * a.hq + head0 + col) * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) *reinterpret_cast<bf16x8*>(qo + 32 * c + 8 * g4) = qreg[c];
    }
  }

  const float c2 = a.scale_log2;
  const float tau_raw = kLazyTau / c2;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share of the row sum
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{};
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto consume = [&](BlockRegs<D>& r, int blk) {
    // S^T = K Q^T (16 tokens x 16 heads)
    f32x4 sacc = f32x4{};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) sacc = mfma16(r.k[c], qreg[c], sacc);
    // tokens past the partition: masked; past the context the cache holds
    // arbitrary bits (0 * NaN is NaN), so their values are zeroed too
    const int t0 = blk * 16 + 4 * g4;
    if (blk * 16 + 16 > tok_end) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + i >= tok_end) sacc[i] = -INFINITY;
      // this lane's 4 tokens t0 .. t0+3 are two dwords of two bf16 each
      const int nvalid = tok_end - t0;
      const uint32_t keep0 = nvalid >= 2 ? 0xffffffffu : (nvalid == 1 ? 0xffffu : 0u);
      const uint32_t keep1 = nvalid >= 4 ? 0xffffffffu : (nvalid == 3 ? 0xffffu : 0u);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) r.v[dt] = u32x2{r.v[dt][0] & keep0, r.v[dt][1] & keep1};
    }
    float tmax = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    tmax = fmaxf(tmax, xor16(tmax));
    tmax = fmaxf(tmax, xor32(tmax));
    if (__any(tmax > m_run + tau_raw)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY ? 0.f : m_run) * c2;
    bf16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[i], c2, -mc)));
    l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0], pb[1]}, ones, l_run, false);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2], pb[3]}, ones, l_run, false);
    const v4i16 pbi = __builtin_bit_cast(v4i16, pb);
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = mfma16k16(__builtin_bit_cast(v4i16, r.v[dt]), pbi, oacc[dt]);
  };

  // ---- this wavefront's blocks: blk_begin + wave, + DWT, ...; three register
  // buffers keep two blocks in flight while one is consumed
  // (the scheduling barriers pin the issue order of the load groups, which
  // the wait counters rely on: loads retire in issue order)
  BlockRegs<D> r0, r1, r2;
  const __bf16 *kb, *vb;
  const int first = blk_begin + wave;
  block_ptrs(first, kb, vb);
  load_block<D>(r0, kb, vb);
  __builtin_amdgcn_sched_barrier(0);
  block_ptrs(first + DWT, kb, vb);
  load_block<D>(r1, kb, vb);
  __builtin_amdgcn_sched_barrier(0);
  for (int blk = first; blk < blk_end; blk += 3 * DWT) {
    block_ptrs(blk + 2 * DWT, kb, vb);
    load_block<D>(r2, kb, vb);
    __builtin_amdgcn_sched_barrier(0);
    consume(r0, blk);
    if (blk + DWT >= blk_end) break;
    block_ptrs(blk + 3 * DWT, kb, vb);
    load_block<D>(r0, kb, vb);
    __builtin_amdgcn_sched_barrier(0);
    consume(r1, blk + DWT);
    if (blk + 2 * DWT >= blk_end) break;
    block_ptrs(blk + 4 * DWT, kb, vb);
    load_block<D>(r1, kb, vb);
    __builtin_amdgcn_sched_barrier(0);
    consume(r2, blk + 2 * DWT);
  }

  // ---- combine the wavefronts (lane holds head `col`, channels 16dt + 4*g4 .. +3)
  float (*sm_m)[16] = reinterpret_cast<float (*)[16]>(lds);
  float (*sm_l)[16] = reinterpret_cast<float (*)[16]>(lds + DWT * 16 * 4);
  f32x4 (*sm_o)[D / 16][4][17] = reinterpret_cast<f32x4 (*)[D / 16][4][17]>(lds + DWT * 16 * 8);
  float l_all = l_run + xor16(l_run);
  l_all += xor32(l_all);
  if (g4 == 0) {
    sm_m[wave][col] = m_run;
    sm_l[wave][col] = l_all;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) sm_o[wave][dt][g4][col] = oacc[dt];
  __syncthreads();

  // thread = (head, 4 channels)
  const bool single = nparts == 1;
  for (int t = tid; t < nh * (D / 4); t += 64 * DWT) {
    const int hl = t / (D / 4), d4 = t % (D / 4);
    const int dt = d4 >> 2, gg = d4 & 3;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < DWT; ++w) mx = fmaxf(mx, sm_m[w][hl]);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float lsum = 0.f;
    f32x4 osum = f32x4{};
#pragma unroll
    for (int w = 0; w < DWT; ++w) {
      const float f = __builtin_amdgcn_exp2f((sm_m[w][hl] - mu) * c2);
      lsum = fmaf(f, sm_l[w][hl], lsum);
      osum += f * sm_o[w][dt][gg][hl];
    }
    const int64_t row = (int64_t)s * a.hq + head0 + hl;
    if (single) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const u32x2 w2 = {pack_bf16x2(osum[0] * inv, osum[1] * inv), pack_bf16x2(osum[2] * inv, osum[3] * inv)};
      *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + row * D + 4 * d4) = w2;
    } else {
      const int64_t slot = row * a.max_parts + p;
      store_coherent(a.ws_o + slot * D + 4 * d4, osum[0], osum[1]);
      store_coherent(a.ws_o + slot * D + 4 * d4 + 2, osum[2], osum[3]);
      if (d4 == 0) store_coherent(a.ws_ml + slot * 2, mx, lsum);
    }
  }
  if (single) return;

  // ---- arrival: every partial store of the workgroup has completed before
  // the count; the workgroup that brings the count to nparts merges, then
  // restores the counter to its value before the call (zero), for the next
  // call
  __builtin_amdgcn_s_waitcnt(0);
  // (the barrier in arrive_last also ends the combine's LDS reads)
  if (!arrive_last(a.counters + (int64_t)s * (a.hkv * a.head_groups) + yy, nparts, reinterpret_cast<int*>(lds)))
    return;
  merge_partials<D>(a, s, head0, nh, nparts, tid, 64 * DWT);
}

// LDS of a DWT-wavefront workgroup's combine: per wave 16 maxima, 16 sums and
// a padded (dt, g4, head) block of partial outputs
template <int D, int DWT>
constexpr int decode_lds_bytes() { return DWT * 16 * 8 + DWT * (D / 16) * 4 * 17 * 16; }

// Planned grid: workgroup = (item, kv slice), item = (sequence, partition)
// from a list built on the host (attn_decode_paged_plan), longest sequences
// first.  Only real partitions are dispatched: the padded grid's empty
// workgroups (most of it for a batch of mixed lengths) each take a CU slot
// on their way out.  Entries out of range are skipped.
// Workgroup `bid` of a planned launch, its combine LDS at `lds`
// (decode_lds_bytes<D, DW>() bytes).
template <int D, bool FUSED>
__device__ __attribute__((always_inline)) inline void planned_body(const DecodeArgs& a, const uint32_t bid, char* lds) {
  const int Y = a.hkv * a.head_groups;
  const int yy = (int)(bid % (uint32_t)Y);
  const int it = (int)(bid / (uint32_t)Y);
  const int s = a.plan[2 * it], p = a.plan[2 * it + 1];
  if (s < 0 || s >= a.num_seqs || p < 0 || p >= a.max_parts) return;
  decode_body<D, DW, FUSED>(a, p, yy, s, lds);
}

}  // namespace dc
}  // namespace
}  // namespace mi_attn
