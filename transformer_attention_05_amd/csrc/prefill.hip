// Prefill attention for gfx950: O = softmax(Q K^T * scale + M) V computed
// tile by tile with an online softmax, as "Fast Attention Kernels and
// Operator Fusion" (§FlashAttention-Style Kernels) describes FlashAttention:
// a workgroup owns a tile of queries and walks the key/value tiles; per tile
// it forms the scores, folds them into the running row max and row sum, and
// adds their share to the output kept on chip.  The Tq x Tk score matrix
// never reaches HBM.
//
// bf16 path (both contractions on MFMA, fp32 accumulate):
//   * workgroup = HPW query heads of one kv group x WPH wavefronts; each
//     wavefront owns 32 queries of one head, and every K/V tile in LDS
//     serves all HPW heads.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q^T stays in registers
//     for the whole kernel, K comes from LDS.  In the S^T accumulator a lane
//     holds one query (lane % 32) and 16 of the 32 keys of the subtile, so the
//     row max and sum need only one cross-lane step (lane ^ 32).
//   * O^T += V^T P^T with the same instruction: P leaves the S accumulator as
//     the B operand without touching LDS.  The order of the 16 keys of each
//     contraction step is permuted to match the accumulator layout, and the
//     V^T operand is read from a transposed LDS copy of the V tile in the same
//     permuted order.  Each lane owns one query of O^T, so the rescale by
//     exp(m_old - m_new) is lane-local.
//   * software pipeline: the MFMAs of S(j+1) run interleaved with the
//     exponentials of S(j), the PV MFMAs of tile j with the row max of S(j+1);
//     the running-max update for S(j+1) waits until the MFMAs of S(j+2) are
//     issued.  The exponent of each score, s * scale * log2 e - m, is formed
//     in place in the PV phase, whose VALU is otherwise nearly idle; when the
//     max update moves m, it shifts those exponents by the change.
//   * K/V tiles of 64 keys cycle through LDS rings fed by global->LDS DMA one
//     or two iterations ahead.  With 4 wavefronts a workgroup needs 80 KiB,
//     so two workgroups share a CU and overlap each other's phases.  When
//     every key tile is whole (contiguous, unmasked, D 128), an iteration's
//     DMAs are issued inside its two phases rather than at its top.  The
//     workgroup start waits only for Q and the first K tile.
//   * causal tiles wholly above the diagonal are never loaded; masking runs
//     only on tiles that cross the diagonal or the sequence end.
//   * workgroups are ordered heaviest first (last query tile first).  The
//     hardware deals workgroup ids round-robin over the 8 XCDs, so every XCD
//     receives an equal share of heavy and light tiles; workgroups that start
//     together walk the same key tiles, so K/V is still shared in each L2.
//   * P is rounded to bf16 for the PV MFMA and the row sum l accumulates the
//     same rounded values (v_dot2 in the PV phase, whose VALU is otherwise
//     idle), so the output weights stay exactly normalised.
// The paged variant is the same loop with K/V rows gathered through the
// block table (16-token blocks): token t of sequence s lives in block
// block_table[s][t / 16] at offset t % 16.  Its V^T tile stays block-major
// in LDS (the four token-minor value blocks as stored), so each V DMA and
// each 16-key contraction step touches one block.
//
// f32 path: a plain VALU kernel (one query per one or two lanes), used for
// full-precision parity runs.

#include "prefill_body.h"

namespace mi_attn {

namespace {

using namespace pf;

template <int D, bool PAGED, int HPW, int WPH, bool MASKED = false, bool DEEP_V = false, bool SPREAD = false>
__global__ __launch_bounds__(64 * HPW * WPH) __attribute__((amdgpu_waves_per_eu(MASKED ? 1 : 2)))
void prefill_bf16_kernel(const PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) __bf16 sm[lds_elems<D, HPW, WPH, MASKED, DEEP_V>()];
  bf16_body<D, PAGED, HPW, WPH, MASKED, DEEP_V, SPREAD>(a, blockIdx.x, sm);
}

// ---------------------------------------------------------------------------
// Merge of the split-KV partials of one query tile (the same geometry as the
// attention kernel): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with
// M = max_s m_s, the exact recombination of softmax statistics, taken here
// as one online pass over the shares (their loads do not depend on each
// other).  Thread = (head, query row, four channels); a query tile's items
// are spread over MERGE_PARTS workgroups of 256 threads.
template <int D, int HPW, int WPH>
constexpr int merge_parts() { return HPW * 32 * WPH * (D / 4) / 256; }

template <int D, bool PAGED, int HPW, int WPH>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillArgs a) {
  constexpr int BM = 32 * WPH;
  constexpr int PARTS = merge_parts<D, HPW, WPH>();
  const uint32_t id = blockIdx.x / PARTS;
  const int it = (int)(blockIdx.x % PARTS) * 256 + (int)threadIdx.x;
  const int hgroups = a.hq / HPW;
  const uint32_t per_tile = (uint32_t)hgroups * (uint32_t)a.batch;
  const int mt = a.num_m_tiles - 1 - (int)(id / per_tile);
  const uint32_t rem = id % per_tile;
  const int b = (int)(rem / hgroups);
  const int h0 = (int)(rem % hgroups) * HPW;
  int32_t tq, tk;
  int64_t q_row0 = 0;
  if constexpr (PAGED) {
    const int32_t c0 = a.cu_seqlens_q[b];
    tq = max(0, min(a.cu_seqlens_q[b + 1], a.total_q) - max(c0, 0));
    tk = min(a.context_lens[b], a.bt_stride * kBlockSize);
    q_row0 = max(c0, 0);
  } else {
    tq = a.tq;
    tk = a.tk;
  }
  const int m0 = mt * BM;
  if (m0 >= tq) return;
  int n_all = (tk + BN - 1) / BN;
  if (a.causal) {
    const int q_hi = min(m0 + BM, tq) - 1;
    const int kmax = min(tk - 1, q_hi + tk - tq);
    n_all = kmax < 0 ? 0 : kmax / BN + 1;
  }
  const int L = split_len(n_all, a);
  const int nsplit = max(1, (n_all + L - 1) / L);
  if (nsplit <= 1) return;  // that query tile wrote its output itself
  const int hl = it / (BM * (D / 4));
  const int r = (it / (D / 4)) % BM;
  const int d0 = 4 * (it % (D / 4));
  const int qi = m0 + r;
  if (qi >= tq) return;
  const int h = h0 + hl;
  const int64_t row = PAGED ? (q_row0 + qi) * a.hq + h : ((int64_t)b * tq + qi) * a.hq + h;
  float mx = -INFINITY, lsum = 0.f;
  f32x4 acc = f32x4{};
#pragma unroll 4
  for (int sp = 0; sp < nsplit; ++sp) {
    const int64_t slot = (int64_t)sp * a.ws_rows + row;
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ws_ml + slot * 2);
    const f32x4 ov = *reinterpret_cast<const f32x4*>(a.ws_o + slot * D + d0);
    const float mn = fmaxf(mx, ml[0]);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float f_old = __builtin_amdgcn_exp2f(mx - mu);    // 0 while mx is -inf
    const float f_new = __builtin_amdgcn_exp2f(ml[0] - mu);
    lsum = lsum * f_old + f_new * ml[1];
    acc = acc * f_old + f_new * ov;
    mx = mn;
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  __bf16* op = static_cast<__bf16*>(a.o);
  __bf16* orow = PAGED ? op + ((q_row0 + qi) * a.hq + h) * D : op + b * a.os_b + (int64_t)qi * a.os_t + h * a.os_h;
  *reinterpret_cast<u32x2*>(orow + d0) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                               pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (!PAGED && a.lse != nullptr && d0 == 0)
    a.lse[((int64_t)b * a.hq + h) * tq + qi] = lsum > 0.f ? (mx + __log2f(lsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// f32 VALU kernel: LPQ = D / 64 lanes per query, each holding 64 channels.
// PAGED: packed queries (cu_seqlens_q) over keys and values gathered
// through the block table (K blocks token-major, V blocks token-minor).
template <int D, bool PAGED>
__global__ __launch_bounds__(64 * (D / 64)) void prefill_f32_kernel(const PrefillArgs a) {
  constexpr int LPQ = D / 64;
  constexpr int TN = 32;  // keys per tile
  constexpr int QM = kPrefillF32BlockM;
  __shared__ float ks[TN][D];
  __shared__ float vs[TN][D];

  const uint32_t per_tile = (uint32_t)a.hq * (uint32_t)a.batch;
  const uint32_t id = blockIdx.x;
  const int mt = a.num_m_tiles - 1 - (int)(id / per_tile);
  const uint32_t rem = id % per_tile;
  const int b = (int)(rem / a.hq);
  const int h = (int)(rem % a.hq);
  const int g = h / a.group;
  int tq, tk;
  int64_t q_row0 = 0;
  const int32_t* bt_row = nullptr;
  if constexpr (PAGED) {
    const int32_t c0 = a.cu_seqlens_q[b];
    // a malformed cu_seqlens / context_lens can shrink the work, never widen
    // the memory it touches
    tq = max(0, min(a.cu_seqlens_q[b + 1], a.total_q) - max(c0, 0));
    tk = min(a.context_lens[b], a.bt_stride * kBlockSize);
    q_row0 = max(c0, 0);
    bt_row = a.block_table + (int64_t)b * a.bt_stride;
    DEBUG_ONLY(debug_check_seqlens(a.cu_seqlens_q, b, a.total_q));
    DEBUG_ONLY(debug_check_length(a.context_lens[b], a.bt_stride * kBlockSize));
  } else {
    tq = a.tq;
    tk = a.tk;
  }
  const int off = tk - tq;
  const int m0 = mt * QM;
  if (m0 >= tq) return;

  const int tid = threadIdx.x;
  const int qi = m0 + tid / LPQ;
  const int part = tid % LPQ;
  const int64_t q_stride = PAGED ? (int64_t)a.hq * D : a.qs_t;
  const int64_t o_stride = PAGED ? (int64_t)a.hq * D : a.os_t;
  const float* qp = static_cast<const float*>(a.q) + (PAGED ? (q_row0 * a.hq + h) * D : b * a.qs_b + h * a.qs_h);
  float* op = static_cast<float*>(a.o) + (PAGED ? (q_row0 * a.hq + h) * D : b * a.os_b + h * a.os_h);
  const float* kp = static_cast<const float*>(a.k);
  const float* vp = static_cast<const float*>(a.v);
  // additive mask row of this query (rows past the queries read the last
  // row); paged rows hold mask_keys entries, later keys count as masked
  const float* mrow = nullptr;
  int mk = tk;
  if (a.mask != nullptr) {
    const int64_t mq = (PAGED ? q_row0 : 0) + min(qi, tq - 1);
    mrow = a.mask + (PAGED ? 0 : b * a.ms_b) + h * a.ms_h + mq * a.ms_q;
    if (PAGED) mk = min(tk, a.mask_keys);
  }

  float qr[64];
#pragma unroll
  for (int d = 0; d < 64; ++d) qr[d] = qi < tq ? qp[(int64_t)qi * q_stride + part * 64 + d] : 0.f;
  float acc[64];
#pragma unroll
  for (int d = 0; d < 64; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;

  int n_keys = tk;
  if (a.causal) n_keys = min(tk, min(m0 + QM, tq) - 1 + off + 1);
  for (int n0 = 0; n0 < n_keys; n0 += TN) {
    __syncthreads();
    for (int e = tid; e < TN * D / 4; e += blockDim.x) {
      const int row = e / (D / 4), c4 = e % (D / 4);
      const int key = n0 + row;
      float4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (key < tk) {
        if constexpr (PAGED) {
          const int64_t base = ((int64_t)safe_block(bt_row[key >> 4], a.num_blocks) * a.hkv + g) * (kBlockSize * D);
          kv = *reinterpret_cast<const float4*>(kp + base + (key & 15) * D + 4 * c4);
          // value blocks are token-minor: channel d of token t at d * 16 + t
          const float* vb = vp + base + (4 * c4) * kBlockSize + (key & 15);
          vv = float4{vb[0], vb[kBlockSize], vb[2 * kBlockSize], vb[3 * kBlockSize]};
        } else {
          kv = *reinterpret_cast<const float4*>(kp + b * a.ks_b + (int64_t)key * a.ks_t + g * a.ks_h + 4 * c4);
          vv = *reinterpret_cast<const float4*>(vp + b * a.vs_b + (int64_t)key * a.vs_t + g * a.vs_h + 4 * c4);
        }
      }
      *reinterpret_cast<float4*>(&ks[row][4 * c4]) = kv;
      *reinterpret_cast<float4*>(&vs[row][4 * c4]) = vv;
    }
    __syncthreads();
    float s[TN];
    float tmax = -INFINITY;
    const int lim = a.causal ? min(tk - 1, qi + off) : tk - 1;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < 64; ++d) dot = fmaf(qr[d], ks[j][part * 64 + d], dot);
      if (LPQ == 2) dot += __shfl_xor(dot, 1);
      // scores are kept in log2 units (scale * log2 e folded in once), so the
      // exponent below is a plain difference of stored values and the row
      // maximum gets weight exactly 1
      if (mrow != nullptr && n0 + j <= lim) dot = n0 + j < mk ? fmaf(mrow[n0 + j], a.mask_scale, dot) : -INFINITY;
      s[j] = (n0 + j <= lim) ? dot * c2 : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < 64; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float p = exp2f(s[j] - m_use);
      l_run += p;
#pragma unroll
      for (int d = 0; d < 64; ++d) acc[d] = fmaf(p, vs[j][part * 64 + d], acc[d]);
    }
    m_run = m_new;
  }
  if (qi < tq) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int d = 0; d < 64; ++d) op[(int64_t)qi * o_stride + part * 64 + d] = acc[d] * inv;
    if (!PAGED && a.lse != nullptr && part == 0)
      a.lse[((int64_t)b * a.hq + h) * tq + qi] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

}  // namespace


template <int D, bool PAGED, int HPW, int WPH>
static void launch_one(const PrefillArgs& a, bool deep_v, hipStream_t s) {
  dim3 grid(a.num_wg * (uint32_t)a.num_splits);
  if constexpr (PAGED && HPW * WPH == 4) {
    if (deep_v) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, true, HPW, WPH, false, true>), grid, dim3(64 * HPW * WPH), 0, s, a);
      if (a.num_splits > 1)
        hipLaunchKernelGGL((prefill_merge_kernel<D, PAGED, HPW, WPH>), dim3(a.num_wg * merge_parts<D, HPW, WPH>()),
                           dim3(256), 0, s, a);
      return;
    }
  }
  if constexpr ((HPW == 2 && WPH == 2) || (HPW == 1 && WPH == 4)) {
    // the masked variant exists for the default tiles only (the host picks
    // one of them and never splits a masked launch)
    if (a.mask != nullptr) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, PAGED, HPW, WPH, true>), grid, dim3(64 * HPW * WPH), 0, s, a);
      return;
    }
  }
  bool spread = false;
  if constexpr (D == 128 && !PAGED && HPW * WPH == 4) {
    // every key tile whole: the K DMAs spread over the PV phase
    spread = a.tk % BN == 0;
    if (spread)
      hipLaunchKernelGGL((prefill_bf16_kernel<D, false, HPW, WPH, false, false, true>), grid, dim3(64 * HPW * WPH), 0,
                         s, a);
  }
  if (!spread) hipLaunchKernelGGL((prefill_bf16_kernel<D, PAGED, HPW, WPH>), grid, dim3(64 * HPW * WPH), 0, s, a);
  if (a.num_splits > 1)
    hipLaunchKernelGGL((prefill_merge_kernel<D, PAGED, HPW, WPH>), dim3(a.num_wg * merge_parts<D, HPW, WPH>()),
                       dim3(256), 0, s, a);
}

template <int D, bool PAGED>
static void launch_cfg(const PrefillArgs& a, int hpw, int wph, bool deep_v, hipStream_t s) {
  if (hpw == 2 && wph == 4) launch_one<D, PAGED, 2, 4>(a, deep_v, s);
  else if (hpw == 2 && wph == 2) launch_one<D, PAGED, 2, 2>(a, deep_v, s);
  else if (hpw == 1 && wph == 4) launch_one<D, PAGED, 1, 4>(a, deep_v, s);
  else launch_one<D, PAGED, 1, 2>(a, deep_v, s);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, bool paged, int hpw, int wph, bool deep_v,
                               hipStream_t s) {
  if (head_dim == 128) {
    if (paged) launch_cfg<128, true>(a, hpw, wph, deep_v, s);
    else launch_cfg<128, false>(a, hpw, wph, deep_v, s);
  } else {
    if (paged) launch_cfg<64, true>(a, hpw, wph, deep_v, s);
    else launch_cfg<64, false>(a, hpw, wph, deep_v, s);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, bool paged, hipStream_t s) {
  dim3 grid(a.num_wg);
  if (paged) {
    if (head_dim == 128) hipLaunchKernelGGL((prefill_f32_kernel<128, true>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((prefill_f32_kernel<64, true>), grid, dim3(64), 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((prefill_f32_kernel<128, false>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((prefill_f32_kernel<64, false>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

// debug builds: this file's report word (nothing in release builds)
hipError_t debug_take_prefill(uint32_t* acc, bool clear) { return debug_take_word(acc, clear); }

}  // namespace mi_attn
