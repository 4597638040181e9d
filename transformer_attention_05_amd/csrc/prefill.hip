// Prefill attention for gfx950: O = softmax(Q K^T * scale + M) V computed
// tile by tile with an online softmax, as "Fast Attention Kernels and
// Operator Fusion" (§FlashAttention-Style Kernels) describes FlashAttention:
// each workgroup owns a tile of queries, walks the key/value tiles, forms a
// block of scores, updates the running row max and row sum and accumulates
// the output on chip.  The Tq x Tk score matrix never reaches HBM.
//
// bf16 path (both contractions on MFMA, fp32 accumulate):
//   * workgroup = 4 wavefronts = 128 queries of one (batch, query head);
//     each wavefront owns 32 queries.
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
//   * K/V tiles of 64 keys are double-buffered in LDS; the next tile's global
//     loads are issued before the current tile's MFMAs.
//   * causal tiles wholly above the diagonal are never loaded; masking runs
//     only on tiles that cross the diagonal or the sequence end.
//   * workgroups are ordered heaviest first (last query tile first) and
//     renumbered so each XCD receives a contiguous range (K/V sharing in L2).
//   * P is rounded to bf16 for the PV MFMA and the row sum l accumulates the
//     same rounded values, so the output weights stay exactly normalised.
// The paged variant is the same loop with K/V rows gathered through the
// block table (16-token blocks): token t of sequence s lives in block
// block_table[s][t / 16] at offset t % 16.
//
// f32 path: a plain VALU kernel (one query per one or two lanes), used for
// full-precision parity runs.

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

constexpr int BM = kPrefillBlockM;  // queries per workgroup
constexpr int BN = kPrefillBlockN;  // keys per tile
constexpr int NW = 4;               // wavefronts per workgroup
constexpr int NT = NW * 64;

template <int D>
struct PrefillSmem {
  static constexpr int KS = D + 8;   // K row stride (elements): 16B-aligned rows, conflict-free b128 reads
  static constexpr int VS = BN + 4;  // V^T row stride: 8B-aligned, conflict-free b64 reads
  __bf16 k[2][BN * KS];
  __bf16 vt[2][D * VS];
};

template <int D, bool PAGED>
__global__ __launch_bounds__(NT) void prefill_bf16_kernel(const PrefillArgs a) {
  using S = PrefillSmem<D>;
  __shared__ S sm;

  const uint32_t id = xcd_logical_id(blockIdx.x, a.num_wg);
  const uint32_t per_tile = (uint32_t)a.hq * (uint32_t)a.batch;
  const int mt = a.num_m_tiles - 1 - (int)(id / per_tile);
  const uint32_t rem = id % per_tile;
  const int b = (int)(rem / a.hq);
  const int h = (int)(rem % a.hq);
  const int g = h / a.group;

  int32_t tq, tk;
  int64_t q_row0 = 0;
  const int32_t* bt_row = nullptr;
  if constexpr (PAGED) {
    const int32_t c0 = a.cu_seqlens_q[b];
    // a malformed cu_seqlens / context_lens can shrink the work, never widen
    // the memory it touches
    tq = max(0, min(a.cu_seqlens_q[b + 1], a.total_q) - max(c0, 0));
    tk = min(a.context_lens[b], a.bt_stride * kBlockSize);
    q_row0 = c0;
    bt_row = a.block_table + (int64_t)b * a.bt_stride;
  } else {
    tq = a.tq;
    tk = a.tk;
  }
  const int m0 = mt * BM;
  if (m0 >= tq) return;  // whole workgroup: no barrier is skipped by part of it

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;  // half of the wavefront
  const int lq = lane & 31;
  const int off = tk - tq;   // bottom-right causal alignment (tk >= tq for causal calls)

  const __bf16* qp = static_cast<const __bf16*>(a.q);
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* vp = static_cast<const __bf16*>(a.v);
  __bf16* op = static_cast<__bf16*>(a.o);

  // Row addresses.  Contiguous: batch/token/head strides.  Paged: packed q
  // rows [total_q][Hq][D]; K/V from the caches.
  const int64_t q_stride_t = PAGED ? (int64_t)a.hq * D : a.qs_t;
  const __bf16* q_base = PAGED ? qp + (q_row0 * a.hq + h) * D : qp + b * a.qs_b + h * a.qs_h;
  __bf16* o_base = PAGED ? op + (q_row0 * a.hq + h) * D : op + b * a.os_b + h * a.os_h;
  const int64_t o_stride_t = PAGED ? (int64_t)a.hq * D : a.os_t;

  // ---- Q^T operand, resident for the whole kernel
  const int wq0 = m0 + wave * 32;
  const int qi = wq0 + lq;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (qi < tq)
      qreg[c] = *reinterpret_cast<const bf16x8*>(q_base + (int64_t)qi * q_stride_t + 16 * c + 8 * hh);
    else
      qreg[c] = bf16x8{};
  }

  // ---- number of key tiles
  int n_tiles = (tk + BN - 1) / BN;
  if (a.causal) {
    const int q_hi = min(m0 + BM, tq) - 1;
    const int kmax = min(tk - 1, q_hi + off);
    n_tiles = kmax < 0 ? 0 : kmax / BN + 1;
  }

  // ---- global -> register staging of one K/V tile
  constexpr int CPR = D / 8;              // 16-byte chunks per K row
  constexpr int KPT = BN * CPR / NT;      // K chunks per thread
  static_assert(KPT * NT == BN * CPR, "K tile must split evenly");
  u32x4 kreg[KPT];
  // contiguous V: groups of 4 keys x 8 channels, transposed in registers
  constexpr int VG = (BN / 4) * CPR;
  constexpr int VPT_C = (VG + NT - 1) / NT;
  // paged V: the cache is token-minor, chunks of 8 tokens x 1 channel
  constexpr int VPT_P = (D * BN / 8) / NT;
  constexpr int VREGS = PAGED ? VPT_P : 4 * VPT_C;
  u32x4 vreg[VREGS];

  auto k_row_ptr = [&](int key) -> const __bf16* {
    if constexpr (PAGED) {
      const int32_t blk = safe_block(bt_row[key >> 4], a.num_blocks);
      return static_cast<const __bf16*>(a.k) + (((int64_t)blk * a.hkv + g) * kBlockSize + (key & 15)) * D;
    } else {
      return kp + b * a.ks_b + (int64_t)key * a.ks_t + g * a.ks_h;
    }
  };

  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPR, col = c % CPR;
      const int key = n0 + row;
      kreg[i] = key < tk ? *reinterpret_cast<const u32x4*>(k_row_ptr(key) + col * 8) : u32x4{0, 0, 0, 0};
    }
    if constexpr (PAGED) {
#pragma unroll
      for (int i = 0; i < VPT_P; ++i) {
        const int c = tid + i * NT;
        const int d = c >> 3, part = c & 7;
        const int bi = part >> 1, half = part & 1;
        const int tok0 = n0 + 16 * bi + 8 * half;
        u32x4 val = {0, 0, 0, 0};
        if (tok0 < tk) {
          const int32_t blk = safe_block(bt_row[tok0 >> 4], a.num_blocks);
          const __bf16* src = static_cast<const __bf16*>(a.v) +
                              (((int64_t)blk * a.hkv + g) * D + d) * kBlockSize + 8 * half;
          val = *reinterpret_cast<const u32x4*>(src);
          const int valid = tk - tok0;  // tokens of this chunk inside the context
          if (valid < 8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (2 * e >= valid) val[e] = 0;
              else if (2 * e + 1 >= valid) val[e] &= 0xffffu;
            }
          }
        }
        vreg[i] = val;
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT_C; ++i) {
        const int grp = tid + i * NT;
#pragma unroll
        for (int r = 0; r < 4; ++r) vreg[4 * i + r] = u32x4{0, 0, 0, 0};
        if (grp < VG) {
          const int k4 = grp / CPR, dc = grp % CPR;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = n0 + 4 * k4 + r;
            if (key < tk)
              vreg[4 * i + r] = *reinterpret_cast<const u32x4*>(vp + b * a.vs_b + (int64_t)key * a.vs_t +
                                                                 g * a.vs_h + dc * 8);
          }
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      const int row = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(&sm.k[buf][row * S::KS + col * 8]) = kreg[i];
    }
    if constexpr (PAGED) {
#pragma unroll
      for (int i = 0; i < VPT_P; ++i) {
        const int c = tid + i * NT;
        const int d = c >> 3, part = c & 7;
        const int bi = part >> 1, half = part & 1;
        __bf16* dst = &sm.vt[buf][d * S::VS + 16 * bi + 8 * half];
        reinterpret_cast<u32x2*>(dst)[0] = u32x2{vreg[i][0], vreg[i][1]};
        reinterpret_cast<u32x2*>(dst)[1] = u32x2{vreg[i][2], vreg[i][3]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT_C; ++i) {
        const int grp = tid + i * NT;
        if (grp < VG) {
          const int k4 = grp / CPR, dc = grp % CPR;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x0 = vreg[4 * i + 0][w], x1 = vreg[4 * i + 1][w];
            const uint32_t x2 = vreg[4 * i + 2][w], x3 = vreg[4 * i + 3][w];
            // channel 2w: low halves; channel 2w+1: high halves
            const u32x2 lo = {(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
            const u32x2 hi = {(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
            *reinterpret_cast<u32x2*>(&sm.vt[buf][(dc * 8 + 2 * w) * S::VS + 4 * k4]) = lo;
            *reinterpret_cast<u32x2*>(&sm.vt[buf][(dc * 8 + 2 * w + 1) * S::VS + 4 * k4]) = hi;
          }
        }
      }
    }
  };

  // ---- running statistics (raw-score units) and output accumulator
  const float c2 = a.scale_log2;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's half of the row sum
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};

  const int wq_hi = min(wq0 + 31, tq - 1);
  const bool wave_has_rows = wq0 < tq;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int n0 = j * BN;
    if (j + 1 < n_tiles) load_tile(n0 + BN);

    const bool active = wave_has_rows && (!a.causal || n0 <= wq_hi + off);
    if (active) {
      // S^T = K Q^T for two 32-key subtiles
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sacc[kt] = f32x16{};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8 kv = *reinterpret_cast<const bf16x8*>(&sm.k[buf][(kt * 32 + lq) * S::KS + 16 * c + 8 * hh]);
          sacc[kt] = mfma32(kv, qreg[c], sacc[kt]);
        }
      }
      // mask: only tiles crossing the diagonal or the end of the keys
      const bool need_mask = (n0 + BN > tk) || (a.causal && n0 + BN - 1 > wq0 + off);
      if (need_mask) {
        const int lim = a.causal ? min(tk - 1, qi + off) : tk - 1;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n0 + kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key > lim) sacc[kt][r] = -INFINITY;
          }
      }
      // online softmax
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kt][r]);
      tmax = fmaxf(tmax, xor32(tmax));
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      const float mc = m_use * c2;
      bf16x8 pb[4];
      float lsum = 0.f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kc >> 1][8 * (kc & 1) + i], c2, -mc));
          const __bf16 pbf = static_cast<__bf16>(p);
          pb[kc][i] = pbf;
          lsum += static_cast<float>(pbf);
        }
      }
      l_run = fmaf(l_run, alpha, lsum);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
      // O^T += V^T P^T, keys of step kc in the accumulator's order
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const __bf16* vrow = &sm.vt[buf][(dt * 32 + lq) * S::VS];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 16 * kc + 4 * hh);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 * kc + 8 + 4 * hh);
          const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
          oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, w), pb[kc], oacc[dt]);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, optional LSE
  const float l_tot = l_run + xor32(l_run);  // both halves of the row, wave-uniform call
  if (qi < tq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* orow = o_base + (int64_t)qi * o_stride_t;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * hh;
        const u32x2 w = {pack_bf16x2(oacc[dt][4 * rg + 0] * inv, oacc[dt][4 * rg + 1] * inv),
                         pack_bf16x2(oacc[dt][4 * rg + 2] * inv, oacc[dt][4 * rg + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (!PAGED && a.lse != nullptr && hh == 0) {
      const float lse = l_tot > 0.f ? (m_run * c2 + __log2f(l_tot)) * kLn2 : -INFINITY;
      a.lse[((int64_t)b * a.hq + h) * tq + qi] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// f32 VALU kernel: LPQ = D / 64 lanes per query, each holding 64 channels.
template <int D>
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
  const int tq = a.tq, tk = a.tk, off = tk - tq;
  const int m0 = mt * QM;
  if (m0 >= tq) return;

  const int tid = threadIdx.x;
  const int qi = m0 + tid / LPQ;
  const int part = tid % LPQ;
  const float* qp = static_cast<const float*>(a.q) + b * a.qs_b + h * a.qs_h;
  const float* kp = static_cast<const float*>(a.k) + b * a.ks_b + g * a.ks_h;
  const float* vp = static_cast<const float*>(a.v) + b * a.vs_b + g * a.vs_h;
  float* op = static_cast<float*>(a.o) + b * a.os_b + h * a.os_h;

  float qr[64];
#pragma unroll
  for (int d = 0; d < 64; ++d) qr[d] = qi < tq ? qp[(int64_t)qi * a.qs_t + part * 64 + d] : 0.f;
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
        kv = *reinterpret_cast<const float4*>(kp + (int64_t)key * a.ks_t + 4 * c4);
        vv = *reinterpret_cast<const float4*>(vp + (int64_t)key * a.vs_t + 4 * c4);
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
    for (int d = 0; d < 64; ++d) op[(int64_t)qi * a.os_t + part * 64 + d] = acc[d] * inv;
    if (a.lse != nullptr && part == 0)
      a.lse[((int64_t)b * a.hq + h) * tq + qi] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, bool paged, hipStream_t s) {
  dim3 grid(a.num_wg), block(NT);
  if (head_dim == 128) {
    if (paged) hipLaunchKernelGGL((prefill_bf16_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((prefill_bf16_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (paged) hipLaunchKernelGGL((prefill_bf16_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((prefill_bf16_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, hipStream_t s) {
  dim3 grid(a.num_wg);
  if (head_dim == 128) hipLaunchKernelGGL((prefill_f32_kernel<128>), grid, dim3(128), 0, s, a);
  else hipLaunchKernelGGL((prefill_f32_kernel<64>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace mi_attn
