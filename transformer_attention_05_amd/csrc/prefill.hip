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

constexpr int BN = kPrefillBlockN;  // keys per tile
constexpr float kLazyTau = 8.f;     // rescale only when the row max grows by more than 2^8

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// LDS tiles are unpadded and XOR-swizzled at 16-byte granularity so that
// the MFMA operand reads are free of bank conflicts.  (row, chunk) is stored
// in chunk slot  chunk ^ swizzle(row).
template <int D>
__device__ __forceinline__ int k_swz(int r) {    // K rows: 16 consecutive rows hit 16 distinct slots
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {    // V rows, read 4 rows x 64 B at a time by the transpose read
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}
__device__ __forceinline__ int vt_swz(int d) {   // V^T rows (paged, 64 keys = 8 chunks per row)
  return (d >> 1) & 7;
}

// Tile geometry: HPW query heads share every K/V tile (same kv head under
// GQA); each head has WPH wavefronts of 32 queries.
template <int D, bool PAGED, int HPW, int WPH>
__global__ __launch_bounds__(64 * HPW * WPH) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_bf16_kernel(const PrefillArgs a) {
  constexpr int NW = HPW * WPH;
  constexpr int BM = 32 * WPH;
  constexpr int CH = D / 8;                  // 16-byte chunks per K/V row
  constexpr int LOADS = BN * D * 2 / 1024;   // 1 KiB wave-wide DMA instructions per tile
  constexpr int LPW = LOADS / NW;
  static_assert(LPW * NW == LOADS, "tile DMA must split evenly over the wavefronts");
  constexpr int RPI = 64 / CH;               // rows per DMA instruction

  __shared__ __attribute__((aligned(1024))) __bf16 smk0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 smk1[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 smv0[BN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 smv1[BN * D];

  const uint32_t id = xcd_logical_id(blockIdx.x, a.num_wg);
  const int hgroups = a.hq / HPW;
  const uint32_t per_tile = (uint32_t)hgroups * (uint32_t)a.batch;
  const int mt = a.num_m_tiles - 1 - (int)(id / per_tile);
  const uint32_t rem = id % per_tile;
  const int b = (int)(rem / hgroups);
  const int h0 = (int)(rem % hgroups) * HPW;
  const int g = h0 / a.group;

  int32_t tq, tk;
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
  } else {
    tq = a.tq;
    tk = a.tk;
  }
  const int m0 = mt * BM;
  if (m0 >= tq) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int lq = lane & 31;
  const int h = h0 + wave / WPH;
  const int off = tk - tq;  // bottom-right causal alignment

  const __bf16* qp = static_cast<const __bf16*>(a.q);
  __bf16* op = static_cast<__bf16*>(a.o);
  const int64_t q_stride_t = PAGED ? (int64_t)a.hq * D : a.qs_t;
  const __bf16* q_base = PAGED ? qp + (q_row0 * a.hq + h) * D : qp + b * a.qs_b + h * a.qs_h;
  __bf16* o_base = PAGED ? op + (q_row0 * a.hq + h) * D : op + b * a.os_b + h * a.os_h;
  const int64_t o_stride_t = PAGED ? (int64_t)a.hq * D : a.os_t;

  // ---- Q^T operand (lane: query lq, channels 16c + 8hh .. +7), resident
  const int wq0 = m0 + (wave % WPH) * 32;
  const int qi = wq0 + lq;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qreg[c] = qi < tq ? *reinterpret_cast<const bf16x8*>(q_base + (int64_t)qi * q_stride_t + 16 * c + 8 * hh)
                      : bf16x8{};

  // ---- key tiles this workgroup visits
  int n_tiles = (tk + BN - 1) / BN;
  if (a.causal) {
    const int q_hi = min(m0 + BM, tq) - 1;
    const int kmax = min(tk - 1, q_hi + off);
    n_tiles = kmax < 0 ? 0 : kmax / BN + 1;
  }

  // ---- global -> LDS DMA of one K/V tile (rows past the keys re-read the
  // last key: finite values whose weights are masked to zero)
  const __bf16* kbase = static_cast<const __bf16*>(a.k);
  const __bf16* vbase = static_cast<const __bf16*>(a.v);
  auto key_row = [&](const __bf16* base, int64_t sb, int64_t st, int64_t sh, int key) -> const __bf16* {
    if constexpr (PAGED) {
      const int32_t blk = safe_block(bt_row[key >> 4], a.num_blocks);
      return base + (((int64_t)blk * a.hkv + g) * kBlockSize + (key & 15)) * D;
    } else {
      return base + b * sb + (int64_t)key * st + g * sh;
    }
  };
  auto issue_tile = [&](__bf16* dk, __bf16* dv, int n0) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int ii = wave * LPW + i;
      const int r = ii * RPI + lane / CH;
      const int slot = lane % CH;
      const int key = min(n0 + r, tk - 1);
      const __bf16* ksrc = key_row(kbase, a.ks_b, a.ks_t, a.ks_h, key) + 8 * (slot ^ k_swz<D>(r));
      __builtin_amdgcn_global_load_lds(ksrc, (lds_void*)(dk + ii * 512), 16, 0, 0);
      if constexpr (!PAGED) {
        const __bf16* vsrc = key_row(vbase, a.vs_b, a.vs_t, a.vs_h, key) + 8 * (slot ^ v_swz<D>(r));
        __builtin_amdgcn_global_load_lds(vsrc, (lds_void*)(dv + ii * 512), 16, 0, 0);
      } else {
        // V^T tile: row d holds the tile's 64 keys (8 chunks of 8 tokens),
        // read straight from the token-minor value blocks
        const int d = ii * 8 + lane / 8;
        const int c = (lane % 8) ^ vt_swz(d);
        int tok0 = n0 + 8 * c;
        if (tok0 >= tk) tok0 = ((tk - 1) >> 3) << 3;
        const int32_t blk = safe_block(bt_row[tok0 >> 4], a.num_blocks);
        const __bf16* vsrc = vbase + (((int64_t)blk * a.hkv + g) * D + d) * kBlockSize + (tok0 & 8);
        __builtin_amdgcn_global_load_lds(vsrc, (lds_void*)(dv + ii * 512), 16, 0, 0);
      }
    }
  };
  // Paged V^T: past the context a block holds arbitrary bits and 0 * NaN is
  // NaN, so the tokens of the last tile beyond the context are zeroed.
  auto zero_tail = [&](__bf16* dv, int n0) {
    if constexpr (PAGED) {
      const int nz = n0 + BN - tk;
      if (nz > 0) {
        for (int e = tid; e < D * nz; e += 64 * NW) {
          const int d = e / nz, kl = BN - nz + e % nz;
          dv[d * BN + 8 * ((kl >> 3) ^ vt_swz(d)) + (kl & 7)] = __bf16{};
        }
      }
    }
  };

  const float c2 = a.scale_log2;
  const float tau_raw = kLazyTau / c2;
  float m_run = -INFINITY;  // running max of raw scores (the one the weights are relative to)
  float l_run = 0.f;        // this lane's half of the row sum
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};

  const int wq_hi = min(wq0 + 31, tq - 1);
  const bool wave_has_rows = wq0 < tq;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto compute_tile = [&](const __bf16* sk, const __bf16* sv, int n0) {
    if (!(wave_has_rows && (!a.causal || n0 <= wq_hi + off))) return;
    // S^T = K Q^T, two 32-key subtiles.  The K operand reads run ahead of
    // the MFMAs (first subtile's reads, then one read of the second subtile
    // per MFMA of the first), so the MFMAs issue back to back.
    constexpr int NC = D / 16;
    f32x16 sacc[2];
    bf16x8 kop[2][NC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int r = kt * 32 + lq;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kop[kt][c] = *reinterpret_cast<const bf16x8*>(sk + r * D + 8 * ((2 * c + hh) ^ k_swz<D>(r)));
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc[kt] = mfma32(kop[kt][c], qreg[c], sacc[kt]);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if ((n0 + BN > tk) || (a.causal && n0 + BN - 1 > wq0 + off)) {
      const int lim = a.causal ? min(tk - 1, qi + off) : tk - 1;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > lim) sacc[kt][r] = -INFINITY;
        }
    }
    // online softmax; the reference max moves only when it grows by > 2^8
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kt][r]);
    tmax = fmaxf(tmax, xor32(tmax));
    if (__any(tmax > m_run + tau_raw)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY ? 0.f : m_run) * c2;
    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pb[kc][i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(sacc[kc >> 1][8 * (kc & 1) + i], c2, -mc)));
    // row sum of exactly the bf16 weights that enter the PV product
    float lsum = l_run;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 pr = {pb[kc][2 * i], pb[kc][2 * i + 1]};
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
      }
    l_run = lsum;
    // O^T += V^T P^T; keys of step kc in the accumulator's order.  The V^T
    // operand reads run one channel tile ahead of the MFMAs.
    u32x4 vop[D / 32][4];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        if constexpr (PAGED) {
          const int d = dt * 32 + lq;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(sv + d * BN + 8 * ((2 * kc) ^ vt_swz(d)) + 4 * hh);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(sv + d * BN + 8 * ((2 * kc + 1) ^ vt_swz(d)) + 4 * hh);
          vop[dt][kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          // transpose read: lane j of each 16-lane group addresses row
          // (key) base + j/4, channels 4*(j%4) .. +3 of its 16-channel slice
          const int grp = lane >> 4, j = lane & 15;
          const int dch = dt * 32 + 16 * (grp & 1) + 4 * (j & 3);  // first channel of the 8-byte piece
          const int r0 = 16 * kc + 4 * hh + (j >> 2);
          const int r1 = r0 + 8;
          const __bf16* p0 = sv + r0 * D + 8 * ((dch >> 3) ^ v_swz<D>(r0)) + (dch & 4);
          const __bf16* p1 = sv + r1 * D + 8 * ((dch >> 3) ^ v_swz<D>(r1)) + (dch & 4);
          const v4i16 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
          const v4i16 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
          const u32x2 lo = __builtin_bit_cast(u32x2, t0);
          const u32x2 hi = __builtin_bit_cast(u32x2, t1);
          vop[dt][kc] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, vop[dt][kc]), pb[kc], oacc[dt]);
#pragma unroll
    for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // DS read
#pragma unroll
    for (int i = 0; i < 4 * (D / 32) - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // 2 DS reads
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
  };

  // ---- main loop: DMA of tile j+1 overlaps the MFMAs of tile j.  The two
  // buffers are separate LDS objects and the loop is unrolled by two, so the
  // DMA into one buffer never forces a wait before reading the other.
  if (n_tiles > 0) {
    issue_tile(smk0, smv0, 0);
    __builtin_amdgcn_s_waitcnt(0);   // also retires the Q loads
    __syncthreads();
    zero_tail(smv0, 0);
    if (PAGED && BN > tk) __syncthreads();
  }
  for (int j = 0; j < n_tiles; j += 2) {
    const int n0 = j * BN;
    if (j + 1 < n_tiles) issue_tile(smk1, smv1, n0 + BN);
    compute_tile(smk0, smv0, n0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 >= n_tiles) break;
    if (PAGED && n0 + 2 * BN > tk) {
      zero_tail(smv1, n0 + BN);
      __syncthreads();
    }
    if (j + 2 < n_tiles) issue_tile(smk0, smv0, n0 + 2 * BN);
    compute_tile(smk1, smv1, n0 + BN);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (PAGED && j + 2 < n_tiles && n0 + 3 * BN > tk) {
      zero_tail(smv0, n0 + 2 * BN);
      __syncthreads();
    }
  }

  // ---- epilogue: O = O / l, optional LSE (natural log)
  const float l_tot = l_run + xor32(l_run);
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

template <int D, bool PAGED>
static void launch_cfg(const PrefillArgs& a, int hpw, int wph, hipStream_t s) {
  dim3 grid(a.num_wg);
  if (hpw == 2 && wph == 4) hipLaunchKernelGGL((prefill_bf16_kernel<D, PAGED, 2, 4>), grid, dim3(512), 0, s, a);
  else if (hpw == 2 && wph == 2) hipLaunchKernelGGL((prefill_bf16_kernel<D, PAGED, 2, 2>), grid, dim3(256), 0, s, a);
  else if (hpw == 1 && wph == 4) hipLaunchKernelGGL((prefill_bf16_kernel<D, PAGED, 1, 4>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((prefill_bf16_kernel<D, PAGED, 1, 2>), grid, dim3(128), 0, s, a);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, bool paged, int hpw, int wph, hipStream_t s) {
  if (head_dim == 128) {
    if (paged) launch_cfg<128, true>(a, hpw, wph, s);
    else launch_cfg<128, false>(a, hpw, wph, s);
  } else {
    if (paged) launch_cfg<64, true>(a, hpw, wph, s);
    else launch_cfg<64, false>(a, hpw, wph, s);
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
