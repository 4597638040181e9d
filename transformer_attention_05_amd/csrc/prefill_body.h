// Device code of the bf16 prefill workgroup: tile constants, the
// global->LDS DMA helpers, the LDS swizzles and bf16_body, one whole
// workgroup (the method is described at the top of prefill.hip).  Shared by
// prefill.hip and mixed.hip, each compiling its own copy.
#pragma once

#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {
namespace {
namespace pf {

constexpr int BN = kPrefillBlockN;  // keys per tile
constexpr float kLazyTau = 8.f;     // rescale only when the row max grows by more than 2^8

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte global -> LDS DMA of one lane (lane l's bytes land at lds + 16 l).
// Issued as inline asm so that the compiler does not track the LDS write:
// completion is ordered by the explicit vmcnt waits before the barriers that
// publish a tile, and the LDS ring buffers can then live in one array
// addressed by a uniform buffer offset.
// `lds` is the LDS byte address (uniform); the instruction takes it in M0.
// The compiler warns that M0, a register it reserves, is clobbered here: in
// these kernels nothing else uses M0 (every M0 write in their ISA is one of
// these DMAs), so no value of the compiler's lives in it across the asm.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
// the same from a uniform (scalar) base plus a 32-bit per-lane byte offset
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  const uint64_t p = (uint64_t)(uintptr_t)base;
  // readfirstlane returns int: widen through uint32_t (no sign extension)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "s"(lds) : "memory", "m0");
}

// Key tiles per split-KV share of a query tile that sees n_all key tiles:
// the planned length, or more when n_all exceeds what num_splits shares of
// that length cover (a context longer than the host planned for), so the
// shares always cover every tile.
__device__ __forceinline__ int split_len(int n_all, const PrefillArgs& a) {
  return a.num_splits > 1 ? max(a.split_tiles, (n_all + a.num_splits - 1) / a.num_splits) : max(n_all, 1);
}

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
__device__ __forceinline__ int vt_swz(int d) {   // V^T rows (paged): the two 16-byte halves of a
  return (d >> 3) & 1;                            // block's 32-byte row swap every 8 rows
}

// Tile geometry: HPW query heads share every K/V tile (same kv head under
// GQA); each head has WPH wavefronts of 32 queries.  MASKED adds the caller's
// additive mask M to every score and carries the weights P of the PV
// product as a bf16 pair (rounded value and rounded remainder).  SPREAD
// (contiguous, unmasked, D 128, two-deep V ring, every key tile whole: the
// key count a multiple of the tile) issues an iteration's tile DMAs inside
// its two phases instead of all at its top, V(j+1) one per odd chunk of the
// S phase and K(j+3) one per chunk of the PV phase, so their issue overlaps
// the matrix work; the DMA stream keeps its order (V(j+1), then K(j+3)), so
// every wait on it holds.
// LDS of one workgroup of bf16_body, in bf16 elements: the K and V rings
// and (MASKED) the mask ring.
template <int D, int HPW, int WPH, bool MASKED, bool DEEP_V>
constexpr int lds_elems() {
  return (3 + ((HPW * WPH == 4 && !DEEP_V) ? 2 : 3)) * BN * D + (MASKED ? 2 * HPW * WPH * 32 * BN * 2 : 0);
}

// One attention workgroup: number `bid` of the launch's num_wg * num_splits,
// its LDS at `sm` (lds_elems() elements, 1 KiB aligned).  The body of
// prefill_bf16_kernel, and of the serving-step kernel that runs these
// workgroups beside decode workgroups in one launch.
template <int D, bool PAGED, int HPW, int WPH, bool MASKED = false, bool DEEP_V = false, bool SPREAD = false>
__device__ __attribute__((always_inline)) inline void bf16_body(const PrefillArgs& a, const uint32_t bid, __bf16* sm) {
  constexpr int NW = HPW * WPH;
  constexpr int BM = 32 * WPH;
  constexpr int CH = D / 8;                  // 16-byte chunks per K/V row
  constexpr int LOADS = BN * D * 2 / 1024;   // 1 KiB wave-wide DMA instructions per tile
  constexpr int LPW = LOADS / NW;
  static_assert(LPW * NW == LOADS, "tile DMA must split evenly over the wavefronts");
  constexpr int RPI = 64 / CH;               // rows per DMA instruction

  // LDS: a ring of three K tiles followed by a ring of three V tiles
  constexpr int TILE = BN * D;
  // V ring depth: three tiles, or two for 4-wavefront workgroups, which
  // keeps them at 80 KiB of LDS so that two fit on a CU.  DEEP_V keeps three
  // (96 KiB) for a paged launch that shares the GPU with a decode: one such
  // workgroup per CU leaves the rest of the CU to a decode workgroup.
  constexpr int NVB = (NW == 4 && !DEEP_V) ? 2 : 3;
  static_assert(!SPREAD || (D == 128 && !PAGED && !MASKED && NVB == 2 && LPW == 4),
                "SPREAD: contiguous, unmasked, D 128, two-deep V ring (four DMAs of each tile per wavefront)");
  // MASKED: a two-slot ring of mask tiles after the K/V rings, one 32-row x
  // BN-key fp32 sub-tile per wavefront and slot (144 KiB in all at D 128:
  // one workgroup per CU, which also gives the masked variant's extra
  // registers room without spilling to memory)
  constexpr int MSUB = 32 * BN;  // floats of one sub-tile
  static_assert(lds_elems<D, HPW, WPH, MASKED, DEEP_V>() == (3 + NVB) * TILE + (MASKED ? 2 * NW * MSUB * 2 : 0),
                "LDS layout");

  // split-KV share index fastest: all shares of the longest query tiles
  // (dispatched first) start together
  const int split = (int)(bid % (uint32_t)a.num_splits);
  const uint32_t id = bid / (uint32_t)a.num_splits;
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
    DEBUG_ONLY(debug_check_seqlens(a.cu_seqlens_q, b, a.total_q));
    DEBUG_ONLY(debug_check_length(a.context_lens[b], a.bt_stride * kBlockSize));
  } else {
    tq = a.tq;
    tk = a.tk;
  }
  const int m0 = mt * BM;
  if (m0 >= tq) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets wave-derived values live in SGPRs
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

  // ---- key tiles this query tile visits, and this split's share of them
  int n_all = (tk + BN - 1) / BN;
  if (a.causal) {
    const int q_hi = min(m0 + BM, tq) - 1;
    const int kmax = min(tk - 1, q_hi + off);
    n_all = kmax < 0 ? 0 : kmax / BN + 1;
  }
  const int L = split_len(n_all, a);
  const int nsplit = max(1, (n_all + L - 1) / L);
  const int T0 = split * L;                    // first key tile of this split
  if (split > 0 && T0 >= n_all) return;        // uniform: no tiles left for this split
  int n_tiles = max(0, min(n_all - T0, L));        // tiles of this split
  // opaque to the optimiser: reasoning over how the count is derived costs
  // ~15 registers in the loop below
  asm volatile("" : "+s"(n_tiles));

  // ---- global -> LDS DMA of one K or V tile.  Rows past the keys re-read
  // the last key: finite values whose weights are masked to zero.  A paged
  // tile spans four 16-token blocks; their table entries are uniform over the
  // workgroup and come through scalar loads, so no vector-memory wait is ever
  // needed to form an address.
  const __bf16* kbase = static_cast<const __bf16*>(a.k);
  const __bf16* vbase = static_cast<const __bf16*>(a.v);
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  auto tile_blocks = [&](int t, int32_t (&blk)[4]) {
    if constexpr (PAGED) {
      const int last = (tk - 1) >> 4;
      const const_i32* row = (const const_i32*)bt_row;
#pragma unroll
      for (int i = 0; i < 4; ++i) blk[i] = safe_block(row[min(4 * t + i, last)], a.num_blocks);
    }
  };
  // one of the four block entries by a per-lane index (selects, no branches)
  auto pick4 = [](const int32_t (&blk)[4], int i) -> int32_t {
    const int32_t lo = (i & 1) ? blk[1] : blk[0];
    const int32_t hi = (i & 1) ? blk[3] : blk[2];
    return (i & 2) ? hi : lo;
  };
  // contiguous layout: a DMA of a whole tile in range reads from a scalar
  // row base plus this lane's byte offset (row within the DMA, swizzled
  // chunk); the offset fits in 32 bits for token strides below 2^28
  // elements, which attn_prefill requires
  uint32_t koff[LPW], voff[LPW];  // bytes
  // Scalar parts, formed once: the (batch, kv head) bases, and the element
  // offset of each DMA slot's first row within a tile, so a tile's DMA costs
  // one scalar multiply plus a 64-bit add per slot.
  const __bf16* const kb0 = kbase + b * a.ks_b + g * a.ks_h;
  const __bf16* const vb0 = vbase + b * a.vs_b + g * a.vs_h;
  int64_t krow[LPW], vrow[LPW];
  if constexpr (!PAGED) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = (wave * LPW + i) * RPI + lane / CH;
      koff[i] = 2u * (uint32_t)((lane / CH) * (int32_t)a.ks_t + 8 * ((lane % CH) ^ k_swz<D>(r)));
      voff[i] = 2u * (uint32_t)((lane / CH) * (int32_t)a.vs_t + 8 * ((lane % CH) ^ v_swz<D>(r)));
      krow[i] = (int64_t)((wave * LPW + i) * RPI) * a.ks_t;
      vrow[i] = (int64_t)((wave * LPW + i) * RPI) * a.vs_t;
    }
  } else {
    // paged K rows: the RPI rows of one DMA lie in one block, so a DMA reads
    // from that block's (scalar) base plus this lane's byte offset within
    // it, the same for every tile.  V^T: a DMA covers 32 channel rows of
    // one block (lane = row pair x half), so one offset serves every DMA
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int r = (wave * LPW + i) * RPI + lane / CH;
      koff[i] = 2u * (uint32_t)((r & 15) * D + 8 * ((lane % CH) ^ k_swz<D>(r)));
      voff[i] = 32u * (uint32_t)(lane >> 1) + 16u * (uint32_t)((lane & 1) ^ vt_swz(lane >> 1));
    }
  }
  // LDS byte address of the ring array (the one generic-to-LDS conversion);
  // a DMA destination is this plus a uniform byte offset
  const uint32_t sm_lds = (uint32_t)(uintptr_t)(lds_void*)sm;
  auto lds_of = [&](const __bf16* p) { return sm_lds + 2u * (uint32_t)(p - sm); };
  // Paged rows past the context read a valid slot of the last block (the
  // table entries are clamped to it); their scores are masked and their
  // values zeroed, so only the address has to stay inside the pool.
  auto issue_k = [&](__bf16* dk, int t, const int32_t (&blk)[4]) {
    const int n0 = t * BN;
    if constexpr (PAGED) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int ii = wave * LPW + i;     // uniform: so is the block of its rows
        const int32_t bk = pick4(blk, (ii * RPI) >> 4);
        dma16s(kbase + ((int64_t)bk * a.hkv + g) * (kBlockSize * D), koff[i], lds_of(dk) + ii * 1024);
      }
    } else if (n0 + BN <= tk) {
      const __bf16* tb = kb0 + (int64_t)n0 * a.ks_t;
      const uint32_t l0 = lds_of(dk) + wave * LPW * 1024;
#pragma unroll
      for (int i = 0; i < LPW; ++i) dma16s(tb + krow[i], koff[i], l0 + i * 1024);
    } else {
      // last partial tile: rows past the keys re-read the last key
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int ii = wave * LPW + i;
        const int r = ii * RPI + lane / CH;
        const int key = min(n0 + r, tk - 1);
        dma16(kbase + b * a.ks_b + (int64_t)key * a.ks_t + g * a.ks_h + 8 * ((lane % CH) ^ k_swz<D>(r)),
              lds_of(dk) + ii * 1024);
      }
    }
  };
  auto issue_v = [&](__bf16* dv, int t, const int32_t (&blk)[4]) {
    const int n0 = t * BN;
    if constexpr (PAGED) {
      // V^T tile, block-major: the tile's four token-minor value blocks
      // (D rows of 16 keys each) one after the other, as stored; DMA ii
      // takes rows 32 (ii % (D / 32)) .. +31 of block ii / (D / 32)
      constexpr int DPB = D / 32;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int ii = wave * LPW + i;
        const int32_t bk = pick4(blk, ii / DPB);
        dma16s(vbase + ((int64_t)bk * a.hkv + g) * (D * kBlockSize) + (ii % DPB) * (32 * kBlockSize), voff[i],
               lds_of(dv) + ii * 1024);
      }
    } else if (n0 + BN <= tk) {
      const __bf16* tb = vb0 + (int64_t)n0 * a.vs_t;
      const uint32_t l0 = lds_of(dv) + wave * LPW * 1024;
#pragma unroll
      for (int i = 0; i < LPW; ++i) dma16s(tb + vrow[i], voff[i], l0 + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int ii = wave * LPW + i;
        const int r = ii * RPI + lane / CH;
        const int key = min(n0 + r, tk - 1);
        dma16(vbase + b * a.vs_b + (int64_t)key * a.vs_t + g * a.vs_h + 8 * ((lane % CH) ^ v_swz<D>(r)),
              lds_of(dv) + ii * 1024);
      }
    }
  };
  // Paged V^T: past the context a block holds arbitrary bits and 0 * NaN is
  // NaN, so the tokens of the last tile beyond the context are zeroed.
  auto zero_tail = [&](__bf16* dv, int t) {
    const int nz = (t + 1) * BN - tk;
    for (int e = tid; e < D * nz; e += 64 * NW) {
      const int d = e / nz, kl = BN - nz + e % nz;
      dv[(kl >> 4) * (D * kBlockSize) + d * kBlockSize + 8 * (((kl >> 3) & 1) ^ vt_swz(d)) + (kl & 7)] = __bf16{};
    }
  };
  auto tail_tile = [&](int t) { return PAGED && t == n_all - 1 && (t + 1) * BN > tk; };
  // MASKED: the wavefront's 32 mask rows x BN keys of key tile src_t, by DMA
  // into ring slot slot_t % 2 (its own sub-tile; no other wavefront reads
  // it).  Row r of a sub-tile keeps 16-byte chunk c at position c ^ (r & 15),
  // so the reads of mask_tile (32 rows, one chunk each) hit distinct banks.
  // A chunk not wholly inside the row's first mk keys is not fetched (the
  // lane reads a harmless address inside q) and mask_tile loads those keys
  // one by one.
  const float* const mbase = MASKED ? a.mask + (PAGED ? 0 : b * a.ms_b) + h * a.ms_h : nullptr;
  const int mask_k = PAGED ? min(tk, a.mask_keys) : tk;
  const uint32_t mring_lds = sm_lds + 2u * (uint32_t)((3 + NVB) * TILE);
  auto issue_mask = [&](int slot_t, int src_t) {
    if constexpr (MASKED) {
      const uint32_t l0 = mring_lds + 4u * (uint32_t)(((slot_t & 1) * NW + wave) * MSUB);
#pragma unroll
      for (int ii = 0; ii < 8; ++ii) {
        const int r = 4 * ii + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        const int64_t mq = PAGED ? q_row0 + min(wq0 + r, tq - 1) : (int64_t)min(wq0 + r, tq - 1);
        const int k0 = src_t * BN + 4 * c;
        const float* src = k0 + 4 <= mask_k ? mbase + mq * a.ms_q + k0 : static_cast<const float*>(a.q);
        dma16(src, l0 + ii * 1024);
      }
    }
  };

  const float c2 = a.scale_log2;
  const float tau_raw = kLazyTau / c2;
  float m_run = -INFINITY;  // running max of raw scores (the one the weights are relative to)
  float mc = 0.f;           // m_run * c2 (0 while m_run is -inf)
  float l_run = 0.f;        // this lane's half of the row sum
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pb[4];  // P of the current tile, B operand of the PV MFMAs
  // MASKED: the remainder P - bf16(P), rounded to bf16 again.  A general
  // mask can leave a row a few keys with weights far from uniform, where the
  // 8-bit rounding of each weight no longer averages out; the second PV
  // product with the remainder carries the weights to about 16 bits.
  bf16x8 pl[MASKED ? 4 : 1];

  constexpr int NC = D / 16;        // contraction steps of S (16 channels each)
  constexpr int NS = 2 * NC;        // S MFMAs per tile
  constexpr int NP = 4 * (D / 32);  // PV MFMAs per tile

  // K operand of S^T = K Q^T: row kt*32 + lq, channels 16c + 8hh .. +7
  auto k_op = [&](const __bf16* sk, int kt, int c) -> bf16x8 {
    const int r = kt * 32 + lq;
    return *reinterpret_cast<const bf16x8*>(sk + r * D + 8 * ((2 * c + hh) ^ k_swz<D>(r)));
  };
  // V^T operand of O^T += V^T P^T for channel tile dt and key step kc, keys
  // in the order the S accumulator hands P over
  auto v_op = [&](const __bf16* sv, int dt, int kc) -> bf16x8 {
    if constexpr (PAGED) {
      const int d = dt * 32 + lq;
      // key step kc is block kc of the tile: row d, keys 4hh.. and 8 + 4hh..
      const __bf16* row = sv + kc * (D * kBlockSize) + d * kBlockSize;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 8 * vt_swz(d) + 4 * hh);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 8 * (1 ^ vt_swz(d)) + 4 * hh);
      return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    } else {
      // transpose read: lane j of each 16-lane group addresses row (key)
      // base + j/4, channels 4*(j%4) .. +3 of its 16-channel slice
      const int grp = lane >> 4, j = lane & 15;
      const int dch = dt * 32 + 16 * (grp & 1) + 4 * (j & 3);
      const int r0 = 16 * kc + 4 * hh + (j >> 2);
      const int r1 = r0 + 8;
      const __bf16* p0 = sv + r0 * D + 8 * ((dch >> 3) ^ v_swz<D>(r0)) + (dch & 4);
      const __bf16* p1 = sv + r1 * D + 8 * ((dch >> 3) ^ v_swz<D>(r1)) + (dch & 4);
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1));
      return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  };

  // S^T for one tile (two 32-key subtiles, MFMAs alternate between them);
  // used once, before the pipeline starts
  auto s_mfma = [&](const __bf16* sk, f32x16 (&s)[2]) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32(k_op(sk, kt, c), qreg[c], c == 0 ? f32x16{} : s[kt]);
  };
  // P = 2^(S c2 - m c2) for half h of key step kc, rounded to bf16, and
  // the row sum of exactly those rounded weights
  auto exp_half = [&](const f32x16 (&s)[2], int kc, int h) {
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[kc >> 1][8 * (kc & 1) + i]);
      pb[kc][i] = static_cast<__bf16>(p);
      // p - bf16(p) is exact in fp32
      if constexpr (MASKED) pl[kc][i] = static_cast<__bf16>(p - static_cast<float>(pb[kc][i]));
    }
  };
  // the row sum of exactly the rounded weights of key step kc (and of their
  // remainders, MASKED), in the order the weights were formed
  auto row_sum = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 pr = {pb[kc][2 * i], pb[kc][2 * i + 1]};
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
      if constexpr (MASKED) {
        const bf16x2 pq = {pl[kc][2 * i], pl[kc][2 * i + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pq, ones, l_run, false);
      }
    }
  };
  // Phase A: S(next) = K Q^T on the matrix cores while the VALU forms P
  // from S(cur).  Eight chunks; each issues NS/8 MFMAs, reads the K operands
  // of the next chunk and does half a key step of the exponentials.
  // sched_barrier(0) between chunks keeps the operand registers bounded.
  // before_exp runs once the first chunk's MFMAs are issued: the running
  // max update for S(cur) (its row max comes from the previous phase B), so
  // the max's cross-lane step, vote and branch overlap those MFMAs instead
  // of ending the previous iteration.
  constexpr int SPC = NS / 8;  // S MFMAs per chunk
  auto phase_a = [&](const __bf16* sk, const f32x16 (&s)[2], f32x16 (&sn)[2], auto&& before_exp, auto&& per_chunk) {
    bf16x8 kcur[SPC], knxt[SPC];
#pragma unroll
    for (int u = 0; u < SPC; ++u) kcur[u] = k_op(sk, u & 1, u >> 1);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < 7) {
#pragma unroll
        for (int u = 0; u < SPC; ++u) {
          const int m = (q + 1) * SPC + u;
          knxt[u] = k_op(sk, m & 1, m >> 1);
        }
      }
#pragma unroll
      for (int u = 0; u < SPC; ++u) {
        const int m = q * SPC + u;
        const int c = m >> 1, kt = m & 1;
        sn[kt] = mfma32(kcur[u], qreg[c], c == 0 ? f32x16{} : sn[kt]);
      }
      if (q == 0) {
        __builtin_amdgcn_sched_barrier(0);
        before_exp();
      }
      exp_half(s, q >> 1, q & 1);
      per_chunk(q);
      if (q & 1) asm volatile("" : "+v"(pb[q >> 1]));
      if constexpr (MASKED) {
        if (q & 1) asm volatile("" : "+v"(pl[q >> 1]));
      }
      if (q > 0) {
#pragma unroll
        for (int u = 0; u < SPC; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (q < 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read (next chunk)
          __builtin_amdgcn_sched_group_barrier(0x002, 10 / SPC, 0);  // VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (q < 7) {
#pragma unroll
        for (int u = 0; u < SPC; ++u) kcur[u] = knxt[u];
      }
    }
  };
  // Phase B: O^T += V^T P^T, one key step per chunk, V^T operands read a
  // chunk ahead; the VALU takes the row max of S(next) meanwhile.
  constexpr int DT = D / 32;
  auto phase_b = [&](const __bf16* sv, f32x16 (&sn)[2], float& tmax, auto&& per_chunk) {
    bf16x8 vcur[DT], vnxt[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vcur[dt] = v_op(sv, dt, 0);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      if (kc < 3) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vnxt[dt] = v_op(sv, dt, kc + 1);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        oacc[dt] = mfma32(vcur[dt], pb[kc], oacc[dt]);
        if constexpr (MASKED) oacc[dt] = mfma32(vcur[dt], pl[kc], oacc[dt]);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) tmax = fmaxf(tmax, sn[kc >> 1][8 * (kc & 1) + r]);
      // the exponent of the next tile, s * scale * log2 e - m (log2 units),
      // formed here where the VALU is idle; the max update at the start of
      // the next phase A corrects it when m moves
#pragma unroll
      for (int r = 0; r < 8; ++r) sn[kc >> 1][8 * (kc & 1) + r] = fmaf(sn[kc >> 1][8 * (kc & 1) + r], c2, -mc);
      row_sum(kc);
      per_chunk(kc);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        __builtin_amdgcn_sched_group_barrier(0x008, MASKED ? 2 : 1, 1);  // MFMA
        if (kc < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // DS reads (next chunk)
        __builtin_amdgcn_sched_group_barrier(0x002, MASKED ? 5 : 4, 1);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kc < 3) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vcur[dt] = vnxt[dt];
      }
    }
  };
  // Keys of the split end at key_end; the tile after the split's last one
  // (the loop's dummy) lies wholly past it and is masked completely.
  const int key_end = min(tk, (T0 + n_tiles) * BN);
  auto needs_mask = [&](int t) {
    return (t + 1) * BN > key_end || (a.causal && (t + 1) * BN - 1 > wq0 + off);
  };
  auto mask_tile = [&](f32x16 (&s)[2], int t) {
    if constexpr (MASKED) {
      // the additive mask M (natural-log units) enters the raw scores as
      // M / scale, so the exponent becomes (s + M / scale) * scale * log2 e;
      // lane keys t*BN + 32kt + 8g + 4hh + j, j < 4, are four consecutive
      // floats of the mask row (rows past the queries read the last row,
      // keys past the keys read nothing: both are discarded or masked)
      // Paged: the row of packed query q_row0 + qi, keys = positions in the
      // sequence's context; entries at or past mask_keys are never read and
      // those keys are masked out.
      // Chunks wholly inside the first mk keys come from this wavefront's
      // sub-tile in LDS (issue_mask); the others, only in a row's last tile,
      // are loaded here key by key.  The sub-tile of tile t was issued an
      // iteration earlier: only this iteration's DMA (2 * LPW K/V and 8 mask
      // instructions) may still be in flight.
      {
        constexpr int AFTER = 2 * LPW + 8;
        __builtin_amdgcn_s_waitcnt(0x0f70 | (AFTER & 15) | ((AFTER >> 4) << 14));
      }
      const int64_t mq = PAGED ? q_row0 + min(qi, tq - 1) : (int64_t)min(qi, tq - 1);
      const float* mrow = mbase + mq * a.ms_q;
      const int mk = mask_k;
      const float* msub = reinterpret_cast<const float*>(sm + (3 + NVB) * TILE) + ((t & 1) * NW + wave) * MSUB;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 mv[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int key0 = t * BN + kt * 32 + 8 * g4 + 4 * hh;
          if (key0 + 4 <= mk) {
            mv[g4] = *reinterpret_cast<const f32x4*>(msub + lq * BN + 4 * ((kt * 8 + 2 * g4 + hh) ^ (lq & 15)));
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) mv[g4][j] = key0 + j < mk ? mrow[key0 + j] : (key0 + j < tk ? -INFINITY : 0.f);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = fmaf(mv[r >> 2][r & 3], a.mask_scale, s[kt][r]);
      }
    }
    const int lim = a.causal ? min(key_end - 1, qi + off) : key_end - 1;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t * BN + kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key > lim) s[kt][r] = -INFINITY;
      }
  };
  auto row_max = [&](const f32x16 (&s)[2]) -> float {
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[kt][r]);
    return fmaxf(tmax, xor32(tmax));
  };
  // online softmax: the reference max moves only when it grows by > 2^8
  auto update_max = [&](float tmax, f32x16* formed) {
    if (__any(tmax > m_run + tau_raw)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f((m_run - (m_new == -INFINITY ? 0.f : m_new)) * c2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
      const float mc_new = (m_run == -INFINITY ? 0.f : m_run) * c2;
      if (formed != nullptr) {
        // exponents formed with the old reference: shift them to the new one
        const float dm = mc_new - mc;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) formed[kt] -= dm;
      }
      mc = mc_new;
    }
  };
  // DMA instructions of the current iteration that may still be in flight
  // at its end: K(j+3) and V(j+2) with the three-deep V ring; only K(j+3)
  // with the two-deep one (its V(j+1) is issued first and must land); and
  // the mask tile j+2 (issued last, read in the next iteration)
  constexpr int PENDING = (NVB == 3 ? 2 * LPW : LPW) + (MASKED ? 8 : 0);
  auto tile_barrier = [&]() {
    // s_waitcnt vmcnt(PENDING) (expcnt and lgkmcnt fields at their no-wait maximum)
    __builtin_amdgcn_s_waitcnt(0x0f70 | (PENDING & 15) | ((PENDING >> 4) << 14));
    __syncthreads();
  };

  // ---- software pipeline.  Iteration j: S(j+1) = K(j+1) Q^T on the matrix
  // cores while the VALU turns S(j) into P(j); then O += V(j)^T P(j) while
  // the VALU takes the row max of S(j+1).  Tile t of K lives in ring buffer
  // t % 3 and the DMA of K(j+3) issued in iteration j has two iterations to
  // land; tile t of V lives in buffer t % NVB and is loaded NVB - 1
  // iterations ahead.  Every iteration issues the same number of DMA
  // instructions (the tile index is clamped), so one vmcnt covers them.
  __bf16* const kring = sm;
  __bf16* const vring = sm + 3 * TILE;
  f32x16 sa[2], sb[2];
  // paged: block-table entries of the K tile and the V tile the next
  // iteration loads (the V tile of one iteration is the K tile of the one
  // before, and the K entries are fetched an iteration ahead)
  int32_t blk_k[4], blk_v[4], blk_v1[4];
  if (n_tiles > 0) {
    {
      int32_t b0[4], b1[4];
      tile_blocks(T0, b0);
      tile_blocks(T0 + min(1, n_tiles - 1), b1);
      tile_blocks(T0 + min(2, n_tiles - 1), blk_v);
      tile_blocks(T0 + min(3, n_tiles - 1), blk_k);
      issue_k(kring, T0, b0);
      issue_v(vring, T0, b0);
      issue_k(kring + TILE, T0 + min(1, n_tiles - 1), b1);
      if constexpr (NVB == 3) issue_v(vring + TILE, T0 + min(1, n_tiles - 1), b1);
      issue_k(kring + 2 * TILE, T0 + min(2, n_tiles - 1), blk_v);
      issue_mask(T0, T0);
      issue_mask(T0 + 1, T0 + min(1, n_tiles - 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) blk_v1[i] = b1[i];
    }
    if constexpr (MASKED) {
      __builtin_amdgcn_s_waitcnt(0);  // also retires the Q loads
    } else {
      // Q and K(0) only (the Q loads came first): S(0) overlaps the other
      // tiles' arrival.  s_waitcnt vmcnt(N) (expcnt, lgkmcnt at no-wait)
      constexpr int N0 = (NVB == 3 ? 4 : 3) * LPW;  // V(0), K(1), [V(1)], K(2)
      __builtin_amdgcn_s_waitcnt(0x0f70 | (N0 & 15) | ((N0 >> 4) << 14));
    }
    __syncthreads();
    if (tail_tile(T0)) {  // uniform: V(0) is zeroed past the context once it has landed
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      zero_tail(vring, T0);
    }
    s_mfma(kring, sa);
    if (MASKED || needs_mask(T0)) mask_tile(sa, T0);
    update_max(row_max(sa), nullptr);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sa[kt][r] = fmaf(sa[kt][r], c2, -mc);
    if constexpr (!MASKED) {
      // iteration 0 reads K(1) and V(0); K(2) may still be in flight
      constexpr int N1 = LPW;
      __builtin_amdgcn_s_waitcnt(0x0f70 | (N1 & 15) | ((N1 >> 4) << 14));
    }
    __syncthreads();
  }
  // Q^T is in registers by now (the wait above retired its loads), but the
  // compiler's wait insertion keeps them pending and would put a vmcnt(0) in
  // front of the loop's first use of Q^T, which would also wait for the tile
  // DMAs just issued.  Passing the registers through an empty asm makes them
  // the asm's results; any wait it adds sits here, before the loop.
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" : "+v"(qreg[c]));
  // Iteration j (tile T0 + j of the query tile's key tiles).  The last
  // iteration also computes S for the tile after this split's last one: its
  // K buffer holds a re-read of the last tile and every score of it is
  // masked, so it changes nothing and the loop body has a single form.
  // r0, r1, r2 = j % 3, (j + 1) % 3, (j + 2) % 3.
  int r0 = 0, r1 = 1, r2 = 2;
  float pend = -INFINITY;  // row max of the newest S, applied at the start of the next phase A
  auto iteration = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int vcur = NVB == 3 ? r0 : (j & 1);  // ring buffer of V(j)
    const int vnext = NVB == 3 ? r1 : (vcur ^ 1);  // of V(j+1)
    if constexpr (NVB == 3) {
      issue_k(kring + r0 * TILE, T0 + min(j + 3, n_tiles - 1), blk_k);
      issue_v(vring + r2 * TILE, T0 + min(j + 2, n_tiles - 1), blk_v);
    } else if constexpr (!SPREAD) {
      issue_v(vring + vnext * TILE, T0 + min(j + 1, n_tiles - 1), blk_v1);
      issue_k(kring + r0 * TILE, T0 + min(j + 3, n_tiles - 1), blk_k);
    }
    // slot from the tile's own index, source clamped like the K/V tiles
    issue_mask(T0 + j + 2, T0 + min(j + 2, n_tiles - 1));
    if constexpr (PAGED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        blk_v1[i] = blk_v[i];  // tile j + 2 (the two-deep ring's next V)
        blk_v[i] = blk_k[i];   // tile j + 3
      }
      tile_blocks(T0 + min(j + 4, n_tiles - 1), blk_k);
    }
    phase_a(kring + r1 * TILE, sc, sn, [&]() { update_max(fmaxf(pend, xor32(pend)), sc); }, [&](int q) {
      if constexpr (SPREAD) {
        if (q & 1) {  // V(j+1), a whole tile: this wavefront's DMA q/2 of it
          const int i = q >> 1;
          const __bf16* tb = vb0 + (int64_t)((T0 + min(j + 1, n_tiles - 1)) * BN) * a.vs_t;
          dma16s(tb + vrow[i], voff[i], lds_of(vring + vnext * TILE) + (wave * LPW + i) * 1024);
        }
      }
    });
    if (MASKED || needs_mask(T0 + j + 1)) mask_tile(sn, T0 + j + 1);
    pend = -INFINITY;
    phase_b(vring + vcur * TILE, sn, pend, [&](int kc) {
      if constexpr (SPREAD) {
        // K(j+3), a whole tile: this wavefront's DMA kc of it
        const __bf16* tb = kb0 + (int64_t)((T0 + min(j + 3, n_tiles - 1)) * BN) * a.ks_t;
        dma16s(tb + krow[kc], koff[kc], lds_of(kring + r0 * TILE) + (wave * LPW + kc) * 1024);
      }
    });
    tile_barrier();
    if (tail_tile(T0 + j + 1)) {
      zero_tail(vring + vnext * TILE, T0 + j + 1);
      __syncthreads();
    }
    const int t = r0;
    r0 = r1;
    r1 = r2;
    r2 = t;
  };
  if (n_tiles > 0) {
    for (int j = 0; j < n_tiles; j += 2) {
      iteration(j, sa, sb);
      if (j + 1 >= n_tiles) break;
      iteration(j + 1, sb, sa);
    }
    // no DMA may still be writing this workgroup's LDS when it exits
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- epilogue: O = O / l, optional LSE (natural log); with several
  // splits the unnormalised O, the max (log2 units) and the row sum go to
  // the workspace for prefill_merge_kernel
  const float l_tot = l_run + xor32(l_run);
  if (qi < tq) {
    if (nsplit > 1) {
      const int64_t row = PAGED ? (q_row0 + qi) * a.hq + h : ((int64_t)b * tq + qi) * a.hq + h;
      const int64_t slot = (int64_t)split * a.ws_rows + row;
      float* wo = a.ws_o + slot * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = dt * 32 + 8 * rg + 4 * hh;
          *reinterpret_cast<f32x4*>(wo + d0) =
              f32x4{oacc[dt][4 * rg + 0], oacc[dt][4 * rg + 1], oacc[dt][4 * rg + 2], oacc[dt][4 * rg + 3]};
        }
      if (hh == 0) {
        a.ws_ml[slot * 2 + 0] = m_run * c2;
        a.ws_ml[slot * 2 + 1] = l_tot;
      }
    } else if (!PAGED && a.lse != nullptr && hh == 0) {
      const float lse = l_tot > 0.f ? (m_run * c2 + __log2f(l_tot)) * kLn2 : -INFINITY;
      a.lse[((int64_t)b * a.hq + h) * tq + qi] = lse;
    }
  }
  if (nsplit <= 1) {
    // O through LDS, so that global stores cover whole rows: the wave writes
    // its 32 x D tile (row = query, 16-byte chunks XOR-swizzled by row, free
    // of bank conflicts both ways) into its own slice of the ring array, then
    // reads it back 16 bytes per lane in row order.  The barrier first lets
    // every wave finish with the K/V rings.
    __syncthreads();
    constexpr int CPRW = D / 8;         // 16-byte chunks per row
    constexpr int RPS = 64 / CPRW;      // rows per store instruction
    __bf16* st = sm + wave * 32 * D;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c = 4 * dt + rg;  // chunk of channels dt*32 + 8*rg .. +7; this lane has half hh
        const u32x2 w = {pack_bf16x2(oacc[dt][4 * rg + 0] * inv, oacc[dt][4 * rg + 1] * inv),
                         pack_bf16x2(oacc[dt][4 * rg + 2] * inv, oacc[dt][4 * rg + 3] * inv)};
        *reinterpret_cast<u32x2*>(st + lq * D + 8 * (c ^ (lq & (CPRW - 1))) + 4 * hh) = w;
      }
#pragma unroll
    for (int it = 0; it < 32 / RPS; ++it) {
      const int row = it * RPS + lane / CPRW;
      const int c = lane % CPRW;
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + row * D + 8 * (c ^ (row & (CPRW - 1))));
      const int q = wq0 + row;
      if (q < tq) *reinterpret_cast<u32x4*>(o_base + (int64_t)q * o_stride_t + 8 * c) = v;
    }
  }
}

}  // namespace pf
}  // namespace
}  // namespace mi_attn
