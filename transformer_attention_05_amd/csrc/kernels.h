// Argument blocks and launchers shared by the C ABI (api.cpp) and the HIP
// kernel sources.  Launchers assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

// RoPE frequencies theta_i = base^(-2i/D), i < D/2, computed once on the host
// in double and passed by value, so every kernel that rotates uses the same
// values.
constexpr int kMaxRopePairs = 64;
struct RopeFreqs {
  double theta[kMaxRopePairs];
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  // element strides of (batch, token, head); head_dim is contiguous
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int32_t batch, tq, tk, hq, hkv, group;
  int32_t causal;
  float scale_log2;  // softmax scale times log2(e)
  int32_t num_m_tiles;
  uint32_t num_wg;
  // paged variant only
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* cu_seqlens_q;
  const int32_t* context_lens;
  int32_t num_blocks;  // pool size; out-of-range table entries are redirected to block 0
  int32_t total_q;     // packed query rows; rows past it are never touched
  // split-KV (bf16 path): grid = num_wg query tiles x num_splits, the share
  // index fastest; share s of a query tile takes its key tiles
  // [s * L, (s + 1) * L) with L = split_tiles, or longer when the tile has
  // more than num_splits * split_tiles key tiles.  A query tile with more
  // than one share writes fp32 partials, merged by prefill_merge_kernel.
  int32_t num_splits;   // 1: no split
  int32_t split_tiles;  // key tiles per split (when num_splits > 1)
  int64_t ws_rows;      // partial rows per split: (query row, head) pairs
  float* ws_o;          // [num_splits][ws_rows][D], unnormalised output
  float* ws_ml;         // [num_splits][ws_rows][2]: max (log2 units), row sum
  // additive mask, fp32; null: none.  mask_scale = 1 / scale.
  // contiguous: element (b, h, i, j) at mask[b*ms_b + h*ms_h + i*ms_q + j];
  // paged: element (packed query row r, h, key position j) at
  // mask[r*ms_q + h*ms_h + j] for j < mask_keys (later keys are masked out).
  const float* mask;
  int64_t ms_b, ms_h, ms_q;
  float mask_scale;
  int32_t mask_keys;
};

struct DecodeArgs {
  const void* q;        // [S][Hq][D]
  const void* k_cache;  // [NB][Hkv][16][D]
  const void* v_cache;  // [NB][Hkv][D][16]
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* context_lens;
  void* o;              // [S][Hq][D]
  float* ws_ml;         // [S][Hq][max_parts][2]  (running max, running sum)
  float* ws_o;          // [S][Hq][max_parts][D]  (unnormalised output)
  int32_t* counters;    // [S][Hkv * head_groups] partitions finished (zero between calls)
  int32_t num_seqs, hq, hkv, group, head_groups;
  int32_t part_size, max_parts;
  int32_t num_blocks;  // pool size; out-of-range table entries are redirected to block 0
  float scale_log2;
  const int32_t* plan;  // [plan_items][2] (sequence, partition), or null: padded grid
  int32_t plan_items;
  // fused RoPE + cache write of each sequence's new token (decode kernels
  // built with the fused flag only)
  const void* k_new;            // [S][Hkv][D], the new token's key (not rotated)
  const void* v_new;            // [S][Hkv][D]
  const int32_t* positions;     // [S], the new token's position
  const int32_t* slot_mapping;  // [S], its cache slot; -1 or outside the pool: not written
  void* q_rot_out;              // [S][Hq][D] rotated queries, or null
  int32_t rope;                 // 0: no rotation (the write is a plain copy)
  RopeFreqs freqs;
};

struct RopeWriteArgs {
  void* q;
  const void* k;
  const void* v;
  const int32_t* positions;
  const int32_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  int32_t num_tokens, hq, hkv;
  int32_t num_blocks;  // slots at or past num_blocks * 16 are skipped
  int32_t rope;        // 0 = no rotation
  RopeFreqs freqs;
};

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* pairs;  // [num_pairs][2] (src, dst)
  int32_t num_pairs;
  int32_t num_blocks;    // ids outside [0, num_blocks) are skipped
  int64_t block_bytes;   // bytes of one block of one pool (a multiple of 16)
};

struct RmsNormArgs {
  const void* x;         // [rows][hidden]
  const void* residual;  // [rows][hidden]
  const void* weight;    // [hidden]
  void* y;               // [rows][hidden] normalised rows
  void* h_out;           // [rows][hidden] updated residual (may alias x or residual)
  int64_t rows;
  int32_t hidden;        // a multiple of 8, at most 8192
  float eps;
};

// Launchers return the launch status (hipSuccess or the error).
// hpw: query heads sharing each K/V tile (1 or 2); wph: wavefronts of 32
// queries per head (4 or 2).  Query tile = 32 * wph rows.  deep_v (paged,
// 4-wavefront tiles): a three-deep V ring, one workgroup per CU.
hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, bool paged, int hpw, int wph, bool deep_v,
                               hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, bool paged, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool fused, hipStream_t s);

// fp32 decode (no fused write); partitions may be any multiple of 16 tokens
hipError_t launch_decode_f32(const DecodeArgs& a, int head_dim, hipStream_t s);
// The library's fixed decode scratch on the current device (32 MiB, found
// and zero-filled on `s` on the first call per device), for
// attn_decode_paged_noalloc.
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(hipStream_t s, void** out);
// One launch running a paged prefill's workgroups (num_wg of them, no
// split, the 4-wavefront tile hpw x (4 / hpw)) and a decode's (planned, or
// the padded grid when da.plan is null): grid = [gp prefill, gd decode] x
// groups, then the remaining decode workgroups.
struct MixedSched {
  int32_t n_pre;   // prefill workgroups
  int32_t n_dec;   // decode workgroups
  int32_t gp, gd;  // workgroups of each kind per interleaved group
  int32_t groups;  // ceil(n_pre / gp)
};
inline uint32_t mixed_grid(const MixedSched& m) {
  const int64_t head = (int64_t)m.groups * (m.gp + m.gd);
  const int64_t rest = m.n_dec - (int64_t)m.groups * m.gd;
  return (uint32_t)(head + (rest > 0 ? rest : 0));
}
hipError_t launch_mixed(const PrefillArgs& pa, const DecodeArgs& da, const MixedSched& m, int head_dim, int hpw,
                        bool fused, hipStream_t s);
hipError_t launch_rope_write(const RopeWriteArgs& a, int head_dim, bool bf16, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s);
hipError_t launch_residual_rms_norm(const RmsNormArgs& a, bool bf16, hipStream_t s);

// Tile geometry of the bf16 prefill kernel, used to size its grid.
constexpr int kPrefillBlockN = 64;
constexpr int kPrefillF32BlockM = 64;
constexpr int kBlockSizeHost = 16;  // paged KV block, in tokens

// Debug builds: OR the report word of each kernel file on the current device
// into *acc (and zero it when `clear`); release builds leave *acc alone.
hipError_t debug_take_prefill(uint32_t* acc, bool clear);
hipError_t debug_take_decode(uint32_t* acc, bool clear);
hipError_t debug_take_rope_write(uint32_t* acc, bool clear);
hipError_t debug_take_copy_blocks(uint32_t* acc, bool clear);
hipError_t debug_take_mixed(uint32_t* acc, bool clear);

}  // namespace mi_attn
