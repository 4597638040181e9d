// C ABI entry points: argument validation, launch geometry and launch.
//
// Every entry point validates all of its arguments before the first HIP call
// ("Fast Attention Kernels and Operator Fusion" notes that hard-wired
// attention backends fail when they do not support the inputs, and that a
// serving engine validates its backend at initialisation and raises; here an
// unsupported or malformed call returns a status and launches nothing).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kernels.h"
#include "mi_attn.h"
#include "status.h"

using namespace mi_attn;

namespace mi_attn {
char* error_buffer() {
  static thread_local char buf[512];
  return buf;
}
}  // namespace mi_attn

extern "C" const char* attn_last_error(void) { return error_buffer(); }

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_head_dim(int32_t d, const char* fn) {
  if (d != 64 && d != 128) return fail(ATTN_E_UNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", fn, d);
  return ATTN_OK;
}

int check_heads(int32_t hq, int32_t hkv, const char* fn) {
  if (hq < 1 || hkv < 1) return fail(ATTN_E_INVALID, "%s: head counts must be >= 1 (got %d, %d)", fn, hq, hkv);
  if (hq % hkv != 0)
    return fail(ATTN_E_INVALID, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", fn, hq, hkv);
  return ATTN_OK;
}

int check_scale(float scale, int32_t d, float* scale_log2, const char* fn) {
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(ATTN_E_INVALID, "%s: scale must be finite and >= 0 (0 = 1/sqrt(head_dim))", fn);
  const double sc = scale == 0.f ? 1.0 / std::sqrt((double)d) : (double)scale;
  *scale_log2 = (float)(sc * 1.4426950408889634);
  return ATTN_OK;
}

int launched(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

constexpr double kLog2eHost = 1.4426950408889634;

// theta_i = base^(-2i/D) for the D/2 rotation pairs, in double
RopeFreqs rope_freqs(float base, int32_t head_dim) {
  RopeFreqs f{};
  for (int i = 0; i < head_dim / 2 && i < kMaxRopePairs; ++i)
    f.theta[i] = std::pow((double)base, -2.0 * (double)i / (double)head_dim);
  return f;
}

// Tile shape of the bf16 prefill kernel: two query heads of one kv group per
// workgroup (each K/V tile serves both) and 64-query tiles, or one head and
// 128 queries for odd groups: 4 wavefronts.
struct PrefillTile {
  int hpw, wph;
};

PrefillTile prefill_tile(int32_t group) {
  const int hpw = (group % 2 == 0) ? 2 : 1;
  // measured on MI355X: 4-wavefront tiles hold 80 KiB of LDS, so two
  // workgroups share a CU and their phases drift apart (one's matrix work
  // overlaps the other's softmax).  Contiguous: faster than the 8-wavefront
  // tile at every size measured.  Paged (8 chunks of 512 new tokens on
  // 0-2048 cached): 69.7 us against 82.6 for the 8-wavefront tile, which
  // halves the block gathers per query but fits one workgroup per CU.
  return PrefillTile{hpw, hpw == 2 ? 2 : 4};
}

// Split-KV plan of the bf16 prefill.  A launch with too few query tiles to
// fill the chip (a short prompt, one long-context chunk) leaves CUs idle
// while the longest query tile walks all of its key tiles.  Cutting each query
// tile's key tiles into shares of split_tiles tiles multiplies the workgroups
// and shortens that critical path; a merge pass recombines the shares' (m, l,
// O) exactly, as the decode does with its partitions.  A query tile whose key
// tiles fit in one share still writes its output directly.  Every share pays
// a workgroup's fixed cost (Q and the first K/V tiles in, the pipeline's fill
// and drain, the output out: ~6-13 us measured on MI355X) and its fp32
// partials are written and read back, so only launches that would fill less
// than half of the workgroup slots split, into shares of at least 8 tiles.
// A launch that already fills most CUs (the chunks of a serving step, which
// also share the GPU with the decode) gains nothing and runs in one pass.
constexpr int kCUs = 256;           // MI355X compute units
constexpr int kMinSplitTiles = 8;
struct PrefillPlan {
  PrefillTile t;
  bool deep_v = false;  // paged 4-wavefront tile with a three-deep V ring (one per CU)
  int32_t num_m_tiles = 0;
  int64_t num_wg = 0;
  int32_t num_splits = 1, split_tiles = 0;
  int64_t ws_rows = 0;
  size_t o_bytes = 0, ml_bytes = 0;
};

// rows: (query row, head) pairs of the output, the workspace's row count.
// max_k: keys of the longest sequence (an upper bound for a paged batch).
PrefillPlan plan_prefill(int64_t max_q, int64_t max_k, int32_t hq, int32_t group, int64_t batch,
                         int32_t d, bool paged, int64_t rows, bool share_cu = false) {
  PrefillPlan p;
  p.t = prefill_tile(group);
  // sharing the GPU with a decode: the paged 4-wavefront tile with a
  // three-deep V ring (96 KiB of LDS, 264 VGPRs) fits once per CU, which
  // leaves room beside it for one decode workgroup (232 VGPRs); two of the
  // two-deep tiles (80 KiB, 256 VGPRs each) fill a CU.  Measured on MI355X
  // with 8 chunks of 512 new tokens beside a 128-sequence decode: 190-191
  // vs 193-195 us per step, while alone the chunks take 82.6 vs 69.7 us.
  p.deep_v = paged && share_cu && p.t.hpw * p.t.wph == 4;
  p.num_m_tiles = ceil_div(max_q, 32 * p.t.wph);
  p.num_wg = (int64_t)p.num_m_tiles * (hq / p.t.hpw) * batch;
  // two 4-wavefront workgroups share a CU (80 KiB of LDS each)
  const int64_t slots = (int64_t)kCUs * ((p.t.hpw * p.t.wph == 4 && !p.deep_v) ? 2 : 1);
  const int64_t t_max = (max_k + 63) / 64;  // key tiles of the longest query tile
  int64_t L = 0;
  if (2 * p.num_wg <= slots && t_max >= 2 * kMinSplitTiles) {
    const int64_t s = std::min((slots + p.num_wg - 1) / p.num_wg, (t_max + kMinSplitTiles - 1) / kMinSplitTiles);
    if (s > 1) L = (t_max + s - 1) / s;
  }
  if (L > 0 && L < t_max) {
    p.split_tiles = (int32_t)L;
    p.num_splits = (int32_t)((t_max + L - 1) / L);
    p.ws_rows = rows;
    p.o_bytes = ((size_t)p.num_splits * rows * d * sizeof(float) + 255) / 256 * 256;
    p.ml_bytes = (size_t)p.num_splits * rows * 2 * sizeof(float);
  }
  return p;
}

// Checks a caller's workspace against a plan: NULL runs the single pass.
int use_workspace(PrefillPlan& p, void* workspace, size_t workspace_bytes, PrefillArgs& a, const char* fn) {
  a.num_splits = 1;
  if (p.num_splits <= 1 || !workspace) return ATTN_OK;
  if (!aligned(workspace, 256)) return fail(ATTN_E_INVALID, "%s: workspace must be 256-byte aligned", fn);
  const size_t need = p.o_bytes + p.ml_bytes;
  if (workspace_bytes < need) return fail(ATTN_E_NOMEM, "%s: workspace %zu bytes, %zu needed", fn, workspace_bytes, need);
  a.num_splits = p.num_splits;
  a.split_tiles = p.split_tiles;
  a.ws_rows = p.ws_rows;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.o_bytes);
  return ATTN_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
extern "C" size_t attn_prefill_workspace_size(int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                              attn_dtype dtype) {
  if (dtype != ATTN_BF16 || batch <= 0 || seqlen_q <= 0 || seqlen_k <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || (head_dim != 64 && head_dim != 128))
    return 0;
  const PrefillPlan p = plan_prefill(seqlen_q, seqlen_k, num_q_heads, num_q_heads / num_kv_heads, batch, head_dim,
                                     false, (int64_t)batch * seqlen_q * num_q_heads);
  return p.o_bytes + p.ml_bytes;
}

extern "C" size_t attn_prefill_paged_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                                    int32_t max_context_len, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim) {
  if (num_seqs <= 0 || total_q <= 0 || max_seqlen_q <= 0 || max_context_len <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || (head_dim != 64 && head_dim != 128))
    return 0;
  const PrefillPlan p = plan_prefill(max_seqlen_q, max_context_len, num_q_heads, num_q_heads / num_kv_heads,
                                     num_seqs, head_dim, true, (int64_t)total_q * num_q_heads);
  return p.o_bytes + p.ml_bytes;
}

// ---------------------------------------------------------------------------
namespace {
int prefill_common(const char* fn, const void* q, const void* k, const void* v, void* o, float* lse,
                   const float* mask, const int64_t* mask_strides, int32_t batch, int32_t seqlen_q,
                   int32_t seqlen_k, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   const int64_t q_strides[3], const int64_t k_strides[3], const int64_t v_strides[3],
                   const int64_t o_strides[3], float scale, int32_t causal, attn_dtype dtype, void* workspace,
                   size_t workspace_bytes, attn_stream_t stream) {
  if (!q || !k || !v || !o) return fail(ATTN_E_INVALID, "%s: q, k, v and o must be non-NULL", fn);
  if (!q_strides || !k_strides || !v_strides || !o_strides)
    return fail(ATTN_E_INVALID, "%s: stride arrays must be non-NULL", fn);
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0) return fail(ATTN_E_INVALID, "%s: negative size", fn);
  int st;
  if ((st = check_heads(num_q_heads, num_kv_heads, fn)) != ATTN_OK) return st;
  if ((st = check_head_dim(head_dim, fn)) != ATTN_OK) return st;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_E_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (causal && seqlen_k < seqlen_q)
    return fail(ATTN_E_INVALID, "%s: causal needs seqlen_k >= seqlen_q (%d < %d)", fn, seqlen_k, seqlen_q);
  float scale_log2;
  if ((st = check_scale(scale, head_dim, &scale_log2, fn)) != ATTN_OK) return st;
  const int64_t mult = dtype == ATTN_BF16 ? 8 : 4;
  const void* ptrs[] = {q, k, v, o};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(ATTN_E_INVALID, "%s: tensor pointers must be 16-byte aligned", fn);
  if (lse && !aligned(lse, 4)) return fail(ATTN_E_INVALID, "%s: lse must be 4-byte aligned", fn);
  const int64_t* strides[] = {q_strides, k_strides, v_strides, o_strides};
  for (const int64_t* sa : strides)
    for (int i = 0; i < 3; ++i)
      if (sa[i] < 0 || sa[i] % mult != 0)
        return fail(ATTN_E_INVALID, "%s: strides must be >= 0 and multiples of %lld elements", fn, (long long)mult);
  // the bf16 kernel forms each lane's key/value load address as a 32-bit
  // byte offset from a row base: up to 7 token strides of 2 bytes
  if (dtype == ATTN_BF16 && (k_strides[1] >= (int64_t(1) << 28) || v_strides[1] >= (int64_t(1) << 28)))
    return fail(ATTN_E_UNSUPPORTED, "%s: key/value token strides must be below 2^28 elements", fn);
  if (mask != nullptr) {
    // the kernels read four consecutive mask floats with one 16-byte load
    if (!aligned(mask, 16)) return fail(ATTN_E_INVALID, "%s: mask must be 16-byte aligned", fn);
    for (int i = 0; i < 3; ++i)
      if (mask_strides[i] < 0 || mask_strides[i] % 4 != 0)
        return fail(ATTN_E_INVALID, "%s: mask strides must be >= 0 and multiples of 4 elements", fn);
  }
  if (batch == 0 || seqlen_q == 0) return ok();

  PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.qs_b = q_strides[0]; a.qs_t = q_strides[1]; a.qs_h = q_strides[2];
  a.ks_b = k_strides[0]; a.ks_t = k_strides[1]; a.ks_h = k_strides[2];
  a.vs_b = v_strides[0]; a.vs_t = v_strides[1]; a.vs_h = v_strides[2];
  a.os_b = o_strides[0]; a.os_t = o_strides[1]; a.os_h = o_strides[2];
  a.batch = batch; a.tq = seqlen_q; a.tk = seqlen_k;
  a.hq = num_q_heads; a.hkv = num_kv_heads; a.group = num_q_heads / num_kv_heads;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = scale_log2;
  if (mask != nullptr) {
    a.mask = mask;
    a.ms_b = mask_strides[0]; a.ms_h = mask_strides[1]; a.ms_q = mask_strides[2];
    a.mask_scale = (float)((double)kLog2eHost / (double)scale_log2);  // 1 / scale
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16) {
    PrefillPlan p = plan_prefill(seqlen_q, seqlen_k, num_q_heads, a.group, batch, head_dim, false,
                                 (int64_t)batch * seqlen_q * num_q_heads);
    if (mask != nullptr) {
      // one pass on the default tile (the masked kernel's only shapes)
      p.t = PrefillTile{a.group % 2 == 0 ? 2 : 1, a.group % 2 == 0 ? 2 : 4};
      p.num_m_tiles = ceil_div(seqlen_q, 32 * p.t.wph);
      p.num_wg = (int64_t)p.num_m_tiles * (num_q_heads / p.t.hpw) * batch;
      p.num_splits = 1;
    }
    if ((st = use_workspace(p, workspace, workspace_bytes, a, fn)) != ATTN_OK) return st;
    a.num_m_tiles = p.num_m_tiles;
    if (p.num_wg * a.num_splits > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "%s: problem too large for one launch", fn);
    a.num_wg = (uint32_t)p.num_wg;
    return launched(launch_prefill_bf16(a, head_dim, false, p.t.hpw, p.t.wph, false, s), fn);
  }
  a.num_splits = 1;
  a.num_m_tiles = ceil_div(seqlen_q, kPrefillF32BlockM);
  const int64_t nwg = (int64_t)a.num_m_tiles * num_q_heads * batch;
  if (nwg > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "%s: problem too large for one launch", fn);
  a.num_wg = (uint32_t)nwg;
  return launched(launch_prefill_f32(a, head_dim, false, s), fn);
}
}  // namespace

extern "C" int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                            int32_t batch, int32_t seqlen_q, int32_t seqlen_k,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t v_strides[3], const int64_t o_strides[3],
                            float scale, int32_t causal, attn_dtype dtype,
                            void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  return prefill_common("attn_prefill", q, k, v, o, lse, nullptr, nullptr, batch, seqlen_q, seqlen_k,
                        num_q_heads, num_kv_heads, head_dim, q_strides, k_strides, v_strides, o_strides, scale,
                        causal, dtype, workspace, workspace_bytes, stream);
}

extern "C" int attn_prefill_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const float* mask, const int64_t mask_strides[3], int32_t batch,
                                   int32_t seqlen_q, int32_t seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, const int64_t q_strides[3], const int64_t k_strides[3],
                                   const int64_t v_strides[3], const int64_t o_strides[3], float scale,
                                   int32_t causal, attn_dtype dtype, attn_stream_t stream) {
  static const char* fn = "attn_prefill_masked";
  if (!mask || !mask_strides) return fail(ATTN_E_INVALID, "%s: mask and mask_strides must be non-NULL", fn);
  return prefill_common(fn, q, k, v, o, lse, mask, mask_strides, batch, seqlen_q, seqlen_k, num_q_heads,
                        num_kv_heads, head_dim, q_strides, k_strides, v_strides, o_strides, scale, causal, dtype,
                        nullptr, 0, stream);
}

// ---------------------------------------------------------------------------
extern "C" int attn_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                  void* o, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                  int32_t max_context_len,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks,
                                  float scale, int32_t causal, attn_dtype dtype,
                                  void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  return attn_prefill_paged_ex(q, k_cache, v_cache, block_table, max_blocks_per_seq, cu_seqlens_q, context_lens, o,
                               num_seqs, total_q, max_seqlen_q, max_context_len, num_q_heads, num_kv_heads,
                               head_dim, block_size, num_blocks, scale, causal, dtype, 0, workspace,
                               workspace_bytes, stream);
}

namespace {
// Paged mask: row of packed query row r and head h at mask + r*ms[0] + h*ms[1],
// mask_keys entries each.
struct PagedMask {
  const float* mask;
  const int64_t* strides;
  int32_t keys;
};

int prefill_paged_common(const char* fn, const PagedMask* pm, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* cu_seqlens_q, const int32_t* context_lens, void* o, int32_t num_seqs,
                         int32_t total_q, int32_t max_seqlen_q, int32_t max_context_len, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                         int32_t causal, attn_dtype dtype, int32_t flags, void* workspace, size_t workspace_bytes,
                         attn_stream_t stream, PrefillArgs* prep = nullptr, int* prep_hpw = nullptr) {
  // prep: validate and fill *prep (bf16, no mask, no split) instead of
  // launching; num_wg 0 when there is nothing to compute
  if (prep != nullptr) {
    *prep = PrefillArgs{};
    *prep_hpw = 0;
    if (dtype != ATTN_BF16 || pm != nullptr || flags != 0 || workspace != nullptr)
      return fail(ATTN_E_UNSUPPORTED, "%s: the prefill part runs in bf16, unmasked, without split-KV", fn);
  }
  if ((flags & ~ATTN_PREFILL_SHARE_CU) != 0) return fail(ATTN_E_INVALID, "%s: unknown flags 0x%x", fn, flags);
  if (!q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !context_lens || !o)
    return fail(ATTN_E_INVALID, "%s: pointer arguments must be non-NULL", fn);
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_context_len < 0 || max_blocks_per_seq < 1 ||
      num_blocks < 1)
    return fail(ATTN_E_INVALID, "%s: bad size", fn);
  if (max_seqlen_q > total_q) return fail(ATTN_E_INVALID, "%s: max_seqlen_q > total_q", fn);
  int st;
  if ((st = check_heads(num_q_heads, num_kv_heads, fn)) != ATTN_OK) return st;
  if ((st = check_head_dim(head_dim, fn)) != ATTN_OK) return st;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return fail(ATTN_E_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (block_size != kBlockSizeHost) return fail(ATTN_E_UNSUPPORTED, "%s: block_size %d (supported: 16)", fn, block_size);
  float scale_log2;
  if ((st = check_scale(scale, head_dim, &scale_log2, fn)) != ATTN_OK) return st;
  const void* ptrs[] = {q, k_cache, v_cache, o};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(ATTN_E_INVALID, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned(block_table, 4) || !aligned(cu_seqlens_q, 4) || !aligned(context_lens, 4))
    return fail(ATTN_E_INVALID, "%s: int32 arrays must be 4-byte aligned", fn);
  if (pm != nullptr) {
    if (!pm->mask || !pm->strides) return fail(ATTN_E_INVALID, "%s: mask and mask_strides must be non-NULL", fn);
    // the kernels read four consecutive mask floats with one 16-byte load
    if (!aligned(pm->mask, 16)) return fail(ATTN_E_INVALID, "%s: mask must be 16-byte aligned", fn);
    for (int i = 0; i < 2; ++i)
      if (pm->strides[i] < 0 || pm->strides[i] % 4 != 0)
        return fail(ATTN_E_INVALID, "%s: mask strides must be >= 0 and multiples of 4 elements", fn);
    if (pm->keys < 0) return fail(ATTN_E_INVALID, "%s: mask_keys must be >= 0", fn);
  }
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();

  PrefillArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = nullptr;
  a.batch = num_seqs;
  a.hq = num_q_heads; a.hkv = num_kv_heads; a.group = num_q_heads / num_kv_heads;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = scale_log2;
  if (dtype == ATTN_F32) {
    // fp32: the VALU kernel, one pass per 64-query tile and head (no
    // split, no flags; the workspace is not used)
    if (pm != nullptr) {
      a.mask = pm->mask;
      a.ms_q = pm->strides[0]; a.ms_h = pm->strides[1]; a.ms_b = 0;
      a.mask_keys = pm->keys;
      a.mask_scale = (float)((double)kLog2eHost / (double)scale_log2);
    }
    a.num_splits = 1;
    a.num_m_tiles = ceil_div(max_seqlen_q, kPrefillF32BlockM);
    const int64_t nwg = (int64_t)a.num_m_tiles * num_q_heads * num_seqs;
    if (nwg > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "%s: problem too large for one launch", fn);
    a.num_wg = (uint32_t)nwg;
    a.block_table = block_table; a.bt_stride = max_blocks_per_seq;
    a.cu_seqlens_q = cu_seqlens_q; a.context_lens = context_lens;
    a.num_blocks = num_blocks;
    a.total_q = total_q;
    return launched(launch_prefill_f32(a, head_dim, true, reinterpret_cast<hipStream_t>(stream)), fn);
  }
  // the plan's key bound: the caller's, else what the block table can hold
  const int64_t ctx_bound = max_context_len > 0 ? max_context_len : (int64_t)max_blocks_per_seq * kBlockSizeHost;
  PrefillPlan p = plan_prefill(max_seqlen_q, ctx_bound, num_q_heads, a.group, num_seqs, head_dim, true,
                               (int64_t)total_q * num_q_heads, (flags & ATTN_PREFILL_SHARE_CU) != 0);
  if (pm != nullptr) {
    // one pass on the default tile (the masked kernel's only shapes)
    a.mask = pm->mask;
    a.ms_q = pm->strides[0]; a.ms_h = pm->strides[1]; a.ms_b = 0;
    a.mask_keys = pm->keys;
    a.mask_scale = (float)((double)kLog2eHost / (double)scale_log2);  // 1 / scale
    p.t = prefill_tile(a.group);
    p.deep_v = false;
    p.num_m_tiles = ceil_div(max_seqlen_q, 32 * p.t.wph);
    p.num_wg = (int64_t)p.num_m_tiles * (num_q_heads / p.t.hpw) * num_seqs;
    p.num_splits = 1;
  }
  if ((st = use_workspace(p, workspace, workspace_bytes, a, fn)) != ATTN_OK) return st;
  a.num_m_tiles = p.num_m_tiles;
  if (p.num_wg * a.num_splits > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "%s: problem too large for one launch", fn);
  a.num_wg = (uint32_t)p.num_wg;
  a.block_table = block_table; a.bt_stride = max_blocks_per_seq;
  a.cu_seqlens_q = cu_seqlens_q; a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.total_q = total_q;
  if (prep != nullptr) {
    *prep = a;
    *prep_hpw = p.t.hpw;
    return ok();
  }
  return launched(launch_prefill_bf16(a, head_dim, true, p.t.hpw, p.t.wph, p.deep_v,
                                      reinterpret_cast<hipStream_t>(stream)), fn);
}
}  // namespace

extern "C" int attn_prefill_paged_ex(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                     void* o, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                     int32_t max_context_len,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks,
                                     float scale, int32_t causal, attn_dtype dtype, int32_t flags,
                                     void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  return prefill_paged_common("attn_prefill_paged", nullptr, q, k_cache, v_cache, block_table, max_blocks_per_seq,
                              cu_seqlens_q, context_lens, o, num_seqs, total_q, max_seqlen_q, max_context_len,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, causal, dtype,
                              flags, workspace, workspace_bytes, stream);
}

extern "C" int attn_prefill_paged_masked(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, int32_t max_blocks_per_seq,
                                         const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                         const float* mask, const int64_t mask_strides[2], int32_t mask_keys,
                                         void* o, int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                         int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                         int32_t causal, attn_dtype dtype, attn_stream_t stream) {
  const PagedMask pm{mask, mask_strides, mask_keys};
  return prefill_paged_common("attn_prefill_paged_masked", &pm, q, k_cache, v_cache, block_table,
                              max_blocks_per_seq, cu_seqlens_q, context_lens, o, num_seqs, total_q, max_seqlen_q,
                              max_context_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                              causal, dtype, 0, nullptr, 0, stream);
}

// ---------------------------------------------------------------------------
extern "C" int32_t attn_decode_paged_auto_partition(int32_t num_seqs, int32_t num_kv_heads,
                                                    int32_t max_context_len) {
  // Largest partition from {1024, 768, 512, 384, 256, 128} tokens that
  // still gives enough partition workgroups if every sequence were as long
  // as the longest: about 512 (two per CU), or 1024 for the 1024-token
  // partition.  Measured on MI355X: 128 sequences with contexts up to 32768
  // decode in the same time at 768 and 1024 (130 us) and a serving step that
  // runs that decode beside a chunked prefill is faster at 1024 (190 vs
  // 194 us); 64 sequences up to 4096 tokens are faster at 768 (36.7 vs
  // 39.0 us); smaller partitions keep the CUs busy when contexts are short.
  static const int32_t cand[] = {1024, 768, 512, 384, 256, 128};
  const int64_t units = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  for (int32_t p : cand)
    if (units * ((ctx + p - 1) / p) >= (p == 1024 ? 1024 : 512)) return p;
  return 128;
}

extern "C" int32_t attn_decode_paged_partition_for(const int32_t* context_lens, int32_t num_seqs,
                                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  static const char* fn = "attn_decode_paged_partition_for";
  if (num_seqs < 0 || (num_seqs > 0 && !context_lens) || num_kv_heads < 1 || num_q_heads < num_kv_heads ||
      num_q_heads % num_kv_heads != 0 || (head_dim != 64 && head_dim != 128))
    return fail(ATTN_E_INVALID, "%s: bad argument", fn);
  // Workgroups resident at once: the decode kernel holds two per CU at
  // head_dim 128 (232 VGPRs per wavefront) and four at 64.  A sweep on MI355X
  // over six batches (16 to 256 sequences, contexts up to 16384) found the
  // fastest partition to be the shortest one whose items all fit in one round,
  // or within 2 % of it (64 sequences U[128, 4096]: 640 tokens, 32.9 us,
  // against 34.5 at 768 and 36.5 at 512, whose 566 workgroups need a second
  // round).
  const int64_t slots = (int64_t)kCUs * (head_dim == 128 ? 2 : 4);
  const int64_t per_item = (int64_t)num_kv_heads * ((num_q_heads / num_kv_heads + 15) / 16);
  for (int32_t p = 128; p <= 1024; p += 128) {
    int64_t items = 0;
    for (int32_t s = 0; s < num_seqs; ++s) items += (std::max(context_lens[s], 0) + p - 1) / p;
    if (items * per_item <= slots) {
      ok();
      return p;
    }
  }
  ok();
  return 1024;
}

namespace {
constexpr int32_t kMaxF32Partition = 65536;
// Decode workspace, used only when a context can span several partitions:
// the arrival counters (one int32 per sequence and kv head slice, zero
// between calls), then the partial outputs, then the (m, l) pairs.  The
// counter block has room for the most sequences a call may have (65535)
// with the call's head geometry, so where it ends does not depend on the
// sequence count: a later call with more sequences finds its counters where
// only counters ever were, not where an earlier, smaller call left partials.
// The fixed scratch of attn_decode_paged_noalloc, shared by calls of every
// geometry, begins with a block of its own for up to 16 slices.
constexpr int64_t kMaxDecodeSeqs = 65535;
constexpr size_t kScratchCounterBytes = size_t(kMaxDecodeSeqs) * 16 * sizeof(int32_t) / 256 * 256 + 256;
struct DecodeGeom {
  int32_t part, max_parts;
  size_t cnt_bytes, o_bytes, ml_bytes;
  size_t total() const { return cnt_bytes + o_bytes + ml_bytes; }
};

DecodeGeom decode_geom(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t max_ctx, int32_t part) {
  DecodeGeom gm{};
  gm.part = part > 0 ? part : attn_decode_paged_auto_partition(num_seqs, hkv, max_ctx);
  gm.max_parts = ceil_div(max_ctx, gm.part);
  if (gm.max_parts > 1) {
    const size_t slices = (size_t)hkv * ceil_div(hq / hkv, 16);
    gm.cnt_bytes = ((size_t)kMaxDecodeSeqs * slices * sizeof(int32_t) + 255) / 256 * 256;
    const size_t rows = (size_t)num_seqs * hq * gm.max_parts;
    gm.o_bytes = (rows * d * sizeof(float) + 255) / 256 * 256;
    gm.ml_bytes = rows * 2 * sizeof(float);
  }
  return gm;
}
}  // namespace

extern "C" size_t attn_decode_paged_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t max_context_len,
                                                   int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len <= 0 ||
      partition_size < 0)
    return 0;
  DecodeGeom gm = decode_geom(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size);
  return gm.total();
}

extern "C" int64_t attn_decode_paged_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                          int32_t max_context_len, int32_t partition_size, int32_t* items,
                                          int64_t capacity) {
  static const char* fn = "attn_decode_paged_plan";
  if (num_seqs < 0 || num_kv_heads < 1 || max_context_len < 1 || capacity < 0 || (num_seqs > 0 && !context_lens))
    return fail(ATTN_E_INVALID, "%s: bad argument", fn);
  if (partition_size < 0 || partition_size % 16 != 0 || partition_size > kMaxF32Partition)
    return fail(ATTN_E_INVALID, "%s: partition_size must be 0 or a multiple of 16 up to %d", fn, kMaxF32Partition);
  const int32_t part = partition_size > 0 ? partition_size
                                          : attn_decode_paged_auto_partition(num_seqs, num_kv_heads, max_context_len);
  // the kernel's own view of a context: clamped to max_context_len
  auto parts_of = [&](int32_t s) {
    const int64_t ctx = std::min<int64_t>(std::max(context_lens[s], 0), max_context_len);
    return (ctx + part - 1) / part;
  };
  int64_t count = 0;
  for (int32_t s = 0; s < num_seqs; ++s) count += parts_of(s);
  if (items == nullptr || capacity < count) {
    ok();
    return count;
  }
  // longest sequences first: their partitions start together
  std::vector<int32_t> order(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) order[s] = s;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return parts_of(x) > parts_of(y); });
  int64_t k = 0;
  for (int32_t s : order)
    for (int64_t p = 0; p < parts_of(s); ++p) {
      items[2 * k] = s;
      items[2 * k + 1] = (int32_t)p;
      ++k;
    }
  ok();
  return count;
}

namespace {
// The new token of each sequence, rotated and written by the decode launch
// itself (attn_decode_paged_rope); null for attn_decode_paged.
struct DecodeWrite {
  void* q_rot_out;
  const void* k_new;
  const void* v_new;
  const int32_t* positions;
  const int32_t* slot_mapping;
  float rope_base;
};

// The fused write's own arguments (the new tokens of attn_decode_paged_rope).
int check_decode_write(const char* fn, const DecodeWrite& w, const void* q, int32_t num_blocks) {
  if (!w.k_new || !w.v_new || !w.positions || !w.slot_mapping)
    return fail(ATTN_E_INVALID, "%s: k_new, v_new, positions and slot_mapping must be non-NULL", fn);
  if (!std::isfinite(w.rope_base) || w.rope_base < 0.f || (w.rope_base > 0.f && w.rope_base <= 1.f))
    return fail(ATTN_E_INVALID, "%s: rope_base must be 0 (no rotation) or > 1", fn);
  if (!aligned(w.k_new, 16) || !aligned(w.v_new, 16) || (w.q_rot_out && !aligned(w.q_rot_out, 16)))
    return fail(ATTN_E_INVALID, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned(w.positions, 4) || !aligned(w.slot_mapping, 4))
    return fail(ATTN_E_INVALID, "%s: int32 arrays must be 4-byte aligned", fn);
  if (w.q_rot_out != nullptr && w.q_rot_out == q)
    return fail(ATTN_E_INVALID, "%s: q_rot_out must not alias q (other workgroups still read q)", fn);
  if ((int64_t)num_blocks * kBlockSizeHost > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "%s: pool too large", fn);
  return ATTN_OK;
}

// use_scratch: the workspace is the library's fixed device scratch
// (attn_decode_paged_noalloc); workspace / workspace_bytes are ignored.
int decode_common(const char* fn, const DecodeWrite* w, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* context_lens, void* o, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                  int32_t partition_size, float scale, attn_dtype dtype, const int32_t* plan,
                  int32_t plan_items, void* workspace, size_t workspace_bytes, attn_stream_t stream,
                  bool use_scratch = false, DecodeArgs* prep = nullptr) {
  // prep: validate and fill *prep (bf16) instead of launching; num_seqs 0
  // when there is nothing to compute
  if (prep != nullptr) {
    *prep = DecodeArgs{};
    if (dtype != ATTN_BF16 || use_scratch) return fail(ATTN_E_UNSUPPORTED, "%s: the decode part runs in bf16", fn);
  }
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !o)
    return fail(ATTN_E_INVALID, "%s: pointer arguments must be non-NULL", fn);
  if (num_seqs < 0 || num_blocks < 1 || max_context_len < 1)
    return fail(ATTN_E_INVALID, "%s: bad size", fn);
  int st;
  if ((st = check_heads(num_q_heads, num_kv_heads, fn)) != ATTN_OK) return st;
  if ((st = check_head_dim(head_dim, fn)) != ATTN_OK) return st;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return fail(ATTN_E_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (dtype == ATTN_F32 && w != nullptr)
    return fail(ATTN_E_UNSUPPORTED, "%s: the decode with the new token's write fused takes bf16 only", fn);
  if (block_size != kBlockSizeHost) return fail(ATTN_E_UNSUPPORTED, "%s: block_size %d (supported: 16)", fn, block_size);
  if (max_blocks_per_seq < ceil_div(max_context_len, kBlockSizeHost))
    return fail(ATTN_E_INVALID, "%s: max_blocks_per_seq %d cannot hold max_context_len %d", fn,
                max_blocks_per_seq, max_context_len);
  if (dtype == ATTN_BF16 && (partition_size < 0 || partition_size % 16 != 0 || partition_size > 1024))
    return fail(ATTN_E_INVALID, "%s: bf16 partition_size must be 0 or a multiple of 16 up to 1024", fn);
  if (dtype == ATTN_F32 && (partition_size < 0 || partition_size % 16 != 0 || partition_size > kMaxF32Partition))
    return fail(ATTN_E_INVALID, "%s: fp32 partition_size must be 0 or a multiple of 16 up to %d", fn,
                kMaxF32Partition);
  float scale_log2;
  if ((st = check_scale(scale, head_dim, &scale_log2, fn)) != ATTN_OK) return st;
  const void* ptrs[] = {q, k_cache, v_cache, o};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(ATTN_E_INVALID, "%s: tensor pointers must be 16-byte aligned", fn);
  if (!aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(plan, 4))
    return fail(ATTN_E_INVALID, "%s: int32 arrays must be 4-byte aligned", fn);
  if (plan_items < 0 || (plan == nullptr && plan_items != 0))
    return fail(ATTN_E_INVALID, "%s: plan_items must be >= 0, and 0 without a plan", fn);
  DecodeGeom gm = decode_geom(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size);
  if (plan != nullptr && (int64_t)plan_items > (int64_t)num_seqs * gm.max_parts)
    return fail(ATTN_E_INVALID, "%s: plan_items %d exceeds num_seqs x partitions", fn, plan_items);
  if (use_scratch && gm.max_parts > 1) {
    if ((size_t)num_kv_heads * ceil_div(num_q_heads / num_kv_heads, 16) > 16)
      return fail(ATTN_E_NOMEM, "%s: the fixed scratch holds arrival counters for at most 16 kv head slices "
                  "(kv heads x ceil(query heads per kv head / 16))", fn);
    gm.cnt_bytes = kScratchCounterBytes;
  }
  const size_t need = gm.total();
  if (use_scratch) {
    if (need > kDecodeScratchBytes)
      return fail(ATTN_E_NOMEM, "%s: the call needs %zu bytes of scratch, above the fixed %zu (fewer sequences, or "
                  "a larger partition_size, fit)", fn, need, kDecodeScratchBytes);
  } else if (need > 0) {
    if (!workspace) return fail(ATTN_E_INVALID, "%s: workspace of %zu bytes required", fn, need);
    if (!aligned(workspace, 256)) return fail(ATTN_E_INVALID, "%s: workspace must be 256-byte aligned", fn);
    if (workspace_bytes < need)
      return fail(ATTN_E_NOMEM, "%s: workspace %zu bytes, %zu needed", fn, workspace_bytes, need);
  }
  if ((int64_t)plan_items * num_kv_heads * ceil_div(num_q_heads / num_kv_heads, 16) > INT32_MAX)
    return fail(ATTN_E_UNSUPPORTED, "%s: plan too large for one launch", fn);
  if ((int64_t)num_kv_heads * ceil_div(num_q_heads / num_kv_heads, 16) > 65535 || num_seqs > kMaxDecodeSeqs)
    return fail(ATTN_E_UNSUPPORTED, "%s: at most 65535 sequences (and kv head slices) per call", fn);
  if (num_seqs == 0) return ok();
  if (use_scratch && need > 0) {
    const hipError_t e = decode_scratch(reinterpret_cast<hipStream_t>(stream), &workspace);
    if (e != hipSuccess) return fail(ATTN_E_DEVICE, "%s: decode scratch: %s", fn, hipGetErrorString(e));
  }
  const int32_t group = num_q_heads / num_kv_heads;
  DecodeArgs a{};
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_table = block_table; a.bt_stride = max_blocks_per_seq;
  a.context_lens = context_lens; a.o = o;
  char* ws = static_cast<char*>(workspace);
  a.counters = need ? reinterpret_cast<int32_t*>(ws) : nullptr;
  a.ws_o = need ? reinterpret_cast<float*>(ws + gm.cnt_bytes) : nullptr;
  a.ws_ml = need ? reinterpret_cast<float*>(ws + gm.cnt_bytes + gm.o_bytes) : nullptr;
  a.num_seqs = num_seqs; a.hq = num_q_heads; a.hkv = num_kv_heads;
  a.group = group; a.head_groups = ceil_div(group, 16);
  a.part_size = gm.part; a.max_parts = gm.max_parts;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale_log2;
  a.plan = plan;
  a.plan_items = plan_items;
  if (w != nullptr) {
    a.q_rot_out = w->q_rot_out;
    a.k_new = w->k_new;
    a.v_new = w->v_new;
    a.positions = w->positions;
    a.slot_mapping = w->slot_mapping;
    a.rope = w->rope_base > 0.f;
    if (a.rope) a.freqs = rope_freqs(w->rope_base, head_dim);
  }
  if (prep != nullptr) {
    *prep = a;
    return ok();
  }
  if (dtype == ATTN_F32) return launched(launch_decode_f32(a, head_dim, reinterpret_cast<hipStream_t>(stream)), fn);
  return launched(launch_decode(a, head_dim, w != nullptr, reinterpret_cast<hipStream_t>(stream)), fn);
}
}  // namespace

extern "C" int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* context_lens, void* o,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 int32_t partition_size, float scale, attn_dtype dtype,
                                 const int32_t* plan, int32_t plan_items,
                                 void* workspace, size_t workspace_bytes, attn_stream_t stream) {
  return decode_common("attn_decode_paged", nullptr, q, k_cache, v_cache, block_table, context_lens, o, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, partition_size, scale, dtype, plan, plan_items, workspace, workspace_bytes,
                       stream);
}

extern "C" int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* context_lens, void* o,
                                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         int32_t partition_size, float scale, attn_dtype dtype,
                                         const int32_t* plan, int32_t plan_items, attn_stream_t stream) {
  return decode_common("attn_decode_paged_noalloc", nullptr, q, k_cache, v_cache, block_table, context_lens, o,
                       num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, partition_size, scale, dtype, plan, plan_items, nullptr, 0, stream, true);
}

extern "C" int attn_decode_paged_rope(void* q_rot_out, const void* q, const void* k_new, const void* v_new,
                                      const int32_t* positions, const int32_t* slot_mapping, float rope_base,
                                      void* k_cache, void* v_cache, const int32_t* block_table,
                                      const int32_t* context_lens, void* o, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                                      int32_t partition_size, float scale, attn_dtype dtype, const int32_t* plan,
                                      int32_t plan_items, void* workspace, size_t workspace_bytes,
                                      attn_stream_t stream) {
  static const char* fn = "attn_decode_paged_rope";
  const DecodeWrite w{q_rot_out, k_new, v_new, positions, slot_mapping, rope_base};
  int st;
  if ((st = check_decode_write(fn, w, q, num_blocks)) != ATTN_OK) return st;
  return decode_common(fn, &w, q, k_cache, v_cache, block_table, context_lens, o, num_seqs, num_q_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                       partition_size, scale, dtype, plan, plan_items, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Mixed launch: the interleave of prefill and decode workgroups in its grid.
// Measured on MI355X with 8 chunks of 512 new tokens (384 prefill
// workgroups) beside a 128-sequence decode (1390 workgroups), RoPE write
// included, us per step: groups of 32 prefill and 64 decode workgroups
// 172-177 against 189-194 for the two-launch, two-stream step; 32 + 32
// 175-178, 16 + 16 184, all prefill first 177-180.  With the prefill's waves
// at raised priority (mixed.hip), same box, configurations interleaved:
// 32 + 72 169.0, 32 + 56 169.4, 32 + 64 171.6, 32 + 80 171.2, 24 + 48 171.2,
// 24 + 56 174.2; spreading the prefill thinner (16 + 64, 32 + 128) 199.
constexpr int32_t kMixedPrefillPerGroup = 32;
constexpr int32_t kMixedDecodePerGroup = 72;

extern "C" int attn_prefill_decode_paged(const attn_paged_prefill_part* prefill, const attn_paged_decode_part* decode,
                                         void* k_cache, void* v_cache, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                         int32_t num_blocks, float scale, attn_dtype dtype, attn_stream_t stream) {
  static const char* fn = "attn_prefill_decode_paged";
  if (!prefill || !decode) return fail(ATTN_E_INVALID, "%s: prefill and decode must be non-NULL", fn);
  if (dtype != ATTN_BF16) return fail(ATTN_E_UNSUPPORTED, "%s: bf16 only", fn);
  // a part with num_seqs 0 is absent (its other fields are not read)
  PrefillArgs pa{};
  int hpw = 0;
  int st = ATTN_OK;
  if (prefill->num_seqs != 0)
    st = prefill_paged_common(fn, nullptr, prefill->q, k_cache, v_cache, prefill->block_table,
                              prefill->max_blocks_per_seq, prefill->cu_seqlens_q, prefill->context_lens, prefill->o,
                              prefill->num_seqs, prefill->total_q, prefill->max_seqlen_q, prefill->max_context_len,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, prefill->causal,
                              dtype, 0, nullptr, 0, stream, &pa, &hpw);
  if (st != ATTN_OK) return st;
  const bool fused = decode->k_new != nullptr || decode->v_new != nullptr || decode->positions != nullptr ||
                     decode->slot_mapping != nullptr;
  const DecodeWrite w{decode->q_rot_out, decode->k_new, decode->v_new, decode->positions, decode->slot_mapping,
                      decode->rope_base};
  if (decode->num_seqs != 0 && fused && (st = check_decode_write(fn, w, decode->q, num_blocks)) != ATTN_OK) return st;
  if (decode->num_seqs != 0 && !fused && decode->q_rot_out != nullptr)
    return fail(ATTN_E_INVALID, "%s: q_rot_out needs the fused write's arguments", fn);
  DecodeArgs da{};
  if (decode->num_seqs != 0)
    st = decode_common(fn, fused ? &w : nullptr, decode->q, k_cache, v_cache, decode->block_table,
                       decode->context_lens, decode->o, decode->num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, decode->max_blocks_per_seq, decode->max_context_len,
                       decode->partition_size, scale, dtype, decode->plan, decode->plan_items, decode->workspace,
                       decode->workspace_bytes, stream, false, &da);
  if (st != ATTN_OK) return st;
  MixedSched m{};
  m.n_pre = (int32_t)pa.num_wg;
  if (da.num_seqs > 0) {
    const int64_t Y = (int64_t)da.hkv * da.head_groups;
    const int64_t n = da.plan != nullptr ? (int64_t)da.plan_items * Y : (int64_t)(da.max_parts | 1) * Y * da.num_seqs;
    if (n > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "%s: problem too large for one launch", fn);
    m.n_dec = (int32_t)n;
  }
  m.gp = kMixedPrefillPerGroup;
  m.gd = kMixedDecodePerGroup;
  m.groups = ceil_div(m.n_pre, m.gp);
  if ((int64_t)m.groups * (m.gp + m.gd) + m.n_dec > INT32_MAX)
    return fail(ATTN_E_UNSUPPORTED, "%s: problem too large for one launch", fn);
  if (hpw == 0) hpw = prefill_tile(num_q_heads / num_kv_heads).hpw;  // no prefill part: any tile
  return launched(launch_mixed(pa, da, m, head_dim, hpw, fused, reinterpret_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
extern "C" int attn_kv_cache_write_rope(void* q, const void* k, const void* v, const int32_t* positions,
                                        const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                        int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        float rope_base, attn_dtype dtype, attn_stream_t stream) {
  static const char* fn = "attn_kv_cache_write_rope";
  if (!k || !v || !positions || !slot_mapping || !k_cache || !v_cache)
    return fail(ATTN_E_INVALID, "%s: pointer arguments (except q) must be non-NULL", fn);
  if (num_tokens < 0 || num_blocks < 1) return fail(ATTN_E_INVALID, "%s: bad size", fn);
  int st;
  if ((st = check_heads(num_q_heads, num_kv_heads, fn)) != ATTN_OK) return st;
  if ((st = check_head_dim(head_dim, fn)) != ATTN_OK) return st;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_E_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (block_size != kBlockSizeHost) return fail(ATTN_E_UNSUPPORTED, "%s: block_size %d (supported: 16)", fn, block_size);
  if (!std::isfinite(rope_base) || rope_base < 0.f || (rope_base > 0.f && rope_base <= 1.f))
    return fail(ATTN_E_INVALID, "%s: rope_base must be 0 (no rotation) or > 1", fn);
  if ((int64_t)num_blocks * kBlockSizeHost > INT32_MAX) return fail(ATTN_E_UNSUPPORTED, "%s: pool too large", fn);
  const void* ptrs[] = {k, v, k_cache, v_cache};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(ATTN_E_INVALID, "%s: tensor pointers must be 16-byte aligned", fn);
  if (q && !aligned(q, 16)) return fail(ATTN_E_INVALID, "%s: q must be 16-byte aligned", fn);
  if (!aligned(positions, 4) || !aligned(slot_mapping, 4))
    return fail(ATTN_E_INVALID, "%s: int32 arrays must be 4-byte aligned", fn);
  if (num_tokens == 0) return ok();
  RopeWriteArgs a{};
  a.q = q; a.k = k; a.v = v; a.positions = positions; a.slot_mapping = slot_mapping;
  a.k_cache = k_cache; a.v_cache = v_cache;
  a.num_tokens = num_tokens; a.hq = num_q_heads; a.hkv = num_kv_heads;
  a.num_blocks = num_blocks;
  a.rope = rope_base > 0.f;
  if (a.rope) a.freqs = rope_freqs(rope_base, head_dim);
  return launched(launch_rope_write(a, head_dim, dtype == ATTN_BF16, reinterpret_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
extern "C" int attn_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                attn_dtype dtype, attn_stream_t stream) {
  static const char* fn = "attn_copy_blocks";
  if (!k_cache || !v_cache || (num_pairs > 0 && !pairs))
    return fail(ATTN_E_INVALID, "%s: k_cache, v_cache and pairs must be non-NULL", fn);
  if (num_pairs < 0 || num_blocks < 1 || num_kv_heads < 1) return fail(ATTN_E_INVALID, "%s: bad size", fn);
  int st;
  if ((st = check_head_dim(head_dim, fn)) != ATTN_OK) return st;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_E_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (block_size != kBlockSizeHost) return fail(ATTN_E_UNSUPPORTED, "%s: block_size %d (supported: 16)", fn, block_size);
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(ATTN_E_INVALID, "%s: cache pointers must be 16-byte aligned", fn);
  if (!aligned(pairs, 4)) return fail(ATTN_E_INVALID, "%s: pairs must be 4-byte aligned", fn);
  if (num_pairs == 0) return ok();
  CopyBlocksArgs a{};
  a.k_cache = k_cache; a.v_cache = v_cache; a.pairs = pairs;
  a.num_pairs = num_pairs; a.num_blocks = num_blocks;
  a.block_bytes = (int64_t)num_kv_heads * kBlockSizeHost * head_dim * (dtype == ATTN_BF16 ? 2 : 4);
  return launched(launch_copy_blocks(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
extern "C" int attn_residual_rms_norm(const void* x, const void* residual, const void* weight, void* y,
                                      void* residual_out, int32_t rows, int32_t hidden, float eps, attn_dtype dtype,
                                      attn_stream_t stream) {
  static const char* fn = "attn_residual_rms_norm";
  if (!x || !residual || !weight || !y || !residual_out)
    return fail(ATTN_E_INVALID, "%s: pointer arguments must be non-NULL", fn);
  if (rows < 0) return fail(ATTN_E_INVALID, "%s: rows < 0", fn);
  if (hidden < 8 || hidden % 8 != 0 || hidden > 8192)
    return fail(ATTN_E_UNSUPPORTED, "%s: hidden %d (supported: multiples of 8 up to 8192)", fn, hidden);
  if (!std::isfinite(eps) || eps < 0.f) return fail(ATTN_E_INVALID, "%s: eps must be finite and >= 0", fn);
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_E_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  const void* ptrs[] = {x, residual, weight, y, residual_out};
  for (const void* p : ptrs)
    if (!aligned(p, 16)) return fail(ATTN_E_INVALID, "%s: pointers must be 16-byte aligned", fn);
  if (y == x || y == residual || y == residual_out)
    return fail(ATTN_E_INVALID, "%s: y must not alias an input or residual_out", fn);
  if (rows == 0) return ok();
  RmsNormArgs a{};
  a.x = x; a.residual = residual; a.weight = weight; a.y = y; a.h_out = residual_out;
  a.rows = rows; a.hidden = hidden; a.eps = eps;
  return launched(launch_residual_rms_norm(a, dtype == ATTN_BF16, reinterpret_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
extern "C" int attn_debug_flags(uint32_t* flags_out, int clear) {
  static const char* fn = "attn_debug_flags";
  if (!flags_out) return fail(ATTN_E_INVALID, "%s: flags_out must be non-NULL", fn);
  *flags_out = 0;
#if MI_ATTN_DEBUG
  hipError_t e = hipDeviceSynchronize();
  uint32_t acc = 0;
  const bool c = clear != 0;
  if (e == hipSuccess) e = debug_take_prefill(&acc, c);
  if (e == hipSuccess) e = debug_take_decode(&acc, c);
  if (e == hipSuccess) e = debug_take_rope_write(&acc, c);
  if (e == hipSuccess) e = debug_take_copy_blocks(&acc, c);
  if (e == hipSuccess) e = debug_take_mixed(&acc, c);
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  *flags_out = acc;
  return ok();
#else
  (void)clear;
  return fail(ATTN_E_UNSUPPORTED, "%s: this is the release library (the debug one is built with MI_ATTN_DEBUG=1)",
              fn);
#endif
}
