// Copy of whole paged-cache blocks: the copy-on-write step of prefix sharing.
//
// "Fast Attention Kernels and Operator Fusion", §Paged Attention Kernels:
// sequences that begin with the same tokens may hold the same blocks.  A
// sequence that
// appends into a partly filled shared block first gets its own copy of that
// block (attn_seq_reserve_cow names the pair); this kernel makes the copies.
// One (block, pool) is contiguous, [Hkv][16][D] for keys and [Hkv][D][16]
// for values, so each is one run of bytes: workgroup = (pair, pool), 16-byte
// loads and stores, consecutive lanes on consecutive chunks.

#include "device_common.h"
#include "kernels.h"

namespace mi_attn {

namespace {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(const CopyBlocksArgs a) {
  const int p = (int)blockIdx.x;
  const int32_t src = a.pairs[2 * p], dst = a.pairs[2 * p + 1];
  DEBUG_ONLY(debug_report(threadIdx.x == 0 && (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks),
                          kDebugCopyPair));
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks || src == dst) return;
  char* base = static_cast<char*>(blockIdx.y == 0 ? a.k_cache : a.v_cache);
  const u32x4* s = reinterpret_cast<const u32x4*>(base + (int64_t)src * a.block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + (int64_t)dst * a.block_bytes);
  const int chunks = (int)(a.block_bytes / 16);
  // all of a thread's loads are issued before its stores (source and
  // destination could alias as far as the compiler knows)
  constexpr int U = 4;
  for (int i0 = threadIdx.x; i0 < chunks; i0 += U * kCopyThreads) {
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u * kCopyThreads < chunks) r[u] = s[i0 + u * kCopyThreads];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u * kCopyThreads < chunks) d[i0 + u * kCopyThreads] = r[u];
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)a.num_pairs, 2), dim3(kCopyThreads), 0, st, a);
  return hipGetLastError();
}

// debug builds: this file's report word (nothing in release builds)
hipError_t debug_take_copy_blocks(uint32_t* acc, bool clear) { return debug_take_word(acc, clear); }

}  // namespace mi_attn
