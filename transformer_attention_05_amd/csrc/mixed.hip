// A chunked prefill and a decode over the same paged cache in one launch.
//
// "Fast Attention Kernels and Operator Fusion" treats prefill (many queries
// at once, bound by the matrix work) and decode (one query per request,
// bound by reading the KV cache) as the two regimes of attention
// (§FlashAttention-Style Kernels), and a serving step has both.  They touch
// disjoint outputs and only read the cache, so their workgroups can share
// the GPU.  Run as two launches on two streams, each pays a cross-stream
// start and join, and the hardware queues decide how the CUs are shared;
// here one grid holds both kinds of workgroup, in an order chosen for it:
//
//   grid = [gp prefill, gd decode] x ceil(n_pre / gp), then the remaining
//          decode workgroups,
//
// so the prefill workgroups, the longest ones, start within the first
// rounds and every CU holds a mix from the start (the hardware deals
// consecutive workgroups round-robin over the XCDs and their CUs).  A slot
// past the end of its kind exits at once.  Each workgroup runs the same code
// as its own kernel would (prefill_body.h, decode_body.h), so the outputs are
// those of the two separate launches, bit for bit.  The LDS of the launch is
// the larger of the two (the prefill tile's rings); registers are what the
// prefill tile uses (256), which keeps two workgroups per CU like either
// kernel alone.

#include "decode_body.h"
#include "prefill_body.h"

namespace mi_attn {

namespace {

template <int D, int HPW, int WPH>
constexpr int mixed_lds_bytes() {
  constexpr int p = pf::lds_elems<D, HPW, WPH, false, false>() * 2;
  constexpr int d = dc::decode_lds_bytes<D, dc::DW>();
  return p > d ? p : d;
}

template <int D, int HPW, int WPH, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void mixed_kernel(const PrefillArgs pa, const DecodeArgs da, const MixedSched m) {
  static_assert(64 * HPW * WPH == 64 * dc::DW, "both kinds of workgroup have 256 threads");
  __shared__ __attribute__((aligned(1024))) char lds[mixed_lds_bytes<D, HPW, WPH>()];
  const uint32_t i = blockIdx.x;
  const uint32_t G = (uint32_t)(m.gp + m.gd);
  const uint32_t head = (uint32_t)m.groups * G;  // the interleaved part of the grid
  uint32_t did;
  if (i < head) {
    const uint32_t k = i / G, r = i % G;
    if (r < (uint32_t)m.gp) {
      const uint32_t pid = k * (uint32_t)m.gp + r;
      // the prefill's waves issue first where they share a SIMD with a
      // decode wave (mixed launch 159.5 -> 157.3 us on the mixed step; the
      // decode's waves first instead: 166 us)
      __builtin_amdgcn_s_setprio(1);
      if (pid < (uint32_t)m.n_pre)
        pf::bf16_body<D, true, HPW, WPH, false, false, false>(pa, pid, reinterpret_cast<__bf16*>(lds));
      return;
    }
    did = k * (uint32_t)m.gd + (r - (uint32_t)m.gp);
  } else {
    did = (uint32_t)m.groups * (uint32_t)m.gd + (i - head);
  }
  if (did >= (uint32_t)m.n_dec) return;
  if (da.plan != nullptr) {
    dc::planned_body<D, FUSED>(da, did, lds);
  } else {
    // padded grid (partition fastest, then kv slice, then sequence)
    const uint32_t P = (uint32_t)(da.max_parts | 1), Y = (uint32_t)(da.hkv * da.head_groups);
    dc::decode_body<D, dc::DW, FUSED>(da, (int)(did % P), (int)(did / P % Y), (int)(did / P / Y), lds);
  }
}

template <int D, int HPW, int WPH>
void launch_mixed_t(const PrefillArgs& pa, const DecodeArgs& da, const MixedSched& m, bool fused, hipStream_t s) {
  const dim3 grid(mixed_grid(m));
  if (fused) hipLaunchKernelGGL((mixed_kernel<D, HPW, WPH, true>), grid, dim3(256), 0, s, pa, da, m);
  else hipLaunchKernelGGL((mixed_kernel<D, HPW, WPH, false>), grid, dim3(256), 0, s, pa, da, m);
}

}  // namespace

hipError_t launch_mixed(const PrefillArgs& pa, const DecodeArgs& da, const MixedSched& m, int head_dim, int hpw,
                        bool fused, hipStream_t s) {
  if (mixed_grid(m) == 0) return hipSuccess;
  if (head_dim == 128) {
    if (hpw == 2) launch_mixed_t<128, 2, 2>(pa, da, m, fused, s);
    else launch_mixed_t<128, 1, 4>(pa, da, m, fused, s);
  } else {
    if (hpw == 2) launch_mixed_t<64, 2, 2>(pa, da, m, fused, s);
    else launch_mixed_t<64, 1, 4>(pa, da, m, fused, s);
  }
  return hipGetLastError();
}

// debug builds: this file's report word (nothing in release builds)
hipError_t debug_take_mixed(uint32_t* acc, bool clear) { return debug_take_word(acc, clear); }

}  // namespace mi_attn
