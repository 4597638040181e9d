"""Benchmark of the attention hot path on one MI355X.

A step is one serving step over a shared paged KV cache, the workload that
touches every stage of the path: the fused RoPE + paged cache write of all
new tokens, chunked prefill of 8 requests (512 new tokens each on 0-2048
cached tokens) and decode of 128 sequences (context log-uniform in
[16, 32768]), partitions and merge in one launch; 12 query / 2 kv heads,
head_dim 128, bf16, 16-token blocks, RoPE base 10000, pool pre-fragmented
(seed 1004).  The decode-only step of the 64-sequence workload is also
timed both ways: RoPE write then decode, and the decode launch that writes
its own tokens.
Inputs are synthetic and already resident in HBM when timing starts.

Timing: the headline times --steps steps (200) after --warmup untimed ones (20),
between two device synchronisations (eager launches).  Every component
figure takes 20 untimed calls and then 100 timed calls in samples of 20
back-to-back calls between a pair of HIP events on the launching stream,
the 20 calls captured once in a HIP graph and replayed per sample (so the
binding's host-side cost does not pace short kernels); it reports the
median (`us`), the min and the mean per call.  A graph replay costs about
22 us before its first kernel starts (measured on MI355X: a replay of one
near-empty kernel takes 28 us, each further one adds 1.1 us), so a sample
of 20 calls charges each call about 1.1 us of it.  The roofline figure
(the mixed launch) uses the mean (the average launch duration), as the
profiler summary does; the step is also timed eagerly in samples of 20, and
the mixed launch inside runs of 20 back-to-back steps, by events around it.

value = percent of the step's roofline time reached:
    100 * max(F / 2.5 PFLOP/s, B / 8 TB/s) / measured step time
with F the chunked-prefill flops (4 * D per unmasked query-key pair) and B the
algorithmic HBM bytes of the write, the chunked prefill and the decode (the
chunked prefill and the decode run at once, so the bound is the busier of
the two resources).  The step is two launches on one stream: the chunk
tokens' RoPE write, then one launch that runs the chunked prefill's and the
decode's workgroups together (the decode writing its own tokens).  The line
also carries the roofline of that dominant launch, the oracle timed on the host cores
and the per-stage figures, plus the contiguous long prefill (T 16384) and the
uniform-context decode (64 sequences, U[128, 4096]) measured on their own.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s + paged-decode KV GB/s on 1 MI355X (% of roofline)"
PEAK_BF16_FLOPS = 2.5e15
TRAFFIC_PROBE_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mixed_traffic.json")
# the sources the counted kernel is compiled from
MIXED_SRCS = [os.path.join(ROOT, "transformer_attention_05_amd", "csrc", f)
              for f in ("mixed.hip", "prefill_body.h", "decode_body.h", "device_common.h", "kernels.h")]
PEAK_HBM = 8.0e12
HQ, HKV, D, BS = 12, 2, 128, 16
ELT = 2  # bf16 bytes


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic work

def prefill_pairs_causal(cached, new):
    """Unmasked (query, key) pairs of a chunk of `new` rows on `cached` keys."""
    return int(new) * int(cached) + int(new) * (int(new) + 1) // 2


def chunk_flops(case):
    pairs = sum(prefill_pairs_causal(c, case.chunk) for c in case.cached)
    return 4 * D * HQ * pairs


def decode_bytes(lengths, num_blocks_used=None):
    """K and V read once per kv head, plus q, o, the used block-table entries
    and the context lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    kv = int(lengths.sum()) * HKV * D * ELT * 2
    qo = len(lengths) * HQ * D * ELT * 2
    bt = int(((lengths + BS - 1) // BS).sum()) * 4
    return kv + qo + bt + len(lengths) * 4


def prefill_io_bytes(case):
    """Chunked prefill: new queries read and outputs written, plus every
    request's keys and values (cached and new) read once per kv head."""
    ctx = np.asarray(case.cached, dtype=np.int64) + case.chunk
    qo = len(case.cached) * case.chunk * HQ * D * ELT * 2
    return qo + int(ctx.sum()) * HKV * D * ELT * 2


def write_bytes(n_tokens):
    """q read + written, k and v read, rotated k and v written, positions and
    slots read."""
    return n_tokens * (HQ * D * ELT * 2 + HKV * D * ELT * 2 * 2 + 8)


# ----------------------------------------------------------------------------- timing helpers

WARM_CALLS, TIMED_CALLS, PER_SAMPLE = 20, 100, 20
IN_STEP_SAMPLES = 5  # runs of PER_SAMPLE back-to-back steps with events around the mixed launch


def timed(torch, fn, warm=None, calls=None, per=PER_SAMPLE, graph=True):
    """Per-call duration of fn(i), in ms: `warm` untimed calls, then `calls`
    timed ones as calls / per samples, each a pair of HIP events on the
    current stream around `per` back-to-back calls.  With `graph`, the `per`
    calls are captured once in a HIP graph and each sample replays it: the
    kernels then run back to back on the GPU whatever the host-side cost of
    a call (the Python binding's argument checks take longer than the
    shortest kernels), so the figure is the GPU time per call plus a share
    of the replay's start (about 22 us over the `per` calls).  (An event
    recorded between two kernels leaves the GPU idle for several
    microseconds on this stack, so there is no event pair around every
    single call.)  Returns mean, median and min over the samples, and the
    call counts."""
    warm = WARM_CALLS if warm is None else warm
    calls = TIMED_CALLS if calls is None else calls
    per = min(per, calls)
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(per):
                fn(j)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
    samples = []
    for k in range(calls // per):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        if g is not None:
            g.replay()
        else:
            for j in range(per):
                fn(k * per + j)
        b.record()
        torch.cuda.synchronize()
        samples.append(a.elapsed_time(b) / per)
    return dict(mean=float(np.mean(samples)), median=float(np.median(samples)), min=float(np.min(samples)),
                warm=warm, calls=(calls // per) * per, per_sample=per, graph=g is not None)


def fig(t, work=None, unit=None, peak=None, key="frac_of_peak"):
    """A component figure: median us (the primary), min and mean us, the
    iteration counts, and the median's rate (and fraction of peak)."""
    how = "graph replays of" if t.get("graph") else "eager,"
    d = {"us": round(t["median"] * 1e3, 2), "us_min": round(t["min"] * 1e3, 2), "us_mean": round(t["mean"] * 1e3, 2),
         "iters": f"{t['warm']} warm-up + {t['calls']} timed calls ({how} {t['per_sample']} calls per event pair)"}
    if t.get("back_to_back"):
        d["iters"] = (f"{t['warm']} warm-up + {t['calls']} timed launches (eager, events around the launch in each "
                      f"step of runs of {t['back_to_back']} back-to-back steps)")
    if work is not None:
        rate = work / (t["median"] / 1e3)
        d[unit] = round(rate / (1e12 if unit == "TFLOP/s" else 1e9), 1)
        if peak:
            d[key] = round(rate / peak, 4)
    return d


def main():
    global WARM_CALLS, TIMED_CALLS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 steps (about 35 ms of GPU time): the window's own start and end
    # (the first launch's latency, the final synchronisation) then cost
    # under 1 % of a step; over 20 steps they added ~5-9 us to each
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--only", choices=["mixed", "prefill", "decode"], default=None,
                    help="run one workload only (for profiling)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="first copy a 256 MiB buffer (known bytes) so hardware byte counters can be scaled")
    ap.add_argument("--calls", type=int, default=TIMED_CALLS,
                    help="timed calls per component figure (default 100; fewer for profiler runs)")
    ap.add_argument("--warm-calls", type=int, default=WARM_CALLS, help="untimed calls before each figure (default 20)")
    args = ap.parse_args()
    WARM_CALLS, TIMED_CALLS = max(0, args.warm_calls), max(1, args.calls)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is a design note, not implemented)"}))
        sys.exit(2)

    import torch
    import transformer_attention_05_amd as mi
    from transformer_attention_05_amd.step import MixedStep
    from workloads import (additive_mask, assign_blocks, build_decode_pool, decode_case, mixed_case, prefill_case,
                           scatter_to_pool)

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    mi.load()
    dev = "cuda"
    out = {}
    # no cyclic garbage collection while timing (reference counting still
    # frees everything): a collection pass inside a timed window stalled the
    # host for tens of milliseconds; the cpu_baseline leg runs with it on
    gc.collect()
    gc.disable()
    if args.traffic_probe:
        src = torch.empty(TRAFFIC_PROBE_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------------------------------ the step (mixed)
    if args.only in (None, "mixed"):
        log("bench: building the mixed step (seed 1004)")
        case = mixed_case(1004)
        step = MixedStep(case, assign_blocks, dev, scatter=scatter_to_pool, single_launch=True)
        n_new = case.q_new.shape[0]
        F = chunk_flops(case)
        B_dec = decode_bytes(case.dec_lengths)
        B_wr = write_bytes(n_new)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            step.run()
        torch.cuda.synchronize()
        # the timed steps: nothing between the launches (an event recorded
        # between two kernels leaves the GPU idle for ~10 us on this stack)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step.run()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        # the step again, event-timed (median and min over samples)
        t_step = timed(torch, lambda i: step.run(), graph=False)
        # the mixed launch inside the step: events around it in each of
        # PER_SAMPLE back-to-back steps (the queue stays ahead of the GPU, so
        # no host latency falls between a step's events)
        in_mix = []
        for k in range(WARM_CALLS + IN_STEP_SAMPLES):
            marks = [{n: torch.cuda.Event(enable_timing=True) for n in ("mixed0", "mixed1")} for _ in range(PER_SAMPLE)]
            for mk in marks:
                step.run(mk)
            torch.cuda.synchronize()
            if k >= WARM_CALLS:
                in_mix += [mk["mixed0"].elapsed_time(mk["mixed1"]) for mk in marks]
        in_step = dict(mean=float(np.mean(in_mix)), median=float(np.median(in_mix)), min=float(np.min(in_mix)),
                       warm=WARM_CALLS * PER_SAMPLE, calls=len(in_mix), per_sample=1, back_to_back=PER_SAMPLE)
        # the step's two launches on their own, back to back, between HIP
        # events on their stream: the chunk tokens' write and the mixed launch
        # (chunked prefill + decode with its tokens' write)
        t_wchunk = timed(torch, lambda i: step.write(0, step.n_prefill))
        t_mix = timed(torch, lambda i: step.prefill_and_decode())
        # the stages as separate kernels, for reference: every token's write,
        # the chunked prefill (default tile) and the decode
        stages = [timed(torch, lambda i, f=fn: f()) for fn in (step.write, step.prefill, step.decode)]
        ms_wr, ms_pre, ms_dec = (t["mean"] for t in stages)
        # the same step captured in a HIP graph, replays back to back
        graph_s = None
        if not args.no_components:
            step.capture()
            for _ in range(3):
                step.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                step.replay()
            torch.cuda.synchronize()
            graph_s = (time.perf_counter() - t0) / args.steps
        # the former schedule: the prefill and the decode as two launches on
        # two streams (each stream writing its own tokens first)
        two_s = None
        if not args.no_components:
            two = MixedStep(case, assign_blocks, dev, scatter=scatter_to_pool)
            for _ in range(args.warmup):
                two.run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                two.run()
            torch.cuda.synchronize()
            two_s = (time.perf_counter() - t0) / args.steps
            del two
        # prefill and decode overlap, so the step's bound is the larger of its
        # total HBM bytes and its total matrix-core flops
        B_pre = prefill_io_bytes(case)
        t_roof = max(F / PEAK_BF16_FLOPS, (B_dec + B_wr + B_pre) / PEAK_HBM)
        S = len(case.dec_lengths)
        B_mix = B_dec + B_pre + write_bytes(S)  # the mixed launch: decode, chunked prefill, decode tokens' write
        out["mixed"] = dict(wall_s=wall, ms_write=ms_wr, ms_prefill=ms_pre, ms_decode=ms_dec, stages=stages,
                            t_step=t_step, in_step=in_step, t_wchunk=t_wchunk, t_mix=t_mix, F=F, B_dec=B_dec,
                            B_wr=B_wr, B_pre=B_pre, B_mix=B_mix, B_wchunk=write_bytes(step.n_prefill), t_roof=t_roof,
                            n_new=n_new, part=step.partition_size, dec_tokens=int(case.dec_lengths.sum()),
                            pool_blocks=case.num_blocks, graph_s=graph_s, two_s=two_s)
        log(f"bench: mixed step wall {wall * 1e3:.3f} ms | chunk write {t_wchunk['mean']:.3f} mixed launch "
            f"{t_mix['mean']:.3f} ms | two streams {two_s * 1e3 if two_s else float('nan'):.3f} ms")
        del step

    # ------------------------------------------------------------------ contiguous long prefill
    if not args.no_components and args.only in (None, "prefill"):
        log("bench: contiguous prefill T 16384")
        q, k, v = prefill_case(1003, 1, 16384, HQ, HKV, D, torch.bfloat16)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(qd)
        t = timed(torch, lambda i: mi.attn_prefill(qd, kd, vd, o=o))
        fl = 4 * D * HQ * 16384 * 16385 // 2
        out["prefill_c4"] = dict(t=t, flops=fl)
        log(f"bench: prefill C4 median {t['median']:.3f} ms  {fl / t['median'] / 1e9:.1f} TFLOP/s")
        del qd, kd, vd, o
        # the 2048-token prompt: too few query tiles for the GPU, so split-KV
        log("bench: contiguous prefill T 2048")
        q, k, v = prefill_case(1001, 1, 2048, HQ, HKV, D, torch.bfloat16)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(qd)
        ws = torch.empty(max(256, mi.attn_prefill_workspace_size(1, 2048, 2048, HQ, HKV, D)), dtype=torch.uint8,
                         device=dev)
        t = timed(torch, lambda i: mi.attn_prefill(qd, kd, vd, o=o, workspace=ws))
        fl = 4 * D * HQ * 2048 * 2049 // 2
        out["prefill_c2"] = dict(t=t, flops=fl)
        log(f"bench: prefill C2 median {t['median'] * 1e3:.1f} us  {fl / t['median'] / 1e9:.1f} TFLOP/s")
        # the same shape with a general additive mask (one fp32 [T, T] mask for
        # every head, no causal structure): every (query, key) pair is computed
        mask = additive_mask(1006, (2048, 2048), amp=1.0, p_masked=0.1).to(dev)
        t = timed(torch, lambda i: mi.attn_prefill_masked(qd, kd, vd, mask, o=o))
        fl = 4 * D * HQ * 2048 * 2048
        out["prefill_masked"] = dict(t=t, flops=fl)
        log(f"bench: masked prefill T 2048 median {t['median'] * 1e3:.1f} us  {fl / t['median'] / 1e9:.1f} TFLOP/s")
        del qd, kd, vd, o, ws, mask

    # ------------------------------------------------------------------ uniform decode
    if not args.no_components and args.only in (None, "decode"):
        log("bench: decode 64 seqs ctx U[128, 4096] (3 rotating pool copies)")
        dc = decode_case(1002, 64, 128, 4096)
        pools = [build_decode_pool(dc, dev) for _ in range(3)]
        qd = dc.q.to(dev)
        bt = torch.from_numpy(dc.block_tables).to(dev)
        cl = torch.from_numpy(dc.lengths.astype(np.int32)).to(dev)
        mx = int(dc.lengths.max())
        # the partition chosen from the lengths (host side, as the plan is)
        part = mi.attn_decode_paged_partition_for(dc.lengths, HQ, HKV, D)
        ws = torch.zeros(max(256, mi.attn_decode_paged_workspace_size(64, HQ, HKV, D, mx, part)), dtype=torch.uint8,
                         device=dev)
        o = torch.empty_like(qd)
        plan = torch.from_numpy(mi.attn_decode_paged_plan(dc.lengths, HKV, mx, part)).to(dev)
        t = timed(torch, lambda i: mi.attn_decode_paged(qd, *pools[i % 3], bt, cl, mx, o=o, partition_size=part,
                                                        workspace=ws, plan=plan))
        by = decode_bytes(dc.lengths)
        out["decode_c3"] = dict(t=t, bytes=by, part=part)
        log(f"bench: decode C3 median {t['median'] * 1e3:.1f} us  {by / t['median'] / 1e6:.0f} GB/s")
        # a decode-only serving step: each sequence's new token (the last of
        # its context) rotated and written into its slot, then the decode;
        # as two launches, and as the one decode launch that writes it
        last = dc.lengths - 1
        slots_np = (dc.block_tables[np.arange(64), last // 16].astype(np.int64) * 16 + last % 16).astype(np.int32)
        slots = torch.from_numpy(slots_np).to(dev)
        pos = torch.from_numpy(last.astype(np.int32)).to(dev)
        k_new = torch.stack([k[-1] for k in dc.k]).to(dev)
        v_new = torch.stack([v[-1] for v in dc.v]).to(dev)
        q_rot = torch.empty_like(qd)
        q_w = qd.clone()

        def two_launches(i):
            mi.attn_kv_cache_write_rope(q_w, k_new, v_new, pos, slots, *pools[i % 3])
            mi.attn_decode_paged(q_w, *pools[i % 3], bt, cl, mx, o=o, partition_size=part, workspace=ws, plan=plan)

        def one_launch(i):
            mi.attn_decode_paged_rope(qd, k_new, v_new, pos, slots, *pools[i % 3], bt, cl, mx, o=o, q_rot_out=q_rot,
                                      partition_size=part, workspace=ws, plan=plan)
        step_t = {name: timed(torch, fn) for name, fn in (("write_then_decode", two_launches), ("fused", one_launch))}
        out["decode_step_c3"] = dict(bytes=by + write_bytes(64), **step_t)
        log(f"bench: decode-only step C3: write + decode {step_t['write_then_decode']['median'] * 1e3:.1f} us, "
            f"fused {step_t['fused']['median'] * 1e3:.1f} us")
        del pools
        # copy on write of prefix sharing: 4096 whole blocks (both pools, 2 kv
        # heads, D 128, bf16: 8 KiB per block and pool) copied in one launch;
        # three disjoint pair sets in rotation (400 MB touched) so the 256 MB
        # MALL cannot hold the sources
        kc = torch.zeros(30000, HKV, 16, D, dtype=torch.bfloat16, device=dev)
        vc = torch.zeros(30000, HKV, D, 16, dtype=torch.bfloat16, device=dev)
        perm = np.random.default_rng(1007).permutation(30000)
        sets = [torch.from_numpy(np.stack([perm[i * 8192:i * 8192 + 4096], perm[i * 8192 + 4096:(i + 1) * 8192]],
                                          1).astype(np.int32)).to(dev) for i in range(3)]
        t = timed(torch, lambda i: mi.attn_copy_blocks(kc, vc, sets[i % 3]))
        out["copy_blocks"] = dict(t=t, bytes=4096 * 2 * HKV * 16 * D * ELT * 2)
        log(f"bench: copy 4096 blocks median {t['median'] * 1e3:.1f} us")
        del kc, vc

    # ------------------------------------------------------------------ fused residual + RMSNorm
    if not args.no_components and args.only in (None, "decode"):
        # the mixed step's 4224 new tokens at the tutorial model's hidden width
        # 1536, bf16; three input sets in rotation (78 MB touched)
        g = np.random.default_rng(1008)
        sets = [tuple(torch.from_numpy(g.standard_normal((4224, 1536)).astype(np.float32)).to(dev, torch.bfloat16)
                      for _ in range(2)) for _ in range(3)]
        wgt = torch.ones(1536, dtype=torch.bfloat16, device=dev)
        yb = torch.empty(4224, 1536, dtype=torch.bfloat16, device=dev)
        hb = torch.empty_like(yb)
        t = timed(torch, lambda i: mi.attn_residual_rms_norm(*sets[i % 3], wgt, y=yb, residual_out=hb))
        out["rmsnorm"] = dict(t=t, bytes=4224 * 1536 * ELT * 4 + 1536 * ELT)
        log(f"bench: residual + RMSNorm 4224 x 1536 median {t['median'] * 1e3:.1f} us")
        del sets, yb, hb

    # ------------------------------------------------------------------ CPU baseline (oracle)
    cpu = None
    gc.enable()
    if not args.no_cpu_baseline and "mixed" in out:
        cpu = cpu_baseline(case, out["mixed"])

    emit(args, out, cpu)


def cpu_baseline(case, m):
    """The oracle on the whole mixed step (a few seconds of host work)."""
    import oracle
    from workloads import to_f64
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(threads)
        blas = [f"{i.get('internal_api')}:{i.get('num_threads')}" for i in threadpool_info()]
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas, used = [], threads
    log(f"bench: oracle on the host ({threads} cores visible, BLAS {blas})")
    t0 = time.perf_counter()
    pos = case.positions
    q_rot = oracle.round_bf16(oracle.rope(to_f64(case.q_new), pos, case.rope_base))
    k_rot = oracle.round_bf16(oracle.rope(to_f64(case.k_new), pos, case.rope_base))
    v_new = to_f64(case.v_new)
    R, C = len(case.cached), case.chunk
    qs, ks, vs = [], [], []
    for r in range(R):
        sl = slice(r * C, (r + 1) * C)
        qs.append(q_rot[sl])
        ks.append(np.concatenate([to_f64(case.k_old[r]), k_rot[sl]]))
        vs.append(np.concatenate([to_f64(case.v_old[r]), v_new[sl]]))
    oracle.chunked_prefill(qs, ks, vs)
    dk, dv = [], []
    for s in range(len(case.dec_lengths)):
        n = R * C + s
        dk.append(np.concatenate([to_f64(case.k_old[R + s]), k_rot[n:n + 1]]))
        dv.append(np.concatenate([to_f64(case.v_old[R + s]), v_new[n:n + 1]]))
    oracle.decode(q_rot[R * C:], dk, dv)
    t = time.perf_counter() - t0
    return dict(value=round(100.0 * m["t_roof"] / t, 6), unit="% of roofline", cores=int(used),
                kind="oracle", seconds_per_step=round(t, 3),
                sample="the whole mixed step (RoPE on all 4224 new tokens, 8 chunked prefills, 128 decodes), "
                       "fp64 NumPy, once")


def mixed_src_sha256():
    """sha256 over the sources of the mixed launch's kernel, in order."""
    import hashlib
    h = hashlib.sha256()
    for path in MIXED_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per mixed launch from the committed counter profile, or
    None if its sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        sha = mixed_src_sha256()
    except (OSError, ValueError):
        return None
    if t.get("src_sha256") != sha:
        return None
    return t.get("hbm_bytes_per_launch")


def emit(args, out, cpu):
    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    comps = {}
    if "mixed" in out:
        m = out["mixed"]
        step_s = m["wall_s"]
        res["value"] = round(100.0 * m["t_roof"] / step_s, 3)
        res["unit"] = "% of roofline"
        res["ms_per_step"] = round(step_s * 1e3, 4)
        res["config"] = {"workload": "mixed serving step: fused RoPE+paged KV write (4224 tokens), chunked "
                                     "prefill 8x512 new on 0-2048 cached, decode 128 seqs ctx log-U[16,32768]; "
                                     "Hq 12 / Hkv 2, D 128, bf16, block 16, fragmented pool, seed 1004",
                         "new_tokens": m["n_new"], "decode_context_tokens": m["dec_tokens"],
                         "pool_blocks": m["pool_blocks"], "decode_partition": m["part"],
                         "schedule": "one stream: the chunk tokens' RoPE write, then one launch running the chunked "
                                     "prefill's and the decode's workgroups together (attn_prefill_decode_paged; the "
                                     "decode writes its own tokens); stage figures run alone, default tiles",
                         "parallelism": "single GPU"}
        mix_s = m["t_mix"]["mean"] / 1e3
        gbps = m["B_mix"] / mix_s / 1e9
        ins = m["in_step"]
        res["roofline"] = {"kernel": "mixed_kernel: the chunked prefill's and the paged decode's workgroups (decode "
                                     "tokens' write, partitions and merge included) in one launch",
                           "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                           "frac": round(gbps * 1e9 / PEAK_HBM, 4), "traffic": measured_traffic(),
                           "algorithmic_bytes_per_launch": m["B_mix"],
                           "flops_per_launch": m["F"],
                           "frac_of_bf16_peak": round(m["F"] / mix_s / PEAK_BF16_FLOPS, 4),
                           "avg_launch_us": round(m["t_mix"]["mean"] * 1e3, 2),
                           "launches_timed": m["t_mix"]["calls"],
                           "in_step": {"avg_launch_us": round(ins["mean"] * 1e3, 2),
                                       "median_launch_us": round(ins["median"] * 1e3, 2),
                                       "frac": round(m["B_mix"] / (ins["mean"] / 1e3) / PEAK_HBM, 4),
                                       "note": "the same launch inside back-to-back steps (events around it)"}}
        st_w, st_p, st_d = m["stages"]
        comps["step"] = fig(m["t_step"])
        comps["step"]["frac_of_step_roofline"] = round(m["t_roof"] / (m["t_step"]["median"] / 1e3), 4)
        comps["step_chunk_write"] = fig(m["t_wchunk"], m["B_wchunk"], "GB/s", PEAK_HBM, "frac_of_hbm_peak")
        comps["step_mixed_launch"] = fig(m["t_mix"], m["B_mix"], "GB/s", PEAK_HBM, "frac_of_hbm_peak")
        comps["step_mixed_launch_in_step"] = fig(m["in_step"], m["B_mix"], "GB/s", PEAK_HBM, "frac_of_hbm_peak")
        comps["write_all_4224_tokens"] = fig(st_w, m["B_wr"], "GB/s", PEAK_HBM, "frac_of_hbm_peak")
        comps["chunked_prefill_alone"] = fig(st_p, m["F"], "TFLOP/s", PEAK_BF16_FLOPS, "frac_of_bf16_peak")
        comps["decode_alone"] = fig(st_d, m["B_dec"], "GB/s", PEAK_HBM, "frac_of_hbm_peak")
        comps["step_roofline_us"] = round(m["t_roof"] * 1e6, 2)
        if m.get("two_s"):
            comps["step_two_streams_us"] = round(m["two_s"] * 1e6, 2)
        if m.get("graph_s"):
            comps["step_graph_replay_us"] = round(m["graph_s"] * 1e6, 2)
    if "prefill_c4" in out:
        comps["prefill_T16384"] = fig(out["prefill_c4"]["t"], out["prefill_c4"]["flops"], "TFLOP/s", PEAK_BF16_FLOPS,
                                      "frac_of_bf16_peak")
    if "prefill_c2" in out:
        comps["prefill_T2048"] = fig(out["prefill_c2"]["t"], out["prefill_c2"]["flops"], "TFLOP/s", PEAK_BF16_FLOPS,
                                     "frac_of_bf16_peak")
    if "prefill_masked" in out:
        comps["prefill_T2048_additive_mask"] = fig(out["prefill_masked"]["t"], out["prefill_masked"]["flops"],
                                                   "TFLOP/s", PEAK_BF16_FLOPS, "frac_of_bf16_peak")
    if "decode_c3" in out:
        d = out["decode_c3"]
        comps["decode_64seq_U128_4096"] = fig(d["t"], d["bytes"], "GB/s", PEAK_HBM, "frac_of_hbm_peak")
        comps["decode_64seq_U128_4096"]["partition"] = d["part"]
    if "decode_step_c3" in out:
        d = out["decode_step_c3"]
        comps["decode_only_step_64seq"] = {"bytes": d["bytes"],
                                           "write_then_decode": fig(d["write_then_decode"]),
                                           "fused": fig(d["fused"], d["bytes"], "GB/s", PEAK_HBM, "frac_of_hbm_peak")}
    if "rmsnorm" in out:
        comps["residual_rmsnorm_4224x1536"] = fig(out["rmsnorm"]["t"], out["rmsnorm"]["bytes"], "GB/s", PEAK_HBM,
                                                  "frac_of_hbm_peak")
    if "copy_blocks" in out:
        comps["copy_on_write_4096_blocks"] = fig(out["copy_blocks"]["t"], out["copy_blocks"]["bytes"], "GB/s",
                                                 PEAK_HBM, "frac_of_hbm_peak")
    res["components"] = comps
    if "value" not in res:
        res["value"] = None
        res["unit"] = "% of roofline"
        res["ms_per_step"] = None
        res["config"] = {"workload": f"partial run ({args.only})"}
    res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
