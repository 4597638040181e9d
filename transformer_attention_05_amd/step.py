"""One serving step over a shared paged cache: fused RoPE + cache write for
every new token, chunked prefill for the prefill requests, decode for the
decode sequences (one launch: partitions and their merge), with no host
synchronisation in between.  The chunked prefill (bound by the matrix cores)
and the decode (bound by HBM) do not depend on each other, and each needs
only its own new tokens rotated and written (the two sets of tokens and of
cache slots are disjoint).  So with ``concurrent`` the write is split in two
launches: the caller's stream writes the chunk tokens and runs the prefill,
a second stream writes the decode tokens and runs the decode, and the
caller's stream then waits for the second one.  With ``fuse_decode_write``
the second stream instead runs one decode launch that rotates and writes its
own tokens (attn_decode_paged_rope; rotated queries in ``q_dec_rot``), after
waiting for the chunk write (see below).  Nothing waits on the other stream
mid-step.  The prefill is enqueued first: each of its workgroups needs a
whole CU's registers, so it must be placed before the decode's thousands of
small workgroups spread over every CU (enqueued the other way round, the
prefill waits for the decode to drain and the step takes ~250 us instead of
~212 us on MI355X).

With ``single_launch`` (the default of the benchmark) the step is two
launches on the caller's stream: the chunk tokens' write, then one launch
whose grid holds the chunked prefill's workgroups and the decode's (which
writes its own tokens), interleaved (attn_prefill_decode_paged): no second
stream, no cross-stream start or join, same results bit for bit.

The host side (block pool, block tables, slot mapping) is built once in
``__init__``; ``run()`` only enqueues the launches, so the same buffers can be
replayed step after step.
"""

from __future__ import annotations

import numpy as np
import torch

from . import (Pool, attn_decode_paged, attn_decode_paged_partition_for, attn_decode_paged_plan,
               attn_decode_paged_rope, attn_decode_paged_workspace_size, attn_kv_cache_write_rope,
               attn_prefill_decode_paged, attn_prefill_paged, attn_prefill_paged_workspace_size)


class MixedStep:
    """Device state of one mixed step.

    ``case`` supplies the new tokens (q, k, v, positions), the cached keys and
    values of every sequence and the chunk/decode lengths; ``assign`` is a
    callable (case, pool) -> case that reserves blocks and fills
    ``case.tables`` and ``case.slots`` through the pool.
    """

    def __init__(self, case, assign, device="cuda", partition_size=0, scatter=None, concurrent=True,
                 fuse_decode_write=False, single_launch=False):
        self.case = case
        self.concurrent = concurrent
        self.single_launch = single_launch
        self.fuse_decode_write = fuse_decode_write
        self.device = device
        self.pool = Pool(case.num_blocks)
        assign(case, self.pool)
        R = len(case.cached)
        S = len(case.dec_lengths)
        self.R, self.S = R, S
        self.n_prefill = R * case.chunk
        hkv, d = case.hkv, case.d
        dt = case.q_new.dtype
        self.k_cache = torch.zeros(case.num_blocks, hkv, 16, d, dtype=dt, device=device)
        self.v_cache = torch.zeros(case.num_blocks, hkv, d, 16, dtype=dt, device=device)
        if scatter is not None:
            for s in range(R + S):
                scatter(self.k_cache, self.v_cache, case.tables[s], case.k_old[s], case.v_old[s])
        self.q = case.q_new.to(device).contiguous()
        self.k = case.k_new.to(device).contiguous()
        self.v = case.v_new.to(device).contiguous()
        self.positions = torch.from_numpy(case.positions.astype(np.int32)).to(device)
        self.slots = torch.from_numpy(case.slots.astype(np.int32)).to(device)
        self.tables = torch.from_numpy(case.tables).to(device)
        ctx = np.concatenate([case.cached + case.chunk, case.dec_lengths]).astype(np.int32)
        self.context_lens = torch.from_numpy(ctx).to(device)
        cu = np.arange(R + 1, dtype=np.int32) * case.chunk
        self.cu_seqlens_q = torch.from_numpy(cu).to(device)
        self.max_dec_ctx = int(case.dec_lengths.max()) if S else 1
        # 0: the partition chosen from the decode lengths (host side), passed
        # explicitly to the plan and to every decode call
        if partition_size == 0 and S:
            partition_size = attn_decode_paged_partition_for(case.dec_lengths, case.hq, hkv, d)
        self.partition_size = partition_size
        self.o_prefill = torch.empty(self.n_prefill, case.hq, d, dtype=dt, device=device)
        self.o_decode = torch.empty(S, case.hq, d, dtype=dt, device=device)
        # rotated decode queries of the fused decode (the concurrent schedule)
        self.q_dec_rot = torch.empty(S, case.hq, d, dtype=dt, device=device)
        need = attn_decode_paged_workspace_size(S, case.hq, hkv, d, self.max_dec_ctx, partition_size)
        # zeroed once: the decode's arrival counters start at zero and every call leaves them so
        self.workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=device)
        # decode plan: the real (sequence, partition) pairs, built on the host
        # from the host copy of the lengths, as the block tables are
        self.plan = (torch.from_numpy(attn_decode_paged_plan(case.dec_lengths, hkv, self.max_dec_ctx,
                                                             partition_size)).to(device) if S else None)
        # split-KV workspace of the chunked prefill (its own: the two run at once)
        self.max_pre_ctx = int((case.cached + case.chunk).max()) if R else 1
        need = attn_prefill_paged_workspace_size(R, max(self.n_prefill, 1), case.chunk, self.max_pre_ctx, case.hq,
                                                 hkv, d) if R else 0
        self.pre_workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        # second stream (default priority) for the decode tokens' write and the decode
        self.side = torch.cuda.Stream(device=device)

    def write(self, lo=0, hi=None):
        """RoPE + cache write of new tokens lo .. hi-1 (all by default)."""
        hi = self.q.shape[0] if hi is None else hi
        if hi <= lo:
            return
        attn_kv_cache_write_rope(self.q[lo:hi], self.k[lo:hi], self.v[lo:hi], self.positions[lo:hi],
                                 self.slots[lo:hi], self.k_cache, self.v_cache, rope_base=self.case.rope_base)

    def prefill(self, share_cu=False):
        """Chunked prefill; ``share_cu`` when a decode runs beside it (the
        concurrent schedules): same results, a tile that leaves every CU room
        for a decode workgroup."""
        R = self.R
        attn_prefill_paged(self.q[: self.n_prefill], self.k_cache, self.v_cache, self.tables[:R],
                           self.cu_seqlens_q, self.context_lens[:R], self.case.chunk, o=self.o_prefill,
                           causal=True, max_context_len=self.max_pre_ctx, workspace=self.pre_workspace,
                           share_cu=share_cu)

    def decode(self):
        """Decode over the cache, whose decode tokens are already written."""
        R = self.R
        attn_decode_paged(self.q[self.n_prefill:], self.k_cache, self.v_cache, self.tables[R:],
                          self.context_lens[R:], self.max_dec_ctx, o=self.o_decode,
                          partition_size=self.partition_size, workspace=self.workspace, plan=self.plan)

    def decode_fused(self):
        """Decode that rotates and writes the decode tokens itself (q left
        unrotated; rotated queries in q_dec_rot)."""
        R, n = self.R, self.n_prefill
        attn_decode_paged_rope(self.q[n:], self.k[n:], self.v[n:], self.positions[n:], self.slots[n:],
                               self.k_cache, self.v_cache, self.tables[R:], self.context_lens[R:],
                               self.max_dec_ctx, o=self.o_decode, q_rot_out=self.q_dec_rot,
                               rope_base=self.case.rope_base, partition_size=self.partition_size,
                               workspace=self.workspace, plan=self.plan)

    def prefill_and_decode(self):
        """The chunked prefill and the decode (which rotates and writes the
        decode tokens itself) in one launch; the chunk tokens are written."""
        R, n = self.R, self.n_prefill
        pre = dict(q=self.q[:n], block_table=self.tables[:R], cu_seqlens_q=self.cu_seqlens_q,
                   context_lens=self.context_lens[:R], max_seqlen_q=self.case.chunk, o=self.o_prefill, causal=True,
                   max_context_len=self.max_pre_ctx) if R else None
        dec = dict(q=self.q[n:], block_table=self.tables[R:], context_lens=self.context_lens[R:],
                   max_context_len=self.max_dec_ctx, o=self.o_decode, partition_size=self.partition_size,
                   workspace=self.workspace, plan=self.plan, k_new=self.k[n:], v_new=self.v[n:],
                   positions=self.positions[n:], slot_mapping=self.slots[n:], q_rot_out=self.q_dec_rot,
                   rope_base=self.case.rope_base) if self.S else None
        attn_prefill_decode_paged(self.k_cache, self.v_cache, prefill=pre, decode=dec)

    def capture(self):
        """Record run() into a HIP graph (torch.cuda.CUDAGraph) for replay().

        The launches allocate nothing, issue no memset and read no length on
        the host, so the step captures as it is; both streams join the
        capture through the events run() records.  A replay re-runs the same
        launches on the same buffers: the RoPE write rotates q in place, so
        the caller restores q (or writes new tokens) between replays, as it
        would between eager steps."""
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()

    def _fused(self):
        return (self.single_launch or (self.concurrent and self.fuse_decode_write)) and self.R and self.S

    def rotated_q(self):
        """Rotated queries of every new token after run()."""
        if self._fused():
            return torch.cat([self.q[: self.n_prefill], self.q_dec_rot])
        return self.q

    def run(self, marks=None):
        """Enqueue one step.  ``marks``: optional dict of torch.cuda.Event
        ("prefill0", "prefill1" on the caller's stream and "decode0",
        "decode1" on the second stream) recorded around the chunked prefill
        and the decode of the concurrent schedule, or ("mixed0", "mixed1")
        around the single launch, to time them inside the step."""
        def mark(name, stream):
            if marks is not None and name in marks:
                marks[name].record(stream)
        if self.single_launch and self.R and self.S:
            self.write(0, self.n_prefill)    # the chunk tokens
            mark("mixed0", torch.cuda.current_stream())
            self.prefill_and_decode()
            mark("mixed1", torch.cuda.current_stream())
            return
        if self._fused():
            main = torch.cuda.current_stream()
            self.side.wait_stream(main)      # the step's inputs come from the caller's stream
            self.write(0, self.n_prefill)    # the chunk tokens
            # the decode is released with the prefill, when the chunk write
            # ends: started at once, its workgroups would take every CU
            # before the prefill's (MI355X: 234 us per step instead of 207)
            after_write = torch.cuda.Event()
            after_write.record(main)
            self.prefill(share_cu=True)
            with torch.cuda.stream(self.side):
                self.side.wait_event(after_write)
                self.decode_fused()          # writes the decode tokens itself
            main.wait_stream(self.side)
            return
        if self.concurrent and self.R and self.S:
            main = torch.cuda.current_stream()
            self.side.wait_stream(main)      # the step's inputs come from the caller's stream
            self.write(0, self.n_prefill)    # the chunk tokens
            mark("prefill0", main)
            self.prefill(share_cu=True)
            mark("prefill1", main)
            with torch.cuda.stream(self.side):
                self.write(self.n_prefill)   # the decode tokens
                mark("decode0", self.side)
                self.decode()
                mark("decode1", self.side)
            main.wait_stream(self.side)
            return
        self.write()
        if self.R:
            self.prefill()
        if self.S:
            self.decode()
