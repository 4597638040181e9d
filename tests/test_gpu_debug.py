"""The debug library (libmi_attn_debug.so: the same kernels built with
MI_ATTN_DEBUG=1).  On well-formed inputs it records nothing and gives the
release library's results bit for bit; on malformed device-side inputs
(block ids, slots, copy pairs, lengths, query offsets) it records the
matching ATTN_DEBUG_* bit while doing what the release library does with
them (clamp or skip).  Every malformed input here is one that the kernels'
own bounds handling keeps inside the buffers: out-of-pool block ids read
block 0, out-of-pool slots and pairs are skipped, lengths and query offsets
are cut to what the table row, the launch and total_q cover."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, f64, say
from transformer_attention_05_amd import (ATTN_DEBUG_BLOCK_ID, ATTN_DEBUG_CONTEXT, ATTN_DEBUG_COPY_PAIR,
                                          ATTN_DEBUG_SEQLENS, ATTN_DEBUG_SLOT)
from workloads import BLOCK_SIZE, build_decode_pool, decode_case, normal, rng, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def both(fn):
    """fn() through the release library, then through the debug one; returns
    (release result, debug result, debug flags)."""
    with mi.debug_library(False):
        r = fn()
        torch.cuda.synchronize()
    with mi.debug_library(True):
        mi.attn_debug_flags(clear=True)
        d = fn()
        flags = mi.attn_debug_flags(clear=True)
    return r, d, flags


def same_bits(a, b):
    iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(iv), b.view(iv))


def decode_inputs(case, dtype=torch.bfloat16):
    kc, vc = build_decode_pool(case, DEV, dtype=dtype)
    return (case.q.to(DEV, dtype), kc, vc, torch.from_numpy(case.block_tables).to(DEV),
            torch.from_numpy(case.lengths.astype(np.int32)).to(DEV))


def oracle_decode(case):
    ref, _ = oracle.decode(to_f64(case.q), [to_f64(k) for k in case.k], [to_f64(v) for v in case.v])
    return ref


def test_well_formed_inputs_record_nothing():
    """Decode (bf16, fp32, fused), chunked prefill, RoPE write and block copy
    on well-formed inputs, with -1 table padding, -1 slots and a src == dst
    copy pair (all documented as normal): no bit, same output bits."""
    say("case: debug library, well-formed inputs")
    case = decode_case(71, 16, 1, 3000)
    q, kc, vc, bt, cl = decode_inputs(case)
    mx = int(case.lengths.max())
    r, d, flags = both(lambda: mi.attn_decode_paged(q, kc, vc, bt, cl, mx))
    assert flags == 0, f"flags {flags:#x}"
    assert same_bits(r, d)
    check(f64(d.cpu()), oracle_decode(case), torch.bfloat16, "debug decode bf16")

    case32 = decode_case(72, 6, 1, 700, dtype=torch.float32)
    q32, kc32, vc32, bt32, cl32 = decode_inputs(case32, torch.float32)
    r, d, flags = both(lambda: mi.attn_decode_paged(q32, kc32, vc32, bt32, cl32, int(case32.lengths.max()),
                                                    partition_size=64))
    assert flags == 0 and same_bits(r, d)
    check(f64(d.cpu()), oracle_decode(case32), torch.float32, "debug decode fp32")

    # fused RoPE + write + decode, one sequence skipped (slot -1)
    last = case.lengths - 1
    slots = (case.block_tables[np.arange(16), last // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE
             + last % BLOCK_SIZE).astype(np.int32)
    slots[3] = -1
    k_new = torch.stack([k[-1] for k in case.k]).to(DEV)
    v_new = torch.stack([v[-1] for v in case.v]).to(DEV)
    pos = torch.from_numpy(last.astype(np.int32)).to(DEV)
    sl = torch.from_numpy(slots).to(DEV)

    def fused():
        k2, v2 = kc.clone(), vc.clone()
        return mi.attn_decode_paged_rope(q.clone(), k_new, v_new, pos, sl, k2, v2, bt, cl, mx)
    r, d, flags = both(fused)
    assert flags == 0 and same_bits(r, d)

    # chunked prefill
    from tests.test_gpu_paged_prefill import paged_setup
    qs, ks, vs, pbt, pkc, pvc, total = paged_setup(73, [100, 0, 37], [64, 130, 5])
    pq = torch.cat(qs).to(DEV)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum([len(x) for x in qs])]).astype(np.int32)).to(DEV)
    ctx = torch.from_numpy(total.astype(np.int32)).to(DEV)
    pbt_d = torch.from_numpy(pbt).to(DEV)
    r, d, flags = both(lambda: mi.attn_prefill_paged(pq, pkc, pvc, pbt_d, cu, ctx, 130, causal=True))
    assert flags == 0 and same_bits(r, d)

    # RoPE write (every 5th token skipped) and a copy with a src == dst pair
    g = rng(74)
    nb, n = 40, 200
    wq, wk, wv = (normal(g, (n, h, 128), torch.bfloat16).to(DEV) for h in (12, 2, 2))
    wslots = g.permutation(nb * BLOCK_SIZE)[:n].astype(np.int32)
    wslots[::5] = -1
    wpos = torch.from_numpy(g.integers(0, 4096, n).astype(np.int32)).to(DEV)
    wsl = torch.from_numpy(wslots).to(DEV)

    def write():
        k2 = torch.zeros(nb, 2, BLOCK_SIZE, 128, dtype=torch.bfloat16, device=DEV)
        v2 = torch.zeros(nb, 2, 128, BLOCK_SIZE, dtype=torch.bfloat16, device=DEV)
        q2 = wq.clone()
        mi.attn_kv_cache_write_rope(q2, wk, wv, wpos, wsl, k2, v2)
        mi.attn_copy_blocks(k2, v2, torch.tensor([[1, 2], [7, 7]], dtype=torch.int32, device=DEV))
        return torch.cat([q2.flatten(), k2.flatten(), v2.flatten()])
    r, d, flags = both(write)
    assert flags == 0 and same_bits(r, d)


def test_block_ids_outside_the_pool():
    """Table entries in use outside [0, num_blocks) (decode bf16 and fp32,
    chunked prefill) read block 0 in both libraries; the debug one records
    ATTN_DEBUG_BLOCK_ID.  Sequences with a good table keep the oracle's
    result."""
    say("case: debug library, block ids outside the pool")
    case = decode_case(75, 8, 40, 1500)
    bad = case.block_tables.copy()
    bad[1, 1] = case.num_blocks + 7
    bad[3, 0] = -3
    q, kc, vc, _, cl = decode_inputs(case)
    btb = torch.from_numpy(bad).to(DEV)
    mx = int(case.lengths.max())
    r, d, flags = both(lambda: mi.attn_decode_paged(q, kc, vc, btb, cl, mx, partition_size=256))
    assert flags == ATTN_DEBUG_BLOCK_ID, f"flags {flags:#x}"
    assert same_bits(r, d) and torch.isfinite(d.float()).all()
    good = [s for s in range(8) if s not in (1, 3)]
    check(f64(d.cpu())[good], oracle_decode(case)[good], torch.bfloat16, "good sequences")

    case32 = decode_case(76, 4, 40, 300, dtype=torch.float32)
    bad32 = case32.block_tables.copy()
    bad32[2, 0] = 1 << 30
    q32, kc32, vc32, _, cl32 = decode_inputs(case32, torch.float32)
    bt32 = torch.from_numpy(bad32).to(DEV)
    r, d, flags = both(lambda: mi.attn_decode_paged(q32, kc32, vc32, bt32, cl32, int(case32.lengths.max()),
                                                    partition_size=64))
    assert flags == ATTN_DEBUG_BLOCK_ID and same_bits(r, d)

    from tests.test_gpu_paged_prefill import paged_setup
    qs, ks, vs, pbt, pkc, pvc, total = paged_setup(77, [100, 20], [64, 70])
    pbt = pbt.copy()
    pbt[0, 2] = -9
    pq = torch.cat(qs).to(DEV)
    cu = torch.from_numpy(np.array([0, 64, 134], np.int32)).to(DEV)
    ctx = torch.from_numpy(total.astype(np.int32)).to(DEV)
    pbt_d = torch.from_numpy(pbt).to(DEV)
    r, d, flags = both(lambda: mi.attn_prefill_paged(pq, pkc, pvc, pbt_d, cu, ctx, 70, causal=True))
    assert flags == ATTN_DEBUG_BLOCK_ID and same_bits(r, d)


def test_lengths_and_query_offsets():
    """A negative context length, one past the block-table row, cu_seqlens_q
    past total_q and not starting at 0: cut to what the launch covers in
    both libraries; the debug one records CONTEXT / SEQLENS."""
    say("case: debug library, malformed lengths")
    case = decode_case(78, 6, 40, 900)
    q, kc, vc, bt, _ = decode_inputs(case)
    mx = int(case.lengths.max())
    lens = case.lengths.astype(np.int32).copy()
    lens[2] = -4
    cl = torch.from_numpy(lens).to(DEV)
    _, _, flags = both(lambda: mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=256))
    assert flags == ATTN_DEBUG_CONTEXT, f"flags {flags:#x}"
    # past the row and the launch: the extra table entries it would need
    # are -1 padding or past the row, so BLOCK_ID may come with it
    lens = case.lengths.astype(np.int32).copy()
    lens[int(np.argmax(case.lengths))] = case.block_tables.shape[1] * BLOCK_SIZE + 40
    cl = torch.from_numpy(lens).to(DEV)
    _, _, flags = both(lambda: mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=256))
    assert flags & ATTN_DEBUG_CONTEXT and not flags & ~(ATTN_DEBUG_CONTEXT | ATTN_DEBUG_BLOCK_ID), f"{flags:#x}"

    from tests.test_gpu_paged_prefill import paged_setup
    qs, ks, vs, pbt, pkc, pvc, total = paged_setup(79, [30, 50], [64, 70])
    pq = torch.cat(qs).to(DEV)
    pbt_d = torch.from_numpy(pbt).to(DEV)
    ctx = torch.from_numpy(total.astype(np.int32)).to(DEV)
    for cu_host, bit in (([0, 64, 140], ATTN_DEBUG_SEQLENS),   # past total_q = 134
                         ([3, 64, 134], ATTN_DEBUG_SEQLENS),   # not starting at 0
                         ([0, 70, 64], ATTN_DEBUG_SEQLENS)):   # falling
        cu = torch.from_numpy(np.array(cu_host, np.int32)).to(DEV)
        r, d, flags = both(lambda: mi.attn_prefill_paged(pq, pkc, pvc, pbt_d, cu, ctx, 76, causal=True))
        assert flags == bit, f"cu {cu_host}: flags {flags:#x}"
    cu = torch.from_numpy(np.array([0, 64, 134], np.int32)).to(DEV)
    big = torch.from_numpy(np.array([int(total[0]), pbt.shape[1] * BLOCK_SIZE + 1], np.int32)).to(DEV)
    _, _, flags = both(lambda: mi.attn_prefill_paged(pq, pkc, pvc, pbt_d, cu, big, 70, causal=True))
    assert flags & ATTN_DEBUG_CONTEXT and not flags & ~(ATTN_DEBUG_CONTEXT | ATTN_DEBUG_BLOCK_ID), f"{flags:#x}"


def test_slots_and_copy_pairs_outside_the_pool():
    """Slots below -1 or past the pool (RoPE write, fused decode) and copy
    pairs outside the pool are skipped in both libraries (caches bit-equal)
    and recorded by the debug one; a read without clearing keeps the bits."""
    say("case: debug library, slots and copy pairs outside the pool")
    g = rng(80)
    nb, n = 30, 100
    wq, wk, wv = (normal(g, (n, h, 64), torch.bfloat16).to(DEV) for h in (4, 4, 4))
    slots = g.permutation(nb * BLOCK_SIZE)[:n].astype(np.int32)
    slots[5], slots[50] = nb * BLOCK_SIZE + 3, -7
    pos = torch.from_numpy(g.integers(0, 4096, n).astype(np.int32)).to(DEV)
    sl = torch.from_numpy(slots).to(DEV)

    def write():
        k2 = torch.zeros(nb, 4, BLOCK_SIZE, 64, dtype=torch.bfloat16, device=DEV)
        v2 = torch.zeros(nb, 4, 64, BLOCK_SIZE, dtype=torch.bfloat16, device=DEV)
        mi.attn_kv_cache_write_rope(wq.clone(), wk, wv, pos, sl, k2, v2)
        return torch.cat([k2.flatten(), v2.flatten()])
    r, d, flags = both(write)
    assert flags == ATTN_DEBUG_SLOT and same_bits(r, d)

    case = decode_case(81, 5, 40, 600)
    q, kc, vc, bt, cl = decode_inputs(case)
    k_new = torch.stack([k[-1] for k in case.k]).to(DEV)
    v_new = torch.stack([v[-1] for v in case.v]).to(DEV)
    p = torch.from_numpy((case.lengths - 1).astype(np.int32)).to(DEV)
    fs = torch.from_numpy(np.array([-1, case.num_blocks * BLOCK_SIZE, -1, -1, -1], np.int32)).to(DEV)

    def fused():
        k2, v2 = kc.clone(), vc.clone()
        o = mi.attn_decode_paged_rope(q.clone(), k_new, v_new, p, fs, k2, v2, bt, cl, int(case.lengths.max()))
        return torch.cat([o.flatten(), k2.flatten(), v2.flatten()])
    r, d, flags = both(fused)
    assert flags == ATTN_DEBUG_SLOT and same_bits(r, d)

    k3 = normal(g, (nb, 2, BLOCK_SIZE, 128), torch.bfloat16).to(DEV)
    v3 = normal(g, (nb, 2, 128, BLOCK_SIZE), torch.bfloat16).to(DEV)
    pairs = torch.tensor([[1, 2], [-1, 5], [5, nb], [7, 7]], dtype=torch.int32, device=DEV)

    def copy():
        k4, v4 = k3.clone(), v3.clone()
        mi.attn_copy_blocks(k4, v4, pairs)
        return torch.cat([k4.flatten(), v4.flatten()])
    r, d, flags = both(copy)
    assert flags == ATTN_DEBUG_COPY_PAIR and same_bits(r, d)

    with mi.debug_library(True):
        mi.attn_copy_blocks(k3.clone(), v3.clone(), pairs)
        assert mi.attn_debug_flags(clear=False) == ATTN_DEBUG_COPY_PAIR
        assert mi.attn_debug_flags(clear=True) == ATTN_DEBUG_COPY_PAIR
        assert mi.attn_debug_flags(clear=True) == 0
