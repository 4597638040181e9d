"""Chunked prefill over the paged cache (attn_prefill_paged) and the whole
mixed step (RoPE + cache write, chunked prefill, decode) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, check_stored, f64, say
from transformer_attention_05_amd.step import MixedStep
from workloads import (BLOCK_SIZE, assign_blocks, mixed_case, normal, prefill_case, rng, scatter_to_pool,
                       to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def paged_setup(seed, cached, new, hq=12, hkv=2, d=128, order="random", dtype=torch.bfloat16):
    """Sequences with `cached` + `new` tokens laid out in a paged pool."""
    g = rng(seed)
    total = np.asarray(cached) + np.asarray(new)
    nblk = (total + BLOCK_SIZE - 1) // BLOCK_SIZE
    nb = int(nblk.sum()) + 8
    perm = g.permutation(nb) if order == "random" else np.arange(nb)
    maxb = int(nblk.max())
    bt = np.full((len(total), maxb), -1, dtype=np.int32)
    p = 0
    for s, n in enumerate(nblk):
        bt[s, :n] = perm[p:p + n]
        p += n
    ks = [normal(g, (int(t), hkv, d), dtype) for t in total]
    vs = [normal(g, (int(t), hkv, d), dtype) for t in total]
    qs = [normal(g, (int(n), hq, d), dtype) for n in new]
    kc = torch.full((nb, hkv, BLOCK_SIZE, d), float("nan"), dtype=dtype, device=DEV)
    vc = torch.full((nb, hkv, d, BLOCK_SIZE), float("nan"), dtype=dtype, device=DEV)
    for s in range(len(total)):
        scatter_to_pool(kc, vc, bt[s], ks[s], vs[s])
    return qs, ks, vs, bt, kc, vc, total


def run_paged(qs, bt, kc, vc, total, causal=True, **kw):
    q = torch.cat(qs).to(DEV)
    cu = np.concatenate([[0], np.cumsum([x.shape[0] for x in qs])]).astype(np.int32)
    o = mi.attn_prefill_paged(q, kc, vc, torch.from_numpy(bt).to(DEV), torch.from_numpy(cu).to(DEV),
                              torch.from_numpy(total.astype(np.int32)).to(DEV), int(np.diff(cu).max()),
                              causal=causal, **kw)
    torch.cuda.synchronize()
    return o.cpu(), cu


@pytest.mark.parametrize("cached,new", [
    ([0], [1]), ([0], [64]), ([5], [1]), ([15], [17]), ([16], [16]), ([17], [129]),
    ([0, 100, 1, 300], [300, 17, 128, 5]), ([2048, 0, 777], [512, 512, 100]),
])
def test_chunked_prefill(cached, new):
    say(f"case: paged prefill cached {cached} new {new}")
    qs, ks, vs, bt, kc, vc, total = paged_setup(70 + sum(cached) + sum(new), cached, new)
    o, cu = run_paged(qs, bt, kc, vc, total)
    refs = oracle.chunked_prefill([to_f64(q) for q in qs], [to_f64(k) for k in ks], [to_f64(v) for v in vs])
    check(f64(o), np.concatenate(refs), torch.bfloat16, "chunked")


def test_chunk_equals_rows_of_contiguous_prefill():
    """Chunked prefill at cached c = rows c .. c+n-1 of the contiguous causal
    prefill over c + n tokens (paged and contiguous kernels agree bit for bit
    when each query tile is one pass)."""
    c, n = 300, 200
    qs, ks, vs, bt, kc, vc, total = paged_setup(80, [c], [n])
    o, _ = run_paged(qs, bt, kc, vc, total, workspace=False)
    qfull = torch.cat([normal(rng(1), (c, 12, 128), torch.bfloat16), qs[0]])[None]
    full = mi.attn_prefill(qfull.to(DEV), ks[0][None].to(DEV), vs[0][None].to(DEV), causal=True,
                           workspace=False).cpu()
    assert torch.equal(full[0, c:], o)


@pytest.mark.parametrize("ctx_hint,d", [(0, 128), (3200, 128), (1100, 128), (3200, 64)])
def test_split_kv_chunked_prefill(ctx_hint, d):
    """Split-KV shares + merge = one pass per query tile = the oracle, for a
    context bound from the block table (0), the exact longest context, and a
    bound below it (the kernel lengthens the shares to cover every key)."""
    cached, new = [3000, 100], [200, 50]
    say(f"case: paged split-KV, max_context_len hint {ctx_hint}, D {d}")
    s, tot, mq = len(new), sum(new), max(new)
    bound = ctx_hint or 3200
    assert mi.attn_prefill_paged_workspace_size(s, tot, mq, bound, 12, 2, d) > 0   # the plan splits
    qs, ks, vs, bt, kc, vc, total = paged_setup(90, cached, new, d=d)
    o_split, _ = run_paged(qs, bt, kc, vc, total, max_context_len=ctx_hint)
    o_one, _ = run_paged(qs, bt, kc, vc, total, workspace=False)
    refs = np.concatenate(oracle.chunked_prefill([to_f64(q) for q in qs], [to_f64(k) for k in ks],
                                                 [to_f64(v) for v in vs]))
    check(f64(o_split), refs, torch.bfloat16, "split-KV chunked")
    check(f64(o_one), refs, torch.bfloat16, "one-pass chunked")
    check(f64(o_split), f64(o_one), torch.bfloat16, "split vs one pass")


def test_share_cu_tile_bit_identical():
    """ATTN_PREFILL_SHARE_CU runs the 4-wavefront tile with a three-deep V
    ring (one workgroup per CU) where the default has a two-deep one (two
    per CU); every row is computed in the same order, so the outputs match
    bit for bit, and both match the oracle."""
    cached, new = [0, 300, 1000, 17, 2048, 64, 500, 5], [512] * 8
    say("case: paged prefill, share-CU tile vs default, 8 x 512")
    qs, ks, vs, bt, kc, vc, total = paged_setup(95, cached, new)
    o_def, _ = run_paged(qs, bt, kc, vc, total)
    o_sh, _ = run_paged(qs, bt, kc, vc, total, share_cu=True)
    assert torch.equal(o_def.view(torch.int16), o_sh.view(torch.int16))
    refs = oracle.chunked_prefill([to_f64(q) for q in qs], [to_f64(k) for k in ks], [to_f64(v) for v in vs])
    check(f64(o_sh), np.concatenate(refs), torch.bfloat16, "share-CU chunked")


@pytest.mark.parametrize("d", [128, 64])
def test_share_cu_split_kv(d):
    """The flagged form through split-KV: few query tiles over long contexts
    split into shares (fewer than the default's, one workgroup per CU) and
    merge; the workspace sized for the default plan suffices.  Checked
    against the oracle (share boundaries differ from the default's, so the
    rounding may too)."""
    cached, new = [3000, 100], [200, 50]
    say(f"case: paged split-KV with the share-CU form, D {d}")
    qs, ks, vs, bt, kc, vc, total = paged_setup(96, cached, new, d=d)
    o, _ = run_paged(qs, bt, kc, vc, total, max_context_len=3200, share_cu=True)
    refs = np.concatenate(oracle.chunked_prefill([to_f64(q) for q in qs], [to_f64(k) for k in ks],
                                                 [to_f64(v) for v in vs]))
    check(f64(o), refs, torch.bfloat16, "share-CU split-KV chunked")


def test_noncausal_paged():
    qs, ks, vs, bt, kc, vc, total = paged_setup(81, [40, 0], [30, 70])
    o, _ = run_paged(qs, bt, kc, vc, total, causal=False)
    refs = [oracle.attention(to_f64(q)[None], to_f64(k)[None], to_f64(v)[None], causal=False)[0][0]
            for q, k, v in zip(qs, ks, vs)]
    check(f64(o), np.concatenate(refs), torch.bfloat16, "non-causal paged")


# ------------------------------------------------------------------ the mixed step

def mixed_reference(case):
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
    pre = np.concatenate(oracle.chunked_prefill(qs, ks, vs)) if R else np.zeros((0, case.hq, case.d))
    dk, dv = [], []
    for s in range(len(case.dec_lengths)):
        n = R * C + s
        dk.append(np.concatenate([to_f64(case.k_old[R + s]), k_rot[n:n + 1]]))
        dv.append(np.concatenate([to_f64(case.v_old[R + s]), v_new[n:n + 1]]))
    dec, _ = oracle.decode(q_rot[R * C:], dk, dv)
    return pre, dec, q_rot


def run_mixed(case, partition_size=0, single_launch=False):
    step = MixedStep(case, assign_blocks, DEV, partition_size=partition_size, scatter=scatter_to_pool,
                     single_launch=single_launch)
    step.run()
    torch.cuda.synchronize()
    return step


def test_mixed_step_small():
    say("case: mixed step small")
    case = mixed_case(77, num_req=3, chunk=100, cached_max=300, num_dec=9, dec_lo=1, dec_hi=3000)
    step = run_mixed(case, partition_size=256)
    pre, dec, _ = mixed_reference(case)
    check_stored(f64(step.rotated_q()), oracle.rope(to_f64(case.q_new), case.positions, case.rope_base), torch.bfloat16,
                 "rotated q")
    check(f64(step.o_prefill), pre, torch.bfloat16, "mixed prefill")
    check(f64(step.o_decode), dec, torch.bfloat16, "mixed decode")
    # foreign tenants' blocks were never handed to the workload
    used = set(case.tables[case.tables >= 0].tolist())
    assert not used & set(case.foreign.tolist())


@pytest.mark.parametrize("schedule", ["two streams", "two streams, fused decode write", "single launch"])
def test_concurrent_step_equals_serial(schedule):
    """The two-stream schedule (the decode tokens written and decoded on a
    second stream beside the chunk write and prefill, or with the decode
    writing its own tokens) and the single launch of prefill and decode
    workgroups give the serial order's outputs, rotated queries and caches
    bit for bit."""
    say(f"case: {schedule} vs serial step")
    case = mixed_case(78, num_req=3, chunk=200, cached_max=900, num_dec=20, dec_lo=1, dec_hi=5000)
    steps = []
    for conc in (False, True):
        st = MixedStep(case, assign_blocks, DEV, scatter=scatter_to_pool, concurrent=conc,
                       fuse_decode_write=schedule.endswith("fused decode write"),
                       single_launch=conc and schedule == "single launch")
        st.run()
        torch.cuda.synchronize()
        steps.append(st)
    a, b = steps
    for name in ("o_prefill", "o_decode", "rotated_q", "k_cache", "v_cache"):
        x, y = getattr(a, name), getattr(b, name)
        if callable(x):
            x, y = x(), y()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), name


@pytest.mark.parametrize("fused,single", [(False, False), (True, False), (False, True)])
def test_graph_replay_equals_eager(fused, single):
    """The step captured in a HIP graph and replayed three times, with eager
    work (restoring the unrotated queries) and synchronisations between the
    replays: every replay matches the oracle (outputs at the bf16 bar, rotated
    queries within the storage bound) and gives the eager step's outputs,
    rotated queries and caches bit for bit."""
    say(f"case: graph-captured step, fused decode write {fused}, single launch {single}")
    case = mixed_case(79, num_req=3, chunk=150, cached_max=700, num_dec=17, dec_lo=1, dec_hi=6000)
    pre, dec, q_rot = mixed_reference(case)
    q_exact = oracle.rope(to_f64(case.q_new), case.positions, case.rope_base)
    st = MixedStep(case, assign_blocks, DEV, scatter=scatter_to_pool, fuse_decode_write=fused, single_launch=single)
    q0 = st.q.clone()
    st.run()
    torch.cuda.synchronize()
    check(f64(st.o_prefill), pre, torch.bfloat16, "eager prefill")
    check(f64(st.o_decode), dec, torch.bfloat16, "eager decode")
    names = ("o_prefill", "o_decode", "k_cache", "v_cache")
    eager = {n: getattr(st, n).clone() for n in names}
    eager["rotated_q"] = st.rotated_q().clone()
    st.capture()
    for rep in range(3):
        st.q.copy_(q0)
        st.o_prefill.zero_()
        st.o_decode.zero_()
        torch.cuda.synchronize()
        st.replay()
        torch.cuda.synchronize()
        check(f64(st.o_prefill), pre, torch.bfloat16, f"replay {rep} prefill")
        check(f64(st.o_decode), dec, torch.bfloat16, f"replay {rep} decode")
        check_stored(f64(st.rotated_q()), q_exact, torch.bfloat16, f"replay {rep} rotated q")
        for n in names:
            assert torch.equal(getattr(st, n).view(torch.int16), eager[n].view(torch.int16)), (rep, n)
        assert torch.equal(st.rotated_q().view(torch.int16), eager["rotated_q"].view(torch.int16)), rep


@pytest.mark.parametrize("single", [True, False])
def test_c5_mixed_step(single):
    """8 chunks of 512 new tokens on 0-2048 cached tokens + 128 decode
    sequences with context log-U[16, 32768], RoPE base 10000, fragmented pool
    (seed 1004), in the benchmark's launch configuration (the single launch)
    and in the two-stream one."""
    say(f"case: C5 mixed step, single launch {single}")
    case = mixed_case(1004)
    step = run_mixed(case, single_launch=single)
    say(f"  pool {case.num_blocks} blocks, decode tokens {int(case.dec_lengths.sum())}")
    pre, dec, _ = mixed_reference(case)
    check(f64(step.o_prefill), pre, torch.bfloat16, "C5 prefill")
    check(f64(step.o_decode), dec, torch.bfloat16, "C5 decode")
