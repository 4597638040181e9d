"""attn_prefill_decode_paged: a chunked prefill and a decode over one paged
cache in one launch, against the two separate calls (bit for bit) and the
oracle: either part alone, the padded and the planned decode grid, with and
without the decode's own token write, head_dim 64, and the 1 x 4 tile of odd
GQA groups."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, f64, say
from transformer_attention_05_amd.step import MixedStep
from workloads import BLOCK_SIZE, assign_blocks, mixed_case, normal, rng, scatter_to_pool, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def setup(case, partition_size=0):
    st = MixedStep(case, assign_blocks, DEV, partition_size=partition_size, scatter=scatter_to_pool)
    st.write()  # every new token rotated and in the cache (the parts read it)
    torch.cuda.synchronize()
    return st


def parts(st, plan=True, fused=False):
    R, n = st.R, st.n_prefill
    pre = dict(q=st.q[:n], block_table=st.tables[:R], cu_seqlens_q=st.cu_seqlens_q, context_lens=st.context_lens[:R],
               max_seqlen_q=st.case.chunk, causal=True, max_context_len=st.max_pre_ctx)
    dec = dict(q=st.q[n:], block_table=st.tables[R:], context_lens=st.context_lens[R:], max_context_len=st.max_dec_ctx,
               partition_size=st.partition_size, workspace=st.workspace, plan=st.plan if plan else None)
    return pre, dec


def separate(st, plan=True):
    """The two calls one after the other."""
    R, n = st.R, st.n_prefill
    o_pre = mi.attn_prefill_paged(st.q[:n], st.k_cache, st.v_cache, st.tables[:R], st.cu_seqlens_q,
                                  st.context_lens[:R], st.case.chunk, causal=True, max_context_len=st.max_pre_ctx,
                                  workspace=False)
    o_dec = mi.attn_decode_paged(st.q[n:], st.k_cache, st.v_cache, st.tables[R:], st.context_lens[R:], st.max_dec_ctx,
                                 partition_size=st.partition_size, workspace=st.workspace,
                                 plan=st.plan if plan else None)
    torch.cuda.synchronize()
    return o_pre, o_dec


def same(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


@pytest.mark.parametrize("plan", [True, False])
def test_both_parts_equal_separate_calls(plan):
    say(f"case: prefill + decode in one launch, planned decode {plan}")
    case = mixed_case(81, num_req=4, chunk=300, cached_max=1000, num_dec=30, dec_lo=1, dec_hi=9000)
    st = setup(case)
    ref_pre, ref_dec = separate(st, plan)
    pre, dec = parts(st, plan)
    o_pre, o_dec = mi.attn_prefill_decode_paged(st.k_cache, st.v_cache, prefill=pre, decode=dec)
    torch.cuda.synchronize()
    same(o_pre, ref_pre, "prefill")
    same(o_dec, ref_dec, "decode")


def test_one_part_only():
    say("case: prefill part alone, decode part alone")
    case = mixed_case(82, num_req=2, chunk=130, cached_max=500, num_dec=11, dec_lo=1, dec_hi=4000)
    st = setup(case)
    ref_pre, ref_dec = separate(st)
    pre, dec = parts(st)
    o_pre, o_none = mi.attn_prefill_decode_paged(st.k_cache, st.v_cache, prefill=pre)
    o_none2, o_dec = mi.attn_prefill_decode_paged(st.k_cache, st.v_cache, decode=dec)
    torch.cuda.synchronize()
    assert o_none is None and o_none2 is None
    same(o_pre, ref_pre, "prefill alone")
    same(o_dec, ref_dec, "decode alone")


@pytest.mark.parametrize("hq,hkv,d", [(12, 2, 64), (6, 2, 128), (4, 4, 64)])
def test_shapes_against_oracle(hq, hkv, d):
    """head_dim 64, and odd groups (3 and 1 query heads per kv head: the
    1 x 4 prefill tile), with the decode writing its own tokens: equal to
    the serial step bit for bit, and to the oracle."""
    say(f"case: single launch, Hq {hq} Hkv {hkv} D {d}")
    case = mixed_case(83, num_req=3, chunk=96, cached_max=400, num_dec=13, dec_lo=1, dec_hi=3000, hq=hq, hkv=hkv, d=d)
    st = MixedStep(case, assign_blocks, DEV, scatter=scatter_to_pool, single_launch=True)
    st.run()
    ser = MixedStep(case, assign_blocks, DEV, scatter=scatter_to_pool, concurrent=False)
    ser.run()
    torch.cuda.synchronize()
    for name in ("o_prefill", "o_decode", "k_cache", "v_cache"):
        same(getattr(st, name), getattr(ser, name), name)
    same(st.rotated_q(), ser.rotated_q(), "rotated q")
    # the oracle, as the mixed-step tests compute it
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
    check(f64(st.o_prefill), np.concatenate(oracle.chunked_prefill(qs, ks, vs)), torch.bfloat16, "prefill")
    dk, dv = [], []
    for s in range(len(case.dec_lengths)):
        n = R * C + s
        dk.append(np.concatenate([to_f64(case.k_old[R + s]), k_rot[n:n + 1]]))
        dv.append(np.concatenate([to_f64(case.v_old[R + s]), v_new[n:n + 1]]))
    dec, _ = oracle.decode(q_rot[R * C:], dk, dv)
    check(f64(st.o_decode), dec, torch.bfloat16, "decode")


def test_rejects_before_launch():
    """Invalid parts are refused with nothing launched: a partition size that
    is not a multiple of 16, and q_rot_out without the token write."""
    case = mixed_case(84, num_req=1, chunk=64, cached_max=64, num_dec=3, dec_lo=1, dec_hi=500)
    st = setup(case)
    pre, dec = parts(st)
    bad = dict(dec, partition_size=40)
    with pytest.raises(mi.AttnError):
        mi.attn_prefill_decode_paged(st.k_cache, st.v_cache, prefill=pre, decode=bad)
    with pytest.raises(mi.AttnError):
        mi.attn_prefill_decode_paged(st.k_cache, st.v_cache, decode=dict(dec, q_rot_out=st.q_dec_rot[:3]))
    assert "attn_prefill_decode_paged" in mi.attn_last_error()


def ragged_pool(seed, pre_cached, pre_new, dec_ctx, hq=12, hkv=2, d=128, dtype=torch.bfloat16):
    """One NaN-filled pool holding the chunked sequences (cached + new
    tokens) and the decode sequences, blocks scattered at random."""
    g = rng(seed)
    totals = [int(c) + int(n) for c, n in zip(pre_cached, pre_new)] + [int(c) for c in dec_ctx]
    nblk = [(t + BLOCK_SIZE - 1) // BLOCK_SIZE for t in totals]
    nb = sum(nblk) + 8
    perm = g.permutation(nb)
    bt = np.zeros((len(totals), max(nblk)), dtype=np.int32)
    p = 0
    for s, n in enumerate(nblk):
        bt[s, :n] = perm[p:p + n]
        p += n
    ks = [normal(g, (t, hkv, d), dtype) for t in totals]
    vs = [normal(g, (t, hkv, d), dtype) for t in totals]
    kc = torch.full((nb, hkv, BLOCK_SIZE, d), float("nan"), dtype=dtype, device=DEV)
    vc = torch.full((nb, hkv, d, BLOCK_SIZE), float("nan"), dtype=dtype, device=DEV)
    for s in range(len(totals)):
        scatter_to_pool(kc, vc, bt[s], ks[s], vs[s])
    q_pre = [normal(g, (int(n), hq, d), dtype) for n in pre_new]
    q_dec = normal(g, (len(dec_ctx), hq, d), dtype)
    return q_pre, q_dec, ks, vs, bt, kc, vc, np.array(totals, dtype=np.int32)


@pytest.mark.parametrize("part,plan", [(0, True), (64, True), (64, False)])
def test_ragged_chunks_and_short_contexts(part, plan):
    """Ragged chunks (1 to 512 new tokens on 0 to 2048 cached, unaligned to
    blocks and tiles) beside decodes of 1, 16, 17, 1024, 1025 and 3000
    tokens, over one NaN-filled pool: bit-identical to the separate calls,
    and the oracle."""
    say(f"case: ragged mixed launch, partition {part}, plan {plan}")
    cached, new = [0, 17, 2048, 5], [1, 129, 512, 64]
    dec_ctx = [1, 16, 17, 1024, 1025, 3000]
    q_pre, q_dec, ks, vs, bt, kc, vc, totals = ragged_pool(85 + part, cached, new, dec_ctx)
    R, S = len(cached), len(dec_ctx)
    q = torch.cat(q_pre).to(DEV)
    qd = q_dec.to(DEV)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(new)]).astype(np.int32)).to(DEV)
    tables = torch.from_numpy(bt).to(DEV)
    lens = torch.from_numpy(totals).to(DEV)
    mx = int(max(dec_ctx))
    part_eff = part if part else mi.attn_decode_paged_partition_for(np.array(dec_ctx, np.int32), 12, 2, 128)
    ws = torch.zeros(max(256, mi.attn_decode_paged_workspace_size(S, 12, 2, 128, mx, part_eff)), dtype=torch.uint8,
                     device=DEV)
    pl = torch.from_numpy(mi.attn_decode_paged_plan(np.array(dec_ctx, np.int32), 2, mx, part_eff)).to(DEV) if plan else None
    pre = dict(q=q, block_table=tables[:R], cu_seqlens_q=cu, context_lens=lens[:R], max_seqlen_q=max(new), causal=True)
    dec = dict(q=qd, block_table=tables[R:], context_lens=lens[R:], max_context_len=mx, partition_size=part_eff,
               workspace=ws, plan=pl)
    o_pre, o_dec = mi.attn_prefill_decode_paged(kc, vc, prefill=pre, decode=dec)
    ref_pre = mi.attn_prefill_paged(q, kc, vc, tables[:R], cu, lens[:R], max(new), causal=True, workspace=False)
    ref_dec = mi.attn_decode_paged(qd, kc, vc, tables[R:], lens[R:], mx, partition_size=part_eff, workspace=ws,
                                   plan=pl)
    torch.cuda.synchronize()
    same(o_pre, ref_pre, "prefill")
    same(o_dec, ref_dec, "decode")
    exp_pre = oracle.chunked_prefill([to_f64(x) for x in q_pre], [to_f64(k) for k in ks[:R]],
                                     [to_f64(v) for v in vs[:R]])
    check(f64(o_pre), np.concatenate(exp_pre), torch.bfloat16, "prefill vs oracle")
    exp_dec, _ = oracle.decode(to_f64(q_dec), [to_f64(k) for k in ks[R:]], [to_f64(v) for v in vs[R:]])
    check(f64(o_dec), exp_dec, torch.bfloat16, "decode vs oracle")


def test_workspace_reused_by_growing_launches():
    """Two single launches in a row on one decode workspace, the second with
    more decode sequences than the first (its arrival counters reach past
    the first's): both equal the separate calls bit for bit, and the
    counter block is zero after each."""
    say("case: mixed launches on one workspace, 9 then 60 decode sequences")
    small = mixed_case(86, num_req=2, chunk=100, cached_max=300, num_dec=9, dec_lo=1000, dec_hi=3000)
    big = mixed_case(87, num_req=2, chunk=100, cached_max=300, num_dec=60, dec_lo=1, dec_hi=3000)
    need = 0
    for case in (small, big):
        mx = int(case.dec_lengths.max())
        need = max(need, mi.attn_decode_paged_workspace_size(len(case.dec_lengths), 12, 2, 128, mx, 128))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    cnt = (65535 * 2 * 4 + 255) // 256 * 256
    for case in (small, big, small):
        st = MixedStep(case, assign_blocks, DEV, partition_size=128, scatter=scatter_to_pool)
        st.write()
        torch.cuda.synchronize()
        st.workspace = ws
        ref_pre, ref_dec = separate(st)
        assert int((ws[:cnt] != 0).sum().item()) == 0
        pre, dec = parts(st)
        o_pre, o_dec = mi.attn_prefill_decode_paged(st.k_cache, st.v_cache, prefill=pre, decode=dec)
        torch.cuda.synchronize()
        same(o_pre, ref_pre, "prefill")
        same(o_dec, ref_dec, f"decode, {len(case.dec_lengths)} sequences")
        assert int((ws[:cnt] != 0).sum().item()) == 0, "counter block not left zero"
