"""Parity of the paged decode (attn_decode_paged: partitions, merged by the
last workgroup of each sequence in the same launch) with the fp64 oracle,
plus the paging and split-KV invariants."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, f64, say
from workloads import BLOCK_SIZE, build_decode_pool, decode_case, prefill_case, rng, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_decode(case, kc, vc, partition_size=0, max_ctx=None):
    max_ctx = int(case.lengths.max()) if max_ctx is None else max_ctx
    q = case.q.to(DEV)
    bt = torch.from_numpy(case.block_tables).to(DEV)
    cl = torch.from_numpy(case.lengths.astype(np.int32)).to(DEV)
    o = mi.attn_decode_paged(q, kc, vc, bt, cl, max_ctx, partition_size=partition_size)
    torch.cuda.synchronize()
    return o.cpu()


def oracle_decode(case):
    ref, _ = oracle.decode(to_f64(case.q), [to_f64(k) for k in case.k], [to_f64(v) for v in case.v])
    return ref


def test_c3_decode():
    """64 sequences, context U[128, 4096], 12/2 heads, D 128, bf16, block
    tables a random permutation of the pool (seed 1002)."""
    say("case: C3 decode")
    case = decode_case(1002, 64, 128, 4096)
    kc, vc = build_decode_pool(case, DEV)
    o = run_decode(case, kc, vc)
    check(f64(o), oracle_decode(case), torch.bfloat16, "C3")


@pytest.mark.parametrize("part", [16, 32, 48, 128, 256, 512, 1024])
def test_split_kv_partition_sizes(part):
    """Merging P partitions equals the single pass, for every partition size
    (16 and 32: one or two blocks, so most wavefronts of a partition have no
    block); sequences shorter than the longest leave empty partitions in the
    grid."""
    say(f"case: split-KV partition {part}")
    case = decode_case(31, 24, 1, 4096, lengths=np.array([1, 2, 15, 16, 17, 127, 128, 129, 255, 256, 257, 511, 512,
                                                           513, 1000, 1023, 1024, 1025, 2047, 2048, 3000, 4095, 4096,
                                                           77]))
    kc, vc = build_decode_pool(case, DEV)
    o = run_decode(case, kc, vc, partition_size=part)
    check(f64(o), oracle_decode(case), torch.bfloat16, f"partition {part}")


def test_workspace_counters_reset_and_reuse():
    """The arrival counters at the head of the decode workspace are zero after
    every call, so one workspace serves consecutive calls of different shapes:
    a long batch, then a smaller one with shorter contexts, then the first
    again, each equal to the oracle (and the repeat bit-identical)."""
    say("case: decode workspace reuse")
    big = decode_case(41, 20, 1, 3000)
    small = decode_case(42, 7, 1, 700)
    part = 128
    need = mi.attn_decode_paged_workspace_size(20, 12, 2, 128, int(big.lengths.max()), part)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    outs = []
    for case in (big, small, big):
        kc, vc = build_decode_pool(case, DEV)
        q = case.q.to(DEV)
        bt = torch.from_numpy(case.block_tables).to(DEV)
        cl = torch.from_numpy(case.lengths.astype(np.int32)).to(DEV)
        mx = int(case.lengths.max())
        assert mi.attn_decode_paged_workspace_size(len(case.lengths), 12, 2, 128, mx, part) <= need
        plan = torch.from_numpy(mi.attn_decode_paged_plan(case.lengths, 2, mx, part)).to(DEV)
        o = mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=part, workspace=ws, plan=plan)
        torch.cuda.synchronize()
        # counters: one int32 per (sequence, kv head) at the start of the workspace
        assert int(ws[:20 * 2 * 4].view(torch.int32).abs().sum().item()) == 0
        check(f64(o.cpu()), oracle_decode(case), torch.bfloat16, f"reuse {len(case.lengths)} seqs, max {mx}")
        outs.append(o.cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


def test_workspace_reuse_with_more_sequences():
    """A call with few sequences and many partitions, then one with more
    sequences on the same workspace.  The counter block is sized for the
    most sequences a call may have, so the second call's counters lie where
    only counters ever were (not where the first call left partials): every
    call finds them zero, leaves them zero, and equals the oracle."""
    say("case: decode workspace reuse, 7 then 100 sequences")
    few = decode_case(43, 7, 1000, 3000)
    many = decode_case(44, 100, 1, 3000)
    part = 128
    need = max(mi.attn_decode_paged_workspace_size(len(c.lengths), 12, 2, 128, int(c.lengths.max()), part)
               for c in (few, many))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for case in (few, many, few):
        kc, vc = build_decode_pool(case, DEV)
        q = case.q.to(DEV)
        bt = torch.from_numpy(case.block_tables).to(DEV)
        cl = torch.from_numpy(case.lengths.astype(np.int32)).to(DEV)
        mx = int(case.lengths.max())
        o = mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=part, workspace=ws)
        torch.cuda.synchronize()
        check(f64(o.cpu()), oracle_decode(case), torch.bfloat16, f"reuse {len(case.lengths)} seqs")
        cnt = (65535 * 2 * 4 + 255) // 256 * 256
        assert int((ws[:cnt] != 0).sum().item()) == 0, "counter block not left zero"


@pytest.mark.parametrize("part", [0, 128])
def test_planned_grid_equals_padded(part):
    """The planned launch (only the real partitions, longest sequences first)
    gives the padded grid's output bit for bit; plan entries out of range are
    skipped."""
    say(f"case: planned decode, partition {part}")
    case = decode_case(33, 40, 1, 9000, dist="loguniform")
    kc, vc = build_decode_pool(case, DEV)
    q = case.q.to(DEV)
    bt = torch.from_numpy(case.block_tables).to(DEV)
    cl = torch.from_numpy(case.lengths.astype(np.int32)).to(DEV)
    mx = int(case.lengths.max())
    o_pad = mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=part)
    items = mi.attn_decode_paged_plan(case.lengths, case.hkv, mx, part)
    o_plan = mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=part,
                                  plan=torch.from_numpy(items).to(DEV))
    junk = np.concatenate([items, np.array([[-1, 0], [0, 99999], [len(case.lengths), 0], [3, -2]], np.int32)])
    o_junk = mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=part, plan=torch.from_numpy(junk).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o_plan.view(torch.int16), o_pad.view(torch.int16))
    assert torch.equal(o_junk.view(torch.int16), o_pad.view(torch.int16))
    check(f64(o_plan), oracle_decode(case), torch.bfloat16, "planned")


@pytest.mark.parametrize("d", [128, 64])
def test_merge_of_many_partitions(d):
    """Long contexts cut into 128-token partitions (up to 157 per sequence):
    the merge walks the partials in several passes of its partition groups."""
    say(f"case: many partitions, D {d}")
    case = decode_case(32, 5, 1, 1, d=d, lengths=np.array([20000, 9000, 8193, 16, 129]))
    kc, vc = build_decode_pool(case, DEV)
    o = run_decode(case, kc, vc, partition_size=128)
    check(f64(o), oracle_decode(case), torch.bfloat16, f"157 partitions, D {d}")


def test_block_order_invariance_and_worked_table(golden_dir):
    """Identity, reversed and random block tables give bit-identical outputs
    (paging does not change the logical K/V), and the tutorial's worked table
    (logical 0 1 2 3 -> physical 17 4 29 8) gives the contiguous answer."""
    say("case: block orders")
    lengths = np.array([64, 100, 700, 1500, 33])
    outs = []
    for order in ("identity", "reversed", "random"):
        case = decode_case(41, 5, 1, 1, lengths=lengths, block_order=order)
        kc, vc = build_decode_pool(case, DEV)
        outs.append(run_decode(case, kc, vc, partition_size=256))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    check(f64(outs[0]), oracle_decode(case), torch.bfloat16, "orders")

    case = decode_case(42, 1, 1, 1, lengths=np.array([64]), slack_blocks=30 - 4, block_order="identity")
    ident = run_decode(case, *build_decode_pool(case, DEV))
    case.block_tables[0, :4] = [17, 4, 29, 8]
    kc, vc = build_decode_pool(case, DEV)
    worked = run_decode(case, kc, vc)
    assert torch.equal(ident, worked)
    check(f64(worked), oracle_decode(case), torch.bfloat16, "worked table")


def test_gather_is_bit_exact():
    """Each sequence's query selects one target token: its score exceeds every
    other by more than 150 in log2 units, so every other weight is exactly 0
    in fp32.  The value of every token encodes its position exactly in bf16,
    so the output names the token the kernel read through the block table."""
    say("case: gather")
    g = rng(43)
    lengths = g.integers(1, 3000, 40)
    case = decode_case(44, 40, 1, 1, lengths=lengths)
    big = 40.0   # score 1600 / sqrt(128) = 141.4, i.e. 204 in log2 units
    targets = np.array([int(g.integers(0, L)) for L in lengths])
    q = torch.zeros_like(case.q)
    q[:, :, 0] = big
    case.q = q
    for s, L in enumerate(lengths):
        k = torch.zeros(L, 2, 128, dtype=torch.bfloat16)
        k[targets[s], :, 0] = big
        t = torch.arange(L, dtype=torch.float32)
        v = torch.zeros(L, 2, 128, dtype=torch.float32)
        v[:, :, 0] = (t // 256)[:, None]
        v[:, :, 1] = (t % 256)[:, None]
        case.k[s] = k
        case.v[s] = v.to(torch.bfloat16)
    kc, vc = build_decode_pool(case, DEV)
    o = f64(run_decode(case, kc, vc, partition_size=256))
    got = o[:, :, 0] * 256 + o[:, :, 1]
    np.testing.assert_array_equal(got, np.repeat(targets[:, None], 12, axis=1))


def test_single_token_and_garbage_past_the_end():
    """ctx = 1 returns V[0] exactly; cache slots past the context hold NaN
    bit patterns that must not leak into the result."""
    case = decode_case(45, 6, 1, 1, lengths=np.array([1, 5, 16, 17, 31, 130]))
    kc, vc = build_decode_pool(case, DEV, fill=float("nan"))
    o = run_decode(case, kc, vc, partition_size=128)
    assert torch.isfinite(o).all()
    np.testing.assert_array_equal(f64(o)[0], f64(case.v[0][0]).repeat(6, axis=0))
    check(f64(o), oracle_decode(case), torch.bfloat16, "short")


def test_decode_equals_prefill_row():
    """decode(q_t, ctx = t + 1) is row t of the causal prefill (two kernels)."""
    T = 777
    q, k, v = prefill_case(46, 1, T, 12, 2, 128, torch.bfloat16)
    full = mi.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True).cpu()
    rows = [0, 100, 776]
    case = decode_case(47, len(rows), 1, 1, lengths=np.array([r + 1 for r in rows]))
    case.q = torch.stack([q[0, r] for r in rows])
    case.k = [k[0, :r + 1] for r in rows]
    case.v = [v[0, :r + 1] for r in rows]
    kc, vc = build_decode_pool(case, DEV)
    o = run_decode(case, kc, vc, partition_size=128)
    for i, r in enumerate(rows):
        d = np.abs(f64(o[i]) - f64(full[0, r])).max()
        assert d <= 1e-2, (r, d)


@pytest.mark.parametrize("hq,hkv", [(40, 2), (34, 1)])
def test_query_head_slices(hq, hkv):
    """Groups of more than 16 query heads per kv head run as slices of at
    most 16 heads (20 = 16 + 4, 34 = 16 + 16 + 2), each with its own
    workgroups and arrival counter; several partitions per sequence."""
    say(f"case: decode {hq}/{hkv} heads (head slices)")
    case = decode_case(34, 9, 1, 2500, hq=hq, hkv=hkv)
    kc, vc = build_decode_pool(case, DEV)
    o = run_decode(case, kc, vc, partition_size=256)
    check(f64(o), oracle_decode(case), torch.bfloat16, f"{hq}/{hkv} heads")
