"""Decode with the new token's RoPE and cache write fused into the launch
(attn_decode_paged_rope): bit-identical to the separate write
(attn_kv_cache_write_rope) followed by attn_decode_paged, and equal to the
fp64 oracle on the rotated queries and keys."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, f64, say
from workloads import BLOCK_SIZE, build_decode_pool, decode_case, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAN16 = -1  # int16 0xFFFF: a NaN bit pattern in bf16


def new_token_slots(case):
    """Slot of logical position ctx - 1 of every sequence."""
    last = case.lengths - 1
    blk = case.block_tables[np.arange(len(case.lengths)), last // BLOCK_SIZE]
    return (blk.astype(np.int64) * BLOCK_SIZE + last % BLOCK_SIZE).astype(np.int32)


def setup(case, skip=()):
    """Pool holding every context token; the new token's slot holds NaN bits
    (the fused write must land before the attention reads it), except for
    sequences in `skip`, whose slot mapping is -1 and whose cache already
    holds the token."""
    kc, vc = build_decode_pool(case, DEV)
    slots = new_token_slots(case)
    for s in range(len(case.lengths)):
        if s in skip:
            continue
        b, off = divmod(int(slots[s]), BLOCK_SIZE)
        kc.view(torch.int16)[b, :, off, :] = NAN16
        vc.view(torch.int16)[b, :, :, off] = NAN16
    slots_in = slots.copy()
    slots_in[list(skip)] = -1
    k_new = torch.stack([k[-1] for k in case.k]).to(DEV)   # [S, Hkv, D]
    v_new = torch.stack([v[-1] for v in case.v]).to(DEV)
    pos = torch.from_numpy((case.lengths - 1).astype(np.int32)).to(DEV)
    return kc, vc, k_new, v_new, pos, torch.from_numpy(slots_in).to(DEV)


def oracle_out(case, base, skip=()):
    """Rotated q (stored in bf16) over the context whose last key is the new
    key rotated and stored in bf16; skipped sequences keep their cached key."""
    pos = case.lengths - 1
    q_rot = oracle.round_bf16(oracle.rope(to_f64(case.q), pos, base)) if base else to_f64(case.q)
    ks = []
    for s, k in enumerate(case.k):
        k64 = to_f64(k)
        if s not in skip and base:
            k64 = k64.copy()
            k64[-1] = oracle.round_bf16(oracle.rope(k64[-1:], pos[s:s + 1], base))[0]
        ks.append(k64)
    ref, _ = oracle.decode(q_rot, ks, [to_f64(v) for v in case.v])
    return ref, q_rot


def run_pair(case, base=10000.0, part=0, planned=True, skip=()):
    S = len(case.lengths)
    mx = int(case.lengths.max())
    q = case.q.to(DEV)
    bt = torch.from_numpy(case.block_tables).to(DEV)
    cl = torch.from_numpy(case.lengths.astype(np.int32)).to(DEV)
    plan = torch.from_numpy(mi.attn_decode_paged_plan(case.lengths, case.hkv, mx, part)).to(DEV) if planned else None
    # fused
    kc1, vc1, k_new, v_new, pos, slots = setup(case, skip)
    kc2, vc2 = kc1.clone(), vc1.clone()
    q_in = q.clone()
    q_rot = torch.empty_like(q)
    o1 = mi.attn_decode_paged_rope(q_in, k_new, v_new, pos, slots, kc1, vc1, bt, cl, mx, q_rot_out=q_rot,
                                   rope_base=base, partition_size=part, plan=plan)
    # separate: write (rotates q in place) then decode
    q2 = q.clone()
    mi.attn_kv_cache_write_rope(q2, k_new, v_new, pos, slots, kc2, vc2, rope_base=base)
    o2 = mi.attn_decode_paged(q2, kc2, vc2, bt, cl, mx, partition_size=part, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(q_in.view(torch.int16), q.view(torch.int16)), "q must be left unchanged"
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "k cache differs from the separate write"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "v cache differs from the separate write"
    assert torch.equal(q_rot.view(torch.int16), q2.view(torch.int16)), "rotated q differs from the separate write"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "output differs from write + decode"
    ref, q_ref = oracle_out(case, base, skip)
    check(f64(o1), ref, torch.bfloat16, f"fused decode S {S} part {part} base {base}")
    return q_rot, q_ref


def test_c3_shape_fused():
    """64 sequences, context U[128, 4096], 12/2 heads, D 128 (seed 1002)."""
    say("case: fused RoPE write + decode, C3 shape")
    case = decode_case(1002, 64, 128, 4096)
    q_rot, q_ref = run_pair(case)
    # rotated queries: each within the bf16 storage bound of the exact value
    # (the same check as the standalone write's), here via the oracle's own rounding
    assert np.mean(f64(q_rot.cpu()) == q_ref) > 0.999


@pytest.mark.parametrize("planned", [True, False])
def test_many_partitions_fused(planned):
    """Log-uniform contexts 1..9000 with 128-token partitions: the new token
    lands in the last partition, alone in its block or not; planned and
    padded grids."""
    say(f"case: fused decode, many partitions, planned={planned}")
    case = decode_case(51, 40, 1, 9000, dist="loguniform")
    run_pair(case, part=128, planned=planned)


def test_skip_and_plain_copy():
    """slot -1 skips a sequence's write (its cache already holds the token);
    rope_base 0 makes the write a plain copy and leaves q unrotated."""
    say("case: fused decode, skipped slots, no rotation")
    case = decode_case(52, 12, 1, 2000)
    run_pair(case, base=10000.0, part=256, skip=(0, 5))
    run_pair(case, base=0.0, part=256)


def test_head_dim_64_mha():
    """D 64, 8 query heads on 8 kv heads."""
    say("case: fused decode, D 64, 8/8 heads")
    case = decode_case(53, 10, 1, 3000, hq=8, hkv=8, d=64)
    run_pair(case, part=128)


def test_head_slices_fused():
    """40 query heads on 2 kv heads: two head slices per kv head, each of
    whose last-partition workgroups writes the (same) new token."""
    say("case: fused decode, 40/2 heads")
    case = decode_case(54, 8, 1, 2500, hq=40, hkv=2)
    run_pair(case, part=256)
