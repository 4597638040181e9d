"""fp32 over the paged cache (attn_decode_paged and attn_prefill_paged, plus
the paged mask) against the fp64 oracle at the fp32 bar (max |err| <= 1e-5),
and the split-KV pin at fp32: partitions of 16, 32, 256 tokens and a single
pass agree with each other within 1e-6 relative, empty partitions included."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, f64, say
from tests.test_gpu_paged_prefill import paged_setup
from workloads import additive_mask, build_decode_pool, decode_case, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

F32 = torch.float32
LENGTHS = np.array([1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 256, 257, 511, 512, 1000, 1025, 2047, 3000])


def decode_f32(case, kc, vc, part, plan=False):
    mx = int(case.lengths.max())
    q = case.q.to(DEV)
    bt = torch.from_numpy(case.block_tables).to(DEV)
    cl = torch.from_numpy(case.lengths.astype(np.int32)).to(DEV)
    pl = torch.from_numpy(mi.attn_decode_paged_plan(case.lengths, case.hkv, mx, part)).to(DEV) if plan else None
    o = mi.attn_decode_paged(q, kc, vc, bt, cl, mx, partition_size=part, plan=pl)
    torch.cuda.synchronize()
    return f64(o.cpu())


@pytest.mark.parametrize("hq,hkv,d", [(12, 2, 128), (8, 8, 64), (40, 2, 64)])
def test_f32_decode_split_kv_pin(hq, hkv, d):
    """fp32 decode at partition sizes 16, 32 and 256 (padded grid and host
    plan) and in one pass (partition >= the longest context): each within
    1e-5 of the oracle, and each within 1e-6 (relative to max |O|) of the
    single pass."""
    say(f"case: fp32 decode {hq}/{hkv} heads, D {d}")
    case = decode_case(41, len(LENGTHS), 1, 3000, hq=hq, hkv=hkv, d=d, dtype=F32, lengths=LENGTHS)
    kc, vc = build_decode_pool(case, DEV, dtype=F32, fill=float("nan"))   # NaN past every context
    ref, _ = oracle.decode(to_f64(case.q), [to_f64(k) for k in case.k], [to_f64(v) for v in case.v])
    one = decode_f32(case, kc, vc, 3008)
    check(one, ref, F32, "single pass")
    scale = np.abs(one).max()
    for part, plan in ((16, False), (32, True), (256, False), (256, True)):
        o = decode_f32(case, kc, vc, part, plan)
        check(o, ref, F32, f"partition {part}{' (plan)' if plan else ''}")
        rel = np.abs(o - one).max() / scale
        say(f"  partition {part}: max |merged - single pass| / max |O| {rel:.2e}")
        assert rel <= 1e-6


def test_f32_decode_noalloc_and_c3_shape():
    """The 64-sequence shape in fp32 (automatic partition), through the
    workspace and through the library's fixed scratch."""
    say("case: fp32 decode, 64 seqs U[128, 4096]")
    case = decode_case(1002, 64, 128, 4096, dtype=F32)
    kc, vc = build_decode_pool(case, DEV, dtype=F32)
    ref, _ = oracle.decode(to_f64(case.q), [to_f64(k) for k in case.k], [to_f64(v) for v in case.v])
    o = decode_f32(case, kc, vc, 0)
    check(o, ref, F32, "fp32 64 seqs")
    q = case.q.to(DEV)
    o2 = torch.empty_like(q)
    mi.attn_decode_paged_noalloc(q, kc, vc, torch.from_numpy(case.block_tables).to(DEV),
                                 torch.from_numpy(case.lengths.astype(np.int32)).to(DEV), int(case.lengths.max()), o2)
    torch.cuda.synchronize()
    assert np.array_equal(f64(o2.cpu()), o)


def run_paged_f32(qs, bt, kc, vc, total, causal=True, mask=None):
    q = torch.cat(qs).to(DEV)
    cu = np.concatenate([[0], np.cumsum([x.shape[0] for x in qs])]).astype(np.int32)
    args = (q, kc, vc, torch.from_numpy(bt).to(DEV), torch.from_numpy(cu).to(DEV),
            torch.from_numpy(total.astype(np.int32)).to(DEV), int(np.diff(cu).max()))
    if mask is None:
        o = mi.attn_prefill_paged(*args, causal=causal)
    else:
        o = mi.attn_prefill_paged_masked(*args, mask, causal=causal)
    torch.cuda.synchronize()
    return f64(o.cpu())


@pytest.mark.parametrize("cached,new,hq,hkv,d,causal", [
    ([0], [1], 12, 2, 128, True),
    ([5], [64], 12, 2, 128, True),
    ([0, 100, 1, 300], [300, 17, 128, 5], 12, 2, 128, True),
    ([17, 40], [129, 70], 6, 6, 64, True),
    ([40, 0], [30, 70], 4, 1, 128, False),
])
def test_f32_chunked_prefill(cached, new, hq, hkv, d, causal):
    say(f"case: fp32 paged prefill cached {cached} new {new} {hq}/{hkv} D {d} causal {causal}")
    qs, ks, vs, bt, kc, vc, total = paged_setup(170 + sum(cached), cached, new, hq=hq, hkv=hkv, d=d, dtype=F32)
    o = run_paged_f32(qs, bt, kc, vc, total, causal=causal)
    refs = [oracle.attention(to_f64(q)[None], to_f64(k)[None], to_f64(v)[None], causal=causal)[0][0]
            for q, k, v in zip(qs, ks, vs)]
    check(o, np.concatenate(refs), F32, "fp32 chunked")


def test_f32_masked_paged_prefill():
    """The paged mask in fp32: per-head rows, keys past mask_keys masked out,
    one (row, head) with every key masked."""
    from tests.test_gpu_prefill_mask import paged_mask_reference
    cached, new, hq = [40, 260], [90, 33], 4
    say("case: fp32 masked paged prefill")
    qs, ks, vs, bt, kc, vc, total = paged_setup(215, cached, new, hq=hq, hkv=2, d=128, dtype=F32)
    kmax = 200
    mask = additive_mask(216, (sum(new), hq, kmax), amp=3.0, p_masked=0.25)
    mask[5, 1, :] = -np.inf
    o = run_paged_f32(qs, bt, kc, vc, total, causal=False, mask=mask.to(DEV))
    ref = paged_mask_reference(qs, ks, vs, mask.numpy().astype(np.float64), False)
    assert np.all(o[5, 1] == 0.0)
    check(o, ref, F32, "fp32 masked paged")
