"""Parity of the contiguous prefill kernel (attn_prefill) with the fp64
oracle, on the same seeded host inputs."""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, check_bf16_output, f64, say
from workloads import prefill_case, rng, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


# LSE bar.  bf16 path: the row sum accumulates the bf16-rounded weights that
# feed the PV product.  bf16 carries 8 significant bits, so rounding to
# nearest moves a weight by at most half an ulp, a relative 2**-8 at the
# bottom of a binade; hence |LSE - exact| <= ln(1 + 2**-8) ~ 3.9e-3 plus fp32
# rounding.  (Averaged over many keys the errors mostly cancel; a row that
# sees only a few keys, as under a strong mask, can come close to the bound.)
# fp32 path: 1e-5.
LSE_BF16 = 4.0e-3
LSE_F32 = 1e-5


def check_lse(got, ref, dtype, what):
    e = np.abs(np.asarray(got, dtype=np.float64) - ref)
    bar = LSE_BF16 if dtype == torch.bfloat16 else LSE_F32
    say(f"  {what} LSE: max |err| {e.max():.3e} (bar {bar})")
    assert e.max() <= bar


def run(q, k, v, causal=True, want_lse=False, scale=0.0, workspace=None):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lse = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=DEV) if want_lse else None
    o = mi.attn_prefill(qd, kd, vd, lse=lse, causal=causal, scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return (o.cpu(), lse.cpu() if want_lse else None)


def test_c1_single_head_f32():
    """Single head, T 64, D 64, fp32, causal, scale 1/8 (seed 1000)."""
    say("case: C1 f32 T64 D64")
    q, k, v = prefill_case(1000, 1, 64, 1, 1, 64, torch.float32)
    o, lse = run(q, k, v, want_lse=True)
    ref, ref_lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=True, scale=0.125)
    check(f64(o), ref, torch.float32, "C1 O")
    check_lse(f64(lse), ref_lse, torch.float32, "C1")


def test_c2_qwen_shape_bf16():
    """T 2048, 12 query / 2 kv heads, D 128, bf16, causal (seed 1001)."""
    say("case: C2 bf16 T2048 Hq12 Hkv2 D128")
    q, k, v = prefill_case(1001, 1, 2048, 12, 2, 128, torch.bfloat16)
    o, lse = run(q, k, v, want_lse=True)
    ref, ref_lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=True)
    check(f64(o), ref, torch.bfloat16, "C2 O")
    check_lse(f64(lse), ref_lse, torch.bfloat16, "C2")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tutorial_sdpa_shape(dtype):
    """(B, H, T, D) = (2, 16, 512, 64), causal: the tutorial's SDPA example,
    passed in its own head-major layout through strides."""
    say(f"case: tutorial shape {dtype}")
    g = rng(7)
    shape = (2, 16, 512, 64)   # (B, H, T, D)
    q, k, v = (torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(dtype) for _ in range(3))
    qd, kd, vd = (t.to(DEV).transpose(1, 2) for t in (q, k, v))   # [B, T, H, D] views
    o = mi.attn_prefill(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(to_f64(q.transpose(1, 2)), to_f64(k.transpose(1, 2)), to_f64(v.transpose(1, 2)))
    check(f64(o), ref, dtype, "tutorial")


CASES = [
    # (tq, tk, hq, hkv, d, causal)
    (1, 1, 1, 1, 64, True),
    (15, 15, 2, 1, 64, True),
    (16, 16, 6, 1, 128, True),
    (17, 17, 12, 2, 128, True),
    (63, 63, 4, 2, 64, True),
    (65, 65, 6, 6, 128, True),
    (127, 127, 12, 2, 128, True),
    (129, 129, 12, 2, 128, True),
    (300, 300, 2, 2, 64, False),
    (1000, 1000, 12, 2, 128, True),
    (37, 101, 12, 2, 128, True),     # bottom-right causal, tq < tk
    (130, 400, 6, 3, 64, True),
    (200, 77, 4, 1, 128, False),     # tk < tq, non-causal
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", CASES, ids=[f"tq{c[0]}_tk{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_{'c' if c[5] else 'nc'}" for c in CASES])
def test_ragged_shapes(case, dtype):
    tq, tk, hq, hkv, d, causal = case
    say(f"case: ragged {case} {dtype}")
    q, k, v = prefill_case(2000 + CASES.index(case), 2, tq, hq, hkv, d, dtype, seqlen_k=tk)
    o, lse = run(q, k, v, causal=causal, want_lse=True)
    ref, ref_lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=causal)
    check(f64(o), ref, dtype, f"ragged {case}")
    check_lse(f64(lse), ref_lse, dtype, "ragged")


# Key counts a multiple of the 64-key tile at D 128 (bf16, no mask): every key
# tile is whole, and the kernel issues each K tile's loads spread over the
# preceding tile's PV phase.  Fewer key tiles than the ring is deep, one query
# row, tq < tk and tq > tk, non-causal, MHA (odd group: the 1 x 4 tile) and
# batches of two.
WHOLE_TILE_CASES = [
    # (batch, tq, tk, hq, hkv, causal)
    (2, 64, 64, 12, 2, True),
    (1, 128, 192, 6, 1, True),
    (1, 1, 1024, 12, 2, True),
    (2, 256, 256, 5, 5, False),
    (1, 100, 640, 4, 2, False),
    (1, 700, 320, 12, 2, False),
    (2, 511, 1024, 12, 2, True),
]


@pytest.mark.parametrize("case", WHOLE_TILE_CASES, ids=[f"b{c[0]}_tq{c[1]}_tk{c[2]}_h{c[3]}x{c[4]}_{'c' if c[5] else 'nc'}"
                                                        for c in WHOLE_TILE_CASES])
def test_whole_key_tiles(case):
    b, tq, tk, hq, hkv, causal = case
    say(f"case: whole key tiles {case}")
    q, k, v = prefill_case(5000 + WHOLE_TILE_CASES.index(case), b, tq, hq, hkv, 128, torch.bfloat16, seqlen_k=tk)
    o, lse = run(q, k, v, causal=causal, want_lse=True)
    ref, ref_lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=causal)
    check_bf16_output(f64(o), ref, f"whole tiles {case}")
    check_lse(f64(lse), ref_lse, torch.bfloat16, "whole tiles")


def test_whole_key_tiles_head_major_strides():
    """(B, H, T, D) = (2, 8, 512, 128) passed through strides (head-major),
    causal: the spread K loads with token strides other than H*D."""
    say("case: whole key tiles, head-major")
    g = rng(8)
    shape = (2, 8, 512, 128)
    q, k, v = (torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16) for _ in range(3))
    qd, kd, vd = (t.to(DEV).transpose(1, 2) for t in (q, k, v))
    o = mi.attn_prefill(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    ref, _ = oracle.attention(to_f64(q.transpose(1, 2)), to_f64(k.transpose(1, 2)), to_f64(v.transpose(1, 2)))
    check_bf16_output(f64(o), ref, "head-major D 128")


SPLIT_CASES = [
    # (batch, tq, tk, hq, hkv, d, causal): few query tiles, many key tiles
    (1, 2048, 2048, 12, 2, 128, True),
    (2, 1000, 1000, 12, 2, 128, True),
    (1, 300, 1800, 4, 2, 64, False),
    (1, 77, 3001, 6, 1, 128, True),
    (3, 129, 1400, 2, 2, 128, True),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"b{c[0]}_tq{c[1]}_tk{c[2]}_h{c[3]}x{c[4]}_d{c[5]}"
                                                   for c in SPLIT_CASES])
def test_split_kv_equals_single_pass(case):
    """Split-KV (key shares on separate workgroups, merged) against the
    oracle and against one pass per query tile, output and LSE."""
    b, tq, tk, hq, hkv, d, causal = case
    say(f"case: split-KV {case}")
    assert mi.attn_prefill_workspace_size(b, tq, tk, hq, hkv, d) > 0   # the plan splits
    q, k, v = prefill_case(4000 + SPLIT_CASES.index(case), b, tq, hq, hkv, d, torch.bfloat16, seqlen_k=tk)
    o_s, lse_s = run(q, k, v, causal=causal, want_lse=True)
    o_1, lse_1 = run(q, k, v, causal=causal, want_lse=True, workspace=False)
    ref, ref_lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=causal)
    check(f64(o_s), ref, torch.bfloat16, "split O")
    check(f64(o_1), ref, torch.bfloat16, "one-pass O")
    check_lse(f64(lse_s), ref_lse, torch.bfloat16, "split")
    check(f64(o_s), f64(o_1), torch.bfloat16, "split vs one pass")


def test_explicit_scale():
    q, k, v = prefill_case(3, 1, 100, 4, 2, 64, torch.float32)
    o, _ = run(q, k, v, scale=0.3)
    ref, _ = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=True, scale=0.3)
    check(f64(o), ref, torch.float32, "scale 0.3")


# ------------------------------------------------------------------ invariants on the GPU

def test_identity_v_gives_probabilities_f32():
    """V = I (T = D = 64): O is the probability matrix itself.  Rows sum to 1,
    entries above the diagonal are exactly 0, and P equals the oracle's."""
    say("case: V = I")
    q, k, _ = prefill_case(1000, 1, 64, 1, 1, 64, torch.float32)
    v = torch.eye(64, dtype=torch.float32)[None, :, None, :]
    o, _ = run(q, k, v)
    p = f64(o)[0, :, 0, :]
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-5)
    assert np.all(np.triu(p, 1) == 0.0)
    _, _, ref_p = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=True, return_probs=True)
    np.testing.assert_allclose(p, ref_p[0, 0], rtol=0, atol=1e-5)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_constant_v_and_first_row(dtype):
    say(f"case: constant V {dtype}")
    q, k, v = prefill_case(11, 1, 333, 12, 2, 128, dtype)
    c = v[:, :1].clone()
    vc = c.expand_as(v).contiguous()
    o, _ = run(q, k, vc)
    want = f64(c).repeat(6, axis=2)     # head h reads kv head h // 6
    if dtype == torch.bfloat16:
        # rows are convex combinations of one bf16 vector: exact up to output rounding
        assert np.array_equal(f64(o), np.broadcast_to(want, o.shape))
    else:
        np.testing.assert_allclose(f64(o), np.broadcast_to(want, o.shape), rtol=0, atol=1e-5)
    o2, _ = run(q, k, v)
    # first causal row is V[0] exactly
    np.testing.assert_array_equal(f64(o2)[:, 0], f64(v)[:, 0].repeat(6, axis=1))


def test_gqa_equals_repeated_heads():
    q, k, v = prefill_case(12, 1, 200, 12, 2, 128, torch.bfloat16)
    o1, _ = run(q, k, v)
    o2, _ = run(q, k.repeat_interleave(6, dim=2), v.repeat_interleave(6, dim=2))
    assert torch.equal(o1, o2)


def test_c4_long_prefill_sampled_rows():
    """T 16384, 12/2 heads, D 128, bf16, causal (seed 1003), the benchmark's
    launch: sampled rows against the oracle, computed one row at a time."""
    say("case: C4 T16384 sampled rows")
    q, k, v = prefill_case(1003, 1, 16384, 12, 2, 128, torch.bfloat16)
    o, lse = run(q, k, v, want_lse=True)
    g = rng(99)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 129, 8191, 8192, 16255, 16256, 16383],
                                     g.integers(0, 16384, 36)]))
    ref, ref_lse = oracle.attention_rows(to_f64(q[0]), to_f64(k[0]), to_f64(v[0]), rows, chunk=16)
    check(f64(o)[0, rows], ref, torch.bfloat16, "C4 rows")
    check_lse(f64(lse)[0][:, rows].T, ref_lse, torch.bfloat16, "C4 rows")
    # every row finite; first row exact
    assert torch.isfinite(o).all()
    np.testing.assert_array_equal(f64(o)[0, 0], f64(v)[0, 0].repeat(6, axis=0))
