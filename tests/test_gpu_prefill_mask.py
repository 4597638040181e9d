"""Contiguous prefill with a general additive mask (attn_prefill_masked):
softmax(Q K^T / sqrt(d) + M) V against the fp64 oracle, which adds the same
M to its materialised scores."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, bf16_ulp, check, f64, say
from tests.test_gpu_prefill import LSE_BF16, LSE_F32
from workloads import additive_mask, prefill_case, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def oracle_masked(q, k, v, mask4, causal):
    """Per (batch, query head): the oracle on one head with its own mask.
    Also returns P|V| (the weights times |V|), which bounds the effect of
    rounding the weights."""
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    b, tq, hq, d = q64.shape
    g = hq // k64.shape[2]
    m = np.broadcast_to(mask4.numpy().astype(np.float64), (b, hq, tq, k64.shape[1]))
    out = np.zeros_like(q64)
    pv_abs = np.zeros_like(q64)
    lse = np.zeros((b, hq, tq))
    for bi in range(b):
        for h in range(hq):
            vv = v64[bi:bi + 1, :, h // g:h // g + 1]
            o, l_, p = oracle.attention(q64[bi:bi + 1, :, h:h + 1], k64[bi:bi + 1, :, h // g:h // g + 1], vv,
                                        causal=causal, mask=m[bi, h], return_probs=True)
            out[bi, :, h] = o[0, :, 0]
            lse[bi, h] = l_[0, 0]
            pv_abs[bi, :, h] = p[0, 0] @ np.abs(vv[0, :, 0])
    return out, lse, pv_abs


def device_mask(mask):
    """The mask on the GPU with its rows padded to a multiple of 4 floats
    (the library reads four consecutive mask entries at a time)."""
    tk = mask.shape[-1]
    buf = torch.zeros(*mask.shape[:-1], (tk + 3) // 4 * 4, dtype=torch.float32, device=DEV)
    buf[..., :tk] = mask.to(DEV)
    return buf[..., :tk]


def check_rounding_bound(out, ref, pv_abs, what):
    """bf16 under a strong mask: a row left a few keys has weights far from
    uniform, and the two bf16 roundings the method makes dominate, so the bar
    is derived per element from them: the weights, each moved by at most a
    relative 2**-8 (8 significant bits) and normalised by their own rounded
    sum, move O by at most 2**-8 (P|V| + |O|); the stored output adds half a
    bf16 ulp of O.  Plus 1e-4 for the fp32 arithmetic.  The mean stays
    within 1e-3."""
    out = np.asarray(out, dtype=np.float64)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref)
    bound = 2.0 ** -8 * (pv_abs + np.abs(ref)) + 0.5 * bf16_ulp(ref) + 1e-4
    worst = (err / bound).max()
    say(f"  {what}: max |err| {err.max():.3e}, max |err| / bound {worst:.3f}, mean |err| {err.mean():.3e}")
    assert worst <= 1.0 and err.mean() <= 1e-3


def check_lse(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    dead = np.isneginf(ref)
    assert np.all(np.isneginf(got[dead])), f"{what}: fully masked rows must give LSE -inf"
    e = np.abs(got[~dead] - ref[~dead])
    bar = LSE_BF16 if dtype == torch.bfloat16 else LSE_F32
    say(f"  {what} LSE: max |err| {e.max():.3e} (bar {bar})")
    assert e.max() <= bar


CASES = [
    # (seed, batch, tq, tk, hq, hkv, d, dtype, causal, mask shape, mask strength)
    (201, 1, 300, 300, 12, 2, 128, torch.bfloat16, True, "qk", "strong"),   # one mask for all heads, causal on top
    (202, 2, 197, 413, 4, 2, 128, torch.bfloat16, False, "bhqk", "strong"),  # per (batch, head), ragged, Tk > Tq
    (203, 1, 130, 130, 6, 6, 64, torch.bfloat16, False, "hqk", "strong"),    # per head, D 64, odd group
    (206, 1, 512, 512, 12, 2, 128, torch.bfloat16, True, "qk", "mild"),      # the plain bf16 bar
    (207, 2, 197, 413, 4, 2, 64, torch.bfloat16, False, "bhqk", "mild"),
    (204, 1, 64, 64, 1, 1, 64, torch.float32, True, "qk", "strong"),         # the single-head fp32 shape
    (205, 2, 100, 250, 4, 1, 128, torch.float32, False, "bhqk", "strong"),
]
STRENGTH = {"strong": dict(amp=3.0, p_masked=0.25), "mild": dict(amp=1.0, p_masked=0.1)}


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_{c[7]}_{c[9]}_{c[10]}" for c in CASES])
def test_masked_prefill(case):
    seed, b, tq, tk, hq, hkv, d, dtype, causal, kind, strength = case
    say(f"case: masked prefill {case}")
    q, k, v = prefill_case(seed, b, tq, hq, hkv, d, dtype, seqlen_k=tk)
    shape = {"qk": (tq, tk), "hqk": (hq, tq, tk), "bhqk": (b, hq, tq, tk)}[kind]
    mask = additive_mask(seed + 1, shape, masked_rows=(3, tq - 1), **STRENGTH[strength])  # two rows see no key
    lse = torch.empty(b, hq, tq, dtype=torch.float32, device=DEV)
    o = mi.attn_prefill_masked(q.to(DEV), k.to(DEV), v.to(DEV), device_mask(mask), lse=lse, causal=causal)
    torch.cuda.synchronize()
    m4 = mask.reshape((1,) * (4 - mask.dim()) + tuple(mask.shape))
    ref, ref_lse, pv_abs = oracle_masked(q, k, v, m4, causal)
    out = f64(o.cpu())
    assert np.all(out[:, [3, tq - 1]] == 0.0), "rows with every key masked give O = 0"
    if dtype == torch.bfloat16 and strength == "strong":
        check_rounding_bound(out, ref, pv_abs, "masked O")
    else:
        check(out, ref, dtype, "masked O")
    check_lse(f64(lse.cpu()), ref_lse, dtype, "masked")


def test_causal_mask_as_additive_mask():
    """The causal mask passed as M (0 / -inf) with causal off gives the
    causal kernel's result within the bf16 bar (T 2048 at 12/2 heads)."""
    say("case: causal as an additive mask, T 2048")
    q, k, v = prefill_case(1001, 1, 2048, 12, 2, 128, torch.bfloat16)
    t = torch.arange(2048)
    m = torch.where(t[None, :] <= t[:, None], 0.0, float("-inf")).to(torch.float32)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_mask = mi.attn_prefill_masked(qd, kd, vd, m.to(DEV), causal=False)
    o_causal = mi.attn_prefill(qd, kd, vd, causal=True, workspace=False)
    torch.cuda.synchronize()
    check(f64(o_mask.cpu()), f64(o_causal.cpu()), torch.bfloat16, "mask vs causal")
    ref, _ = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal=True)
    check(f64(o_mask.cpu()), ref, torch.bfloat16, "mask vs oracle")
