"""Pins for the CPU oracle, checked against things other than itself:
brute force on tiny inputs, PyTorch's own SDPA on the CPU in float64,
closed forms and invariants of exact attention, and the worked block-table
example of the tutorial "Fast Attention Kernels and Operator Fusion"."""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import rng


# ------------------------------------------------------------------ helpers

def brute_attention(q, k, v, mask, scale):
    """Pure-Python triple loop with math.fsum, one head, no max subtraction."""
    tq, d = len(q), len(q[0])
    tk = len(k)
    out = [[0.0] * d for _ in range(tq)]
    for i in range(tq):
        w = []
        for j in range(tk):
            if mask[i][j] == -math.inf:
                w.append(0.0)
                continue
            s = math.fsum(q[i][c] * k[j][c] for c in range(d)) * scale + mask[i][j]
            w.append(math.exp(s))
        z = math.fsum(w)
        for c in range(d):
            out[i][c] = math.fsum(w[j] * v[j][c] for j in range(tk)) / z if z > 0 else 0.0
    return np.array(out)


def torch_sdpa_f64(q, k, v, **kw):
    """PyTorch's CPU scaled_dot_product_attention in float64 on [B,T,H,D] arrays."""
    tq = torch.from_numpy(np.ascontiguousarray(q)).transpose(1, 2)
    tk = torch.from_numpy(np.ascontiguousarray(k)).transpose(1, 2)
    tv = torch.from_numpy(np.ascontiguousarray(v)).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, **kw)
    return o.transpose(1, 2).numpy()


# ------------------------------------------------------------------ brute force

@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    g = rng(seed)
    tq = int(g.integers(1, 9))
    tk = int(g.integers(1, 9))
    d = int(g.integers(1, 9))
    q = g.standard_normal((tq, d))
    k = g.standard_normal((tk, d))
    v = g.standard_normal((tk, d))
    # random additive mask: finite offsets and -inf holes; keep one key per row
    mask = g.standard_normal((tq, tk))
    holes = g.random((tq, tk)) < 0.3
    holes[np.arange(tq), g.integers(0, tk, size=tq)] = False
    mask = np.where(holes, -np.inf, mask)
    scale = 1.0 / math.sqrt(d)
    ref = brute_attention(q.tolist(), k.tolist(), v.tolist(), mask.tolist(), scale)
    o, _ = oracle.attention(q[None, :, None, :], k[None, :, None, :], v[None, :, None, :],
                            causal=False, mask=mask)
    np.testing.assert_allclose(o[0, :, 0, :], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_causal_gqa(seed):
    g = rng(100 + seed)
    tq = int(g.integers(1, 7))
    tk = tq + int(g.integers(0, 4))
    d = 4
    hkv = 2
    hq = 6
    q = g.standard_normal((1, tq, hq, d))
    k = g.standard_normal((1, tk, hkv, d))
    v = g.standard_normal((1, tk, hkv, d))
    o, _ = oracle.attention(q, k, v, causal=True)
    for h in range(hq):
        kv = h // 3
        mask = [[0.0 if j <= i + (tk - tq) else -math.inf for j in range(tk)] for i in range(tq)]
        ref = brute_attention(q[0, :, h].tolist(), k[0, :, kv].tolist(), v[0, :, kv].tolist(), mask,
                              1.0 / math.sqrt(d))
        np.testing.assert_allclose(o[0, :, h], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ library routine

def test_sdpa_c1_shape():
    """Single head, T 64, D 64, causal, scale 1/8: the library routine agrees."""
    g = rng(7)
    q, k, v = (g.standard_normal((1, 64, 1, 64)) for _ in range(3))
    o, _ = oracle.attention(q, k, v, causal=True)
    ref = torch_sdpa_f64(q, k, v, is_causal=True)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    o2, _ = oracle.attention(q, k, v, causal=True, scale=0.125)
    np.testing.assert_allclose(o2, o, rtol=0, atol=0)


def test_sdpa_tutorial_shape():
    """The tutorial's SDPA example shape (2, 16, 512, 64), causal."""
    g = rng(8)
    q, k, v = (g.standard_normal((2, 512, 16, 64)) for _ in range(3))
    o, _ = oracle.attention(q, k, v, causal=True)
    ref = torch_sdpa_f64(q, k, v, is_causal=True)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_sdpa_gqa_and_bottom_right():
    """GQA head mapping and bottom-right causal alignment, against torch's
    enable_gqa and causal_lower_right bias."""
    from torch.nn.attention.bias import causal_lower_right
    g = rng(9)
    tq, tk = 37, 101
    q = g.standard_normal((1, tq, 12, 32))
    k = g.standard_normal((1, tk, 2, 32))
    v = g.standard_normal((1, tk, 2, 32))
    o, _ = oracle.attention(q, k, v, causal=True)
    tq_ = torch.from_numpy(q).transpose(1, 2)
    tk_ = torch.from_numpy(k).transpose(1, 2).repeat_interleave(6, dim=1)
    tv_ = torch.from_numpy(v).transpose(1, 2).repeat_interleave(6, dim=1)
    bias = causal_lower_right(tq, tk)
    ref = torch.nn.functional.scaled_dot_product_attention(tq_, tk_, tv_, attn_mask=bias)
    np.testing.assert_allclose(o, ref.transpose(1, 2).numpy(), rtol=0, atol=1e-12)
    keep = torch.ones(tq, tk, dtype=torch.bool).tril(diagonal=tk - tq)
    ref2 = torch_sdpa_f64(q, k, v, attn_mask=keep, enable_gqa=True)
    np.testing.assert_allclose(o, ref2, rtol=0, atol=1e-12)


def test_lse_matches_logsumexp():
    g = rng(10)
    q, k, v = (g.standard_normal((1, 20, 2, 8)) for _ in range(3))
    _, lse = oracle.attention(q, k, v, causal=True)
    ql = torch.from_numpy(q[0]).transpose(0, 1)
    kl = torch.from_numpy(k[0]).transpose(0, 1)
    s = ql @ kl.transpose(1, 2) / math.sqrt(8)
    s = s + torch.full((20, 20), -math.inf, dtype=torch.float64).triu(1)
    np.testing.assert_allclose(lse[0], torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ invariants

def test_rows_sum_to_one_and_causal_zeros():
    g = rng(11)
    q, k, v = (g.standard_normal((1, 64, 1, 64)) for _ in range(3))
    _, _, p = oracle.attention(q, k, v, causal=True, return_probs=True)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.triu(p[0, 0], 1) == 0.0)
    # V = I returns P itself
    o, _ = oracle.attention(q, k, np.eye(64)[None, :, None, :], causal=True)
    np.testing.assert_allclose(o[0, :, 0, :], p[0, 0], rtol=0, atol=1e-15)


def test_constant_v_and_first_row():
    g = rng(12)
    q = g.standard_normal((2, 33, 4, 16))
    k = g.standard_normal((2, 33, 2, 16))
    c = g.standard_normal(16)
    v = np.broadcast_to(c, (2, 33, 2, 16)).copy()
    o, _ = oracle.attention(q, k, v, causal=True)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)
    v2 = g.standard_normal((2, 33, 2, 16))
    o2, _ = oracle.attention(q, k, v2, causal=True)
    for h in range(4):
        np.testing.assert_array_equal(o2[:, 0, h, :], v2[:, 0, h // 2, :])


def test_affine_in_v():
    g = rng(13)
    q, k, v = (g.standard_normal((1, 17, 2, 8)) for _ in range(3))
    a, b = 2.5, g.standard_normal(8)
    o1, _ = oracle.attention(q, k, v, causal=True)
    o2, _ = oracle.attention(q, k, a * v + b, causal=True)
    np.testing.assert_allclose(o2, a * o1 + b, rtol=0, atol=1e-13)


def test_key_permutation_noncausal():
    g = rng(14)
    q, k, v = (g.standard_normal((1, 23, 3, 8)) for _ in range(3))
    perm = g.permutation(23)
    o1, l1 = oracle.attention(q, k, v, causal=False)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm], causal=False)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_gqa_equals_repeated_mha():
    g = rng(15)
    q = g.standard_normal((1, 19, 12, 16))
    k = g.standard_normal((1, 19, 2, 16))
    v = g.standard_normal((1, 19, 2, 16))
    o1, _ = oracle.attention(q, k, v, causal=True)
    o2, _ = oracle.attention(q, np.repeat(k, 6, axis=2), np.repeat(v, 6, axis=2), causal=True)
    np.testing.assert_array_equal(o1, o2)


def test_fully_masked_row_is_zero():
    q = np.ones((1, 2, 1, 4))
    k = np.ones((1, 3, 1, 4))
    v = np.ones((1, 3, 1, 4))
    mask = np.array([[0.0, -np.inf, -np.inf], [-np.inf, -np.inf, -np.inf]])
    o, lse = oracle.attention(q, k, v, causal=False, mask=mask)
    assert np.all(o[0, 1] == 0.0) and lse[0, 0, 1] == -np.inf
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])


def test_rows_subset_matches_full():
    g = rng(16)
    q = g.standard_normal((1, 300, 4, 16))
    k = g.standard_normal((1, 300, 2, 16))
    v = g.standard_normal((1, 300, 2, 16))
    o, lse = oracle.attention(q, k, v, causal=True)
    rows = np.array([0, 1, 57, 128, 299])
    o2, l2 = oracle.attention_rows(q[0], k[0], v[0], rows, chunk=2)
    np.testing.assert_allclose(o2, o[0, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, lse[0][:, rows].T, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ split KV, decode, chunks

@pytest.mark.parametrize("nparts", [1, 2, 5])
def test_merge_lse_equals_single_pass(nparts):
    g = rng(20 + nparts)
    tk = 80
    q = g.standard_normal((1, 1, 6, 16))
    k = g.standard_normal((1, tk, 1, 16))
    v = g.standard_normal((1, tk, 1, 16))
    o_full, l_full = oracle.attention(q, k, v, causal=False)
    cuts = np.sort(g.choice(np.arange(1, tk), size=nparts - 1, replace=False)) if nparts > 1 else []
    edges = [0, *cuts, tk]
    parts = []
    for a, b in zip(edges[:-1], edges[1:]):
        o_p, l_p = oracle.attention(q, k[:, a:b], v[:, a:b], causal=False)
        parts.append((o_p, l_p.transpose(0, 2, 1)))      # LSE laid out like O[..., 0]
    # an empty subset contributes nothing
    parts.append((np.zeros_like(o_full), np.full(o_full.shape[:-1], -np.inf)))
    o, lse = oracle.merge_lse(parts)
    np.testing.assert_allclose(o, o_full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, l_full.transpose(0, 2, 1), rtol=0, atol=1e-13)


def test_decode_is_last_row_of_prefill():
    g = rng(30)
    t = 45
    q = g.standard_normal((1, t, 12, 16))
    k = g.standard_normal((1, t, 2, 16))
    v = g.standard_normal((1, t, 2, 16))
    o, _ = oracle.attention(q, k, v, causal=True)
    for row in (0, 7, 44):
        od, _ = oracle.decode(q[0, row][None], [k[0, :row + 1]], [v[0, :row + 1]])
        np.testing.assert_allclose(od[0], o[0, row], rtol=0, atol=1e-14)


def test_chunk_is_rows_of_full_prefill():
    g = rng(31)
    c, n = 37, 20
    q = g.standard_normal((1, c + n, 12, 16))
    k = g.standard_normal((1, c + n, 2, 16))
    v = g.standard_normal((1, c + n, 2, 16))
    o, _ = oracle.attention(q, k, v, causal=True)
    oc = oracle.chunked_prefill([q[0, c:]], [k[0]], [v[0]])[0]
    np.testing.assert_allclose(oc, o[0, c:], rtol=0, atol=1e-14)


# ------------------------------------------------------------------ bf16 rounding

def test_round_bf16_matches_torch_on_float32_values():
    g = rng(40)
    x = g.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** g.integers(-3, 4, 100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    # 1 + 2**-8 is the midpoint between 1 and 1 + 2**-7: ties go to the even 1.0.
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2**-8 is the midpoint between 1 + 2**-7 (odd) and 1 + 2**-6 (even).
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert oracle.round_bf16(np.array([-(1.0 + 2.0 ** -8 + 2.0 ** -30)]))[0] == -(1.0 + 2.0 ** -7)


# ------------------------------------------------------------------ RoPE

def test_rope_d2_closed_form():
    for p in (0, 1, 3, 1000, 32767):
        r = oracle.rope(np.array([[[1.0, 0.0]]]), np.array([p]))
        np.testing.assert_allclose(r[0, 0], [math.cos(p), math.sin(p)], rtol=0, atol=1e-12)


def test_rope_d4_frequencies_and_pairing():
    base = 10000.0
    p = 7
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]])   # pair (x[1], x[3]) uses angle p * base**(-1/2)
    r = oracle.rope(x, np.array([p]), base)
    a = p / math.sqrt(base)
    np.testing.assert_allclose(r[0, 0], [0.0, math.cos(a), 0.0, math.sin(a)], rtol=0, atol=1e-15)


def test_rope_properties():
    g = rng(41)
    x = g.standard_normal((5, 3, 128))
    y = g.standard_normal((5, 3, 128))
    zero = oracle.rope(x, np.zeros(5))
    np.testing.assert_array_equal(zero, x)
    a = g.integers(0, 30000, 5)
    b = g.integers(0, 3000, 5)
    ra = oracle.rope(x, a)
    half = 64
    np.testing.assert_allclose(ra[..., :half] ** 2 + ra[..., half:] ** 2,
                               x[..., :half] ** 2 + x[..., half:] ** 2, rtol=1e-12)
    np.testing.assert_allclose(oracle.rope(ra, b), oracle.rope(x, a + b), rtol=0, atol=1e-9)
    m, n = a, b
    lhs = np.sum(oracle.rope(x, m) * oracle.rope(y, n), axis=-1)
    rhs = np.sum(oracle.rope(x, m - n) * y, axis=-1)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-9)


# ------------------------------------------------------------------ paged cache

def _read_block_table_fixture(golden_dir):
    rows = {}
    with open(os.path.join(golden_dir, "paged_block_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows[key] = [int(x) for x in vals]
    return rows


def test_worked_block_table_example(golden_dir):
    tab = _read_block_table_fixture(golden_dir)
    assert tab["logical"] == [0, 1, 2, 3]
    phys = tab["physical"]
    assert phys == [17, 4, 29, 8]
    g = rng(50)
    bs, hkv, d = 16, 2, 8
    T = 64
    k = g.standard_normal((T, hkv, d))
    v = g.standard_normal((T, hkv, d))
    kc0 = np.full((30, hkv, bs, d), 7.0)
    vc0 = np.full((30, hkv, d, bs), 7.0)
    slots = np.array([phys[t // bs] * bs + t % bs for t in range(T)])
    kc, vc = oracle.kv_cache_write_expected(kc0, vc0, k, v, np.arange(T), slots, rope_base=0.0, bf16=False)
    np.testing.assert_array_equal(oracle.gather_paged(kc, phys, T), k)
    np.testing.assert_array_equal(oracle.gather_paged(vc, phys, T, token_minor=True), v)
    untouched = [b for b in range(30) if b not in phys]
    assert np.all(kc[untouched] == 7.0) and np.all(vc[untouched] == 7.0)
    # logical token 16 is the first row of physical block 4
    np.testing.assert_array_equal(kc[4, :, 0, :], k[16])


def test_cache_write_rotates_keys_only_and_skips():
    g = rng(51)
    n, hkv, d, bs, nb = 10, 2, 8, 16, 4
    k = g.standard_normal((n, hkv, d))
    v = g.standard_normal((n, hkv, d))
    pos = g.integers(0, 100, n)
    slots = g.permutation(nb * bs)[:n]
    slots[3] = -1
    kc, vc = oracle.kv_cache_write_expected(np.zeros((nb, hkv, bs, d)), np.zeros((nb, hkv, d, bs)),
                                            k, v, pos, slots, rope_base=10000.0, bf16=False)
    kr = oracle.rope(k, pos)
    for i in range(n):
        if slots[i] < 0:
            continue
        np.testing.assert_array_equal(kc[slots[i] // bs, :, slots[i] % bs], kr[i])
        np.testing.assert_array_equal(vc[slots[i] // bs, :, :, slots[i] % bs], v[i])
    assert np.count_nonzero(np.abs(kc).sum(axis=-1)) == (n - 1) * hkv


# ------------------------------------------------------------------ fused residual + RMSNorm

def brute_rms_norm(x, r, w, eps):
    """Pure-Python loops with math.fsum: one row at a time."""
    out, hs = [], []
    for xi, ri in zip(x, r):
        h = [float(np.float32(a) + np.float32(b)) for a, b in zip(xi, ri)]
        ms = math.fsum(v * v for v in h) / len(h)
        out.append([v / math.sqrt(ms + eps) * wj for v, wj in zip(h, w)])
        hs.append(h)
    return np.array(out), np.array(hs)


def test_rms_norm_brute_force():
    g = rng(71)
    x, r = g.standard_normal((5, 24)), g.standard_normal((5, 24))
    w = g.standard_normal(24)
    y, h = oracle.residual_rms_norm(x, r, w, eps=1e-3, bf16=False)
    yb, hb = brute_rms_norm(x, r, w, 1e-3)
    np.testing.assert_allclose(h, hb, rtol=0, atol=0)
    np.testing.assert_allclose(y, yb, rtol=1e-13, atol=1e-14)


def test_rms_norm_one_hot_closed_form():
    """A row whose sum is a * e_k: mean square a^2 / H, so the output is
    a w_k / sqrt(a^2 / H + eps) at k and 0 elsewhere."""
    H, a, k, eps = 16, 3.0, 5, 1e-6
    x = np.zeros((1, H)); r = np.zeros((1, H)); x[0, k] = 1.0; r[0, k] = a - 1.0
    w = np.arange(1, H + 1, dtype=np.float64)
    y, h = oracle.residual_rms_norm(x, r, w, eps=eps)
    want = np.zeros(H); want[k] = a * w[k] / math.sqrt(a * a / H + eps)
    np.testing.assert_allclose(y[0], want, rtol=1e-15, atol=0)
    assert h[0, k] == a


def test_rms_norm_invariants():
    """With unit weights each output row has root mean square
    sqrt(ms / (ms + eps)); the map commutes with a permutation of the hidden
    dimension (weights permuted alike); with eps = 0 it is invariant to
    scaling the row by a power of two (exact in float32 and bf16)."""
    g = rng(72)
    x, r = g.standard_normal((6, 40)), g.standard_normal((6, 40))
    eps = 1e-2
    y, h = oracle.residual_rms_norm(x, r, np.ones(40), eps=eps)
    ms = np.mean(h * h, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-14)
    w = g.standard_normal(40)
    perm = g.permutation(40)
    y1, _ = oracle.residual_rms_norm(x, r, w)
    y2, _ = oracle.residual_rms_norm(x[:, perm], r[:, perm], w[perm])
    np.testing.assert_allclose(y2, y1[:, perm], rtol=1e-14, atol=0)
    y3, _ = oracle.residual_rms_norm(8 * x, 8 * r, w, eps=0.0)
    y4, _ = oracle.residual_rms_norm(x, r, w, eps=0.0)
    np.testing.assert_allclose(y3, y4, rtol=1e-14, atol=0)


def test_rms_norm_stored_residual_is_bf16_of_the_float32_sum():
    """The updated residual: 1 + 2^-8 (exact in float32) rounds to nearest
    even in bf16 (to 1.0); 1 + 3 * 2^-8 rounds up to 1 + 2^-6."""
    x = np.array([[1.0, 1.0]])
    r = np.array([[2.0 ** -8, 3 * 2.0 ** -8]])
    _, h = oracle.residual_rms_norm(x, r, np.ones(2))
    assert h[0, 0] == 1.0 and h[0, 1] == 1.0 + 2.0 ** -6
