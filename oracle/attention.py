"""CPU oracle for exact scaled-dot-product attention, paged decode, chunked
prefill and the fused RoPE + paged KV-cache write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code with the HIP library (no kernels, headers, tables or
helpers); its inputs are the same host arrays the GPU path receives.

Everything is NumPy float64.  The functions materialise the full score rows
on purpose: this is the plain definition, not the tiled method.

Source: the tutorial "Fast Attention Kernels and Operator Fusion"
(Machine Learning Mastery).  Citations below name its sections.

Readings of points the page leaves open:
  * d in 1/sqrt(d) is the head dimension.
  * The mask M is additive with entries 0 or -inf; "causal" keeps key j
    visible to query i iff j <= i + (Tk - Tq) (bottom-right alignment, the
    only reading under which a prefill chunk equals rows of the full prefill).
  * Grouped-query heads: query head h reads key/value head h // (Hq // Hkv).
  * A row with no visible key returns 0 and LSE = -inf.
  * RoPE uses the half-split pairing (x[i], x[i + D/2]) with angle
    pos * base**(-2i/D).  The page only names the fusion, so the pairing
    convention is a reading; its parity is unpinned beyond the closed-form
    properties the tests check.
  * Values the method stores into a bf16 buffer (the rotated keys in the
    cache, the rotated queries written back in place) are rounded to bf16
    with round-to-nearest-even before later steps read them.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "attention",
    "attention_rows",
    "merge_lse",
    "rope",
    "round_bf16",
    "kv_cache_write_expected",
    "decode",
    "chunked_prefill",
    "gather_paged",
]


def _scale(d: int, scale: float | None) -> float:
    # "Fast Attention Kernels and Operator Fusion", §FlashAttention-Style
    # Kernels, attention equation: scores are divided by sqrt(d).
    return 1.0 / math.sqrt(d) if not scale else float(scale)


def _causal_mask(tq: int, tk: int, rows: np.ndarray | None = None) -> np.ndarray:
    """Additive mask M (0 / -inf), bottom-right aligned.

    §FlashAttention-Style Kernels uses an additive mask M and the causal flag;
    query i sits at absolute position (tk - tq) + i and sees keys j <= that.
    """
    qi = np.arange(tq) if rows is None else np.asarray(rows)
    pos = qi[:, None] + (tk - tq)
    kj = np.arange(tk)[None, :]
    return np.where(kj <= pos, 0.0, -np.inf)


def _softmax_rows(s: np.ndarray):
    """Row softmax with max subtraction; returns (P, lse).

    Max subtraction is exact in real arithmetic: softmax(s) = softmax(s - c).
    A row that is entirely -inf yields P = 0 and lse = -inf.
    """
    m = np.max(s, axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    z = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)
        lse = np.where(z[..., 0] > 0, m_safe[..., 0] + np.log(np.where(z[..., 0] > 0, z[..., 0], 1.0)), -np.inf)
    return p, lse


def attention(q, k, v, causal=True, scale=None, mask=None, return_probs=False):
    """O = softmax(Q K^T / sqrt(d) + M) V for every batch and query head.

    Layout is token-major, as the library takes it: q [B, Tq, Hq, D],
    k and v [B, Tk, Hkv, D].  Returns (O [B, Tq, Hq, D], LSE [B, Hq, Tq]) and,
    if asked, P [B, Hq, Tq, Tk].

    Follows the attention equation of §FlashAttention-Style Kernels exactly:
    the full Tq x Tk score matrix is materialised per head (the "simple
    implementation" that the same section describes), then a row softmax,
    then the product with V.  ``mask`` is an optional additive [Tq, Tk] (or
    broadcastable) array added on top of the causal mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, tq, hq, d = q.shape
    _, tk, hkv, _ = k.shape
    assert hq % hkv == 0
    grp = hq // hkv
    sc = _scale(d, scale)
    m_add = np.zeros((tq, tk))
    if causal:
        m_add = m_add + _causal_mask(tq, tk)
    if mask is not None:
        m_add = m_add + np.asarray(mask, dtype=np.float64)
    out = np.zeros((b, tq, hq, d))
    lse = np.zeros((b, hq, tq))
    probs = np.zeros((b, hq, tq, tk)) if return_probs else None
    for bi in range(b):
        for h in range(hq):
            g = h // grp
            s = (q[bi, :, h, :] @ k[bi, :, g, :].T) * sc + m_add
            p, l_ = _softmax_rows(s)
            out[bi, :, h, :] = p @ v[bi, :, g, :]
            lse[bi, h, :] = l_
            if return_probs:
                probs[bi, h] = p
    if return_probs:
        return out, lse, probs
    return out, lse


def attention_rows(q, k, v, rows, heads=None, causal=True, scale=None, chunk=1024):
    """Selected query rows of :func:`attention` for one batch element.

    q [Tq, Hq, D], k and v [Tk, Hkv, D].  Each requested row still gets its
    full Tk-wide score vector (the definition is per row); rows are processed
    ``chunk`` at a time only to bound memory.  Returns O [len(rows), nh, D] and
    LSE [len(rows), nh] for heads ``heads`` (default all).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = hq // hkv
    rows = np.asarray(rows, dtype=np.int64)
    heads = list(range(hq)) if heads is None else list(heads)
    sc = _scale(d, scale)
    out = np.zeros((len(rows), len(heads), d))
    lse = np.zeros((len(rows), len(heads)))
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        m_add = _causal_mask(tq, tk, rr) if causal else 0.0
        for hi, h in enumerate(heads):
            g = h // grp
            s = (q[rr, h, :] @ k[:, g, :].T) * sc + m_add
            p, l_ = _softmax_rows(s)
            out[c0:c0 + len(rr), hi, :] = p @ v[:, g, :]
            lse[c0:c0 + len(rr), hi] = l_
    return out, lse


def merge_lse(parts):
    """Combine attention over disjoint key subsets.

    ``parts`` is a list of (O_p, LSE_p) with O_p already normalised over its
    own subset and LSE_p shaped like O_p without its last axis.  Since softmax over the union weights subset p by
    exp(LSE_p - LSE), the exact result is O = sum_p exp(LSE_p - LSE) O_p with
    LSE = log sum_p exp(LSE_p).  This is the running-max / running-sum
    statistic of §FlashAttention-Style Kernels applied to whole subsets.
    Empty subsets carry LSE = -inf and contribute nothing.
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    os_ = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    m = np.max(lses, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lses - m_safe)
    z = np.sum(w, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(z[..., None] > 0, np.sum(w[..., None] * os_, axis=0) / np.where(z > 0, z, 1.0)[..., None], 0.0)
        lse = np.where(z > 0, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return o, lse


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even).

    bfloat16 keeps 8 significant bits and float32's exponent range; the
    rounding is done directly from float64 (no float32 double rounding).
    Only normal-range finite values occur in these workloads.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, ex = np.frexp(x)  # x = mant * 2**ex, 0.5 <= |mant| < 1
    return np.ldexp(np.rint(mant * 256.0), ex - 8)


def rope(x, positions, base=10000.0):
    """Rotary position embedding in float64.

    §Operator Fusion counts the rotary embedding of queries and keys among
    its fusion targets but gives no formula; the reading used here
    is the half-split form: for i < D/2, the pair (x[i], x[i + D/2]) is
    rotated by angle pos * base**(-2i/D).  x is [N, H, D], positions [N].
    """
    x = np.asarray(x, dtype=np.float64)
    n, h, d = x.shape
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def kv_cache_write_expected(k_cache, v_cache, k, v, positions, slot_mapping,
                            rope_base=10000.0, bf16=True):
    """Expected paged caches after the fused RoPE + KV-cache write.

    §Operator Fusion counts the KV-cache update made as keys and values are
    transformed among its fusion targets; §Paged Attention Kernels fixes the
    storage as fixed-size
    blocks addressed through a table.  Token n with slot s >= 0 lands in
    physical block s // bs at offset s % bs.  Cache layouts (the library's):
    k_cache [NB, Hkv, bs, D] and v_cache [NB, Hkv, D, bs] (values stored
    token-minor inside a block).  Keys are rotated (unless rope_base == 0),
    values are copied unchanged; slot -1 is skipped.  Returns new arrays.
    """
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bs = kc.shape[2]
    kr = rope(k, positions, rope_base) if rope_base else k
    if bf16:
        kr = round_bf16(kr)
    for n, s in enumerate(np.asarray(slot_mapping)):
        if s < 0:
            continue
        blk, off = int(s) // bs, int(s) % bs
        kc[blk, :, off, :] = kr[n]
        vc[blk, :, :, off] = v[n]
    return kc, vc


def gather_paged(cache, block_table_row, length, token_minor=False):
    """Read a sequence's logical K or V rows back out of a paged cache.

    §Paged Attention Kernels: logical position t lives in physical block
    table[t // bs] at offset t % bs; K[t + 1] need not sit next to K[t].
    Returns [length, Hkv, D].
    """
    cache = np.asarray(cache)
    bs = cache.shape[3] if token_minor else cache.shape[2]
    out = []
    for t in range(length):
        blk = int(block_table_row[t // bs])
        off = t % bs
        out.append(cache[blk, :, :, off] if token_minor else cache[blk, :, off, :])
    return np.stack(out) if out else np.zeros((0,) + (cache.shape[1], cache.shape[2] if token_minor else cache.shape[3]))


def decode(q, ks, vs, scale=None):
    """One decode query per sequence over its whole logical context.

    §FlashAttention-Style Kernels: decode has one new query per request and
    reads the growing KV cache.  q [S, Hq, D]; ks[s], vs[s] are the logical
    [ctx_s, Hkv, D] keys/values (the new token included).  No mask beyond the
    context length.  Returns (O [S, Hq, D], LSE [S, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    s_n, hq, d = q.shape
    out = np.zeros((s_n, hq, d))
    lse = np.zeros((s_n, hq))
    for s in range(s_n):
        o, l_ = attention(q[s][None, None], np.asarray(ks[s])[None], np.asarray(vs[s])[None],
                          causal=False, scale=scale)
        out[s] = o[0, 0]
        lse[s] = l_[0, :, 0]
    return out, lse


def chunked_prefill(qs, ks, vs, scale=None):
    """Prefill of new query chunks over cached plus new keys.

    qs[r] is [n_r, Hq, D]; ks[r], vs[r] are [c_r + n_r, Hkv, D] with the
    chunk's own keys last.  Bottom-right causal: chunk row i sees keys
    0 .. c_r + i.  Returns a list of O [n_r, Hq, D].
    """
    outs = []
    for q, k, v in zip(qs, ks, vs):
        o, _ = attention(np.asarray(q)[None], np.asarray(k)[None], np.asarray(v)[None],
                         causal=True, scale=scale)
        outs.append(o[0])
    return outs
