"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module draws random numbers and lays data out; it holds none of the
attention arithmetic.  Values are float32 draws from N(0, 1) made with
NumPy's PCG64 generator, then rounded to bfloat16 (round-to-nearest-even, via
torch) when the workload is bf16.  Draw order inside one case: lengths, then
block permutations, then Q, K, V.

Workload shapes follow the tutorial "Fast Attention Kernels and Operator
Fusion": its serving example (§Paged Attention Kernels) uses a
Qwen2.5-1.5B-Instruct decoder with 16-token KV blocks, whose attention has
12 query heads, 2 key/value heads and head dimension 128; its SDPA example
(§FlashAttention-Style Kernels) uses (B, H, T, D) = (2, 16, 512, 64).
No model weights or prompts are involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(g: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    a = g.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(a).to(dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a host tensor (bf16 or fp32) to a float64 array."""
    return t.detach().to("cpu", torch.float64).numpy()


# --------------------------------------------------------------------------
# contiguous prefill
# --------------------------------------------------------------------------

def prefill_case(seed, batch, seqlen, hq, hkv, d, dtype, seqlen_k=None):
    """q [B, Tq, Hq, D], k and v [B, Tk, Hkv, D] on the host."""
    g = rng(seed)
    tk = seqlen if seqlen_k is None else seqlen_k
    q = normal(g, (batch, seqlen, hq, d), dtype)
    k = normal(g, (batch, tk, hkv, d), dtype)
    v = normal(g, (batch, tk, hkv, d), dtype)
    return q, k, v


def additive_mask(seed, shape, amp=3.0, p_masked=0.25, masked_rows=()):
    """fp32 additive mask: amp * N(0,1) with a fraction p_masked of the entries
    set to -inf, and the rows listed in masked_rows (indices on the second to
    last axis) wholly -inf."""
    g = rng(seed)
    m = (amp * g.standard_normal(shape)).astype(np.float32)
    m[g.random(shape) < p_masked] = -np.inf
    for r in masked_rows:
        m[..., r, :] = -np.inf
    return torch.from_numpy(m)


# --------------------------------------------------------------------------
# paged decode
# --------------------------------------------------------------------------

def lengths_uniform(g, n, lo, hi):
    """Integers uniform on [lo, hi] inclusive."""
    return g.integers(lo, hi + 1, size=n).astype(np.int64)


def lengths_loguniform(g, n, lo, hi):
    """round(exp(U(ln lo, ln hi))), clipped to [lo, hi]."""
    x = np.exp(g.uniform(np.log(lo), np.log(hi), size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


@dataclass
class DecodeCase:
    lengths: np.ndarray          # [S] context lengths (new token included)
    q: torch.Tensor              # [S, Hq, D]
    k: list                      # per sequence [ctx, Hkv, D]
    v: list
    block_tables: np.ndarray     # [S, max_blocks] int32, -1 past the end
    num_blocks: int              # physical blocks in the pool
    hq: int = 12
    hkv: int = 2
    d: int = 128


def decode_case(seed, num_seqs, lo, hi, hq=12, hkv=2, d=128, dtype=torch.bfloat16,
                dist="uniform", slack_blocks=16, lengths=None, block_order="random"):
    """Decode inputs whose block tables take consecutive ids of a seeded
    permutation of the pool (so logical neighbours are physically scattered).

    block_order: "random" (permutation), "identity" (0, 1, 2, ...),
    "reversed" (descending ids).
    """
    g = rng(seed)
    if lengths is None:
        lengths = (lengths_uniform if dist == "uniform" else lengths_loguniform)(g, num_seqs, lo, hi)
    lengths = np.asarray(lengths, dtype=np.int64)
    nblk = (lengths + BLOCK_SIZE - 1) // BLOCK_SIZE
    num_blocks = int(nblk.sum()) + slack_blocks
    perm = g.permutation(num_blocks)  # always drawn, so values do not depend on block_order
    if block_order == "random":
        pass
    elif block_order == "identity":
        perm = np.arange(num_blocks)
    elif block_order == "reversed":
        perm = np.arange(num_blocks)[::-1].copy()
    else:
        raise ValueError(block_order)
    maxb = int(max(1, nblk.max()))
    bt = np.full((len(lengths), maxb), -1, dtype=np.int32)
    pos = 0
    for s, nb in enumerate(nblk):
        bt[s, :nb] = perm[pos:pos + nb]
        pos += nb
    q = normal(g, (len(lengths), hq, d), dtype)
    ks, vs = [], []
    for L in lengths:
        ks.append(normal(g, (int(L), hkv, d), dtype))
        vs.append(normal(g, (int(L), hkv, d), dtype))
    return DecodeCase(lengths, q, ks, vs, bt, num_blocks, hq, hkv, d)


def scatter_to_pool(k_cache, v_cache, block_table_row, k, v, start=0):
    """Place logical rows [start, start+len) of one sequence into the paged
    caches (k_cache [NB, Hkv, bs, D], v_cache [NB, Hkv, D, bs]) with torch
    indexing.  Harness plumbing: it stands in for earlier steps that wrote
    the cache."""
    n = k.shape[0]
    if n == 0:
        return
    dev = k_cache.device
    t = torch.arange(start, start + n, device=dev)
    bt = torch.as_tensor(np.asarray(block_table_row, dtype=np.int64), device=dev)
    blk = bt[t // BLOCK_SIZE]
    off = t % BLOCK_SIZE
    kk = k.to(dev, k_cache.dtype)
    vv = v.to(dev, v_cache.dtype)
    k_cache[blk, :, off, :] = kk
    # v_cache[blk, :, :, off] with advanced indices on dims 0 and 3 yields
    # [n, Hkv, D] in that order.
    v_cache[blk, :, :, off] = vv


def build_decode_pool(case: DecodeCase, device, dtype=torch.bfloat16, fill=0.0):
    """Allocate caches for a DecodeCase and scatter every sequence into them."""
    kc = torch.full((case.num_blocks, case.hkv, BLOCK_SIZE, case.d), fill, dtype=dtype, device=device)
    vc = torch.full((case.num_blocks, case.hkv, case.d, BLOCK_SIZE), fill, dtype=dtype, device=device)
    for s in range(len(case.lengths)):
        scatter_to_pool(kc, vc, case.block_tables[s], case.k[s], case.v[s])
    return kc, vc


# --------------------------------------------------------------------------
# the mixed step: chunked prefill + decode over one fragmented pool
# --------------------------------------------------------------------------

@dataclass
class MixedCase:
    cached: np.ndarray           # [R] cached tokens of each chunked-prefill request
    chunk: int                   # new tokens per request
    dec_lengths: np.ndarray      # [S] decode context lengths (new token included)
    free_order: np.ndarray       # permutation used to fragment the pool
    num_blocks: int
    q_new: torch.Tensor          # [N, Hq, D] raw (un-rotated) queries, N = R*chunk + S
    k_new: torch.Tensor          # [N, Hkv, D] raw keys
    v_new: torch.Tensor          # [N, Hkv, D]
    positions: np.ndarray        # [N] absolute positions of the new tokens
    k_old: list                  # per sequence (requests, then decode) cached keys (already rotated)
    v_old: list
    hq: int = 12
    hkv: int = 2
    d: int = 128
    rope_base: float = 10000.0
    tables: np.ndarray | None = None       # filled by assign_blocks
    slots: np.ndarray | None = None        # [N] slot of each new token
    foreign: np.ndarray | None = None      # blocks held by other tenants
    extra: dict = field(default_factory=dict)


def mixed_case(seed, num_req=8, chunk=512, cached_max=2048, num_dec=128, dec_lo=16, dec_hi=32768,
               hq=12, hkv=2, d=128, dtype=torch.bfloat16, rope_base=10000.0):
    g = rng(seed)
    cached = g.integers(0, cached_max + 1, size=num_req).astype(np.int64)
    dec = lengths_loguniform(g, num_dec, dec_lo, dec_hi)
    need = int(((cached + chunk + BLOCK_SIZE - 1) // BLOCK_SIZE).sum() + ((dec + BLOCK_SIZE - 1) // BLOCK_SIZE).sum())
    num_blocks = 2 * need + 64
    free_order = g.permutation(num_blocks)
    n_new = num_req * chunk + num_dec
    q_new = normal(g, (n_new, hq, d), dtype)
    k_new = normal(g, (n_new, hkv, d), dtype)
    v_new = normal(g, (n_new, hkv, d), dtype)
    pos = np.concatenate([np.arange(c, c + chunk) for c in cached] + [dec - 1]).astype(np.int64)
    k_old, v_old = [], []
    for c in list(cached) + list(dec - 1):
        k_old.append(normal(g, (int(c), hkv, d), dtype))
        v_old.append(normal(g, (int(c), hkv, d), dtype))
    return MixedCase(cached, chunk, dec, free_order, num_blocks, q_new, k_new, v_new, pos,
                     k_old, v_old, hq, hkv, d, rope_base)


def assign_blocks(case: MixedCase, pool):
    """Fragment the pool and reserve every sequence's blocks through ``pool``.

    Reading of "pre-fragmented by allocating and freeing 50% of blocks at
    random": allocate every block, then free a seeded half of them in seeded
    order; the other half stays held by foreign tenants and the workload's
    sequences take blocks from the holes.  ``pool`` is the library's host
    allocator wrapper (alloc / free / seq_reserve).
    """
    nb = case.num_blocks
    all_ids = pool.alloc(nb)
    assert len(all_ids) == nb
    half = case.free_order[: nb // 2]
    pool.free(np.asarray(half, dtype=np.int32))
    case.foreign = np.setdiff1d(np.arange(nb), half)
    lens_total = np.concatenate([case.cached + case.chunk, case.dec_lengths])
    maxb = int(((lens_total + BLOCK_SIZE - 1) // BLOCK_SIZE).max())
    S = len(lens_total)
    tables = np.full((S, maxb), -1, dtype=np.int32)
    slots = []
    old_lens = np.concatenate([case.cached, case.dec_lengths - 1])
    new_lens = np.concatenate([np.full(len(case.cached), case.chunk), np.ones(len(case.dec_lengths), np.int64)])
    for s in range(S):
        row = tables[s]
        if old_lens[s] > 0:
            pool.seq_reserve(row, 0, int(old_lens[s]))
        slots.append(pool.seq_reserve(row, int(old_lens[s]), int(new_lens[s])))
    case.tables = tables
    case.slots = np.concatenate(slots).astype(np.int32)
    return case
