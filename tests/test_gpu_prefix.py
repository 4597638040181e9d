"""Prefix sharing with copy on write: the block copy (attn_copy_blocks) is
bit-exact, and a forked sequence that appends into a shared, partly filled
block decodes against its own context while the parent's cache stays
untouched (oracle on the logical sequences)."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_05_amd as mi
from tests.gpu_util import DEV, check, f64, say
from workloads import BLOCK_SIZE, normal, rng, scatter_to_pool, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_copy_blocks_bit_exact(dtype, d):
    say(f"case: copy blocks {dtype} D {d}")
    g = rng(61)
    nb, hkv = 300, 2
    kc = normal(g, (nb, hkv, BLOCK_SIZE, d), dtype).to(DEV)
    vc = normal(g, (nb, hkv, d, BLOCK_SIZE), dtype).to(DEV)
    perm = g.permutation(nb)
    pairs = np.stack([perm[:100], perm[100:200]], axis=1).astype(np.int32)
    junk = np.array([[-1, 5], [5, nb], [7, 7]], np.int32)          # skipped
    k0, v0 = kc.clone(), vc.clone()
    mi.attn_copy_blocks(kc, vc, torch.from_numpy(np.concatenate([pairs, junk])).to(DEV))
    torch.cuda.synchronize()
    k1, v1 = k0.clone(), v0.clone()
    k1[pairs[:, 1]] = k0[pairs[:, 0]]
    v1[pairs[:, 1]] = v0[pairs[:, 0]]
    iv = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(kc.view(iv), k1.view(iv)) and torch.equal(vc.view(iv), v1.view(iv))


def test_fork_append_decode():
    """A parent of 37 tokens (the last block holds 5), a child forked from
    all of it that appends 20 tokens (copy on write of the shared block), a
    second child forked at 32 tokens (no copy) that appends 9, and the
    parent appending 3 of its own: every sequence decodes against its
    logical context, and the blocks the parent never wrote stay
    bit-identical."""
    say("case: fork + copy on write + decode")
    g = rng(62)
    hq, hkv, d, nb = 12, 2, 128, 64
    pool = mi.Pool(nb)
    kc = torch.zeros(nb, hkv, BLOCK_SIZE, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(nb, hkv, d, BLOCK_SIZE, dtype=torch.bfloat16, device=DEV)
    rows = {n: np.full(8, -1, np.int32) for n in ("parent", "a", "b")}
    kv = {}
    # the parent's 37 cached tokens
    pk, pv = normal(g, (37, hkv, d), torch.bfloat16), normal(g, (37, hkv, d), torch.bfloat16)
    pool.seq_reserve(rows["parent"], 0, 37)
    scatter_to_pool(kc, vc, rows["parent"], pk, pv)
    torch.cuda.synchronize()
    parent_blocks = rows["parent"][:3].copy()
    snapshot = (kc[parent_blocks].clone(), vc[parent_blocks].clone())
    pool.seq_fork(rows["parent"], 37, rows["a"])
    pool.seq_fork(rows["parent"], 32, rows["b"])
    kv["parent"], kv["a"], kv["b"] = (pk, pv), (pk, pv), (pk[:32], pv[:32])
    lens = {"parent": 37, "a": 37, "b": 32}
    copies = 0
    for name, n_new in (("a", 20), ("b", 9), ("parent", 3)):
        slots, pair = pool.seq_reserve_cow(rows[name], lens[name], n_new)
        if pair is not None:
            copies += 1
            mi.attn_copy_blocks(kc, vc, torch.tensor([pair], dtype=torch.int32, device=DEV))
        nk, nv = normal(g, (n_new, hkv, d), torch.bfloat16), normal(g, (n_new, hkv, d), torch.bfloat16)
        pos = torch.arange(lens[name], lens[name] + n_new, dtype=torch.int32, device=DEV)
        mi.attn_kv_cache_write_rope(None, nk.to(DEV), nv.to(DEV), pos, torch.from_numpy(slots).to(DEV), kc, vc,
                                    rope_base=0.0)
        kv[name] = (torch.cat([kv[name][0], nk]), torch.cat([kv[name][1], nv]))
        lens[name] += n_new
    torch.cuda.synchronize()
    assert copies == 1                      # only "a" appended into a shared partial block
    # the parent's first two blocks are still shared and unwritten, its third
    # was copied for "a" before the parent appended in place
    assert torch.equal(kc[parent_blocks[:2]].view(torch.int16), snapshot[0][:2].view(torch.int16))
    assert torch.equal(vc[parent_blocks[:2]].view(torch.int16), snapshot[1][:2].view(torch.int16))
    names = ("parent", "a", "b")
    q = normal(g, (3, hq, d), torch.bfloat16)
    bt = torch.from_numpy(np.stack([rows[n] for n in names])).to(DEV)
    cl = torch.tensor([lens[n] for n in names], dtype=torch.int32, device=DEV)
    o = mi.attn_decode_paged(q.to(DEV), kc, vc, bt, cl, max(lens.values()), partition_size=128)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(to_f64(q), [to_f64(kv[n][0]) for n in names], [to_f64(kv[n][1]) for n in names])
    check(f64(o.cpu()), ref, torch.bfloat16, "forked decode")
