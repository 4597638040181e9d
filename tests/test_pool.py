"""Host block pool and block-table growth, checked bit-exactly against a
brute-force set model (§Paged Attention Kernels of "Fast Attention Kernels
and Operator Fusion": blocks allocated on demand, returned when a request
ends, shared by sequences with a common prefix)."""

import numpy as np
import pytest

from transformer_attention_05_amd import ATTN_E_INVALID, ATTN_E_NOMEM, ATTN_E_STATE, AttnError, Pool
from workloads import rng


def test_fresh_pool_hands_out_ascending_ids():
    p = Pool(10)
    assert p.num_free == 10 and p.num_blocks == 10
    np.testing.assert_array_equal(p.alloc(4), [0, 1, 2, 3])
    assert [p.refcount(i) for i in range(5)] == [1, 1, 1, 1, 0]


def test_lifo_reuse_order():
    p = Pool(8)
    p.alloc(8)
    p.free([5, 2, 7])
    np.testing.assert_array_equal(p.alloc(3), [7, 2, 5])


def test_alloc_all_or_nothing():
    p = Pool(6)
    p.alloc(4)
    with pytest.raises(AttnError) as e:
        p.alloc(3)
    assert e.value.status == ATTN_E_NOMEM
    assert p.num_free == 2
    np.testing.assert_array_equal(p.alloc(2), [4, 5])


def test_free_validates_everything_first():
    p = Pool(6)
    ids = p.alloc(3)
    with pytest.raises(AttnError) as e:
        p.free([0, 1, 99])
    assert e.value.status == ATTN_E_INVALID
    assert p.num_free == 3 and all(p.refcount(int(i)) == 1 for i in ids)
    with pytest.raises(AttnError) as e:
        p.free([0, 0])  # refcount 1, released twice
    assert e.value.status == ATTN_E_STATE
    assert p.refcount(0) == 1
    p.free([0])
    with pytest.raises(AttnError) as e:
        p.free([0])     # double free
    assert e.value.status == ATTN_E_STATE


def test_retain_and_shared_release():
    p = Pool(4)
    a = p.alloc(2)
    p.retain(a)          # a second sequence shares the prefix
    assert p.refcount(int(a[0])) == 2
    p.free(a)
    assert p.num_free == 2 and p.refcount(int(a[0])) == 1
    p.free(a)
    assert p.num_free == 4
    with pytest.raises(AttnError) as e:
        p.retain([3])    # free block
    assert e.value.status == ATTN_E_STATE


def test_seq_reserve_slots_and_growth():
    p = Pool(20)
    row = np.full(8, -1, dtype=np.int32)
    s1 = p.seq_reserve(row, 0, 20)       # needs 2 blocks
    np.testing.assert_array_equal(row[:2], [0, 1])
    assert row[2] == -1
    np.testing.assert_array_equal(s1, [row[t // 16] * 16 + t % 16 for t in range(20)])
    s2 = p.seq_reserve(row, 20, 13)      # 33 tokens -> 3 blocks
    np.testing.assert_array_equal(row[:3], [0, 1, 2])
    np.testing.assert_array_equal(s2, [row[t // 16] * 16 + t % 16 for t in range(20, 33)])
    s3 = p.seq_reserve(row, 33, 15)      # 48 tokens still 3 blocks
    assert p.num_free == 17 and len(s3) == 15
    with pytest.raises(AttnError) as e:
        p.seq_reserve(row, 48, 100)      # would need 10 blocks, row holds 8
    assert e.value.status == ATTN_E_INVALID
    assert p.num_free == 17


def test_seq_reserve_out_of_memory_leaves_pool_unchanged():
    p = Pool(3)
    row = np.full(10, -1, dtype=np.int32)
    p.seq_reserve(row, 0, 16)
    with pytest.raises(AttnError) as e:
        p.seq_reserve(row, 16, 64)       # 4 more blocks, 2 free
    assert e.value.status == ATTN_E_NOMEM
    assert p.num_free == 2 and row[1] == -1


def test_seq_reserve_rejects_unallocated_row_entries():
    p = Pool(4)
    row = np.array([3, -1], dtype=np.int32)   # block 3 was never allocated
    with pytest.raises(AttnError) as e:
        p.seq_reserve(row, 10, 10)
    assert e.value.status == ATTN_E_STATE


@pytest.mark.parametrize("seed", range(3))
def test_random_ops_against_set_model(seed):
    g = rng(seed)
    nb = 64
    p = Pool(nb)
    ref = {}            # id -> refcount
    stack = list(range(nb - 1, -1, -1))
    for _ in range(400):
        op = g.integers(0, 3)
        if op == 0:
            n = int(g.integers(0, 10))
            if n > len(stack):
                with pytest.raises(AttnError):
                    p.alloc(n)
            else:
                got = p.alloc(n)
                exp = [stack.pop() for _ in range(n)]
                np.testing.assert_array_equal(got, exp)
                for i in exp:
                    ref[i] = 1
        elif op == 1 and ref:
            ids = g.choice(sorted(ref), size=min(len(ref), int(g.integers(1, 4))), replace=False)
            p.free(ids)
            for i in ids:
                ref[int(i)] -= 1
                if ref[int(i)] == 0:
                    del ref[int(i)]
                    stack.append(int(i))
        elif op == 2 and ref:
            ids = g.choice(sorted(ref), size=1)
            p.retain(ids)
            ref[int(ids[0])] += 1
        assert p.num_free == len(stack) == nb - len(ref)
        for i in range(nb):
            assert p.refcount(i) == ref.get(i, 0)


def test_fragmentation_readings():
    """Two readings of 'allocate and free 50% of blocks at random': (a) every
    block allocated, a random half freed (holes between foreign tenants);
    (b) half allocated then all freed (only the free-list order scrambled).
    Either way the pool stays consistent and hands out distinct ids."""
    g = rng(5)
    nb = 100
    p = Pool(nb)
    p.alloc(nb)
    half = g.permutation(nb)[: nb // 2]
    p.free(half)
    got = p.alloc(nb // 2)
    assert sorted(got.tolist()) == sorted(half.tolist())
    q = Pool(nb)
    first = q.alloc(nb // 2)
    q.free(g.permutation(first))
    got2 = q.alloc(nb)
    assert sorted(got2.tolist()) == list(range(nb))


# ------------------------------------------------------------------ prefix sharing, copy on write

def test_fork_shares_blocks():
    p = Pool(20, 16)
    parent = np.full(8, -1, np.int32)
    p.seq_reserve(parent, 0, 37)                 # 3 blocks, the last holds 5 tokens
    child = np.full(8, -1, np.int32)
    p.seq_fork(parent, 37, child)
    np.testing.assert_array_equal(child[:3], parent[:3])
    assert np.all(child[3:] == -1)
    assert [p.refcount(int(b)) for b in parent[:3]] == [2, 2, 2]
    p.seq_fork(parent, 0, child)                 # nothing to share
    assert [p.refcount(int(b)) for b in parent[:3]] == [2, 2, 2]


def test_fork_validates_first():
    p = Pool(10, 16)
    parent = np.array([0, 1, 7, -1], np.int32)   # block 7 was never allocated
    p.alloc(2)
    child = np.full(4, -1, np.int32)
    with pytest.raises(AttnError) as e:
        p.seq_fork(parent, 40, child)
    assert e.value.status == ATTN_E_STATE
    assert [p.refcount(i) for i in (0, 1, 7)] == [1, 1, 0] and np.all(child == -1)
    with pytest.raises(AttnError) as e:
        p.seq_fork(parent, 40, np.full(2, -1, np.int32))   # the child row is too short
    assert e.value.status == ATTN_E_INVALID


def test_reserve_cow_copies_a_shared_partial_block():
    p = Pool(20, 16)
    parent = np.full(8, -1, np.int32)
    p.seq_reserve(parent, 0, 37)
    child = np.full(8, -1, np.int32)
    p.seq_fork(parent, 37, child)
    shared = int(parent[2])
    slots, pair = p.seq_reserve_cow(child, 37, 20)   # tokens 37..56: block 2 (11 more), block 3
    assert pair == (shared, int(child[2])) and child[2] != shared
    assert p.refcount(shared) == 1 and p.refcount(int(child[2])) == 1 and p.refcount(int(child[3])) == 1
    np.testing.assert_array_equal(child[:2], parent[:2])       # full blocks stay shared
    assert p.refcount(int(parent[0])) == 2
    t = np.arange(37, 57)
    np.testing.assert_array_equal(slots, child[t // 16] * 16 + t % 16)
    assert not set(slots // 16) & set(parent[:3].tolist())     # no new token lands in a parent block
    # the parent, now the only holder of its last block, appends without a copy
    _, pair = p.seq_reserve_cow(parent, 37, 3)
    assert pair is None


def test_reserve_cow_no_copy_cases():
    p = Pool(20, 16)
    parent = np.full(8, -1, np.int32)
    p.seq_reserve(parent, 0, 32)                 # two full blocks
    child = np.full(8, -1, np.int32)
    p.seq_fork(parent, 32, child)
    _, pair = p.seq_reserve_cow(child, 32, 5)    # the next token starts a new block
    assert pair is None and child[2] not in parent[:2]
    other = np.full(8, -1, np.int32)
    p.seq_fork(parent, 30, other)                # shares two blocks, the second partly filled
    _, pair = p.seq_reserve_cow(other, 30, 0)    # nothing appended: nothing copied
    assert pair is None and other[1] == parent[1]


def test_reserve_cow_out_of_memory_changes_nothing():
    p = Pool(5, 16)
    parent = np.full(4, -1, np.int32)
    p.seq_reserve(parent, 0, 37)                 # 3 of 5 blocks
    child = np.full(4, -1, np.int32)
    p.seq_fork(parent, 37, child)
    p.alloc(1)                                   # one block left: the copy fits, the growth does not
    before = ([p.refcount(i) for i in range(5)], p.num_free, child.copy())
    with pytest.raises(AttnError) as e:
        p.seq_reserve_cow(child, 37, 20)
    assert e.value.status == ATTN_E_NOMEM
    assert ([p.refcount(i) for i in range(5)], p.num_free) == before[:2]
    np.testing.assert_array_equal(child, before[2])


@pytest.mark.parametrize("seed", [11, 12])
def test_cow_random_against_model(seed):
    """Random forks, appends and releases: the pool's refcounts and free count
    follow a brute-force model, and after every append the block receiving the
    sequence's next token is held by that sequence alone."""
    g = rng(seed)
    NB, BS, MAXB = 64, 16, 12
    p = Pool(NB, BS)
    ref = np.zeros(NB, np.int64)
    seqs = []                                    # [row, length]
    for _ in range(300):
        op = g.integers(0, 4)
        if op == 0 or not seqs:                  # new sequence
            row = np.full(MAXB, -1, np.int32)
            n = int(g.integers(1, 60))
            try:
                p.seq_reserve(row, 0, n)
            except AttnError:
                continue
            ref[row[: -(-n // BS)]] += 1
            seqs.append([row, n])
        elif op == 1:                            # fork a prefix of a sequence
            row, n = seqs[g.integers(len(seqs))]
            k = int(g.integers(0, n + 1))
            child = np.full(MAXB, -1, np.int32)
            p.seq_fork(row, k, child)
            ref[child[: -(-k // BS)]] += 1
            seqs.append([child, k])
        elif op == 2:                            # append
            s = seqs[g.integers(len(seqs))]
            row, n = s
            k = int(g.integers(1, 30))
            if -(-(n + k) // BS) > MAXB:
                continue
            old = row.copy()
            try:
                slots, pair = p.seq_reserve_cow(row, n, k)
            except AttnError as e:
                assert e.status == ATTN_E_NOMEM
                np.testing.assert_array_equal(row, old)
                continue
            if pair is not None:
                assert n % BS and pair[0] == old[n // BS] and row[n // BS] == pair[1]
                ref[pair[0]] -= 1
                ref[pair[1]] += 1
            have, need = -(-n // BS), -(-(n + k) // BS)
            ref[row[have:need]] += 1
            assert p.refcount(int(row[n // BS])) == 1    # the next token's block is private
            s[1] = n + k
        else:                                    # release a sequence
            row, n = seqs.pop(g.integers(len(seqs)))
            ids = row[: -(-n // BS)]
            p.free(ids)
            ref[ids] -= 1
        assert [p.refcount(i) for i in range(NB)] == ref.tolist()
        assert p.num_free == int((ref == 0).sum())
