"""The host block manager (pkv_bm_*, pkv_xxh64, pkv_block_hash) on the CPU:
the hash against published XXH64 vectors and the xxhash package, the chained
block hash against its definition in "nano-vLLM-1" ("2. BlockManager 初始化与
链式哈希"), the allocation / append / release rules of that page's sections 3-6
on its worked examples and invariants, and the manager feeding the packers."""
import json
import os

import numpy as np
import pytest

import oracle
import paged_kv_cache_125_amd as pkv

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- hashing

def test_xxh64_published_vectors():
    g = json.load(open(os.path.join(HERE, "golden", "xxh64_vectors.json")))
    for v in g["vectors"]:
        assert pkv.xxh64(v["input"].encode(), v["seed"]) == int(v["xxh64"], 16), v


def test_xxh64_matches_the_xxhash_package():
    xxhash = pytest.importorskip("xxhash")
    rng = np.random.default_rng(1)
    for n in list(range(0, 70)) + [127, 128, 129, 1000, 4099]:
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        for seed in (0, 1, 0x9E3779B97F4A7C15):
            assert pkv.xxh64(data, seed) == xxhash.xxh64(data, seed=seed).intdigest(), (n, seed)


def test_block_hash_is_the_chained_definition():
    # xxh64 of [previous hash as 8 little-endian bytes] + token ids as int64
    xxhash = pytest.importorskip("xxhash")
    toks = [7, 0, 151643, 2 ** 40 + 3, 5]
    first = xxhash.xxh64(np.array(toks, dtype=np.int64).tobytes()).intdigest()
    assert pkv.block_hash(toks) == first
    second = xxhash.xxh64(first.to_bytes(8, "little") + np.array(toks[::-1], dtype=np.int64).tobytes()).intdigest()
    assert pkv.block_hash(toks[::-1], prefix=first) == second
    assert pkv.block_hash(toks[::-1]) != second          # the chain matters


# ---------------------------------------------------------------- allocation

def _toks(*blocks, bs=4):
    out = []
    for b in blocks:
        out += [b * 100 + i for i in range(bs)] if isinstance(b, int) else list(b)
    return out


def test_shared_prefix_blocks_are_reused_until_the_first_difference():
    # the page's example: [A, B, C] and [A, B, D] share A and B, not C / D
    A, B, C, D = 1, 2, 3, 4
    m = pkv.BlockManager(16, 4)
    assert m.allocate(10, _toks(A, B, C)) == 0
    assert m.allocate(11, _toks(A, B, D)) == 8
    t10, t11 = m.block_table(10), m.block_table(11)
    assert t10[:2] == t11[:2] and t10[2] != t11[2]
    assert m.num_free == 16 - 4
    # a different first block breaks the chain even where later tokens agree
    assert m.allocate(12, _toks(D, B, C)) == 0
    assert not set(m.block_table(12)) & set(t10)
    # releasing one sharer keeps the shared blocks in use
    m.deallocate(10)
    assert m.num_free == 16 - 7 + 1
    m.deallocate(11)
    assert m.num_free == 16 - 3


def test_only_full_blocks_are_shared():
    m = pkv.BlockManager(8, 4)
    seq = _toks(1, [5, 6, 7])              # 7 tokens: one full block + 3
    assert m.allocate(1, seq) == 0
    assert m.allocate(2, seq) == 4          # the partial block is never a hit
    assert m.block_table(1)[0] == m.block_table(2)[0]
    assert m.block_table(1)[1] != m.block_table(2)[1]


def test_decode_state_machine_on_the_seven_token_example():
    # bs 4, 7 tokens hold logical blocks 0 and 1; the 8th token fills block 1
    # (it is registered then), the 9th opens a new block
    m = pkv.BlockManager(8, 4)
    seq = list(range(1, 8))
    m.allocate(1, seq)
    assert len(m.block_table(1)) == 2 and m.num_free == 6
    m.append_token(1, 8)
    assert m.can_append(1)
    m.may_append(1)                         # len 8: block 1 full -> registered
    assert len(m.block_table(1)) == 2 and m.num_free == 6
    assert m.allocate(2, list(range(1, 9))) == 8      # both blocks now hit
    m.append_token(1, 9)
    m.may_append(1)                         # len 9: a new block
    assert len(m.block_table(1)) == 3 and m.num_free == 5
    m.append_token(1, 10)
    m.may_append(1)                         # len 10: nothing changes
    m.may_append(1)                         # (and again: still nothing)
    assert len(m.block_table(1)) == 3
    m.append_token(1, 11)
    m.append_token(1, 12)
    m.may_append(1)                         # len 12: block 2 full -> registered
    with pytest.raises(pkv.PkvError):
        m.may_append(1)                     # the same fill twice is inconsistent
    m.deallocate(2)
    m.deallocate(1)
    assert m.num_free == 8


def test_fifo_order_and_release_order():
    m = pkv.BlockManager(6, 2)
    m.allocate(1, [1, 2, 3, 4, 5])          # blocks 0, 1, 2 from the front
    assert m.block_table(1) == [0, 1, 2]
    m.allocate(2, [9, 9])                   # block 3
    assert m.block_table(2) == [3]
    m.deallocate(1)                         # back of the FIFO, last block first: 2, 1, 0
    m.allocate(3, [7, 7, 8, 8, 6, 6, 5])    # takes 4, 5, then 2, 1
    assert m.block_table(3) == [4, 5, 2, 1]


def test_released_blocks_stay_hits_until_reused():
    m = pkv.BlockManager(4, 2)
    m.allocate(1, [1, 2, 3, 4])
    t = m.block_table(1)
    m.deallocate(1)                         # preempted: blocks free but registered
    assert m.allocate(2, [1, 2, 3, 4, 5]) == 4
    assert m.block_table(2)[:2] == t
    assert m.num_free == 1


def test_a_revived_block_stays_registered():
    # blocks released by one sequence and taken back by a later prompt with
    # the same prefix keep their registration: a third prompt with that prefix
    # still finds them while the second holds them
    m = pkv.BlockManager(6, 2)
    m.allocate(1, [1, 2, 3, 4])
    t = m.block_table(1)
    m.deallocate(1)
    assert m.allocate(2, [1, 2, 3, 4, 5]) == 4
    assert m.allocate(3, [1, 2, 3, 4, 9]) == 4
    assert m.block_table(3)[:2] == t == m.block_table(2)[:2]


def test_a_stale_entry_with_the_same_tokens_is_a_miss():
    # block X holds tokens T after prefix P1, is freed, and is reused for T
    # after prefix P2; P1 + T must then miss although X's tokens equal T
    m = pkv.BlockManager(4, 2)
    m.allocate(1, [1, 1, 5, 5])             # blocks 0 (P1), 1 (T after P1)
    m.allocate(9, [8, 8])                   # block 2
    m.deallocate(1)                         # FIFO: 3, 1, 0
    m.allocate(2, [2, 2, 5, 5])             # takes 3 (P2) and 1 (T after P2)
    assert m.block_table(2) == [3, 1]
    m.deallocate(9)                         # FIFO: 0, 2
    cached = m.allocate(3, [1, 1, 5, 5])    # P1 hits block 0; T after P1 must miss
    assert cached == 2 and m.block_table(3) == [0, 2]


def test_capacity_checks_and_failures_leave_the_state_unchanged():
    m = pkv.BlockManager(3, 4)
    assert m.can_allocate(12) and not m.can_allocate(13)
    m.allocate(1, list(range(9)))           # 3 blocks
    assert m.num_free == 0
    with pytest.raises(pkv.PkvError):
        m.allocate(2, [1])
    assert m.num_free == 0
    with pytest.raises(pkv.PkvError):
        m.allocate(1, [1])                  # already holds blocks
    for t in (9, 10, 11):
        m.append_token(1, t)
        assert m.can_append(1)
        m.may_append(1)                     # lengths 10..12 stay in block 2
    m.append_token(1, 12)                   # length 13 opens a block: none free
    assert not m.can_append(1)
    with pytest.raises(pkv.PkvError):
        m.may_append(1)
    m.deallocate(1)
    assert m.num_free == 3


def test_block_size_one():
    m = pkv.BlockManager(8, 1)
    assert m.allocate(1, [4, 5]) == 0
    m.append_token(1, 6)
    assert m.can_append(1)
    m.may_append(1)
    assert len(m.block_table(1)) == 3
    assert m.allocate(2, [4, 5, 6, 7]) == 3


# ---------------------------------------------------------------- packing

def test_manager_feeds_the_packers():
    bs = 16
    m = pkv.BlockManager(64, bs)
    rng = np.random.default_rng(3)
    prefix = [int(x) for x in rng.integers(0, 50000, 48)]
    prompts = {1: prefix + [1, 2, 3], 2: prefix[:40] + [9] * 30, 3: prefix + list(range(70)),
               4: [int(x) for x in rng.integers(0, 50000, 5)]}
    cached = {s: m.allocate(s, p) for s, p in prompts.items()}
    assert cached == {1: 0, 2: 32, 3: 48, 4: 0}
    ids = [1, 2, 3, 4]
    lens, nc, tables = m.gather(ids)
    assert lens == [len(prompts[s]) for s in ids] and nc == [cached[s] for s in ids]
    meta = pkv.pack_prefill(lens, nc, tables, bs, device="cpu")
    ranges = [(i, c, n) for i, (n, c) in enumerate(zip(lens, nc))]
    assert np.array_equal(meta["slot_mapping"].numpy(), oracle.slots(ranges, tables, bs))
    assert meta["block_tables"] is not None           # the batch reads a cached prefix
    # decode: every sequence grows by one token
    for s in ids:
        m.append_token(s, 7)
        m.may_append(s)
    lens, _, tables = m.gather(ids)
    dm = pkv.pack_decode(lens, tables, bs, device="cpu")
    want = oracle.slots([(i, n - 1, n) for i, n in enumerate(lens)], tables, bs)
    assert np.array_equal(dm["slot_mapping"].numpy(), want)
