"""Host-side checks of the seeded workload generator and its block allocator."""
import json
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_seeded_and_reproducible():
    a = W.tiny_fp32()
    b = W.tiny_fp32()
    for name in ("q", "prefix_k", "prefix_v", "prefix_slots", "new_k", "new_v", "new_slots",
                 "block_tables", "context_lens"):
        assert getattr(a, name).tobytes() == getattr(b, name).tobytes(), name


def test_tiny_config_shape():
    c = W.tiny_fp32()
    assert list(c.context_lens) == [1, 17, 100, 250]
    assert (c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, c.num_blocks) == (8, 8, 64, 16, 64)
    assert c.dtype == np.float32 and c.scale == 1.0 / 8.0


def _check_tables(case):
    B = case.block_size
    used = []
    for s in range(case.num_seqs):
        ctx = int(case.context_lens[s])
        nb = -(-ctx // B)
        row = case.block_tables[s]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < case.num_blocks)
        assert np.all(row[nb:] == -1)
        # internal fragmentation: at most B-1 unused slots in the last block
        assert 0 <= nb * B - ctx <= B - 1
        used.extend(row[:nb].tolist())
    return used


def test_p13_blocks_and_fragmentation_bound():
    g = json.load(open(os.path.join(GOLDEN, "kv_bytes.json")))["fragmentation_bound"]
    case = W.make_case(seed=3, context_lens=[1, 15, 16, 17, 31, 32, 33, 250], num_q_heads=4,
                       num_kv_heads=2, head_dim=8, block_size=g["block_size"])
    used = _check_tables(case)
    assert len(used) == len(set(used))  # private blocks are distinct
    waste = [-(-int(c) // 16) * 16 - int(c) for c in case.context_lens]
    assert max(waste) == g["expected_max_waste_tokens"]


def test_p13_shared_prefix_refcounts_and_private_appends():
    case = W.shared_prefix(num_prompts=3, samples=4, prompt_len=64, max_tail=40)
    _check_tables(case)
    pb = 64 // 16
    for p in range(3):
        rows = case.block_tables[p * 4:(p + 1) * 4, :pb]
        assert np.all(rows == rows[0])  # samples point at the same prompt blocks
        assert np.all(case.refcount[rows[0]] == 4)
    # this step's appends never land in a shared block
    for s in range(case.num_seqs):
        blk = int(case.new_slots[s]) // case.block_size
        assert case.refcount[blk] == 1
    # every stored slot is written exactly once
    all_slots = np.concatenate([case.prefix_slots, case.new_slots])
    assert len(all_slots) == len(set(all_slots.tolist()))


def test_full_config_shared_prefix_is_block_aligned():
    case = W.shared_prefix()
    assert case.num_seqs == 128
    assert np.all(case.context_lens >= 2001) and np.all(case.context_lens <= 2257)
    assert all(case.refcount[case.new_slots // 16] == 1)
    assert case.unique_kv_bytes() < case.kv_bytes() / 4


def test_pool_exhaustion_raises():
    alloc = W.BlockAllocator(3, np.random.default_rng(0))
    got = [alloc.allocate() for _ in range(3)]
    assert sorted(got) == [0, 1, 2]
    with pytest.raises(W.PoolExhausted):
        alloc.allocate()
    alloc.release(got[0])
    assert alloc.allocate() == got[0]


def test_share_and_release_refcounts():
    alloc = W.BlockAllocator(4, np.random.default_rng(1))
    b = alloc.allocate()
    alloc.share(b)
    assert alloc.refcount[b] == 2
    alloc.release(b)
    assert alloc.num_free == 3
    alloc.release(b)
    assert alloc.num_free == 4
    with pytest.raises(ValueError):
        alloc.release(b)


def test_placement_is_scattered():
    case = W.make_case(seed=9, context_lens=[400], num_q_heads=2, num_kv_heads=2, head_dim=8,
                       block_size=16)
    row = case.block_tables[0, :25]
    assert not np.all(np.diff(row) == 1)


def test_variants_change_only_what_they_say():
    plain = W.make_case(seed=5, context_lens=[30, 40], num_q_heads=4, num_kv_heads=2,
                        head_dim=16, block_size=8)
    needle = W.make_case(seed=5, context_lens=[30, 40], num_q_heads=4, num_kv_heads=2,
                         head_dim=16, block_size=8, variant="needle")
    pos = W.make_case(seed=5, context_lens=[30, 40], num_q_heads=4, num_kv_heads=2,
                      head_dim=16, block_size=8, variant="poscode")
    assert np.array_equal(plain.q, needle.q) and np.array_equal(plain.prefix_v, needle.prefix_v)
    assert np.array_equal(plain.prefix_k, pos.prefix_k)
    for s in range(2):
        k, _ = W.logical_kv(needle, s)
        kp, _ = W.logical_kv(plain, s)
        assert (k != kp).any(axis=(1, 2)).sum() == 1  # exactly one planted position
        _, v = W.logical_kv(pos, s)
        np.testing.assert_allclose(v[:, 0, 0].astype(np.float64),
                                   np.arange(len(v)) / 40.0, atol=1e-3)


def test_long_context_logical_data_independent_of_block_size():
    a = W.long_context(block_size=8, num_seqs=2, lo=64, hi=200)
    b = W.long_context(block_size=32, num_seqs=2, lo=64, hi=200)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.q, b.q)
    for s in range(2):
        ka, va = W.logical_kv(a, s)
        kb, vb = W.logical_kv(b, s)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    assert not np.array_equal(a.new_slots, b.new_slots)
