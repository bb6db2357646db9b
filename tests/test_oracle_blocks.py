"""Pins for the oracle's block copies and block manager (sharing, copy-on-write, swap).

Pinned to what the pages fix: several tables may point at one block, writes into a
shared block must not be seen by the other tables (reference counts plus
copy-on-write), a preempted sequence's blocks can move to another pool and back, and
the block is the unit of all of it.  The strongest pin is content-level: random forks,
appends, frees and swaps over a pool of token ids must leave every live sequence
reading back exactly its own token history through its table.
"""
import numpy as np
import pytest

from oracle import pa_oracle as O

B = 4


def _pool(n):
    # one kv head, B slots, one "dim": the slot holds a token id (NaN = never written)
    return np.full((n, 1, B, 1), np.nan), np.full((n, 1, B, 1), np.nan)


def _read(pool, table, n_tokens):
    flat = [pool[table[p // B], 0, p % B, 0] for p in range(n_tokens)]
    return np.array(flat)


def _check_refcounts(mgr, tables):
    counts = np.zeros(len(mgr.refcount), dtype=int)
    for t in tables:
        for b in t:
            counts[b] += 1
    assert list(counts) == mgr.refcount
    assert sorted(mgr.free) == [b for b in range(len(counts)) if counts[b] == 0]


class _World:
    """Sequences = (table, history of token ids); the pools hold the ids."""

    def __init__(self, n_blocks, seed, cow=True):
        self.rng = np.random.default_rng(seed)
        self.mgr = O.BlockManager(n_blocks, B, order=self.rng.permutation(n_blocks))
        self.k, self.v = _pool(n_blocks)
        self.seqs = []
        self.next_id = 1
        self.cow = cow

    def append(self, i):
        table, hist = self.seqs[i]
        slot, pair = self.mgr.append_slot(table, len(hist))
        if pair is not None and self.cow:  # cow=False plants a mistake: the copy is dropped
            self.k, self.v = O.copy_blocks(self.k, self.v, self.k, self.v, [pair])
        tok = self.next_id
        self.next_id += 1
        self.k[slot // B, 0, slot % B, 0] = tok
        self.v[slot // B, 0, slot % B, 0] = -tok
        hist.append(tok)

    def check(self):
        for table, hist in self.seqs:
            assert np.array_equal(_read(self.k, table, len(hist)), np.array(hist, float))
            assert np.array_equal(_read(self.v, table, len(hist)), -np.array(hist, float))
        _check_refcounts(self.mgr, [t for t, _ in self.seqs])


# --------------------------------------------------------------------- BM1-BM3
@pytest.mark.parametrize("seed", range(6))
def test_bm1_random_forks_appends_frees_keep_every_history(seed):
    w = _World(400, seed)
    w.seqs.append(([], []))
    for _ in range(int(w.rng.integers(1, 23))):  # a prompt of 1..22 tokens
        w.append(0)
    for step in range(300):
        op = w.rng.random()
        live = len(w.seqs)
        if op < 0.15 and live < 12:  # parallel sampling: fork a sequence
            i = int(w.rng.integers(live))
            w.seqs.append((w.mgr.fork(w.seqs[i][0]), list(w.seqs[i][1])))
        elif op < 0.22 and live > 1:  # a sequence finishes
            i = int(w.rng.integers(live))
            w.mgr.free_table(w.seqs[i][0])
            w.seqs.pop(i)
        else:
            w.append(int(w.rng.integers(live)))
        w.check()


def test_bm2_appends_never_land_in_a_shared_block():
    w = _World(64, 7)
    w.seqs.append(([], []))
    for _ in range(6):  # 6 tokens: the second block is half full
        w.append(0)
    for _ in range(3):
        w.seqs.append((w.mgr.fork(w.seqs[0][0]), list(w.seqs[0][1])))
    for i in range(4):
        table, hist = w.seqs[i]
        slot, pair = w.mgr.append_slot(table, len(hist))
        assert w.mgr.refcount[slot // B] == 1
        # the first three writers copy the shared half-full block; the last owns it alone
        assert (pair is not None) == (i < 3)
        if pair is not None:
            w.k, w.v = O.copy_blocks(w.k, w.v, w.k, w.v, [pair])
        w.k[slot // B, 0, slot % B, 0] = 100 + i
        w.v[slot // B, 0, slot % B, 0] = -(100 + i)
        hist.append(100 + i)
    w.check()
    assert w.mgr.refcount[w.seqs[0][0][0]] == 4  # the full first block stays shared


def test_bm3_sharing_costs_one_copy_of_the_prompt():
    """N samples of a block-aligned prompt hold the prompt once (O(prompt) memory)."""
    mgr = O.BlockManager(100, 16)
    t0 = []
    for p in range(32):  # a block-aligned prompt of two blocks
        mgr.append_slot(t0, p)
    tables = [t0] + [mgr.fork(t0) for _ in range(7)]
    assert len(mgr.free) == 100 - 2 and all(mgr.refcount[b] == 8 for b in t0)
    for t in tables:  # the first generated token: aligned prompt, so no copy, one new block each
        _, pair = mgr.append_slot(t, 32)
        assert pair is None
    assert len(mgr.free) == 100 - 2 - 8


# --------------------------------------------------------------------- BM4 swap
@pytest.mark.parametrize("seed", range(3))
def test_bm4_swap_out_and_in_keeps_content_and_sharing(seed):
    w = _World(200, 20 + seed)
    w.seqs.append(([], []))
    for _ in range(13):
        w.append(0)
    for _ in range(3):
        w.seqs.append((w.mgr.fork(w.seqs[0][0]), list(w.seqs[0][1])))
        for _ in range(int(w.rng.integers(0, 9))):
            w.append(len(w.seqs) - 1)
    w.check()
    distinct = len({b for t, _ in w.seqs for b in t})
    cpu = O.BlockManager(300, B, order=w.rng.permutation(300))
    ck, cv = _pool(300)
    group = [t for t, _ in w.seqs]
    pairs = w.mgr.move(group, cpu)
    assert len(pairs) == distinct
    ck, cv = O.copy_blocks(w.k, w.v, ck, cv, pairs)
    assert len(w.mgr.free) == 200  # every GPU block came back
    w.k, w.v = _pool(200)          # the GPU pool is reused by others meanwhile
    pairs = cpu.move(group, w.mgr)
    w.k, w.v = O.copy_blocks(ck, cv, w.k, w.v, pairs)
    assert len(cpu.free) == 300
    w.check()
    assert len({b for t, _ in w.seqs for b in t}) == distinct


# --------------------------------------------------------------------- copies
def test_copy_blocks_moves_whole_blocks_and_skips_invalid_pairs():
    rng = np.random.default_rng(3)
    src_k, src_v = rng.standard_normal((6, 2, 4, 3)), rng.standard_normal((6, 2, 4, 3))
    dst_k, dst_v = np.zeros((5, 2, 4, 3)), np.zeros((5, 2, 4, 3))
    k, v = O.copy_blocks(src_k, src_v, dst_k, dst_v, [(4, 0), (-1, 1), (2, 9), (0, 3), (6, 2)])
    assert np.array_equal(k[0], src_k[4]) and np.array_equal(v[0], src_v[4])
    assert np.array_equal(k[3], src_k[0]) and np.array_equal(v[3], src_v[0])
    assert not k[[1, 2, 4]].any() and not v[[1, 2, 4]].any()


# --------------------------------------------------------------------- planted mistakes
def test_planted_missing_copy_is_caught():
    w = _World(64, 11, cow=False)
    w.seqs.append(([], []))
    for _ in range(6):
        w.append(0)
    w.seqs.append((w.mgr.fork(w.seqs[0][0]), list(w.seqs[0][1])))
    w.append(1)
    with pytest.raises(AssertionError):
        w.check()


def test_planted_write_into_shared_block_is_caught(monkeypatch):
    """Without the copy-on-write branch the writer overwrites a slot its sibling reads."""
    def no_cow(self, table, ctx):
        idx, off = divmod(int(ctx), self.block_size)
        if off == 0:
            table.append(self.allocate())
        return table[idx] * self.block_size + off, None
    monkeypatch.setattr(O.BlockManager, "append_slot", no_cow)
    w = _World(64, 12)
    w.seqs.append(([], []))
    for _ in range(6):
        w.append(0)
    w.seqs.append((w.mgr.fork(w.seqs[0][0]), list(w.seqs[0][1])))
    w.append(0)
    w.append(1)
    with pytest.raises(AssertionError):
        w.check()
