"""Seeded synthetic inputs for paged KV-cache decode.

This module builds inputs only: query vectors, per-token K/V for every logical
position, block tables handed out by a shuffled host allocator, context
lengths and the slot of every token.  It holds none of the attention
arithmetic; both the GPU path and the CPU oracle consume what it returns,
and each builds its own KV pool from the tokens with its own cache write.

Every sequence ends with the token that the current decode step appends: its
K/V and slot are kept apart (``new_k``, ``new_v``, ``new_slots``) because the
step writes it before attending, and context lengths count it.

Workload shapes follow the five benchmark settings of the project: a tiny fp32
case, a Llama-3-8B-shaped decode layer, a Llama-2-70B-shaped 8K-context layer,
parallel sampling with shared prompt blocks, and a 32K-128K context sweep over
block sizes 8/16/32.  No dataset or trained weight is involved; values are
normal with a stated standard deviation, rounded once to the cache dtype.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "BlockAllocator",
    "PoolExhausted",
    "PagedDecodeCase",
    "make_case",
    "logical_kv",
    "tiny_fp32",
    "llama3_8b",
    "llama2_70b",
    "shared_prefix",
    "long_context",
    "CONFIGS",
    "PagedPrefillCase",
    "make_prefill_case",
    "prefill_llama3_8b",
    "prefill_llama2_70b",
    "PREFILL_CONFIGS",
]


class PoolExhausted(RuntimeError):
    """Raised when the host allocator has no free physical block left."""


class BlockAllocator:
    """Free list of physical block ids with reference counts.

    Blocks come out in the order of a seeded random permutation, so physical
    placement is scattered over the pool.  ``share`` adds a reference to an
    allocated block (several block tables pointing at one physical block).
    """

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.num_blocks = int(num_blocks)
        # pop() takes from the end; reverse so the permutation is used front to back
        self._free = list(rng.permutation(self.num_blocks)[::-1])
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise PoolExhausted(f"all {self.num_blocks} physical blocks are in use")
        b = int(self._free.pop())
        self.refcount[b] = 1
        return b

    def share(self, block: int) -> int:
        if self.refcount[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self.refcount[block] += 1
        return int(block)

    def release(self, block: int) -> None:
        if self.refcount[block] <= 0:
            raise ValueError(f"block {block} is not allocated")
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            self._free.append(int(block))


@dataclass
class PagedDecodeCase:
    """One decode step's inputs.  Shapes:

    q            [S, Hq, D]           cache dtype
    block_tables [S, max_blocks]      int32, -1 past each sequence's last block
    context_lens [S]                  int32, counts the token written this step
    prefix_k/v   [Tp, Hkv, D]         every stored token except the new ones
                                      (a shared prompt is listed once)
    prefix_slots [Tp]                 int64 slot of each prefix token
    new_k/v      [S, Hkv, D]          the token each sequence appends this step
    new_slots    [S]                  int64 slot of that token
    """

    name: str
    dtype: np.dtype
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    prefix_k: np.ndarray
    prefix_v: np.ndarray
    prefix_slots: np.ndarray
    new_k: np.ndarray
    new_v: np.ndarray
    new_slots: np.ndarray
    refcount: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elt_bytes(self) -> int:
        return int(np.dtype(self.dtype).itemsize)

    def empty_pool(self) -> np.ndarray:
        """A NaN-filled [N, Hkv, B, D] pool: every slot nobody writes stays NaN."""
        return np.full((self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim),
                       np.nan, dtype=self.dtype)

    def kv_bytes(self) -> int:
        """Logical K+V bytes one decode step reads: sum(ctx) * Hkv * D * 2 * elt."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * \
            self.head_dim * 2 * self.elt_bytes

    def unique_kv_bytes(self) -> int:
        """Bytes of distinct physical slots read (shared prompt blocks counted once)."""
        seen = set()
        tokens = 0
        for s in range(self.num_seqs):
            ctx = int(self.context_lens[s])
            for j in range(-(-ctx // self.block_size)):
                phys = int(self.block_tables[s, j])
                if phys not in seen:
                    seen.add(phys)
                    tokens += min(self.block_size, ctx - j * self.block_size)
        return tokens * self.num_kv_heads * self.head_dim * 2 * self.elt_bytes


def logical_kv(case: PagedDecodeCase, s: int):
    """Sequence s's K and V in logical order, [ctx, Hkv, D] each (the dense form)."""
    rows = case.meta["seq_rows"][s]
    k = np.concatenate([case.prefix_k[rows], case.new_k[s:s + 1]], axis=0)
    v = np.concatenate([case.prefix_v[rows], case.new_v[s:s + 1]], axis=0)
    return k, v


# ---------------------------------------------------------------------------
# helpers (input construction only)
# ---------------------------------------------------------------------------

def _slots(table_row: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Slot of each logical position: physical block * B + offset in the block."""
    positions = np.asarray(positions, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[positions // block_size]
    return phys * block_size + positions % block_size


def _normal(rng: np.random.Generator, shape, sigma: float, dtype) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x.astype(dtype)  # one round-to-nearest-even to the cache dtype


def _plant_needle(keys: np.ndarray, q_seq: np.ndarray, pos: int, group: int, dtype) -> None:
    """Make position ``pos`` dominate every query head of each kv-head group.

    The planted key is alpha * u / |u| with u the sum of the group's query
    vectors and alpha = 16 * sqrt(D), so the group's scores at ``pos`` exceed
    all others by a wide margin and the output is close to that token's V.
    """
    num_kv_heads, d = keys.shape[1], keys.shape[2]
    alpha = 16.0 * np.sqrt(d)
    for kvh in range(num_kv_heads):
        u = q_seq[kvh * group:(kvh + 1) * group].astype(np.float64).sum(axis=0)
        keys[pos, kvh] = (alpha * u / np.linalg.norm(u)).astype(dtype)


def _poscode(vals: np.ndarray, first_pos: int, denom: float, dtype) -> None:
    """Coordinate 0 of every V row carries its logical position / denom."""
    n = vals.shape[0]
    pos = np.arange(first_pos, first_pos + n, dtype=np.float64)
    vals[:, :, 0] = (pos / denom)[:, None].astype(dtype)


def _assemble(name, dtype, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
              scale, ctx, tables, q, seq_tokens, refcount, meta) -> PagedDecodeCase:
    """Split per-sequence token lists into the prefix store and the new tokens.

    ``seq_tokens`` is a list over sequences of (k, v, slots) triples holding the
    tokens that sequence itself stores (shared prompt tokens appear only under
    the sequence that first owned them); the last triple row of each sequence
    is its new token.
    """
    num_seqs = len(ctx)
    pk, pv, ps, nk, nv, ns = [], [], [], [], [], []
    own_rows = []
    row = 0
    for s in range(num_seqs):
        k, v, slots = seq_tokens[s]
        pk.append(k[:-1])
        pv.append(v[:-1])
        ps.append(slots[:-1])
        own_rows.append(np.arange(row, row + len(k) - 1, dtype=np.int64))
        row += len(k) - 1
        nk.append(k[-1])
        nv.append(v[-1])
        ns.append(slots[-1])
    extra_rows = []
    for extra_k, extra_v, extra_slots in meta.pop("_extra_prefix", []):
        pk.append(extra_k)
        pv.append(extra_v)
        ps.append(extra_slots)
        extra_rows.append(np.arange(row, row + len(extra_k), dtype=np.int64))
        row += len(extra_k)
    # rows of the prefix store holding each sequence's positions 0..ctx-2, in order
    shared_of = meta.pop("_shared_of", None)
    seq_rows = []
    for s in range(num_seqs):
        parts = [] if shared_of is None or shared_of[s] < 0 else [extra_rows[shared_of[s]]]
        parts.append(own_rows[s])
        seq_rows.append(np.concatenate(parts))
    meta["seq_rows"] = seq_rows
    d = head_dim
    prefix_k = np.concatenate(pk, axis=0) if pk else np.zeros((0, num_kv_heads, d), dtype)
    prefix_v = np.concatenate(pv, axis=0) if pv else np.zeros((0, num_kv_heads, d), dtype)
    prefix_slots = np.concatenate(ps).astype(np.int64) if ps else np.zeros(0, np.int64)
    return PagedDecodeCase(
        name=name, dtype=np.dtype(dtype), num_seqs=num_seqs, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=int(num_blocks), scale=float(scale),
        context_lens=np.asarray(ctx, dtype=np.int32), block_tables=tables, q=q,
        prefix_k=prefix_k, prefix_v=prefix_v, prefix_slots=prefix_slots,
        new_k=np.stack(nk).astype(dtype) if nk else np.zeros((0, num_kv_heads, d), dtype),
        new_v=np.stack(nv).astype(dtype) if nv else np.zeros((0, num_kv_heads, d), dtype),
        new_slots=np.asarray(ns, dtype=np.int64),
        refcount=refcount, meta=meta)


def _tables_from(allocator: BlockAllocator, blocks_per_seq, width: int) -> np.ndarray:
    tables = np.full((len(blocks_per_seq), max(width, 1)), -1, dtype=np.int32)
    for s, nb in enumerate(blocks_per_seq):
        for j in range(nb):
            tables[s, j] = allocator.allocate()
    return tables


# ---------------------------------------------------------------------------
# generic case
# ---------------------------------------------------------------------------

_LOGICAL_MEMO = {}  # one entry: the last logical data set (lets block-size sweeps reuse it)
_PROGRESS = None    # optional callable(message): told as each sequence's data is generated


def set_progress(fn) -> None:
    """Report generation progress through fn(message) (None: silent)."""
    global _PROGRESS
    _PROGRESS = fn


def _logical_data(lseed, ctx, num_q_heads, num_kv_heads, head_dim, sigma, dtype, variant):
    """Queries and per-sequence logical K/V; a function of the logical seed only."""
    if variant not in ("plain", "needle", "poscode"):
        raise ValueError(f"unknown variant {variant!r}")
    key = (lseed, tuple(int(c) for c in ctx), num_q_heads, num_kv_heads, head_dim, float(sigma),
           np.dtype(dtype).str, variant)
    if key in _LOGICAL_MEMO:
        return _LOGICAL_MEMO[key]
    _LOGICAL_MEMO.clear()
    group = num_q_heads // num_kv_heads
    q = _normal(np.random.default_rng([lseed, 0]), (len(ctx), num_q_heads, head_dim), sigma, dtype)
    denom = float(max(int(max(ctx)) if len(ctx) else 1, 1))
    needle_rng = np.random.default_rng([lseed, 9])
    logical = []
    for s, c in enumerate(ctx):
        c = int(c)
        rng = np.random.default_rng([lseed, 1, s])
        k = _normal(rng, (c, num_kv_heads, head_dim), sigma, dtype)
        v = _normal(rng, (c, num_kv_heads, head_dim), sigma, dtype)
        if variant == "needle":
            _plant_needle(k, q[s], int(needle_rng.integers(0, c)), group, dtype)
        elif variant == "poscode":
            _poscode(v, 0, denom, dtype)
        logical.append((k, v))
        if _PROGRESS is not None:
            _PROGRESS(f"sequence {s + 1}/{len(ctx)}: {c} tokens generated")
    _LOGICAL_MEMO[key] = (q, logical)
    return q, logical


def clear_memo() -> None:
    _LOGICAL_MEMO.clear()


def make_case(*, name="custom", seed=0, dtype=np.float16, context_lens, num_q_heads,
              num_kv_heads, head_dim, block_size, pool_factor=1.2, num_blocks=None,
              sigma=0.5, scale=None, variant="plain", extra_table_cols=0,
              logical_seed=None) -> PagedDecodeCase:
    """Independent sequences, each with its own scattered blocks.

    ``logical_seed`` fixes the per-sequence K/V streams independently of the
    pool seed, so the same logical data can be laid out with different block
    sizes or placements.  ``extra_table_cols`` widens the table with -1 columns.
    """
    assert num_q_heads % num_kv_heads == 0
    ctx = np.asarray(context_lens, dtype=np.int64)
    if np.any(ctx < 1):
        raise ValueError("every sequence needs ctx >= 1: the step appends a token before attending")
    group = num_q_heads // num_kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    lseed = seed if logical_seed is None else logical_seed
    blocks_per_seq = [int(-(-c // block_size)) for c in ctx]
    needed = sum(blocks_per_seq)
    if num_blocks is None:
        num_blocks = max(1, int(np.ceil(pool_factor * needed)))
    alloc = BlockAllocator(num_blocks, np.random.default_rng([seed, 7, block_size]))
    width = (max(blocks_per_seq) if blocks_per_seq else 1) + extra_table_cols
    tables = _tables_from(alloc, blocks_per_seq, width)
    q, logical = _logical_data(lseed, ctx, num_q_heads, num_kv_heads, head_dim, sigma, dtype,
                               variant)
    seq_tokens = []
    for s, c in enumerate(ctx):
        k, v = logical[s]
        slots = _slots(tables[s], np.arange(int(c)), block_size)
        seq_tokens.append((k, v, slots))
    meta = {"variant": variant, "seed": seed, "sigma": sigma}
    return _assemble(name, dtype, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     scale, ctx, tables, q, seq_tokens, alloc.refcount, meta)


# ---------------------------------------------------------------------------
# the five benchmark workloads
# ---------------------------------------------------------------------------

def tiny_fp32(variant="plain") -> PagedDecodeCase:
    """4 sequences, ctx {1,17,100,250}, 8/8 heads, D 64, B 16, 64-block pool, N(0,1), fp32."""
    return make_case(name="tiny_fp32", seed=1001, dtype=np.float32,
                     context_lens=[1, 17, 100, 250], num_q_heads=8, num_kv_heads=8,
                     head_dim=64, block_size=16, num_blocks=64, sigma=1.0,
                     scale=1.0 / 8.0, variant=variant)


def llama3_8b(variant="plain", num_seqs=64) -> PagedDecodeCase:
    """Batch 64, 32 q / 8 kv heads, D 128, B 16, ctx uniform [512, 4096], pool 1.2x, fp16."""
    rng = np.random.default_rng(1002)
    ctx = rng.integers(512, 4096, size=num_seqs, endpoint=True)
    return make_case(name="llama3_8b", seed=1002, dtype=np.float16, context_lens=ctx,
                     num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                     pool_factor=1.2, sigma=0.5, variant=variant)


def llama2_70b(variant="plain", num_seqs=32, context_len=8192) -> PagedDecodeCase:
    """Batch 32, ctx 8192 each, 64 q / 8 kv heads, D 128, B 16, pool 1.2x, fp16."""
    return make_case(name="llama2_70b", seed=1003, dtype=np.float16,
                     context_lens=[context_len] * num_seqs, num_q_heads=64, num_kv_heads=8,
                     head_dim=128, block_size=16, pool_factor=1.2, sigma=0.5, variant=variant)


def shared_prefix(variant="plain", num_prompts=16, samples=8, prompt_len=2000,
                  max_tail=256) -> PagedDecodeCase:
    """Parallel sampling: each prompt's blocks are shared by its samples (refcount = samples).

    Each sample owns a private tail of uniform [0, max_tail] tokens plus the
    token it appends this step, so ctx = prompt_len + tail + 1.  A prompt of
    2000 tokens fills exactly 125 blocks of 16, so no append lands in a shared
    block.  32 q / 8 kv heads, D 128, B 16, fp16, N(0, 0.5^2).
    """
    seed, B, hq, hkv, d, sigma = 1004, 16, 32, 8, 128, 0.5
    dtype = np.float16
    group = hq // hkv
    rng = np.random.default_rng(seed)
    tails = rng.integers(0, max_tail, size=num_prompts * samples, endpoint=True)
    ctx = prompt_len + tails + 1
    prompt_blocks = -(-prompt_len // B)
    own_blocks = [int(-(-c // B)) - (prompt_len // B) for c in ctx]
    needed = num_prompts * prompt_blocks + sum(own_blocks)
    num_blocks = int(np.ceil(1.2 * needed))
    alloc = BlockAllocator(num_blocks, np.random.default_rng([seed, 7, B]))
    width = int(max(-(-c // B) for c in ctx))
    tables = np.full((len(ctx), width), -1, dtype=np.int32)
    q = _normal(np.random.default_rng([seed, 0]), (len(ctx), hq, d), sigma, dtype)
    denom = float(ctx.max())
    seq_tokens = []
    extra = []
    needle_rng = np.random.default_rng([seed, 9])
    for p in range(num_prompts):
        prng = np.random.default_rng([seed, 2, p])
        pk = _normal(prng, (prompt_len, hkv, d), sigma, dtype)
        pv = _normal(prng, (prompt_len, hkv, d), sigma, dtype)
        if variant == "poscode":
            _poscode(pv, 0, denom, dtype)
        pblocks = [alloc.allocate() for _ in range(prompt_blocks)]
        for b in pblocks:  # one reference per sample
            for _ in range(samples - 1):
                alloc.share(b)
        pslots = _slots(np.asarray(pblocks), np.arange(prompt_len), B)
        extra.append((pk, pv, pslots))
        for i in range(samples):
            s = p * samples + i
            c = int(ctx[s])
            tables[s, :prompt_blocks] = pblocks
            for j in range(prompt_blocks, -(-c // B)):
                tables[s, j] = alloc.allocate()
            trng = np.random.default_rng([seed, 3, s])
            n_own = c - prompt_len
            tk = _normal(trng, (n_own, hkv, d), sigma, dtype)
            tv = _normal(trng, (n_own, hkv, d), sigma, dtype)
            if variant == "needle":
                # planted in the private part: the shared prompt is common to 8 different queries
                _plant_needle(tk, q[s], int(needle_rng.integers(0, n_own)), group, dtype)
            elif variant == "poscode":
                _poscode(tv, prompt_len, denom, dtype)
            tslots = _slots(tables[s], np.arange(prompt_len, c), B)
            seq_tokens.append((tk, tv, tslots))
    meta = {"variant": variant, "seed": seed, "sigma": sigma, "prompt_len": prompt_len,
            "samples": samples, "_extra_prefix": extra,
            "_shared_of": [s // samples for s in range(len(ctx))]}
    return _assemble("shared_prefix", dtype, hq, hkv, d, B, num_blocks, 1.0 / np.sqrt(d), ctx,
                     tables, q, seq_tokens, alloc.refcount, meta)


def shared_groups(layout, seed=2024, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                  dtype=np.float16, sigma=0.5, variant="plain") -> PagedDecodeCase:
    """A batch of prefix-sharing groups and independent sequences, in the order of ``layout``.

    Each item is ("g", prompt_len, tails): a group of len(tails) sequences whose tables hold
    the same physical blocks for the prompt_len prompt tokens (a multiple of block_size),
    each with a private tail of that many tokens plus the token it appends this step
    (ctx = prompt_len + tail + 1); or ("s", ctx): an independent sequence.  meta holds the
    group arrays pa_decode_shared takes: "seq_group" [S], "group_first", "group_size",
    "group_prefix" [NG].
    """
    B, d = block_size, head_dim
    group = num_q_heads // num_kv_heads
    ctx, seq_group, groups = [], [], []
    for item in layout:
        if item[0] == "g":
            _, plen, tails = item
            assert plen % B == 0 and plen > 0
            groups.append((len(ctx), len(tails), plen))
            for t in tails:
                ctx.append(plen + int(t) + 1)
                seq_group.append(len(groups) - 1)
        else:
            ctx.append(int(item[1]))
            seq_group.append(-1)
    ctx = np.asarray(ctx, dtype=np.int64)
    own_blocks = []
    for s, c in enumerate(ctx):
        gi = seq_group[s]
        plen = groups[gi][2] if gi >= 0 else 0
        own_blocks.append(int(-(-int(c) // B)) - plen // B)
    needed = sum(g[2] // B for g in groups) + sum(own_blocks)
    num_blocks = max(4, int(np.ceil(1.3 * needed)) + 2)
    alloc = BlockAllocator(num_blocks, np.random.default_rng([seed, 7, B]))
    width = int(max(-(-int(c) // B) for c in ctx)) + 1
    tables = np.full((len(ctx), width), -1, dtype=np.int32)
    q = _normal(np.random.default_rng([seed, 0]), (len(ctx), num_q_heads, d), sigma, dtype)
    denom = float(ctx.max())
    extra, gblocks = [], []
    for gi, (first, size, plen) in enumerate(groups):
        prng = np.random.default_rng([seed, 2, gi])
        pk = _normal(prng, (plen, num_kv_heads, d), sigma, dtype)
        pv = _normal(prng, (plen, num_kv_heads, d), sigma, dtype)
        if variant == "poscode":
            _poscode(pv, 0, denom, dtype)
        pblocks = [alloc.allocate() for _ in range(plen // B)]
        for b in pblocks:
            for _ in range(size - 1):
                alloc.share(b)
        extra.append((pk, pv, _slots(np.asarray(pblocks), np.arange(plen), B)))
        gblocks.append(pblocks)
    needle_rng = np.random.default_rng([seed, 9])
    seq_tokens = []
    for s, c in enumerate(ctx):
        c = int(c)
        gi = seq_group[s]
        plen = groups[gi][2] if gi >= 0 else 0
        if gi >= 0:
            tables[s, :plen // B] = gblocks[gi]
        for j in range(plen // B, -(-c // B)):
            tables[s, j] = alloc.allocate()
        trng = np.random.default_rng([seed, 3, s])
        n_own = c - plen
        tk = _normal(trng, (n_own, num_kv_heads, d), sigma, dtype)
        tv = _normal(trng, (n_own, num_kv_heads, d), sigma, dtype)
        if variant == "needle":
            _plant_needle(tk, q[s], int(needle_rng.integers(0, n_own)), group, dtype)
        elif variant == "poscode":
            _poscode(tv, plen, denom, dtype)
        seq_tokens.append((tk, tv, _slots(tables[s], np.arange(plen, c), B)))
    meta = {"variant": variant, "seed": seed, "sigma": sigma, "_extra_prefix": extra,
            "_shared_of": list(seq_group),
            "seq_group": np.asarray(seq_group, np.int32),
            "group_first": np.asarray([g[0] for g in groups], np.int32),
            "group_size": np.asarray([g[1] for g in groups], np.int32),
            "group_prefix": np.asarray([g[2] for g in groups], np.int32)}
    return _assemble("shared_groups", dtype, num_q_heads, num_kv_heads, head_dim, B, num_blocks,
                     1.0 / np.sqrt(d), ctx, tables, q, seq_tokens, alloc.refcount, meta)


def shared_prefix_groups(case: PagedDecodeCase):
    """The group arrays of a shared_prefix() batch: prompt p's samples are group p."""
    samples, plen = case.meta["samples"], case.meta["prompt_len"]
    ng = case.num_seqs // samples
    return (np.arange(case.num_seqs, dtype=np.int32) // samples,
            np.arange(ng, dtype=np.int32) * samples, np.full(ng, samples, np.int32),
            np.full(ng, plen, np.int32))


def long_context(block_size=16, variant="plain", num_seqs=8, lo=32768, hi=131072) -> PagedDecodeCase:
    """Batch 8, ctx uniform [32768, 131072], 56 q / 8 kv heads, D 128, fp16.

    The logical K/V and queries depend only on the sequence (seed 1005), so the
    outputs for block sizes 8, 16 and 32 are comparable; each block size gets
    its own shuffled 1.2x pool (seed 1005 + 100 * B).
    """
    rng = np.random.default_rng(1005)
    ctx = rng.integers(lo, hi, size=num_seqs, endpoint=True)
    return make_case(name=f"long_context_b{block_size}", seed=1005 + 100 * block_size,
                     logical_seed=1005, dtype=np.float16, context_lens=ctx, num_q_heads=56,
                     num_kv_heads=8, head_dim=128, block_size=block_size, pool_factor=1.2,
                     sigma=0.5, variant=variant)


CONFIGS = {
    "tiny_fp32": tiny_fp32,
    "llama3_8b": llama3_8b,
    "llama2_70b": llama2_70b,
    "shared_prefix": shared_prefix,
    "long_context": long_context,
}


# ---------------------------------------------------------------------------
# several query tokens per sequence (a prompt chunk)
# ---------------------------------------------------------------------------

@dataclass
class PagedPrefillCase:
    """One chunked-prefill step's inputs.  Shapes:

    q            [Tq, Hq, D]          the chunk's queries, sequences one after another
    query_start  [S + 1]              int32 offsets of each sequence's rows in q
    context_lens [S]                  int32, counting the chunk (its tokens are the last ones)
    block_tables [S, max_blocks]      int32, -1 past each sequence's last block
    prefix_k/v   [Tp, Hkv, D]         the tokens before each chunk, already stored
    prefix_slots [Tp]                 int64
    new_k/v      [Tq, Hkv, D]         the chunk's own K/V, written in the step
    new_slots    [Tq]                 int64
    """

    name: str
    dtype: np.dtype
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray
    query_start: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    prefix_k: np.ndarray
    prefix_v: np.ndarray
    prefix_slots: np.ndarray
    new_k: np.ndarray
    new_v: np.ndarray
    new_slots: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return int(self.query_start[-1])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start).astype(np.int64)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elt_bytes(self) -> int:
        return int(np.dtype(self.dtype).itemsize)

    def empty_pool(self) -> np.ndarray:
        return np.full((self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim),
                       np.nan, dtype=self.dtype)

    def flops(self) -> int:
        """Causal attention work: 4 D flops per (query head, query token, visible key)."""
        n = self.query_lens
        c = self.context_lens.astype(np.int64)
        # keys visible to the chunk's rows: sum over i < n of (c - n + i + 1)
        visible = n * (c - n) + n * (n + 1) // 2
        return int(4 * self.head_dim * self.num_q_heads * visible.sum())

    def kv_bytes(self) -> int:
        """K+V bytes of every context, read once."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * \
            self.head_dim * 2 * self.elt_bytes


def make_prefill_case(*, name="custom_prefill", seed=0, dtype=np.float16, context_lens, query_lens,
                      num_q_heads, num_kv_heads, head_dim, block_size, pool_factor=1.2,
                      num_blocks=None, sigma=0.5, scale=None, variant="plain",
                      logical_seed=None, extra_table_cols=0) -> PagedPrefillCase:
    """Each sequence holds ctx tokens, the last n of which are the chunk being prefilled.

    K/V come from the same per-sequence streams as make_case (so a logical seed fixes them
    independently of the block size); the chunk's queries from their own streams.
    Variants: "plain", or "poscode" (coordinate 0 of V is position / max ctx).
    """
    assert num_q_heads % num_kv_heads == 0
    ctx = np.asarray(context_lens, dtype=np.int64)
    qlen = np.asarray(query_lens, dtype=np.int64)
    if ctx.shape != qlen.shape or np.any(qlen < 0) or np.any(qlen > ctx):
        raise ValueError("need 0 <= query_lens <= context_lens, one per sequence")
    if variant not in ("plain", "poscode"):
        raise ValueError(f"unknown prefill variant {variant!r}")
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    lseed = seed if logical_seed is None else logical_seed
    blocks_per_seq = [int(-(-c // block_size)) for c in ctx]
    if num_blocks is None:
        num_blocks = max(1, int(np.ceil(pool_factor * max(sum(blocks_per_seq), 1))))
    alloc = BlockAllocator(num_blocks, np.random.default_rng([seed, 7, block_size]))
    width = (max(blocks_per_seq) if blocks_per_seq else 1) + extra_table_cols
    tables = _tables_from(alloc, blocks_per_seq, width)
    _, logical = _logical_data(lseed, np.maximum(ctx, 1), num_q_heads, num_kv_heads, head_dim,
                               sigma, dtype, variant)
    pk, pv, ps, nk, nv, ns, qs = [], [], [], [], [], [], []
    for s, c in enumerate(ctx):
        c, n = int(c), int(qlen[s])
        k, v = logical[s]
        k, v = k[:c], v[:c]
        slots = _slots(tables[s], np.arange(c), block_size)
        pk.append(k[:c - n])
        pv.append(v[:c - n])
        ps.append(slots[:c - n])
        nk.append(k[c - n:])
        nv.append(v[c - n:])
        ns.append(slots[c - n:])
        qs.append(_normal(np.random.default_rng([lseed, 10, s]), (n, num_q_heads, head_dim), sigma,
                          dtype))
    cat = lambda xs, shape: np.concatenate(xs, axis=0) if xs else np.zeros(shape, dtype)  # noqa: E731
    d = head_dim
    return PagedPrefillCase(
        name=name, dtype=np.dtype(dtype), num_seqs=len(ctx), num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=int(num_blocks), scale=float(scale), context_lens=ctx.astype(np.int32),
        query_start=np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32),
        block_tables=tables, q=cat(qs, (0, num_q_heads, d)),
        prefix_k=cat(pk, (0, num_kv_heads, d)), prefix_v=cat(pv, (0, num_kv_heads, d)),
        prefix_slots=np.concatenate(ps).astype(np.int64) if ps else np.zeros(0, np.int64),
        new_k=cat(nk, (0, num_kv_heads, d)), new_v=cat(nv, (0, num_kv_heads, d)),
        new_slots=np.concatenate(ns).astype(np.int64) if ns else np.zeros(0, np.int64),
        meta={"variant": variant, "seed": seed, "sigma": sigma})


def prefill_llama3_8b(variant="plain", num_seqs=8, chunk=512) -> PagedPrefillCase:
    """Chunked prefill: 8 sequences, each with U[1024, 3584] tokens already cached and a
    512-token chunk; 32 q / 8 kv heads, D 128, B 16, pool 1.2x, fp16."""
    rng = np.random.default_rng(1006)
    prior = rng.integers(1024, 3584, size=num_seqs, endpoint=True)
    return make_prefill_case(name="prefill_llama3_8b", seed=1006, dtype=np.float16,
                             context_lens=prior + chunk, query_lens=[chunk] * num_seqs,
                             num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                             sigma=0.5, variant=variant)


def prefill_llama2_70b(variant="plain", num_seqs=4, prompt=2048) -> PagedPrefillCase:
    """Whole prompts: 4 sequences of 2048 tokens prefilled at once (ctx = n = 2048);
    64 q / 8 kv heads, D 128, B 16, pool 1.2x, fp16."""
    return make_prefill_case(name="prefill_llama2_70b", seed=1007, dtype=np.float16,
                             context_lens=[prompt] * num_seqs, query_lens=[prompt] * num_seqs,
                             num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                             sigma=0.5, variant=variant)


PREFILL_CONFIGS = {
    "prefill_llama3_8b": prefill_llama3_8b,
    "prefill_llama2_70b": prefill_llama2_70b,
}
