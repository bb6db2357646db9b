"""Plain CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
package (``paged_kv_cache_167_amd``) never imports it, and the two share no
code: no kernels, headers, helpers, tables or pre/post-processing.  The only
thing both sides consume is the seeded synthetic input from ``workloads/``,
which contains none of the arithmetic below.

Everything here is numpy, float64 for all floating point.  It is slow and
written to be checked against the pages by eye.

Sources (page title, section):
  [DRV]  "揭开 NVIDIA 驱动栈的面纱：GPU 显存页表与 vLLM 中的 PagedAttention
         是如何在底层协同的" (kwkd.cn) -- section 6 gives the logical-token to
         (physical block, offset) translation with a worked example, and the
         k_cache pointer formula.
  [SRC]  vLLM source walk-through page (peacm.com) -- section 3.2 shows the
         append of a new token into the last block, section 3.4 the per-block
         paged attention loop, the tail mask and the online-softmax update.
  [CON]  "PagedAttention：当 KV Cache 遇到操作系统分页" (forceinjection.github.io)
         -- section 3.1 (block = B tokens of one layer; block table maps logical
         to physical blocks), section 3.2 (the kernel walks the table and
         gathers block by block).
  [SOSP] "《Efficient Memory Management for LLM Serving with PagedAttention》
         深度解读报告" (zako-mio.github.io) -- section 2.3 (K and V blocks are
         managed separately; the fill count keeps padding out of the result),
         section 3.3 (the result equals the one on contiguously stored KV),
         section 3.4 (write the new token first, then attend over all valid KV),
         section 4.4 (the attention mathematics is unchanged).

Readings where the pages are silent (each listed in the design notes):
  * slot encoding: slot = physical_block * B + offset; slot < 0 means "skip".
  * GQA: query head h reads kv head h // G, G = num_q_heads / num_kv_heads.
  * context_lens count the token just written (write first, then attend).
  * ctx == 0 yields an all-zero output row.
  * pool layout [num_blocks, num_kv_heads, B, head_dim], K and V separate.

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
(worked example from [DRV] section 6, brute force, torch SDPA on contiguous
K/V, permutation / block-size / sharing invariants, closed forms); the FP8 part
([CON] section 6) by ``tests/test_oracle_fp8.py`` (code values fixed by the E4M3
definition, torch's float8_e4m3fn table and rounding, brute-force nearest code,
ties, saturation, and lossless round trips that reduce FP8 decode to the fp64 one);
``copy_blocks`` and ``BlockManager`` by ``tests/test_oracle_blocks.py`` (every sequence
reads back its own token history through random forks, appends, frees and swaps; reference
counts equal table references; planted copy-on-write mistakes are caught);
``prefill`` by ``tests/test_oracle_prefill.py`` (torch SDPA with a causal or bottom-right
mask in float64, pure-Python loops, reduction to ``decode`` at one token per sequence,
chunk-split invariance).
"""

from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Address translation  ([DRV] section 6; [CON] section 3.1)
# ---------------------------------------------------------------------------

def locate_kv(logical_pos: int, block_table, block_size: int) -> tuple[int, int]:
    """Map a logical token position to (physical block id, offset in block).

    The logical block is the position divided by the block size, the offset is
    the remainder, and the block table turns the logical block into the
    physical one ([DRV] section 6; [SRC] section 3.2 does the same split when
    appending a token).
    """
    logical_block = logical_pos // block_size
    offset = logical_pos % block_size
    return int(block_table[logical_block]), int(offset)


def slot_to_block_offset(slot: int, block_size: int) -> tuple[int, int]:
    """Decode the flat slot index (reading: slot = phys * B + offset)."""
    return int(slot) // block_size, int(slot) % block_size


# ---------------------------------------------------------------------------
# Cache write  ([SRC] section 3.2 append_token; [SOSP] sections 3.2 and 3.4)
# ---------------------------------------------------------------------------

def cache_write(k, v, slot_mapping, k_cache, v_cache, block_size: int):
    """Return copies of the two pools with each new token's K/V stored in its slot.

    k, v:          [T, Hkv, D]
    slot_mapping:  [T] integers, slot = phys * B + offset; negative = skip
    k_cache/v_cache: [N, Hkv, B, D], same dtype as k/v

    The store is a plain element copy in the cache dtype (no arithmetic), so
    the result is bit-exact by construction.  K and V are separate pools
    ([SOSP] section 2.3).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, off = slot_to_block_offset(slot, block_size)
        kc[blk, :, off, :] = k[t]  # every kv head of token t
        vc[blk, :, off, :] = v[t]
    return kc, vc


# ---------------------------------------------------------------------------
# Gather through the block table  ([CON] section 3.2; [SOSP] section 2.3)
# ---------------------------------------------------------------------------

def gather_head(cache, table_row, ctx: int, block_size: int, kv_head: int) -> np.ndarray:
    """Collect one kv head of one sequence into a contiguous [ctx, D] float64 array.

    Logical blocks 0..ceil(ctx/B)-1 are looked up in the table in order, their
    [B, D] tiles are concatenated, and only the first ctx positions are kept:
    the unfilled tail of the last block never enters the result ([SOSP]
    section 2.3; [SRC] section 3.4 masks the same positions).
    """
    n_blocks = -(-ctx // block_size)
    tiles = [np.asarray(cache[int(table_row[j]), kv_head], dtype=np.float64)
             for j in range(n_blocks)]
    if not tiles:
        return np.zeros((0, cache.shape[-1]), dtype=np.float64)
    return np.concatenate(tiles, axis=0)[:ctx]


# ---------------------------------------------------------------------------
# Decode attention: the plain definition  ([SOSP] sections 3.3 and 4.4)
# ---------------------------------------------------------------------------

def softmax(z: np.ndarray) -> np.ndarray:
    """Textbook softmax with the max subtracted ([SRC] section 3.4, 'traditional' form)."""
    e = np.exp(z - z.max())
    return e / e.sum()


def decode_one(q, k_cache, v_cache, block_tables, context_lens, scale: float,
               block_size: int, num_kv_heads: int, s: int, h: int) -> np.ndarray:
    """Attention output of query head h of sequence s, float64 [D].

    Paged attention computes exactly the attention over the contiguously
    stored KV ([SOSP] sections 3.3, 4.4), so this is that definition:
    out = softmax(scale * K q) V over the sequence's first ctx positions.
    """
    num_q_heads = q.shape[1]
    group = num_q_heads // num_kv_heads
    kv_head = h // group
    ctx = int(context_lens[s])
    d = q.shape[2]
    if ctx == 0:
        return np.zeros(d, dtype=np.float64)
    keys = gather_head(k_cache, block_tables[s], ctx, block_size, kv_head)
    vals = gather_head(v_cache, block_tables[s], ctx, block_size, kv_head)
    qv = np.asarray(q[s, h], dtype=np.float64)
    p = softmax(float(scale) * (keys @ qv))
    return p @ vals


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
           block_size: int, num_kv_heads: int) -> np.ndarray:
    """All outputs, float64 [S, Hq, D]; one gather per (sequence, kv head)."""
    num_seqs, num_q_heads, d = q.shape
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_seqs, num_q_heads, d), dtype=np.float64)
    for s in range(num_seqs):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        for kvh in range(num_kv_heads):
            keys = gather_head(k_cache, block_tables[s], ctx, block_size, kvh)
            vals = gather_head(v_cache, block_tables[s], ctx, block_size, kvh)
            for g in range(group):
                h = kvh * group + g
                qv = np.asarray(q[s, h], dtype=np.float64)
                p = softmax(float(scale) * (keys @ qv))
                out[s, h] = p @ vals
    return out


# ---------------------------------------------------------------------------
# Algebra the GPU path relies on, written as plain mirrors so the tests can pin
# them to the definition above.  Neither is used to produce expected values for
# the GPU comparison; those come from decode()/decode_one().
# ---------------------------------------------------------------------------

def decode_one_online(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                      block_size: int, num_kv_heads: int, s: int, h: int) -> np.ndarray:
    """Block-by-block online softmax ([SRC] section 3.4, the running max / sum update).

    Per logical block: new max = max(old max, block max); correction =
    exp(old max - new max); running sum = old sum * correction + sum of
    exp(score - new max) over the block; running output likewise; divide by
    the running sum at the end.  The page's code snippet has defects (an
    undefined previous max, a final division by the output's own sum); the
    recurrence stated beside it is what is followed here.
    """
    num_q_heads = q.shape[1]
    group = num_q_heads // num_kv_heads
    kv_head = h // group
    ctx = int(context_lens[s])
    d = q.shape[2]
    if ctx == 0:
        return np.zeros(d, dtype=np.float64)
    qv = np.asarray(q[s, h], dtype=np.float64)
    m = -math.inf
    ell = 0.0
    acc = np.zeros(d, dtype=np.float64)
    n_blocks = -(-ctx // block_size)
    for j in range(n_blocks):
        phys = int(block_tables[s][j])
        valid = min(block_size, ctx - j * block_size)
        kb = np.asarray(k_cache[phys, kv_head, :valid], dtype=np.float64)
        vb = np.asarray(v_cache[phys, kv_head, :valid], dtype=np.float64)
        z = float(scale) * (kb @ qv)
        m_new = max(m, float(z.max()))
        corr = math.exp(m - m_new) if m != -math.inf else 0.0
        e = np.exp(z - m_new)
        ell = ell * corr + float(e.sum())
        acc = acc * corr + e @ vb
        m = m_new
    return acc / ell


def decode_one_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                           block_size: int, num_kv_heads: int, s: int, h: int,
                           partition_size: int) -> np.ndarray:
    """Split the context into partitions, normalise each, merge by log-sum-exp.

    Not on the pages: it is the online-softmax merge of [SRC] section 3.4
    applied to whole partitions instead of blocks.  Partition p covers logical
    positions [p*P, min((p+1)*P, ctx)); it yields its max m_p, its sum l_p and
    its normalised output o_p.  The merge takes M = max m_p, weights
    w_p = l_p * exp(m_p - M), and returns sum(w_p o_p) / sum(w_p), adding
    partitions in index order.
    """
    num_q_heads = q.shape[1]
    group = num_q_heads // num_kv_heads
    kv_head = h // group
    ctx = int(context_lens[s])
    d = q.shape[2]
    if ctx == 0:
        return np.zeros(d, dtype=np.float64)
    keys = gather_head(k_cache, block_tables[s], ctx, block_size, kv_head)
    vals = gather_head(v_cache, block_tables[s], ctx, block_size, kv_head)
    qv = np.asarray(q[s, h], dtype=np.float64)
    z = float(scale) * (keys @ qv)
    parts = []
    for start in range(0, ctx, partition_size):
        zp = z[start:start + partition_size]
        m_p = float(zp.max())
        e = np.exp(zp - m_p)
        l_p = float(e.sum())
        o_p = (e @ vals[start:start + partition_size]) / l_p
        parts.append((m_p, l_p, o_p))
    big_m = max(m_p for m_p, _, _ in parts)
    num = np.zeros(d, dtype=np.float64)
    den = 0.0
    for m_p, l_p, o_p in parts:
        w = l_p * math.exp(m_p - big_m)
        num += w * o_p
        den += w
    return num / den


# ---------------------------------------------------------------------------
# Block copies and the block manager  ([SRC] section 3.2: the free pool, allocate,
# append a token; [SRC] section 3.3: swap a preempted sequence's blocks out to CPU
# memory; [DRV] section 4 and [SOSP] section 2.4: several tables point at one block,
# reference counts and copy-on-write protect writes; [CON] section 4.3).
# Readings where the pages are silent: the free list is a stack (a released block is
# the next one handed out) over an initial order; a copy-on-write happens when a token
# is appended into a partly filled block that another table also points at; a swap
# moves every distinct block of a group of tables once, keeping their sharing.
# ---------------------------------------------------------------------------

def copy_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """Copies of the destination pools with dst[d] = src[s] for every (s, d) pair, in
    order; a pair naming a block outside its pool is skipped.  All kv heads, slots and
    dims of a block move together: a block is the unit of sharing and of swapping."""
    dk, dv = np.array(dst_k, copy=True), np.array(dst_v, copy=True)
    for s_blk, d_blk in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= s_blk < len(src_k) and 0 <= d_blk < len(dk)):
            continue
        dk[d_blk] = src_k[s_blk]
        dv[d_blk] = src_v[s_blk]
    return dk, dv


class BlockManager:
    """Reference counts over a pool of num_blocks physical blocks of block_size slots."""

    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if order is None else [int(b) for b in order]
        assert sorted(order) == list(range(num_blocks)), "order must be a permutation"
        self.free = order[::-1]  # a stack: the first block of order is handed out first
        self.refcount = [0] * num_blocks

    def allocate(self) -> int:
        if not self.free:
            raise MemoryError("no free block")
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def share(self, b: int) -> None:
        assert self.refcount[b] > 0
        self.refcount[b] += 1

    def release(self, b: int) -> None:
        assert self.refcount[b] > 0
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    def append_slot(self, table: list, ctx: int):
        """Slot of the token at position ctx of a sequence whose table is `table` (list of
        block ids, updated in place), and the (source, destination) copy it needs or None.
        A new block is taken when the position starts one; a shared last block is first
        copied into a block of its own."""
        idx, off = divmod(int(ctx), self.block_size)
        cow = None
        if off == 0:
            assert idx == len(table)
            table.append(self.allocate())
        else:
            last = table[idx]
            if self.refcount[last] > 1:
                new = self.allocate()
                self.release(last)
                table[idx] = new
                cow = (last, new)
        return table[idx] * self.block_size + off, cow

    def fork(self, table: list) -> list:
        """A second table over the same blocks (parallel sampling of one prompt)."""
        for b in table:
            self.share(b)
        return list(table)

    def free_table(self, table: list) -> None:
        for b in table:
            self.release(b)
        table.clear()

    def move(self, tables: list, dst: "BlockManager") -> list:
        """Move every block of the given tables to the pool dst manages: each distinct block
        once, the tables rewritten in place, sharing among them kept.  Returns the
        (source, destination) copies, in the order the blocks are first met."""
        if len({b for table in tables for b in table}) > len(dst.free):
            raise MemoryError("not enough free blocks in the destination pool")  # nothing moved
        mapping, pairs = {}, []
        for table in tables:
            for j, b in enumerate(table):
                if b not in mapping:
                    mapping[b] = dst.allocate()
                    pairs.append((b, mapping[b]))
                else:
                    dst.share(mapping[b])
                self.release(b)
                table[j] = mapping[b]
        return pairs


# ---------------------------------------------------------------------------
# Several query tokens per sequence: the prompt phase, in chunks, over the paged
# cache  ([SOSP] section 2.1: the prompt is taken in at once, as matrix work;
# [SOSP] section 5.1, item 5 and [VATT] "3 分钟速读" point 1: paged prefill,
# later done in chunks).  Reading: the chunk's n tokens are the last n positions
# of the context (written before attention, as a decode step writes its token:
# [SOSP] section 3.4), and query i, at position ctx - n + i, attends causally to
# positions 0 .. ctx - n + i.  n = 1 is the decode step.
# ---------------------------------------------------------------------------

def visible_keys(ctx: int, n: int, i: int) -> int:
    """Keys that query i of an n-token chunk ending a ctx-token context sees: positions
    0 .. ctx - n + i, its own included."""
    return ctx - n + i + 1


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
            block_size: int, num_kv_heads: int) -> np.ndarray:
    """Outputs of every query token, float64 [total_q, Hq, D].

    q:            [total_q, Hq, D]; sequence s owns rows query_start[s] .. query_start[s+1]-1
    query_start:  [S + 1] non-decreasing offsets, query_start[0] = 0
    context_lens: [S], counting the chunk; a chunk longer than its context is
                  invalid and gives NaN rows.
    For each row: softmax(scale * K[:p+1] q_row) V[:p+1] with p the row's position.
    """
    total_q, num_q_heads, d = q.shape
    group = num_q_heads // num_kv_heads
    out = np.zeros((total_q, num_q_heads, d), dtype=np.float64)
    for s in range(len(context_lens)):
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        n, ctx = r1 - r0, int(context_lens[s])
        if n == 0:
            continue
        if n > ctx:
            out[r0:r1] = np.nan
            continue
        for kvh in range(num_kv_heads):
            keys = gather_head(k_cache, block_tables[s], ctx, block_size, kvh)
            vals = gather_head(v_cache, block_tables[s], ctx, block_size, kvh)
            for i in range(n):
                m = visible_keys(ctx, n, i)
                for g in range(group):
                    h = kvh * group + g
                    qv = np.asarray(q[r0 + i, h], dtype=np.float64)
                    p = softmax(float(scale) * (keys[:m] @ qv))
                    out[r0 + i, h] = p @ vals[:m]
    return out


# ---------------------------------------------------------------------------
# FP8 KV cache  ([CON] section 6: the blocks hold compressed K/V and the kernel
# dequantizes them).  The pages name FP8 but no format or scaling; the reading
# taken: the OCP FP8 E4M3 format (4 exponent bits, bias 7, 3 mantissa bits, no
# infinities, the all-ones exponent with mantissa 7 is NaN, largest finite 448),
# one scale for all of K and one for all of V.  Storing x means the code nearest
# to x / scale (ties to an even code, i.e. an even mantissa), saturated to +-448;
# a NaN is stored as 0x7F whatever its sign bit (a NaN's sign carries no value,
# and arithmetic need not keep it); loading a code means its value times the scale.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return math.nan
    if exponent == 0:  # subnormal: mantissa/8 * 2^(1 - bias)
        return sign * (mantissa / 8.0) * 2.0 ** -6
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Values of an array of codes (uint8), float64."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest FP8 E4M3 code of each value (ties to the even code), saturating at +-448.

    The positive finite codes 0x00..0x7E have increasing values; the magnitude is
    clamped to 448 and matched against that list, and the sign bit is the sign of x
    (so -0.0 gives 0x80).  NaN gives 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = E4M3_TABLE[:0x7F]  # codes 0x00..0x7E, values 0 .. 448 increasing
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(pos, mag, side="left"), 0, 0x7E)  # first value >= mag
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - pos[lo]
    d_hi = pos[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def fp8_quotient(x, scale: float) -> np.ndarray:
    """x / scale in float64, with scale taken as the single-precision value the library
    receives.  For fp16 (or fp32) x this is the exact quotient up to one float64 rounding,
    which cannot move it across or onto a midpoint between two E4M3 values: a midpoint has
    at most 5 significant bits, so a quotient that is not exactly on one differs from it by
    far more than 2^-53 relative."""
    s = np.float64(np.float32(scale))
    with np.errstate(invalid="ignore", over="ignore"):
        return np.asarray(x, dtype=np.float64) / s


def cache_write_fp8(k, v, slot_mapping, k_cache, v_cache, block_size: int, k_scale: float,
                    v_scale: float):
    """Like cache_write, but each stored element is the E4M3 code nearest to x / scale
    (ties to the even code, saturating, NaN to 0x7F), the quotient taken exactly."""
    kq = e4m3_encode(fp8_quotient(k, k_scale))
    vq = e4m3_encode(fp8_quotient(v, v_scale))
    return cache_write(kq, vq, slot_mapping, k_cache, v_cache, block_size)


def dequantize_pool(codes, scale: float) -> np.ndarray:
    """float64 pool of code values times the scale (the load of [CON] section 6)."""
    return e4m3_decode(codes) * float(scale)


def decode_fp8(q, k_codes, v_codes, k_scale: float, v_scale: float, block_tables,
               context_lens, scale: float, block_size: int, num_kv_heads: int) -> np.ndarray:
    """Attention over the dequantized pools: the plain definition, unchanged."""
    return decode(q, dequantize_pool(k_codes, k_scale), dequantize_pool(v_codes, v_scale),
                  block_tables, context_lens, scale, block_size, num_kv_heads)
