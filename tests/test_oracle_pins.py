"""Pins for the CPU oracle: each checks it against something other than itself.

The pins come from what the pages fix (worked example, byte arithmetic,
equality with contiguous attention, block sharing) and from mathematics
(brute force, closed forms, invariants).  ``test_planted_mistakes_are_caught``
plants plausible mistakes in the oracle (on the CPU) and shows that a pin
fails for each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import pa_oracle as O
from tests._helpers import oracle_decode, oracle_pools

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(**kw):
    base = dict(seed=11, dtype=np.float32, context_lens=[1, 5, 16, 17, 40], num_q_heads=4,
                num_kv_heads=2, head_dim=8, block_size=4, num_blocks=None, sigma=1.0)
    base.update(kw)
    return W.make_case(**base)


# --------------------------------------------------------------------- P1
def test_p1_locate_kv_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "locate_kv_example.json")))
    phys, off = O.locate_kv(g["logical_pos"], g["block_table"], g["block_size"])
    assert (phys, off) == (g["expected_physical_block"], g["expected_offset"])
    # the workload generator's slot encoding agrees with the translation
    slot = W._slots(np.array(g["block_table"]), np.array([g["logical_pos"]]), g["block_size"])[0]
    assert O.slot_to_block_offset(slot, g["block_size"]) == (phys, off)


def test_p1_every_workload_slot_matches_translation():
    case = _case()
    for s in range(case.num_seqs):
        ctx = int(case.context_lens[s])
        rows = case.meta["seq_rows"][s]
        slots = list(case.prefix_slots[rows]) + [case.new_slots[s]]
        for pos in range(ctx):
            assert O.slot_to_block_offset(slots[pos], case.block_size) == \
                O.locate_kv(pos, case.block_tables[s], case.block_size)


# --------------------------------------------------------------------- P2
def _brute_force(q_s, k_log, v_log, scale, group):
    """Pure-Python attention over the dense logical K/V of one sequence."""
    hq, d = q_s.shape
    out = np.zeros((hq, d))
    for h in range(hq):
        kvh = h // group
        z = [scale * math.fsum(float(q_s[h, i]) * float(k_log[t, kvh, i]) for i in range(d))
             for t in range(k_log.shape[0])]
        m = max(z)
        e = [math.exp(x - m) for x in z]
        den = math.fsum(e)
        for i in range(d):
            out[h, i] = math.fsum(e[t] * float(v_log[t, kvh, i]) for t in range(len(e))) / den
    return out


@pytest.mark.parametrize("block_size", [1, 4, 16])
@pytest.mark.parametrize("group", [1, 2, 4])
def test_p2_brute_force_tiny(block_size, group):
    case = _case(context_lens=[3, 17, 40], num_q_heads=2 * group, num_kv_heads=2,
                 head_dim=8, block_size=block_size, seed=100 + block_size + group)
    kc, vc = oracle_pools(case)
    ref = oracle_decode(case, kc, vc)
    for s in range(case.num_seqs):
        k_log, v_log = W.logical_kv(case, s)
        bf = _brute_force(case.q[s], k_log, v_log, case.scale, group)
        np.testing.assert_allclose(ref[s], bf, rtol=0, atol=1e-12)


# --------------------------------------------------------------------- P3
def _sdpa_dense(case):
    """torch SDPA in float64 on each sequence's contiguous K/V, kv heads repeated G times."""
    group = case.num_q_heads // case.num_kv_heads
    outs = []
    for s in range(case.num_seqs):
        k_log, v_log = W.logical_kv(case, s)
        k_t = torch.from_numpy(k_log.astype(np.float64)).permute(1, 0, 2)  # [Hkv, L, D]
        v_t = torch.from_numpy(v_log.astype(np.float64)).permute(1, 0, 2)
        k_t = k_t.repeat_interleave(group, dim=0).unsqueeze(0).contiguous()
        v_t = v_t.repeat_interleave(group, dim=0).unsqueeze(0).contiguous()
        q_t = torch.from_numpy(case.q[s].astype(np.float64)).unsqueeze(0).unsqueeze(2)
        o = torch.nn.functional.scaled_dot_product_attention(q_t, k_t, v_t, scale=case.scale)
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(dtype=np.float16, num_q_heads=8, num_kv_heads=2, head_dim=16, block_size=8,
         context_lens=[1, 7, 8, 9, 63, 64, 65]),
    dict(dtype=np.float16, num_q_heads=7, num_kv_heads=1, head_dim=32, block_size=32,
         context_lens=[100, 33]),
    dict(num_q_heads=3, num_kv_heads=3, head_dim=64, block_size=16, context_lens=[250, 1, 17]),
])
def test_p3_equals_dense_sdpa(kw):
    case = _case(**kw)
    kc, vc = oracle_pools(case)
    np.testing.assert_allclose(oracle_decode(case, kc, vc), _sdpa_dense(case), rtol=0, atol=1e-12)


def test_p3_shared_prefix_equals_dense_sdpa():
    case = W.shared_prefix(num_prompts=2, samples=3, prompt_len=48, max_tail=20)
    kc, vc = oracle_pools(case)
    np.testing.assert_allclose(oracle_decode(case, kc, vc), _sdpa_dense(case), rtol=0, atol=1e-12)


# --------------------------------------------------------------------- P4
def test_p4_physical_permutation_bit_identical():
    case = _case(dtype=np.float16, context_lens=[9, 31, 40], block_size=4)
    kc, vc = oracle_pools(case)
    ref = oracle_decode(case, kc, vc)
    perm = np.random.default_rng(5).permutation(case.num_blocks)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    out2 = O.decode(case.q, kc2, vc2, bt2, case.context_lens, case.scale, case.block_size,
                    case.num_kv_heads)
    assert np.array_equal(ref, out2)


# --------------------------------------------------------------------- P5
def test_p5_context_one_returns_v():
    case = _case(context_lens=[1, 1, 1], seed=3)
    kc, vc = oracle_pools(case)
    out = oracle_decode(case, kc, vc)
    group = case.num_q_heads // case.num_kv_heads
    for s in range(case.num_seqs):
        for h in range(case.num_q_heads):
            assert np.array_equal(out[s, h], case.new_v[s, h // group].astype(np.float64))


# --------------------------------------------------------------------- P6
def test_p6_duplicated_rows_identical():
    case = _case(context_lens=[23, 40])
    kc, vc = oracle_pools(case)
    q = np.concatenate([case.q, case.q[:1]], axis=0)
    bt = np.concatenate([case.block_tables, case.block_tables[:1]], axis=0)
    ctx = np.concatenate([case.context_lens, case.context_lens[:1]])
    out = O.decode(q, kc, vc, bt, ctx, case.scale, case.block_size, case.num_kv_heads)
    assert np.array_equal(out[0], out[-1])


def test_p6_shared_prompt_blocks_identical_for_identical_queries():
    case = W.shared_prefix(num_prompts=1, samples=4, prompt_len=32, max_tail=0)
    kc, vc = oracle_pools(case)
    # samples share the prompt; give them one query and one (prompt-only) context
    q = np.repeat(case.q[:1], case.num_seqs, axis=0)
    ctx = np.full(case.num_seqs, 32, dtype=np.int32)
    out = O.decode(q, kc, vc, case.block_tables, ctx, case.scale, case.block_size,
                   case.num_kv_heads)
    for s in range(1, case.num_seqs):
        assert np.array_equal(out[0], out[s])
    assert case.refcount[case.block_tables[0, 0]] == 4


# --------------------------------------------------------------------- P7 / P8
def test_p7_online_softmax_equals_two_pass():
    case = _case(context_lens=[1, 4, 5, 37, 40], seed=21)
    kc, vc = oracle_pools(case)
    for s in range(case.num_seqs):
        for h in range(case.num_q_heads):
            a = O.decode_one(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                             case.block_size, case.num_kv_heads, s, h)
            b = O.decode_one_online(case.q, kc, vc, case.block_tables, case.context_lens,
                                    case.scale, case.block_size, case.num_kv_heads, s, h)
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("psize", [1000, 4, 8, 12, 64])
def test_p8_partition_merge_equals_unsplit(psize):
    case = _case(context_lens=[1, 11, 40, 97], seed=23, block_size=4)
    kc, vc = oracle_pools(case)
    for s in range(case.num_seqs):
        for h in range(case.num_q_heads):
            a = O.decode_one(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                             case.block_size, case.num_kv_heads, s, h)
            b = O.decode_one_partitioned(case.q, kc, vc, case.block_tables, case.context_lens,
                                         case.scale, case.block_size, case.num_kv_heads, s, h,
                                         psize)
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# --------------------------------------------------------------------- P9
def test_p9_block_size_invariance_bit_identical():
    outs = []
    for B in (8, 16, 32):
        case = W.make_case(seed=500 + B, logical_seed=77, dtype=np.float16,
                           context_lens=[1, 31, 100, 257], num_q_heads=4, num_kv_heads=2,
                           head_dim=16, block_size=B, sigma=0.5)
        kc, vc = oracle_pools(case)
        outs.append(oracle_decode(case, kc, vc))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


# --------------------------------------------------------------------- P10
def test_p10_closed_forms():
    case = _case(context_lens=[7, 40], seed=31)
    kc, vc = oracle_pools(case)
    group = case.num_q_heads // case.num_kv_heads
    # all K rows of a head equal -> uniform weights -> mean of the V rows
    kc_eq = kc.copy()
    for s in range(case.num_seqs):
        for pos in range(int(case.context_lens[s])):
            blk, off = O.locate_kv(pos, case.block_tables[s], case.block_size)
            kc_eq[blk, :, off, :] = 0.25
    out = O.decode(case.q, kc_eq, vc, case.block_tables, case.context_lens, case.scale,
                   case.block_size, case.num_kv_heads)
    for s in range(case.num_seqs):
        _, v_log = W.logical_kv(case, s)
        for h in range(case.num_q_heads):
            np.testing.assert_allclose(out[s, h], v_log[:, h // group].astype(np.float64).mean(0),
                                       rtol=0, atol=1e-12)
    # all V rows equal to c -> c
    c = np.linspace(-1, 1, case.head_dim).astype(vc.dtype).astype(np.float64)
    vc_eq = vc.copy()
    vc_eq[...] = c
    out = O.decode(case.q, kc, vc_eq, case.block_tables, case.context_lens, case.scale,
                   case.block_size, case.num_kv_heads)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=0, atol=1e-12)


# --------------------------------------------------------------------- P11
def test_p11_padding_poison_does_not_leak():
    case = _case(context_lens=[5, 18, 39], block_size=8, extra_table_cols=3)
    kc, vc = oracle_pools(case)
    assert np.isnan(kc).any() and (case.block_tables == -1).any()
    out = oracle_decode(case, kc, vc)
    assert np.all(np.isfinite(out))
    out_zero = oracle_decode(case, np.nan_to_num(kc), np.nan_to_num(vc))
    assert np.array_equal(out, out_zero)


# --------------------------------------------------------------------- P12
def test_p12_write_is_a_slot_scatter_and_nothing_else():
    case = _case(dtype=np.float16, context_lens=[3, 9, 17])
    rng = np.random.default_rng(4)
    sentinel_k = rng.standard_normal(case.empty_pool().shape).astype(np.float16)
    sentinel_v = rng.standard_normal(case.empty_pool().shape).astype(np.float16)
    slots = case.new_slots.copy()
    slots[1] = -1  # a padding entry is skipped
    kc, vc = O.cache_write(case.new_k, case.new_v, slots, sentinel_k, sentinel_v, case.block_size)
    # independent formulation: view the pool as [N*B] slots of [Hkv, D]
    flat = lambda pool: pool.transpose(0, 2, 1, 3).reshape(-1, pool.shape[1], pool.shape[3])
    exp_k, exp_v = flat(sentinel_k).copy(), flat(sentinel_v).copy()
    for t, sl in enumerate(slots):
        if sl >= 0:
            exp_k[sl] = case.new_k[t]
            exp_v[sl] = case.new_v[t]
    assert flat(kc).tobytes() == exp_k.tobytes()
    assert flat(vc).tobytes() == exp_v.tobytes()


# --------------------------------------------------------------------- P14
def test_p14_byte_accounting_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "kv_bytes.json")))
    t = g["per_token_per_layer"]
    case = W.make_case(seed=1, dtype=np.float16, context_lens=[1], num_q_heads=8,
                       num_kv_heads=t["num_kv_heads"], head_dim=t["head_dim"], block_size=16)
    assert case.kv_bytes() == t["expected_bytes_per_token_per_layer"]
    assert case.kv_bytes() * t["num_layers"] == t["expected_kib_per_token_all_layers"] * 1024
    b = g["per_block_per_layer"]
    pool = np.zeros((1, b["num_kv_heads"], b["block_size"], b["head_dim"]), dtype=np.float16)
    assert pool.nbytes == b["expected_k_bytes"] and 2 * pool.nbytes == b["expected_kv_bytes"]
    e = g["block_table_entries"]
    assert -(-e["context_len"] // e["block_size"]) == e["expected_entries"]


# --------------------------------------------------------------------- planted mistakes
def _p3_passes(case):
    kc, vc = oracle_pools(case)
    out = oracle_decode(case, kc, vc)
    return np.all(np.isfinite(out)) and np.allclose(out, _sdpa_dense(case), rtol=0, atol=1e-9)


_real_gather = O.gather_head
_real_softmax = O.softmax


def _reversed_blocks(cache, row, ctx, B, kvh):
    nb = -(-ctx // B)
    return _real_gather(cache, list(row[:nb])[::-1] + list(row[nb:]), ctx, B, kvh)


def _no_tail_mask(cache, row, ctx, B, kvh):
    return _real_gather(cache, row, -(-ctx // B) * B, B, kvh)


def _drops_last_token(cache, row, ctx, B, kvh):
    out = _real_gather(cache, row, ctx, B, kvh)
    return out[:-1] if len(out) > 1 else out


def _wrong_head(cache, row, ctx, B, kvh):
    return _real_gather(cache, row, ctx, B, 0)


def _offset_transposed(cache, row, ctx, B, kvh):
    nb = -(-ctx // B)
    tiles = [np.asarray(cache[int(row[j]), kvh], dtype=np.float64)[::-1] for j in range(nb)]
    return np.concatenate(tiles, 0)[:ctx]


def _unnormalised(z):
    return np.exp(z - z.max())


def _sign_flip(z):
    return _real_softmax(-z)


@pytest.mark.parametrize("where,mutant", [
    ("gather_head", _reversed_blocks),
    ("gather_head", _no_tail_mask),
    ("gather_head", _drops_last_token),
    ("gather_head", _wrong_head),
    ("gather_head", _offset_transposed),
    ("softmax", _unnormalised),
    ("softmax", _sign_flip),
])
def test_planted_mistakes_are_caught(monkeypatch, where, mutant):
    case = _case(context_lens=[6, 17, 40], block_size=4, seed=41)
    assert _p3_passes(case)
    monkeypatch.setattr(O, where, mutant)
    assert not _p3_passes(case)


def test_planted_dropped_scale_is_caught():
    case = _case(context_lens=[17, 40], seed=43)
    kc, vc = oracle_pools(case)
    wrong = O.decode(case.q, kc, vc, case.block_tables, case.context_lens, 1.0,
                     case.block_size, case.num_kv_heads)
    assert not np.allclose(wrong, _sdpa_dense(case), atol=1e-6)
