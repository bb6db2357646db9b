"""GPU checks of pa_decode_append (store each sequence's new token at position ctx - 1 and
attend over the whole context, in one call) through the C ABI.

The call must give exactly what pa_cache_write (at the slot the table gives that position)
followed by pa_decode gives: the same output bit for bit and the same pools byte for byte.
The outputs are also held to the oracle (cache write, then decode) within the decode
tolerance, and the slots the workloads use for the new token are checked against the
table arithmetic first.
"""
import numpy as np
import pytest

import paged_kv_cache_167_amd as P
import workloads as W
from tests import _gpu as G
from tests._helpers import oracle_decode, oracle_pools

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _table_slots(case):
    """Slot of position ctx - 1 of every sequence from its block table (the append of a
    token into the sequence's last block)."""
    B = case.block_size
    p = case.context_lens.astype(np.int64) - 1
    return case.block_tables[np.arange(case.num_seqs), p // B].astype(np.int64) * B + p % B


def _same_bits(a, b):
    """Pools compared bit for bit (unwritten slots hold NaN, which == would reject)."""
    torch = _torch()
    return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))


def _two_calls(case, d, partition):
    """Reference on the device: pa_cache_write of the new tokens, then pa_decode."""
    torch = _torch()
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    P.pa_cache_write(d.new_k, d.new_v, d.new_slots, kc, vc)
    out = torch.empty_like(d.q)
    P.pa_decode(out, d.q, kc, vc, d.tables, d.ctx, case.scale, case.block_size, case.num_kv_heads,
                max_context_len=case.max_context_len, partition_size=partition)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kc, vc


def _append(case, d, partition, ctx=None, tables=None):
    """pa_decode_append on copies of the prefix-only pools; returns (out, k pool, v pool)."""
    torch = _torch()
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    out = torch.empty_like(d.q)
    P.pa_decode_append(out, d.q, d.new_k, d.new_v, kc, vc, d.tables if tables is None else tables,
                       d.ctx if ctx is None else ctx, case.scale, case.block_size, case.num_kv_heads,
                       max_context_len=case.max_context_len, partition_size=partition)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kc, vc


SHAPES = [
    # D, B, Hq, Hkv: group sizes 1-32 (32 query heads per kv head take two 16-row units)
    (128, 16, 32, 8),
    (128, 8, 16, 2),
    (128, 32, 14, 2),
    (64, 16, 8, 8),
    (64, 8, 12, 2),
    (128, 16, 64, 2),
]
CTX = [1, 2, 15, 16, 17, 31, 32, 33, 100, 511, 512, 513, 2049]


@pytest.mark.parametrize("partition", [0, 64])
@pytest.mark.parametrize("D,B,hq,hkv", SHAPES)
def test_equals_write_then_decode_and_the_oracle(D, B, hq, hkv, partition):
    label = f"append D{D} B{B} {hq}/{hkv} P{partition}"
    G.say(label)
    case = W.make_case(seed=D + B + hq + partition, dtype=np.float16, context_lens=CTX,
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=D, block_size=B, sigma=0.5)
    assert np.array_equal(_table_slots(case), case.new_slots)
    d = G.to_device(case, write_new=False)
    got, kc, vc = _append(case, d, partition)
    ref, rkc, rvc = _two_calls(case, d, partition)
    assert got.tobytes() == ref.tobytes(), f"{label}: output differs from write + decode"
    assert kc.cpu().numpy().tobytes() == rkc.cpu().numpy().tobytes(), f"{label}: K pool differs"
    assert vc.cpu().numpy().tobytes() == rvc.cpu().numpy().tobytes(), f"{label}: V pool differs"
    okc, ovc = oracle_pools(case)
    assert kc.cpu().numpy().tobytes() == okc.tobytes(), f"{label}: K pool differs from the oracle's"
    G.assert_close(got, oracle_decode(case, okc, ovc), np.float16, label)


@pytest.mark.parametrize("name", ["llama3_8b", "llama2_70b"])
def test_workloads_equal_write_then_decode(name):
    G.say(f"append {name}: generating")
    case = W.CONFIGS[name]("plain")
    assert np.array_equal(_table_slots(case), case.new_slots)
    d = G.to_device(case, write_new=False)
    G.say(f"append {name}: device")
    got, kc, vc = _append(case, d, 0)
    ref, rkc, rvc = _two_calls(case, d, 0)
    assert got.tobytes() == ref.tobytes()
    assert _same_bits(kc, rkc) and _same_bits(vc, rvc)


def test_split_launches_equal_the_single_call():
    """pa_decode_append_partitions + pa_decode_reduce attend exactly as pa_decode_append does,
    and store nothing."""
    torch = _torch()
    case = W.make_case(seed=91, dtype=np.float16, context_lens=CTX, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, block_size=16, sigma=0.5)
    d = G.to_device(case, write_new=False)
    one, _, _ = _append(case, d, 64)
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    out = torch.empty_like(d.q)
    ws = P.pa_decode_append_partitions(out, d.q, d.new_k, d.new_v, kc, vc, d.tables, d.ctx, case.scale,
                                       case.block_size, case.num_kv_heads,
                                       max_context_len=case.max_context_len, partition_size=64)
    P.pa_decode_reduce(out, d.ctx, case.num_kv_heads, case.max_context_len, 64, ws)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tobytes() == one.tobytes()
    assert _same_bits(kc, d.k_cache) and _same_bits(vc, d.v_cache)


def test_empty_invalid_and_out_of_pool_sequences_store_nothing():
    """Context 0: zero rows; a context beyond max_context_len, or a last-position table
    entry outside the pool: NaN rows.  None of them stores its token; the others do."""
    torch = _torch()
    case = W.make_case(seed=92, dtype=np.float16, context_lens=[40, 70, 33, 90, 17], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, sigma=0.5)
    d = G.to_device(case, write_new=False)
    ctx = d.ctx.clone()
    ctx[1] = 0
    ctx[2] = case.max_context_len + 5
    tables = d.tables.clone()
    tables[3, (int(case.context_lens[3]) - 1) // 16] = case.num_blocks + 3
    got, kc, vc = _append(case, d, 0, ctx=ctx, tables=tables)
    assert np.all(got[1] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    written = np.zeros(case.num_seqs, bool)
    written[[0, 4]] = True
    # the expected pools: the prefix-only pools plus the new tokens of sequences 0 and 4
    ek, ev = d.k_cache.clone(), d.v_cache.clone()
    keep = torch.from_numpy(np.flatnonzero(written)).cuda()
    P.pa_cache_write(d.new_k[keep].contiguous(), d.new_v[keep].contiguous(), d.new_slots[keep].contiguous(),
                     ek, ev)
    torch.cuda.synchronize()
    assert _same_bits(kc, ek) and _same_bits(vc, ev)
    ref, _, _ = _two_calls(case, d, 0)
    assert got[[0, 4]].tobytes() == ref[[0, 4]].tobytes()


# ------------------------------------------------------------------ E4M3 pools
def _f8():
    from tests import test_gpu_fp8 as F
    return F


def _f8_device(case, ks, vs):
    """Pools of codes holding every token but the new ones; the new rows as fp16."""
    torch = _torch()
    F = _f8()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    d = type("D", (), {})()
    d.q, d.tables, d.ctx = t(case.q), t(case.block_tables), t(case.context_lens)
    d.k_cache, d.v_cache = t(F._empty_codes(case)), t(F._empty_codes(case))
    P.pa_cache_write_fp8(t(case.prefix_k), t(case.prefix_v), t(case.prefix_slots), d.k_cache, d.v_cache,
                         ks, vs)
    d.new_k, d.new_v, d.new_slots = t(case.new_k), t(case.new_v), t(case.new_slots)
    torch.cuda.synchronize()
    return d


def _f8_two_calls(case, d, ks, vs, partition):
    torch = _torch()
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    P.pa_cache_write_fp8(d.new_k, d.new_v, d.new_slots, kc, vc, ks, vs)
    out = torch.empty_like(d.q)
    P.pa_decode_fp8(out, d.q, kc, vc, d.tables, d.ctx, case.scale, ks, vs, case.block_size,
                    case.num_kv_heads, max_context_len=case.max_context_len, partition_size=partition)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kc, vc


def _f8_append(case, d, ks, vs, partition, ctx=None, tables=None):
    torch = _torch()
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    out = torch.empty_like(d.q)
    P.pa_decode_fp8_append(out, d.q, d.new_k, d.new_v, kc, vc, d.tables if tables is None else tables,
                           d.ctx if ctx is None else ctx, case.scale, ks, vs, case.block_size,
                           case.num_kv_heads, max_context_len=case.max_context_len,
                           partition_size=partition)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kc, vc


F8_SHAPES = [(128, 16, 32, 8), (128, 8, 16, 2), (128, 32, 14, 2), (64, 16, 8, 8), (64, 8, 12, 2),
             (128, 16, 64, 2)]


@pytest.mark.parametrize("partition", [0, 64])
@pytest.mark.parametrize("D,B,hq,hkv", F8_SHAPES)
def test_fp8_equals_write_then_decode_and_the_oracle(D, B, hq, hkv, partition):
    F = _f8()
    label = f"fp8 append D{D} B{B} {hq}/{hkv} P{partition}"
    G.say(label)
    case = W.make_case(seed=3 * D + B + hq + partition, dtype=np.float16, context_lens=CTX,
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=D, block_size=B, sigma=0.5)
    assert np.array_equal(_table_slots(case), case.new_slots)
    ks, vs = F._scales(case)
    d = _f8_device(case, ks, vs)
    got, kc, vc = _f8_append(case, d, ks, vs, partition)
    ref, rkc, rvc = _f8_two_calls(case, d, ks, vs, partition)
    assert got.tobytes() == ref.tobytes(), f"{label}: output differs from write + decode"
    assert bool(torch_equal(kc, rkc)) and bool(torch_equal(vc, rvc)), f"{label}: pools differ"
    okc, ovc = F._oracle_pools(case, ks, vs)
    assert kc.cpu().numpy().tobytes() == okc.tobytes(), f"{label}: K codes differ from the oracle's"
    assert vc.cpu().numpy().tobytes() == ovc.tobytes(), f"{label}: V codes differ from the oracle's"
    F._check(got, F._oracle_decode(case, okc, ovc, ks, vs), ovc, vs, label)


def torch_equal(a, b):
    return _torch().equal(a, b)  # uint8 codes: NaN codes compare as bytes


@pytest.mark.parametrize("name", ["llama3_8b", "llama2_70b"])
def test_fp8_workloads_equal_write_then_decode(name):
    F = _f8()
    G.say(f"fp8 append {name}")
    case = W.CONFIGS[name]("plain")
    ks, vs = F._scales(case)
    d = _f8_device(case, ks, vs)
    got, kc, vc = _f8_append(case, d, ks, vs, 0)
    ref, rkc, rvc = _f8_two_calls(case, d, ks, vs, 0)
    assert got.tobytes() == ref.tobytes()
    assert torch_equal(kc, rkc) and torch_equal(vc, rvc)


def test_fp8_split_launches_and_nothing_stored_for_bad_sequences():
    torch = _torch()
    F = _f8()
    case = W.make_case(seed=93, dtype=np.float16, context_lens=[40, 70, 33, 90, 17, 1, 16], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, sigma=0.5)
    ks, vs = F._scales(case)
    d = _f8_device(case, ks, vs)
    one, _, _ = _f8_append(case, d, ks, vs, 64)
    kc, vc = d.k_cache.clone(), d.v_cache.clone()
    out = torch.empty_like(d.q)
    ws = P.pa_decode_fp8_append_partitions(out, d.q, d.new_k, d.new_v, kc, vc, d.tables, d.ctx, case.scale,
                                           ks, vs, case.block_size, case.num_kv_heads,
                                           max_context_len=case.max_context_len, partition_size=64)
    P.pa_decode_reduce(out, d.ctx, case.num_kv_heads, case.max_context_len, 64, ws)
    torch.cuda.synchronize()
    assert out.cpu().numpy().tobytes() == one.tobytes()
    assert torch_equal(kc, d.k_cache) and torch_equal(vc, d.v_cache)  # the first launch stores nothing
    ctx = d.ctx.clone()
    ctx[1] = 0
    ctx[2] = case.max_context_len + 5
    tables = d.tables.clone()
    tables[3, (int(case.context_lens[3]) - 1) // 16] = case.num_blocks + 3
    got, kc, vc = _f8_append(case, d, ks, vs, 0, ctx=ctx, tables=tables)
    assert np.all(got[1] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    keep = torch.tensor([0, 4, 5, 6], device="cuda")
    ek, ev = d.k_cache.clone(), d.v_cache.clone()
    P.pa_cache_write_fp8(d.new_k[keep].contiguous(), d.new_v[keep].contiguous(), d.new_slots[keep].contiguous(),
                         ek, ev, ks, vs)
    torch.cuda.synchronize()
    assert torch_equal(kc, ek) and torch_equal(vc, ev)
    ref, _, _ = _f8_two_calls(case, d, ks, vs, 0)
    assert got[[0, 4, 5, 6]].tobytes() == ref[[0, 4, 5, 6]].tobytes()


@pytest.mark.parametrize("D,B", [(128, 16), (64, 8)])
def test_fp8_append_rounds_near_midpoint_quotients_exactly(D, B):
    """New rows made of fp16 values whose quotient by the scale lies within an fp32 step of a
    midpoint between two codes: the reduce kernel's store and the operands the attention kernel
    substitutes for the new token must both take the code nearest to the exact quotient."""
    F = _f8()
    ks, vs = F._near_midpoint_scales(3)[1:3]
    case = W.make_case(seed=5 + D, dtype=np.float16, context_lens=[1, 17, 40, 100], num_q_heads=8,
                       num_kv_heads=2, head_dim=D, block_size=B, sigma=0.5)
    rng = np.random.default_rng(D)
    for arr, sc in ((case.new_k, ks), (case.new_v, vs)):
        hard = F._ALL_F16[(F._reciprocal_reading(sc) != F._codes(F._ALL_F16, sc)) & np.isfinite(F._ALL_F16)]
        assert hard.size > 0
        arr[...] = rng.choice(hard, size=arr.shape)
    G.say(f"fp8 append near-midpoint D{D} B{B} scales {ks!r} {vs!r}")
    d = _f8_device(case, ks, vs)
    got, kc, vc = _f8_append(case, d, ks, vs, 0)
    ref, rkc, rvc = _f8_two_calls(case, d, ks, vs, 0)
    assert got.tobytes() == ref.tobytes(), "output differs from write + decode"
    assert torch_equal(kc, rkc) and torch_equal(vc, rvc), "pools differ from write + decode"
    okc, ovc = F._oracle_pools(case, ks, vs)
    assert kc.cpu().numpy().tobytes() == okc.tobytes(), "K codes differ from the oracle's"
    assert vc.cpu().numpy().tobytes() == ovc.tobytes(), "V codes differ from the oracle's"
    F._check(got, F._oracle_decode(case, okc, ovc, ks, vs), ovc, vs, "near-midpoint append")
