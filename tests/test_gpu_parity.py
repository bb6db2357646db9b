"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Writes must match byte for byte; attention must be within |d| <= 2e-3 + 1e-2|ref|
and the normalised error bound, and fp16 results also within the bound that the fp16
rounding of probabilities and outputs implies.  Exact invariants (physical relabelling,
context 1, padding poison, block size, split launches, repeat runs) are checked bitwise
on the GPU.  With the default split, where a context is cut between waves depends on the
whole batch, so the same sequence at another batch position (duplicated rows, a changed
neighbour) is checked to within that rounding bound; with fixed partitions it is bitwise.
"""
import functools

import numpy as np
import pytest

import paged_kv_cache_167_amd as P
import workloads as W
from oracle import pa_oracle as O
from tests import _gpu as G
from tests._helpers import oracle_decode, oracle_pools

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------ small sweep
SMALL = [
    # dtype, D, B, Hq, Hkv
    (np.float32, 64, 16, 4, 4),
    (np.float16, 128, 16, 8, 2),
    (np.float16, 128, 8, 16, 2),
    (np.float16, 128, 32, 14, 2),
    (np.float16, 64, 8, 4, 2),
    (np.float32, 128, 32, 6, 2),
    (np.float16, 128, 16, 12, 1),
    (np.float32, 64, 8, 10, 2),
]
SMALL_CTX = [1, 2, 15, 16, 17, 100, 511, 512, 513, 1100, 2049]


@pytest.mark.parametrize("partition", [0, 64, 512])
@pytest.mark.parametrize("dtype,D,B,hq,hkv", SMALL)
def test_small_shapes(dtype, D, B, hq, hkv, partition):
    label = f"small {np.dtype(dtype).name} D{D} B{B} {hq}/{hkv} P{partition}"
    G.say(label)
    case = W.make_case(seed=D + B + hq, dtype=dtype, context_lens=SMALL_CTX, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=D, block_size=B, sigma=0.5,
                       extra_table_cols=2)
    part = partition if partition == 0 else max(partition, B)
    d = G.to_device(case)
    got = G.decode(case, d, partition_size=part)
    kc, vc = oracle_pools(case)
    assert d.k_cache.cpu().numpy().tobytes() == kc.tobytes(), f"{label}: K pool differs"
    assert d.v_cache.cpu().numpy().tobytes() == vc.tobytes(), f"{label}: V pool differs"
    ref = oracle_decode(case, kc, vc)
    G.assert_close(got, ref, dtype, label)
    _fp16_bound(got, ref, case, label)


def _fp16_bound(got, ref, case, label):
    """fp16: probabilities rounded to fp16 (relative 2^-11) before P.V and the output
    rounded to fp16 give |gpu - exact| <= 2^-11 (|out| + max|v|); twice that leaves room
    for the fp32 sums."""
    if np.dtype(case.dtype) != np.float16:
        return
    err = np.abs(np.asarray(got, np.float64) - ref)
    bound = 2.0 * 2.0 ** -11 * (np.abs(ref) + _vmax(case)) + 1e-6
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{label}: {err[worst]:.3e} > {bound[worst]:.3e} at {worst}"


# ------------------------------------------------------------------ the five workloads
@functools.lru_cache(maxsize=1)
def _config(name, variant):
    if name.startswith("long_context_b"):  # the block-size sweep: B = 8, 16, 32
        return W.long_context(int(name[len("long_context_b"):]), variant)
    return W.CONFIGS[name](variant)


CONFIG_RUNS = [
    ("tiny_fp32", "plain", 64), ("tiny_fp32", "needle", 64), ("tiny_fp32", "poscode", 0),
    ("llama3_8b", "plain", 0), ("llama3_8b", "needle", 256), ("llama3_8b", "poscode", 512),
    ("llama2_70b", "plain", 0), ("llama2_70b", "needle", 512),
    ("shared_prefix", "plain", 0), ("shared_prefix", "needle", 512),
    ("shared_prefix", "poscode", 0),
    ("long_context_b16", "plain", 0), ("long_context_b16", "needle", 512),
    ("long_context_b8", "plain", 0), ("long_context_b8", "needle", 512),
    ("long_context_b32", "plain", 0), ("long_context_b32", "needle", 512),
]


@pytest.mark.parametrize("name,variant,partition", CONFIG_RUNS)
def test_config_parity(name, variant, partition):
    label = f"{name}/{variant} P{partition}"
    G.say(f"{label}: generating")
    case = _config(name, variant)
    G.say(f"{label}: device pools via pa_cache_write")
    d = G.to_device(case)
    G.say(f"{label}: decode")
    got = G.decode(case, d, partition_size=partition)
    G.say(f"{label}: oracle")
    kc, vc = oracle_pools(case)
    assert d.k_cache.cpu().numpy().tobytes() == kc.tobytes(), f"{label}: K pool differs"
    assert d.v_cache.cpu().numpy().tobytes() == vc.tobytes(), f"{label}: V pool differs"
    del d
    _torch().cuda.empty_cache()
    ref = oracle_decode(case, kc, vc)
    err, norm = G.assert_close(got, ref, case.dtype, label)
    _fp16_bound(got, ref, case, label)
    G.say(f"{label}: max err {err:.2e}, normalised {norm:.2e}")
    if variant == "needle":  # the planted key dominates: output is close to one V row
        assert np.abs(ref).max() > 0.2


def test_new_token_write_only_touches_its_slots():
    case = _config("shared_prefix", "plain")
    d = G.to_device(case, write_new=False)
    before_k = d.k_cache.cpu().numpy()
    before_v = d.v_cache.cpu().numpy()
    P.pa_cache_write(d.new_k, d.new_v, d.new_slots, d.k_cache, d.v_cache)
    _torch().cuda.synchronize()
    exp_k, exp_v = O.cache_write(case.new_k, case.new_v, case.new_slots, before_k, before_v,
                                 case.block_size)
    assert d.k_cache.cpu().numpy().tobytes() == exp_k.tobytes()
    assert d.v_cache.cpu().numpy().tobytes() == exp_v.tobytes()


def test_cache_write_skips_padding_slots():
    torch = _torch()
    case = W.make_case(seed=3, dtype=np.float16, context_lens=[5, 9, 40], num_q_heads=4,
                       num_kv_heads=2, head_dim=128, block_size=8)
    d = G.to_device(case, write_new=False)
    slots = case.new_slots.copy()
    slots[1] = -1
    before_k = d.k_cache.cpu().numpy()
    before_v = d.v_cache.cpu().numpy()
    P.pa_cache_write(d.new_k, d.new_v, torch.from_numpy(slots).cuda(), d.k_cache, d.v_cache)
    torch.cuda.synchronize()
    exp_k, exp_v = O.cache_write(case.new_k, case.new_v, slots, before_k, before_v,
                                 case.block_size)
    assert d.k_cache.cpu().numpy().tobytes() == exp_k.tobytes()
    assert d.v_cache.cpu().numpy().tobytes() == exp_v.tobytes()


# ------------------------------------------------------------------ exact invariants on the GPU
def _mid_case(dtype=np.float16, B=16):
    return W.make_case(seed=77, logical_seed=78, dtype=dtype,
                       context_lens=[1, 16, 17, 300, 1025, 3001], num_q_heads=32,
                       num_kv_heads=8, head_dim=128, block_size=B, sigma=0.5)


@pytest.mark.parametrize("partition", [0, 512])
def test_physical_permutation_bit_identical(partition):
    torch = _torch()
    case = _mid_case()
    d = G.to_device(case)
    ref = G.decode(case, d, partition_size=partition)
    perm = np.random.default_rng(5).permutation(case.num_blocks)
    permt = torch.from_numpy(perm).cuda()
    kc2 = torch.empty_like(d.k_cache)
    vc2 = torch.empty_like(d.v_cache)
    kc2[permt] = d.k_cache
    vc2[permt] = d.v_cache
    bt2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], -1)
    bt2 = bt2.astype(np.int32)
    got = G.decode(case, d, partition_size=partition, tables=torch.from_numpy(bt2).cuda(),
                   k_cache=kc2, v_cache=vc2)
    assert got.tobytes() == ref.tobytes()


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_context_one_returns_v_exactly(dtype):
    case = W.make_case(seed=9, dtype=dtype, context_lens=[1, 1, 1, 1], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, sigma=0.5)
    d = G.to_device(case)
    got = G.decode(case, d, partition_size=512)
    for s in range(case.num_seqs):
        for h in range(case.num_q_heads):
            assert got[s, h].tobytes() == case.new_v[s, h // 4].tobytes()


def _vmax(case):
    return float(max(np.abs(case.prefix_v).max(initial=0.0), np.abs(case.new_v).max(initial=0.0)))


def _within_rounding(a, b, dtype, label, vmax):
    """Two results of the same rows computed with different split points.

    fp16: the kernel rounds each probability to fp16 (relative 2^-11) before P.V and the
    output to fp16, so each result lies within 2^-11 (|o| + max|v|) of the exact row (the
    fp32 sums add far less); two results lie within the sum of their bounds.
    fp32: probabilities stay fp32, so the results agree to a few fp32 roundings."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), label
    if np.dtype(dtype) == np.float16:
        tol = 2.0 ** -11 * (np.abs(a) + np.abs(b) + 2.0 * vmax) + 2.0 ** -24
    else:
        tol = 1e-5 * np.abs(b) + 1e-7
    diff = np.abs(a - b)
    worst = np.unravel_index(np.argmax(diff - tol), diff.shape)
    assert np.all(diff <= tol), f"{label}: {a[worst]} vs {b[worst]} at {worst}"


def test_duplicated_rows_within_rounding():
    torch = _torch()
    case = _mid_case()
    d = G.to_device(case)
    idx = torch.tensor([5, 0, 5, 3, 5], device="cuda")
    q = d.q[idx].contiguous()
    bt = d.tables[idx].contiguous()
    ctx = d.ctx[idx].contiguous()
    got = G.decode(case, d, q=q, tables=bt, ctx=ctx)
    vm = _vmax(case)
    _within_rounding(got[0], got[2], case.dtype, "copy 2", vm)
    _within_rounding(got[0], got[4], case.dtype, "copy 4", vm)
    full = G.decode(case, d)
    _within_rounding(got[0], full[5], case.dtype, "seq 5", vm)
    _within_rounding(got[1], full[0], case.dtype, "seq 0", vm)


@pytest.mark.parametrize("dtype,partition", [(np.float16, 512), (np.float16, 64),
                                             (np.float32, 512), (np.float16, 16)])
def test_fixed_partitions_are_independent_of_the_batch(dtype, partition):
    """With partition_size > 0 a context is cut at fixed multiples of the partition size
    and each partition is one piece: a row does not depend on its batch position or on the
    rest of the batch, so duplicated, reordered and lone sequences agree bitwise."""
    torch = _torch()
    case = _mid_case(dtype=dtype)
    d = G.to_device(case)
    full = G.decode(case, d, partition_size=partition)

    def sub(rows):
        idx = torch.tensor(rows, device="cuda")
        return G.decode(case, d, partition_size=partition, q=d.q[idx].contiguous(),
                        tables=d.tables[idx].contiguous(), ctx=d.ctx[idx].contiguous())

    got = sub([5, 0, 5, 3, 5, 4])
    for j, s in enumerate([5, 0, 5, 3, 5, 4]):
        assert got[j].tobytes() == full[s].tobytes(), f"P{partition}: batch row {j} (seq {s})"
    for s in (5, 4, 0):
        assert sub([s])[0].tobytes() == full[s].tobytes(), f"P{partition}: seq {s} alone"
    rev = sub(list(range(case.num_seqs))[::-1])
    assert rev[::-1].tobytes() == full.tobytes(), f"P{partition}: reversed batch"
    kc, vc = oracle_pools(case)
    G.assert_close(full, oracle_decode(case, kc, vc), dtype, f"P{partition}")


def test_shared_prompt_blocks_agree_for_identical_queries():
    torch = _torch()
    case = _config("shared_prefix", "plain")
    d = G.to_device(case)
    # the 8 samples of prompt 0 with one query and the prompt-only context
    q = d.q[:8].clone()
    q[:] = d.q[0]
    ctx = torch.full((8,), 2000, dtype=torch.int32, device="cuda")
    got = G.decode(case, d, q=q.contiguous(), tables=d.tables[:8].contiguous(), ctx=ctx)
    for s in range(1, 8):
        _within_rounding(got[s], got[0], case.dtype, f"sample {s}", _vmax(case))
    # with fixed partitions the samples are bitwise equal
    got = G.decode(case, d, q=q.contiguous(), tables=d.tables[:8].contiguous(), ctx=ctx,
                   partition_size=512)
    for s in range(1, 8):
        assert got[s].tobytes() == got[0].tobytes(), f"sample {s}, partition 512"


def test_padding_poison_has_no_effect():
    torch = _torch()
    case = _mid_case()
    d = G.to_device(case)
    got_nan = G.decode(case, d)
    kz = torch.nan_to_num(d.k_cache)
    vz = torch.nan_to_num(d.v_cache)
    assert torch.isnan(d.k_cache).any()
    got_zero = G.decode(case, d, k_cache=kz, v_cache=vz)
    assert np.all(np.isfinite(got_nan))
    assert got_nan.tobytes() == got_zero.tobytes()


def test_block_size_invariance_bit_identical():
    outs = []
    for B in (8, 16, 32):
        case = _mid_case(B=B)
        d = G.to_device(case)
        outs.append(G.decode(case, d))
    assert outs[0].tobytes() == outs[1].tobytes() == outs[2].tobytes()


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_partition_size_invariance(dtype):
    case = _mid_case(dtype=dtype)
    d = G.to_device(case)
    base = G.decode(case, d, partition_size=0)
    for part in (16, 64, 256, 512, 1024):
        got = G.decode(case, d, partition_size=part)
        _within_rounding(got, base, dtype, f"partition {part}", _vmax(case))


def test_split_launches_equal_single_call():
    case = _mid_case()
    d = G.to_device(case)
    one = G.decode(case, d, partition_size=256)
    two = G.decode(case, d, partition_size=256, split=True)
    assert one.tobytes() == two.tobytes()


def test_repeatable_bitwise():
    case = _mid_case()
    d = G.to_device(case)
    a = G.decode(case, d)
    b = G.decode(case, d)
    assert a.tobytes() == b.tobytes()


def test_context_zero_gives_zero_rows():
    torch = _torch()
    case = _mid_case()
    d = G.to_device(case)
    ctx = d.ctx.clone()
    ctx[2] = 0
    got = G.decode(case, d, ctx=ctx)
    assert np.all(got[2] == 0)
    full = G.decode(case, d)
    keep = [0, 1, 3, 4, 5]
    _within_rounding(got[keep], full[keep], case.dtype, "other rows", _vmax(case))


def test_no_sequences_is_a_no_op():
    torch = _torch()
    q = torch.empty((0, 8, 128), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.float16, device="cuda")
    bt = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    ctx = torch.zeros((0,), dtype=torch.int32, device="cuda")
    P.pa_decode(out, q, kc, kc, bt, ctx, 0.1, 16, 2, max_context_len=64)
    torch.cuda.synchronize()


def test_long_context_block_sizes_agree():
    """Same logical K/V laid out with block sizes 8, 16 and 32: bitwise equal outputs."""
    outs = {}
    for B in (16, 8, 32):
        G.say(f"long_context B{B}: generating")
        case = W.long_context(B, "plain", num_seqs=3)
        d = G.to_device(case)
        G.say(f"long_context B{B}: decode")
        outs[B] = G.decode(case, d, partition_size=512)
        del d
        _torch().cuda.empty_cache()
    assert outs[8].tobytes() == outs[16].tobytes() == outs[32].tobytes()
    # and the first sequence against the oracle (sampled heads)
    case = W.long_context(16, "plain", num_seqs=3)
    kc, vc = oracle_pools(case)
    for h in (0, 13, 55):
        ref = O.decode_one(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                           case.block_size, case.num_kv_heads, 0, h)
        G.assert_close(outs[16][0, h], ref, case.dtype, f"long_context seq0 head {h}")


# ------------------------------------------------------------------ extreme sizes
def test_many_short_sequences():
    """2000 sequences of 1..80 tokens (past the 256-sequence register index), some of them
    emptied on the device: every row against the oracle, empty rows exactly zero."""
    torch = _torch()
    rng = np.random.default_rng(2000)
    ctx = rng.integers(1, 80, size=2000, endpoint=True)
    case = W.make_case(seed=2001, dtype=np.float16, context_lens=ctx, num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, sigma=0.5)
    d = G.to_device(case)
    zero = np.array([0, 7, 1999, 1024])
    ctx_dev = d.ctx.clone()
    ctx_dev[torch.from_numpy(zero).cuda()] = 0
    G.say("2000 sequences: decode")
    got = G.decode(case, d, ctx=ctx_dev)
    assert np.all(got[zero] == 0)
    kc, vc = oracle_pools(case)
    ref = oracle_decode(case, kc, vc)
    keep = np.setdiff1d(np.arange(case.num_seqs), zero)
    G.assert_close(got[keep], ref[keep], case.dtype, "2000 sequences")
    _fp16_bound(got[keep], ref[keep], case, "2000 sequences")


def test_one_context_split_over_every_wave():
    """One 200K-token context (GQA 8): the default split cuts it into about a thousand
    pieces that the reduce merges; against the oracle."""
    case = W.make_case(seed=2002, dtype=np.float16, context_lens=[200_000], num_q_heads=8,
                       num_kv_heads=1, head_dim=128, block_size=16, sigma=0.5)
    d = G.to_device(case)
    G.say("200K context: decode")
    got = G.decode(case, d)
    kc, vc = oracle_pools(case)
    ref = oracle_decode(case, kc, vc)
    G.assert_close(got, ref, case.dtype, "200K context")
    _fp16_bound(got, ref, case, "200K context")


def test_many_small_partitions():
    """32-token partitions cut the 3001-token context into 94 pieces, merged by the second
    launch: results agree with the oracle and, within rounding, with the default split."""
    case = _mid_case()
    d = G.to_device(case)
    got = G.decode(case, d, partition_size=32)
    kc, vc = oracle_pools(case)
    ref = oracle_decode(case, kc, vc)
    G.assert_close(got, ref, case.dtype, "partition 32")
    _within_rounding(got, G.decode(case, d), case.dtype, "partition 32 vs default", _vmax(case))
