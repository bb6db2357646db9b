"""GPU parity of a bf16 path (q, pools and out in bfloat16) through the C ABI against the
fp64 CPU oracle.  The path is not in the library (see the skip reason below); the tests
are kept for the record and for when it returns.

The inputs are the workloads' fp32 values rounded once to bf16 (to nearest, ties to even),
so the oracle computes with exactly the values the GPU reads.  Writes must match byte for
byte.  Attention: the kernel rounds each probability to bf16 for the P.V product and the
output to bf16, so every element lies within 2^-8 (|exact| + max|v|) of exact attention
(bf16 keeps 8 significant bits, where fp16's 11 give the 2^-11 of the fp16 bound); the
fp32 sums and exponentials add far less.  The fp16 gate (2e-3 + 1e-2 |ref|) is below what
bf16 storage itself can hold, so this bound is the gate here.  Exact invariants (physical
relabelling, block size, split launches, partition independence, the allocation-free
entry) are checked bitwise.
"""
import numpy as np
import pytest

import paged_kv_cache_167_amd as P
import workloads as W
from tests import _gpu as G
from tests._helpers import oracle_decode, oracle_pools

# The first run of this file on MI355X went silent inside test_bf16_small_shapes (D128, B16,
# 32/8 heads, default split) and was killed after 180 s.  The bf16 stream and reduce kernels
# compiled to the fp16 ones' code apart from the product and conversion instructions, and no
# cause was found; the bf16 decode path was taken out of the library and these tests stay
# skipped until one is.
pytestmark = [pytest.mark.gpu,
              pytest.mark.skip(reason="bf16 decode is not built: its first GPU run went silent for "
                                      "180 s in test_bf16_small_shapes and no cause was found")]

SMALL_CTX = [1, 2, 15, 16, 17, 100, 511, 512, 513, 1100, 2049]


def _torch():
    import torch
    return torch


def _bf16_values(x):
    """fp32 array -> the nearest bf16 values (ties to even), still as fp32 (exact)."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _bf16_case(case):
    """The case with every value input rounded to bf16 (the oracle then sees the GPU's inputs)."""
    for name in ("q", "prefix_k", "prefix_v", "new_k", "new_v"):
        setattr(case, name, _bf16_values(getattr(case, name)))
    return case


def _make(seed, context_lens, hq, hkv, D, B, **kw):
    case = W.make_case(seed=seed, dtype=np.float32, context_lens=context_lens, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=D, block_size=B, sigma=0.5, **kw)
    return _bf16_case(case)


def _to_device(case):
    """Upload as bf16 (exact) and write every token through pa_cache_write with PA_BF16."""
    from types import SimpleNamespace
    torch = _torch()
    G.check_case_host(case)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    b = lambda a: t(a).to(torch.bfloat16)  # noqa: E731
    d = SimpleNamespace()
    d.q = b(case.q)
    d.tables = t(case.block_tables)
    d.ctx = t(case.context_lens)
    shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    d.k_cache = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    d.v_cache = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    P.pa_cache_write(b(case.prefix_k), b(case.prefix_v), t(case.prefix_slots), d.k_cache, d.v_cache)
    P.pa_cache_write(b(case.new_k), b(case.new_v), t(case.new_slots), d.k_cache, d.v_cache)
    torch.cuda.synchronize()
    return d


def _bits(x):
    """bf16 bit patterns of a bf16 device tensor or of an fp32 array of bf16 values."""
    torch = _torch()
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return x.contiguous().view(torch.int16).cpu().numpy()


def _decode(case, d, partition_size=0, q=None, tables=None, ctx=None, split=False, noalloc=False):
    torch = _torch()
    q = d.q if q is None else q
    out = torch.empty_like(q)
    args = (out, q, d.k_cache, d.v_cache, d.tables if tables is None else tables,
            d.ctx if ctx is None else ctx, case.scale, case.block_size, case.num_kv_heads)
    mcl = case.max_context_len
    if noalloc:
        P.pa_decode_noalloc(*args, max_context_len=mcl, partition_size=partition_size)
    elif split:
        ws = P.pa_decode_partitions(*args, max_context_len=mcl, partition_size=partition_size)
        P.pa_decode_reduce(out, d.ctx if ctx is None else ctx, case.num_kv_heads, mcl, partition_size, ws)
    else:
        P.pa_decode(*args, max_context_len=mcl, partition_size=partition_size)
    torch.cuda.synchronize()
    return out


def _vmax(case):
    return float(max(np.abs(case.prefix_v).max(initial=0.0), np.abs(case.new_v).max(initial=0.0)))


def _assert_bf16_close(out, ref, vmax, label):
    got = out.float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = np.abs(got - ref)
    bound = 1.05 * 2.0 ** -8 * (np.abs(ref) + vmax) + 1e-6
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{label}: {got[worst]} vs {ref[worst]} at {worst}"
    norm = err.max() / max(ref.std(), 1e-30)
    assert norm <= 2e-2, f"{label}: normalised error {norm:.3e}"


SMALL = [(128, 16, 32, 8), (64, 8, 8, 8), (128, 32, 16, 2), (64, 16, 14, 2), (128, 16, 8, 8)]


@pytest.mark.parametrize("partition", [0, 64])
@pytest.mark.parametrize("D,B,hq,hkv", SMALL)
def test_bf16_small_shapes(D, B, hq, hkv, partition):
    label = f"bf16 D{D} B{B} {hq}/{hkv} P{partition}"
    G.say(label)
    case = _make(D + B + hq, SMALL_CTX, hq, hkv, D, B, extra_table_cols=2)
    d = _to_device(case)
    kc, vc = oracle_pools(case)
    assert _bits(d.k_cache).tobytes() == _bits(kc).tobytes(), f"{label}: K pool differs"
    assert _bits(d.v_cache).tobytes() == _bits(vc).tobytes(), f"{label}: V pool differs"
    out = _decode(case, d, partition_size=partition)
    _assert_bf16_close(out, oracle_decode(case, kc, vc), _vmax(case), label)


def test_bf16_llama3_8b_full_size():
    """The Llama-3-8B-shaped batch (64 sequences, 512-4096 tokens, 32/8 heads) at full size in
    bf16: every output element against the oracle, the pools byte for byte."""
    G.say("bf16 llama3_8b: generating")
    rng = np.random.default_rng(1002)
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    case = _make(1002, ctx, 32, 8, 128, 16, pool_factor=1.2)
    G.say("bf16 llama3_8b: device")
    d = _to_device(case)
    out = _decode(case, d)
    G.say("bf16 llama3_8b: oracle")
    kc, vc = oracle_pools(case)
    assert _bits(d.k_cache).tobytes() == _bits(kc).tobytes()
    assert _bits(d.v_cache).tobytes() == _bits(vc).tobytes()
    _assert_bf16_close(out, oracle_decode(case, kc, vc), _vmax(case), "bf16 llama3_8b")


def test_bf16_needle_and_position_code():
    for variant in ("needle", "poscode"):
        case = _make(31, [700, 1537, 2049], 32, 8, 128, 16, variant=variant)
        d = _to_device(case)
        kc, vc = oracle_pools(case)
        _assert_bf16_close(_decode(case, d), oracle_decode(case, kc, vc), _vmax(case), f"bf16 {variant}")


def test_bf16_context_one_returns_v_exactly():
    case = _make(9, [1, 1, 1, 1], 8, 2, 128, 16)
    d = _to_device(case)
    out = _decode(case, d, partition_size=512)
    assert _bits(out).tobytes() == _bits(np.repeat(case.new_v, 4, axis=1)).tobytes()


def test_bf16_physical_relabelling_and_block_size_bitwise():
    torch = _torch()
    outs = []
    for B in (16, 8, 32):
        case = _make(77, [1, 16, 17, 300, 1025, 3001], 32, 8, 128, B, logical_seed=78)
        d = _to_device(case)
        outs.append(_bits(_decode(case, d)))
        if B == 16:
            perm = np.random.default_rng(5).permutation(case.num_blocks)
            inv = np.argsort(perm)
            bt = case.block_tables.copy()
            bt[bt >= 0] = inv[bt[bt >= 0]]
            idx = torch.from_numpy(perm).cuda()
            d.k_cache = d.k_cache[idx].contiguous()
            d.v_cache = d.v_cache[idx].contiguous()
            got = _bits(_decode(case, d, tables=torch.from_numpy(bt).cuda()))
            assert got.tobytes() == outs[0].tobytes(), "relabelled pool"
    assert outs[0].tobytes() == outs[1].tobytes() == outs[2].tobytes(), "block sizes"


def test_bf16_split_launches_partitions_and_noalloc_bitwise():
    torch = _torch()
    case = _make(77, [1, 16, 17, 300, 1025, 3001], 32, 8, 128, 16, logical_seed=78)
    d = _to_device(case)
    for part in (0, 256):
        one = _bits(_decode(case, d, partition_size=part))
        assert _bits(_decode(case, d, partition_size=part, split=True)).tobytes() == one.tobytes()
        assert _bits(_decode(case, d, partition_size=part, noalloc=True)).tobytes() == one.tobytes()
    # fixed partitions: a row does not depend on the rest of the batch
    full = _bits(_decode(case, d, partition_size=512))
    idx = torch.tensor([5, 0, 5, 3], device="cuda")
    got = _bits(_decode(case, d, partition_size=512, q=d.q[idx].contiguous(),
                        tables=d.tables[idx].contiguous(), ctx=d.ctx[idx].contiguous()))
    for j, s in enumerate([5, 0, 5, 3]):
        assert got[j].tobytes() == full[s].tobytes(), f"batch row {j}"


def test_bf16_is_refused_where_it_is_not_built():
    torch = _torch()
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    ctx = torch.ones((1,), dtype=torch.int32, device="cuda")
    with pytest.raises(P.PaError):
        P.pa_decode_append(torch.empty_like(q), q, kc[0, :, 0].contiguous(), kc[0, :, 0].contiguous(),
                           kc, kc, bt, ctx, 0.1, 16, 2, max_context_len=16)
