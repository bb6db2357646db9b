"""GPU checks of the virtually contiguous cache (HIP virtual memory) and pa_decode_dense.

The dense path runs the same tiles, work split and arithmetic as pa_decode, only with each
tile's address computed instead of looked up, so on the same tokens its output must equal
the paged output bit for bit; both are also held to the oracle.  Page accounting, writes
past the backed capacity, freeing and re-mapping are checked from the host.
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


def _fill(kv, case):
    """Write every token of the case into the dense cache (prefix, then the new tokens)."""
    torch = _torch()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    seq, pos = [], []
    for s in range(case.num_seqs):
        n = int(case.context_lens[s]) - 1
        seq.append(np.full(n, s, np.int32))
        pos.append(np.arange(n, dtype=np.int32))
    order = np.concatenate(case.meta["seq_rows"]) if case.num_seqs else np.zeros(0, np.int64)
    kv.write(t(case.prefix_k[order]), t(case.prefix_v[order]), t(np.concatenate(seq)), t(np.concatenate(pos)))
    kv.write(t(case.new_k), t(case.new_v), t(np.arange(case.num_seqs, dtype=np.int32)),
             t((case.context_lens - 1).astype(np.int32)))
    torch.cuda.synchronize()


def _dense_decode(kv, case, partition=0):
    torch = _torch()
    q = torch.from_numpy(case.q).cuda()
    out = torch.empty_like(q)
    kv.decode(out, q, case.scale, partition_size=partition)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("D,hkv,hq", [(128, 8, 32), (64, 2, 16)])
def test_dense_equals_paged_bitwise_and_the_oracle(D, hkv, hq):
    case = W.make_case(seed=61, dtype=np.float16, context_lens=[1, 15, 16, 17, 1023, 1024, 1025, 2049, 3000],
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=D, block_size=16, sigma=0.5)
    kv = P.DenseKV(case.num_seqs, 3000, hkv, D)
    kv.step(case.context_lens.tolist())
    tpp = kv.page_bytes // (hkv * D * 2)
    assert tpp % 16 == 0
    for s, c in enumerate(case.context_lens):
        assert kv.capacity(s) == min(3000, -(-int(c) // tpp) * tpp)
    pages = sum(-(-int(c) // tpp) for c in case.context_lens)
    assert kv.mapped_bytes == 2 * (pages + 1) * kv.page_bytes  # K and V, guard pages included
    _fill(kv, case)
    for part in (0, 64):
        dense = _dense_decode(kv, case, part)
        d = G.to_device(case)
        paged = G.decode(case, d, partition_size=part)
        assert dense.tobytes() == paged.tobytes(), f"partition {part}"
    kc, vc = oracle_pools(case)
    G.assert_close(dense, oracle_decode(case, kc, vc), np.float16, f"dense D{D}")
    kv.close()


def test_writes_past_the_backed_capacity_are_skipped():
    torch = _torch()
    case = W.make_case(seed=62, dtype=np.float16, context_lens=[40, 70], num_q_heads=8, num_kv_heads=2,
                       head_dim=128, block_size=16, sigma=0.5)
    kv = P.DenseKV(4, 100000, 2, 128)
    kv.step(case.context_lens.tolist())
    _fill(kv, case)
    before = _dense_decode(kv, case)
    cap = kv.capacity(0)
    junk = torch.full((3, 2, 128), 1000.0, dtype=torch.float16, device="cuda")
    kv.write(junk, junk, torch.tensor([0, 1, 3], dtype=torch.int32, device="cuda"),
             torch.tensor([cap, cap + 5000, 0], dtype=torch.int32, device="cuda"))  # unbacked: skipped
    torch.cuda.synchronize()
    assert _dense_decode(kv, case).tobytes() == before.tobytes()
    kv.close()


def test_free_and_remap_a_sequence():
    torch = _torch()
    case = W.make_case(seed=63, dtype=np.float16, context_lens=[500, 2000, 33], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, block_size=16, sigma=0.5)
    kv = P.DenseKV(3, 4096, 2, 128)
    kv.step(case.context_lens.tolist())
    _fill(kv, case)
    first = _dense_decode(kv, case)
    mapped = kv.mapped_bytes
    kv.free_seq(1)
    assert kv.capacity(1) == 0 and kv.mapped_bytes < mapped
    kv.step(case.context_lens.tolist())  # sequence 1 comes back (fresh pages) ...
    assert kv.mapped_bytes == mapped
    _fill(kv, case)                      # ... and is written again
    assert _dense_decode(kv, case).tobytes() == first.tobytes()
    with pytest.raises(P.PaError):
        kv.step([500, 5000, 33])  # beyond max_context_len: refused, nothing mapped
    assert kv.mapped_bytes == mapped
    kv.close()


def test_contexts_of_zero_and_invalid_lengths():
    torch = _torch()
    case = W.make_case(seed=64, dtype=np.float16, context_lens=[100, 1, 300], num_q_heads=4,
                       num_kv_heads=1, head_dim=64, block_size=16, sigma=0.5)
    kv = P.DenseKV(3, 512, 1, 64)
    kv.step(case.context_lens.tolist())
    _fill(kv, case)
    full = _dense_decode(kv, case)
    kv.step([100, 0, 300])  # sequence 1 now has no tokens: a zero row
    got = _dense_decode(kv, case)
    assert np.all(got[1] == 0)
    kc, vc = oracle_pools(case)
    ref = oracle_decode(case, kc, vc)
    G.assert_close(got[[0, 2]], ref[[0, 2]], np.float16, "others")
    assert np.isfinite(full).all()
    kv.close()


def test_dense_equals_paged_after_many_other_kernels():
    """The work split depends on the resident-wave count of each kernel, which the library
    memoises.  Regression: with more kernels in use than its table held, a kernel seen late got
    another split (and different rounding) than the paged kernel seen early.  Here the paged
    kernel runs first, then a dozen other decode kernels, then the dense one."""
    torch = _torch()
    case = W.make_case(seed=65, dtype=np.float16, context_lens=[1, 15, 16, 17, 1023, 1024, 1025, 2049, 3000],
                       num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, sigma=0.5)
    d = G.to_device(case)
    paged = G.decode(case, d)
    for D, hq, hkv in ((64, 4, 4), (64, 8, 4), (64, 16, 4), (64, 32, 4),
                       (128, 4, 4), (128, 8, 4), (128, 16, 4), (128, 32, 4)):  # every fp32 group tile
        other = W.make_case(seed=66, dtype=np.float32, context_lens=[5, 40], num_q_heads=hq, num_kv_heads=hkv,
                            head_dim=D, block_size=16, sigma=0.5)
        G.decode(other, G.to_device(other))
    for D in (64, 128):  # fp16 at the other head size, E4M3 and append kernels
        other = W.make_case(seed=67, dtype=np.float16, context_lens=[5, 40], num_q_heads=8, num_kv_heads=2,
                            head_dim=D, block_size=16, sigma=0.5)
        od = G.to_device(other, write_new=False)
        out = torch.empty_like(od.q)
        P.pa_decode_append(out, od.q, od.new_k, od.new_v, od.k_cache, od.v_cache, od.tables, od.ctx,
                           other.scale, 16, 2, max_context_len=other.max_context_len)
        codes = torch.zeros(od.k_cache.shape, dtype=torch.uint8, device="cuda")
        P.pa_decode_fp8(out, od.q, codes, codes, od.tables, od.ctx, other.scale, 1.0, 1.0, 16, 2,
                        max_context_len=other.max_context_len)
        P.pa_decode_fp8_append(out, od.q, od.new_k, od.new_v, codes, codes.clone(), od.tables, od.ctx,
                               other.scale, 1.0, 1.0, 16, 2, max_context_len=other.max_context_len)
        if D == 64:
            G.decode(other, G.to_device(other))
    torch.cuda.synchronize()
    kv = P.DenseKV(case.num_seqs, 3000, 8, 128)
    kv.step(case.context_lens.tolist())
    _fill(kv, case)
    assert _dense_decode(kv, case).tobytes() == paged.tobytes()
    kv.close()
