"""GPU-side test helpers: move a workload to cuda:0, fill its pools through
pa_cache_write, run pa_decode, and compare against the CPU oracle."""
import sys
from types import SimpleNamespace

import numpy as np

import paged_kv_cache_167_amd as P


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_case_host(case):
    """Host-side precondition check before any launch: every table entry a sequence
    uses is a valid block, slots are distinct and inside the pool."""
    B = case.block_size
    for s in range(case.num_seqs):
        nb = -(-int(case.context_lens[s]) // B)
        row = case.block_tables[s, :nb]
        assert np.all(row >= 0) and np.all(row < case.num_blocks), f"bad table row {s}"
    assert int(case.context_lens.max()) <= case.block_tables.shape[1] * B
    slots = np.concatenate([case.prefix_slots, case.new_slots])
    assert np.all(slots >= 0) and np.all(slots < case.num_blocks * B)
    assert len(np.unique(slots)) == len(slots), "duplicate slots"


def to_device(case, dev="cuda:0", write_new=True):
    import torch
    check_case_host(case)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    d = SimpleNamespace()
    d.q = t(case.q)
    d.tables = t(case.block_tables)
    d.ctx = t(case.context_lens)
    d.k_cache = t(case.empty_pool())
    d.v_cache = t(case.empty_pool())
    d.new_k, d.new_v, d.new_slots = t(case.new_k), t(case.new_v), t(case.new_slots)
    pk, pv, ps = t(case.prefix_k), t(case.prefix_v), t(case.prefix_slots)
    P.pa_cache_write(pk, pv, ps, d.k_cache, d.v_cache)
    del pk, pv, ps
    if write_new:
        P.pa_cache_write(d.new_k, d.new_v, d.new_slots, d.k_cache, d.v_cache)
    torch.cuda.synchronize()
    return d


def decode(case, d, partition_size=P.DEFAULT_PARTITION, max_context_len=None, q=None,
           tables=None, ctx=None, k_cache=None, v_cache=None, split=False):
    import torch
    q = d.q if q is None else q
    out = torch.empty_like(q)
    mcl = case.max_context_len if max_context_len is None else max_context_len
    args = (out, q, d.k_cache if k_cache is None else k_cache,
            d.v_cache if v_cache is None else v_cache, d.tables if tables is None else tables,
            d.ctx if ctx is None else ctx, case.scale, case.block_size, case.num_kv_heads)
    if split:
        ws = P.pa_decode_partitions(*args, max_context_len=mcl, partition_size=partition_size)
        P.pa_decode_reduce(out, d.ctx if ctx is None else ctx, case.num_kv_heads, mcl,
                           partition_size, ws)
    else:
        P.pa_decode(*args, max_context_len=mcl, partition_size=partition_size)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_close(got, ref, dtype, label):
    """The pass/fail gate |gpu - ref| <= 2e-3 + 1e-2 |ref|, plus the sharper normalised check
    max|gpu - ref| / std(ref) <= 2e-2 (fp16) or 1e-4 (fp32)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = np.abs(got - ref)
    bound = 2e-3 + 1e-2 * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{label}: tolerance exceeded at {worst}: got {got[worst]} "
                                  f"ref {ref[worst]}")
    norm = err.max() / max(ref.std(), 1e-30)
    lim = 1e-4 if np.dtype(dtype) == np.float32 else 2e-2
    assert norm <= lim, f"{label}: normalised error {norm:.3e} > {lim}"
    return float(err.max()), float(norm)
