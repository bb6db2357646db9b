"""Test-side helpers: build the oracle's pools for a workload and compare results."""
import numpy as np

from oracle import pa_oracle


def oracle_pools(case, *, include_new=True):
    """NaN-filled pools with every prefix token (and the new tokens) written by the oracle."""
    kc, vc = pa_oracle.cache_write(case.prefix_k, case.prefix_v, case.prefix_slots,
                                   case.empty_pool(), case.empty_pool(), case.block_size)
    if include_new:
        kc, vc = pa_oracle.cache_write(case.new_k, case.new_v, case.new_slots, kc, vc,
                                       case.block_size)
    return kc, vc


def oracle_decode(case, kc, vc):
    return pa_oracle.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                            case.block_size, case.num_kv_heads)


def tol_check(got, ref, atol=2e-3, rtol=1e-2):
    """Element-wise |got - ref| <= atol + rtol * |ref|; returns (ok, worst excess, normalised max err)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    ok = bool(np.all(err <= bound)) and bool(np.all(np.isfinite(got)))
    std = float(ref.std()) if ref.size else 1.0
    return ok, float((err - bound).max()) if err.size else 0.0, float(err.max() / max(std, 1e-300))
