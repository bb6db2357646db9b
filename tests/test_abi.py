"""CPU-side checks of the C ABI: the library loads, exports what include/pa.h declares,
and rejects invalid arguments before launching anything (no GPU is touched)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_167_amd as P
from paged_kv_cache_167_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libpa.so not built (run __graft_entry__.build())")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(pa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    names = _declared_functions()
    for want in ("pa_cache_write", "pa_decode", "pa_decode_workspace_bytes",
                 "pa_decode_partitions", "pa_decode_reduce", "pa_last_error", "pa_abi_version",
                 "pa_cache_write_fp8", "pa_decode_fp8", "pa_decode_fp8_partitions",
                 "pa_prefill", "pa_decode_append", "pa_decode_append_partitions",
                 "pa_decode_fp8_append", "pa_decode_fp8_append_partitions", "pa_decode_noalloc",
                 "pa_decode_shared", "pa_decode_shared_partitions", "pa_decode_shared_workspace_bytes"):
        assert want in names


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(handle, name), name
    assert set(_declared_functions()) == set(_lib.SIGNATURES)


def test_abi_version():
    assert P.lib().pa_abi_version() == (2 << 16) | 9


def test_workspace_size_query():
    # per (sequence, unit) a 2-int descriptor; per wave two records, each with fp32 max and
    # sum of R rows and R * head_dim fp32 outputs (every region 256-byte aligned).
    # R = min(rows per unit, group); the larger of the fp32 and fp16 layouts is returned.
    al = lambda x: (x + 255) // 256 * 256

    def layout(S, units, waves, R, d):
        return al(S * units * 8) + 2 * al(2 * waves * R * 4) + al(2 * waves * R * d * 4)

    S, hq, hkv, d = 64, 32, 8, 128  # group 4: one unit per kv head, 4 rows per record
    waves = 4096
    assert P.pa_decode_workspace_bytes(S, hq, hkv, d, 4096, 0) == layout(S, hkv, waves, 4, d)
    # 56 query / 8 kv heads: groups of 7, one unit per kv head
    assert P.pa_decode_workspace_bytes(8, 56, 8, d, 131072, 0) == layout(8, 8, waves, 7, d)
    # fixed partitions: one record per partition, ceil(max_ctx / partition_size) per segment
    big = P.pa_decode_workspace_bytes(8, 56, 8, d, 131072, 512)
    recs = 8 * 8 * ((131072 + 511) // 512)
    assert big == al(8 * 8 * 8) + 2 * al(recs * 7 * 4) + al(recs * 7 * d * 4)
    # 64 query heads per kv head: four units of 16 rows (fp16) or eight of 8 (fp32)
    wide = P.pa_decode_workspace_bytes(2, 64, 1, d, 1024, 0)
    assert wide == max(layout(2, 4, waves, 16, d), layout(2, 8, waves, 8, d))
    assert P.pa_decode_workspace_bytes(0, hq, hkv, d, 4096, 0) == 0
    assert P.pa_decode_workspace_bytes(4, 30, 8, d, 4096, 0) == 0  # 30 % 8 != 0


FAKE = 1 << 20  # a 16-byte aligned non-null address that is never dereferenced


def _decode(**over):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, scale=1.0, B=16, hkv=8, S=4,
             hq=32, D=128, mb=16, mcl=256, N=100, P=64, dt=_lib.PA_F16, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(over)
    return P.lib().pa_decode(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["scale"],
                             a["B"], a["hkv"], a["S"], a["hq"], a["D"], a["mb"], a["mcl"], a["N"],
                             a["P"], a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=64), _lib.PA_ERR_UNSUPPORTED),
    (dict(dt=7), _lib.PA_ERR_UNSUPPORTED),
    (dict(hq=30), _lib.PA_ERR_INVALID_ARG),          # not a multiple of the kv heads
    (dict(hkv=0), _lib.PA_ERR_INVALID_ARG),
    (dict(S=-1), _lib.PA_ERR_INVALID_ARG),
    (dict(P=24), _lib.PA_ERR_INVALID_ARG),           # not a multiple of the block size
    (dict(B=8, P=8), _lib.PA_ERR_INVALID_ARG),       # a multiple of the block size, not of 16
    (dict(mcl=257), _lib.PA_ERR_INVALID_ARG),        # beyond max_blocks * block_size
    (dict(N=0), _lib.PA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), _lib.PA_ERR_INVALID_ARG),     # misaligned
    (dict(bt=None), _lib.PA_ERR_INVALID_ARG),
    (dict(scale=0.0), _lib.PA_ERR_INVALID_ARG),      # the scale must be positive and finite
    (dict(scale=-0.1), _lib.PA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.PA_ERR_INVALID_ARG),
    (dict(ws=None), _lib.PA_ERR_WORKSPACE),
    (dict(wsb=16), _lib.PA_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.PA_ERR_WORKSPACE),     # not 256-byte aligned
    (dict(S=65536), _lib.PA_ERR_INVALID_ARG),        # grid dimension limits
    (dict(hq=65536, hkv=8), _lib.PA_ERR_INVALID_ARG),
    # more than 2^31 - 1 segments (sequence x kv head), even with empty contexts
    (dict(S=65535, hkv=40000, hq=40000, D=64, B=8, mcl=0, wsb=1 << 50), _lib.PA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_arguments(over, code):
    assert _decode(**over) == code
    assert P.last_error() != ""


def test_decode_counts_every_partition_in_the_split_bound():
    # 1.5e9-token contexts at fp32 (8-token tiles): the default split's cost (tiles plus one
    # per segment) fits in 32 bits, 16-token partitions (one more per partition) do not
    big = dict(S=1, hkv=8, hq=32, mcl=1_500_000_000, mb=1_500_000_000 // 16, dt=_lib.PA_F32, wsb=1 << 62)
    assert _decode(P=16, **big) == _lib.PA_ERR_INVALID_ARG
    assert "tiles and pieces" in P.last_error()
    _decode(P=0, **big)  # fails later, on the fake workspace pointer, not on the bound
    assert "tiles and pieces" not in P.last_error()


def test_other_element_types_are_refused():
    assert _decode(dt=2) == _lib.PA_ERR_UNSUPPORTED
    assert "dtype" in P.last_error()
    assert P.lib().pa_cache_write(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 100, 2, None) == \
        _lib.PA_ERR_UNSUPPORTED


def test_binding_refuses_mixed_element_types():
    import torch
    q = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.float16)
    bt = torch.zeros((2, 4), dtype=torch.int32)
    ctx = torch.ones((2,), dtype=torch.int32)
    with pytest.raises(P.PaError, match="mixed element types"):
        P.pa_decode(torch.empty_like(q), q, kc, kc, bt, ctx, 0.1, 16, 2, max_context_len=64)
    k = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(P.PaError, match="mixed element types"):
        P.pa_cache_write(k, k, torch.zeros(3, dtype=torch.int64), kc, kc)


def test_decode_with_no_sequences_is_a_no_op():
    assert _decode(S=0, out=None, q=None) == _lib.PA_OK
    assert P.last_error() == ""


def _noalloc(**over):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, scale=1.0, B=16, hkv=8, S=4,
             hq=32, D=128, mb=16, mcl=256, N=100, P=64, dt=_lib.PA_F16, stream=None)
    a.update(over)
    return P.lib().pa_decode_noalloc(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["scale"],
                                     a["B"], a["hkv"], a["S"], a["hq"], a["D"], a["mb"], a["mcl"], a["N"],
                                     a["P"], a["dt"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(dt=7), _lib.PA_ERR_UNSUPPORTED),
    (dict(hq=30), _lib.PA_ERR_INVALID_ARG),
    (dict(P=24), _lib.PA_ERR_INVALID_ARG),
    (dict(mcl=257), _lib.PA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), _lib.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.PA_ERR_INVALID_ARG),
    (dict(S=65536), _lib.PA_ERR_INVALID_ARG),
])
def test_decode_noalloc_rejects_bad_arguments(over, code):
    """Checked on the host before the scratch or the device is touched."""
    assert _noalloc(**over) == code
    assert P.last_error() != ""


def test_decode_noalloc_with_no_sequences_is_a_no_op():
    assert _noalloc(S=0, out=None, q=None) == _lib.PA_OK
    assert P.last_error() == ""


def test_shared_workspace_size_query():
    # per virtual segment (each group's prefix and each sequence's own part, per kv head) a
    # 2-int descriptor and a record; besides, two records per wave of the 4096-wave cap; every
    # record holds fp32 max and sum of 32 rows and 32 * head_dim fp32 outputs
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731

    def layout(S, NG, hkv, d):
        segs = (S + NG) * hkv
        recs = 2 * 4096 + segs
        return al(segs * 8) + 2 * al(recs * 32 * 4) + al(recs * 32 * d * 4)

    assert P.pa_decode_shared_workspace_bytes(256, 16, 32, 8, 128) == layout(256, 16, 8, 128)
    assert P.pa_decode_shared_workspace_bytes(3, 0, 8, 2, 64) == layout(3, 0, 2, 64)
    assert P.pa_decode_shared_workspace_bytes(0, 1, 8, 2, 64) == 0
    assert P.pa_decode_shared_workspace_bytes(4, -1, 8, 2, 64) == 0
    assert P.pa_decode_shared_workspace_bytes(4, 1, 30, 8, 128) == 0  # 30 % 8 != 0


def _shared(fn="pa_decode_shared", **over):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, sg=FAKE, gf=FAKE, gs=FAKE, gp=FAKE, NG=2,
             scale=1.0, B=16, hkv=8, S=4, hq=32, D=128, mb=16, mcl=256, N=100, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(over)
    return getattr(P.lib(), fn)(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["sg"], a["gf"],
                                a["gs"], a["gp"], a["NG"], a["scale"], a["B"], a["hkv"], a["S"], a["hq"],
                                a["D"], a["mb"], a["mcl"], a["N"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("fn", ["pa_decode_shared", "pa_decode_shared_partitions"])
@pytest.mark.parametrize("over,code", [
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=64), _lib.PA_ERR_UNSUPPORTED),
    (dict(hq=8 * 17), _lib.PA_ERR_UNSUPPORTED),      # more than 16 query heads per kv head
    (dict(hq=30), _lib.PA_ERR_INVALID_ARG),
    (dict(mcl=257), _lib.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.PA_ERR_INVALID_ARG),
    (dict(S=65536), _lib.PA_ERR_INVALID_ARG),
    (dict(NG=-1), _lib.PA_ERR_INVALID_ARG),
    (dict(NG=65536), _lib.PA_ERR_INVALID_ARG),
    (dict(sg=None), _lib.PA_ERR_INVALID_ARG),
    (dict(gp=None), _lib.PA_ERR_INVALID_ARG),        # NULL group arrays with groups
    (dict(gf=FAKE + 2), _lib.PA_ERR_INVALID_ARG),    # misaligned
    (dict(q=FAKE + 8), _lib.PA_ERR_INVALID_ARG),
    (dict(ws=None), _lib.PA_ERR_WORKSPACE),
    (dict(wsb=1024), _lib.PA_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.PA_ERR_WORKSPACE),
    # more than 2^31 - 1 tiles over the virtual segments, though the sequences alone fit
    (dict(S=65535, NG=65535, hkv=2, hq=2, mb=8192, mcl=131072, wsb=1 << 50), _lib.PA_ERR_INVALID_ARG),
    # within the tile bound, but the work split's 32-bit cost positions would overflow
    (dict(S=8192, NG=0, hkv=8, hq=32, mb=8192, mcl=131072, wsb=1 << 50), _lib.PA_ERR_INVALID_ARG),
])
def test_decode_shared_rejects_bad_arguments(fn, over, code):
    assert _shared(fn, **over) == code
    assert P.last_error() != ""


def test_decode_shared_with_no_sequences_is_a_no_op():
    assert _shared(S=0, out=None, q=None, ws=None) == _lib.PA_OK
    assert P.last_error() == ""


def _write(**over):
    a = dict(k=FAKE, v=FAKE, sm=FAKE, kc=FAKE, vc=FAKE, T=4, hkv=8, D=128, B=16, N=10,
             dt=_lib.PA_F16, stream=None)
    a.update(over)
    return P.lib().pa_cache_write(a["k"], a["v"], a["sm"], a["kc"], a["vc"], a["T"], a["hkv"],
                                  a["D"], a["B"], a["N"], a["dt"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(D=80), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=4), _lib.PA_ERR_UNSUPPORTED),
    (dict(T=-1), _lib.PA_ERR_INVALID_ARG),
    (dict(hkv=0), _lib.PA_ERR_INVALID_ARG),
    (dict(N=0), _lib.PA_ERR_INVALID_ARG),
    (dict(k=None), _lib.PA_ERR_INVALID_ARG),
    (dict(kc=FAKE + 4), _lib.PA_ERR_INVALID_ARG),
    (dict(sm=FAKE + 4), _lib.PA_ERR_INVALID_ARG),
    (dict(T=(1 << 31) - 1), _lib.PA_ERR_INVALID_ARG),  # more threads than one launch counts
])
def test_cache_write_rejects_bad_arguments(over, code):
    assert _write(**over) == code


def test_cache_write_with_no_tokens_is_a_no_op():
    assert _write(T=0, k=None, v=None) == _lib.PA_OK


def test_reduce_rejects_bad_arguments():
    lib = P.lib()
    assert lib.pa_decode_reduce(FAKE, FAKE, 4, 32, 8, 96, 4096, 0, 1, FAKE, 1 << 30, None) == \
        _lib.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_reduce(FAKE, FAKE, 4, 32, 8, 128, 4096, 0, 1, None, 0, None) == \
        _lib.PA_ERR_WORKSPACE
    assert lib.pa_decode_reduce(FAKE, FAKE, 4, 30, 8, 128, 4096, 0, 1, FAKE, 1 << 30, None) == \
        _lib.PA_ERR_INVALID_ARG
    # more than 2^31 - 1 segments (sequence x kv head), whatever the workspace
    assert lib.pa_decode_reduce(FAKE, FAKE, 65535, 40000, 40000, 64, 0, 0, 1, FAKE, 1 << 50, None) == \
        _lib.PA_ERR_INVALID_ARG
    # partition size not a multiple of 16; partitions whose record rows overflow 32 bits
    assert lib.pa_decode_reduce(FAKE, FAKE, 4, 32, 8, 128, 4096, 24, 1, FAKE, 1 << 30, None) == \
        _lib.PA_ERR_INVALID_ARG
    assert lib.pa_decode_reduce(FAKE, FAKE, 64, 32, 8, 128, 1 << 30, 16, 1, FAKE, 1 << 62, None) == \
        _lib.PA_ERR_INVALID_ARG
    assert "too many partitions" in P.last_error()
    assert lib.pa_decode_reduce(FAKE, FAKE, 0, 32, 8, 128, 4096, 0, 1, None, 0, None) == _lib.PA_OK


def _append(fn="pa_decode_append", **over):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, scale=0.1, B=16,
             hkv=8, S=4, hq=32, D=128, mb=16, mcl=256, N=100, P=64, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return getattr(P.lib(), fn)(a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["ctx"],
                                a["scale"], a["B"], a["hkv"], a["S"], a["hq"], a["D"], a["mb"], a["mcl"],
                                a["N"], a["P"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("fn", ["pa_decode_append", "pa_decode_append_partitions"])
@pytest.mark.parametrize("over,code", [
    (dict(kn=None), _lib.PA_ERR_INVALID_ARG),
    (dict(vn=None), _lib.PA_ERR_INVALID_ARG),
    (dict(kn=FAKE + 8), _lib.PA_ERR_INVALID_ARG),   # misaligned
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=4), _lib.PA_ERR_UNSUPPORTED),
    (dict(scale=0.0), _lib.PA_ERR_INVALID_ARG),
    (dict(mcl=257), _lib.PA_ERR_INVALID_ARG),
    (dict(kc=None), _lib.PA_ERR_INVALID_ARG),
    (dict(wsb=16), _lib.PA_ERR_WORKSPACE),
])
def test_decode_append_rejects_bad_arguments(fn, over, code):
    assert _append(fn, **over) == code
    assert P.last_error() != ""


def test_decode_append_with_no_sequences_is_a_no_op():
    assert _append(S=0, out=None, q=None, kn=None, vn=None) == _lib.PA_OK


def test_decode_append_binding_takes_fp16_only():
    import torch
    h = torch.zeros((2, 4, 64), dtype=torch.float32)
    pool = torch.zeros((3, 2, 16, 64), dtype=torch.float32)
    with pytest.raises(P.PaError):
        P.pa_decode_append(h, h, h[:, :2], h[:, :2], pool, pool, None, None, 0.1, 16, 2)


def _append_fp8(fn="pa_decode_fp8_append", **over):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, scale=0.1, ks=0.01,
             vs=0.02, B=16, hkv=8, S=4, hq=32, D=128, mb=16, mcl=256, N=100, P=64, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(over)
    return getattr(P.lib(), fn)(a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["ctx"],
                                a["scale"], a["ks"], a["vs"], a["B"], a["hkv"], a["S"], a["hq"], a["D"],
                                a["mb"], a["mcl"], a["N"], a["P"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("fn", ["pa_decode_fp8_append", "pa_decode_fp8_append_partitions"])
@pytest.mark.parametrize("over,code", [
    (dict(kn=None), _lib.PA_ERR_INVALID_ARG),
    (dict(vn=FAKE + 4), _lib.PA_ERR_INVALID_ARG),
    (dict(ks=0.0), _lib.PA_ERR_INVALID_ARG),
    (dict(vs=float("inf")), _lib.PA_ERR_INVALID_ARG),
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(hq=30), _lib.PA_ERR_INVALID_ARG),
    (dict(wsb=16), _lib.PA_ERR_WORKSPACE),
])
def test_decode_fp8_append_rejects_bad_arguments(fn, over, code):
    assert _append_fp8(fn, **over) == code
    assert P.last_error() != ""


def test_decode_fp8_append_with_no_sequences_is_a_no_op():
    assert _append_fp8(S=0, out=None, q=None, kn=None, vn=None) == _lib.PA_OK


def _decode_fp8(fn="pa_decode_fp8", **over):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, scale=0.1, ks=0.01, vs=0.02,
             B=16, hkv=8, S=4, hq=32, D=128, mb=16, mcl=256, N=100, P=64, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(over)
    return getattr(P.lib(), fn)(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["scale"],
                                a["ks"], a["vs"], a["B"], a["hkv"], a["S"], a["hq"], a["D"], a["mb"],
                                a["mcl"], a["N"], a["P"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("fn", ["pa_decode_fp8", "pa_decode_fp8_partitions"])
@pytest.mark.parametrize("over,code", [
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=4), _lib.PA_ERR_UNSUPPORTED),
    (dict(ks=0.0), _lib.PA_ERR_INVALID_ARG),          # scales: positive and finite
    (dict(vs=-1.0), _lib.PA_ERR_INVALID_ARG),
    (dict(ks=float("nan")), _lib.PA_ERR_INVALID_ARG),
    (dict(vs=float("inf")), _lib.PA_ERR_INVALID_ARG),
    (dict(scale=1e30, ks=1e30), _lib.PA_ERR_INVALID_ARG),  # scale * k_scale overflows fp32
    (dict(scale=0.0), _lib.PA_ERR_INVALID_ARG),
    (dict(hq=30), _lib.PA_ERR_INVALID_ARG),
    (dict(mcl=257), _lib.PA_ERR_INVALID_ARG),
    (dict(kc=FAKE + 8), _lib.PA_ERR_INVALID_ARG),
    (dict(wsb=16), _lib.PA_ERR_WORKSPACE),
])
def test_decode_fp8_rejects_bad_arguments(fn, over, code):
    assert _decode_fp8(fn, **over) == code
    assert P.last_error() != ""


def test_decode_fp8_with_no_sequences_is_a_no_op():
    assert _decode_fp8(S=0, out=None, q=None) == _lib.PA_OK


def _write_fp8(**over):
    a = dict(k=FAKE, v=FAKE, sm=FAKE, kc=FAKE, vc=FAKE, ks=0.5, vs=0.25, T=4, hkv=8, D=128, B=16,
             N=10, stream=None)
    a.update(over)
    return P.lib().pa_cache_write_fp8(a["k"], a["v"], a["sm"], a["kc"], a["vc"], a["ks"], a["vs"],
                                      a["T"], a["hkv"], a["D"], a["B"], a["N"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(D=80), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=64), _lib.PA_ERR_UNSUPPORTED),
    (dict(ks=0.0), _lib.PA_ERR_INVALID_ARG),
    (dict(vs=float("nan")), _lib.PA_ERR_INVALID_ARG),
    (dict(ks=float("-inf")), _lib.PA_ERR_INVALID_ARG),
    (dict(T=-1), _lib.PA_ERR_INVALID_ARG),
    (dict(N=0), _lib.PA_ERR_INVALID_ARG),
    (dict(v=None), _lib.PA_ERR_INVALID_ARG),
    (dict(vc=FAKE + 4), _lib.PA_ERR_INVALID_ARG),
    (dict(sm=FAKE + 4), _lib.PA_ERR_INVALID_ARG),
    (dict(T=(1 << 31) - 1), _lib.PA_ERR_INVALID_ARG),  # more threads than one launch counts
])
def test_cache_write_fp8_rejects_bad_arguments(over, code):
    assert _write_fp8(**over) == code
    assert P.last_error() != ""


def test_cache_write_fp8_with_no_tokens_is_a_no_op():
    assert _write_fp8(T=0, k=None, v=None) == _lib.PA_OK


def test_fp8_binding_checks_element_types():
    import torch
    h = torch.zeros((2, 8, 16, 128), dtype=torch.float16)
    with pytest.raises(P.PaError, match="uint8"):
        P.pa_decode_fp8(h, h, h, h, None, None, 0.1, 1.0, 1.0, 16, 8)
    with pytest.raises(P.PaError, match="uint8"):
        P.pa_cache_write_fp8(h, h, None, h, h, 1.0, 1.0)


def _prefill(**over):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, ctx=FAKE, qs=FAKE, scale=0.1, B=16,
             hkv=8, S=4, hq=32, D=128, mb=16, mql=64, mcl=256, N=100, dt=_lib.PA_F16, stream=None)
    a.update(over)
    return P.lib().pa_prefill(a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], a["qs"],
                              a["scale"], a["B"], a["hkv"], a["S"], a["hq"], a["D"], a["mb"],
                              a["mql"], a["mcl"], a["N"], a["dt"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(dt=_lib.PA_F32), _lib.PA_ERR_UNSUPPORTED),
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(B=4), _lib.PA_ERR_UNSUPPORTED),
    (dict(scale=0.0), _lib.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.PA_ERR_INVALID_ARG),
    (dict(hq=30), _lib.PA_ERR_INVALID_ARG),
    (dict(mql=-1), _lib.PA_ERR_INVALID_ARG),
    (dict(mcl=257), _lib.PA_ERR_INVALID_ARG),
    (dict(N=0), _lib.PA_ERR_INVALID_ARG),
    (dict(S=70000), _lib.PA_ERR_INVALID_ARG),
    (dict(qs=None), _lib.PA_ERR_INVALID_ARG),
    (dict(qs=FAKE + 2), _lib.PA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), _lib.PA_ERR_INVALID_ARG),
])
def test_prefill_rejects_bad_arguments(over, code):
    assert _prefill(**over) == code
    assert P.last_error() != ""


def test_prefill_with_nothing_to_do_is_a_no_op():
    assert _prefill(S=0, out=None, q=None) == _lib.PA_OK
    assert _prefill(mql=0, out=None, q=None) == _lib.PA_OK


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libpa.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()
