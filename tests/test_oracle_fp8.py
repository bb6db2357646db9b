"""Pins for the oracle's FP8 (E4M3) KV cache: the code table, the store's rounding and
saturation, and attention over the dequantized pools.

The pages say only that blocks hold compressed K/V which the kernel dequantizes
([CON] section 6); the format (OCP E4M3), the per-tensor scales and saturation are
readings.  The pins tie the oracle's code table and its encoder to values fixed by the
format's definition and to torch's own float8_e4m3fn conversion, and tie the FP8 decode
to the already pinned fp64 definition.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import pa_oracle as O


def _torch_values(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_f1_code_table_special_values():
    v = O.E4M3_TABLE
    assert v[0x00] == 0.0 and not math.copysign(1.0, v[0x00]) < 0
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0      # -0
    assert v[0x01] == 2.0 ** -9                                    # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                                # largest subnormal
    assert v[0x08] == 2.0 ** -6                                    # smallest normal
    assert v[0x38] == 1.0 and v[0x39] == 1.125
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0                  # largest finite
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])             # the only NaNs
    assert int(np.isnan(v).sum()) == 2


def test_f1_code_table_equals_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    t = _torch_values(codes)
    assert np.array_equal(np.isnan(t), np.isnan(O.E4M3_TABLE))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], O.E4M3_TABLE[ok])
    assert np.array_equal(np.signbit(t[ok]), np.signbit(O.E4M3_TABLE[ok]))


def test_f2_encoder_round_trips_every_code():
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[~np.isnan(O.E4M3_TABLE)]
    assert np.array_equal(O.e4m3_encode(O.E4M3_TABLE[finite]), finite)
    assert O.e4m3_encode([math.nan, -math.nan, np.float32("nan")]).tolist() == [0x7F] * 3


def test_f3_encoder_equals_torch_rounding_in_range():
    """torch rounds float32 to E4M3 to nearest, ties to even; in range the two agree."""
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100_000) * 20.0,                        # typical magnitudes
        rng.standard_normal(20_000) * 0.01,                         # subnormal range
        np.frombuffer(np.arange(65536, dtype=np.uint16).tobytes(), dtype=np.float16).astype(np.float64),
    ])
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)].astype(np.float32)
    got = O.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_f4_midpoints_go_to_the_even_code():
    pos = O.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0
    got = O.e4m3_encode(mids)
    lower = np.arange(0x7E, dtype=np.uint8)
    want = np.where(lower % 2 == 0, lower, lower + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    assert np.array_equal(O.e4m3_encode(-mids), want | 0x80)


def test_f5_saturation_and_brute_force_nearest():
    assert O.e4m3_encode([449.0, 464.0, 1e6, math.inf]).tolist() == [0x7E] * 4
    assert O.e4m3_encode([-449.0, -1e30, -math.inf]).tolist() == [0xFE] * 3
    # brute force: the nearest of all finite values, on a grid that includes far-off values
    x = np.linspace(-500.0, 500.0, 40_001)
    finite = np.arange(256)[~np.isnan(O.E4M3_TABLE)]
    vals = O.E4M3_TABLE[finite]
    dist = np.abs(np.clip(x, -448, 448)[:, None] - vals[None, :])
    best = dist.min(axis=1)
    got = O.E4M3_TABLE[O.e4m3_encode(x)]
    assert np.array_equal(np.abs(np.clip(x, -448, 448) - got), best)


def _exact_code(x: float, scale: float) -> int:
    """Nearest E4M3 code to x / scale in exact rational arithmetic (pure Python): every
    finite non-negative value is compared with |x| / scale (clamped to 448), ties to the even
    code, the sign of x added.  Independent of the oracle's float64 quotient."""
    if math.isnan(x):
        return 0x7F
    q = min(abs(Fraction(x) / Fraction(scale)), Fraction(448))
    best = None
    for c in range(0x7F):
        d = abs(q - Fraction(O.e4m3_value(c)))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if math.copysign(1.0, x) < 0 else 0)


def _near_midpoint_pairs(n, seed):
    """(x, scale) pairs whose exact quotient lies within a few fp32 steps of a midpoint between
    two E4M3 values: scale = fp32(x / m) and its fp32 neighbours."""
    rng = np.random.default_rng(seed)
    pos = O.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0
    f16 = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    f16 = f16[np.isfinite(f16) & (f16 != 0)]
    pairs = []
    while len(pairs) < n:
        x, m = float(rng.choice(f16)), float(rng.choice(mids))
        s = np.float32(abs(x) / m)
        if not (np.isfinite(s) and s > 0):
            continue
        for step in (-1, 0, 1):
            t = s if step == 0 else np.nextafter(s, np.float32(np.inf if step > 0 else 0.0), dtype=np.float32)
            pairs.append((x, float(t)))
    return pairs


def test_f6_store_is_the_nearest_code_to_the_exact_quotient():
    """The stored code of x is the code nearest to x / scale itself.  x = 3.873046875 with the
    fp32 scale 0.050961144268512726 has x / scale = 75.99999825, just below the midpoint 76
    between 72 and 80, so the code is 0x69 (72); the fp32 product x * fp32(1/scale) rounds to
    76.0 exactly and would give the even code 0x6A (80)."""
    x, s = 3.873046875, 0.050961144268512726
    assert float(np.float16(x)) == x and float(np.float32(s)) == s
    assert Fraction(x) / Fraction(s) < 76 and O.e4m3_value(0x69) == 72.0
    assert _exact_code(x, s) == 0x69
    pool = np.zeros((1, 1, 1, 1), np.uint8)
    k = np.array([[[x]]], np.float16)
    kc, vc = O.cache_write_fp8(k, -k, np.array([0], np.int64), pool, pool, 1, s, s)
    assert kc[0, 0, 0, 0] == 0x69 and vc[0, 0, 0, 0] == 0xE9
    # near-midpoint pairs, exact ties among them, and random pairs: exact rational arithmetic
    rng = np.random.default_rng(11)
    pairs = _near_midpoint_pairs(300, 6)
    pairs += [(float(np.float16(v)), float(np.float32(sc))) for v, sc in
              zip(rng.standard_normal(200) * 4, np.exp(rng.uniform(-8, 3, 200)))]
    pairs += [(72.0 * 0.25 + 8.0 * 0.125, 0.25), (3.0, 2.0 ** -5 / 1.0), (-0.0, 1.0), (0.0, 3.0)]
    xs = np.array([p[0] for p in pairs], np.float16)
    ss = [p[1] for p in pairs]
    got = [int(O.e4m3_encode(O.fp8_quotient(xs[i:i + 1], ss[i]))[0]) for i in range(len(pairs))]
    want = [_exact_code(float(xs[i]), ss[i]) for i in range(len(pairs))]
    assert got == want
    # in range, the dequantized error is at most half a code step relative (2^-4) plus half
    # the subnormal step
    ks = 0.037
    ref = xs.astype(np.float64)
    ref = ref[np.abs(ref) <= 448.0 * ks]
    deq = O.dequantize_pool(O.e4m3_encode(O.fp8_quotient(ref, ks)), ks)
    assert ref.size > 100
    assert np.all(np.abs(deq - ref) <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * ks + 1e-12)


def test_f7_fp8_decode_is_attention_on_the_dequantized_pools():
    """With K and V already on the E4M3 grid and scales that are powers of two, the store is
    lossless, so FP8 decode equals the pinned fp64 decode of the original values."""
    rng = np.random.default_rng(7)
    case = W.make_case(seed=8, dtype=np.float16, context_lens=[1, 9, 33], num_q_heads=4,
                       num_kv_heads=2, head_dim=8, block_size=4, sigma=1.0)
    finite = O.E4M3_TABLE[np.isfinite(O.E4M3_TABLE) & (np.abs(O.E4M3_TABLE) <= 8)]
    ks, vs = 0.5, 2.0
    pk = (rng.choice(finite, size=case.prefix_k.shape) * ks).astype(np.float16)
    pv = (rng.choice(finite, size=case.prefix_v.shape) * vs).astype(np.float16)
    nk = (rng.choice(finite, size=case.new_k.shape) * ks).astype(np.float16)
    nv = (rng.choice(finite, size=case.new_v.shape) * vs).astype(np.float16)
    shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    k8, v8 = O.cache_write_fp8(pk, pv, case.prefix_slots, np.zeros(shape, np.uint8),
                               np.zeros(shape, np.uint8), case.block_size, ks, vs)
    k8, v8 = O.cache_write_fp8(nk, nv, case.new_slots, k8, v8, case.block_size, ks, vs)
    got = O.decode_fp8(case.q, k8, v8, ks, vs, case.block_tables, case.context_lens,
                       case.scale, case.block_size, case.num_kv_heads)
    kc, vc = O.cache_write(pk, pv, case.prefix_slots, case.empty_pool(), case.empty_pool(),
                           case.block_size)
    kc, vc = O.cache_write(nk, nv, case.new_slots, kc, vc, case.block_size)
    want = O.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                    case.block_size, case.num_kv_heads)
    assert np.array_equal(got, want)


def test_f8_planted_reciprocal_quotient_is_caught(monkeypatch):
    """Storing the code of the fp32 product x * fp32(1/scale) instead of x / scale fails F6."""
    def recip(x, scale):
        with np.errstate(all="ignore"):
            return np.asarray(x, np.float32) * np.float32(1.0 / float(scale))

    monkeypatch.setattr(O, "fp8_quotient", recip)
    with pytest.raises(AssertionError):
        test_f6_store_is_the_nearest_code_to_the_exact_quotient()


@pytest.mark.parametrize("mutant", ["ties_up", "no_saturation", "lost_sign"])
def test_f8_planted_encoder_mistakes_are_caught(monkeypatch, mutant):
    real = O.e4m3_encode

    def wrong(x):
        x = np.asarray(x, dtype=np.float64)
        c = real(x)
        if mutant == "ties_up":  # round half up instead of to even
            pos = O.E4M3_TABLE[:0x7F]
            mag = np.abs(x)
            i = np.clip(np.searchsorted(pos, mag), 1, 0x7E)
            tie = np.isclose(mag, (pos[i - 1] + pos[i]) / 2, rtol=0, atol=0)
            c = np.where(tie, (i | (c & 0x80)).astype(np.uint8), c)
        elif mutant == "no_saturation":
            c = np.where(np.abs(x) > 464.0, (0x7F | (c & 0x80)).astype(np.uint8), c)
        else:
            c = c & 0x7F
        return c.astype(np.uint8)

    monkeypatch.setattr(O, "e4m3_encode", wrong)
    catcher = {"ties_up": test_f4_midpoints_go_to_the_even_code,
               "no_saturation": test_f5_saturation_and_brute_force_nearest,
               "lost_sign": test_f4_midpoints_go_to_the_even_code}[mutant]
    with pytest.raises(AssertionError):
        catcher()
