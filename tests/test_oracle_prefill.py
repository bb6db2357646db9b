"""Pins for the oracle's chunked-prefill attention (several query tokens per sequence).

The pages describe the prompt phase and paged prefill kernels but give no formula; the
reading is causal attention of each chunk token over the context up to and including its
own position.  The pins tie the oracle to torch's scaled_dot_product_attention in float64
(with is_causal for whole prompts, with an explicit bottom-right mask for chunks), to
pure-Python loops, to the already pinned decode at one token per sequence, and to the
invariance of causal attention under splitting a chunk.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import pa_oracle as O


def _case(**kw):
    base = dict(seed=21, dtype=np.float32, context_lens=[5, 17, 40, 9], query_lens=[5, 3, 16, 1],
                num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4, sigma=1.0)
    base.update(kw)
    return W.make_prefill_case(**base)


def _pools(case):
    kc, vc = O.cache_write(case.prefix_k, case.prefix_v, case.prefix_slots, case.empty_pool(),
                           case.empty_pool(), case.block_size)
    return O.cache_write(case.new_k, case.new_v, case.new_slots, kc, vc, case.block_size)


def _oracle(case, kc=None, vc=None, context_lens=None, query_start=None, q=None):
    if kc is None:
        kc, vc = _pools(case)
    return O.prefill(case.q if q is None else q, kc, vc, case.block_tables,
                     case.context_lens if context_lens is None else context_lens,
                     case.query_start if query_start is None else query_start, case.scale,
                     case.block_size, case.num_kv_heads)


def _dense_kv(case, s):
    """Sequence s's K/V in logical order: the stored prefix, then the chunk."""
    qs = case.query_start
    n, ctx = int(qs[s + 1] - qs[s]), int(case.context_lens[s])
    before = int(sum(int(case.context_lens[j]) - int(qs[j + 1] - qs[j]) for j in range(s)))
    k = np.concatenate([case.prefix_k[before:before + ctx - n], case.new_k[qs[s]:qs[s + 1]]])
    v = np.concatenate([case.prefix_v[before:before + ctx - n], case.new_v[qs[s]:qs[s + 1]]])
    return k, v


def _sdpa(case, explicit_mask=True):
    """torch SDPA, float64, per sequence on its dense K/V with kv heads repeated G times."""
    group = case.num_q_heads // case.num_kv_heads
    out = np.zeros((case.total_q, case.num_q_heads, case.head_dim))
    for s in range(case.num_seqs):
        r0, r1 = int(case.query_start[s]), int(case.query_start[s + 1])
        n, ctx = r1 - r0, int(case.context_lens[s])
        if n == 0:
            continue
        k, v = _dense_kv(case, s)
        kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(group, 0)
        vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(group, 0)
        qt = torch.from_numpy(case.q[r0:r1].astype(np.float64)).permute(1, 0, 2)  # [Hq, n, D]
        if explicit_mask:  # query i sees keys j <= ctx - n + i (the bottom-right diagonal)
            mask = torch.arange(ctx)[None, :] <= (ctx - n + torch.arange(n))[:, None]
            o = torch.nn.functional.scaled_dot_product_attention(
                qt.unsqueeze(0), kt.unsqueeze(0).contiguous(), vt.unsqueeze(0).contiguous(),
                attn_mask=mask, scale=case.scale)
        else:  # whole prompt: n == ctx, the library's own causal mask
            assert n == ctx
            o = torch.nn.functional.scaled_dot_product_attention(
                qt.unsqueeze(0), kt.unsqueeze(0).contiguous(), vt.unsqueeze(0).contiguous(),
                is_causal=True, scale=case.scale)
        out[r0:r1] = o[0].permute(1, 0, 2).numpy()
    return out


# --------------------------------------------------------------------- PF1
def test_pf1_one_token_per_sequence_is_decode():
    """With n = 1 the chunk is a decode step: equal, bit for bit, to the pinned decode."""
    case = _case(context_lens=[1, 7, 33, 64], query_lens=[1, 1, 1, 1], block_size=8)
    kc, vc = _pools(case)
    got = _oracle(case, kc, vc)
    want = O.decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale,
                    case.block_size, case.num_kv_heads)
    assert got.tobytes() == want.tobytes()


# --------------------------------------------------------------------- PF2
@pytest.mark.parametrize("kw", [
    dict(context_lens=[1, 6, 31], query_lens=[1, 6, 31]),
    dict(dtype=np.float16, num_q_heads=8, num_kv_heads=2, head_dim=16, block_size=16,
         context_lens=[64, 17], query_lens=[64, 17]),
])
def test_pf2_whole_prompt_equals_causal_sdpa(kw):
    case = _case(**kw)
    np.testing.assert_allclose(_oracle(case), _sdpa(case, explicit_mask=False), rtol=0, atol=1e-12)


# --------------------------------------------------------------------- PF3
@pytest.mark.parametrize("kw", [
    dict(),
    dict(dtype=np.float16, num_q_heads=12, num_kv_heads=3, head_dim=32, block_size=8,
         context_lens=[100, 3, 70, 16], query_lens=[37, 0, 70, 15]),
    dict(num_q_heads=2, num_kv_heads=2, head_dim=64, block_size=32, context_lens=[200],
         query_lens=[65]),
])
def test_pf3_chunk_equals_masked_sdpa(kw):
    case = _case(**kw)
    np.testing.assert_allclose(_oracle(case), _sdpa(case), rtol=0, atol=1e-12)


# --------------------------------------------------------------------- PF4
def test_pf4_brute_force_tiny():
    case = _case(context_lens=[6, 4], query_lens=[3, 4], head_dim=4, num_q_heads=4,
                 num_kv_heads=1, block_size=2)
    got = _oracle(case)
    group = case.num_q_heads // case.num_kv_heads
    for s in range(case.num_seqs):
        k, v = _dense_kv(case, s)
        r0 = int(case.query_start[s])
        n, ctx = int(case.query_start[s + 1]) - r0, int(case.context_lens[s])
        for i in range(n):
            for h in range(case.num_q_heads):
                kvh = h // group
                z = [case.scale * math.fsum(float(case.q[r0 + i, h, d]) * float(k[t, kvh, d])
                                            for d in range(case.head_dim))
                     for t in range(ctx - n + i + 1)]
                mx = max(z)
                e = [math.exp(x - mx) for x in z]
                den = math.fsum(e)
                for d in range(case.head_dim):
                    want = math.fsum(e[t] * float(v[t, kvh, d]) for t in range(len(e))) / den
                    assert abs(got[r0 + i, h, d] - want) <= 1e-12


# --------------------------------------------------------------------- PF5
@pytest.mark.parametrize("cut", [1, 7, 15])
def test_pf5_splitting_a_chunk_changes_nothing(cut):
    """Rows of one 16-token chunk equal those of two chunks (cut, 16 - cut) processed in turn,
    the first with the context ending at its own last token."""
    case = _case(context_lens=[40], query_lens=[16], block_size=4)
    kc, vc = _pools(case)
    whole = _oracle(case, kc, vc)
    first = _oracle(case, kc, vc, context_lens=np.array([40 - (16 - cut)], np.int32),
                    query_start=np.array([0, cut], np.int32), q=case.q[:cut])
    second = _oracle(case, kc, vc, query_start=np.array([0, 16 - cut], np.int32), q=case.q[cut:])
    assert first.tobytes() == whole[:cut].tobytes()
    assert second.tobytes() == whole[cut:].tobytes()


# --------------------------------------------------------------------- PF6
def test_pf6_empty_and_invalid_chunks():
    case = _case(context_lens=[5, 3, 8], query_lens=[2, 0, 3])
    kc, vc = _pools(case)
    got = _oracle(case, kc, vc)
    assert got.shape == (5, case.num_q_heads, case.head_dim) and np.all(np.isfinite(got))
    bad = _oracle(case, kc, vc, context_lens=np.array([1, 3, 8], np.int32))  # 2 tokens, ctx 1
    assert np.all(np.isnan(bad[:2])) and np.array_equal(bad[2:], got[2:])


def test_pf6_first_token_of_a_prompt_returns_its_v():
    """Position 0 sees only itself: its output is its own V row (closed form)."""
    case = _case(context_lens=[9, 12], query_lens=[9, 12])
    got = _oracle(case)
    group = case.num_q_heads // case.num_kv_heads
    for s in range(case.num_seqs):
        r0 = int(case.query_start[s])
        for h in range(case.num_q_heads):
            np.testing.assert_array_equal(got[r0, h], case.new_v[r0, h // group].astype(np.float64))


# --------------------------------------------------------------------- planted mistakes
@pytest.mark.parametrize("mutant", [
    lambda ctx, n, i: ctx - n + i,      # the query's own key left out
    lambda ctx, n, i: i + 1,            # mask aligned to the top left (ignores the cached prefix)
    lambda ctx, n, i: ctx,              # no causal mask
    lambda ctx, n, i: ctx - n + i + 2 if ctx - n + i + 2 <= ctx else ctx,  # one key too many
])
def test_planted_causal_mistakes_are_caught(monkeypatch, mutant):
    case = _case()
    monkeypatch.setattr(O, "visible_keys", mutant)
    with pytest.raises((AssertionError, ValueError)):  # ValueError: a row left with no key
        np.testing.assert_allclose(_oracle(case), _sdpa(case), rtol=0, atol=1e-9)
