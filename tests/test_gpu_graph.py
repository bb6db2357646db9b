"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph over the library's launches).

A serving loop replays one captured step per iteration, which takes the host's launch work
out of the step.  The library's launches record no memset and allocate nothing, so a
capture holds exactly its kernels.  Each captured call is replayed several times, with
eager work and synchronisations between the replays and new inputs copied into the
captured tensors, and every replay must equal the eager call on the same inputs bit for
bit (pools included).
"""
import numpy as np
import pytest

import paged_kv_cache_167_amd as P
import workloads as W
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _capture(fn):
    torch = _torch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture (the library memoises occupancy queries here)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _bits(t):
    torch = _torch()
    return t.view(torch.uint8) if t.dtype == torch.uint8 else t.view(torch.int16)


@pytest.mark.parametrize("kind", ["append", "fp8_append", "decode"])
def test_replays_equal_eager_calls(kind):
    torch = _torch()
    case = W.make_case(seed=71, dtype=np.float16, context_lens=[1, 17, 300, 1025, 2049, 4000],
                       num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, sigma=0.5)
    d = G.to_device(case, write_new=kind == "decode")
    mcl = case.max_context_len
    ks = vs = 0.05
    if kind == "fp8_append":
        from tests import test_gpu_fp8 as F
        kc = torch.from_numpy(F._empty_codes(case)).cuda()
        vc = kc.clone()
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        P.pa_cache_write_fp8(t(case.prefix_k), t(case.prefix_v), t(case.prefix_slots), kc, vc, ks, vs)
    else:
        kc, vc = d.k_cache, d.v_cache
    q = d.q.clone()
    k_new, v_new = d.new_k.clone(), d.new_v.clone()
    out = torch.empty_like(q)
    ws = torch.empty(max(P.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                                     case.head_dim, mcl), 256), dtype=torch.uint8, device="cuda")

    def step(o, qq, kk, vv, kcache, vcache):
        if kind == "append":
            P.pa_decode_append(o, qq, kk, vv, kcache, vcache, d.tables, d.ctx, case.scale, case.block_size,
                               case.num_kv_heads, max_context_len=mcl, workspace=ws)
        elif kind == "fp8_append":
            P.pa_decode_fp8_append(o, qq, kk, vv, kcache, vcache, d.tables, d.ctx, case.scale, ks, vs,
                                   case.block_size, case.num_kv_heads, max_context_len=mcl, workspace=ws)
        else:
            P.pa_decode(o, qq, kcache, vcache, d.tables, d.ctx, case.scale, case.block_size,
                        case.num_kv_heads, max_context_len=mcl, workspace=ws)

    graph = _capture(lambda: step(out, q, k_new, v_new, kc, vc))
    rng = np.random.default_rng(5)
    for r in range(4):
        # new inputs into the captured tensors, by eager kernels, then a synchronisation
        q.copy_(torch.from_numpy(rng.standard_normal(q.shape).astype(np.float16)).cuda())
        k_new.copy_(torch.from_numpy(rng.standard_normal(k_new.shape).astype(np.float16)).cuda())
        v_new.copy_(torch.from_numpy(rng.standard_normal(v_new.shape).astype(np.float16)).cuda())
        torch.cuda.synchronize()
        # eager reference on copies of everything the step reads or writes
        ref = torch.empty_like(out)
        rkc, rvc = kc.clone(), vc.clone()
        step(ref, q, k_new, v_new, rkc, rvc)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == ref.cpu().numpy().tobytes(), f"{kind}: replay {r}"
        assert torch.equal(_bits(kc), _bits(rkc)) and torch.equal(_bits(vc), _bits(rvc)), f"{kind}: pools {r}"
