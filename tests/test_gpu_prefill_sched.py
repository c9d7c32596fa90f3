"""GPU parity of the scheduled prefill calls (mla_latent_attn_prefill_chunk_sched
and its paged form): persistent workgroups take the chunk's query blocks from
a counter in caller memory. Every block is computed exactly as by the
per-block kernel, so the outputs must be bitwise equal to the plain calls
(which the other prefill tests check against the oracle), the counter must be
zero after every call, and one counter must serve consecutive calls and
graph replays."""
import numpy as np
import pytest
import torch

import lca_inputs as li
import mla_latent_kv_lca_amd as lca
from oracle import lca_oracle as O
from tests.gpu_util import assert_close, dev, host, packed
from tests.test_gpu_parity import _page_pool

pytestmark = pytest.mark.gpu


def _dense_inputs(seed, Hq, m, raw_begin, s0, C):
    L = s0 + C
    c, kr = li.latent_cache(400 + seed, 1, L)
    li.plant_needles(400 + seed, c, kr, min(2, L - raw_begin), 14.0, raw_begin, L)
    rc, rk = li.latent_cache(500 + seed, 1, max(m, 1))
    q = li.queries(400 + seed, 1, C, Hq, rho=0.5)[0]
    return c, kr, rc, rk, q


# (seed, Hq, m, raw_begin, s0, C, bf16_out, q_dtype): 263 blocks of 8 tokens (more blocks
# than persistent workgroups, ragged last block), grouped-query heads, two head
# groups, fewer blocks than workgroups, and Hg = 8 with f32 queries
SHAPES = [(0, 16, 300, 4800, 5000, 2100, True, torch.bfloat16), (1, 4, 0, 0, 0, 1000, False, torch.bfloat16),
          (2, 32, 50, 900, 1000, 700, True, torch.bfloat16), (3, 16, 20, 350, 370, 9, False, torch.bfloat16),
          (4, 8, 64, 2000, 2048, 1531, True, torch.float32)]


@pytest.mark.parametrize("seed,Hq,m,raw_begin,s0,C,bf16_out,q_dtype", SHAPES)
def test_prefill_sched_equals_per_block_kernel(seed, Hq, m, raw_begin, s0, C, bf16_out, q_dtype):
    c, kr, rc, rk, q = _dense_inputs(seed, Hq, m, raw_begin, s0, C)
    cache_t = packed(c, kr)[0]
    reps_t = packed(rc[:, :m], rk[:, :m])[0] if m else None
    rl = lca.packed_latent(reps_t) if m else None
    odt = torch.bfloat16 if bf16_out else torch.float32
    q_t = dev(q, q_dtype)
    ref = torch.empty((C, Hq, 512), dtype=odt, device="cuda")
    ref_lse = torch.empty((C, Hq), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_prefill_chunk(q_t, s0, rl, m, lca.packed_latent(cache_t), raw_begin, 1.0, ref, ref_lse)
    sched = lca.prefill_sched()
    for call in range(3):  # one counter for consecutive calls
        out = torch.full((C, Hq, 512), float("nan"), dtype=odt, device="cuda")
        lse = torch.full((C, Hq), float("nan"), dtype=torch.float32, device="cuda")
        lca.mla_latent_attn_prefill_chunk(q_t, s0, rl, m, lca.packed_latent(cache_t), raw_begin, 1.0, out, lse,
                                          sched=sched)
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), f"call {call}: scheduled output differs"
        assert sched.tolist() == [0, 0], f"call {call}: counter left at {sched.tolist()}"
    if seed == 0:  # and the oracle, on the scheduled output
        ro, rlse = O.prefill_chunk(q, s0, rc[0, :m], rk[0, :m], m, c[0], kr[0], raw_begin, 1.0)
        assert_close(host(out), ro, what="scheduled prefill o_latent")
        assert_close(host(lse), rlse, what="scheduled prefill lse")


def test_prefill_sched_graph_replays():
    """A graph holding two scheduled chunk calls that share one counter,
    replayed three times with eager work in between: every replay gives the
    eager outputs and leaves the counter zeroed."""
    seed, Hq, m, raw_begin, s0, C = 5, 16, 120, 2000, 2100, 1500
    c, kr, rc, rk, q = _dense_inputs(seed, Hq, m, raw_begin, s0, C)
    cache_l = lca.packed_latent(packed(c, kr)[0])
    reps_l = lca.packed_latent(packed(rc[:, :m], rk[:, :m])[0])
    q_t = dev(q)
    half = C // 2
    ref = torch.empty((C, Hq, 512), dtype=torch.bfloat16, device="cuda")
    lca.mla_latent_attn_prefill_chunk(q_t[:half], s0, reps_l, m, cache_l, raw_begin, 1.0, ref[:half])
    lca.mla_latent_attn_prefill_chunk(q_t[half:], s0 + half, reps_l, m, cache_l, raw_begin, 1.0, ref[half:])
    sched = lca.prefill_sched()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            lca.mla_latent_attn_prefill_chunk(q_t[:half], s0, reps_l, m, cache_l, raw_begin, 1.0, out[:half],
                                              sched=sched)
            lca.mla_latent_attn_prefill_chunk(q_t[half:], s0 + half, reps_l, m, cache_l, raw_begin, 1.0,
                                              out[half:], sched=sched)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}: output differs"
        assert sched.tolist() == [0, 0], f"replay {rep}: counter left at {sched.tolist()}"


@pytest.mark.parametrize("page_rows,Hh", [(16, 16), (64, 4)])
def test_prefill_paged_sched_equals_paged(page_rows, Hh):
    """The paged call on shuffled pages, scheduled and per-block, on chunks
    with ragged starts of two sequences sharing one pool and one counter."""
    Ls, w, g = [2600, 1900], 256, 16
    cs, ks, qs = [], [], []
    for b, L in enumerate(Ls):
        c, kr = li.latent_cache(60 + b, 1, L)
        cs.append(c[0]); ks.append(kr[0])
        qs.append(li.queries(60 + b, 1, L, Hh, rho=0.5)[0])
    pool, table = _page_pool([np.concatenate([c, k], -1) for c, k in zip(cs, ks)], page_rows, 19)
    cache_all = lca.paged_latent(dev(pool), torch.from_numpy(table).cuda())
    sched = lca.prefill_sched()
    for b, L in enumerate(Ls):
        s0 = L - 1100 if b == 0 else 700
        C = L - s0
        m = O.prefill_plan(s0, w, g)
        rc, rk = li.latent_cache(70 + b, 1, max(m, 1))
        reps_l = lca.packed_latent(packed(rc[:, :m], rk[:, :m])[0]) if m else None
        q_t = dev(qs[b][s0:])
        outs = []
        for sc in (None, sched):
            out = torch.full((C, Hh, 512), float("nan"), dtype=torch.float32, device="cuda")
            lse = torch.full((C, Hh), float("nan"), dtype=torch.float32, device="cuda")
            lca.mla_latent_attn_prefill_chunk_paged(q_t, s0, reps_l, m, cache_all, b, m * g, 1.0, out, lse, sched=sc)
            outs.append((out, lse))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), f"seq {b} differs"
        assert sched.tolist() == [0, 0]
