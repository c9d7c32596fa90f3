"""GPU parity: every kernel through the C ABI against the fp64 oracle.

Inputs come from lca_inputs (seeded, bf16-rounded on the host); expected
values come only from the oracle. Downstream stages are fed the GPU's own
condensed cache, so a legitimate near-tie anchor cannot cascade.
"""
import numpy as np
import pytest
import torch

import lca_inputs as li
import mla_latent_kv_lca_amd as lca
from oracle import lca_oracle as O
from tests.gpu_util import TOL, AnchorTally, anchors_agree, assert_close, dev, host, packed

pytestmark = pytest.mark.gpu

H = 16


def _condense_gpu(cache_t, B, g, gb, n, q_t, r0, step, sm, m_cap, rep_dtype=None, mode=lca.LCA_MODE_LCA):
    rep_dtype = rep_dtype or cache_t.dtype
    reps = torch.zeros((B, m_cap, 576), dtype=rep_dtype, device="cuda")
    anchor = torch.full((B, m_cap), -1, dtype=torch.int32, device="cuda")
    alpha = torch.zeros((B, m_cap, g), dtype=torch.float32, device="cuda")
    lca.lca_condense(lca.packed_latent(cache_t), B, g, gb, n, q_t, r0, step, sm,
                     lca.packed_latent(reps), anchor, alpha, mode=mode)
    return reps, anchor, alpha


@pytest.mark.parametrize("mode,dtype,g,step", [(lca.LCA_MODE_POOL_ROPE, torch.bfloat16, 16, 0),
                                               (lca.LCA_MODE_POOL_ROPE, torch.float32, 8, 8),
                                               (lca.LCA_MODE_ANCHOR, torch.bfloat16, 16, 0),
                                               (lca.LCA_MODE_ANCHOR, torch.float32, 4, 4)])
def test_condense_ablation_modes_match_oracle(mode, dtype, g, step):
    """The ablation variants (pooled RoPE keys; anchor row only) against the oracle's modes."""
    B, L, w = 2, 2600, 1024
    bf = dtype == torch.bfloat16
    c, kr = li.latent_cache(4, B, L, bf16=bf)
    m = O.plan(L, w, g)["m"]
    T = (m - 1) * step + g
    q = li.queries(4, B, T, H, rho=0.5, bf16=bf)
    reps, anchor, alpha = _condense_gpu(packed(c, kr, dtype), B, g, 0, m, dev(q, dtype), 0, step, 1.0, m,
                                        mode=mode)
    torch.cuda.synchronize()
    rc, rk, ra, ralpha, s = O.condense(c, kr, q, g, 0, m, 0, step, 1.0, mode)
    r = host(reps)
    assert_close(host(alpha), ralpha, tol=1e-5, what="alpha")
    ga = host(anchor).astype(np.int64)
    n_sure = anchors_agree(ga, ra, O.top2_margin(s))
    assert n_sure > 0.5 * B * m
    if mode == lca.LCA_MODE_ANCHOR:
        # the representative is the anchor row itself, bit for bit
        for b in range(B):
            np.testing.assert_array_equal(r[b, :, :512], c[b, ga[b]].astype(np.float64))
            np.testing.assert_array_equal(r[b, :, 512:], kr[b, ga[b]].astype(np.float64))
    else:
        assert_close(r[..., :512], rc, what="rep c_KV")
        assert_close(r[..., 512:], rk, what="pooled rep k_R")


@pytest.mark.parametrize("dtype,rho", [(torch.bfloat16, 0.5), (torch.float32, 0.5), (torch.bfloat16, 0.0)])
def test_condense_matches_oracle(dtype, rho):
    B, L, g, w = 2, 2048, 16, 1024
    bf = dtype == torch.bfloat16
    c, kr = li.latent_cache(1, B, L, bf16=bf)
    q = li.queries(1, B, 16, H, rho=rho, bf16=bf)
    m = O.plan(L, w, g)["m"]
    reps, anchor, alpha = _condense_gpu(packed(c, kr, dtype), B, g, 0, m, dev(q, dtype), 0, 0, 1.0, m)
    torch.cuda.synchronize()
    rc, rk, ra, ralpha, s = O.condense(c, kr, q, g, 0, m, 0, 0, 1.0)
    r = host(reps)
    assert_close(r[..., :512], rc, what="rep c_KV")
    assert_close(host(alpha), ralpha, tol=1e-5, what="alpha")
    np.testing.assert_allclose(host(alpha).sum(-1), 1.0, atol=1e-6)
    n_sure = anchors_agree(host(anchor).astype(np.int64), ra, O.top2_margin(s))
    assert n_sure > 0.5 * B * m
    # the anchor's k_R is copied exactly from the cache row it names
    ga = host(anchor).astype(np.int64)
    for b in range(B):
        np.testing.assert_array_equal(r[b, :, 512:], kr[b, ga[b]].astype(np.float64))


def test_condense_per_group_summary_queries_prefill_style():
    """Chunked-prefill addressing: group j uses the g queries after it."""
    B, L, g = 1, 640, 16
    c, kr = li.latent_cache(4, B, L)
    q = li.queries(4, B, L, H, rho=0.5)
    gb, n = 5, 20
    reps, anchor, alpha = _condense_gpu(packed(c, kr), B, g, gb, n, dev(q), (gb + 1) * g, g, 0.7, gb + n)
    torch.cuda.synchronize()
    rc, rk, ra, ralpha, s = O.condense(c, kr, q, g, gb, n, (gb + 1) * g, g, 0.7)
    r = host(reps)
    assert not r[:, :gb].any(), "rows before group_begin must stay untouched"
    assert_close(r[0, gb:, :512], rc[0], what="rep c_KV")
    assert_close(host(alpha)[0, gb:], ralpha[0], tol=1e-5, what="alpha")
    anchors_agree(host(anchor)[0, gb:].astype(np.int64), ra[0], O.top2_margin(s[0]))


@pytest.mark.parametrize("n_kv,Hq", [(2, 32), (8, 32), (2, 16), (8, 16), (16, 16)])  # Hg = 16, 4, 8, 2, 1
def test_gqa_condense_and_decode_match_oracle(n_kv, Hq):
    """GQA reading (n_kv latent caches, query heads grouped per cache) through
    the existing entry points on B * n_kv sequences of Hg = Hq / n_kv heads,
    against the oracle's GQA condensation and decode; then the per-head W_UV
    up-projection of the decode output over all Hq query heads."""
    B, L, g, w = 2, 2600, 16, 1024
    Hg = Hq // n_kv
    c, kr = li.latent_cache(8, B * n_kv, L)
    li.plant_needles(8, c, kr, 2, 14.0, 0, L)
    q = li.queries(8, B, g, Hq, rho=0.5)
    qd = li.queries(8, B, 1, Hq, rho=0.5, stream=1)[:, 0]
    wuv = li.w_uv(8, Hq)
    m = O.plan(L, w, g)["m"]
    cache = packed(c, kr, torch.bfloat16)                      # [B * n_kv, L, 576]
    reps, anchor, alpha = _condense_gpu(cache, B * n_kv, g, 0, m, lca.gqa_sequences(dev(q), n_kv), 0, 0, 1.0, m)
    o = torch.empty((B * n_kv, Hg, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B * n_kv, Hg), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_decode(dev(qd).view(B * n_kv, Hg, 576), lca.packed_latent(reps), m,
                               lca.packed_latent(cache), m * g, L, 1.0, o, lse)
    y = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lca.mla_up_proj(o.view(B, Hq, 512), dev(wuv), y)         # kv-major heads are the query heads in order
    torch.cuda.synchronize()
    c4, k4 = c.reshape(B, n_kv, L, 512), kr.reshape(B, n_kv, L, 64)
    rc, rk, ra, ralpha, s = O.condense_gqa(c4, k4, q, n_kv, g, 0, m, 0, 0, 1.0)
    r = host(reps).reshape(B, n_kv, m, 576)
    assert_close(r[..., :512], rc, what="GQA rep c_KV")
    assert_close(host(alpha).reshape(B, n_kv, m, g), ralpha, tol=1e-5, what="GQA alpha")
    ga = host(anchor).astype(np.int64).reshape(B, n_kv, m)
    anchors_agree(ga.reshape(-1, m), ra.reshape(-1, m), O.top2_margin(s.reshape(-1, m, g)))
    ro, rl = O.decode_gqa(qd, r[..., :512], r[..., 512:], m, c4, k4, m * g, L, n_kv, 1.0)
    assert_close(host(o).reshape(B, Hq, 512), ro, what="GQA o_latent")
    assert_close(host(lse).reshape(B, Hq), rl, what="GQA lse")
    assert_close(host(y), O.up_proj(ro, wuv), what="GQA up-projected output")


@pytest.mark.parametrize("n_kv,Hq,L,C", [(4, 16, 700, 256), (8, 8, 300, 128), (8, 16, 400, 200), (2, 16, 500, 160)])  # Hg = 4, 1, 2, 8
def test_gqa_prefill_matches_oracle(n_kv, Hq, L, C):
    """GQA chunked prefill: per key-value head k, its cache condensed with its
    own Hg query heads (the g queries after each group) and its Hg heads'
    queries attending it chunk by chunk (query token stride Hq * 576), against
    the oracle's prefill of that group's heads on that cache."""
    w, g, sm = 128, 16, 1.0
    Hg = Hq // n_kv
    c, kr = li.latent_cache(16, n_kv, L)
    li.plant_needles(16, c, kr, 3, 14.0, 0, L)
    q = li.queries(16, 1, L, Hq, rho=0.5)[0]                 # [L, Hq, 576]
    q_t = dev(q)
    m_cap = max(O.prefill_plan(((L - 1) // C) * C, w, g), 1)
    for k in range(n_kv):
        cache_k = packed(c[k], kr[k])
        qk = q_t[:, k * Hg:(k + 1) * Hg]                      # token stride Hq * 576, heads contiguous
        reps = torch.zeros((m_cap, 576), dtype=torch.bfloat16, device="cuda")
        anchor = torch.zeros((1, m_cap), dtype=torch.int32, device="cuda")
        out = torch.empty((L, Hg, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((L, Hg), dtype=torch.float32, device="cuda")
        m = 0
        for s0 in range(0, L, C):
            ms = O.prefill_plan(s0, w, g)
            if ms > m:
                lca.lca_condense(lca.packed_latent(cache_k[None]), 1, g, m, ms - m, qk[None], (m + 1) * g, g, sm,
                                 lca.packed_latent(reps[None]), anchor)
                m = ms
            e = min(L, s0 + C)
            lca.mla_latent_attn_prefill_chunk(qk[s0:e], s0, lca.packed_latent(reps) if m else None, m,
                                              lca.packed_latent(cache_k), m * g, sm, out[s0:e], lse[s0:e])
        torch.cuda.synchronize()
        ro, rl, rep_c, rep_k = O.prefill(q[:, k * Hg:(k + 1) * Hg], c[k], kr[k], w, g, C, sm)
        r = host(reps)[:len(rep_c)]
        assert_close(r[:, :512], rep_c, what=f"GQA prefill reps, kv head {k}")
        # attention checked on the GPU's own representatives
        go = np.zeros_like(ro)
        gl = np.zeros_like(rl)
        for s0 in range(0, L, C):
            ms = O.prefill_plan(s0, w, g)
            e = min(L, s0 + C)
            go[s0:e], gl[s0:e] = O.prefill_chunk(q[s0:e, k * Hg:(k + 1) * Hg], s0, r[:, :512], r[:, 512:], ms,
                                                 c[k], kr[k], ms * g, sm)
        assert_close(host(out), go, what=f"GQA prefill o_latent, kv head {k}")
        assert_close(host(lse), gl, what=f"GQA prefill lse, kv head {k}")


def _page_pool(seqs, page_rows, seed):
    """Scatter each sequence's packed rows [L_b, 576] over shuffled pages of a
    pool; returns (pool [n_pages, page_rows, 576], block table int32 [B, n])."""
    r = np.random.default_rng(seed)
    need = [-(-len(x) // page_rows) for x in seqs]
    order = r.permutation(sum(need))
    pool = np.zeros((sum(need), page_rows, 576), dtype=np.float32)
    table = np.zeros((len(seqs), max(need)), dtype=np.int32)
    k = 0
    for b, x in enumerate(seqs):
        for j in range(need[b]):
            pg = order[k]
            k += 1
            table[b, j] = pg
            rows = x[j * page_rows:(j + 1) * page_rows]
            pool[pg, :len(rows)] = rows
    return pool, table


@pytest.mark.parametrize("page_rows,g,q_dtype,Hh", [(64, 16, torch.bfloat16, 16), (16, 8, torch.bfloat16, 16),
                                                    (64, 16, torch.float32, 16), (64, 16, torch.bfloat16, 4),
                                                    (16, 16, torch.bfloat16, 1)])
def test_decode_paged_ragged_matches_oracle(page_rows, g, q_dtype, Hh):
    """Ragged batch (different lengths, one shorter than the window) over a
    shuffled paged cache against the oracle on each sequence's logical rows.
    With g = 8 the raw ranges start off a 16-row boundary, so tiles straddle
    pages. Hh = 4 and 1: one key-value group of grouped-query attention per
    sequence (reading R8)."""
    H = Hh
    Ls, w = [1500, 2077, 3000, 1040, 777], 1024
    B = len(Ls)
    seqs, reps, ms, rbs = [], [], [], []
    for b, L in enumerate(Ls):
        c, kr = li.latent_cache(20 + b, 1, L)
        li.plant_needles(20 + b, c, kr, 2, 14.0, 0, L)
        seqs.append(np.concatenate([c[0], kr[0]], -1))
        p = O.plan(L, w, g)
        ms.append(p["m"])
        rbs.append(p["raw_begin"])
        rc, rk = li.latent_cache(40 + b, 1, max(p["m"], 1))
        reps.append(np.concatenate([rc[0], rk[0]], -1)[:p["m"]])
    pool, table = _page_pool(seqs, page_rows, 7)
    m_cap = max(max(ms), 1)
    reps_t = torch.zeros((B, m_cap, 576), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        if ms[b]:
            reps_t[b, :ms[b]] = dev(reps[b])
    q = li.queries(9, B, 1, H, rho=0.5)[:, 0]
    pool_t = dev(pool)
    table_t = torch.from_numpy(table).cuda()
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")  # noqa: E731
    o = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    max_entries = max(m + L - rb for m, L, rb in zip(ms, Ls, rbs))
    lca.mla_latent_attn_decode_paged(dev(q, q_dtype), lca.packed_latent(reps_t), i32(ms), lca.paged_latent(pool_t, table_t),
                                     i32(rbs), i32(Ls), max_entries, 1.0, o, lse)
    torch.cuda.synchronize()
    for b in range(B):
        x = seqs[b][None]
        rep = reps[b][None] if ms[b] else None
        ro, rl = O.decode(q[b:b + 1], None if rep is None else rep[..., :512], None if rep is None else rep[..., 512:],
                          ms[b], x[..., :512], x[..., 512:], rbs[b], Ls[b], 1.0)
        assert_close(host(o[b:b + 1]), ro, what=f"paged o_latent seq {b}")
        assert_close(host(lse[b:b + 1]), rl, what=f"paged lse seq {b}")


def test_condense_and_decode_paged_ragged_end_to_end():
    """Ragged batch over shuffled pages: lca_condense_paged against the oracle
    per sequence, then mla_latent_attn_decode_paged over the GPU's own
    representatives against the oracle's decode."""
    Ls, g, w, P = [1500, 2077, 3000, 1040, 777, 2600], 16, 1024, 64
    B = len(Ls)
    cs, ks = [], []
    for b, L in enumerate(Ls):
        c, kr = li.latent_cache(60 + b, 1, L)
        li.plant_needles(60 + b, c, kr, 2, 14.0, 0, L)
        cs.append(c[0])
        ks.append(kr[0])
    pool, table = _page_pool([np.concatenate([c, k], -1) for c, k in zip(cs, ks)], P, 11)
    plans = [O.plan(L, w, g) for L in Ls]
    ms = [p["m"] for p in plans]
    m_cap = max(ms)
    qh = li.queries(61, B, g, H, rho=0.5)
    qd = li.queries(61, B, 1, H, rho=0.5, stream=1)[:, 0]
    pool_t, table_t = dev(pool), torch.from_numpy(table).cuda()
    cache = lca.paged_latent(pool_t, table_t)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")  # noqa: E731
    reps = torch.zeros((B, m_cap, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.full((B, m_cap), -1, dtype=torch.int32, device="cuda")
    alpha = torch.zeros((B, m_cap, g), dtype=torch.float32, device="cuda")
    lca.lca_condense_paged(cache, B, g, i32([0] * B), i32(ms), m_cap, dev(qh), 0, 1.0,
                           lca.packed_latent(reps), anchor, alpha)
    o = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    rbs = [p["raw_begin"] for p in plans]
    lca.mla_latent_attn_decode_paged(dev(qd), lca.packed_latent(reps), i32(ms), cache, i32(rbs), i32(Ls),
                                     max(p["n_entries"] for p in plans), 1.0, o, lse)
    torch.cuda.synchronize()
    r, ga = host(reps), host(anchor).astype(np.int64)
    tally = AnchorTally()
    for b in range(B):
        m = ms[b]
        if m:
            rc, rk, ra, ralpha, s = O.condense(cs[b][None], ks[b][None], qh[b:b + 1], g, 0, m, 0, 0, 1.0)
            assert_close(r[b, :m, :512], rc[0], what=f"paged rep c_KV seq {b}")
            assert_close(host(alpha[b, :m]), ralpha[0], tol=1e-5, what=f"paged alpha seq {b}")
            tally.add(ga[b, :m], ra[0], O.top2_margin(s[0]))
            np.testing.assert_array_equal(r[b, :m, 512:], ks[b][ga[b, :m]].astype(np.float64))
        ro, rl = O.decode(qd[b:b + 1], r[b:b + 1, :m, :512] if m else None, r[b:b + 1, :m, 512:] if m else None, m,
                          cs[b][None], ks[b][None], rbs[b], Ls[b], 1.0)
        assert_close(host(o[b:b + 1]), ro, what=f"paged decode seq {b}")
        assert_close(host(lse[b:b + 1]), rl, what=f"paged lse seq {b}")
    tally.check()


@pytest.mark.parametrize("page_rows,Hh", [(16, 16), (64, 16), (64, 4)])
def test_prefill_paged_ragged_end_to_end(page_rows, Hh):
    """Chunked prefill of three sequences of different lengths over shuffled
    pages: before each chunk (ragged chunk starts) the groups that left the
    window are condensed through lca_condense_paged with the g queries that
    follow each group, then mla_latent_attn_prefill_chunk_paged attends the
    chunk. Representatives against the oracle's condensation; attention
    against the oracle on the GPU's representatives, and bitwise against the
    dense prefill call on the same rows. Hh = 4: one key-value group of
    grouped-query attention (8 tokens x 4 heads per 32-row block)."""
    Ls, w, g, sm = [1500, 2300, 900], 256, 16, 1.0
    bounds = {0: [0, 300, 700, 1100, 1500], 1: [0, 500, 650, 1400, 2300], 2: [0, 257, 900]}
    B, H = len(Ls), Hh
    cs, ks, qs = [], [], []
    for b, L in enumerate(Ls):
        c, kr = li.latent_cache(30 + b, 1, L)
        li.plant_needles(30 + b, c, kr, 3, 14.0, 0, L)
        cs.append(c[0]); ks.append(kr[0])
        qs.append(li.queries(30 + b, 1, L, H, rho=0.5)[0])
    pool, table = _page_pool([np.concatenate([c, k], -1) for c, k in zip(cs, ks)], page_rows, 17)
    pool_t, table_t = dev(pool), torch.from_numpy(table).cuda()
    cache_all = lca.paged_latent(pool_t, table_t)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")  # noqa: E731
    tally = AnchorTally()
    for b, L in enumerate(Ls):
        q_t = dev(qs[b])
        m_cap = max(O.prefill_plan(bounds[b][-2], w, g), 1)
        reps = torch.zeros((1, m_cap, 576), dtype=torch.bfloat16, device="cuda")
        anchor = torch.full((1, m_cap), -1, dtype=torch.int32, device="cuda")
        out = torch.empty((L, H, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((L, H), dtype=torch.float32, device="cuda")
        cache_b = lca.paged_latent(pool_t, table_t[b:b + 1])   # this sequence's block-table row
        m = 0
        for s0, e in zip(bounds[b][:-1], bounds[b][1:]):
            ms = O.prefill_plan(s0, w, g)
            if ms > m:
                lca.lca_condense_paged(cache_b, 1, g, i32([m]), i32([ms - m]), ms - m, q_t[None], (m + 1) * g, sm,
                                       lca.packed_latent(reps), anchor, q_row_step=g)
                m = ms
            lca.mla_latent_attn_prefill_chunk_paged(q_t[s0:e], s0, lca.packed_latent(reps[0]) if m else None, m,
                                                    cache_all, b, m * g, sm, out[s0:e], lse[s0:e])
        # the dense call on the same rows and representatives
        dense = packed(cs[b], ks[b])
        out_d = torch.empty_like(out)
        lse_d = torch.empty_like(lse)
        for s0, e in zip(bounds[b][:-1], bounds[b][1:]):
            ms = O.prefill_plan(s0, w, g)
            lca.mla_latent_attn_prefill_chunk(q_t[s0:e], s0, lca.packed_latent(reps[0]) if ms else None, ms,
                                              lca.packed_latent(dense), ms * g, sm, out_d[s0:e], lse_d[s0:e])
        torch.cuda.synchronize()
        assert torch.equal(out, out_d) and torch.equal(lse, lse_d), f"paged and dense prefill differ (seq {b})"
        r = host(reps)[0]
        ga = host(anchor)[0].astype(np.int64)
        m_final = O.prefill_plan(bounds[b][-2], w, g)
        if m_final:
            rc, rk, ra, ralpha, sc = O.condense(cs[b][None], ks[b][None], qs[b][None], g, 0, m_final, g, g, sm)
            assert_close(r[:m_final, :512], rc[0], what=f"paged prefill reps seq {b}")
            tally.add(ga[:m_final], ra[0], O.top2_margin(sc[0]))
            np.testing.assert_array_equal(r[:m_final, 512:], ks[b][ga[:m_final]].astype(np.float64))
        for s0, e in zip(bounds[b][:-1], bounds[b][1:]):
            ms = O.prefill_plan(s0, w, g)
            ro, rl = O.prefill_chunk(qs[b][s0:e], s0, r[:, :512], r[:, 512:], ms, cs[b], ks[b], ms * g, sm)
            assert_close(host(out[s0:e]), ro, what=f"paged prefill o_latent seq {b} chunk {s0}")
            assert_close(host(lse[s0:e]), rl, what=f"paged prefill lse seq {b} chunk {s0}")
    tally.check()


def test_decode_paged_up_equals_paged_decode_then_up_proj():
    """Paged decode fused with W_UV: bitwise the paged decode followed by
    mla_up_proj, and the up-projected output against the oracle."""
    Ls, w, g, P = [1500, 2077, 3000, 1040, 777], 1024, 16, 64
    B = len(Ls)
    seqs, ms, rbs, reps = [], [], [], []
    for b, L in enumerate(Ls):
        c, kr = li.latent_cache(50 + b, 1, L)
        li.plant_needles(50 + b, c, kr, 2, 14.0, 0, L)
        seqs.append(np.concatenate([c[0], kr[0]], -1))
        p = O.plan(L, w, g)
        ms.append(p["m"]); rbs.append(p["raw_begin"])
        rc, rk = li.latent_cache(70 + b, 1, max(p["m"], 1))
        reps.append(np.concatenate([rc[0], rk[0]], -1)[:p["m"]])
    pool, table = _page_pool(seqs, P, 9)
    reps_t = torch.zeros((B, max(ms), 576), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        if ms[b]:
            reps_t[b, :ms[b]] = dev(reps[b])
    q = li.queries(51, B, 1, H, rho=0.5)[:, 0]
    wuv = li.w_uv(51, H)
    pool_t, table_t = dev(pool), torch.from_numpy(table).cuda()
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")  # noqa: E731
    max_entries = max(m + L - rb for m, L, rb in zip(ms, Ls, rbs))
    args = (dev(q), lca.packed_latent(reps_t), i32(ms), lca.paged_latent(pool_t, table_t), i32(rbs), i32(Ls),
            max_entries, 1.0)
    o1 = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    l1 = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_decode_paged(*args, o1, l1)
    y1 = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lca.mla_up_proj(o1, dev(wuv), y1)
    o2, l2, y2 = torch.empty_like(o1), torch.empty_like(l1), torch.empty_like(y1)
    lca.mla_latent_attn_decode_paged_up(*args, o2, dev(wuv), y2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(y1, y2)
    for b in range(B):
        x = seqs[b][None]
        rep = reps[b][None] if ms[b] else None
        ro, _ = O.decode(q[b:b + 1], None if rep is None else rep[..., :512], None if rep is None else rep[..., 512:],
                         ms[b], x[..., :512], x[..., 512:], rbs[b], Ls[b], 1.0)
        assert_close(host(y2[b:b + 1]), O.up_proj(ro, wuv), what=f"paged decode_up out seq {b}")


@pytest.mark.parametrize("B,L,g,with_alpha,Hq,q_dtype", [
    (3, 5000, 16, True, 16, torch.bfloat16), (2, 4100, 8, False, 16, torch.bfloat16),
    (1, 70000, 16, False, 16, torch.bfloat16),
    (2, 3000, 16, False, 32, torch.float32),    # 512 query rows per summary query, f32 queries
    (2, 3000, 16, False, 48, torch.bfloat16)])  # 768 query rows
def test_condense_streaming_kernel_equals_general_kernel(B, L, g, with_alpha, Hq, q_dtype):
    """Packed bf16 rows with one summary query per sequence take the streaming
    kernel; the same rows given as separate c_KV / k_R tensors (temporary
    copies, kept alive by the description) take the general kernel. Both must
    agree bit for bit (same arithmetic order), and with the oracle on sampled
    groups."""
    c, kr = li.latent_cache(15, B, L)
    li.plant_needles(15, c, kr, 3, 12.0, 0, L)
    q = li.queries(15, B, g, Hq, rho=0.5)
    m = (L - 64) // g
    cache_t = packed(c, kr)
    q_t = dev(q, q_dtype)
    outs = []
    for split in (False, True):
        reps = torch.zeros((B, m, 576), dtype=torch.bfloat16, device="cuda")
        anchor = torch.full((B, m), -1, dtype=torch.int32, device="cuda")
        alpha = torch.zeros((B, m, g), dtype=torch.float32, device="cuda") if with_alpha else None
        src = lca.latent(cache_t[..., :512].contiguous(), cache_t[..., 512:].contiguous()) if split \
            else lca.packed_latent(cache_t)
        lca.lca_condense(src, B, g, 0, m, q_t, 0, 0, 1.0, lca.packed_latent(reps), anchor, alpha)
        outs.append((reps, anchor, alpha))
    torch.cuda.synchronize()
    (r0, a0, al0), (r1, a1, al1) = outs
    assert torch.equal(r0, r1) and torch.equal(a0, a1)
    if with_alpha:
        assert torch.equal(al0, al1)
    r = host(r0)
    tally = AnchorTally()
    for b, j in zip(np.random.default_rng(3).integers(0, B, 24), np.random.default_rng(4).integers(0, m, 24)):
        rc, _, ra, _, sc = O.condense(c[b:b + 1], kr[b:b + 1], q[b:b + 1], g, int(j), 1, 0, 0, 1.0)
        assert_close(r[b, j, :512], rc[0, 0], what=f"rep ({b},{j})")
        tally.add(host(a0)[b, j:j + 1].astype(np.int64), ra[0], O.top2_margin(sc[0]))
    tally.check()


def test_condense_g1_copies_rows_exactly():
    B, L = 2, 100
    c, kr = li.latent_cache(5, B, L)
    q = li.queries(5, B, 1, H)
    reps, anchor, alpha = _condense_gpu(packed(c, kr), B, 1, 0, L, dev(q), 0, 0, 1.0, L)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(reps), np.concatenate([c, kr], -1).astype(np.float64))
    np.testing.assert_array_equal(host(anchor), np.tile(np.arange(L), (B, 1)))
    np.testing.assert_array_equal(host(alpha), 1.0)


def test_condense_identical_rows_pool_to_the_row():
    B, g = 1, 16
    c, kr = li.latent_cache(6, B, 4 * g)
    for j in range(4):  # every group is one row repeated
        c[0, j * g:(j + 1) * g] = c[0, j * g]
        kr[0, j * g:(j + 1) * g] = kr[0, j * g]
    q = li.queries(6, B, g, H, rho=0.5)
    reps, anchor, alpha = _condense_gpu(packed(c, kr), B, g, 0, 4, dev(q), 0, 0, 1.0, 4)
    torch.cuda.synchronize()
    want = np.concatenate([c[0, ::g], kr[0, ::g]], -1).astype(np.float64)
    np.testing.assert_array_equal(host(reps)[0], want)
    np.testing.assert_array_equal(host(anchor)[0], np.arange(4) * g)
    np.testing.assert_array_equal(host(alpha), 1.0 / g)


@pytest.mark.parametrize("g", [2, 4, 8, 32])
def test_condense_other_group_sizes(g):
    B, L = 1, 40 * g
    c, kr = li.latent_cache(7, B, L)
    q = li.queries(7, B, g, H, rho=0.5)
    n = 37
    reps, anchor, alpha = _condense_gpu(packed(c, kr), B, g, 1, n, dev(q), 0, 0, 1.3, n + 1)
    torch.cuda.synchronize()
    rc, rk, ra, ralpha, s = O.condense(c, kr, q, g, 1, n, 0, 0, 1.3)
    assert_close(host(reps)[0, 1:, :512], rc[0], what=f"rep c_KV g={g}")
    assert_close(host(alpha)[0, 1:], ralpha[0], tol=1e-5, what="alpha")
    anchors_agree(host(anchor)[0, 1:].astype(np.int64), ra[0], O.top2_margin(s[0]))


# ------------------------------------------------------------------ decode --
def _decode_gpu(q_t, reps_t, m, cache_t, raw_begin, raw_end, sm):
    B = q_t.shape[0]
    o = torch.empty((B, q_t.shape[1], 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, q_t.shape[1]), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_decode(q_t, None if m == 0 else lca.packed_latent(reps_t), m,
                               lca.packed_latent(cache_t), raw_begin, raw_end, sm, o, lse)
    return o, lse


@pytest.mark.parametrize("dtype,L", [(torch.bfloat16, 2048), (torch.float32, 2048), (torch.bfloat16, 2077)])
def test_decode_condensed_matches_oracle(dtype, L):
    B, g, w = 2, 16, 1024
    bf = dtype == torch.bfloat16
    c, kr = li.latent_cache(1, B, L, bf16=bf)
    li.plant_needles(1, c, kr, 3, 14.0, 0, L, bf16=bf)
    qh = li.queries(1, B, 16, H, rho=0.5, bf16=bf)
    qd = li.queries(1, B, 1, H, rho=0.5, bf16=bf, stream=1)[:, 0]
    p = O.plan(L, w, g)
    cache_t = packed(c, kr, dtype)
    reps, anchor, _ = _condense_gpu(cache_t, B, g, 0, p["m"], dev(qh, dtype), 0, 0, 1.0, p["m"])
    o, lse = _decode_gpu(dev(qd, dtype), reps, p["m"], cache_t, p["raw_begin"], L, 1.0)
    torch.cuda.synchronize()
    r = host(reps)
    ro, rl = O.decode(qd, r[..., :512], r[..., 512:], p["m"], c, kr, p["raw_begin"], L, 1.0)
    assert_close(host(o), ro, what="o_latent")
    assert_close(host(lse), rl, what="lse")


# (seed, heads, representatives m, raw_begin, chunk_start, chunk rows C, bf16 output):
# single-token and odd chunks, two head blocks with C > 128, grouped heads
# (16 / Hg tokens per wave), a window that starts at the chunk, m not a
# multiple of the 32-entry tile
PREFILL_SHAPES = [
    (1, 16, 0, 0, 0, 1, False), (2, 16, 37, 40, 95, 33, True), (3, 32, 5, 0, 7, 130, False),
    (4, 4, 64, 128, 300, 77, False), (5, 1, 10, 20, 60, 200, True), (6, 2, 100, 16, 16, 129, False),
    (7, 8, 0, 0, 250, 251, False), (8, 16, 31, 33, 33, 64, True),
]


@pytest.mark.parametrize("seed,Hq,m,raw_begin,s0,C,bf16_out", PREFILL_SHAPES)
def test_prefill_kernel_shapes(seed, Hq, m, raw_begin, s0, C, bf16_out):
    """The packed-row prefill kernel called directly at assorted (m,
    raw_begin, chunk_start, C, H) against the oracle's chunk attention:
    representatives are arbitrary bf16 rows, raw rows [raw_begin, s0 + i]
    are visible to chunk row i."""
    L, sm = s0 + C, 1.0
    c, kr = li.latent_cache(200 + seed, 1, L)
    li.plant_needles(200 + seed, c, kr, min(2, L - raw_begin), 14.0, raw_begin, L)
    rc, rk = li.latent_cache(300 + seed, 1, max(m, 1))
    q = li.queries(200 + seed, 1, C, Hq, rho=0.5)[0]
    cache_t = packed(c, kr)[0]
    reps_t = packed(rc[:, :m], rk[:, :m])[0] if m else None
    out = torch.empty((C, Hq, 512), dtype=torch.bfloat16 if bf16_out else torch.float32, device="cuda")
    lse = torch.empty((C, Hq), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_prefill_chunk(dev(q), s0, lca.packed_latent(reps_t) if m else None, m,
                                      lca.packed_latent(cache_t), raw_begin, sm, out, lse)
    torch.cuda.synchronize()
    ro, rl = O.prefill_chunk(q, s0, rc[0, :m], rk[0, :m], m, c[0], kr[0], raw_begin, sm)
    assert_close(host(out), ro, what=f"prefill o_latent, shape {seed}")
    assert_close(host(lse), rl, what=f"prefill lse, shape {seed}")


@pytest.mark.parametrize("q_dtype,c_dtype,layout", [
    (torch.float32, torch.bfloat16, "packed"),  # direct-load kernel, f32 queries
    (torch.bfloat16, torch.float32, "packed"),  # register-staged kernel, f32 rows
    (torch.bfloat16, torch.bfloat16, "split"),  # register-staged kernel, c_KV and k_R apart
])
def test_decode_other_dtypes_and_layouts(q_dtype, c_dtype, layout):
    """Decode kernel instantiations not reached by the tests above, against the
    oracle: 3 sequences, needles in the window, seeded bf16 representatives
    given to both sides, several splits; f32 inputs hold bf16-representable values."""
    B, L, g, w = 3, 2600, 16, 1024
    c, kr = li.latent_cache(13, B, L)
    li.plant_needles(13, c, kr, 2, 14.0, L - w, L)
    qd = li.queries(13, B, 1, H, rho=0.5, stream=1)[:, 0]
    p = O.plan(L, w, g)
    m = p["m"]
    rng = np.random.default_rng(13)
    rep_c = li.bf16_round((0.3 * rng.standard_normal((B, m, 512))).astype(np.float32))
    rep_k = li.bf16_round(rng.standard_normal((B, m, 64)).astype(np.float32))

    def describe(xc, xk):
        if layout == "packed":
            t = packed(xc, xk, c_dtype)
            return t, lca.packed_latent(t)
        tc, tk = dev(xc, c_dtype), dev(xk, c_dtype)
        return (tc, tk), lca.latent(tc, tk)

    keep_c, cache_l = describe(c, kr)
    keep_r, reps_l = describe(rep_c, rep_k)
    o = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_decode(dev(qd, q_dtype), reps_l, m, cache_l, p["raw_begin"], L, 1.0, o, lse)
    torch.cuda.synchronize()
    ro, rl = O.decode(qd, rep_c, rep_k, m, c, kr, p["raw_begin"], L, 1.0)
    assert_close(host(o), ro, what=f"decode o_latent ({layout})")
    assert_close(host(lse), rl, what=f"decode lse ({layout})")


def test_decode_plain_mla_matches_oracle():
    B, L = 2, 2048  # w = L: no groups, exact MLA over every row
    c, kr = li.latent_cache(2, B, L)
    li.plant_needles(2, c, kr, 2, 14.0, 0, L)
    qd = li.queries(2, B, 1, H, rho=0.5, stream=1)[:, 0]
    o, lse = _decode_gpu(dev(qd), None, 0, packed(c, kr), 0, L, 1.0)
    torch.cuda.synchronize()
    ro, rl = O.decode(qd, None, None, 0, c, kr, 0, L, 1.0)
    assert_close(host(o), ro, what="o_latent")
    assert_close(host(lse), rl, what="lse")


def test_decode_singleton_groups_equal_plain_mla_bitwise():
    """g = 1 representatives are exact row copies, so LCA decode over them
    equals plain MLA decode bit for bit (same entries, same order)."""
    B, L, w = 2, 1500, 300
    c, kr = li.latent_cache(3, B, L)
    qd = li.queries(3, B, 1, H, rho=0.5, stream=1)[:, 0]
    cache_t = packed(c, kr)
    m = L - w
    reps, _, _ = _condense_gpu(cache_t, B, 1, 0, m, dev(li.queries(3, B, 1, H)), 0, 0, 1.0, m)
    o1, l1 = _decode_gpu(dev(qd), reps, m, cache_t, m, L, 1.0)
    o2, l2 = _decode_gpu(dev(qd), None, 0, cache_t, 0, L, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_independent_of_split_count():
    """The same sequence alone (many splits) and in a batch of 64 (few
    splits). The only split-dependent rounding is that of the softmax
    weights: each split rounds p_e = 2^(z_e - ref) to bf16 (relative error
    <= 2^-9) against its own running reference, while the row sum uses the
    unrounded fp32 weights. Two split counts therefore differ by at most
    2^-8 * sum_e p_e |c_e,d| / sum_e p_e per output element, plus fp32
    accumulation-order error (allowed 1e-4 of the same magnitude)."""
    L = 9000
    c, kr = li.latent_cache(8, 1, L)
    li.plant_needles(8, c, kr, 2, 14.0, 0, L)
    qd = li.queries(8, 1, 1, H, rho=0.5, stream=1)[:, 0]
    cache1 = packed(c, kr)
    o1, l1 = _decode_gpu(dev(qd), None, 0, cache1, 0, L, 1.0)
    cacheB = cache1.expand(64, L, 576)
    oB, lB = _decode_gpu(dev(qd).expand(64, H, 576), None, 0, cacheB, 0, L, 1.0)
    torch.cuda.synchronize()
    s1 = lca.mla_latent_attn_decode_workspace_size(1, H, L)
    sB = lca.mla_latent_attn_decode_workspace_size(64, H, L)
    assert s1 // (16 * 514 * 4) != sB // (64 * 16 * 514 * 4)  # different split counts
    # sum_e p_e |c_e,d| / sum_e p_e with the exact (fp64) softmax weights
    keys = np.concatenate([c[0], kr[0]], -1).astype(np.float64)
    z = qd[0].astype(np.float64) @ keys.T
    pw = np.exp(z - z.max(-1, keepdims=True))
    mag = (pw / pw.sum(-1, keepdims=True)) @ np.abs(c[0].astype(np.float64))   # [H, 512]
    diff = host(oB[0]) - host(o1[0])
    bound = (2.0 ** -8 + 1e-4) * mag + 1e-7
    assert np.all(np.abs(diff) <= bound), f"max excess {np.max(np.abs(diff) - bound):.3e}"
    assert (lB - l1).abs().max().item() <= 1e-5
    # every batch row identical (deterministic)
    assert torch.equal(oB, oB[:1].expand_as(oB))


def test_decode_split_count_exact_on_power_of_two_weights():
    """Split-count invariance within 1e-6 relative (the bound the survey sets
    for the split merge) where no weight rounds: every head's query is one
    unit column, every cached value a small integer, and sm_scale = fp32(ln 2)
    makes the log2-domain logits the integers -2..0. Each weight 2^(z - ref)
    is then an exact power of two in bf16 and fp32, all partial sums are
    exact, and the output may differ between split counts only through the
    hardware exp2 of integer arguments."""
    L = 9000
    r = np.random.default_rng(81)
    rows = r.integers(-2, 1, size=(1, L, 576)).astype(np.float32)
    cols = r.choice(576, H, replace=False)                     # heads in c_KV and in k_R columns
    qd = np.zeros((1, H, 576), dtype=np.float32)
    qd[0, np.arange(H), cols] = 1.0
    sm = float(np.float32(np.log(2.0)))
    cache1 = dev(rows)
    o1, l1 = _decode_gpu(dev(qd), None, 0, cache1, 0, L, sm)
    oB, lB = _decode_gpu(dev(qd).expand(64, H, 576), None, 0, cache1.expand(64, L, 576), 0, L, sm)
    torch.cuda.synchronize()
    rel = (oB - o1).abs().max().item() / o1.abs().max().item()
    assert rel <= 1e-6, rel
    assert (lB - l1).abs().max().item() <= 1e-6 * l1.abs().max().item()
    ro, rl = O.decode(qd, None, None, 0, rows[..., :512], rows[..., 512:], 0, L, sm)
    assert_close(host(o1), ro, what="o_latent")
    assert_close(host(l1), rl, what="lse")


def test_decode_tiny_and_ragged():
    B, L = 3, 5
    c, kr = li.latent_cache(9, B, L)
    qd = li.queries(9, B, 1, 32, rho=0.5, stream=1)[:, 0]  # H = 32: two head blocks
    o, lse = _decode_gpu(dev(qd), None, 0, packed(c, kr), 2, L, 0.8)
    torch.cuda.synchronize()
    ro, rl = O.decode(qd, None, None, 0, c, kr, 2, L, 0.8)
    assert_close(host(o), ro, what="o_latent")
    assert_close(host(lse), rl, what="lse")


# ----------------------------------------------------------------- prefill --
@pytest.mark.parametrize("B,L,wdt,odt,Hh", [(32, 3008, torch.bfloat16, torch.bfloat16, 16),  # fused merge
                                            (5, 1000, torch.float32, torch.float32, 16),    # fused, 32 splits, ragged B
                                            (3, 30, torch.bfloat16, torch.float32, 16),     # one split
                                            (1, 40000, torch.bfloat16, torch.bfloat16, 16),  # many splits
                                            (70, 600, torch.bfloat16, torch.bfloat16, 16),  # B > 64
                                            (24, 3008, torch.bfloat16, torch.float32, 4),   # a GQA group of 4 heads
                                            (2, 40000, torch.bfloat16, torch.bfloat16, 1)])  # one head, many splits
def test_decode_up_equals_decode_then_up_proj(B, L, wdt, odt, Hh):
    """The fused decode + up-projection entry point gives bitwise the results
    of mla_latent_attn_decode followed by mla_up_proj, and the up-projected
    output matches the oracle (also for head counts below 16)."""
    H = Hh
    c, kr = li.latent_cache(13, B, L)
    li.plant_needles(13, c, kr, 2, 12.0, 0, L)
    q = li.queries(13, B, 1, H, rho=0.5)[:, 0]
    w = li.w_uv(13, H)
    cache_t, q_t, w_t = packed(c, kr), dev(q), dev(w, wdt)
    o1, l1 = _decode_gpu(q_t, None, 0, cache_t, 0, L, 1.0)
    y1 = torch.empty((B, H, 128), dtype=odt, device="cuda")
    lca.mla_up_proj(o1, w_t, y1)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    y2 = torch.empty_like(y1)
    lca.mla_latent_attn_decode_up(q_t, None, 0, lca.packed_latent(cache_t), 0, L, 1.0, o2, w_t, y2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(y1, y2)
    ro, _ = O.decode(q, None, None, 0, c, kr, 0, L, 1.0)
    assert_close(host(y2), O.up_proj(ro, w), what="decode_up out")


def test_two_head_blocks_decode_up_and_prefill():
    """H = 32, two blocks of 16 heads (the grids' head-block axis): the fused
    decode + up-projection (4 sequences, several splits) and a causal prefill
    chunk with a ragged last workgroup, against the oracle."""
    H2, B, L = 32, 4, 3000
    c, kr = li.latent_cache(14, B, L)
    li.plant_needles(14, c, kr, 2, 12.0, 0, L)
    q = li.queries(14, B, 1, H2, rho=0.5)[:, 0]
    w = li.w_uv(14, H2)
    cache_t = packed(c, kr)
    o = torch.empty((B, H2, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H2), dtype=torch.float32, device="cuda")
    y = torch.empty((B, H2, 128), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_decode_up(dev(q), None, 0, lca.packed_latent(cache_t), 0, L, 1.0, o, dev(w), y, lse)
    Lp = 150
    qp = li.queries(14, 1, Lp, H2, rho=0.5, stream=2)[0]
    op = torch.empty((Lp, H2, 512), dtype=torch.float32, device="cuda")
    lp = torch.empty((Lp, H2), dtype=torch.float32, device="cuda")
    lca.mla_latent_attn_prefill_chunk(dev(qp), 0, None, 0, lca.packed_latent(cache_t[0]), 0, 1.0, op, lp)
    torch.cuda.synchronize()
    ro, rl = O.decode(q, None, None, 0, c, kr, 0, L, 1.0)
    assert_close(host(o), ro, what="decode o_latent, H = 32")
    assert_close(host(lse), rl, what="decode lse, H = 32")
    assert_close(host(y), O.up_proj(ro, w), what="decode_up out, H = 32")
    rpo, rpl = O.prefill_chunk(qp, 0, np.zeros((0, 512)), np.zeros((0, 64)), 0, c[0], kr[0], 0, 1.0)
    assert_close(host(op), rpo, what="prefill o_latent, H = 32")
    assert_close(host(lp), rpl, what="prefill lse, H = 32")


# chunks of 64 and 40 rows, of 129 rows (a second workgroup of 128 query rows
# holding one token), and of one token
@pytest.mark.parametrize("L,C", [(320, 64), (301, 40), (300, 129), (70, 1)])
def test_prefill_chunks_match_oracle(L, C):
    w, g, sm = 64, 16, 1.0
    c, kr = li.latent_cache(10, 1, L)
    q = li.queries(10, 1, L, H, rho=0.5)[0]
    cache_t = packed(c, kr)[0]
    q_t = dev(q)
    m_cap = O.prefill_plan(((L - 1) // C) * C, w, g)
    reps = torch.zeros((max(m_cap, 1), 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.zeros((1, max(m_cap, 1)), dtype=torch.int32, device="cuda")
    out = torch.empty((L, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, H), dtype=torch.float32, device="cuda")
    m = 0
    for s in range(0, L, C):
        ms = O.prefill_plan(s, w, g)
        if ms > m:
            lca.lca_condense(lca.packed_latent(cache_t[None]), 1, g, m, ms - m, q_t[None],
                             (m + 1) * g, g, sm, lca.packed_latent(reps[None]), anchor)
            m = ms
        e = min(L, s + C)
        lca.mla_latent_attn_prefill_chunk(q_t[s:e], s, lca.packed_latent(reps) if m else None, m,
                                          lca.packed_latent(cache_t), m * g, sm, out[s:e], lse[s:e])
    torch.cuda.synchronize()
    # oracle reps for the anchor check, GPU reps for the attention check
    _, _, rep_c, rep_k = O.prefill(q, c[0], kr[0], w, g, C, sm)
    r = host(reps)[:m_cap]
    assert_close(r[:, :512], rep_c, what="prefill reps")
    ro = np.zeros((L, H, 512))
    rl = np.zeros((L, H))
    for s in range(0, L, C):
        ms = O.prefill_plan(s, w, g)
        e = min(L, s + C)
        ro[s:e], rl[s:e] = O.prefill_chunk(q[s:e], s, r[:, :512], r[:, 512:], ms, c[0], kr[0], ms * g, sm)
    assert_close(host(out), ro, what="prefill o_latent")
    assert_close(host(lse), rl, what="prefill lse")


def test_prefill_bf16_output():
    L, C = 96, 96
    c, kr = li.latent_cache(11, 1, L)
    q = li.queries(11, 1, L, H, rho=0.5)[0]
    out = torch.empty((C, H, 512), dtype=torch.bfloat16, device="cuda")
    lca.mla_latent_attn_prefill_chunk(dev(q), 0, None, 0, lca.packed_latent(packed(c, kr)[0]), 0, 1.0, out)
    torch.cuda.synchronize()
    ro, _ = O.prefill_chunk(q, 0, np.zeros((0, 512)), np.zeros((0, 64)), 0, c[0], kr[0], 0, 1.0)
    assert_close(host(out), ro, what="prefill bf16 o_latent")


@pytest.mark.parametrize("q_dtype,c_dtype,layout", [
    (torch.float32, torch.bfloat16, "packed"),  # direct-load kernel, f32 queries
    (torch.bfloat16, torch.float32, "packed"),  # register-staged kernel, f32 rows
    (torch.bfloat16, torch.bfloat16, "split"),  # register-staged kernel, c_KV and k_R apart
    (torch.float32, torch.float32, "split"),
])
def test_prefill_other_dtypes_and_layouts(q_dtype, c_dtype, layout):
    """Every prefill kernel instantiation against the oracle: several chunks
    with representatives (the oracle's, rounded to bf16 and given to both
    sides), a ragged last chunk; f32 inputs hold bf16-representable values."""
    L, C, w, g, sm = 230, 72, 64, 16, 1.0
    c, kr = li.latent_cache(12, 1, L)
    q = li.queries(12, 1, L, H, rho=0.5)[0]
    _, _, rep_c, rep_k = O.prefill(q, c[0], kr[0], w, g, C, sm)
    rep_c, rep_k = li.bf16_round(rep_c), li.bf16_round(rep_k)

    def describe(xc, xk):
        if layout == "packed":
            t = packed(xc, xk, c_dtype)
            return t, lca.packed_latent(t)
        tc, tk = dev(xc, c_dtype), dev(xk, c_dtype)
        return (tc, tk), lca.latent(tc, tk)

    keep_c, cache_l = describe(c[0], kr[0])
    keep_r, reps_l = describe(rep_c, rep_k)
    q_t = dev(q, q_dtype)
    out = torch.empty((L, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, H), dtype=torch.float32, device="cuda")
    for s in range(0, L, C):
        ms = O.prefill_plan(s, w, g)
        e = min(L, s + C)
        lca.mla_latent_attn_prefill_chunk(q_t[s:e], s, reps_l if ms else None, ms, cache_l, ms * g, sm,
                                          out[s:e], lse[s:e])
    torch.cuda.synchronize()
    ro = np.zeros((L, H, 512))
    rl = np.zeros((L, H))
    for s in range(0, L, C):
        ms = O.prefill_plan(s, w, g)
        e = min(L, s + C)
        ro[s:e], rl[s:e] = O.prefill_chunk(q[s:e], s, rep_c, rep_k, ms, c[0], kr[0], ms * g, sm)
    assert_close(host(out), ro, what=f"prefill o_latent ({layout})")
    assert_close(host(lse), rl, what=f"prefill lse ({layout})")


# --------------------------------------------------------------- up-proj ----
@pytest.mark.parametrize("xdt,ydt,T", [(torch.float32, torch.float32, 37), (torch.bfloat16, torch.bfloat16, 130),
                                      (torch.float32, torch.bfloat16, 64)])
def test_up_proj_matches_oracle(xdt, ydt, T):
    rng = np.random.default_rng(12)
    # unit-scale outputs: latent attention outputs are convex mixes of rows
    x = li.bf16_round((0.25 * rng.standard_normal((T, H, 512))).astype(np.float32))
    w = li.w_uv(12, H)
    out = torch.empty((T, H, 128), dtype=ydt, device="cuda")
    lca.mla_up_proj(dev(x, xdt), dev(w), out)
    torch.cuda.synchronize()
    assert_close(host(out), O.up_proj(x, w), tol=TOL, what="up_proj")


@pytest.mark.parametrize("T,Hh,wdt,ydt", [(65, 16, torch.bfloat16, torch.bfloat16),
                                          (1000, 16, torch.float32, torch.float32),
                                          (4097, 1, torch.bfloat16, torch.bfloat16),
                                          (777, 8, torch.float32, torch.bfloat16),
                                          (600, 128, torch.bfloat16, torch.float32)])
def test_up_proj_bf16_latent_shapes(T, Hh, wdt, ydt):
    """bf16 latent above 64 tokens (the persistent streaming kernel): ragged
    ends of the 32-token tiles, 1 to 128 heads, W_UV and output in either
    precision."""
    rng = np.random.default_rng(13 + T)
    x = li.bf16_round((0.25 * rng.standard_normal((T, Hh, 512))).astype(np.float32))
    w = li.w_uv(13, Hh)
    out = torch.empty((T, Hh, 128), dtype=ydt, device="cuda")
    lca.mla_up_proj(dev(x, torch.bfloat16), dev(w, wdt), out)
    torch.cuda.synchronize()
    assert_close(host(out), O.up_proj(x, w), tol=TOL, what=f"up_proj T={T} H={Hh}")


def test_up_proj_row_independent_of_rows_projected_with_it():
    """mla_up_proj picks its workgroup shape (rows per workgroup, output-column
    blocks) from the row count, so T = 64, 37, 32, 8, 5, 2 and 1 run different
    shapes; a row's output is the same bits in every one, and matches the
    oracle."""
    rng = np.random.default_rng(21)
    x = li.bf16_round((0.25 * rng.standard_normal((64, H, 512))).astype(np.float32))
    w = li.w_uv(21, H)
    xd, wd = dev(x, torch.float32), dev(w)
    ref = None
    for T in (64, 37, 32, 8, 5, 2, 1):
        out = torch.empty((T, H, 128), dtype=torch.float32, device="cuda")
        lca.mla_up_proj(xd[:T].contiguous(), wd, out)
        torch.cuda.synchronize()
        if ref is None:
            ref = host(out)
            assert_close(ref, O.up_proj(x, w), tol=TOL, what="up_proj T=64")
        else:
            assert np.array_equal(host(out), ref[:T]), f"T={T} differs from T=64"


# ------------------------------------------------------------- HIP graphs --
def test_graph_replay_matches_eager():
    """Condense + fused decode captured in a HIP graph: every replay, with
    eager work and synchronisations in between, equals the eager results."""
    B, L, g, w = 4, 2500, 16, 1024
    c, kr = li.latent_cache(14, B, L)
    qh = li.queries(14, B, 16, H, rho=0.5)
    qd = li.queries(14, B, 1, H, rho=0.5, stream=1)[:, 0]
    p = O.plan(L, w, g)
    m = p["m"]
    cache_t, qh_t, qd_t, w_t = packed(c, kr), dev(qh), dev(qd), dev(li.w_uv(14, H))
    reps = torch.zeros((B, m, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.zeros((B, m), dtype=torch.int32, device="cuda")
    o = torch.zeros((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, H), dtype=torch.float32, device="cuda")
    y = torch.zeros((B, H, 128), dtype=torch.bfloat16, device="cuda")
    cws = torch.empty(lca.lca_condense_workspace_size(B, m, 0), dtype=torch.uint8, device="cuda")
    dws = lca.decode_workspace(B, H, p["n_entries"])

    def work():
        lca.lca_condense(lca.packed_latent(cache_t), B, g, 0, m, qh_t, 0, 0, 1.0,
                         lca.packed_latent(reps), anchor, None, cws)
        lca.mla_latent_attn_decode_up(qd_t, lca.packed_latent(reps), m, lca.packed_latent(cache_t),
                                      p["raw_begin"], L, 1.0, o, w_t, y, lse, dws)

    work()
    torch.cuda.synchronize()
    want = [t.clone() for t in (reps, anchor, o, lse, y)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(3):
        for t in (reps, o, lse, y):
            t.fill_(float("nan"))
        anchor.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((reps, anchor, o, lse, y), want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
        _ = (qd_t.float() * 2).sum().item()  # eager work between replays
