"""GPU parity at the full workload sizes, in the launch configurations the
benchmark uses, on outputs the oracle can compute one by one (sampled groups,
sampled sequences, sampled query rows), plus the incremental decode loop of
the million-token workload checked step by step at a small size.

Inputs: lca_inputs (seeded, bf16-rounded on the host); expected values come
only from the oracle, fed the GPU's own condensed rows where the attention is
checked (so a legitimate near-tie anchor cannot cascade).
"""
import numpy as np
import pytest
import torch

import lca_inputs as li
import mla_latent_kv_lca_amd as lca
from oracle import lca_oracle as O
from tests.gpu_util import TOL, AnchorTally, anchors_agree, assert_close, dev, host

pytestmark = pytest.mark.gpu

H, G, W = 16, 16, 1024


def _packed(c, kr):
    t = torch.empty(c.shape[:-1] + (576,), dtype=torch.bfloat16, device="cuda")
    for b in range(c.shape[0]):  # upload sequence by sequence to bound host temporaries
        t[b] = torch.from_numpy(np.concatenate([c[b], kr[b]], -1)).to("cuda", torch.bfloat16)
    return t


@pytest.mark.timeout(400)
def test_batched_decode_32x32k_sampled():
    """B = 32 sequences x L = 32,768: condense every group, one decode step."""
    B, L = 32, 32768
    c, kr = li.latent_cache(2, B, L)
    li.plant_needles(2, c, kr, 4, 14.0, 0, L)
    qh = li.queries(2, B, G, H, rho=0.5)
    qd = li.queries(2, B, 1, H, rho=0.5, stream=1)[:, 0]
    p = O.plan(L, W, G)
    m = p["m"]
    cache = _packed(c, kr)
    reps = torch.empty((B, m, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.empty((B, m), dtype=torch.int32, device="cuda")
    alpha = torch.empty((B, m, G), dtype=torch.float32, device="cuda")
    lca.lca_condense(lca.packed_latent(cache), B, G, 0, m, dev(qh), 0, 0, 1.0,
                     lca.packed_latent(reps), anchor, alpha)
    o = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = lca.decode_workspace(B, H, p["n_entries"])
    lca.mla_latent_attn_decode(dev(qd), lca.packed_latent(reps), m, lca.packed_latent(cache),
                               p["raw_begin"], L, 1.0, o, lse, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    r = host(reps)
    ga = host(anchor).astype(np.int64)
    rng = np.random.default_rng(0)
    tally = AnchorTally()
    for b, j in zip(rng.integers(0, B, 96), rng.integers(0, m, 96)):
        rc, rk, ra, ralpha, s = O.condense(c[b:b + 1], kr[b:b + 1], qh[b:b + 1], G, int(j), 1, 0, 0, 1.0)
        assert_close(r[b, j, :512], rc[0, 0], what=f"rep ({b},{j})")
        assert_close(host(alpha[b, j]), ralpha[0, 0], tol=1e-5, what="alpha")
        tally.add(ga[b, j:j + 1], ra[0], O.top2_margin(s[0]))
        np.testing.assert_array_equal(r[b, j, 512:], kr[b, ga[b, j]])
    tally.check()
    for b in (0, 13, 31):
        ro, rl = O.decode(qd[b:b + 1], r[b:b + 1, :, :512], r[b:b + 1, :, 512:], m,
                          c[b:b + 1], kr[b:b + 1], p["raw_begin"], L, 1.0)
        assert_close(host(o[b]), ro[0], what=f"o_latent seq {b}")
        assert_close(host(lse[b]), rl[0], what=f"lse seq {b}")


def test_incremental_decode_loop_matches_oracle():
    """Decode steps that append a row each and condense every newly
    completed group with the last g decode queries (frozen representatives)."""
    L0, S, w, g = 1300, 40, 1024, 16
    c0, k0 = li.latent_cache(5, 1, L0 + S)
    li.plant_needles(5, c0, k0, 3, 14.0, 0, L0 + S)
    qhist = li.queries(5, 1, g, H, rho=0.5)[0]
    steps = li.queries(5, 1, S, H, rho=0.5, stream=2)[0]
    ro, rl, _, _, m_ref = O.decode_loop(c0[0, :L0], k0[0, :L0], qhist, steps, c0[0, L0:], k0[0, L0:],
                                        w, g, 1.0)
    cache = _packed(c0, k0)           # rows are appended by advancing L
    qall = dev(np.concatenate([qhist, steps])[None])  # [1, g + S, H, 576]
    m_cap = O.plan(L0 + S, w, g)["m"]
    reps = torch.empty((1, m_cap, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.empty((1, m_cap), dtype=torch.int32, device="cuda")
    L = L0
    m = O.plan(L, w, g)["m"]
    lca.lca_condense(lca.packed_latent(cache), 1, g, 0, m, qall, 0, 0, 1.0,
                     lca.packed_latent(reps), anchor)
    o = torch.empty((1, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws = lca.decode_workspace(1, H, L0 + S)
    outs, lses = [], []
    for st in range(S):
        lca.mla_latent_attn_decode(qall[:, g + st], lca.packed_latent(reps) if m else None, m,
                                   lca.packed_latent(cache), m * g, L, 1.0, o, lse, ws)
        outs.append(o.clone())
        lses.append(lse.clone())
        L += 1
        if L - w >= (m + 1) * g:  # the row just appended completed group m
            lca.lca_condense(lca.packed_latent(cache), 1, g, m, 1, qall, st + 1, 0, 1.0,
                             lca.packed_latent(reps), anchor)
            m += 1
    torch.cuda.synchronize()
    assert m == m_ref
    got = np.stack([host(x)[0] for x in outs])
    assert_close(got, ro, what="incremental decode o_latent")
    assert_close(np.stack([host(x)[0] for x in lses]), rl, what="incremental decode lse")


@pytest.mark.timeout(600)
def test_million_token_decode_loop_sampled():
    """L0 = 1,048,576 tokens, one sequence, with needles: condense the 65,472
    groups, then 256 decode steps in the benchmark's launch configuration
    (decode + W_UV up-projection) that each append a row, condensing every
    newly completed group with the last 16 decode queries (16 condensations).
    Checked: 64 sampled initial representatives, every incrementally
    condensed representative, and the outputs of steps 0, 16 and 255."""
    L0, S = 1 << 20, 256
    c, kr = li.latent_cache(6, 1, L0 + S)
    li.plant_needles(6, c, kr, 4, 16.0, 0, L0 - W)            # condensed into representatives
    li.plant_needles(6, c, kr, 2, 16.0, L0 - W, L0 + S)       # in the window / appended rows
    qall = np.concatenate([li.queries(6, 1, G, H, rho=0.5), li.queries(6, 1, S, H, rho=0.5, stream=1)], 1)
    wuv = li.w_uv(6, H)
    p = O.plan(L0, W, G)
    m = p["m"]
    assert m == 65472
    m_cap = O.plan(L0 + S, W, G)["m"]
    cache = _packed(c, kr)                                     # rows past L are appended by advancing L
    q_t = dev(qall)                                            # [1, 16 + S, H, 576]
    w_t = dev(wuv)
    reps = torch.empty((1, m_cap, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.empty((1, m_cap), dtype=torch.int32, device="cuda")
    lca.lca_condense(lca.packed_latent(cache), 1, G, 0, m, q_t, 0, 0, 1.0, lca.packed_latent(reps), anchor)
    o = torch.empty((1, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H), dtype=torch.float32, device="cuda")
    y = torch.empty((1, H, 128), dtype=torch.float32, device="cuda")
    ws = lca.decode_workspace(1, H, m_cap + (L0 + S - m_cap * G))
    check = {0: None, 16: None, 255: None}
    condensed = []                                             # (step, group, q_row0)
    L = L0
    for st in range(S):
        lca.mla_latent_attn_decode_up(q_t[:, G + st], lca.packed_latent(reps), m, lca.packed_latent(cache),
                                      m * G, L, 1.0, o, w_t, y, lse, ws)
        if st in check:
            check[st] = (m, L, o.clone(), lse.clone(), y.clone())
        L += 1                                                 # the step's row is appended
        if L - W >= (m + 1) * G:                               # it completed group m
            lca.lca_condense(lca.packed_latent(cache), 1, G, m, 1, q_t, st + 1, 0, 1.0,
                             lca.packed_latent(reps), anchor)
            condensed.append((st, m, st + 1))
            m += 1
    torch.cuda.synchronize()
    assert len(condensed) == 16 and m == m_cap
    r = host(reps)
    ga = host(anchor).astype(np.int64)
    tally = AnchorTally()
    for j in np.random.default_rng(1).integers(0, p["m"], 64):
        rc, _, ra, _, s = O.condense(c, kr, qall, G, int(j), 1, 0, 0, 1.0)
        assert_close(r[0, j, :512], rc[0, 0], what=f"rep {j}")
        tally.add(ga[0, j:j + 1], ra[0], O.top2_margin(s[0]))
        np.testing.assert_array_equal(r[0, j, 512:], kr[0, ga[0, j]])
    for st, j, r0 in condensed:  # each new group: the 16 most recent decode queries
        rc, _, ra, _, s = O.condense(c, kr, qall, G, j, 1, r0, 0, 1.0)
        assert_close(r[0, j, :512], rc[0, 0], what=f"incremental rep {j} (after step {st})")
        tally.add(ga[0, j:j + 1], ra[0], O.top2_margin(s[0]))
        np.testing.assert_array_equal(r[0, j, 512:], kr[0, ga[0, j]])
    tally.check()
    for st, (ms, Ls, o_s, l_s, y_s) in check.items():
        ro, rl = O.decode(qall[:, G + st], r[:, :, :512], r[:, :, 512:], ms, c, kr, ms * G, Ls, 1.0)
        assert np.abs(ro).max() > 0.5, "needles should make the output unit-scale"
        assert_close(host(o_s), ro, what=f"o_latent step {st}")
        assert_close(host(l_s), rl, what=f"lse step {st}")
        assert_close(host(y_s), O.up_proj(ro, wuv), what=f"up-projected output step {st}")


def _assert_close_bf16_out(got, ref, what):
    """Outputs stored in bf16: the parity gate (max-abs <= 1e-2 and <= 1e-2 of
    max|ref|) applied to what is left after one bf16 rounding of the stored
    value (2^-9 relative, allowed twice)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    excess = np.maximum(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref), 0.0)
    err, scale = float(excess.max()), float(np.abs(ref).max())
    assert err <= TOL, f"{what}: max-abs error beyond bf16 storage {err:.3e} > {TOL}"
    assert err <= TOL * scale, f"{what}: error beyond bf16 storage {err:.3e} vs output scale {scale:.3e}"


@pytest.mark.timeout(600)
def test_prefill_128k_sampled_rows():
    """Chunked prefill of L = 131,072 in 4,096-token chunks, with needles so
    that outputs stay unit-scale: per chunk the newly eligible groups are
    condensed with the 16 queries that follow each group; 256 sampled query
    rows of chunks 0, 1, 15 and 31 (each chunk's first and last row among
    them) and 256 sampled representatives against the oracle; the W_UV
    up-projection of all 131,072 x 16 outputs in one call, on the same rows."""
    L, C = 131072, 4096
    c, kr = li.latent_cache(7, 1, L)
    li.plant_needles(7, c, kr, 2, 14.0, 0, 64)       # visible to (almost) every row of chunk 0
    li.plant_needles(7, c, kr, 30, 14.0, 64, L)
    q = li.queries(7, 1, L, H, rho=0.5)[0]
    cache = _packed(c, kr)[0]
    q_t = torch.empty((L, H, 576), dtype=torch.bfloat16, device="cuda")
    for s0 in range(0, L, 16384):
        q_t[s0:s0 + 16384] = torch.from_numpy(q[s0:s0 + 16384]).to("cuda", torch.bfloat16)
    m_cap = O.prefill_plan(L - C, W, G)
    reps = torch.empty((m_cap, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.empty((1, m_cap), dtype=torch.int32, device="cuda")
    out = torch.empty((L, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((L, H), dtype=torch.float32, device="cuda")
    m = 0
    for s0 in range(0, L, C):
        ms = O.prefill_plan(s0, W, G)
        if ms > m:
            lca.lca_condense(lca.packed_latent(cache[None]), 1, G, m, ms - m, q_t[None], (m + 1) * G, G,
                             1.0, lca.packed_latent(reps[None]), anchor)
            m = ms
        lca.mla_latent_attn_prefill_chunk(q_t[s0:s0 + C], s0, lca.packed_latent(reps) if m else None, m,
                                          lca.packed_latent(cache), m * G, 1.0, out[s0:s0 + C], lse[s0:s0 + C])
    wuv = li.w_uv(7, H)
    y = torch.empty((L, H, 128), dtype=torch.bfloat16, device="cuda")
    lca.mla_up_proj(out, dev(wuv), y)  # the whole prefill's up-projection in one call
    # the scheduled call (persistent workgroups, the benchmark's path) on the
    # full-size chunks 15 and 31: bitwise equal to the per-block kernel
    sched = lca.prefill_sched()
    for chunk in (15, 31):
        s0 = chunk * C
        ms = O.prefill_plan(s0, W, G)
        o_s = torch.empty((C, H, 512), dtype=torch.bfloat16, device="cuda")
        l_s = torch.empty((C, H), dtype=torch.float32, device="cuda")
        lca.mla_latent_attn_prefill_chunk(q_t[s0:s0 + C], s0, lca.packed_latent(reps), ms, lca.packed_latent(cache),
                                          ms * G, 1.0, o_s, l_s, sched=sched)
        torch.cuda.synchronize()
        assert torch.equal(o_s, out[s0:s0 + C]) and torch.equal(l_s, lse[s0:s0 + C]), f"scheduled chunk {chunk}"
    assert sched.tolist() == [0, 0]
    torch.cuda.synchronize()
    r = host(reps)
    ga = host(anchor).astype(np.int64)
    rng = np.random.default_rng(2)
    tally = AnchorTally()
    for j in rng.choice(m_cap, 256, replace=False):  # representatives: per-group summary queries
        rc, _, ra, _, s = O.condense(c, kr, q[None], G, int(j), 1, (int(j) + 1) * G, G, 1.0)
        assert_close(r[j, :512], rc[0, 0], what=f"rep {j}")
        tally.add(ga[0, j:j + 1], ra[0], O.top2_margin(s[0]))
        np.testing.assert_array_equal(r[j, 512:], kr[0, ga[0, j]])
    tally.check()
    for chunk in (0, 1, 15, 31):
        s0 = chunk * C
        ms = O.prefill_plan(s0, W, G)
        rows = np.sort(rng.choice(np.arange(1, C - 1), 254, replace=False))
        rows = np.concatenate([[0], rows, [C - 1]])  # the first row sees the fewest entries, the last the most
        ro, rl = O.prefill_chunk(q[s0:s0 + C], s0, r[:, :512], r[:, 512:], ms, c[0], kr[0], ms * G, 1.0,
                                 rows=rows)
        if chunk > 0:
            assert np.abs(ro).max(axis=(1, 2)).min() > 0.5, "needles should keep every sampled row unit-scale"
        _assert_close_bf16_out(host(out[s0 + rows]), ro, what=f"prefill o_latent chunk {chunk}")
        assert_close(host(lse[s0 + rows]), rl, what=f"prefill lse chunk {chunk}")
        assert_close(host(y[s0 + rows]), O.up_proj(host(out[s0 + rows]), wuv), what=f"up-projected chunk {chunk}")


@pytest.mark.timeout(400)
def test_decode_128k_lca_and_plain_mla_sampled():
    """The 131,072-token shape of the long-context comparison (2 sequences):
    condense all 8,128 groups, then one decode step over the condensed cache
    and one over all rows (plain MLA, m = 0), in the benchmark's launch
    configuration (decode plus W_UV up-projection)."""
    B, L = 2, 131072
    c, kr = li.latent_cache(7, B, L)
    li.plant_needles(7, c, kr, 4, 14.0, 0, L)
    qh = li.queries(7, B, G, H, rho=0.5)
    qd = li.queries(7, B, 1, H, rho=0.5, stream=1)[:, 0]
    wuv = li.w_uv(7, H)
    p = O.plan(L, W, G)
    m = p["m"]
    cache = _packed(c, kr)
    reps = torch.empty((B, m, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.empty((B, m), dtype=torch.int32, device="cuda")
    lca.lca_condense(lca.packed_latent(cache), B, G, 0, m, dev(qh), 0, 0, 1.0, lca.packed_latent(reps), anchor)
    o_l = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    o_m = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    y_l = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    y_m = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    lse_l = torch.empty((B, H), dtype=torch.float32, device="cuda")
    lse_m = torch.empty((B, H), dtype=torch.float32, device="cuda")
    w_t, q_t = dev(wuv), dev(qd)
    lca.mla_latent_attn_decode_up(q_t, lca.packed_latent(reps), m, lca.packed_latent(cache), p["raw_begin"], L,
                                  1.0, o_l, w_t, y_l, lse_l)
    lca.mla_latent_attn_decode_up(q_t, None, 0, lca.packed_latent(cache), 0, L, 1.0, o_m, w_t, y_m, lse_m)
    torch.cuda.synchronize()
    r = host(reps)
    ga = host(anchor).astype(np.int64)
    tally = AnchorTally()
    for j in np.random.default_rng(8).integers(0, m, 24):
        rc, _, ra, _, s = O.condense(c, kr, qh, G, int(j), 1, 0, 0, 1.0)
        for b in range(B):
            assert_close(r[b, j, :512], rc[b, 0], what=f"rep {b}/{j}")
        tally.add(ga[:, j], ra[:, 0], O.top2_margin(s[:, 0]))
    tally.check()
    ro, rl = O.decode(qd, r[..., :512], r[..., 512:], m, c, kr, p["raw_begin"], L, 1.0)
    assert_close(host(o_l), ro, what="LCA o_latent")
    assert_close(host(lse_l), rl, what="LCA lse")
    assert_close(host(y_l), O.up_proj(ro, wuv), what="LCA up-projected output")
    mo, ml = O.decode(qd, None, None, 0, c, kr, 0, L, 1.0)
    assert_close(host(o_m), mo, what="plain MLA o_latent")
    assert_close(host(lse_m), ml, what="plain MLA lse")
    assert_close(host(y_m), O.up_proj(mo, wuv), what="plain MLA up-projected output")
