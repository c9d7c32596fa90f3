"""GPU parity of the projection step in front of the attention: hidden
states -> cache rows [c ; RoPE(k_R)] appended at caller-chosen rows, and
absorbed queries [W_UK q_nope ; RoPE(q_rope)], against the fp64 oracle; then
a decode loop driven by it (project, append, condense each completed group,
attend), against the oracle's incremental decode on the same rows."""
import numpy as np
import pytest
import torch

import lca_inputs as li
import mla_latent_kv_lca_amd as lca
from oracle import lca_oracle as O
from tests.gpu_util import AnchorTally, assert_close, dev, host

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _within(got, ref, rel, floor, what):
    """|got - ref| <= rel |ref| + floor * rms(ref), element by element. For
    outputs stored in bf16 (values of a few units, whose half-ulp alone is
    above 1e-2) rel = 2^-8 covers the storage rounding (2^-9 relative) with
    room for the fp32 accumulation; the floor covers values near zero."""
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + floor * float(np.sqrt(np.mean(ref ** 2)))
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, f"{what}: {bad.size} of {err.size} elements out of bound, worst {err.max():.3e}"


def _absorbed_within(got, ref, x, w, wuk, what):
    """The absorbed query parts, element by element, against a bound that
    holds for any number of elements: the kernels round q_nope to bf16 (unit
    roundoff u = 2^-9) before the W_UK product, which moves output j by at
    most u * sum_k |W_UK[h][j][k]| |q_nope[k]|; storing the result in bf16
    adds at most u |ref|; fp32 accumulation adds far less than the 1e-4
    floor."""
    H = wuk.shape[0]
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    bound = np.empty(ref.shape)
    for h in range(H):
        qn = np.abs(y[:, 576 + 192 * h:576 + 192 * h + 128])
        bound[:, h] = 2.0 ** -9 * (qn @ np.abs(np.asarray(wuk[h], dtype=np.float64)).T)
    bound = 1.01 * bound + 2.0 ** -8 * np.abs(ref) + 1e-4
    err = np.abs(got - ref)
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, f"{what}: {bad.size} of {err.size} elements out of bound, worst {err.max():.3e}"


def _project_gpu(x, pos, w, wuk, dst, n_rows, q_dtype):
    T = x.shape[0]
    H = wuk.shape[0]
    rows = torch.full((n_rows, 576), SENTINEL, dtype=torch.bfloat16, device="cuda")
    q = torch.full((T, H, 576), float("nan"), dtype=q_dtype, device="cuda")
    lca.lca_project(dev(x), dev(pos, torch.int32), dev(w), dev(wuk), rows, dev(dst, torch.int64), q)
    torch.cuda.synchronize()
    return host(rows), host(q)


@pytest.mark.parametrize("T,d,H,q_dtype", [(300, 256, 16, torch.bfloat16),   # 3 token tiles, ragged tail
                                           (37, 2048, 16, torch.float32),    # a decode batch (few-token kernel)
                                           (64, 512, 16, torch.bfloat16),    # few-token kernel, two token chunks
                                           (5, 256, 3, torch.float32),       # few-token kernel, odd H
                                           (129, 96, 3, torch.float32),      # odd H: half-used rotary block
                                           (4000, 256, 16, torch.bfloat16),  # 256-wide tiles, ragged last tile
                                           (11600, 64, 3, torch.float32),    # 256-wide tiles, odd H, f32 queries
                                           (1, 32, 1, torch.bfloat16)])      # one token, one k slice
def test_project_matches_oracle(T, d, H, q_dtype):
    seed = 60 + H
    x = li.hidden_states(seed, T, d)
    w = li.w_proj(seed, H, d)
    wuk = li.w_uk(seed, H)
    r = np.random.default_rng(seed)
    pos = r.integers(0, 1 << 20, T).astype(np.int32)
    pos[0] = 0
    if T > 2:
        pos[1], pos[2] = 131071, -5
    n_rows = T + 9
    dst = r.permutation(n_rows)[:T].astype(np.int64)
    if T > 4:
        dst[3] = -1  # this token's row is not written
    rows, q = _project_gpu(x, pos, w, wuk, dst, n_rows, q_dtype)
    ref_rows, ref_q = O.project(x, pos, w.T, wuk, H)

    written = dst >= 0
    got_rows = rows[dst[written]]
    _within(got_rows, ref_rows[written], 2.0 ** -8, 1e-3, "cache rows")
    untouched = np.setdiff1d(np.arange(n_rows), dst[written])
    assert np.all(rows[untouched] == SENTINEL), "rows outside dst_row were written"
    _within(q[..., 512:], ref_q[..., 512:], 2.0 ** -8, 1e-3, "rotated query part")
    _absorbed_within(q[..., :512], ref_q[..., :512], x, w, wuk, "absorbed query part")
    if q_dtype == torch.float32:
        assert_close(q, ref_q, what="absorbed queries")


def test_project_rotary_part_is_relative():
    """Same hidden state at positions p and p + D: the query's rotary part
    dotted with the key's rotary part depends on the distance only."""
    d, H = 64, 1
    x1 = li.hidden_states(70, 1, d)
    x = np.repeat(x1, 4, axis=0)
    pos = np.array([10, 10 + 300, 5000, 5000 + 300], dtype=np.int32)
    w = li.w_proj(70, H, d)
    wuk = li.w_uk(70, H)
    rows, q = _project_gpu(x, pos, w, wuk, np.arange(4, dtype=np.int64), 4, torch.float32)
    # query of token 1 (p + 300) against key of token 0 (p), at two offsets p
    a = q[1, 0, 512:] @ rows[0, 512:]
    b = q[3, 0, 512:] @ rows[2, 512:]
    assert abs(a - b) <= 2e-2 * max(1.0, abs(a)), (a, b)


def test_projected_incremental_decode_loop():
    """The decode loop from hidden states: a prompt of L0 tokens is projected
    into the cache in one call; every step projects one token (its row is
    appended after the step's attention, its query joins the history), every
    completed group beyond the window is condensed with the last g queries."""
    L0, S, w_, g, d, H = 1300, 40, 1024, 16, 256, 16
    sm = 0.35
    x = li.hidden_states(71, L0 + S, d)
    wp = li.w_proj(71, H, d)
    wuk = li.w_uk(71, H)
    pos = np.arange(L0 + S, dtype=np.int32)
    x_t, wp_t, wuk_t = dev(x), dev(wp), dev(wuk)
    pos_t = dev(pos, torch.int32)
    cache = torch.zeros((1, L0 + S, 576), dtype=torch.bfloat16, device="cuda")
    q_prompt = torch.empty((L0, H, 576), dtype=torch.bfloat16, device="cuda")
    qall = torch.empty((1, g + S, H, 576), dtype=torch.bfloat16, device="cuda")
    lca.lca_project(x_t[:L0], pos_t[:L0], wp_t, wuk_t, cache[0],
                    torch.arange(L0, dtype=torch.int64, device="cuda"), q_prompt)
    qall[0, :g] = q_prompt[L0 - g:]
    m_cap = O.plan(L0 + S, w_, g)["m"]
    reps = torch.empty((1, m_cap, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.empty((1, m_cap), dtype=torch.int32, device="cuda")
    L = L0
    m = O.plan(L, w_, g)["m"]
    lca.lca_condense(lca.packed_latent(cache), 1, g, 0, m, qall, 0, 0, sm, lca.packed_latent(reps), anchor)
    o = torch.empty((1, H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws = lca.decode_workspace(1, H, L0 + S)
    outs = []
    for st in range(S):
        t = L0 + st
        lca.lca_project(x_t[t:t + 1], pos_t[t:t + 1], wp_t, wuk_t, cache[0],
                        torch.full((1,), t, dtype=torch.int64, device="cuda"), qall[0, g + st:g + st + 1])
        lca.mla_latent_attn_decode(qall[:, g + st], lca.packed_latent(reps) if m else None, m,
                                   lca.packed_latent(cache), m * g, L, sm, o, lse, ws)
        outs.append(o.clone())
        L += 1
        if L - w_ >= (m + 1) * g:
            lca.lca_condense(lca.packed_latent(cache), 1, g, m, 1, qall, st + 1, 0, sm,
                             lca.packed_latent(reps), anchor)
            m += 1
    torch.cuda.synchronize()

    # the projection itself, for every token
    ref_rows, ref_q = O.project(x, pos, wp.T, wuk, H)
    rows = host(cache)[0]
    _within(rows, ref_rows, 2.0 ** -8, 1e-3, "projected cache rows")
    qh = host(qall)[0]
    _within(qh[g:, :, 512:], ref_q[L0:, :, 512:], 2.0 ** -8, 1e-3, "projected step queries, rotary part")
    _absorbed_within(qh[g:, :, :512], ref_q[L0:, :, :512], x[L0:], wp, wuk, "projected step queries, absorbed part")
    # the loop, on the rows and queries the GPU produced
    ro, _, _, _, m_ref = O.decode_loop(rows[:L0, :512], rows[:L0, 512:], qh[:g], qh[g:],
                                       rows[L0:, :512], rows[L0:, 512:], w_, g, sm)
    assert m == m_ref
    assert_close(np.stack([host(v)[0] for v in outs]), ro, what="projected decode loop o_latent")


# 3 sequences: 43 splits, so the step runs as its own launch after the merge;
# 8 sequences: 22 splits, so it runs inside the merge / W_UV launch
@pytest.mark.parametrize("L0s", [[1300, 1111, 1057], [1300, 1111, 1057, 1024, 1200, 1033, 1150, 1090]])
def test_projected_decode_step_graph_ragged_paged(L0s):
    """One projected decode step as a fixed launch sequence with its state on
    the device (lca_project -> mla_latent_attn_decode_paged ->
    lca_condense_step), captured once as a HIP graph and replayed for every
    step of a ragged batch on shuffled 64-row pages, so that the sequences
    complete groups at different steps. Per sequence: the step outputs
    against the oracle's incremental loop on the rows and queries the GPU
    produced; the final state, and the representatives and anchors
    condensed during the loop. The same loop with the fused step call
    (mla_latent_attn_decode_paged_up_step) is bitwise equal, and its W_UV
    outputs match the oracle's up-projection."""
    S, w_, g, d, H, P = 40, 1024, 16, 256, 16, 64
    sm = 0.35
    B = len(L0s)
    cap = max(L0s) + S + 1                       # tokens mapped per sequence (the state looks one token ahead)
    n_pg = -(-cap // P)
    perm = np.random.default_rng(81).permutation(B * n_pg).astype(np.int32)
    table = torch.from_numpy(perm.reshape(B, n_pg)).cuda()
    pool = torch.zeros((B * n_pg, P, 576), dtype=torch.bfloat16, device="cuda")
    rows_flat = pool.view(-1, 576)
    cache = lca.paged_latent(pool, table)

    def phys(b, t):
        return int(perm[b * n_pg + t // P]) * P + t % P

    wp, wuk = li.w_proj(81, H, d), li.w_uk(81, H)
    wp_t, wuk_t = dev(wp), dev(wuk)
    xs = [li.hidden_states(82 + b, L0s[b] + S, d) for b in range(B)]
    ring = torch.empty((B, g, H, 576), dtype=torch.bfloat16, device="cuda")
    q_hist = []
    for b in range(B):                           # prompts into their pages; their last g queries fill the ring
        L0 = L0s[b]
        qp = torch.empty((L0, H, 576), dtype=torch.bfloat16, device="cuda")
        dst = torch.tensor([phys(b, t) for t in range(L0)], dtype=torch.int64, device="cuda")
        lca.lca_project(dev(xs[b][:L0]), torch.arange(L0, dtype=torch.int32, device="cuda"), wp_t, wuk_t,
                        rows_flat, dst, qp)
        for t in range(L0 - g, L0):
            ring[b, t % g] = qp[t]
        q_hist.append(qp[L0 - g:].clone())
    m0 = [O.plan(L, w_, g)["m"] for L in L0s]
    m_cap = O.plan(max(L0s) + S, w_, g)["m"] + 1
    reps = torch.zeros((B, m_cap, 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.full((B, m_cap), -1, dtype=torch.int32, device="cuda")
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")  # noqa: E731
    lca.lca_condense_paged(cache, B, g, i32([0] * B), i32(m0), max(m0), ring, 0, sm, lca.packed_latent(reps),
                           anchor)
    state0 = (i32(m0), i32([m * g for m in m0]), i32(L0s), i32(L0s),
              torch.tensor([phys(b, L0s[b]) for b in range(B)], dtype=torch.int64, device="cuda"))
    ring0, reps0, anchor0 = ring.clone(), reps.clone(), anchor.clone()
    x_step = torch.empty((B, d), dtype=torch.bfloat16, device="cuda")
    q_step = torch.empty((B, H, 576), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")
    y = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    wuv = li.w_uv(81, H)
    wuv_t = dev(wuv)
    max_entries = max(m0) + cap
    ws_dec = lca.decode_workspace(B, H, max_entries)
    ws_proj = torch.empty(lca.lca_project_workspace_size(B, H), dtype=torch.uint8, device="cuda")
    x_all = [dev(xs[b]) for b in range(B)]

    def run(fused):
        """The loop from the same initial state: unfused = decode_paged then
        lca_condense_step; fused = mla_latent_attn_decode_paged_up_step."""
        seq_m, seq_rb, seq_re, pos, dst_row = (t.clone() for t in state0)
        ring.copy_(ring0)
        reps.copy_(reps0)
        anchor.copy_(anchor0)
        reps_l = lca.packed_latent(reps)

        def step():
            lca.lca_project(x_step, pos, wp_t, wuk_t, rows_flat, dst_row, q_step, workspace=ws_proj)
            if fused:
                lca.mla_latent_attn_decode_paged_up_step(q_step, reps_l, seq_m, cache, seq_rb, seq_re, max_entries,
                                                         sm, o, wuv_t, y, w_, g, ring, anchor, pos, dst_row,
                                                         workspace=ws_dec)
            else:
                lca.mla_latent_attn_decode_paged(q_step, reps_l, seq_m, cache, seq_rb, seq_re, max_entries, sm, o,
                                                 workspace=ws_dec)
                lca.lca_condense_step(cache, w_, g, q_step, ring, sm, reps_l, anchor, seq_m, seq_rb, seq_re, pos,
                                      dst_row)

        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        outs, qs, ys = [], [], []
        for st in range(S):
            for b in range(B):
                x_step[b].copy_(x_all[b][L0s[b] + st])
            graph.replay()
            outs.append(o.clone())
            qs.append(q_step.clone())
            ys.append(y.clone())
        torch.cuda.synchronize()
        return outs, qs, ys, (seq_m, seq_rb, seq_re, pos, dst_row), reps.clone(), anchor.clone()

    outs_f, _, ys_f, state_f, reps_f, anchor_f = run(True)
    outs, qs, _, (seq_m, seq_rb, seq_re, pos, dst_row), reps, anchor = run(False)
    # the fused call is bitwise the two calls in sequence
    assert all(torch.equal(a, b) for a, b in zip(outs_f, outs))
    assert all(torch.equal(a, b) for a, b in zip(state_f, (seq_m, seq_rb, seq_re, pos, dst_row)))
    assert torch.equal(reps_f, reps) and torch.equal(anchor_f, anchor)

    pool_h = host(pool).reshape(-1, 576)
    reps_h, anchor_h = host(reps), host(anchor).astype(np.int64)
    tally = AnchorTally()
    for b in range(B):
        L0 = L0s[b]
        rows = pool_h[[phys(b, t) for t in range(L0 + S)]]
        steps_q = np.stack([host(v[b]) for v in qs])
        ro, _, rc_ref, rk_ref, m_ref = O.decode_loop(rows[:L0, :512], rows[:L0, 512:], host(q_hist[b]), steps_q,
                                                     rows[L0:, :512], rows[L0:, 512:], w_, g, sm)
        assert_close(np.stack([host(v[b]) for v in outs]), ro, what=f"step outputs, sequence {b}")
        assert_close(np.stack([host(v[b]) for v in ys_f]), O.up_proj(ro, wuv),
                     what=f"fused step W_UV outputs, sequence {b}")
        assert host(seq_m)[b] == m_ref and host(seq_rb)[b] == m_ref * g and host(seq_re)[b] == L0 + S
        assert host(pos)[b] == L0 + S and host(dst_row)[b] == phys(b, L0 + S)
        new = slice(m0[b], m_ref)               # the groups the loop condensed
        assert m_ref > m0[b]
        assert_close(reps_h[b, new, :512], rc_ref[new], what=f"loop representatives, sequence {b}")
        np.testing.assert_array_equal(reps_h[b, new, 512:], rows[anchor_h[b, new], 512:])
        allq = np.concatenate([host(q_hist[b]), steps_q])   # history, then one query per step
        for j in range(m0[b], m_ref):           # anchors: the oracle's argmax wherever it is clear
            st = (j + 1) * g + w_ - L0 - 1     # the step after which group j completes
            _, _, _, a_ref, sc = O.condense_group(rows[j * g:(j + 1) * g, :512], rows[j * g:(j + 1) * g, 512:],
                                                  O.summary_query(allq[st + 1:st + 1 + g]), sm)
            tally.add(anchor_h[b, j:j + 1] - j * g, np.array([a_ref]), O.top2_margin(sc)[None])
    tally.check()


@pytest.mark.parametrize("T", [32, 4096])
def test_project_benchmark_sizes_sampled(T):
    """The benchmark's projection calls (d_model 2,048, H 16; a decode batch of
    32 tokens and a prefill chunk of 4,096 at positions after a 32K context),
    checked on sampled tokens against the oracle."""
    d, H = 2048, 16
    x = li.hidden_states(72, T, d)
    w = li.w_proj(72, H, d)
    wuk = li.w_uk(72, H)
    pos = np.arange(32768, 32768 + T, dtype=np.int32)
    dst = np.arange(T, dtype=np.int64)
    rows, q = _project_gpu(x, pos, w, wuk, dst, T, torch.bfloat16)
    sample = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(73).integers(0, T, 24)]))
    ref_rows, ref_q = O.project(x[sample], pos[sample], w.T, wuk, H)
    _within(rows[sample], ref_rows, 2.0 ** -8, 1e-3, "cache rows")
    _within(q[sample][..., 512:], ref_q[..., 512:], 2.0 ** -8, 1e-3, "rotated query part")
    _absorbed_within(q[sample][..., :512], ref_q[..., :512], x[sample], w, wuk, "absorbed query part")


@pytest.mark.parametrize("T,q_dtype", [(8230, torch.bfloat16),   # 17 tiles of 32 tokens on two workgroups
                                       (6170, torch.float32)])   # 13 tiles on one workgroup, ragged tail
def test_project_absorption_in_batches(T, q_dtype):
    """The absorption's workgroups hold at most 16 (bf16 output) or 12 (f32)
    token tiles of q_nope at once; at these sizes some of them take a second
    batch (and the last, partial tile), checked on every token."""
    d, H = 64, 16
    x = li.hidden_states(76, T, d)
    w = li.w_proj(76, H, d)
    wuk = li.w_uk(76, H)
    pos = np.arange(T, dtype=np.int32)
    dst = np.arange(T, dtype=np.int64)
    rows, q = _project_gpu(x, pos, w, wuk, dst, T, q_dtype)
    ref_rows, ref_q = O.project(x, pos, w.T, wuk, H)
    _within(rows, ref_rows, 2.0 ** -8, 1e-3, "cache rows")
    _within(q[..., 512:], ref_q[..., 512:], 2.0 ** -8, 1e-3, "rotated query part")
    _absorbed_within(q[..., :512], ref_q[..., :512], x, w, wuk, "absorbed query part")


def test_project_strided_inputs_and_outputs():
    """Hidden states with a token stride wider than d_model, absorbed queries
    written into every other slot of a history buffer, cache rows into a
    strided pool: the same values as the dense call."""
    T, d, H = 300, 128, 16
    x = li.hidden_states(74, T, d)
    w = li.w_proj(74, H, d)
    wuk = li.w_uk(74, H)
    pos = np.arange(T, dtype=np.int32) * 3
    xw = torch.zeros((T, d + 40), dtype=torch.bfloat16, device="cuda")
    xw[:, :d] = dev(x)
    pool = torch.full((T, 2, 640), SENTINEL, dtype=torch.bfloat16, device="cuda")  # row stride 1,280
    qbuf = torch.full((T, 2, H, 576), float("nan"), dtype=torch.bfloat16, device="cuda")
    dst = torch.arange(T, dtype=torch.int64, device="cuda")
    lca.lca_project(xw[:, :d], dev(pos, torch.int32), dev(w), dev(wuk), pool[:, 0, :576], dst, qbuf[:, 0])
    rows_d, q_d = _project_gpu(x, pos, w, wuk, np.arange(T, dtype=np.int64), T, torch.bfloat16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(pool[:, 0, :576]), rows_d)
    np.testing.assert_array_equal(host(qbuf[:, 0]), q_d)
    assert np.all(host(pool[:, 0, 576:]) == SENTINEL) and np.all(host(pool[:, 1]) == SENTINEL)
    assert np.isnan(host(qbuf[:, 1])).all()
