"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here runs the oracle against itself: each test checks a value the
pages print, a hand-derived closed form, an invariant of the definition, or a
special case that reduces to a library routine (torch's scaled-dot-product
attention in float64, numpy's least squares / mean / argmax).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import lca_inputs as li
from oracle import lca_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _num(s):
    return float(eval(s, {"ln": math.log}))  # fixture strings like "ln(3)/4", "3/7"


# ------------------------------------------------------------ grouping ------
def test_plan_counts_golden():
    gold = _load("plan_counts.json")
    for case in gold["cases"]:
        p = O.plan(case["L"], case["w"], case["g"])
        assert p["m"] == case["m"], case
        assert p["raw_begin"] == case["m"] * case["g"]
        assert p["n_entries"] == case["m"] + case["L"] - case["m"] * case["g"]
    cc = gold["compression_128k"]
    comp = 1.0 - O.kept_fraction(cc["L"], cc["w"], cc["g"])
    assert abs(comp - cc["claimed_compression"]) <= cc["tolerance"]


def test_plan_window_covers_all():
    for L in (0, 1, 5, 1023, 1024):
        p = O.plan(L, 1024, 16)
        assert p["m"] == 0 and p["raw_begin"] == 0 and p["n_entries"] == L
    # every token is either in a group or raw, and the raw part holds >= w tokens
    for L in range(1024, 1300, 7):
        p = O.plan(L, 1024, 16)
        assert p["m"] * 16 + (L - p["raw_begin"]) == L
        assert 1024 <= L - p["raw_begin"] < 1024 + 16


# -------------------------------------------------------- condensation ------
def _worked_rows(g=4):
    c = np.zeros((g, 512))
    k = np.zeros((g, 64))
    for i in range(g):
        c[i, i] = 4.0
        k[i, 0] = i + 1.0
    return c, k


def _queries_with_mean(qbar, g, H, seed=0):
    r = np.random.default_rng(seed)
    q = np.zeros((g, H, 576))
    for t in range(g):
        d = r.standard_normal(576)
        q[t, 0] = qbar + d
        q[t, 1] = qbar - d
    return q


def test_condense_worked_example_golden():
    gold = _load("condense_worked_example.json")
    g, H = gold["g"], gold["H"]
    c, k = _worked_rows(g)
    qbar = np.zeros(576)
    qbar[:4] = [_num(x) for x in gold["qbar_latent_head"]]
    q = _queries_with_mean(qbar, g, H)
    L = g
    rc, rk, anc, alpha, s = O.condense(c[None], k[None], q[None], g, 0, 1, 0, 0, gold["sm_scale"])
    ex = gold["expected"]
    np.testing.assert_allclose(s[0, 0], [_num(x) for x in ex["scores"]], atol=1e-12)
    np.testing.assert_allclose(alpha[0, 0], [_num(x) for x in ex["alpha"]], atol=1e-12)
    want_c = np.zeros(512)
    want_c[:4] = [_num(x) for x in ex["c_rep_head"]]
    np.testing.assert_allclose(rc[0, 0], want_c, atol=1e-12)
    assert anc[0, 0] == ex["anchor"]
    want_k = np.zeros(64)
    want_k[0] = _num(ex["k_rep_head"][0])
    np.testing.assert_allclose(rk[0, 0], want_k, atol=0)
    assert L == g
    # tie: lowest index wins
    qbar2 = np.zeros(576)
    qbar2[:2] = 0.25
    _, rk2, anc2, a2, _ = O.condense(c[None], k[None], _queries_with_mean(qbar2, g, H)[None],
                                     g, 0, 1, 0, 0, 1.0)
    assert anc2[0, 0] == gold["tie_case"]["anchor"]
    e = math.e
    np.testing.assert_allclose(a2[0, 0], np.array([e, e, 1, 1]) / (2 * e + 2), atol=1e-12)


def test_condense_modes_worked_example_golden():
    """The 消融实验 variants on the hand-derived group (golden values)."""
    gold = _load("condense_worked_example.json")
    g, H = gold["g"], gold["H"]
    c, k = _worked_rows(g)
    qbar = np.zeros(576)
    qbar[:4] = [_num(x) for x in gold["qbar_latent_head"]]
    q = _queries_with_mean(qbar, g, H)
    for mode, key in ((O.MODE_POOL_ROPE, "pool_rope"), (O.MODE_ANCHOR, "anchor")):
        rc, rk, anc, alpha, _ = O.condense(c[None], k[None], q[None], g, 0, 1, 0, 0, gold["sm_scale"], mode)
        ex = gold["modes"][key]
        want_c = np.zeros(512)
        want_c[:4] = [_num(x) for x in ex["c_rep_head"]]
        np.testing.assert_allclose(rc[0, 0], want_c, atol=1e-12)
        want_k = np.zeros(64)
        want_k[0] = _num(ex["k_rep_head"][0])
        np.testing.assert_allclose(rk[0, 0], want_k, atol=1e-12)
        assert anc[0, 0] == gold["expected"]["anchor"]
        np.testing.assert_allclose(alpha[0, 0], [_num(x) for x in gold["expected"]["alpha"]], atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_pool_rope_mode_is_weighted_mean_with_limits(seed):
    """Pooled RoPE key: the alpha-weighted mean (sum_i alpha_i (k_i - k_rep) = 0);
    sm_scale -> 0 gives the plain mean, sm_scale -> inf the anchor's key."""
    c, k, qb = _rand_group(seed, scale=0.5)
    cr, kk, a, anc, _ = O.condense_group(c, k, qb, 1.0, O.MODE_POOL_ROPE)
    np.testing.assert_allclose((a[:, None] * (k - kk)).sum(axis=0), 0.0, atol=1e-12)
    cr_lca, kk_lca, _, anc_lca, _ = O.condense_group(c, k, qb, 1.0, O.MODE_LCA)
    np.testing.assert_array_equal(cr, cr_lca)  # the latent pool is unchanged
    assert anc == anc_lca
    # with spread-out weights the pooled key really differs from the anchor's
    _, kk_s, _, _, _ = O.condense_group(c, k, qb, 0.05, O.MODE_POOL_ROPE)
    _, kk_a, _, _, _ = O.condense_group(c, k, qb, 0.05, O.MODE_LCA)
    assert np.max(np.abs(kk_s - kk_a)) > 0.1
    _, k0, _, _, _ = O.condense_group(c, k, qb, 1e-12, O.MODE_POOL_ROPE)
    np.testing.assert_allclose(k0, k.mean(axis=0), atol=1e-10)
    _, kinf, _, ainf, _ = O.condense_group(c, k, qb, 1e4, O.MODE_POOL_ROPE)
    np.testing.assert_allclose(kinf, k[ainf], atol=1e-9)


@pytest.mark.parametrize("seed", range(3))
def test_anchor_mode_keeps_the_anchor_row(seed):
    """Pure sparse: the representative is the most important token's own row,
    whatever the softmax scale."""
    c, k, qb = _rand_group(seed, scale=0.5)
    s = np.concatenate([c, k], axis=1) @ qb
    i = int(np.argmax(s))
    for sm in (1e-6, 1.0, 30.0):
        cr, kk, a, anc, _ = O.condense_group(c, k, qb, sm, O.MODE_ANCHOR)
        assert anc == i
        np.testing.assert_array_equal(cr, c[i])
        np.testing.assert_array_equal(kk, k[i])
        assert abs(a.sum() - 1.0) <= 1e-12


def test_all_modes_agree_on_singletons_and_identical_rows():
    r = np.random.default_rng(11)
    c1, k1, qb = r.standard_normal((1, 512)), r.standard_normal((1, 64)), r.standard_normal(576)
    row_c, row_k = r.standard_normal(512), r.standard_normal(64)
    for mode in (O.MODE_LCA, O.MODE_POOL_ROPE, O.MODE_ANCHOR):
        cr, kk, a, anc, _ = O.condense_group(c1, k1, qb, 1.0, mode)
        np.testing.assert_array_equal(cr, c1[0])
        np.testing.assert_array_equal(kk, k1[0])
        cr, kk, _, anc, _ = O.condense_group(np.tile(row_c, (16, 1)), np.tile(row_k, (16, 1)), qb, 1.0, mode)
        np.testing.assert_allclose(cr, row_c, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(kk, row_k, rtol=1e-14, atol=1e-14)
        assert anc == 0


def _rand_group(seed, g=16, scale=1.0):
    r = np.random.default_rng(seed)
    return r.standard_normal((g, 512)), r.standard_normal((g, 64)), r.standard_normal(576) * scale


@pytest.mark.parametrize("seed", range(5))
def test_weights_sum_to_one_and_nonnegative(seed):
    c, k, qb = _rand_group(seed, scale=0.3)
    for sm in (0.0, 0.1, 1.0, 7.0):
        _, _, a, _, _ = O.condense_group(c, k, qb, sm)
        assert np.all(a >= 0)
        assert abs(a.sum() - 1.0) <= 1e-12


def test_identical_rows_pool_to_row():
    r = np.random.default_rng(3)
    row_c, row_k = r.standard_normal(512), r.standard_normal(64)
    c = np.tile(row_c, (16, 1))
    k = np.tile(row_k, (16, 1))
    cr, kk, a, anc, _ = O.condense_group(c, k, r.standard_normal(576), 1.0)
    np.testing.assert_allclose(cr, row_c, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(kk, row_k)
    assert anc == 0
    np.testing.assert_allclose(a, np.full(16, 1 / 16), atol=1e-15)


@pytest.mark.parametrize("seed", range(3))
def test_prop1_pool_is_weighted_least_squares(seed):
    """Proposition 1: c_rep minimises sum_i alpha_i |c_i - r|^2 (solved by lstsq)."""
    c, k, qb = _rand_group(seed, scale=0.5)
    cr, _, a, _, _ = O.condense_group(c, k, qb, 1.0)
    sw = np.sqrt(a)[:, None]
    A = np.repeat(sw, 1, axis=1)  # [g, 1] design: every row predicts r
    # minimise sum_i |sqrt(a_i) (c_i - r)|^2 column by column: A r = sqrt(a) c
    r_ls = np.linalg.lstsq(A, sw * c, rcond=None)[0][0]
    np.testing.assert_allclose(cr, r_ls, atol=1e-12)
    obj = lambda r: float((a[:, None] * (c - r) ** 2).sum())  # noqa: E731
    rng = np.random.default_rng(seed + 10)
    for _ in range(5):
        assert obj(cr + 1e-3 * rng.standard_normal(512)) > obj(cr)


@pytest.mark.parametrize("seed", range(3))
def test_scale_limits_mean_pool_and_pure_sparse(seed):
    c, k, qb = _rand_group(seed, scale=0.5)
    cr0, _, _, _, _ = O.condense_group(c, k, qb, 1e-12)
    np.testing.assert_allclose(cr0, np.mean(c, axis=0), atol=1e-10)
    s_lib = np.concatenate([c, k], axis=1) @ qb
    i_lib = int(np.argmax(s_lib))
    crinf, kinf, _, anc, _ = O.condense_group(c, k, qb, 1e4)
    assert anc == i_lib
    np.testing.assert_allclose(crinf, c[i_lib], atol=1e-9)
    np.testing.assert_array_equal(kinf, k[i_lib])


def test_permutation_moves_anchor_with_its_row():
    c, k, qb = _rand_group(7, scale=0.5)
    cr, kk, a, anc, _ = O.condense_group(c, k, qb, 1.0)
    perm = np.random.default_rng(8).permutation(16)
    cr2, kk2, a2, anc2, _ = O.condense_group(c[perm], k[perm], qb, 1.0)
    np.testing.assert_allclose(cr2, cr, atol=1e-12)
    np.testing.assert_array_equal(kk2, kk)
    assert perm[anc2] == anc
    np.testing.assert_allclose(a2, a[perm], atol=1e-15)


def test_top2_margin_hand_values():
    """The anchor-parity rule (anchors must agree where the largest score
    beats the runner-up by more than 1e-3) rests on top2_margin: the gap
    between the largest and the second-largest score of each group, ties
    counted twice. Hand values: unsorted rows, ties, all-negative scores,
    and batched leading axes."""
    assert O.top2_margin(np.array([3.0, 1.0, 2.0])) == 1.0
    assert O.top2_margin(np.array([0.1, -2.0, 0.7, 0.4])) == pytest.approx(0.3, abs=1e-15)
    assert O.top2_margin(np.array([5.0, 1.0, 5.0])) == 0.0          # tie at the top
    assert O.top2_margin(np.array([-5.0, -1.0, -3.0])) == 2.0       # sign of the values
    assert O.top2_margin(np.array([2.0, 2.0, 2.0, 2.0])) == 0.0     # all equal
    assert O.top2_margin(np.array([7.0, 7.0 - 2e-3])) == pytest.approx(2e-3, abs=1e-15)
    batched = np.array([[[1.0, 4.0, 2.0], [0.0, 0.0, -1.0]],
                        [[9.0, -9.0, 8.5], [1.0, 3.0, 3.0 - 5e-4]]])
    np.testing.assert_allclose(O.top2_margin(batched), [[2.0, 0.0], [0.5, 5e-4]], atol=1e-15)
    # the margin is taken along the last axis only, and is never negative
    r = np.random.default_rng(21).standard_normal((3, 5, 16))
    got = O.top2_margin(r)
    assert got.shape == (3, 5) and np.all(got >= 0)
    i, j = 2, 4
    row = r[i, j]
    top = row.max()
    assert got[i, j] == top - row[row != top].max()


def test_scores_are_mean_textbook_logits():
    """R1-R2: s_i is the mean over g queries and H heads of the textbook MLA
    logit [W_UK^T c_i ; k_i^R] . [q_nope ; q_rope] (keys built explicitly)."""
    r = np.random.default_rng(11)
    g, H = 4, 3
    wuk = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    q_nope = r.standard_normal((g, H, 128))
    q_rope = r.standard_normal((g, H, 64))
    c = r.standard_normal((g, 512))
    kr = r.standard_normal((g, 64))
    logits = np.zeros((g, H, g))  # [query token, head, key token]
    for t in range(g):
        for h in range(H):
            keys = np.concatenate([c @ wuk[h], kr], axis=1)
            logits[t, h] = keys @ np.concatenate([q_nope[t, h], q_rope[t, h]])
    q_abs = np.stack([O.absorb_query(q_nope[t], q_rope[t], wuk) for t in range(g)])
    _, _, _, _, s = O.condense_group(c, kr, O.summary_query(q_abs), 1.0)
    np.testing.assert_allclose(s, logits.mean(axis=(0, 1)), atol=1e-12)


def test_summary_query_uses_the_addressed_rows():
    """Group j must take its summary query from rows q_row0 + (j-gb)*step ...:
    only those rows point at one planted token per group."""
    r = np.random.default_rng(5)
    g, H, n = 4, 2, 3
    L = 4 * g + 8
    c = r.standard_normal((1, L, 512)) * 0.1
    kr = r.standard_normal((1, L, 64)) * 0.1
    T = 40
    q = r.standard_normal((1, T, H, 576)) * 0.01
    gb, row0, step = 1, 7, 9
    target = []
    for nn in range(n):
        j = gb + nn
        tok = j * g + (nn + 1) % g
        target.append(tok)
        dirv = np.concatenate([c[0, tok], kr[0, tok]])
        q[0, row0 + nn * step: row0 + nn * step + g] += 50 * dirv / np.linalg.norm(dirv)
    _, _, anc, _, _ = O.condense(c, kr, q, g, gb, n, row0, step, 1.0)
    assert list(anc[0]) == target


# ------------------------------------------------------------- attention ----
def test_attend_worked_example_golden():
    gold = _load("attend_worked_example.json")
    q = np.zeros((1, 576))
    q[0, 1] = math.log(3) / 2
    ec = np.zeros((2, 512))
    ec[0, 0] = 1
    ec[1, 1] = 1
    o, lse = O.attend(q, ec, np.zeros((2, 64)), gold["sm_scale"])
    want = np.zeros(512)
    want[:2] = [_num(x) for x in gold["expected"]["o_head"]]
    np.testing.assert_allclose(o[0], want, atol=1e-14)
    assert abs(lse[0] - _num(gold["expected"]["lse"])) < 1e-14


def _sdpa(q, k, v, sm_scale, mask=None, causal=False):
    """torch's scaled-dot-product attention, float64 CPU, [H, n, d] inputs."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))  # noqa: E731
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(t(q)[None], t(k)[None], t(v)[None], attn_mask=m,
                                          is_causal=causal, scale=sm_scale)[0].numpy()


def _expanded_heads(c, kr, wuk, wuv):
    """Per-head textbook keys [H, n, 192] and values [H, n, 128]."""
    H = wuk.shape[0]
    k = np.stack([np.concatenate([c @ wuk[h], kr], axis=1) for h in range(H)])
    v = np.stack([c @ wuv[h] for h in range(H)])
    return k, v


@pytest.mark.parametrize("L,w,g", [(24, 24, 4), (24, 100, 4), (37, 8, 1)])
def test_no_condensation_is_exact_mla(L, w, g):
    """w >= L (no group) or g = 1 (singleton groups) reproduces exact MLA,
    checked against textbook attention with explicit W_UK / W_UV heads."""
    r = np.random.default_rng(L + w + g)
    H = 4
    c = r.standard_normal((1, L, 512))
    kr = r.standard_normal((1, L, 64))
    wuk = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    wuv = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    q_nope, q_rope = r.standard_normal((H, 128)) * 0.3, r.standard_normal((H, 64)) * 0.3
    q_abs = O.absorb_query(q_nope, q_rope, wuk)
    qh = r.standard_normal((1, g, H, 576)) * 0.1
    p = O.plan(L, w, g)
    rc, rk, anc, _, _ = O.condense(c, kr, qh, g, 0, p["m"], 0, 0, 0.9)
    o_lat, lse = O.decode(q_abs[None], rc, rk, p["m"], c, kr, p["raw_begin"], L, 0.9)
    out = O.up_proj(o_lat, wuv)[0]
    kh, vh = _expanded_heads(c[0], kr[0], wuk, wuv)
    qe = np.concatenate([q_nope, q_rope], axis=1)[:, None, :]
    ref = _sdpa(qe, kh, vh, 0.9)[:, 0]
    np.testing.assert_allclose(out, ref, atol=1e-12)
    # textbook logsumexp from torch
    z = 0.9 * np.einsum("hd,hnd->hn", qe[:, 0], kh)
    np.testing.assert_allclose(lse[0], torch.logsumexp(torch.from_numpy(z), dim=1).numpy(), atol=1e-12)
    if g == 1:
        assert list(anc[0]) == list(range(p["m"]))


def test_mha_expanded_is_textbook_attention_and_equals_absorbed_form():
    """The oracle's expanded-head MLA equals torch's float64 attention over
    explicit W_UK / W_UV heads, and the absorbed decode + up-projection equals
    it (the absorption identity q_nope . (W_UK^T c) = (W_UK q_nope) . c)."""
    r = np.random.default_rng(33)
    n, H = 29, 3
    c = r.standard_normal((n, 512))
    kr = r.standard_normal((n, 64))
    wuk = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    wuv = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    q_nope, q_rope = r.standard_normal((H, 128)) * 0.4, r.standard_normal((H, 64)) * 0.4
    got = O.mha_expanded(q_nope, q_rope, c, kr, wuk, wuv, 0.8)
    kh, vh = _expanded_heads(c, kr, wuk, wuv)
    ref = _sdpa(np.concatenate([q_nope, q_rope], 1)[:, None], kh, vh, 0.8)[:, 0]
    np.testing.assert_allclose(got, ref, atol=1e-12)
    o_lat, _ = O.decode(O.absorb_query(q_nope, q_rope, wuk)[None], None, None, 0, c[None], kr[None],
                        0, n, 0.8)
    np.testing.assert_allclose(O.up_proj(o_lat, wuv)[0], got, atol=1e-12)


def test_condensed_decode_equals_textbook_attention_over_condensed_set():
    """Tiny-L brute force: the absorbed decode over [reps ++ window] equals
    textbook per-head attention whose keys/values are built from the same
    condensed rows."""
    r = np.random.default_rng(21)
    L, w, g, H = 45, 8, 4, 4
    c = r.standard_normal((1, L, 512))
    kr = r.standard_normal((1, L, 64))
    wuk = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    wuv = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    qh = r.standard_normal((1, 16, H, 576)) * 0.2
    p = O.plan(L, w, g)
    assert p["m"] == 9 and p["raw_begin"] == 36
    rc, rk, anc, alpha, _ = O.condense(c, kr, qh, g, 0, p["m"], 16 - g, 0, 1.3)
    q_nope, q_rope = r.standard_normal((H, 128)) * 0.3, r.standard_normal((H, 64)) * 0.3
    q_abs = O.absorb_query(q_nope, q_rope, wuk)
    o_lat, _ = O.decode(q_abs[None], rc, rk, p["m"], c, kr, p["raw_begin"], L, 1.3)
    out = O.up_proj(o_lat, wuv)[0]
    # condensed set built independently: weighted rows by einsum, anchors by index
    reps_c = np.einsum("ng,ngd->nd", alpha[0], c[0, :36].reshape(9, 4, 512))
    reps_k = kr[0, anc[0]]
    set_c = np.concatenate([reps_c, c[0, 36:]])
    set_k = np.concatenate([reps_k, kr[0, 36:]])
    kh, vh = _expanded_heads(set_c, set_k, wuk, wuv)
    ref = _sdpa(np.concatenate([q_nope, q_rope], 1)[:, None], kh, vh, 1.3)[:, 0]
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_prefill_before_first_group_is_causal_mla():
    """Chunks that start before w + g have m_s = 0: causal textbook attention."""
    r = np.random.default_rng(31)
    L, w, g, H, C = 20, 16, 4, 2, 8
    c = r.standard_normal((L, 512))
    kr = r.standard_normal((L, 64))
    q = r.standard_normal((L, H, 576)) * 0.1
    o, lse, _, _ = O.prefill(q, c, kr, w, g, C, 0.7)
    keys = np.concatenate([c, kr], 1)
    ref = _sdpa(np.transpose(q, (1, 0, 2)), np.broadcast_to(keys, (H, L, 576)),
                np.broadcast_to(c, (H, L, 512)), 0.7, causal=True)
    np.testing.assert_allclose(np.transpose(o, (1, 0, 2)), ref, atol=1e-12)


def test_prefill_chunking_is_invisible_without_groups():
    r = np.random.default_rng(32)
    L, H = 30, 2
    c = r.standard_normal((L, 512))
    kr = r.standard_normal((L, 64))
    q = r.standard_normal((L, H, 576)) * 0.1
    o1, l1, _, _ = O.prefill(q, c, kr, 64, 4, 7, 1.1)
    o2, l2, _, _ = O.prefill(q, c, kr, 64, 4, 30, 1.1)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_prefill_with_groups_matches_masked_textbook_attention():
    """Whole chunked prefill with condensation against textbook attention with
    a boolean mask over [reps ++ raw] per chunk; reps built from the group
    rows, the summary queries of the g following tokens (R6), and numpy's
    softmax-free weighting."""
    r = np.random.default_rng(33)
    L, w, g, H, C = 48, 8, 4, 2, 16
    c = r.standard_normal((L, 512))
    kr = r.standard_normal((L, 64))
    q = r.standard_normal((L, H, 576)) * 0.3
    sm = 0.8
    o, _, rep_c, rep_k = O.prefill(q, c, kr, w, g, C, sm)
    # independent reps: weights from exp of summary logits
    m_final = (32 - w) // g
    assert rep_c.shape[0] == m_final
    for j in range(m_final):
        qbar = q[(j + 1) * g:(j + 2) * g].mean(axis=(0, 1))
        rows = np.concatenate([c[j * g:(j + 1) * g], kr[j * g:(j + 1) * g]], 1)
        s = rows @ qbar
        wts = np.exp(sm * s)
        wts /= wts.sum()
        np.testing.assert_allclose(rep_c[j], wts @ c[j * g:(j + 1) * g], atol=1e-12)
        np.testing.assert_array_equal(rep_k[j], kr[j * g + int(np.argmax(s))])
    for s0 in range(0, L, C):
        ms = (s0 - w) // g if s0 > w else 0
        keys = np.concatenate([np.concatenate([rep_c[:ms], rep_k[:ms]], 1),
                               np.concatenate([c[ms * g:s0 + C], kr[ms * g:s0 + C]], 1)])
        vals = np.concatenate([rep_c[:ms], c[ms * g:s0 + C]])
        n = keys.shape[0]
        mask = np.ones((C, n), dtype=bool)
        for i in range(C):
            mask[i, ms + (s0 + i - ms * g) + 1:] = False
        ref = _sdpa(np.transpose(q[s0:s0 + C], (1, 0, 2)), np.broadcast_to(keys, (H, n, 576)),
                    np.broadcast_to(vals, (H, n, 512)), sm, mask=mask)
        np.testing.assert_allclose(np.transpose(o[s0:s0 + C], (1, 0, 2)), ref, atol=1e-12)


def test_decode_loop_singletons_is_exact_mla():
    """Incremental decode with g = 1 keeps every token (singleton reps)."""
    r = np.random.default_rng(41)
    L0, S, H, w = 12, 6, 2, 4
    c0, k0 = r.standard_normal((L0, 512)), r.standard_normal((L0, 64))
    qh = r.standard_normal((3, H, 576)) * 0.1
    sq = r.standard_normal((S, H, 576)) * 0.1
    nc, nk = r.standard_normal((S, 512)), r.standard_normal((S, 64))
    o, lse, _, _, m = O.decode_loop(c0, k0, qh, sq, nc, nk, w, 1, 0.6)
    assert m == L0 + S - w
    for st in range(S):
        cc = np.concatenate([c0, nc[:st]])
        kk = np.concatenate([k0, nk[:st]])
        keys = np.concatenate([cc, kk], 1)
        ref = _sdpa(sq[st][:, None], np.broadcast_to(keys, (H,) + keys.shape),
                    np.broadcast_to(cc, (H,) + cc.shape), 0.6)[:, 0]
        np.testing.assert_allclose(o[st], ref, atol=1e-12)


def test_decode_loop_freezes_reps_and_uses_recent_queries():
    r = np.random.default_rng(42)
    L0, S, H, w, g = 20, 9, 2, 8, 4
    c0, k0 = r.standard_normal((L0, 512)), r.standard_normal((L0, 64))
    qh = r.standard_normal((5, H, 576)) * 0.2
    sq = r.standard_normal((S, H, 576)) * 0.2
    nc, nk = r.standard_normal((S, 512)), r.standard_normal((S, 64))
    _, _, rc, rk, m = O.decode_loop(c0, k0, qh, sq, nc, nk, w, g, 0.9)
    Lf = L0 + S
    assert m == (Lf - w) // g == 5
    allc = np.concatenate([c0, nc])
    allk = np.concatenate([k0, nk])
    allq = np.concatenate([qh, sq])
    # groups 0..2 exist at start (L0=20 -> m=3) and use the last g history rows
    qb0 = qh[-g:].mean(axis=(0, 1))
    for j in range(3):
        rows = np.concatenate([allc[j * g:(j + 1) * g], allk[j * g:(j + 1) * g]], 1)
        wts = np.exp(0.9 * (rows @ qb0))
        np.testing.assert_allclose(rc[j], (wts / wts.sum()) @ allc[j * g:(j + 1) * g], atol=1e-12)
    # group 3 completes when L reaches 8 + 16 = 24, i.e. after step index 3
    # (4 rows appended); its summary query is queries up to and incl. step 3
    qb3 = allq[5 + 3 - g + 1:5 + 3 + 1].mean(axis=(0, 1))
    rows = np.concatenate([allc[12:16], allk[12:16]], 1)
    wts = np.exp(0.9 * (rows @ qb3))
    np.testing.assert_allclose(rc[3], (wts / wts.sum()) @ allc[12:16], atol=1e-12)


def test_up_proj_worked():
    """o[t,h] = o_latent[t,h] @ W_UV[h] on unit vectors picks W_UV rows."""
    H = 3
    wuv = np.arange(H * 512 * 128, dtype=np.float64).reshape(H, 512, 128)
    ol = np.zeros((2, H, 512))
    ol[0, 1, 5] = 1.0
    ol[1, 2, 7] = 2.0
    out = O.up_proj(ol, wuv)
    np.testing.assert_array_equal(out[0, 1], wuv[1, 5])
    np.testing.assert_array_equal(out[1, 2], 2 * wuv[2, 7])
    assert not out[0, 0].any() and not out[0, 2].any()


# ------------------------------------------------------------ inputs --------
def test_bf16_round_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e-39], dtype=np.float32)
    y = li.bf16_round(x)
    assert y[0] == 1.0
    assert y[1] == 1.0            # tie -> even mantissa
    assert y[2] == 1.0 + 2 ** -7  # 1.00586 lies above the midpoint 1.00391 -> rounds up
    assert y[3] == -2.5
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(y, ref)


def test_input_recipe_moments():
    c, k = li.latent_cache(9, 2, 256)
    assert c.shape == (2, 256, 512) and k.shape == (2, 256, 64)
    assert abs(c.std() - 1) < 0.02 and abs(k.std() - 1) < 0.05
    q = li.queries(9, 2, 64, 16, rho=0.5)
    assert abs(q.var() * 576 - 1) < 0.1
    np.testing.assert_array_equal(li.latent_cache(9, 2, 256)[0], c)  # seeded


def test_gqa_decode_is_textbook_grouped_attention():
    """R8: with nothing condensed, GQA decode + up-projection equals torch's
    float64 attention with grouped key/value heads (enable_gqa), keys and
    values built explicitly per head through W_UK / W_UV from its group's
    latent rows."""
    r = np.random.default_rng(44)
    B, n_kv, Hg, L = 2, 2, 3, 21
    H = n_kv * Hg
    c = r.standard_normal((B, n_kv, L, 512))
    kr = r.standard_normal((B, n_kv, L, 64))
    wuk = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    wuv = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    q_nope, q_rope = r.standard_normal((B, H, 128)) * 0.4, r.standard_normal((B, H, 64)) * 0.4
    qa = np.stack([O.absorb_query(q_nope[b], q_rope[b], wuk) for b in range(B)])
    o_lat, _ = O.decode_gqa(qa, None, None, 0, c, kr, 0, L, n_kv, 0.9)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))  # noqa: E731
    for b in range(B):
        # head h's key/value from group h // Hg through its own W_UK[h] / W_UV[h]:
        # with grouped SDPA the per-head key must be shared by the group, so
        # compare head by head against single-head attention over that group
        for h in range(H):
            k = h // Hg
            kh = np.concatenate([c[b, k] @ wuk[h], kr[b, k]], axis=1)[None]
            vh = (c[b, k] @ wuv[h])[None]
            qh = np.concatenate([q_nope[b, h], q_rope[b, h]])[None, None]
            ref = F.scaled_dot_product_attention(t(qh)[None], t(kh)[None], t(vh)[None], scale=0.9)[0, 0, 0]
            np.testing.assert_allclose(O.up_proj(o_lat[b:b + 1, h:h + 1], wuv[h:h + 1])[0, 0], ref.numpy(),
                                       atol=1e-12)
    # grouped SDPA over the latent rows themselves (keys [c ; k_R], values c):
    # query heads h of group k share kv head k
    kk = t(np.concatenate([c, kr], axis=-1))            # [B, n_kv, L, 576]
    vv = t(c)                                            # [B, n_kv, L, 512]
    ref = F.scaled_dot_product_attention(t(qa)[:, :, None], kk, vv, scale=0.9, enable_gqa=True)[:, :, 0]
    np.testing.assert_allclose(o_lat, ref.numpy(), atol=1e-12)


def test_gqa_condense_uses_each_groups_own_heads_and_cache():
    """R8: group k's representative equals condensing cache k with the mean of
    heads [k Hg, (k+1) Hg) only (the other groups' queries do not leak in)."""
    r = np.random.default_rng(45)
    B, n_kv, Hg, g, L = 1, 3, 2, 4, 16
    c = r.standard_normal((B, n_kv, L, 512))
    kr = r.standard_normal((B, n_kv, L, 64))
    q = r.standard_normal((B, g, n_kv * Hg, 576)) * 0.2
    rc, rk, anc, al, s = O.condense_gqa(c, kr, q, n_kv, g, 0, 4, 0, 0, 1.0)
    for k in range(n_kv):
        qbar = q[0, :, k * Hg:(k + 1) * Hg].reshape(-1, 576).mean(axis=0)
        for j in range(4):
            rows = np.concatenate([c[0, k, j * g:(j + 1) * g], kr[0, k, j * g:(j + 1) * g]], axis=1)
            sc = rows @ qbar
            np.testing.assert_allclose(s[0, k, j], sc, atol=1e-12)
            a = np.exp(sc - sc.max()) / np.exp(sc - sc.max()).sum()
            np.testing.assert_allclose(rc[0, k, j], a @ c[0, k, j * g:(j + 1) * g], atol=1e-12)
            assert anc[0, k, j] == j * g + int(np.argmax(sc))


def _rope_complex(x, pos, base=10000.0):
    """RoPE written as a complex rotation (an independent formulation): pair
    (x_i, x_{i+32}) is the complex number x_i + j x_{i+32}, multiplied by
    exp(j p theta_i)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    z = torch.complex(t[..., :32], t[..., 32:])
    theta = base ** (-torch.arange(32, dtype=torch.float64) * 2.0 / 64)
    ang = torch.from_numpy(np.asarray(pos, dtype=np.float64))[..., None] * theta
    z = z * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1).numpy()


def test_rope_matches_complex_rotation_and_is_relative():
    r = np.random.default_rng(50)
    x = r.standard_normal((7, 64))
    pos = np.array([0, 1, 5, 1000, 65535, 1 << 20, 3])
    got = O.rope_rotate(x, pos)
    np.testing.assert_allclose(got, _rope_complex(x, pos), atol=1e-12)
    np.testing.assert_allclose(O.rope_rotate(x[:1], [0]), x[:1], atol=0)     # position 0: identity
    np.testing.assert_allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    a, b = r.standard_normal(64), r.standard_normal(64)
    for p1, p2 in ((10, 3), (70000, 69990), (5, 5)):  # <R(p1) a, R(p2) b> depends on p1 - p2 only
        lhs = O.rope_rotate(a[None], [p1])[0] @ O.rope_rotate(b[None], [p2])[0]
        rhs = O.rope_rotate(a[None], [p1 - p2])[0] @ b
        assert abs(lhs - rhs) < 1e-9


def test_projected_decode_is_textbook_attention_from_hidden_states():
    """R9 end to end: project hidden states (cache rows and absorbed queries),
    decode over the cache rows, up-project through W_UV: equals torch's
    float64 attention with per-head keys [W_UK[h]^T c ; RoPE(k^R)] and values
    W_UV[h]^T c built directly from x, with RoPE as a complex rotation."""
    r = np.random.default_rng(51)
    d, H, L = 48, 3, 19
    x = r.standard_normal((L + 1, d))
    pos = np.arange(L + 1) + 1000
    w_cat = r.standard_normal((d, 576 + 192 * H)) / math.sqrt(d)
    w_uk = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    w_uv = r.standard_normal((H, 512, 128)) / math.sqrt(512)
    rows, q_abs = O.project(x, pos, w_cat, w_uk, H)
    # the last token queries the L cached tokens before it
    o_lat, _ = O.decode(q_abs[L][None], None, None, 0, rows[None, :L, :512], rows[None, :L, 512:], 0, L, 0.7)
    got = O.up_proj(o_lat, w_uv)[0]
    y = x @ w_cat
    c = y[:L, :512]
    kr = _rope_complex(y[:L, 512:576], pos[:L])
    qh = y[L, 576:].reshape(H, 192)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))  # noqa: E731
    for h in range(H):
        k = np.concatenate([c @ w_uk[h], kr], axis=1)
        v = c @ w_uv[h]
        qv = np.concatenate([qh[h, :128], _rope_complex(qh[h, 128:][None], [pos[L]])[0]])
        ref = F.scaled_dot_product_attention(t(qv)[None, None], t(k)[None], t(v)[None], scale=0.7)[0, 0]
        np.testing.assert_allclose(got[h], ref.numpy(), atol=1e-12)
