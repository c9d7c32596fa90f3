"""Plain fp64 CPU oracle for MLA attention over a latent-condensed KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module:
only the tests, the smoke check of the entry script and the CPU-baseline leg
of the benchmark may call it. It shares no code with the HIP library.

Every function follows the method as the pages state it, in NumPy float64,
with no blocking, fusion or reordering beyond the plain definition:

  [LCT]  "Latent-Condensed Transformer for Efficient Long Context Modeling"
         (papernotes.org notes on the ACL 2026 paper, arXiv 2604.12452)
         - 方法详解 / 整体框架: history older than the local window of w tokens
           is cut into m = floor((L - w) / g) groups of g tokens; each group
           becomes one representative; representatives are concatenated with
           the window and standard attention runs over the result (flowchart
           nodes B, W, E, F).
         - 关键设计 1: the summary query is the mean of the most recent g
           queries; every token of a group gets an importance score; the
           scores are softmax-normalised into weights alpha_i^(j); the latent
           representative is the alpha-weighted sum of the group's c_KV rows
           (the displayed pooling equation). Proposition 1: this weighted pool
           minimises the expected reconstruction error.
         - 关键设计 2: the position key of a group is the k_R of its most
           important token I_j (the displayed anchor equation).
         - 关键设计 3: the last w tokens are never compressed.
         - 消融实验 (ablation table): two variants beside full LCA (semantic
           pooling + position anchor): "pure pooling including position" (the
           position keys pooled with the same weights as the latents) and "pure
           sparse" (the group keeps only its most important token).
  [MLA]  "新一代开源大模型架构演进与注意力机制深度对比解析" (cloud.baidu.com),
         三、核心差异分析 1: MLA caches a low-rank latent per token and projects
         it back up at compute time.

Readings where the pages are silent (each is restated where it is used):
  R1 the importance score of token i is the absorbed attention logit of the
     summary query against the full cached row, s_i = qbar . [c_i ; k_i^R];
  R2 "mean of the most recent g queries" averages over the g query tokens and
     over the H heads (one weight per token, so one representative per group);
  R3 the anchor is the lowest index among the maxima of s (ties to the first);
  R4 one softmax scale sm_scale is used for the pooling weights and for the
     attention logits; representatives get no extra logit bias;
  R5 groups are aligned at token 0; the (L - w) mod g leftover tokens stay raw;
  R6 chunked prefill freezes groups before each chunk's window: a chunk that
     starts at s uses m_s = floor((s - w) / g) groups (0 if s < w), each group
     j condensed with the mean of the g queries that follow it (tokens
     (j+1)g .. (j+2)g-1); query t sees all m_s representatives and raw rows
     [m_s g, t];
  R7 in decode, representatives are computed once when a group leaves the
     window and are frozen afterwards; the g most recent decode queries give
     the summary query of the group being condensed;
  R8 GQA (关键发现 says the design extends to GQA, with no mapping): n_kv
     independent latent caches; the H query heads form n_kv groups of
     Hg = H / n_kv consecutive heads, group k attends cache k, and cache k is
     condensed with the summary query of its own Hg heads;
  R9 the step before the path ([MLA] 三.1: per-token latent down-projection,
     and RoPE needs its own handling under MLA; [LCT] 研究背景与动机 / 核心矛盾:
     the position key K^R carries RoPE beside the latent): for hidden state x_t
     at position p_t, c_t = x_t W_DKV, k^R_t = RoPE(x_t W_KR, p_t) and per head
     [q^nope_h ; q^rope_h] = x_t W_Q[h], q^rope rotated by RoPE(p_t); the
     absorbed query is [W_UK[h] q^nope_h ; RoPE(q^rope_h, p_t)]. RoPE is the
     rotate-half convention on 64 dims (pairs (i, i + 32), angle p theta_i,
     theta_i = base^(-2i/64)). The pages give no widths beyond d_c, d_R and H:
     per-head no-RoPE query width 128 as W_UK's shape implies.
"""
from __future__ import annotations

import numpy as np

D_C = 512
D_R = 64
D_ROW = D_C + D_R

# condensation modes: full LCA and the two ablation variants of 消融实验
MODE_LCA = 0          # c_rep = sum alpha_i c_i, k_rep = k_R of the anchor
MODE_POOL_ROPE = 1    # c_rep = sum alpha_i c_i, k_rep = sum alpha_i k_R,i
MODE_ANCHOR = 2       # c_rep = c of the anchor, k_rep = k_R of the anchor


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- grouping ---
def plan(L: int, w: int, g: int) -> dict:
    """Group count and raw range [LCT 整体框架: m = floor((L - w)/g); R5].

    Groups are [j g, (j+1) g) for j < m; the raw (uncompressed) rows are
    [m g, L): the last w tokens plus the (L - w) mod g leftover.
    """
    if L < 0 or w < 0 or g < 1:
        raise ValueError("L, w >= 0 and g >= 1 required")
    m = (L - w) // g if L > w else 0
    raw_begin = m * g
    return {"m": m, "raw_begin": raw_begin, "raw_end": L, "n_entries": m + (L - raw_begin)}


def kept_fraction(L: int, w: int, g: int) -> float:
    """Entries attended after condensation over entries before (1 - compression)."""
    return plan(L, w, g)["n_entries"] / L


# ------------------------------------------------------------ condensation ---
def summary_query(q_rows) -> np.ndarray:
    """qbar from g query tokens [g, H, 576]: mean over tokens and heads [LCT 关键设计 1; R2]."""
    q = _f64(q_rows)
    return q.reshape(-1, q.shape[-1]).mean(axis=0)


def importance_scores(qbar, c_rows, k_rows) -> np.ndarray:
    """s_i = qbar . [c_i ; k_i^R] for each token of a group [LCT 关键设计 1; R1]."""
    rows = np.concatenate([_f64(c_rows), _f64(k_rows)], axis=-1)
    return rows @ _f64(qbar)


def softmax(x) -> np.ndarray:
    x = _f64(x)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def condense_group(c_rows, k_rows, qbar, sm_scale: float, mode: int = MODE_LCA):
    """One group [LCT 关键设计 1 pooling equation, 关键设计 2 anchor equation;
    消融实验 for the other modes].

    Returns (c_rep [512], k_rep [64], alpha [g], anchor (index within the
    group), scores [g]). alpha = softmax(sm_scale * s) (R4); anchor = first
    argmax of s (R3). MODE_LCA: c_rep = sum_i alpha_i c_i, k_rep = k_R of the
    anchor. MODE_POOL_ROPE: k_rep = sum_i alpha_i k_R,i as well. MODE_ANCHOR:
    c_rep and k_rep are the anchor's own row.
    """
    s = importance_scores(qbar, c_rows, k_rows)
    alpha = softmax(sm_scale * s)
    anchor = int(np.flatnonzero(s == s.max())[0])
    c_rep = _f64(c_rows)[anchor] if mode == MODE_ANCHOR else alpha @ _f64(c_rows)
    k_rep = alpha @ _f64(k_rows) if mode == MODE_POOL_ROPE else _f64(k_rows)[anchor]
    return c_rep, k_rep, alpha, anchor, s


def condense(c, kr, q, g: int, group_begin: int, n_groups: int, q_row0: int,
             q_row_step: int, sm_scale: float, mode: int = MODE_LCA):
    """Condense groups [group_begin, group_begin + n_groups) of every sequence.

    c [B, L, 512], kr [B, L, 64], q [B, T, H, 576]. Group j (token rows
    [j g, (j+1) g)) takes its summary query from query tokens
    [q_row0 + (j - group_begin) q_row_step, ... + g) (R2, R6, R7).
    Returns rep_c [B, n, 512], rep_k [B, n, 64], anchor [B, n] (absolute token
    index I_j), alpha [B, n, g], scores [B, n, g]. `mode` selects full LCA or
    one of the ablation variants (condense_group).
    """
    c, kr = np.asarray(c), np.asarray(kr)
    B = c.shape[0]
    rep_c = np.zeros((B, n_groups, D_C))
    rep_k = np.zeros((B, n_groups, D_R))
    anchor = np.zeros((B, n_groups), dtype=np.int64)
    alpha = np.zeros((B, n_groups, g))
    scores = np.zeros((B, n_groups, g))
    for b in range(B):
        for n in range(n_groups):
            j = group_begin + n
            r0 = q_row0 + n * q_row_step
            qbar = summary_query(q[b, r0:r0 + g])
            cr, kk, a, i, s = condense_group(c[b, j * g:(j + 1) * g], kr[b, j * g:(j + 1) * g],
                                             qbar, sm_scale, mode)
            rep_c[b, n], rep_k[b, n], alpha[b, n], scores[b, n] = cr, kk, a, s
            anchor[b, n] = j * g + i
    return rep_c, rep_k, anchor, alpha, scores


def top2_margin(scores) -> np.ndarray:
    """Gap between the largest and second-largest score of each group."""
    s = np.sort(_f64(scores), axis=-1)
    return s[..., -1] - s[..., -2]


# --------------------------------------------------------------- attention ---
def attend(q, ent_c, ent_k, sm_scale: float):
    """Standard softmax attention of H absorbed queries over latent entries.

    q [H, 576]; entries ent_c [n, 512], ent_k [n, 64]. The absorbed query's
    logit against entry e is q . [c_e ; k_e]; the value is c_e itself (the
    up-projection to the head's value space comes later, [MLA] 三.1). Returns
    o_latent [H, 512] and lse [H] (natural-log logsumexp of the logits).
    """
    keys = np.concatenate([_f64(ent_c), _f64(ent_k)], axis=-1)
    z = sm_scale * (_f64(q) @ keys.T)
    zmax = z.max(axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    ssum = e.sum(axis=-1, keepdims=True)
    o = (e / ssum) @ _f64(ent_c)
    return o, zmax[:, 0] + np.log(ssum[:, 0])


def decode(q, rep_c, rep_k, m: int, raw_c, raw_k, raw_begin: int, raw_end: int,
           sm_scale: float):
    """Decode over [representatives [0, m) ++ raw rows [raw_begin, raw_end)].

    [LCT 整体框架, flowchart E -> F]. q [B, H, 576]; rep_* [B, >=m, .];
    raw_* [B, >=raw_end, .]. Plain MLA is m = 0, raw = [0, L).
    Returns o_latent [B, H, 512], lse [B, H].
    """
    B, H = q.shape[0], q.shape[1]
    o = np.zeros((B, H, D_C))
    lse = np.zeros((B, H))
    for b in range(B):
        ec, ek = _f64(raw_c[b, raw_begin:raw_end]), _f64(raw_k[b, raw_begin:raw_end])
        if m > 0:
            ec = np.concatenate([_f64(rep_c[b, :m]), ec])
            ek = np.concatenate([_f64(rep_k[b, :m]), ek])
        o[b], lse[b] = attend(q[b], ec, ek, sm_scale)
    return o, lse


def prefill_chunk(q, chunk_start: int, rep_c, rep_k, m: int, raw_c, raw_k, raw_begin: int,
                  sm_scale: float, rows=None):
    """Chunked prefill for one sequence (R6).

    q [C, H, 576] are the queries at positions chunk_start .. chunk_start+C-1.
    Query at position t sees representatives [0, m) and raw rows
    [raw_begin, t] (causal, inclusive). rows optionally selects which chunk
    rows to evaluate. Returns o_latent [len(rows), H, 512], lse [len(rows), H].
    """
    C, H = q.shape[0], q.shape[1]
    rows = np.arange(C) if rows is None else np.asarray(rows)
    o = np.zeros((len(rows), H, D_C))
    lse = np.zeros((len(rows), H))
    rc = _f64(rep_c[:m]) if m > 0 else np.zeros((0, D_C))
    rk = _f64(rep_k[:m]) if m > 0 else np.zeros((0, D_R))
    for n, i in enumerate(rows):
        t = chunk_start + int(i)
        ec = np.concatenate([rc, _f64(raw_c[raw_begin:t + 1])])
        ek = np.concatenate([rk, _f64(raw_k[raw_begin:t + 1])])
        o[n], lse[n] = attend(q[i], ec, ek, sm_scale)
    return o, lse


def up_proj(o_latent, w_uv) -> np.ndarray:
    """Per-head value up-projection o[t, h] = o_latent[t, h] @ W_UV[h] ([MLA] 三.1)."""
    return np.einsum("thk,hkv->thv", _f64(o_latent), _f64(w_uv))


# ----------------------------------------------------- whole-path drivers ---
def prefill_plan(chunk_start: int, w: int, g: int) -> int:
    """m_s for a chunk starting at position chunk_start (R6)."""
    return (chunk_start - w) // g if chunk_start > w else 0


def prefill(q, c, kr, w: int, g: int, C: int, sm_scale: float):
    """Whole chunked prefill of one sequence (R6), all rows evaluated.

    q [L, H, 576], c [L, 512], kr [L, 64]. Chunk k covers [kC, (k+1)C). Before
    each chunk the newly eligible groups are condensed with the g queries that
    follow them. Returns o_latent [L, H, 512], lse [L, H] and the reps.
    """
    L, H = q.shape[0], q.shape[1]
    m_final = prefill_plan(((L - 1) // C) * C, w, g)
    rep_c = np.zeros((m_final, D_C))
    rep_k = np.zeros((m_final, D_R))
    o = np.zeros((L, H, D_C))
    lse = np.zeros((L, H))
    m = 0
    for s in range(0, L, C):
        ms = prefill_plan(s, w, g)
        if ms > m:
            rc, rk, _, _, _ = condense(c[None], kr[None], q[None], g, m, ms - m,
                                       (m + 1) * g, g, sm_scale)
            rep_c[m:ms], rep_k[m:ms] = rc[0], rk[0]
            m = ms
        e = min(L, s + C)
        o[s:e], lse[s:e] = prefill_chunk(q[s:e], s, rep_c, rep_k, m, c, kr, m * g, sm_scale)
    return o, lse, rep_c, rep_k


def decode_loop(c0, kr0, q_hist, steps_q, new_c, new_k, w: int, g: int, sm_scale: float):
    """Incremental decode of one sequence with frozen representatives (R7).

    c0/kr0 [L0, .] initial cache; q_hist [>=g, H, 576] the decode queries
    before step 0 (the most recent g give the first condensation's summary
    query); steps_q [S, H, 576] the query of each step; new_c/new_k [S, .] the
    row appended after each step. Before step 0 every eligible group is
    condensed with the last g history queries. After each step the row is
    appended, and if the raw history now holds a full group beyond the window
    that group is condensed with the last g queries (steps included).
    Returns o_latent [S, H, 512], lse [S, H], and the final reps and m.
    """
    cache_c = [_f64(x) for x in c0]
    cache_k = [_f64(x) for x in kr0]
    qs = [_f64(x) for x in q_hist]
    L = len(cache_c)
    m0 = plan(L, w, g)["m"]
    rc, rk, _, _, _ = condense(np.asarray(cache_c)[None], np.asarray(cache_k)[None],
                               np.asarray(qs)[None], g, 0, m0, len(qs) - g, 0, sm_scale)
    reps_c = list(rc[0])
    reps_k = list(rk[0])
    m = m0
    S = steps_q.shape[0]
    outs = np.zeros((S, steps_q.shape[1], D_C))
    lses = np.zeros((S, steps_q.shape[1]))
    for st in range(S):
        ec = np.asarray(reps_c[:m] + cache_c[m * g:]).reshape(-1, D_C)
        ek = np.asarray(reps_k[:m] + cache_k[m * g:]).reshape(-1, D_R)
        outs[st], lses[st] = attend(steps_q[st], ec, ek, sm_scale)
        qs.append(_f64(steps_q[st]))
        cache_c.append(_f64(new_c[st]))
        cache_k.append(_f64(new_k[st]))
        L += 1
        if L - w >= (m + 1) * g:
            cr, kk, _, _, _ = condense_group(np.asarray(cache_c[m * g:(m + 1) * g]),
                                             np.asarray(cache_k[m * g:(m + 1) * g]),
                                             summary_query(np.asarray(qs[-g:])), sm_scale)
            reps_c.append(cr)
            reps_k.append(kk)
            m += 1
    return outs, lses, np.asarray(reps_c), np.asarray(reps_k), m


# --------------------------------------------------- textbook MLA (pins) ---
def mha_expanded(q_nope, q_rope, c, kr, w_uk, w_uv, sm_scale: float):
    """Textbook per-head attention with explicitly up-projected keys and values.

    [MLA] 三.1: head h's key for token i is [W_UK[h]^T c_i ; k_i^R] and its
    value is W_UV[h]^T c_i; the head's query is [q_nope_h ; q_rope_h].
    q_nope [H, 128], q_rope [H, 64], c [n, 512], kr [n, 64], w_uk/w_uv
    [H, 512, 128]. Returns o [H, 128].
    """
    H = q_nope.shape[0]
    out = np.zeros((H, w_uv.shape[-1]))
    for h in range(H):
        k = np.concatenate([_f64(c) @ _f64(w_uk[h]), _f64(kr)], axis=-1)
        v = _f64(c) @ _f64(w_uv[h])
        qh = np.concatenate([_f64(q_nope[h]), _f64(q_rope[h])])
        p = softmax(sm_scale * (k @ qh))
        out[h] = p @ v
    return out


def absorb_query(q_nope, q_rope, w_uk) -> np.ndarray:
    """Absorbed query [W_UK[h] q_nope_h ; q_rope_h] ([H, 576])."""
    qa = np.einsum("hkd,hd->hk", _f64(w_uk), _f64(q_nope))
    return np.concatenate([qa, _f64(q_rope)], axis=-1)


def condense_gqa(c, kr, q, n_kv: int, g: int, group_begin: int, n_groups: int, q_row0: int,
                 q_row_step: int, sm_scale: float, mode: int = MODE_LCA):
    """GQA condensation (R8): c [B, n_kv, L, 512], kr [B, n_kv, L, 64],
    q [B, T, H, 576]; kv group k is condensed on its own cache with its own
    heads' queries. Returns condense()'s outputs with a kv axis after B."""
    Hg = q.shape[2] // n_kv
    per = [condense(c[:, k], kr[:, k], q[:, :, k * Hg:(k + 1) * Hg], g, group_begin, n_groups,
                    q_row0, q_row_step, sm_scale, mode) for k in range(n_kv)]
    return tuple(np.stack([o[i] for o in per], axis=1) for i in range(5))


def decode_gqa(q, rep_c, rep_k, m: int, raw_c, raw_k, raw_begin: int, raw_end: int, n_kv: int,
               sm_scale: float):
    """GQA decode (R8): q [B, H, 576]; rep_* [B, n_kv, m, *]; raw_* [B, n_kv, L, *];
    head h attends kv group h // (H / n_kv). Returns (o [B, H, 512], lse [B, H])."""
    Hg = q.shape[1] // n_kv
    os_, ls_ = [], []
    for k in range(n_kv):
        o, l = decode(q[:, k * Hg:(k + 1) * Hg], None if rep_c is None else rep_c[:, k],
                      None if rep_k is None else rep_k[:, k], m, raw_c[:, k], raw_k[:, k], raw_begin,
                      raw_end, sm_scale)
        os_.append(o)
        ls_.append(l)
    return np.concatenate(os_, axis=1), np.concatenate(ls_, axis=1)


def rope_rotate(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of the last axis (64 wide) at positions pos (R9):
    out[i] = x[i] cos(p t_i) - x[i+32] sin(p t_i), out[i+32] = x[i+32] cos(p t_i)
    + x[i] sin(p t_i), t_i = base^(-2i/64), i < 32. x [..., 64], pos broadcast
    over the leading axes."""
    x = _f64(x)
    half = x.shape[-1] // 2
    theta = base ** (-2.0 * np.arange(half) / x.shape[-1])
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def project(x, pos, w_cat, w_uk, H: int, base: float = 10000.0):
    """The step before the path (R9): x [T, d], pos [T], w_cat [d, 576 + 192 H]
    = [W_DKV (512) | W_KR (64) | W_Q (head h: 128 no-RoPE + 64 RoPE columns)],
    w_uk [H, 512, 128]. Returns the cache rows [T, 576] = [c ; RoPE(k^R)] and
    the absorbed queries [T, H, 576] = [W_UK[h] q^nope_h ; RoPE(q^rope_h)]."""
    y = _f64(x) @ _f64(w_cat)
    pos = np.asarray(pos)
    rows = np.concatenate([y[:, :D_C], rope_rotate(y[:, D_C:D_ROW], pos, base)], axis=-1)
    q = y[:, D_ROW:].reshape(len(y), H, 192)
    q_rope = rope_rotate(q[..., 128:], pos[:, None], base)
    return rows, np.stack([absorb_query(q[t, :, :128], q_rope[t], w_uk) for t in range(len(y))])
