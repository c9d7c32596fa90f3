"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/lca.h declares, computes the grouping plan, and rejects
bad arguments before touching the device."""
import ctypes
import json
import os
import re

import pytest

import mla_latent_kv_lca_amd as lca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "lca.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = lca.load()
    declared = _header_functions()
    assert set(declared) == set(lca.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version():
    assert lca.lca_version() == 1004


def test_plan_matches_golden():
    with open(os.path.join(ROOT, "tests", "golden", "plan_counts.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        p = lca.lca_plan(case["L"], case["w"], case["g"])
        assert p["m"] == case["m"]
        assert p["raw_begin"] == case["m"] * case["g"]
        assert p["raw_end"] == case["L"]
        assert p["n_entries"] == case["m"] + case["L"] - case["m"] * case["g"]


def test_plan_rejects_bad_args():
    with pytest.raises(lca.LcaError) as e:
        lca.lca_plan(10, 4, 0)
    assert e.value.status == lca.LCA_ERR_INVALID_ARG
    assert "g >= 1" in lca.lca_last_error()
    assert lca.lca_plan(10, 4, 2)["m"] == 3 and lca.lca_last_error() == ""


def test_workspace_sizes():
    assert lca.lca_condense_workspace_size(32, 1984, 0) == 32 * 9 * 576 * 4  # summary query + 8 partial sums
    assert lca.lca_condense_workspace_size(1, 256, 16) == 256 * 576 * 4
    assert lca.lca_condense_workspace_size(0, 1, 0) == 0
    # one split needs no workspace; more splits need partials of 16 x 514 floats
    small = lca.mla_latent_attn_decode_workspace_size(512, 16, 32)
    assert small == 0
    big = lca.mla_latent_attn_decode_workspace_size(1, 16, 66496)
    assert big > 0 and big % (16 * 514 * 4) == 0
    assert lca.mla_latent_attn_decode_workspace_size(1, 24, 100) == 0  # unsupported H


def _lat(ptr=16, dtype=0, stride=576):
    return lca.LatentT(ptr, ptr, 0, stride, 0, stride, dtype)


def _condense(lib, cache, reps, **kw):
    a = dict(B=1, g=16, gb=0, n=1, q=64, qdt=0, qss=0, qts=576 * 16, T=16, H=16, r0=0, rs=0,
             sm=1.0, anchor=64, aseq=0, alpha=None, alseq=0, ws=64, wsb=4096)
    a.update(kw)
    return lib.lca_condense(None if cache is None else ctypes.byref(cache), a["B"], a["g"], a["gb"],
                            a["n"], a["q"], a["qdt"], a["qss"], a["qts"], a["T"], a["H"], a["r0"],
                            a["rs"], a["sm"], None if reps is None else ctypes.byref(reps),
                            a["anchor"], a["aseq"], a["alpha"], a["alseq"], a["ws"], a["wsb"], None)


def test_condense_argument_errors():
    lib = lca.load()
    ok_lat = _lat()
    assert _condense(lib, None, ok_lat) == lca.LCA_ERR_INVALID_ARG
    assert "cache is null" in lca.lca_last_error()
    assert _condense(lib, ok_lat, ok_lat, g=12) == lca.LCA_ERR_UNSUPPORTED
    assert _condense(lib, ok_lat, ok_lat, g=64) == lca.LCA_ERR_UNSUPPORTED
    assert _condense(lib, _lat(ptr=18), ok_lat) == lca.LCA_ERR_INVALID_ARG  # misaligned
    assert _condense(lib, _lat(stride=577), ok_lat) == lca.LCA_ERR_INVALID_ARG
    assert _condense(lib, _lat(dtype=7), ok_lat) == lca.LCA_ERR_INVALID_ARG
    assert _condense(lib, ok_lat, ok_lat, sm=-1.0) == lca.LCA_ERR_INVALID_ARG
    assert _condense(lib, ok_lat, ok_lat, sm=float("nan")) == lca.LCA_ERR_INVALID_ARG
    assert _condense(lib, ok_lat, ok_lat, T=15) == lca.LCA_ERR_INVALID_ARG  # q rows out of range
    assert "T = 15" in lca.lca_last_error()
    assert _condense(lib, ok_lat, ok_lat, n=3, rs=16, T=40) == lca.LCA_ERR_INVALID_ARG
    assert _condense(lib, ok_lat, ok_lat, anchor=None) == lca.LCA_ERR_INVALID_ARG
    assert _condense(lib, ok_lat, ok_lat, ws=None) == lca.LCA_ERR_WORKSPACE
    assert _condense(lib, ok_lat, ok_lat, wsb=100) == lca.LCA_ERR_WORKSPACE
    assert _condense(lib, ok_lat, ok_lat, n=0) == lca.LCA_OK  # empty range: no launch


def test_condense_mode_argument_errors():
    """lca_condense_mode: the mode is checked first, then the same checks as lca_condense."""
    lib = lca.load()
    ok_lat = _lat()
    a = dict(B=1, g=16, gb=0, n=1, q=64, qdt=0, qss=0, qts=576 * 16, T=16, H=16, r0=0, rs=0)

    def call(mode, **kw):
        b = dict(a, **kw)
        return lib.lca_condense_mode(ctypes.byref(ok_lat), b["B"], b["g"], b["gb"], b["n"], b["q"], b["qdt"],
                                     b["qss"], b["qts"], b["T"], b["H"], b["r0"], b["rs"], 1.0,
                                     ctypes.byref(ok_lat), 64, 0, None, 0, 64, 4096, mode, None)
    for bad in (-1, 3, 99):
        assert call(bad) == lca.LCA_ERR_INVALID_ARG
        assert "mode" in lca.lca_last_error()
    assert call(lca.LCA_MODE_POOL_ROPE, g=12) == lca.LCA_ERR_UNSUPPORTED
    assert call(lca.LCA_MODE_ANCHOR, T=15) == lca.LCA_ERR_INVALID_ARG
    assert call(lca.LCA_MODE_ANCHOR, n=0) == lca.LCA_OK  # empty range: no launch


def test_decode_paged_argument_errors():
    lib = lca.load()
    reps = lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 0)

    def call(pages=64, row_stride=576, page_rows=64, table=128, table_stride=4, seq=256, max_entries=100,
             H=16, reps_=reps):
        cache = lca.PagedT(pages, row_stride, page_rows, table, table_stride)
        return lib.mla_latent_attn_decode_paged(64, 0, 16 * 576, 1, H, ctypes.byref(reps_), seq,
                                                ctypes.byref(cache), seq, seq, max_entries, 1.0, 64, None,
                                                64, 1 << 20, None)
    assert call(page_rows=8) == lca.LCA_ERR_UNSUPPORTED
    assert call(page_rows=40) == lca.LCA_ERR_UNSUPPORTED
    assert call(pages=None) == lca.LCA_ERR_INVALID_ARG
    assert call(pages=72) == lca.LCA_ERR_INVALID_ARG  # misaligned
    assert call(row_stride=570) == lca.LCA_ERR_INVALID_ARG
    assert call(table=None) == lca.LCA_ERR_INVALID_ARG
    assert call(table_stride=0) == lca.LCA_ERR_INVALID_ARG
    assert call(seq=None) == lca.LCA_ERR_INVALID_ARG
    assert call(max_entries=0) == lca.LCA_ERR_INVALID_ARG
    assert call(H=24) == lca.LCA_ERR_UNSUPPORTED
    assert call(row_stride=584) == lca.LCA_ERR_UNSUPPORTED  # reps stride differs from the pages'
    assert call(reps_=lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 1)) == lca.LCA_ERR_UNSUPPORTED  # f32 reps


def test_condense_paged_argument_errors():
    lib = lca.load()
    reps = lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 0)

    def call(page_rows=64, g=16, table=128, seq=256, max_groups=4, T=16, reps_=reps, step=0):
        cache = lca.PagedT(64, 576, page_rows, table, 4)
        return lib.lca_condense_paged(ctypes.byref(cache), 1, g, seq, seq, max_groups, 64, 0, 0, 16 * 576, T, 16,
                                      0, step, 1.0, ctypes.byref(reps_), 64, 0, None, 0, 64, 1 << 20, None)
    assert call(page_rows=40) == lca.LCA_ERR_UNSUPPORTED  # not a multiple of g
    assert call(g=12) == lca.LCA_ERR_UNSUPPORTED
    assert call(table=None) == lca.LCA_ERR_INVALID_ARG
    assert call(seq=None) == lca.LCA_ERR_INVALID_ARG
    assert call(T=15) == lca.LCA_ERR_INVALID_ARG
    assert call(max_groups=-1) == lca.LCA_ERR_INVALID_ARG
    assert call(reps_=lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 1)) == lca.LCA_ERR_UNSUPPORTED
    assert call(max_groups=0) == lca.LCA_OK  # nothing to condense: no launch
    # per-group summary queries: rows q_row0 + n * step .. + g must exist for n < max_groups
    assert call(step=16, T=63) == lca.LCA_ERR_INVALID_ARG
    assert "T = 63" in lca.lca_last_error()
    assert call(step=-16, T=64) == lca.LCA_ERR_INVALID_ARG


def test_paged_prefill_and_paged_decode_up_argument_errors():
    lib = lca.load()
    reps = lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 0)

    def prefill(page_rows=64, table=128, seq=0, H=16, rb=0, cs=10, m=0, reps_=reps, row_stride=576):
        cache = lca.PagedT(64, row_stride, page_rows, table, 4)
        return lib.mla_latent_attn_prefill_chunk_paged(64, 0, 16 * 576, cs, 4, H, ctypes.byref(reps_), m,
                                                       ctypes.byref(cache), seq, rb, 1.0, 64, 0, None, None)
    assert prefill(page_rows=40) == lca.LCA_ERR_UNSUPPORTED
    assert prefill(table=None) == lca.LCA_ERR_INVALID_ARG
    assert prefill(seq=-1) == lca.LCA_ERR_INVALID_ARG
    assert prefill(H=24) == lca.LCA_ERR_UNSUPPORTED
    assert prefill(rb=11) == lca.LCA_ERR_INVALID_ARG               # raw rows must start at or before the chunk
    assert prefill(m=2, reps_=lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 1)) == lca.LCA_ERR_UNSUPPORTED
    assert prefill(m=2, row_stride=640) == lca.LCA_ERR_UNSUPPORTED  # reps and pages share one row stride

    def dec(w=64, out=64, H=16, ws=None, wsb=0, max_entries=8):
        cache = lca.PagedT(64, 576, 64, 128, 4)
        return lib.mla_latent_attn_decode_paged_up(64, 0, 16 * 576, 1, H, ctypes.byref(reps), 256,
                                                   ctypes.byref(cache), 256, 256, max_entries, 1.0, 64, None,
                                                   w, 0, out, 0, ws, wsb, None)
    assert dec(w=None) == lca.LCA_ERR_INVALID_ARG
    assert dec(out=72) == lca.LCA_ERR_INVALID_ARG
    assert dec(H=24) == lca.LCA_ERR_UNSUPPORTED
    assert dec(max_entries=60000) == lca.LCA_ERR_WORKSPACE


def test_condense_step_argument_errors():
    lib = lca.load()
    reps = lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 0)

    def step(page_rows=64, table=128, B=2, w=1024, g=16, q=64, qdt=0, H=16, ring=64, ring_seq=16 * 16 * 576,
             reps_=reps, anchor=64, sm=1.0, sm_arr=64, rb_arr=64, re_arr=64):
        cache = lca.PagedT(64, 576, page_rows, table, 4)
        return lib.lca_condense_step(ctypes.byref(cache), B, w, g, q, qdt, 16 * 576, H, ring, ring_seq, sm,
                                     ctypes.byref(reps_), anchor, 0, sm_arr, rb_arr, re_arr, None, None, None)
    assert step(page_rows=40) == lca.LCA_ERR_UNSUPPORTED          # not a multiple of g
    assert step(g=12) == lca.LCA_ERR_UNSUPPORTED
    assert step(g=64) == lca.LCA_ERR_UNSUPPORTED
    assert step(table=None) == lca.LCA_ERR_INVALID_ARG
    assert step(B=0) == lca.LCA_ERR_INVALID_ARG
    assert step(w=-1) == lca.LCA_ERR_INVALID_ARG
    assert step(q=None) == lca.LCA_ERR_INVALID_ARG
    assert step(qdt=7) == lca.LCA_ERR_INVALID_ARG
    assert step(ring=None) == lca.LCA_ERR_INVALID_ARG
    assert step(ring_seq=16 * 16 * 576 - 8) == lca.LCA_ERR_INVALID_ARG  # ring shorter than g rows of H heads
    assert step(reps_=lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 1)) == lca.LCA_ERR_UNSUPPORTED
    assert step(anchor=None) == lca.LCA_ERR_INVALID_ARG
    assert step(sm_arr=None) == lca.LCA_ERR_INVALID_ARG
    assert step(re_arr=None) == lca.LCA_ERR_INVALID_ARG
    assert step(sm=float("nan")) == lca.LCA_ERR_INVALID_ARG
    assert "g = 12" in (step(g=12), lca.lca_last_error())[1]


def test_decode_paged_up_step_argument_errors():
    lib = lca.load()
    reps = lca.LatentT(64, 64 + 1024, 0, 576, 0, 576, 0)

    def call(step=True, g=16, ring=64, ring_seq=16 * 16 * 576, anchor=64, w=1024, H=16, wuv=64):
        cache = lca.PagedT(64, 576, 64, 128, 4)
        st = lca.StepT(w, g, ring, ring_seq, anchor, 0, None, None)
        return lib.mla_latent_attn_decode_paged_up_step(
            64, 0, 16 * 576, 1, H, ctypes.byref(reps), 256, ctypes.byref(cache), 256, 256, 8, 1.0, 64, None,
            wuv, 0, 64, 0, ctypes.byref(st) if step else None, None, 0, None)
    assert call(step=False) == lca.LCA_ERR_INVALID_ARG
    assert call(g=12) == lca.LCA_ERR_UNSUPPORTED
    assert call(ring=None) == lca.LCA_ERR_INVALID_ARG
    assert call(ring_seq=100) == lca.LCA_ERR_INVALID_ARG
    assert call(anchor=None) == lca.LCA_ERR_INVALID_ARG
    assert call(w=-1) == lca.LCA_ERR_INVALID_ARG
    assert call(H=24) == lca.LCA_ERR_UNSUPPORTED
    assert call(wuv=None) == lca.LCA_ERR_INVALID_ARG


def _decode(lib, reps, raw, **kw):
    a = dict(q=64, qdt=0, qss=16 * 576, B=1, H=16, m=0, rb=0, re=8, sm=1.0, o=64, lse=None,
             ws=None, wsb=0)
    a.update(kw)
    return lib.mla_latent_attn_decode(a["q"], a["qdt"], a["qss"], a["B"], a["H"],
                                      None if reps is None else ctypes.byref(reps), a["m"],
                                      None if raw is None else ctypes.byref(raw), a["rb"], a["re"],
                                      a["sm"], a["o"], a["lse"], a["ws"], a["wsb"], None)


def test_decode_argument_errors():
    lib = lca.load()
    lat = _lat()
    assert _decode(lib, None, lat, H=24) == lca.LCA_ERR_UNSUPPORTED
    assert _decode(lib, None, lat, re=0) == lca.LCA_ERR_INVALID_ARG  # nothing to attend
    assert _decode(lib, None, None) == lca.LCA_ERR_INVALID_ARG       # raw rows but no raw
    assert _decode(lib, None, lat, m=4) == lca.LCA_ERR_INVALID_ARG   # reps missing
    assert _decode(lib, _lat(dtype=1), lat, m=4) == lca.LCA_ERR_UNSUPPORTED  # mixed dtypes
    assert _decode(lib, None, lat, q=None) == lca.LCA_ERR_INVALID_ARG
    assert _decode(lib, None, lat, o=None) == lca.LCA_ERR_INVALID_ARG
    assert _decode(lib, None, lat, rb=5, re=4) == lca.LCA_ERR_INVALID_ARG
    # a long single sequence needs split-K workspace
    assert _decode(lib, None, lat, re=60000) == lca.LCA_ERR_WORKSPACE
    assert "workspace needs" in lca.lca_last_error()


def _decode_up(lib, raw, **kw):
    a = dict(q=64, qdt=0, qss=16 * 576, B=1, H=16, m=0, rb=0, re=8, sm=1.0, o=64, lse=None,
             w=64, wdt=0, out=64, odt=0, ws=None, wsb=0)
    a.update(kw)
    return lib.mla_latent_attn_decode_up(a["q"], a["qdt"], a["qss"], a["B"], a["H"], None, a["m"],
                                         None if raw is None else ctypes.byref(raw), a["rb"], a["re"],
                                         a["sm"], a["o"], a["lse"], a["w"], a["wdt"], a["out"],
                                         a["odt"], a["ws"], a["wsb"], None)


def test_decode_up_argument_errors():
    lib = lca.load()
    lat = _lat()
    assert _decode_up(lib, lat, w=None) == lca.LCA_ERR_INVALID_ARG
    assert _decode_up(lib, lat, out=None) == lca.LCA_ERR_INVALID_ARG
    assert _decode_up(lib, lat, w=72) == lca.LCA_ERR_INVALID_ARG   # misaligned
    assert _decode_up(lib, lat, odt=7) == lca.LCA_ERR_INVALID_ARG
    assert _decode_up(lib, lat, H=24) == lca.LCA_ERR_UNSUPPORTED
    assert _decode_up(lib, lat, re=60000) == lca.LCA_ERR_WORKSPACE


def test_head_group_sizes():
    """Head counts that divide 16 (grouped-query attention groups) use one
    16-row head block, so they need the workspace of 16 heads; other counts
    below 16, or not a multiple of 16, are not supported."""
    for h in (1, 2, 4, 8):
        assert lca.mla_latent_attn_decode_workspace_size(3, h, 66496) == \
            lca.mla_latent_attn_decode_workspace_size(3, 16, 66496) > 0
    for h in (3, 12, 24, 40):
        assert lca.mla_latent_attn_decode_workspace_size(3, h, 66496) == 0
    assert lca.mla_latent_attn_decode_workspace_size(3, 48, 66496) > 0


def test_decode_up_noalloc_argument_errors():
    """The entry point that allocates nothing rejects bad arguments like
    mla_latent_attn_decode_up (it has no workspace argument to get wrong)."""
    lib = lca.load()
    lat = _lat()

    def call(**kw):
        a = dict(q=64, qdt=0, qss=16 * 576, B=1, H=16, m=0, rb=0, re=8, sm=1.0, o=64, lse=None,
                 w=64, wdt=0, out=64, odt=0)
        a.update(kw)
        return lib.mla_latent_attn_decode_up_noalloc(a["q"], a["qdt"], a["qss"], a["B"], a["H"], None, a["m"],
                                                     ctypes.byref(lat), a["rb"], a["re"], a["sm"], a["o"],
                                                     a["lse"], a["w"], a["wdt"], a["out"], a["odt"], None)
    assert call(q=None) == lca.LCA_ERR_INVALID_ARG
    assert call(w=None) == lca.LCA_ERR_INVALID_ARG
    assert call(out=72) == lca.LCA_ERR_INVALID_ARG
    assert call(H=24) == lca.LCA_ERR_UNSUPPORTED
    assert call(rb=9) == lca.LCA_ERR_INVALID_ARG
    assert call(sm=-1.0) == lca.LCA_ERR_INVALID_ARG
    assert "sm_scale" in lca.lca_last_error()


def test_prefill_and_up_proj_argument_errors():
    lib = lca.load()
    lat = _lat()
    pf = lib.mla_latent_attn_prefill_chunk
    assert pf(64, 0, 9216, 10, 4, 16, None, 0, ctypes.byref(lat), 11, 1.0, 64, 0, None, None) == lca.LCA_ERR_INVALID_ARG
    assert pf(64, 0, 9216, 10, 0, 16, None, 0, ctypes.byref(lat), 0, 1.0, 64, 0, None, None) == lca.LCA_ERR_INVALID_ARG
    assert pf(64, 0, 9216, 10, 4, 24, None, 0, ctypes.byref(lat), 0, 1.0, 64, 0, None, None) == lca.LCA_ERR_UNSUPPORTED
    assert pf(64, 0, 9216, 10, 4, 16, None, 0, ctypes.byref(lat), 0, 1.0, 64, 5, None, None) == lca.LCA_ERR_INVALID_ARG
    # the scheduled forms: a null or misaligned counter, then the shared checks
    ps = lib.mla_latent_attn_prefill_chunk_sched
    assert ps(64, 0, 9216, 10, 4, 16, None, 0, ctypes.byref(lat), 0, 1.0, 64, 0, None, None, None) == lca.LCA_ERR_INVALID_ARG
    assert ps(64, 0, 9216, 10, 4, 16, None, 0, ctypes.byref(lat), 0, 1.0, 64, 0, None, 68, None) == lca.LCA_ERR_INVALID_ARG
    assert ps(64, 0, 9216, 10, 4, 24, None, 0, ctypes.byref(lat), 0, 1.0, 64, 0, None, 64, None) == lca.LCA_ERR_UNSUPPORTED
    pps = lib.mla_latent_attn_prefill_chunk_paged_sched
    assert pps(64, 0, 9216, 10, 4, 16, None, 0, None, 0, 0, 1.0, 64, 0, None, None, None) == lca.LCA_ERR_INVALID_ARG
    assert pps(64, 0, 9216, 10, 4, 16, None, 0, None, 0, 0, 1.0, 64, 0, None, 64, None) == lca.LCA_ERR_INVALID_ARG
    up = lib.mla_up_proj
    assert up(64, 0, 0, 16, 64, 0, 64, 0, None) == lca.LCA_OK  # T == 0
    assert up(64, 0, -1, 16, 64, 0, 64, 0, None) == lca.LCA_ERR_INVALID_ARG
    assert up(None, 0, 4, 16, 64, 0, 64, 0, None) == lca.LCA_ERR_INVALID_ARG
    assert up(64, 3, 4, 16, 64, 0, 64, 0, None) == lca.LCA_ERR_INVALID_ARG


def _project(lib, **kw):
    a = dict(x=64, xs=2048, T=4, d=2048, pos=64, base=10000.0, w=64, wuk=64, H=16, rows=64, rs=576,
             dst=64, q=64, qdt=0, qs=16 * 576, ws=64, wsb=4 * 16 * 128 * 2)
    a.update(kw)
    return lib.lca_project(a["x"], a["xs"], a["T"], a["d"], a["pos"], a["base"], a["w"], a["wuk"], a["H"],
                           a["rows"], a["rs"], a["dst"], a["q"], a["qdt"], a["qs"], a["ws"], a["wsb"], None)


def test_project_argument_errors():
    lib = lca.load()
    assert lca.lca_project_workspace_size(4, 16) == 4 * 16 * 128 * 2
    assert lca.lca_project_workspace_size(-1, 16) == 0
    assert _project(lib, T=0) == lca.LCA_OK
    assert _project(lib, T=-1) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, d=100) == lca.LCA_ERR_UNSUPPORTED
    assert _project(lib, H=0) == lca.LCA_ERR_UNSUPPORTED
    assert _project(lib, base=1.0) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, base=float("nan")) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, qdt=5) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, x=None) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, w=72) == lca.LCA_ERR_INVALID_ARG      # misaligned
    assert _project(lib, xs=1000) == lca.LCA_ERR_INVALID_ARG   # shorter than d_model
    assert _project(lib, pos=None) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, dst=None) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, rs=500) == lca.LCA_ERR_INVALID_ARG
    assert _project(lib, qs=576) == lca.LCA_ERR_INVALID_ARG    # heads overlap
    assert _project(lib, wsb=16) == lca.LCA_ERR_WORKSPACE
    assert _project(lib, ws=None) == lca.LCA_ERR_WORKSPACE


def test_binding_rejects_bad_lse():
    """The binding checks lse (fp32, contiguous, rows x H elements) before any
    call reaches the library, since the kernels index it without bounds."""
    import torch
    B, H = 2, 16
    q = torch.zeros((B, H, 576), dtype=torch.bfloat16)
    o = torch.zeros((B, H, 512), dtype=torch.float32)
    raw = lca.packed_latent(torch.zeros((B, 8, 576), dtype=torch.bfloat16))
    for bad in (torch.zeros((B, H), dtype=torch.bfloat16), torch.zeros((B, H - 1)),
                torch.zeros((H, B)).t()):
        with pytest.raises(ValueError, match="lse"):
            lca.mla_latent_attn_decode(q, None, 0, raw, 0, 8, 1.0, o, bad)
        with pytest.raises(ValueError, match="lse"):
            lca.mla_latent_attn_decode_up(q, None, 0, raw, 0, 8, 1.0, o, torch.zeros((H, 512, 128)),
                                          torch.zeros((B, H, 128)), bad)
    C = 3
    with pytest.raises(ValueError, match="lse"):
        lca.mla_latent_attn_prefill_chunk(torch.zeros((C, H, 576), dtype=torch.bfloat16), 0, None, 0, raw, 0, 1.0,
                                          torch.zeros((C, H, 512)), torch.zeros((C * H + 1,)))
    pool = torch.zeros((2, 16, 576), dtype=torch.bfloat16)
    table = torch.zeros((B, 1), dtype=torch.int32)
    i32 = torch.zeros((B,), dtype=torch.int32)
    with pytest.raises(ValueError, match="lse"):
        lca.mla_latent_attn_decode_paged(q, lca.packed_latent(torch.zeros((B, 1, 576), dtype=torch.bfloat16)), i32,
                                         lca.paged_latent(pool, table), i32, i32, 8, 1.0, o,
                                         torch.zeros((B, H), dtype=torch.float64))
