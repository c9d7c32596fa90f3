"""The decode entry point that allocates nothing: mla_latent_attn_decode_up_noalloc
(through the C ABI) against mla_latent_attn_decode_up with a caller workspace,
on two calls in a row, the second with a smaller input (the fixed scratch keeps
the first call's partial results), and against the oracle."""
import numpy as np
import pytest
import torch

import lca_inputs as li
import mla_latent_kv_lca_amd as lca
from oracle import lca_oracle as O
from tests.gpu_util import assert_close, dev, host, packed

pytestmark = pytest.mark.gpu

H, G, W = 16, 16, 1024


def _case(cfg, B, L):
    c, kr = li.latent_cache(cfg, B, L)
    li.plant_needles(cfg, c, kr, 2, 14.0, 0, L)
    qh = li.queries(cfg, B, G, H, rho=0.5)
    qd = li.queries(cfg, B, 1, H, rho=0.5, stream=1)[:, 0]
    wuv = li.w_uv(cfg, H)
    p = O.plan(L, W, G)
    cache = packed(c, kr)
    reps = torch.empty((B, max(p["m"], 1), 576), dtype=torch.bfloat16, device="cuda")
    anchor = torch.empty((B, max(p["m"], 1)), dtype=torch.int32, device="cuda")
    if p["m"]:
        lca.lca_condense(lca.packed_latent(cache), B, G, 0, p["m"], dev(qh), 0, 0, 1.0,
                         lca.packed_latent(reps), anchor)
    return dict(c=c, kr=kr, qd=qd, wuv=wuv, p=p, cache=cache, reps=reps, B=B, L=L)


def _run(case, noalloc):
    B, p = case["B"], case["p"]
    o = torch.full((B, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((B, H, 128), float("nan"), dtype=torch.float32, device="cuda")
    args = (dev(case["qd"]), lca.packed_latent(case["reps"]) if p["m"] else None, p["m"],
            lca.packed_latent(case["cache"]), p["raw_begin"], case["L"], 1.0, o, dev(case["wuv"]), y, lse)
    if noalloc:
        lca.mla_latent_attn_decode_up_noalloc(*args)
    else:
        lca.mla_latent_attn_decode_up(*args)
    return o, lse, y


@pytest.mark.parametrize("shapes", [((32, 3008), (3, 1500)),      # 8 splits (fused merge), then fewer
                                    ((1, 40000), (2, 5000))])     # many splits (separate merge), then fewer
def test_decode_up_noalloc_matches_workspace_entry_point(shapes):
    cases = [_case(60 + i, B, L) for i, (B, L) in enumerate(shapes)]
    torch.cuda.synchronize()
    for case in cases:  # two calls in a row on the shared scratch, the second smaller
        got = _run(case, noalloc=True)
        want = _run(case, noalloc=False)
        torch.cuda.synchronize()
        for g_, w_ in zip(got, want):
            assert torch.equal(g_, w_), "the no-alloc call must equal the workspace call bit for bit"
        r = host(case["reps"])
        p = case["p"]
        ro, rl = O.decode(case["qd"], r[..., :512], r[..., 512:], p["m"], case["c"], case["kr"],
                          p["raw_begin"], case["L"], 1.0)
        assert_close(host(got[0]), ro, what=f"o_latent B={case['B']} L={case['L']}")
        assert_close(host(got[1]), rl, what="lse")
        assert_close(host(got[2]), O.up_proj(ro, case["wuv"]), what="up-projected output")
