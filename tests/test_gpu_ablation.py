"""GPU: the ablation modes inside decode, on the synthetic diffuse regime of
the error-versus-length study (seeded; see bench.py --ablation-study).

Properties checked (the ablation table and the length-independence finding of
"Latent-Condensed Transformer for Efficient Long Context Modeling", 消融实验 and
关键发现, on synthetic inputs): the error of condensed decode against exact MLA
does not grow from 4K to 32K tokens, and keeping only the anchor row ("pure
sparse") is clearly further off than the method. Exact MLA is the decode
kernel over all raw rows, itself checked against the oracle elsewhere.
"""
import numpy as np
import pytest
import torch

import lca_inputs as li
import mla_latent_kv_lca_amd as lca

pytestmark = pytest.mark.gpu

H, G, W = 16, 16, 1024


def _abs_errors(L, B=2, steps=2):
    cfg = 750 + L.bit_length()
    c, kr = li.latent_cache(cfg, B, L)
    plan = lca.lca_plan(L, W, G)
    m, rb = plan["m"], plan["raw_begin"]
    qh = torch.from_numpy(li.queries(cfg, B, G, H, rho=0.5)).to("cuda", torch.bfloat16)
    qd = torch.from_numpy(li.queries(cfg, B, steps, H, rho=0.5, stream=1)).to("cuda", torch.bfloat16)
    cache = torch.empty((B, L, 576), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        cache[b] = torch.from_numpy(np.concatenate([c[b], kr[b]], -1)).to("cuda", torch.bfloat16)
    cl = lca.packed_latent(cache)
    ws = lca.decode_workspace(B, H, L)
    o = torch.empty((B, H, 512), dtype=torch.float32, device="cuda")

    def run(reps, mm, begin):
        outs = []
        for st in range(steps):
            lca.mla_latent_attn_decode(qd[:, st].contiguous(), reps, mm, cl, begin, L, 1.0, o, None, ws)
            outs.append(o.clone())
        return torch.stack(outs)

    ref = run(None, 0, 0)
    errs = {}
    for name, mode in (("lca", lca.LCA_MODE_LCA), ("anchor", lca.LCA_MODE_ANCHOR)):
        reps = torch.empty((B, m, 576), dtype=torch.bfloat16, device="cuda")
        anchor = torch.empty((B, m), dtype=torch.int32, device="cuda")
        lca.lca_condense(cl, B, G, 0, m, qh, 0, 0, 1.0, lca.packed_latent(reps), anchor, mode=mode)
        errs[name] = float((run(lca.packed_latent(reps), m, rb) - ref).norm(dim=-1).mean())
    torch.cuda.synchronize()
    assert all(np.isfinite(v) for v in errs.values())
    return errs


@pytest.mark.timeout(300)
def test_condensed_error_flat_in_length_and_pure_sparse_worse():
    e4, e32 = _abs_errors(4096), _abs_errors(32768)
    assert e32["lca"] <= 1.25 * e4["lca"], (e4, e32)
    assert e32["anchor"] >= 1.5 * e32["lca"], e32
