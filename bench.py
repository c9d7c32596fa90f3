#!/usr/bin/env python3
"""Benchmark of the latent-condensed MLA hot path on one MI355X.

Workload (one "step"): batched decode over a latent cache of B = 32 sequences
x L = 32,768 tokens (bf16 rows of 512 c_KV + 64 k_R), H = 16 heads, group
size g = 16, window w = 1024 (m = 1,984 representatives + 1,024 raw rows per
sequence). A step condenses every group once (summary query = mean of the
last 16 history queries) and then runs 64 decode steps, each with fresh
absorbed queries: attention over the condensed cache plus the W_UV
up-projection. The step is repeated over `--layers` independent caches (the
layers of a model), so the working set of consecutive decode kernels
(4 x 111 MB) exceeds the 256 MB Infinity Cache and the kernels stream HBM.

value = context tokens attended per second = layers * B * L * 64 / time.
All inputs are synthetic (seeded) and resident in HBM before timing.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

B, L, H, G, W = 32, 32768, 16, 16, 1024
DECODE_STEPS = 64
HBM_PEAK_GBS = 8000.0
ROW_BYTES = 576 * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roofline-reps", type=int, default=20)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is described in DESIGN.md, not built)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import lca_inputs as li
    import mla_latent_kv_lca_amd as lca

    torch.cuda.set_device(0)
    dev = "cuda"
    plan = lca.lca_plan(L, W, G)
    m, rb = plan["m"], plan["raw_begin"]
    n_ent = plan["n_entries"]
    NL = args.layers

    caches = [li.latent_cache_torch(100 + i, B, L) for i in range(NL)]
    qhist = [li.queries_torch(200 + i, (B, G, H, 576)) for i in range(NL)]
    qsteps = [li.queries_torch(300 + i, (DECODE_STEPS, B, H, 576)) for i in range(NL)]
    wuv = [li.w_uv_torch(400 + i, H) for i in range(NL)]
    reps = [torch.empty((B, m, 576), dtype=torch.bfloat16, device=dev) for _ in range(NL)]
    anchors = [torch.empty((B, m), dtype=torch.int32, device=dev) for _ in range(NL)]
    o_lat = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)
    cws = torch.empty(lca.lca_condense_workspace_size(B, m, 0), dtype=torch.uint8, device=dev)
    dws = torch.empty(max(16, lca.mla_latent_attn_decode_workspace_size(B, H, n_ent)),
                      dtype=torch.uint8, device=dev)
    cache_lat = [lca.packed_latent(c) for c in caches]
    rep_lat = [lca.packed_latent(r) for r in reps]

    def condense(i):
        lca.lca_condense(cache_lat[i], B, G, 0, m, qhist[i], 0, 0, 1.0, rep_lat[i], anchors[i],
                         None, cws)

    def decode(i, st):
        lca.mla_latent_attn_decode(qsteps[i][st], rep_lat[i], m, cache_lat[i], rb, L, 1.0, o_lat,
                                   lse, dws)
        lca.mla_up_proj(o_lat, wuv[i], out)

    def step():
        for i in range(NL):
            condense(i)
        for st in range(DECODE_STEPS):
            for i in range(NL):
                decode(i, st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ctx_tokens = NL * B * L * DECODE_STEPS
    value = ctx_tokens / (ms_per_step / 1e3)

    # per-kernel times with events on the launch stream, cycling the layers
    stream = torch.cuda.current_stream()

    def timed(fn, reps_):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps_)]
        for k in range(reps_):
            ev[k][0].record(stream)
            fn(k)
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / reps_ * 1e-3  # seconds

    t_dec = timed(lambda k: lca.mla_latent_attn_decode(qsteps[k % NL][k % DECODE_STEPS],
                                                       rep_lat[k % NL], m, cache_lat[k % NL], rb,
                                                       L, 1.0, o_lat, lse, dws), args.roofline_reps)
    t_con = timed(lambda k: condense(k % NL), max(4, args.roofline_reps // 4))
    dec_bytes = B * n_ent * ROW_BYTES + B * H * 576 * 2 + B * H * (512 + 1) * 4
    con_bytes = B * m * G * ROW_BYTES + B * G * H * 576 * 2 + B * m * (ROW_BYTES + 4)
    dec_gbs = dec_bytes / t_dec / 1e9
    con_gbs = con_bytes / t_con / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(caches[0], qhist[0], qsteps[0], args.cpu_seconds)

    rec = {
        "metric": "condensed-MLA context tokens/s (decode, incl. condensation)",
        "value": value,
        "unit": "context tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latent cache with RoPE keys, N(0,1/576) queries)",
        "config": {"workload": f"batched LCA decode: B={B} x L={L}, H={H}, g={G}, w={W}, "
                               f"condense once + {DECODE_STEPS} decode steps (+W_UV), "
                               f"{NL} rotating layer caches",
                   "global_batch": B, "seq_len": L, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "mla_latent_attn_decode (decode + split merge)",
                     "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dec_gbs / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": dec_bytes, "avg_launch_us": t_dec * 1e6},
        "condense": {"achieved_gbs": con_gbs, "frac": con_gbs / HBM_PEAK_GBS,
                     "bytes_per_launch": con_bytes, "avg_launch_us": t_con * 1e6},
        "decode_context_tokens_per_s": B * L / t_dec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


def cpu_baseline(cache, qhist, qsteps, budget_s):
    """The fp64 oracle on the first sequences of layer 0 (condense + all 64
    decode steps per sequence) until about budget_s seconds have passed."""
    import numpy as np

    from oracle import lca_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    plan = O.plan(L, W, G)
    m, rb = plan["m"], plan["raw_begin"]
    done, t_total = 0, 0.0
    while done < B and t_total < budget_s:
        b = done
        x = cache[b].float().cpu().numpy().astype(np.float64)
        qh = qhist[b].float().cpu().numpy().astype(np.float64)
        qs = qsteps[:, b].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        rc, rk, _, _, _ = O.condense(x[None, :, :512], x[None, :, 512:], qh[None], G, 0, m, 0, 0, 1.0)
        for st in range(DECODE_STEPS):
            O.decode(qs[st][None], rc, rk, m, x[None, :, :512], x[None, :, 512:], rb, L, 1.0)
        t_total += time.perf_counter() - t0
        done += 1
    return {"value": done * L * DECODE_STEPS / t_total, "unit": "context tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{done} of {B} sequences of one layer (condense + {DECODE_STEPS} decode "
                      f"steps each), {t_total:.1f} s"}


if __name__ == "__main__":
    main()
