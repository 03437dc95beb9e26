"""Time the two schedules of the attention backward on a set of shapes.

The pages describe a backward that picks a Q-parallel or a KV-parallel
schedule by shape, to keep the gradient reductions cheap (gist.science
Technical Summary §2.2, "Asymmetric Backward Variants").  libwhalefuse has
both: the hybrid (a Q-parallel dQ kernel plus a KV-parallel dK/dV kernel) and
the KV-parallel one (one kernel forms dK, dV and dQ).  This script forces each
in turn through WHALE_XATTN_BWD_SCHEDULE, times whale_jagged_xattn_bwd with
HIP events (median of --reps calls after --warmup), and prints one JSON line
per shape with both times.

    python -m candidate_conditioned_sequence_amd.bwd_schedule_sweep [--reps 20]

Inputs are seeded N(0,1) bf16 tensors; only the timing matters here (the
parity tests check the results).
"""
import argparse
import json
import os
import sys

import numpy as np
import torch

from . import binding as wb
from . import synth

# name, B, C, n_q, d, h, lengths (as in synth.Config.lengths)
SHAPES = [
    ("short_L64", 256, 64, 32, 256, 4, ("fixed", 64)),
    ("short_L128", 256, 64, 32, 256, 4, ("fixed", 128)),
    ("short_U32_128", 256, 64, 32, 256, 4, ("uniform", 32, 128)),
    ("short_L256", 256, 64, 32, 256, 4, ("fixed", 256)),
    ("short_L512", 128, 64, 32, 256, 4, ("fixed", 512)),
    ("c2_shape", 64, 16, 16, 128, 4, ("lognormal", 1500, 0.5, 512, 3000)),
    ("c5_shape", 64, 64, 32, 256, 4, ("lognormal", 6000, 0.5, 3000, 15000)),
    ("few_candidates_L96", 2048, 4, 16, 256, 4, ("fixed", 96)),
]


def time_bwd(dm, t, reps, warmup):
    ws = torch.empty(max(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb.BF16), 256), dtype=torch.uint8,
                     device=t["Q"].device)
    dQ, dK, dV = torch.empty_like(t["Q"]), torch.empty_like(t["K"]), torch.empty_like(t["V"])

    def call():
        wb.whale_jagged_xattn_bwd(dm, t["Q"], t["K"], t["V"], t["off"], 0.0, t["A"], t["lse"], t["dA"], dQ, dK, dV,
                                  ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return float(np.median(ms)), int(ws.numel())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default=None, help="comma-separated shape names")
    args = ap.parse_args()
    wb.load()
    dev = torch.device("cuda:0")
    only = set(args.only.split(",")) if args.only else None
    for name, B, C, n_q, d, h, lengths in SHAPES:
        if only and name not in only:
            continue
        cfg = synth.Config(name, 90, B=B, C=C, n_q=n_q, d=d, h=h, dtype="bf16", lengths=lengths)
        L = synth.lengths(cfg)
        off = synth.offsets_of(L)
        M, T = B * C * n_q, int(off[-1])
        g = torch.Generator(device=dev).manual_seed(7)
        t = {k: torch.randn(n, d, generator=g, device=dev).to(torch.bfloat16)
             for k, n in (("Q", M), ("K", T), ("V", T), ("dA", M))}
        t["off"] = torch.from_numpy(off).to(dev)
        dm = wb.dims(B, C, n_q, d, h, int(L.max()), T)
        t["A"], t["lse"] = torch.empty_like(t["Q"]), torch.empty((M, h), device=dev)
        wb.whale_jagged_xattn_fwd(dm, t["Q"], t["K"], t["V"], t["off"], 0.0, t["A"], t["lse"])
        res = {"shape": name, "B": B, "C": C, "n_q": n_q, "d": d, "h": h, "max_L": int(L.max()), "T": T,
               "mean_L": round(float(L.mean()), 1)}
        flops = 2.5 * 4.0 * d * C * n_q * T
        for sched in ("q", "kv"):
            os.environ["WHALE_XATTN_BWD_SCHEDULE"] = sched
            ms, wsb = time_bwd(dm, t, args.reps, args.warmup)
            res[f"{sched}_ms"] = round(ms, 4)
            res[f"{sched}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
            res[f"{sched}_workspace_mb"] = round(wsb / 2 ** 20, 1)
        del os.environ["WHALE_XATTN_BWD_SCHEDULE"]
        print(json.dumps(res), flush=True)
        del t
        torch.cuda.empty_cache()


if __name__ == "__main__":
    sys.exit(main())
