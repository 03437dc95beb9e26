"""Benchmark: one fusion-layer step (forward + backward of the whole module)
on the L = 10k, d = 256, C = 64 workload, through the libwhalefuse C ABI.

Workload: B = 128 requests, C = 64 candidates, n_q = 32 query tokens, d = 256,
h = 4 heads (d_h = 64), FFN hidden 4d, shared gate, LayerNorm, every history
L_b = 10000 (T = 1.28M rows), bf16, seeded synthetic inputs already resident
in HBM.  One step = projections, jagged cross-attention, fusion MLP, SwiGLU
FFN, then the backward of all of them with a synthetic upstream gradient.

Prints one JSON line.  `value` is algorithmic TFLOP/s of the whole step (K/V
projections counted once per request, jagged sum of L_b, attention backward
counted as 2.5x its forward).  Per-call times come from HIP events on the
stream the calls run on.  The fp64 CPU oracle is timed on a bounded sample of
requests of the same workload as the CPU baseline.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0

# HBM traffic of one xattn_fwd_pp_kernel<64> launch on this workload:
# rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what
# the counter reads for a 512 MiB elementwise copy (x2.000 and x1.000).  Taken
# from profiles/xattn_fwd_pp_kernel_c3_L10k_hbm_traffic.md; must be re-measured
# (or set to None) whenever that kernel changes.
XATTN_FWD_TRAFFIC = {"kernel": "xattn_fwd_pp_kernel<64>",
                     "fetch_kib": 706662, "fetch_scale": 2.000, "write_kib": 140220, "write_scale": 1.000}
METRIC = "fusion-attn TFLOP/s + requests/s at L=10k,d=256,C=64; % bf16 MFMA peak"


def flops(cfg, T, H, gate_sep=False, shared_kv=False, M=None, pairs=None):
    """Algorithmic FLOPs of one layer (forward, backward) for T history rows.
    With shared keys and values the history side has one projection, not two.
    M (query rows) and pairs (query row, history row of the same request)
    default to the fixed-count layout: B*C*n_q and C*n_q*T."""
    d = cfg.d
    M = cfg.M if M is None else M
    pairs = cfg.C * cfg.n_q * T if pairs is None else pairs
    Hu = 2 * H if gate_sep else H
    attn_f = 4.0 * d * pairs
    kv_f = (2.0 if shared_kv else 4.0) * T * d * d
    gemm_f = 2.0 * M * d * d + kv_f + 2.0 * M * 2 * d * d + 2.0 * M * d * Hu + 2.0 * M * H * d
    return {"attn_fwd": attn_f, "gemm_fwd": gemm_f, "fwd": attn_f + gemm_f,
            "attn_bwd": 2.5 * attn_f, "gemm_bwd": 2.0 * gemm_f, "bwd": 2.5 * attn_f + 2.0 * gemm_f}


def mfma_probe(torch, wb, dev, blocks=2048, iters=10000, reps=5):
    """bf16 MFMA rate the GPU sustains with no memory traffic (TFLOP/s, best
    of `reps` launches of about 5 ms): 8 waves per SIMD of four independent
    MFMA chains.  Run after the warm-up, with the clock already under load."""
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    wb.whale_mfma_peak_probe(out, iters, blocks)
    torch.cuda.synchronize()
    flop = float(blocks) * 4 * iters * 4 * 32 * 32 * 16 * 2
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        wb.whale_mfma_peak_probe(out, iters, blocks)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return {"tflops": round(best, 1), "blocks": blocks, "iters": iters, "kernel": "mfma_peak_kernel"}


def cpu_baseline(cfg, p, L, n_req, shared_kv=False):
    """fp64 oracle, forward + backward of the first n_req requests."""
    from candidate_conditioned_sequence_amd import synth
    from oracle import whale_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    reqs = list(range(n_req))
    H_w, H_s, off = synth.inputs(cfg, requests=reqs)
    dY = np.concatenate([synth.dy_rows(cfg, b) for b in reqs])
    t0 = time.perf_counter()
    O.layer_bwd(H_w, H_s, off, cfg.C, cfg.n_q, cfg.h, p, dY)
    dt = time.perf_counter() - t0
    sub = synth.scaled(cfg, B=n_req)
    f = flops(sub, int(off[-1]), cfg.H, shared_kv=shared_kv)
    total = f["fwd"] + f["bwd"]
    return {"value": total / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "requests_per_s": n_req / dt, "seconds": dt,
            "sample": f"{n_req} request(s) of the same workload (L_b = {int(L[0])}), forward + backward "
                      f"(layer_bwd recomputes the forward), fp64 numpy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-requests", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward only")
    ap.add_argument("--serving", action="store_true",
                    help="forward only, each request with its own candidate count C_b ~ U{16..112} (mean 64)")
    ap.add_argument("--shared-kv", action="store_true",
                    help="shared key-value layer: one history-side projection whose output serves as K and V")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain elementwise copy (negation) of 512 MiB fp32, 3 times: the reference kernel "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the module shards by request "
              "with no exchange in the forward; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from candidate_conditioned_sequence_amd import binding as wb
    from candidate_conditioned_sequence_amd import synth
    from candidate_conditioned_sequence_amd.layer import FusionLayer

    wb.load()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS["c3L10k"]
    L = synth.lengths(cfg)
    T = int(L.sum())
    p = synth.layer_params(cfg)
    if args.shared_kv:
        del p["W_V"]
    print(f"[bench] generating inputs: B={cfg.B} C={cfg.C} n_q={cfg.n_q} d={cfg.d} h={cfg.h} T={T}", file=sys.stderr,
          flush=True)
    H_w, H_s, off = synth.inputs(cfg)
    dY = np.concatenate([synth.dy_rows(cfg, b) for b in range(cfg.B)])
    bf = torch.bfloat16
    tHw = torch.from_numpy(H_w).to(dev).to(bf)
    tHs = torch.from_numpy(H_s).to(dev).to(bf)
    del H_s
    tdY = torch.from_numpy(dY).to(dev).to(bf)
    toff = torch.from_numpy(off).to(dev)
    tp = {k: (torch.from_numpy(v).to(dev).to(bf) if k.startswith("W_") else torch.from_numpy(v).to(dev))
          for k, v in p.items()}
    lay = FusionLayer(tp, cfg.C, cfg.n_q, cfg.h)
    max_L = int(L.max())
    fwd_kw = {"save": not args.fwd_only}
    if args.serving:
        # Serving: forward only; request b scores C_b candidates against its
        # one history (K/V formed once per request).
        args.fwd_only = True
        Cb = synth.candidate_counts(cfg, 16, 112)
        tHw = torch.from_numpy(np.concatenate([synth.h_w_rows_n(cfg, b, int(Cb[b])) for b in range(cfg.B)])).to(
            dev).to(bf)
        fwd_kw = {"save": False, "cand_offsets": torch.from_numpy(synth.offsets_of(Cb)).to(dev),
                  "max_C": int(Cb.max())}

    calls = ["proj_qkv", "xattn_fwd", "fusion_mlp", "swiglu_ffn", "ffn_bwd", "fusion_bwd", "xattn_bwd", "proj_bwd"]

    class Timed:
        """Events around each C-ABI call, on the stream the calls use."""

        def __init__(self):
            self.ev = []

        def mark(self, name):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            self.ev.append((name, e))

    def step(tm=None):
        # forward, call by call (same sequence as FusionLayer.forward/backward)
        if tm: tm.mark("start")
        out = lay.forward(tHw, tHs, toff, max_L, **fwd_kw)
        if tm: tm.mark("fwd_end")
        if not args.fwd_only:
            lay.backward(tdY)
        if tm: tm.mark("end")
        return out

    # Per-call timing uses a wrapped binding: record an event after every call.
    per_call = {c: [] for c in calls}
    orig = {}
    names = {"whale_proj_qkv": "proj_qkv", "whale_jagged_xattn_fwd": "xattn_fwd",
             "whale_jagged_xattn_fwd_varc": "xattn_fwd", "whale_fusion_mlp": "fusion_mlp",
             "whale_swiglu_ffn": "swiglu_ffn", "whale_swiglu_ffn_bwd": "ffn_bwd",
             "whale_fusion_mlp_bwd": "fusion_bwd", "whale_jagged_xattn_bwd": "xattn_bwd",
             "whale_proj_qkv_bwd": "proj_bwd"}
    record = {"on": False, "events": []}
    for fn, short in names.items():
        orig[fn] = getattr(wb, fn)

        def wrapped(*a, _f=orig[fn], _n=short, **k):
            if record["on"]:
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record()
            _f(*a, **k)
            if record["on"]:
                e1 = torch.cuda.Event(enable_timing=True)
                e1.record()
                record["events"].append((_n, e0, e1))
        setattr(wb, fn, wrapped)
    import candidate_conditioned_sequence_amd.layer as layer_mod
    layer_mod.wb = wb

    if args.calibrate_copy:
        # torch.neg over 2^27 fp32 values: one elementwise kernel that reads
        # and writes exactly 512 MiB.
        src = torch.ones(1 << 27, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    probe = mfma_probe(torch, wb, dev)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    record["on"] = True
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    record["on"] = False
    ms = ev0.elapsed_time(ev1) / args.steps
    for n, e0, e1 in record["events"]:
        per_call[n].append(e0.elapsed_time(e1))
    avg = {n: float(np.mean(v)) for n, v in per_call.items() if v}

    if args.serving:
        f = flops(cfg, T, cfg.H, shared_kv=args.shared_kv, M=int(tHw.shape[0]), pairs=cfg.n_q * float(np.dot(Cb, L)))
    else:
        f = flops(cfg, T, cfg.H, shared_kv=args.shared_kv)
    step_flops = f["fwd"] + (0.0 if args.fwd_only else f["bwd"])
    fwd_ms = sum(avg[c] for c in ("proj_qkv", "xattn_fwd", "fusion_mlp", "swiglu_ffn"))
    value = step_flops / (ms * 1e-3) / 1e12

    # Roofline of the dominant call.  xattn_fwd is a single kernel launch.
    attn_ms = avg["xattn_fwd"]
    attn_tflops = f["attn_fwd"] / (attn_ms * 1e-3) / 1e12
    kname = "xattn_fwd_pp_kernel<64>"
    tr = XATTN_FWD_TRAFFIC
    traffic = None
    if tr is not None and tr["kernel"] == kname and not (args.shared_kv or args.serving):
        traffic = int(1024 * (tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]))
    M, d = cfg.M, cfg.d
    if args.serving:
        M = int(tHw.shape[0])
    algo_bytes = 2 * (M * d + (1 if args.shared_kv else 2) * T * d + M * d) + 4 * M * cfg.h
    roof = {"bound": "mfma", "kernel": kname, "achieved": round(attn_tflops, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic, "traffic_unit": "bytes per launch", "algorithmic_bytes": algo_bytes,
            "algorithmic_flops": f["attn_fwd"],
            "measured_peak": probe["tflops"], "frac_of_measured_peak": round(attn_tflops / probe["tflops"], 4)}
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("fusion layer fwd, serving, C_b ~ U{16..112}" if args.serving else
                                "fusion layer fwd+bwd" if not args.fwd_only else "fusion layer fwd"),
                   "B": cfg.B, "C": cfg.C, "n_q": cfg.n_q, "d": cfg.d, "h": cfg.h, "H": cfg.H, "L_b": int(L[0]),
                   "T": T, "gate": "shared", "norm": "layer", "kv": "shared" if args.shared_kv else "separate"},
        "requests_per_s": round(cfg.B / (ms * 1e-3), 1),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 3), "tflops": round(f["fwd"] / (fwd_ms * 1e-3) / 1e12, 1),
                "requests_per_s": round(cfg.B / (fwd_ms * 1e-3), 1),
                "pct_bf16_peak": round(100 * f["fwd"] / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)},
        "attn_fwd": {"ms": round(attn_ms, 3), "tflops": round(attn_tflops, 1)},
        "per_call_ms": {k: round(v, 3) for k, v in avg.items()},
        "roofline": roof,
        "mfma_probe": probe,
        "wall_s": round(wall, 2),
    }
    if not args.no_cpu:
        print(f"[bench] cpu baseline ({args.cpu_requests} requests, fp64 oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, p, L, args.cpu_requests, args.shared_kv)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
