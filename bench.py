"""Benchmark of the WHALE fusion layer through the libwhalefuse C ABI.

Default workload (the headline): one fusion-layer step, forward + backward of
the whole module, at B = 128 requests, C = 64 candidates, n_q = 32 query
tokens, d = 256, h = 4 heads (d_h = 64), FFN hidden 4d, shared gate,
LayerNorm, every history L_b = 10000 (T = 1.28M rows), bf16, seeded synthetic
inputs already resident in HBM.

`--config` selects one of the workload configurations instead (shapes and
length distributions follow the pages' sweeps: widths 64-512, histories
3k-15k, 2-8 layers):
  c3L10k  the headline above (forward + backward)
  c2      B=64, C=16, n_q=16, d=128, h=4, L_b ~ lognormal(1500) in [512, 3000];
          projections + attention + fusion MLP, forward
  c3      B=128, C=64, n_q=32, d=256, h=4, L_b ~ U{3000..10000}; whole module, forward
  c4      B=64, C=128, n_q=32, d=512, h=8, L_b ~ U{10000..15000}; 8 stacked layers, forward
  c5      B=64, C=64, n_q=32, d=256, h=4, L_b ~ lognormal(6000) in [3000, 15000];
          whole module, forward + backward

Prints one JSON line.  `value` is algorithmic TFLOP/s of the step (K/V
projections counted once per request, jagged sum of L_b, attention backward
counted as 2.5x its forward), from the median step time.  Per-call times come
from HIP events on the stream the calls run on.  `roofline` covers the
dominant call; `cpu_baseline` times the fp64 CPU oracle on a bounded sample of
requests of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_ALU_TLANE = 39.3          # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, lane-instructions / s
HSTU_INSTR_PER_SCORE = 9.5     # HSTU forward, per-element form (fixed reference count)

# HBM traffic of one xattn_fwd_pp_kernel<64> launch on the headline workload
# (profiles/hbm_traffic_c3_L10k_all_kernels.md):
# rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what
# the counter reads for a 512 MiB elementwise copy (x2.000 and x1.000), taken
# on the kernel source whose SHA-256 prefix is recorded here.  When the source
# differs, the figure no longer describes the kernel and is reported as null.
XATTN_FWD_TRAFFIC = {"kernel": "xattn_fwd_pp_kernel<64>", "config": "c3L10k",
                     "source": "candidate_conditioned_sequence_amd/csrc/xattn_fwd.hip",
                     "source_sha256_16": "1a65f62065d3bc51",
                     "fetch_kib": 705704, "fetch_scale": 2.000, "write_kib": 147456, "write_scale": 1.000}
METRIC = "fusion-attn TFLOP/s + requests/s at L=10k,d=256,C=64; % bf16 MFMA peak"

# Per configuration: what one step covers, and the CPU-oracle sample.
SCOPE = {
    "c3L10k": dict(backward=True, cpu_requests=8),
    "c2": dict(backward=False, cpu_requests=64),
    "c3": dict(backward=False, cpu_requests=12),
    "c4": dict(backward=False, cpu_requests=1),
    "c5": dict(backward=True, cpu_requests=6),
}


def source_sha16(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def flops(cfg, T, H, gate_sep=False, shared_kv=False, M=None, pairs=None, ffn=True):
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
    gemm_f = 2.0 * M * d * d + kv_f + 2.0 * M * 2 * d * d
    if ffn:
        gemm_f += 2.0 * M * d * Hu + 2.0 * M * H * d
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


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return None


def cpu_baseline(cfg, key, n_req, backward, shared_kv=False):
    """The fp64 oracle on the first n_req requests of the workload (each
    layer of a stack in turn), forward, or forward + backward."""
    from candidate_conditioned_sequence_amd import synth
    from oracle import whale_oracle as O
    L = synth.lengths(cfg)
    reqs = list(range(min(n_req, cfg.B)))
    off = synth.offsets_of(L[reqs])
    x = synth.gather(cfg, lambda c, b: synth.h_w_rows(c, b, 0), reqs)
    H_s = [np.concatenate([synth.h_s_rows(cfg, b, L[b], ell) for b in reqs]) for ell in range(cfg.layers)]
    ps = []
    for ell in range(cfg.layers):
        p = synth.layer_params(cfg, ell)
        if shared_kv:
            del p["W_V"]
        ps.append(p)
    dY = np.concatenate([synth.dy_rows(cfg, b) for b in reqs]) if backward else None
    t0 = time.perf_counter()
    for ell in range(cfg.layers):
        if backward and ell == cfg.layers - 1:
            O.layer_bwd(x, H_s[ell], off, cfg.C, cfg.n_q, cfg.h, ps[ell], dY, ffn=cfg.ffn)
        else:
            x = O.layer_fwd(x, H_s[ell], off, cfg.C, cfg.n_q, cfg.h, ps[ell], ffn=cfg.ffn)["Y"]
    dt = time.perf_counter() - t0
    sub = synth.scaled(cfg, B=len(reqs))
    f = flops(sub, int(off[-1]), cfg.H, shared_kv=shared_kv, ffn=cfg.ffn)
    total = cfg.layers * f["fwd"] + (f["bwd"] if backward else 0.0)
    what = "forward + backward (layer_bwd recomputes the forward)" if backward else "forward"
    return {"value": total / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads() or host_cores(),
            "host_cores": host_cores(), "blas_threads": blas_threads(), "kind": "oracle",
            "requests_per_s": len(reqs) / dt, "seconds": dt,
            "sample": f"{len(reqs)} request(s) of the {key} workload (L_b = {L[reqs].tolist()[:8]}"
                      f"{'...' if len(reqs) > 8 else ''}), {cfg.layers} layer(s), {what}, fp64 numpy"}


def bench_hstu(args, torch, wb, synth, dev):
    """HSTU self-attention forward on one configuration's histories: every
    request attends causally over its own history (pairs = sum L_b (L_b + 1) / 2
    per head), inputs N(0, 1) bf16 resident in HBM."""
    key = "c5" if args.config == "c3L10k" else args.config
    cfg = synth.CONFIGS[key]
    L = synth.lengths(cfg)
    off = synth.offsets_of(L)
    T, d, h = int(off[-1]), cfg.d, cfg.h
    print(f"[bench] hstu on {key} histories: B={cfg.B} T={T} d={d} h={h}", file=sys.stderr, flush=True)
    g = torch.Generator(device=dev).manual_seed(0)
    Q, K, V = (torch.randn(T, d, generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    ts = torch.from_numpy(np.concatenate([synth.timestamps(cfg, b, L[b]) for b in range(cfg.B)])).to(dev)
    wp, wt = (torch.from_numpy(x).to(dev) for x in synth.hstu_tables(cfg, 4096, 32))
    toff = torch.from_numpy(off).to(dev)
    dm = wb.dims(cfg.B, 1, 1, d, h, int(L.max()), T)
    A = torch.empty_like(Q)

    def call():
        wb.whale_hstu_attn_fwd(dm, Q, K, V, toff, ts, wp, wt, 0.0, A)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    pairs = float(np.sum(L * (L + 1) // 2))
    flop = 4.0 * d * pairs
    scores = pairs * h
    tflops = flop / (ms * 1e-3) / 1e12
    res = {"metric": "HSTU self-attention TFLOP/s (causal pairs) and Gscore/s", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"HSTU jagged causal self-attention with rab on the {key} histories", "name": key,
                      "B": cfg.B, "d": d, "h": h, "T": T, "n_pos": 4096, "n_time": 32},
           "gscore_per_s": round(scores / (ms * 1e-3) / 1e9, 1),
           "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2)}
    # Roofline: the kernel is bound by vector ALU issue.  Work per score in
    # the straightforward per-element form: bias add, fused multiply-add,
    # exp2, add, reciprocal, multiply, the saturating time difference, its
    # leading-zero count and address shift, half a bf16 pack (9.5; the
    # kernel folds the first two into its MFMAs and issues 8.5).  Fixed, so
    # that the fraction compares kernel versions.
    # Peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-instructions/s.
    gsc = scores / (ms * 1e-3)
    achieved = gsc * HSTU_INSTR_PER_SCORE / 1e12
    res["roofline"] = {"bound": "alu", "kernel": f"hstu_fwd_kernel<bf16,{d // h}>", "call": "whale_hstu_attn_fwd",
                       "achieved": round(achieved, 2), "peak": PEAK_ALU_TLANE, "unit": "T lane-instr/s",
                       "frac": round(achieved / PEAK_ALU_TLANE, 4), "traffic": None,
                       "instr_per_score": HSTU_INSTR_PER_SCORE,
                       "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    if not args.no_cpu:
        res["cpu_baseline"] = hstu_cpu_baseline(cfg, key, L, d, h)
    print(json.dumps(res))


def hstu_cpu_baseline(cfg, key, L, d, h, n_req=25):
    """The fp64 oracle on the n_req shortest histories of the workload."""
    from oracle import whale_oracle as O
    from candidate_conditioned_sequence_amd import synth
    reqs = [int(b) for b in np.argsort(L, kind="stable")[:n_req]]
    Ls = L[reqs]
    off = synth.offsets_of(Ls)
    T = int(off[-1])
    r = np.random.default_rng(1)
    q, k, v = (r.standard_normal((T, d)) for _ in range(3))
    ts = np.concatenate([synth.timestamps(cfg, b, L[b]) for b in reqs])
    wp, wt = synth.hstu_tables(cfg, 4096, 32)
    t0 = time.perf_counter()
    O.hstu_attn_fwd(q, k, v, off, h, ts, wp, wt)
    dt = time.perf_counter() - t0
    pairs = float(np.sum(Ls * (Ls + 1) // 2))
    return {"value": 4.0 * d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads() or host_cores(),
            "host_cores": host_cores(), "blas_threads": blas_threads(), "kind": "oracle",
            "gscore_per_s": pairs * h / dt / 1e9, "seconds": dt,
            "sample": f"the {len(reqs)} shortest request(s) of the {key} histories (L_b = {Ls.tolist()}), "
                      f"N(0, 1) inputs, fp64 numpy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3L10k", choices=sorted(SCOPE))
    ap.add_argument("--cpu-requests", type=int, default=None, help="requests in the CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward only")
    ap.add_argument("--serving", action="store_true",
                    help="forward only, each request with its own candidate count C_b ~ U{16..112} (mean 64)")
    ap.add_argument("--shared-kv", action="store_true",
                    help="shared key-value layer: one history-side projection whose output serves as K and V")
    ap.add_argument("--hstu", action="store_true",
                    help="time the HSTU self-attention (whale_hstu_attn_fwd) on the history shapes of --config "
                         "(c5 by default for this mode), position table 4096, time table 32")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward replayed from one HIP graph capture (forward-only steps)")
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
    if args.hstu:
        return bench_hstu(args, torch, wb, synth, dev)
    key = args.config
    cfg = synth.CONFIGS[key]
    backward = SCOPE[key]["backward"] and not (args.fwd_only or args.serving)
    L = synth.lengths(cfg)
    T = int(L.sum())
    bf = torch.bfloat16
    print(f"[bench] {key}: generating inputs: B={cfg.B} C={cfg.C} n_q={cfg.n_q} d={cfg.d} h={cfg.h} T={T} "
          f"layers={cfg.layers}", file=sys.stderr, flush=True)
    H_w, H_s0, off = synth.inputs(cfg)
    tHw = torch.from_numpy(H_w).to(dev).to(bf)
    toff = torch.from_numpy(off).to(dev)
    layers, tHs = [], []
    for ell in range(cfg.layers):
        p = synth.layer_params(cfg, ell)
        if args.shared_kv:
            del p["W_V"]
        hs = H_s0 if ell == 0 else np.concatenate([synth.h_s_rows(cfg, b, L[b], ell) for b in range(cfg.B)])
        tHs.append(torch.from_numpy(hs).to(dev).to(bf))
        del hs
        tp = {k: (torch.from_numpy(v).to(dev).to(bf) if k.startswith("W_") else torch.from_numpy(v).to(dev))
              for k, v in p.items()}
        layers.append(FusionLayer(tp, cfg.C, cfg.n_q, cfg.h, ffn=cfg.ffn))
    del H_s0
    tdY = torch.from_numpy(np.concatenate([synth.dy_rows(cfg, b) for b in range(cfg.B)])).to(dev).to(bf) \
        if backward else None
    max_L = int(L.max())
    fwd_kw = {"save": backward}
    Cb = None
    if args.serving:
        # Serving: forward only; request b scores C_b candidates against its
        # one history (K/V formed once per request).
        Cb = synth.candidate_counts(cfg, 16, 112)
        tHw = torch.from_numpy(np.concatenate([synth.h_w_rows_n(cfg, b, int(Cb[b])) for b in range(cfg.B)])).to(
            dev).to(bf)
        fwd_kw = {"save": False, "cand_offsets": torch.from_numpy(synth.offsets_of(Cb)).to(dev),
                  "max_C": int(Cb.max())}

    # Per-call timing: each C-ABI call is wrapped with events on the current
    # stream, the stream every call is enqueued on.
    names = {"whale_proj_qkv": "proj_qkv", "whale_jagged_xattn_fwd": "xattn_fwd",
             "whale_jagged_xattn_fwd_varc": "xattn_fwd", "whale_fusion_mlp": "fusion_mlp",
             "whale_swiglu_ffn": "swiglu_ffn", "whale_swiglu_ffn_bwd": "ffn_bwd",
             "whale_fusion_mlp_bwd": "fusion_bwd", "whale_jagged_xattn_bwd": "xattn_bwd",
             "whale_proj_qkv_bwd": "proj_bwd"}
    record = {"on": False, "events": []}
    for fn, short in names.items():
        def wrapped(*a, _f=getattr(wb, fn), _n=short, **k):
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

    def step():
        """One step; returns the events bracketing it and its forward."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        x = tHw
        for ell, lay in enumerate(layers):
            x = lay.forward(x, tHs[ell], toff, max_L, **fwd_kw)["Y"]
        ev[1].record()
        if backward:
            layers[-1].backward(tdY)
        ev[2].record()
        return ev

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
    torch.cuda.synchronize()
    steps = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    record["on"] = False
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in steps])
    fwd_span = np.array([e[0].elapsed_time(e[1]) for e in steps])
    ms_total = steps[0][0].elapsed_time(steps[-1][2])
    ms = float(np.median(step_ms))
    per_call = {}
    for n, e0, e1 in record["events"]:
        per_call.setdefault(n, []).append(e0.elapsed_time(e1))
    # per step: a stack runs each forward call once per layer
    avg = {n: float(np.sum(v)) / args.steps for n, v in per_call.items()}

    graph_ms, graph_equal = None, None
    if args.graph:
        # The same forward captured once in a HIP graph and replayed: no host
        # launch gaps between the calls.  The replay's output is checked bit
        # for bit against an eager forward before it is timed.
        if backward:
            print("--graph times forward-only steps (use --fwd-only)", file=sys.stderr)
            sys.exit(2)

        def run_fwd():
            x = tHw
            for ell, lay in enumerate(layers):
                x = lay.forward(x, tHs[ell], toff, max_L, **fwd_kw)["Y"]
            return x
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_fwd()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            y_graph = run_fwd()
        torch.cuda.synchronize()
        y_eager = run_fwd().clone()
        g.replay()
        torch.cuda.synchronize()
        graph_equal = bool(torch.equal(y_graph, y_eager))
        gev = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            gev.append((e0, e1))
        torch.cuda.synchronize()
        graph_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in gev]))
        del g, y_graph, y_eager

    if args.serving:
        f = flops(cfg, T, cfg.H, shared_kv=args.shared_kv, M=int(tHw.shape[0]), pairs=cfg.n_q * float(np.dot(Cb, L)),
                  ffn=cfg.ffn)
    else:
        f = flops(cfg, T, cfg.H, shared_kv=args.shared_kv, ffn=cfg.ffn)
    fwd_flops = cfg.layers * f["fwd"]
    step_flops = fwd_flops + (f["bwd"] if backward else 0.0)
    fwd_ms = float(np.median(fwd_span))
    value = step_flops / (ms * 1e-3) / 1e12

    # Roofline of the dominant call: the attention forward (one kernel launch
    # per layer) or, in a step with the backward where it dominates, the
    # attention backward (the dQ and dK/dV kernels of one call).
    per_layer_attn_ms = avg["xattn_fwd"] / cfg.layers
    attn_tflops = f["attn_fwd"] / (per_layer_attn_ms * 1e-3) / 1e12
    M, d = (int(tHw.shape[0]) if args.serving else cfg.M), cfg.d
    nkv = 1 if args.shared_kv else 2
    algo_bytes = 2 * (M * d + nkv * T * d + M * d) + 4 * M * cfg.h
    pp = d // cfg.h == 64 and cfg.C * cfg.n_q >= 1024
    kname = "xattn_fwd_pp_kernel<64>" if pp else f"xattn_fwd_kernel<bf16,{d // cfg.h},...>"
    tr = XATTN_FWD_TRAFFIC
    traffic = None
    if (tr["kernel"] == kname and tr["config"] == key and not (args.shared_kv or args.serving)
            and source_sha16(tr["source"]) == tr["source_sha256_16"]):
        traffic = int(1024 * (tr["fetch_kib"] * tr["fetch_scale"] + tr["write_kib"] * tr["write_scale"]))
    ai = f["attn_fwd"] / algo_bytes
    bound_tflops = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)
    roof = {"bound": "mfma", "kernel": kname, "call": "whale_jagged_xattn_fwd",
            "achieved": round(attn_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "traffic_unit": "bytes per launch",
            "algorithmic_bytes": algo_bytes, "algorithmic_flops": f["attn_fwd"],
            "arithmetic_intensity": round(ai, 1), "roofline_tflops": round(bound_tflops, 1),
            "frac_of_roofline": round(attn_tflops / bound_tflops, 4),
            "measured_peak": probe["tflops"], "frac_of_measured_peak": round(attn_tflops / probe["tflops"], 4)}
    if backward and key != "c3L10k" and avg.get("xattn_bwd", 0.0) > avg["xattn_fwd"]:
        bwd_tflops = f["attn_bwd"] / (avg["xattn_bwd"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": "bwd_dq_kernel<bf16,64,8> + bwd_dkdv_kernel<bf16,64,8>",
                "call": "whale_jagged_xattn_bwd", "achieved": round(bwd_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "traffic_unit": "bytes per launch", "algorithmic_flops": f["attn_bwd"],
                "measured_peak": probe["tflops"], "frac_of_measured_peak": round(bwd_tflops / probe["tflops"], 4),
                "attn_fwd": {"kernel": kname, "achieved": round(attn_tflops, 1),
                             "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4)}}
    workload = {"c3L10k": "fusion layer fwd+bwd", "c2": "fusion layer fwd without FFN",
                "c3": "fusion layer fwd", "c4": "8-layer fusion stack fwd", "c5": "fusion layer fwd+bwd"}[key]
    if args.serving:
        workload = "fusion layer fwd, serving, C_b ~ U{16..112}"
    elif args.fwd_only:
        workload = workload.replace("fwd+bwd", "fwd")
    lk = cfg.lengths
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload, "name": key, "B": cfg.B, "C": cfg.C, "n_q": cfg.n_q, "d": cfg.d, "h": cfg.h,
                   "H": cfg.H if cfg.ffn else None, "layers": cfg.layers,
                   "L_b": lk[1] if lk[0] == "fixed" else list(lk), "T": T, "gate": "shared", "norm": "layer",
                   "kv": "shared" if args.shared_kv else "separate"},
        "ms_per_step_mean": round(float(np.mean(step_ms)), 3), "ms_per_step_min": round(float(np.min(step_ms)), 3),
        "ms_all_steps": round(ms_total, 3),
        "requests_per_s": round(cfg.B / (ms * 1e-3), 1),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 3), "tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 1),
                "requests_per_s": round(cfg.B / (fwd_ms * 1e-3), 1),
                "pct_bf16_peak": round(100 * fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                "target_pct_bf16_peak": 50.0},
        "attn_fwd": {"ms_per_layer": round(per_layer_attn_ms, 3), "tflops": round(attn_tflops, 1)},
        "per_call_ms": {k: round(v, 3) for k, v in avg.items()},
        "roofline": roof,
        "mfma_probe": probe,
        "wall_s": round(wall, 2),
    }
    if graph_ms is not None:
        res["graph"] = {"ms_per_step": round(graph_ms, 3),
                        "tflops": round(step_flops / (graph_ms * 1e-3) / 1e12, 2),
                        "requests_per_s": round(cfg.B / (graph_ms * 1e-3), 1),
                        "output_equal_to_eager": graph_equal}
    if not args.no_cpu:
        n_req = args.cpu_requests or SCOPE[key]["cpu_requests"]
        print(f"[bench] cpu baseline ({n_req} requests, fp64 oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, key, n_req, backward, args.shared_kv)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
