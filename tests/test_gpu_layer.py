"""GPU parity of the whole fusion layer against the fp64 oracle for the five
workload configurations.

* reduced: the configuration with fewer requests (the oracle computes every
  output element);
* full size: the configuration at its full shape, run in the launch
  configuration the benchmark uses, checked on sampled requests (shortest,
  median, longest history).  Requests do not interact in the forward, so the
  sampled rows are exact; the weight gradients are checked with the upstream
  gradient zeroed outside the sampled requests, which makes them equal to the
  sampled requests' contribution.
Tolerances: relative Frobenius error <= 1e-5 (fp32), <= 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

from candidate_conditioned_sequence_amd import synth
from candidate_conditioned_sequence_amd.layer import FusionLayer
from oracle import whale_oracle as O
from tests.util import assert_close, host, tdt

pytestmark = pytest.mark.gpu

GRADS = ("dH_w", "dH_s", "dW_Q", "dW_K", "dW_V", "dW_F", "dW_U", "dW_D")


def dev_params(p, dtype, gpu):
    return {k: (torch.from_numpy(v).to(gpu).to(tdt(dtype)) if k.startswith("W_") else torch.from_numpy(v).to(gpu))
            for k, v in p.items()}


def run_layers(cfg, gpu, requests=None, backward=False, dy_mask=None, tied=False):
    """Run cfg.layers stacked layers on the GPU for `requests` (all by default).
    Returns per-layer outputs (host fp64) and, if backward, the gradients of
    the last layer.  tied: shared key-value layers (no W_V)."""
    L = synth.lengths(cfg)
    reqs = list(range(cfg.B)) if requests is None else list(requests)
    H_w = synth.gather(cfg, lambda c, b: synth.h_w_rows(c, b, 0), reqs)
    off = synth.offsets_of(L[reqs])
    toff = torch.from_numpy(off).to(gpu)
    x = torch.from_numpy(H_w).to(gpu).to(tdt(cfg.dtype))
    outs, layer = [], None
    for ell in range(cfg.layers):
        H_s = np.concatenate([synth.h_s_rows(cfg, b, L[b], ell) for b in reqs])
        tHs = torch.from_numpy(H_s).to(gpu).to(tdt(cfg.dtype))
        del H_s
        p = dev_params(synth.layer_params(cfg, ell, random_affine=backward), cfg.dtype, gpu)
        if tied:
            del p["W_V"]
        layer = FusionLayer(p, cfg.C, cfg.n_q, cfg.h, ffn=cfg.ffn)
        out = layer.forward(x, tHs, toff, int(L[reqs].max()), save=backward)
        x = out["Y"]
        outs.append(out)
    res = {"Y": x}
    if backward:
        dY = np.concatenate([synth.dy_rows(cfg, b) for b in reqs])
        if dy_mask is not None:
            per = cfg.C * cfg.n_q
            for i, b in enumerate(reqs):
                if b not in dy_mask:
                    dY[i * per:(i + 1) * per] = 0
        res["grads"] = layer.backward(torch.from_numpy(dY).to(gpu).to(tdt(cfg.dtype)))
    torch.cuda.synchronize()
    return res, outs


def oracle_layers(cfg, requests, backward=False, tied=False):
    L = synth.lengths(cfg)
    H_w = synth.gather(cfg, lambda c, b: synth.h_w_rows(c, b, 0), requests)
    off = synth.offsets_of(L[list(requests)])
    x = H_w
    for ell in range(cfg.layers):
        H_s = np.concatenate([synth.h_s_rows(cfg, b, L[b], ell) for b in requests])
        p = synth.layer_params(cfg, ell, random_affine=backward)
        if tied:
            del p["W_V"]
        if backward and ell == cfg.layers - 1:
            dY = np.concatenate([synth.dy_rows(cfg, b) for b in requests])
            g = O.layer_bwd(x, H_s, off, cfg.C, cfg.n_q, cfg.h, p, dY, ffn=cfg.ffn)
            y = O.layer_fwd(x, H_s, off, cfg.C, cfg.n_q, cfg.h, p, ffn=cfg.ffn)["Y"]
            return y, g
        x = O.layer_fwd(x, H_s, off, cfg.C, cfg.n_q, cfg.h, p, ffn=cfg.ffn)["Y"]
    return x, None


REDUCED = {
    "c1": dict(),
    "c2": dict(B=4),
    "c3": dict(B=2),
    "c4": dict(B=2),
    "c5": dict(B=2),
}


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_config_reduced(gpu, key):
    cfg = synth.scaled(synth.CONFIGS[key], **REDUCED[key])
    backward = key in ("c1", "c5")
    print(f"\n[layer reduced] {cfg.name} B={cfg.B} L={synth.lengths(cfg).tolist()} layers={cfg.layers} "
          f"bwd={backward}", flush=True)
    res, _ = run_layers(cfg, gpu, backward=backward)
    y_ref, g_ref = oracle_layers(cfg, list(range(cfg.B)), backward=backward)
    assert_close("Y", res["Y"], y_ref, cfg.dtype)
    if backward:
        for k in GRADS:
            assert_close(k, res["grads"][k], g_ref[k], cfg.dtype)
        for k in ("dg_q", "db_q", "dg_kv", "db_kv", "dg_f", "db_f"):
            assert_close(k, res["grads"][k], g_ref[k], cfg.dtype)


@pytest.mark.parametrize("key,h", [("c5", 2), ("c4", 4)])
def test_layer_head_width_128(gpu, key, h):
    """Whole layers with d_h = 128 (d = 256, h = 2 forward + backward; d = 512,
    h = 4 forward of one layer of the stack)."""
    cfg = synth.scaled(synth.CONFIGS[key], h=h, **REDUCED[key])
    if key == "c4":
        cfg = synth.scaled(cfg, layers=1)
    backward = key == "c5"
    print(f"\n[layer d_h=128] {cfg.name} d={cfg.d} h={cfg.h} B={cfg.B} L={synth.lengths(cfg).tolist()} "
          f"bwd={backward}", flush=True)
    res, _ = run_layers(cfg, gpu, backward=backward)
    y_ref, g_ref = oracle_layers(cfg, list(range(cfg.B)), backward=backward)
    assert_close("Y", res["Y"], y_ref, cfg.dtype)
    if backward:
        for k in GRADS + ("dg_q", "db_q", "dg_kv", "db_kv", "dg_f", "db_f"):
            assert_close(k, res["grads"][k], g_ref[k], cfg.dtype)


@pytest.mark.parametrize("key", ["c1", "c5"])
def test_shared_kv_layer_reduced(gpu, key):
    """Shared key-value layers: forward and every gradient against the oracle."""
    cfg = synth.scaled(synth.CONFIGS[key], **REDUCED[key])
    print(f"\n[shared kv layer] {cfg.name} B={cfg.B} L={synth.lengths(cfg).tolist()}", flush=True)
    res, _ = run_layers(cfg, gpu, backward=True, tied=True)
    y_ref, g_ref = oracle_layers(cfg, list(range(cfg.B)), backward=True, tied=True)
    assert_close("Y", res["Y"], y_ref, cfg.dtype)
    assert "dW_V" not in res["grads"] and "dW_V" not in g_ref
    for k in GRADS + ("dg_q", "db_q", "dg_kv", "db_kv", "dg_f", "db_f"):
        if k != "dW_V":
            assert_close(k, res["grads"][k], g_ref[k], cfg.dtype)


def test_serving_layer_variable_candidates(gpu):
    """Serving forward with a different number of candidates per request (one
    with none, one with an empty history): the row-wise calls see all query
    rows as one batch, the attention call the candidate offsets."""
    cfg = synth.scaled(synth.CONFIGS["c3"], B=5)
    C_b, L = [64, 5, 0, 33, 2], [3000, 200, 100, 1500, 0]
    coff, off = synth.offsets_of(C_b), synth.offsets_of(L)
    n_q, d = cfg.n_q, cfg.d
    M, T = n_q * int(coff[-1]), int(off[-1])
    r = np.random.default_rng(51)
    H_w = synth.round_bf16(r.standard_normal((M, d)).astype(np.float32))
    H_s = synth.round_bf16(r.standard_normal((T, d)).astype(np.float32))
    p = synth.layer_params(cfg)
    print(f"\n[serving layer] C_b={C_b} L={L}", flush=True)
    layer = FusionLayer(dev_params(p, cfg.dtype, gpu), cfg.C, n_q, cfg.h, ffn=cfg.ffn)
    out = layer.forward(torch.from_numpy(H_w).to(gpu).to(torch.bfloat16),
                        torch.from_numpy(H_s).to(gpu).to(torch.bfloat16), torch.from_numpy(off).to(gpu), max(L),
                        save=False, cand_offsets=torch.from_numpy(coff).to(gpu), max_C=max(C_b))
    torch.cuda.synchronize()
    y_ref = O.layer_fwd(H_w, H_s, off, None, n_q, cfg.h, p, ffn=cfg.ffn, cand_offsets=coff)["Y"]
    assert_close("Y", out["Y"], y_ref, cfg.dtype)


def test_serving_forward_graph_capture(gpu):
    """The serving forward (candidate offsets, host shape hints) captured in a
    HIP graph: every replay, with eager work between replays, gives the eager
    result bit for bit."""
    cfg = synth.scaled(synth.CONFIGS["c3"], B=4)
    C_b, L = [40, 0, 17, 64], [900, 30, 0, 1500]
    coff, off = synth.offsets_of(C_b), synth.offsets_of(L)
    n_q, d = cfg.n_q, cfg.d
    M, T = n_q * int(coff[-1]), int(off[-1])
    r = np.random.default_rng(61)
    tHw = torch.from_numpy(synth.round_bf16(r.standard_normal((M, d)).astype(np.float32))).to(gpu).to(torch.bfloat16)
    tHs = torch.from_numpy(synth.round_bf16(r.standard_normal((T, d)).astype(np.float32))).to(gpu).to(torch.bfloat16)
    toff, tcoff = torch.from_numpy(off).to(gpu), torch.from_numpy(coff).to(gpu)
    layer = FusionLayer(dev_params(synth.layer_params(cfg), cfg.dtype, gpu), cfg.C, n_q, cfg.h, ffn=cfg.ffn)

    def fwd():
        return layer.forward(tHw, tHs, toff, max(L), save=False, cand_offsets=tcoff, max_C=max(C_b))["Y"]

    print(f"\n[serving graph capture] C_b={C_b} L={L}", flush=True)
    eager = fwd().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y = fwd()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
        assert torch.equal(fwd(), eager)
        torch.cuda.synchronize()


def _rows(cfg, L, reqs, sample):
    """Row slices of the sampled requests inside the full-size layout."""
    per = cfg.C * cfg.n_q
    off = synth.offsets_of(L[reqs])
    pos = {b: i for i, b in enumerate(reqs)}
    m = np.concatenate([np.arange(pos[b] * per, (pos[b] + 1) * per) for b in sample])
    t = np.concatenate([np.arange(off[pos[b]], off[pos[b] + 1]) for b in sample])
    return m, t


@pytest.mark.timeout(400)
@pytest.mark.parametrize("key", ["c2", "c3", "c4"])
def test_config_full_size_forward_sampled(gpu, key):
    cfg = synth.CONFIGS[key]
    L = synth.lengths(cfg)
    sample = synth.sample_requests(L, 3 if key != "c4" else 2)
    print(f"\n[layer full] {cfg.name} B={cfg.B} T={int(L.sum())} sample={sample} L={L[sample].tolist()}", flush=True)
    res, _ = run_layers(cfg, gpu)
    m, _ = _rows(cfg, L, list(range(cfg.B)), sample)
    y_ref, _ = oracle_layers(cfg, sample)
    assert_close("Y[sampled]", host(res["Y"])[m], y_ref, cfg.dtype)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("key", ["c5", "c3L10k"])
def test_config_full_size_backward_sampled(gpu, key):
    """Forward and backward at full size in the launch configuration the
    benchmark times (c3L10k is the benchmarked step itself: B = 128, every
    L_b = 10000), checked on sampled requests."""
    cfg = synth.CONFIGS[key]
    L = synth.lengths(cfg)
    sample = synth.sample_requests(L, 2)
    if len(sample) < 2:                        # equal lengths: first and last request
        sample = [0, cfg.B - 1]
    print(f"\n[layer full bwd] {cfg.name} B={cfg.B} T={int(L.sum())} sample={sample} L={L[sample].tolist()}",
          flush=True)
    res, _ = run_layers(cfg, gpu, backward=True, dy_mask=set(sample))
    m, t = _rows(cfg, L, list(range(cfg.B)), sample)
    y_ref, g_ref = oracle_layers(cfg, sample, backward=True)
    g = res["grads"]
    assert_close("Y[sampled]", host(res["Y"])[m], y_ref, cfg.dtype)
    assert_close("dH_w[sampled]", host(g["dH_w"])[m], g_ref["dH_w"], cfg.dtype)
    assert_close("dH_s[sampled]", host(g["dH_s"])[t], g_ref["dH_s"], cfg.dtype)
    # requests outside the sample got a zero upstream gradient: their
    # input gradients are exactly zero
    others = np.setdiff1d(np.arange(cfg.B), sample)[:3]
    mo, to = _rows(cfg, L, list(range(cfg.B)), list(others))
    assert not host(g["dH_w"])[mo].any() and not host(g["dH_s"])[to].any()
    for k in ("dW_Q", "dW_K", "dW_V", "dW_F", "dW_U", "dW_D", "dg_q", "db_q", "dg_kv", "db_kv", "dg_f", "db_f"):
        assert_close(k, g[k], g_ref[k], cfg.dtype)
