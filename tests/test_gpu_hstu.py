"""GPU parity of the HSTU self-attention (reading R12) against the fp64
oracle through the C ABI: ragged histories (lengths 0, 1, 63-65, 129, 257,
...), every head width, position tables shorter and longer than the
histories (the far-tile path and the gathers), one-entry tables, and the
full c5 history shapes on sampled requests; bitwise causality and request
independence.  Tolerances as for the fusion attention (relative Frobenius
1e-5 fp32, 2e-2 bf16, with the per-row bound)."""
import numpy as np
import pytest
import torch

from candidate_conditioned_sequence_amd import binding as wb
from candidate_conditioned_sequence_amd import synth
from oracle import whale_oracle as O
from tests.util import assert_close, f32_dev, host, i64_dev, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, L, d, dtype, n_pos, n_time):
    cfg = synth.scaled(synth.CONFIGS["c5"], B=len(L), lengths=("list", list(L)))
    off = synth.offsets_of(L)
    T = int(off[-1])
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((T, d)).astype(np.float32) for _ in range(3))
    if dtype == "bf16":
        q, k, v = synth.round_bf16(q), synth.round_bf16(k), synth.round_bf16(v)
    ts = np.concatenate([synth.timestamps(cfg, b, L[b]) for b in range(len(L))]) if T else np.zeros(0, np.int64)
    wp, wt = synth.hstu_tables(cfg, n_pos, n_time)
    return q, k, v, off, ts, wp, wt


def _run(gpu, q, k, v, off, ts, wp, wt, h, dtype, scale=0.0):
    L = np.diff(off)
    T, d = q.shape
    dm = wb.dims(len(L), 1, 1, d, h, int(L.max()) if len(L) else 0, T)
    tq, tk, tv = to_dev(q, dtype, gpu), to_dev(k, dtype, gpu), to_dev(v, dtype, gpu)
    A = torch.full_like(tq, float("nan"))
    wb.whale_hstu_attn_fwd(dm, tq, tk, tv, i64_dev(off, gpu), i64_dev(ts, gpu), f32_dev(wp, gpu), f32_dev(wt, gpu),
                           scale, A)
    torch.cuda.synchronize()
    return A


CASES = [
    # dtype, d, h, lengths, n_pos, n_time
    ("f32", 64, 2, [0, 1, 63, 64, 65, 257], 50, 20),
    ("bf16", 128, 4, [130, 1, 700, 64], 300, 32),
    ("bf16", 256, 4, [1000, 333, 129], 64, 16),
    ("bf16", 256, 2, [300, 77, 0], 4096, 32),
    ("f32", 256, 2, [200, 65], 100, 7),
    ("bf16", 512, 8, [2000], 128, 24),
    ("bf16", 256, 4, [190, 5], 1, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-d{c[1]}h{c[2]}-L{c[3]}-P{c[4]}-T{c[5]}")
def test_hstu_attn_fwd(gpu, case):
    dtype, d, h, L, n_pos, n_time = case
    print(f"\n[hstu fwd] {case}", flush=True)
    q, k, v, off, ts, wp, wt = _inputs(3, L, d, dtype, n_pos, n_time)
    A = _run(gpu, q, k, v, off, ts, wp, wt, h, dtype)
    ref = O.hstu_attn_fwd(q, k, v, off, h, ts, wp, wt)
    assert_close("A", A, ref, dtype)


def test_hstu_is_causal_bitwise(gpu):
    """Rows after i (their K, V and timestamps) do not move row i by one bit."""
    L, d, h = [1000], 256, 4
    q, k, v, off, ts, wp, wt = _inputs(5, L, d, "bf16", 256, 32)
    A0 = _run(gpu, q, k, v, off, ts, wp, wt, h, "bf16")
    k2, v2, ts2 = k.copy(), v.copy(), ts.copy()
    k2[600:] = synth.round_bf16(np.float32(3.0) * k2[600:])
    v2[600:] = -v2[600:]
    ts2[600:] += 10 ** 6
    A1 = _run(gpu, q, k2, v2, off, ts2, wp, wt, h, "bf16")
    assert torch.equal(A0[:600], A1[:600])
    assert not torch.equal(A0[600:], A1[600:])


def test_hstu_requests_independent_bitwise(gpu):
    L, d, h = [700, 300, 128], 128, 4
    q, k, v, off, ts, wp, wt = _inputs(7, L, d, "bf16", 200, 32)
    A0 = _run(gpu, q, k, v, off, ts, wp, wt, h, "bf16")
    q2 = q.copy()
    q2[off[1]:off[2]] = synth.round_bf16(np.float32(0.5) * q2[off[1]:off[2]])
    A1 = _run(gpu, q2, k, v, off, ts, wp, wt, h, "bf16")
    assert torch.equal(A0[:off[1]], A1[:off[1]]) and torch.equal(A0[off[2]:], A1[off[2]:])
    # one request alone gives the same bits as inside the batch
    sl = slice(int(off[2]), int(off[3]))
    A2 = _run(gpu, q[sl], k[sl], v[sl], np.array([0, L[2]]), ts[sl], wp, wt, h, "bf16")
    assert torch.equal(A2, A0[sl])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hstu_unordered_and_extreme_timestamps(gpu, dtype):
    """Timestamps out of order (negative differences fall in bucket 0), runs
    of equal timestamps (difference 0), and values up to 2^30 - 1 either side
    of the request's first (differences near 2^31: buckets 29 and 30)."""
    L, d, h = [300, 130, 65], 128, 2
    q, k, v, off, _, wp, wt = _inputs(9, L, d, dtype, 200, 32)
    r = np.random.default_rng(19)
    parts = []
    for b, n in enumerate(L):
        first = 1_700_000_000 + 10 ** 9 * b
        t = first + r.integers(-(2 ** 30) + 1, 2 ** 30, n)
        t[0] = first
        t[5:25] = t[5]                                  # equal timestamps
        t[-3:] = [first + 2 ** 30 - 1, first - 2 ** 30 + 1, first]
        parts.append(t.astype(np.int64))
    ts = np.concatenate(parts)
    A = _run(gpu, q, k, v, off, ts, wp, wt, h, dtype)
    ref = O.hstu_attn_fwd(q, k, v, off, h, ts, wp, wt)
    assert_close("A", A, ref, dtype)


@pytest.mark.timeout(300)
def test_hstu_c5_histories_full_size_sampled(gpu):
    """The c5 history shapes (B = 64, L_b ~ lognormal(6000) in [3000, 15000],
    d = 256, h = 4) in one launch, the benchmark's launch configuration,
    checked on the shortest and the median request."""
    cfg = synth.CONFIGS["c5"]
    L = synth.lengths(cfg)
    off = synth.offsets_of(L)
    T, d, h = int(off[-1]), cfg.d, cfg.h
    sample = synth.sample_requests(L, 2)
    print(f"\n[hstu full] B={cfg.B} T={T} sample={sample} L={L[sample].tolist()}", flush=True)
    g = torch.Generator(device=gpu).manual_seed(11)
    tq, tk, tv = (torch.randn(T, d, generator=g, device=gpu).to(torch.bfloat16) for _ in range(3))
    ts = np.concatenate([synth.timestamps(cfg, b, L[b]) for b in range(cfg.B)])
    wp, wt = synth.hstu_tables(cfg, 4096, 32)
    dm = wb.dims(cfg.B, 1, 1, d, h, int(L.max()), T)
    A = torch.empty_like(tq)
    wb.whale_hstu_attn_fwd(dm, tq, tk, tv, i64_dev(off, gpu), i64_dev(ts, gpu), f32_dev(wp, gpu), f32_dev(wt, gpu),
                           0.0, A)
    torch.cuda.synchronize()
    for b in sample:
        sl = slice(int(off[b]), int(off[b + 1]))
        ref = O.hstu_attn_fwd(host(tq[sl]), host(tk[sl]), host(tv[sl]), np.array([0, L[b]]), h, ts[sl], wp, wt)
        assert_close(f"A[request {b}]", A[sl], ref, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hstu_explicit_scale_and_large_biases(gpu, dtype):
    """A scale other than 1/sqrt(d_h) (the kernel folds -log2(e) scale into
    Q once) and bias tables twenty times larger (the position bias starts
    the score accumulators; far tiles read the time table with the last
    position entry folded in): ragged lengths across far, interior and edge
    tiles, including the position table's last entry."""
    L, d, h = [700, 65, 300], 128, 2
    q, k, v, off, ts, wp, wt = _inputs(13, L, d, dtype, 200, 24)
    wp, wt = 20.0 * wp, 20.0 * wt
    A = _run(gpu, q, k, v, off, ts, wp, wt, h, dtype, scale=0.37)
    ref = O.hstu_attn_fwd(q, k, v, off, h, ts, wp, wt, scale=0.37)
    assert_close("A", A, ref, dtype)
