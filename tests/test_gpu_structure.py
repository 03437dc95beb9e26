"""Structural GPU checks that hold bit for bit: jagged indexing and masking,
empty and single-row histories, saturated softmax, independence of requests
and of candidates, memory past the history never read, determinism of every
output, and replay of the forward captured in a HIP graph."""
import numpy as np
import pytest
import torch

from candidate_conditioned_sequence_amd import binding as wb
from candidate_conditioned_sequence_amd import synth
from candidate_conditioned_sequence_amd.layer import FusionLayer
from tests.util import i64_dev, to_dev

pytestmark = pytest.mark.gpu


def _draw(seed, shape, dtype):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if dtype == "bf16" else x


def _fwd(gpu, dtype, Q, K, V, L, C, n_q, h, extra_rows=0, poison=None):
    off = synth.offsets_of(L)
    T = int(off[-1])
    d = Q.shape[1]
    tK = torch.empty((T + extra_rows, d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=gpu)
    tV = torch.empty_like(tK)
    if extra_rows:
        tK[T:] = poison
        tV[T:] = poison
    tK[:T] = to_dev(K, dtype, gpu)
    tV[:T] = to_dev(V, dtype, gpu)
    tQ = to_dev(Q, dtype, gpu)
    A = torch.full_like(tQ, float("nan"))
    lse = torch.full((Q.shape[0], h), float("nan"), device=gpu)
    wb.whale_jagged_xattn_fwd(wb.dims(len(L), C, n_q, d, h, max(L), T), tQ, tK, tV, i64_dev(off, gpu), 0.0, A, lse)
    torch.cuda.synchronize()
    return A.cpu(), lse.cpu()


@pytest.mark.parametrize("dtype,d,h,C,n_q", [("bf16", 256, 4, 3, 5), ("f32", 64, 2, 3, 5), ("bf16", 128, 4, 3, 5),
                                             ("bf16", 256, 4, 40, 30)])
def test_single_key_returns_value_row_bitwise(gpu, dtype, d, h, C, n_q):
    L = [1, 1, 0, 1]
    M = len(L) * C * n_q
    Q, K, V = _draw(1, (M, d), dtype), _draw(2, (3, d), dtype), _draw(3, (3, d), dtype)
    A, lse = _fwd(gpu, dtype, Q, K, V, L, C, n_q, h)
    per = C * n_q
    rows = {0: 0, 1: 1, 3: 2}
    for b, t in rows.items():
        ref = torch.from_numpy(np.repeat(V[t:t + 1], per, 0)).to(A.dtype)
        assert torch.equal(A[b * per:(b + 1) * per], ref)
    assert torch.all(A[2 * per:3 * per] == 0) and torch.all(torch.isneginf(lse[2 * per:3 * per]))


@pytest.mark.parametrize("hot,C,n_q", [(0, 4, 8), (63, 4, 8), (64, 4, 8), (700, 4, 8), (1299, 4, 8),
                                       (0, 32, 32), (64, 32, 32), (1299, 32, 32)])
def test_one_hot_saturated_picks_exact_row(gpu, hot, C, n_q):
    # Score gap of 512 natural-log units: every other weight underflows to 0,
    # in any history tile.  V rows hold small integers (exact in bf16) naming
    # the row, so the exact value proves the indexing.
    dtype, d, h, L = "bf16", 128, 2, [1300]
    M = C * n_q
    Q = np.zeros((M, d), np.float32)
    Q[:, 0] = 64.0
    Q[:, 64] = 64.0
    K = synth.round_bf16(0.01 * _draw(5, (L[0], d), "f32"))
    K[hot, 0] = 64.0
    K[hot, 64] = 64.0
    V = np.zeros((L[0], d), np.float32)
    V[:, :] = (np.arange(L[0])[:, None] % 97) + (np.arange(d)[None, :] % 7)
    A, _ = _fwd(gpu, dtype, Q, K, V, L, C, n_q, h)
    assert torch.equal(A.float(), torch.from_numpy(np.repeat(V[hot:hot + 1], M, 0)))


@pytest.mark.parametrize("C,n_q", [(5, 7), (40, 30)])
def test_memory_past_the_history_is_never_read(gpu, C, n_q):
    dtype, d, h, L = "bf16", 256, 4, [77, 0, 130]
    M = len(L) * C * n_q
    Q, K, V = _draw(7, (M, d), dtype), _draw(8, (sum(L), d), dtype), _draw(9, (sum(L), d), dtype)
    A0, l0 = _fwd(gpu, dtype, Q, K, V, L, C, n_q, h)
    A1, l1 = _fwd(gpu, dtype, Q, K, V, L, C, n_q, h, extra_rows=300, poison=float("nan"))
    assert torch.isfinite(A1).all()
    assert torch.equal(A0, A1) and torch.equal(l0, l1)


def test_requests_and_candidates_are_independent_bitwise(gpu):
    dtype, d, h, C, n_q = "bf16", 256, 4, 64, 32
    L = [900, 333, 64]
    off = synth.offsets_of(L)
    M = len(L) * C * n_q
    Q, K, V = _draw(11, (M, d), dtype), _draw(12, (sum(L), d), dtype), _draw(13, (sum(L), d), dtype)
    A, lse = _fwd(gpu, dtype, Q, K, V, L, C, n_q, h)
    # change request 1 entirely: request 0 and 2 must not move by one bit
    K2, V2 = K.copy(), V.copy()
    K2[off[1]:off[2]] = _draw(14, (L[1], d), dtype)
    V2[off[1]:off[2]] = _draw(15, (L[1], d), dtype)
    A2, _ = _fwd(gpu, dtype, Q, K2, V2, L, C, n_q, h)
    per = C * n_q
    assert torch.equal(A[:per], A2[:per]) and torch.equal(A[2 * per:], A2[2 * per:])
    assert not torch.equal(A[per:2 * per], A2[per:2 * per])
    # each candidate alone (C = 1) against the same shared K/V: same bits
    for c in (0, 17, 63):
        rows = slice((0 * C + c) * n_q, (0 * C + c + 1) * n_q)
        A1, _ = _fwd(gpu, dtype, Q[rows], K[:L[0]], V[:L[0]], [L[0]], 1, n_q, h)
        assert torch.equal(A1, A[rows])


def _layer_case(gpu, key="c5", B=3):
    cfg = synth.scaled(synth.CONFIGS[key], B=B, lengths=("list", [700, 1, 257][:B]))
    L = synth.lengths(cfg)
    H_w, H_s, off = synth.inputs(cfg)
    p = synth.layer_params(cfg, random_affine=True)
    tp = {k: (torch.from_numpy(v).to(gpu).to(torch.bfloat16) if k.startswith("W_") else torch.from_numpy(v).to(gpu))
          for k, v in p.items()}
    x = (torch.from_numpy(H_w).to(gpu).to(torch.bfloat16), torch.from_numpy(H_s).to(gpu).to(torch.bfloat16),
         torch.from_numpy(off).to(gpu), int(L.max()))
    dY = torch.from_numpy(np.concatenate([synth.dy_rows(cfg, b) for b in range(cfg.B)])).to(gpu).to(torch.bfloat16)
    return cfg, tp, x, dY


def test_forward_and_backward_are_deterministic(gpu):
    cfg, tp, x, dY = _layer_case(gpu)
    results = []
    for _ in range(3):
        lay = FusionLayer(tp, cfg.C, cfg.n_q, cfg.h)
        out = lay.forward(*x)
        g = lay.backward(dY)
        torch.cuda.synchronize()
        results.append({**{k: v.clone() for k, v in out.items() if isinstance(v, torch.Tensor)},
                        **{k: v.clone() for k, v in g.items()}})
    for k in results[0]:
        for r in results[1:]:
            assert torch.equal(results[0][k], r[k]), k


def test_forward_replays_from_a_captured_graph(gpu):
    cfg, tp, x, _ = _layer_case(gpu)
    lay = FusionLayer(tp, cfg.C, cfg.n_q, cfg.h)
    eager = lay.forward(*x, save=False)["Y"].clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lay.forward(*x, save=False)   # warm the allocator on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = lay.forward(*x, save=False)["Y"]
    for i in range(4):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {i}"
        _ = (x[0].float() * 2).sum()      # unrelated eager work between replays
        torch.cuda.synchronize()


def test_mfma_probe_does_the_products_it_counts(gpu):
    """The matrix-core probe's per-wave output sums to 4 * iters * sum(A B),
    with A and B the register operands it builds: its FLOP count is real."""
    blocks, iters = 3, 7
    out = torch.empty(blocks * 256, dtype=torch.float32, device=gpu)
    wb.whale_mfma_peak_probe(out, iters, blocks)
    torch.cuda.synchronize()
    lane = np.arange(64)
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for u in range(8):
        # the kernel's fp32 product 1e-3f * x, rounded to bf16
        a = synth.round_bf16(np.float32(1e-3) * (lane + u).astype(np.float32)).astype(np.float64)
        b = synth.round_bf16(np.float32(1e-3) * (lane - u).astype(np.float32)).astype(np.float64)
        A[lane % 32, 8 * (lane // 32) + u] = a
        Bm[8 * (lane // 32) + u, lane % 32] = b
    want = 4 * iters * (A @ Bm).sum()
    got = out.double().cpu().numpy().reshape(-1, 64).sum(1)
    np.testing.assert_allclose(got, want, rtol=1e-4)
