"""GPU parity of every C-ABI call against the fp64 oracle, element by element,
at sizes the oracle finishes in seconds that still span several tiles and a
ragged tail (history lengths 0, 1, 63, 64, 65, 257, ...; query blocks with a
partial last block).  Tolerance: relative Frobenius error <= 1e-5 (fp32) and
<= 2e-2 (bf16), max-abs error printed."""
import numpy as np
import pytest
import torch

from candidate_conditioned_sequence_amd import binding as wb
from candidate_conditioned_sequence_amd import synth
from oracle import whale_oracle as O
from tests.util import assert_close, f32_dev, host, i64_dev, to_dev

pytestmark = pytest.mark.gpu


def draw(seed, shape, dtype, scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * scale
    return synth.round_bf16(x) if dtype == "bf16" else x


def weights(seed, out_f, in_f, dtype):
    a = np.sqrt(6.0 / (in_f + out_f))
    w = np.random.default_rng(seed).uniform(-a, a, (out_f, in_f)).astype(np.float32)
    return synth.round_bf16(w) if dtype == "bf16" else w


def offsets(lengths):
    return synth.offsets_of(lengths)


XATTN_CASES = [
    # dtype, d, h, C, n_q, lengths
    ("f32", 64, 2, 4, 8, [256]),
    ("f32", 128, 2, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 128, 4, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 256, 4, 20, 15, [130, 1, 700, 64]),
    ("bf16", 256, 4, 64, 32, [1000, 333]),
    ("bf16", 512, 8, 8, 16, [97, 640]),
    ("f32", 128, 2, 40, 8, [300, 5]),
    # C*n_q >= 1024 with d_h = 64: the 8-wave ping-pong kernel (partial last
    # query block, every ragged length class)
    ("bf16", 256, 4, 40, 30, [0, 1, 63, 64, 65, 257, 130]),
    ("bf16", 512, 8, 32, 32, [700, 1]),
    # d_h = 128 (d = 256, h = 2 and d = 512, h = 4): the general kernel with
    # one key block of K operands at a time
    ("f32", 256, 2, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 256, 2, 20, 15, [130, 1, 700, 64]),
    ("bf16", 512, 4, 8, 16, [97, 640]),
    ("f32", 512, 4, 4, 8, [300, 5]),
    ("bf16", 256, 2, 40, 30, [1000, 65, 0]),
]


@pytest.mark.parametrize("case", XATTN_CASES, ids=lambda c: f"{c[0]}-d{c[1]}h{c[2]}-C{c[3]}nq{c[4]}-L{c[5]}")
def test_xattn_fwd(gpu, case):
    dtype, d, h, C, n_q, L = case
    print(f"\n[xattn_fwd] {case}", flush=True)
    B = len(L)
    M, off = B * C * n_q, offsets(L)
    T = int(off[-1])
    Q, K, V = draw(1, (M, d), dtype), draw(2, (T, d), dtype), draw(3, (T, d), dtype)
    A_ref, lse_ref = O.xattn_fwd(Q, K, V, off, C, n_q, h)
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tQ, tK, tV = to_dev(Q, dtype, gpu), to_dev(K, dtype, gpu), to_dev(V, dtype, gpu)
    A = torch.full_like(tQ, float("nan"))
    lse = torch.full((M, h), float("nan"), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, tQ, tK, tV, i64_dev(off, gpu), 0.0, A, lse)
    torch.cuda.synchronize()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(host(lse)), fin), "empty-history rows must give lse = -inf exactly"
    assert np.all(host(lse)[~fin] == -np.inf)
    assert_close("A", A, A_ref, dtype)
    got = host(lse)
    assert_close("lse", got[fin], lse_ref[fin], dtype, factor=0.1)


# bf16 at d = 256 runs the row-streaming kernels (32-row blocks, one
# workgroup per CU); the long histories give workgroups several blocks each,
# so the transfers run two blocks ahead, and leave a ragged last block.
PROJ_L = [0, 200, 77]
PROJ_LONG = [9000, 17000, 5, 31]
PROJ_CASES = [
    ("f32", O.NORM_LAYER, False, 128, PROJ_L), ("bf16", O.NORM_LAYER, False, 128, PROJ_L),
    ("bf16", O.NORM_RMS, False, 128, PROJ_L), ("f32", O.NORM_NONE, False, 128, PROJ_L),
    ("f32", O.NORM_LAYER, True, 128, PROJ_L), ("bf16", O.NORM_LAYER, True, 128, PROJ_L),
    ("bf16", O.NORM_RMS, True, 128, PROJ_L),
    ("bf16", O.NORM_LAYER, True, 256, PROJ_L), ("bf16", O.NORM_LAYER, False, 256, PROJ_L),
    ("bf16", O.NORM_RMS, True, 256, PROJ_L), ("bf16", O.NORM_NONE, False, 256, PROJ_L),
    ("bf16", O.NORM_LAYER, True, 256, PROJ_LONG), ("bf16", O.NORM_RMS, False, 256, [1, 33, 64]),
    # d = 512: the row-streaming kernels in column groups of 256 (K = 512
    # rows as two panels; 2 groups for Q, 4 for K and V)
    ("bf16", O.NORM_LAYER, True, 512, PROJ_L), ("bf16", O.NORM_RMS, False, 512, PROJ_LONG),
    ("bf16", O.NORM_NONE, False, 512, [1, 33, 64]),
]


@pytest.mark.parametrize("dtype,norm,keep,d,L", PROJ_CASES,
                         ids=lambda v: str(len(v)) if isinstance(v, list) else str(v))
def test_proj_qkv(gpu, dtype, norm, keep, d, L):
    """keep: the normalised inputs are written out once (X_q, X_s) and the
    projections read them; otherwise the projections normalise per tile."""
    print(f"\n[proj_qkv] {dtype} norm={norm} keep={keep} d={d} L={L}", flush=True)
    B, C, n_q, h = len(L), 5, 7, d // 64
    M, off = B * C * n_q, offsets(L)
    T = int(off[-1])
    Hw, Hs = draw(4, (M, d), dtype, 2.0) + 0.5, draw(5, (T, d), dtype)
    Wq, Wk, Wv = (weights(s, d, d, dtype) for s in (6, 7, 8))
    g = 1 + 0.2 * draw(9, (2, d), "f32")
    bt = 0.2 * draw(10, (2, d), "f32")
    Qr, Kr, Vr = O.proj_qkv(Hw, Hs, norm, 1e-5, g[0], bt[0], g[1], bt[1], Wq, Wk, Wv)
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    Q, K, V = (torch.empty((n, d), dtype=to_dev(Hw[:1], dtype, gpu).dtype, device=gpu) for n in (M, T, T))
    sq, skv = torch.empty((M, 2), device=gpu), torch.empty((T, 2), device=gpu)
    Xq, Xs = (torch.empty_like(Q), torch.empty_like(K)) if keep else (None, None)
    wb.whale_proj_qkv(dm, to_dev(Hw, dtype, gpu), to_dev(Hs, dtype, gpu), norm, 1e-5, f32_dev(g[0], gpu),
                      f32_dev(bt[0], gpu), f32_dev(g[1], gpu), f32_dev(bt[1], gpu), to_dev(Wq, dtype, gpu),
                      to_dev(Wk, dtype, gpu), to_dev(Wv, dtype, gpu), Q, K, V, sq, skv, Xq, Xs)
    torch.cuda.synchronize()
    for name, got, ref in (("Q", Q, Qr), ("K", K, Kr), ("V", V, Vr)):
        assert_close(name, got, ref, dtype)
    if keep:
        assert_close("X_q", Xq, O.norm_fwd(Hw, norm, g[0], bt[0], 1e-5)[0], dtype)
        assert_close("X_s", Xs, O.norm_fwd(Hs, norm, g[1], bt[1], 1e-5)[0], dtype)
    if norm != O.NORM_NONE:
        # (statistics of the rows as the device holds them: H_w + 0.5 is
        # rounded to bf16 again on upload)
        for name, got, x in (("stats_q", sq, Hw), ("stats_kv", skv, Hs)):
            x = (synth.round_bf16(x) if dtype == "bf16" else x).astype(np.float64)
            mean = x.mean(1) if norm == O.NORM_LAYER else np.zeros(len(x))
            var = ((x - mean[:, None]) ** 2).mean(1)
            want = np.stack([mean, 1 / np.sqrt(var + 1e-5)], 1)
            assert_close(name, got, want, "f32")


# bf16 with SiLU at d = 256: the row-streaming kernel (M = 9001: several
# 32-row blocks per workgroup and a ragged one; keepz False: Z not saved).
@pytest.mark.parametrize("dtype,act,M,keepz", [("f32", O.ACT_SILU, 300, True), ("bf16", O.ACT_SILU, 300, True),
                                               ("bf16", O.ACT_NONE, 300, True), ("bf16", O.ACT_SILU, 9001, True),
                                               ("bf16", O.ACT_SILU, 77, False)])
def test_fusion_mlp(gpu, dtype, act, M, keepz):
    print(f"\n[fusion_mlp] {dtype} act={act} M={M} keepz={keepz}", flush=True)
    d = 256
    A, Hw = draw(11, (M, d), dtype), draw(12, (M, d), dtype)
    Wf = weights(13, d, 2 * d, dtype)
    F_ref, Z_ref = O.fusion_mlp(A, Hw, Wf, act)
    dm = wb.dims(1, M, 1, d, 4, 0, 0)
    tA = to_dev(A, dtype, gpu)
    F, Z = torch.empty_like(tA), torch.empty_like(tA)
    wb.whale_fusion_mlp(dm, tA, to_dev(Hw, dtype, gpu), to_dev(Wf, dtype, gpu), act, F, Z if keepz else None)
    torch.cuda.synchronize()
    assert_close("F", F, F_ref, dtype)
    if act == O.ACT_SILU and keepz:
        assert_close("Z", Z, Z_ref, dtype)


# bf16, shared gate, d = 256 and H a multiple of 512: the up projection runs
# in the row-streaming kernel (column groups of 512; M = 9001 gives its
# workgroups several 32-row blocks and a ragged last one).  d = 512 runs the
# tiled path.
@pytest.mark.parametrize("dtype,gate,norm,d,M,H", [("f32", O.GATE_SHARED, O.NORM_LAYER, 128, 200, 512),
                                                   ("bf16", O.GATE_SHARED, O.NORM_LAYER, 256, 200, 1024),
                                                   ("bf16", O.GATE_SEPARATE, O.NORM_RMS, 128, 200, 512),
                                                   ("f32", O.GATE_SEPARATE, O.NORM_NONE, 64, 200, 256),
                                                   ("bf16", O.GATE_SHARED, O.NORM_RMS, 256, 9001, 1024),
                                                   ("bf16", O.GATE_SHARED, O.NORM_NONE, 256, 333, 512),
                                                   ("bf16", O.GATE_SHARED, O.NORM_LAYER, 256, 77, 2048),
                                                   ("bf16", O.GATE_SHARED, O.NORM_LAYER, 256, 333, -1024),
                                                   ("bf16", O.GATE_SHARED, O.NORM_LAYER, 512, 9001, 2048),
                                                   ("bf16", O.GATE_SHARED, O.NORM_NONE, 512, 333, -1024)])
def test_swiglu_ffn(gpu, dtype, gate, norm, d, M, H):
    """H < 0: the same with |H| and U not kept (the product goes to the workspace)."""
    keepu = H > 0
    H = abs(H)
    print(f"\n[swiglu_ffn] {dtype} gate={gate} norm={norm} d={d} M={M} H={H} keepu={keepu}", flush=True)
    Fm = draw(14, (M, d), dtype)
    Wu = weights(15, (2 if gate == O.GATE_SEPARATE else 1) * H, d, dtype)
    Wd = weights(16, d, H, dtype)
    g, bt = 1 + 0.2 * draw(17, (d,), "f32"), 0.2 * draw(18, (d,), "f32")
    Y_ref, U_ref = O.swiglu_ffn(Fm, norm, 1e-5, g, bt, Wu, gate, Wd)
    dm = wb.dims(1, M, 1, d, d // 64 if d >= 64 else 1, 0, 0)
    tF = to_dev(Fm, dtype, gpu)
    Y = torch.empty_like(tF)
    U = torch.empty((M, Wu.shape[0]), dtype=tF.dtype, device=gpu)
    sf = torch.empty((M, 2), device=gpu)
    ws = torch.empty(wb.whale_swiglu_ffn_workspace_size(dm, wb._dtype_code(tF), gate, H), dtype=torch.uint8,
                     device=gpu)
    wb.whale_swiglu_ffn(dm, tF, norm, 1e-5, f32_dev(g, gpu), f32_dev(bt, gpu), to_dev(Wu, dtype, gpu), gate, H,
                        to_dev(Wd, dtype, gpu), Y, U if keepu else None, sf, ws)
    torch.cuda.synchronize()
    assert_close("Y", Y, Y_ref, dtype)
    if keepu:
        assert_close("U", U, U_ref, dtype)
    if norm != O.NORM_NONE:
        x = Fm.astype(np.float64)
        mean = x.mean(1) if norm == O.NORM_LAYER else np.zeros(M)
        want = np.stack([mean, 1 / np.sqrt(((x - mean[:, None]) ** 2).mean(1) + 1e-5)], 1)
        assert_close("stats_f", sf, want, "f32")


BWD_CASES = [
    ("f32", 64, 2, 4, 8, [256]),
    ("f32", 128, 2, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 128, 4, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 256, 4, 20, 15, [130, 1, 700, 64]),
    ("bf16", 256, 4, 64, 32, [900, 333]),
    # d_h = 128
    ("f32", 256, 2, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 256, 2, 20, 15, [130, 1, 700, 64]),
    ("bf16", 512, 4, 8, 16, [97, 640]),
    ("bf16", 256, 2, 64, 32, [900, 333]),
    ("f32", 512, 4, 4, 8, [300, 5]),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"{c[0]}-d{c[1]}h{c[2]}-C{c[3]}nq{c[4]}-L{c[5]}")
def test_xattn_bwd(gpu, case):
    dtype, d, h, C, n_q, L = case
    print(f"\n[xattn_bwd] {case}", flush=True)
    B = len(L)
    M, off = B * C * n_q, offsets(L)
    T = int(off[-1])
    Q, K, V, dA = draw(21, (M, d), dtype), draw(22, (T, d), dtype), draw(23, (T, d), dtype), draw(24, (M, d), dtype)
    dQ_ref, dK_ref, dV_ref = O.xattn_bwd(Q, K, V, off, C, n_q, h, None, dA)
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tQ, tK, tV, tdA = (to_dev(x, dtype, gpu) for x in (Q, K, V, dA))
    toff = i64_dev(off, gpu)
    A, lse = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, tQ, tK, tV, toff, 0.0, A, lse)
    dQ, dK, dV = torch.empty_like(tQ), torch.empty_like(tK), torch.empty_like(tV)
    ws = torch.empty(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb._dtype_code(tQ)), dtype=torch.uint8, device=gpu)
    wb.whale_jagged_xattn_bwd(dm, tQ, tK, tV, toff, 0.0, A, lse, tdA, dQ, dK, dV, ws)
    torch.cuda.synchronize()
    assert_close("dQ", dQ, dQ_ref, dtype)
    assert_close("dK", dK, dK_ref, dtype)
    assert_close("dV", dV, dV_ref, dtype)


# Shared key-value form: V is K, and the backward returns one gradient dK + dV.
# The first three cases run split query ranges with fp32 partials (ragged and
# empty histories among them); the last has enough history tiles for no split.
SHARED_KV_CASES = [
    ("f32", 128, 2, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 128, 4, 3, 5, [0, 1, 63, 64, 65, 257]),
    ("bf16", 256, 4, 20, 15, [130, 1, 700, 64]),
    ("bf16", 256, 4, 16, 32, [2100, 2050, 1999, 2100, 7, 2100, 1500, 2048]),
    ("bf16", 256, 2, 20, 15, [130, 1, 700, 64]),
]


@pytest.mark.parametrize("case", SHARED_KV_CASES, ids=lambda c: f"{c[0]}-d{c[1]}h{c[2]}-C{c[3]}nq{c[4]}-B{len(c[5])}")
def test_xattn_shared_kv(gpu, case):
    dtype, d, h, C, n_q, L = case
    print(f"\n[xattn shared kv] {case}", flush=True)
    B = len(L)
    M, off = B * C * n_q, offsets(L)
    T = int(off[-1])
    Q, K, dA = draw(71, (M, d), dtype), draw(72, (T, d), dtype), draw(73, (M, d), dtype)
    A_ref, _ = O.xattn_fwd(Q, K, K, off, C, n_q, h)
    dQ_ref, dK_ref, dV_ref = O.xattn_bwd(Q, K, K, off, C, n_q, h, None, dA)
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tQ, tK, tdA = (to_dev(x, dtype, gpu) for x in (Q, K, dA))
    toff = i64_dev(off, gpu)
    A, lse = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, tQ, tK, tK, toff, 0.0, A, lse)
    dQ, dK = torch.empty_like(tQ), torch.empty_like(tK)
    ws = torch.empty(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb._dtype_code(tQ)), dtype=torch.uint8, device=gpu)
    wb.whale_jagged_xattn_bwd(dm, tQ, tK, tK, toff, 0.0, A, lse, tdA, dQ, dK, None, ws)
    torch.cuda.synchronize()
    assert_close("A", A, A_ref, dtype)
    assert_close("dQ", dQ, dQ_ref, dtype)
    assert_close("dK+dV", dK, dK_ref + dV_ref, dtype)


# bf16 with SiLU at d = 256: the row-streaming kernel (dZ, dA and dH_w in one
# pass; M = 9001 gives several 32-row blocks per workgroup and a ragged one).
@pytest.mark.parametrize("dtype,act,M,d", [("f32", O.ACT_SILU, 300, 128), ("bf16", O.ACT_SILU, 300, 128),
                                           ("bf16", O.ACT_NONE, 300, 128), ("bf16", O.ACT_SILU, 9001, 256),
                                           ("bf16", O.ACT_SILU, 77, 256), ("bf16", O.ACT_NONE, 300, 256)])
def test_fusion_mlp_bwd(gpu, dtype, act, M, d):
    print(f"\n[fusion_mlp_bwd] {dtype} act={act} M={M} d={d}", flush=True)
    A, Hw, dF = draw(31, (M, d), dtype), draw(32, (M, d), dtype), draw(33, (M, d), dtype)
    Wf = weights(34, d, 2 * d, dtype)
    dA_ref, dHw_ref, dWf_ref = O.fusion_mlp_bwd(A, Hw, Wf, act, dF)
    _, Z = O.fusion_mlp(A, Hw, Wf, act)
    dm = wb.dims(1, M, 1, d, d // 64, 0, 0)
    tA, tHw, tWf = to_dev(A, dtype, gpu), to_dev(Hw, dtype, gpu), to_dev(Wf, dtype, gpu)
    F, tZ = torch.empty_like(tA), torch.empty_like(tA)
    wb.whale_fusion_mlp(dm, tA, tHw, tWf, act, F, tZ if act == O.ACT_SILU else None)
    dA, dHw = torch.empty_like(tA), torch.empty_like(tA)
    dWf = torch.empty((d, 2 * d), device=gpu)
    ws = torch.empty(wb.whale_fusion_mlp_bwd_workspace_size(dm, wb._dtype_code(tA)), dtype=torch.uint8, device=gpu)
    wb.whale_fusion_mlp_bwd(dm, tA, tHw, tWf, act, tZ if act == O.ACT_SILU else None, to_dev(dF, dtype, gpu), dA,
                            dHw, dWf, ws)
    torch.cuda.synchronize()
    assert_close("dA", dA, dA_ref, dtype)
    assert_close("dH_w", dHw, dHw_ref, dtype)
    assert_close("dW_F", dWf, dWf_ref, dtype)


# bf16, shared gate, d = 256: the gate backward runs in the row-streaming
# kernel (M = 9001: several 32-row blocks per workgroup and a ragged one).
# keep: the forward writes X_f = Norm_f(F) and the backward reads it.
@pytest.mark.parametrize("dtype,gate,norm,d,M,H,keep", [
    ("f32", O.GATE_SHARED, O.NORM_LAYER, 128, 300, 512, False), ("bf16", O.GATE_SHARED, O.NORM_LAYER, 256, 300, 1024, False),
    ("bf16", O.GATE_SEPARATE, O.NORM_RMS, 128, 300, 512, True), ("f32", O.GATE_SEPARATE, O.NORM_NONE, 64, 300, 256, False),
    ("bf16", O.GATE_SHARED, O.NORM_LAYER, 512, 300, 2048, False), ("bf16", O.GATE_SHARED, O.NORM_RMS, 256, 9001, 1024, True),
    ("bf16", O.GATE_SHARED, O.NORM_NONE, 256, 77, 512, True), ("bf16", O.GATE_SHARED, O.NORM_LAYER, 256, 300, 1024, True),
    ("f32", O.GATE_SHARED, O.NORM_LAYER, 128, 300, 512, True)])
def test_swiglu_ffn_bwd(gpu, dtype, gate, norm, d, M, H, keep):
    print(f"\n[swiglu_ffn_bwd] {dtype} gate={gate} norm={norm} d={d} M={M} H={H} keep={keep}", flush=True)
    Fm, dY = draw(41, (M, d), dtype), draw(42, (M, d), dtype)
    Wu = weights(43, (2 if gate == O.GATE_SEPARATE else 1) * H, d, dtype)
    Wd = weights(44, d, H, dtype)
    g, bt = 1 + 0.2 * draw(45, (d,), "f32"), 0.2 * draw(46, (d,), "f32")
    ref = O.swiglu_ffn_bwd(Fm, norm, 1e-5, g, bt, Wu, gate, Wd, dY)
    dm = wb.dims(1, M, 1, d, d // 64, 0, 0)
    tF, tWu, tWd = to_dev(Fm, dtype, gpu), to_dev(Wu, dtype, gpu), to_dev(Wd, dtype, gpu)
    tg, tb = f32_dev(g, gpu), f32_dev(bt, gpu)
    Y, U = torch.empty_like(tF), torch.empty((M, Wu.shape[0]), dtype=tF.dtype, device=gpu)
    sf = torch.empty((M, 2), device=gpu)
    code = wb._dtype_code(tF)
    ws = torch.empty(wb.whale_swiglu_ffn_workspace_size(dm, code, gate, H), dtype=torch.uint8, device=gpu)
    Xf = torch.empty_like(tF) if keep else None
    wb.whale_swiglu_ffn(dm, tF, norm, 1e-5, tg, tb, tWu, gate, H, tWd, Y, U, sf, ws, X_f=Xf)
    if keep and norm != O.NORM_NONE:
        assert_close("X_f", Xf, O.norm_fwd(Fm, norm, g, bt, 1e-5)[0], dtype)
    dF = torch.empty_like(tF)
    dWu, dWd = torch.empty(tuple(Wu.shape), device=gpu), torch.empty(tuple(Wd.shape), device=gpu)
    dg, db = torch.empty(d, device=gpu), torch.empty(d, device=gpu)
    ws = torch.empty(wb.whale_swiglu_ffn_bwd_workspace_size(dm, code, gate, H), dtype=torch.uint8, device=gpu)
    wb.whale_swiglu_ffn_bwd(dm, tF, norm, 1e-5, tg, tb, sf, tWu, gate, H, tWd, U, to_dev(dY, dtype, gpu), dF, dWu,
                            dWd, dg, db, ws, X_f=Xf)
    torch.cuda.synchronize()
    assert_close("dF", dF, ref["dF"], dtype)
    assert_close("dW_U", dWu, ref["dW_U"], dtype)
    assert_close("dW_D", dWd, ref["dW_D"], dtype)
    if norm != O.NORM_NONE:
        assert_close("dg_f", dg, ref["dg_f"], dtype)
    if norm == O.NORM_LAYER:
        assert_close("db_f", db, ref["db_f"], dtype)


@pytest.mark.parametrize("dtype,norm,d,keep,L", [
    ("f32", O.NORM_LAYER, 128, False, PROJ_L), ("bf16", O.NORM_LAYER, 128, False, PROJ_L),
    ("bf16", O.NORM_RMS, 256, False, PROJ_L), ("f32", O.NORM_LAYER, 64, False, PROJ_L),
    ("bf16", O.NORM_LAYER, 512, False, PROJ_L), ("f32", O.NORM_NONE, 128, False, PROJ_L),
    ("bf16", O.NORM_LAYER, 256, True, PROJ_L), ("f32", O.NORM_RMS, 128, True, PROJ_L),
    ("bf16", O.NORM_NONE, 256, False, PROJ_L), ("bf16", O.NORM_LAYER, 256, True, PROJ_LONG),
    ("bf16", O.NORM_RMS, 256, True, [1, 33, 64])], ids=lambda v: str(len(v)) if isinstance(v, list) else str(v))
def test_proj_qkv_bwd(gpu, dtype, norm, d, keep, L):
    """keep: the forward's normalised inputs are handed to the backward."""
    print(f"\n[proj_qkv_bwd] {dtype} norm={norm} d={d} keep={keep} L={L}", flush=True)
    B, C, n_q = len(L), 5, 7
    h = d // 64
    M, off = B * C * n_q, offsets(L)
    T = int(off[-1])
    Hw, Hs = draw(51, (M, d), dtype), draw(52, (T, d), dtype)
    Wq, Wk, Wv = (weights(s, d, d, dtype) for s in (53, 54, 55))
    dQ, dK, dV, extra = draw(56, (M, d), dtype), draw(57, (T, d), dtype), draw(58, (T, d), dtype), \
        draw(59, (M, d), dtype)
    g = 1 + 0.2 * draw(60, (2, d), "f32")
    bt = 0.2 * draw(61, (2, d), "f32")
    ref = O.proj_qkv_bwd(Hw, Hs, norm, 1e-5, g[0], bt[0], g[1], bt[1], Wq, Wk, Wv, dQ, dK, dV)
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tHw, tHs = to_dev(Hw, dtype, gpu), to_dev(Hs, dtype, gpu)
    tW = [to_dev(w, dtype, gpu) for w in (Wq, Wk, Wv)]
    tg = [f32_dev(x, gpu) for x in (g[0], bt[0], g[1], bt[1])]
    Q, K, V = torch.empty_like(tHw), torch.empty_like(tHs), torch.empty_like(tHs)
    sq, skv = torch.empty((M, 2), device=gpu), torch.empty((T, 2), device=gpu)
    Xq, Xs = (torch.empty_like(tHw), torch.empty_like(tHs)) if keep else (None, None)
    wb.whale_proj_qkv(dm, tHw, tHs, norm, 1e-5, *tg, *tW, Q, K, V, sq, skv, Xq, Xs)
    dHw, dHs = torch.empty_like(tHw), torch.empty_like(tHs)
    dW = [torch.empty((d, d), device=gpu) for _ in range(3)]
    dgb = [torch.empty(d, device=gpu) for _ in range(4)]
    ws = torch.empty(wb.whale_proj_qkv_bwd_workspace_size(dm, wb._dtype_code(tHw)), dtype=torch.uint8, device=gpu)
    wb.whale_proj_qkv_bwd(dm, tHw, tHs, norm, 1e-5, *tg, sq, skv, *tW, to_dev(dQ, dtype, gpu),
                          to_dev(dK, dtype, gpu), to_dev(dV, dtype, gpu), to_dev(extra, dtype, gpu), dHw, dHs, *dW,
                          *dgb, ws, Xq, Xs)
    torch.cuda.synchronize()
    assert_close("dH_w", dHw, ref["dH_w"] + extra, dtype)
    assert_close("dH_s", dHs, ref["dH_s"], dtype)
    for name, got in zip(("dW_Q", "dW_K", "dW_V"), dW):
        assert_close(name, got, ref[name], dtype)
    if norm != O.NORM_NONE:
        assert_close("dg_q", dgb[0], ref["dg_q"], dtype)
        assert_close("dg_kv", dgb[2], ref["dg_kv"], dtype)
    if norm == O.NORM_LAYER:
        assert_close("db_q", dgb[1], ref["db_q"], dtype)
        assert_close("db_kv", dgb[3], ref["db_kv"], dtype)


@pytest.mark.parametrize("dtype,norm,d,L", [("f32", O.NORM_LAYER, 128, PROJ_L), ("bf16", O.NORM_RMS, 128, PROJ_L),
                                            ("bf16", O.NORM_LAYER, 256, PROJ_LONG),
                                            ("bf16", O.NORM_NONE, 256, PROJ_L), ("bf16", O.NORM_LAYER, 512, PROJ_L)],
                         ids=lambda v: str(len(v)) if isinstance(v, list) else str(v))
def test_proj_qkv_shared_kv(gpu, dtype, norm, d, L):
    """Shared key-value form: no W_V, no V; the backward takes one dK."""
    print(f"\n[proj_qkv shared kv] {dtype} norm={norm} d={d} L={L}", flush=True)
    B, C, n_q = len(L), 5, 7
    h = d // 64
    M, off = B * C * n_q, offsets(L)
    T = int(off[-1])
    Hw, Hs = draw(81, (M, d), dtype), draw(82, (T, d), dtype)
    Wq, Wk = weights(83, d, d, dtype), weights(84, d, d, dtype)
    dQ, dK = draw(85, (M, d), dtype), draw(86, (T, d), dtype)
    g = 1 + 0.2 * draw(87, (2, d), "f32")
    bt = 0.2 * draw(88, (2, d), "f32")
    Q_ref, K_ref, V_ref = O.proj_qkv(Hw, Hs, norm, 1e-5, g[0], bt[0], g[1], bt[1], Wq, Wk, None)
    assert V_ref is K_ref
    ref = O.proj_qkv_bwd(Hw, Hs, norm, 1e-5, g[0], bt[0], g[1], bt[1], Wq, Wk, None, dQ, dK, None)
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tHw, tHs = to_dev(Hw, dtype, gpu), to_dev(Hs, dtype, gpu)
    tWq, tWk = to_dev(Wq, dtype, gpu), to_dev(Wk, dtype, gpu)
    tg = [f32_dev(x, gpu) for x in (g[0], bt[0], g[1], bt[1])]
    Q, K = torch.empty_like(tHw), torch.empty_like(tHs)
    sq, skv = torch.empty((M, 2), device=gpu), torch.empty((T, 2), device=gpu)
    wb.whale_proj_qkv(dm, tHw, tHs, norm, 1e-5, *tg, tWq, tWk, None, Q, K, None, sq, skv, None, None)
    dHw, dHs = torch.empty_like(tHw), torch.empty_like(tHs)
    dWq, dWk = torch.empty((d, d), device=gpu), torch.empty((d, d), device=gpu)
    dgb = [torch.empty(d, device=gpu) for _ in range(4)]
    ws = torch.empty(wb.whale_proj_qkv_bwd_workspace_size(dm, wb._dtype_code(tHw)), dtype=torch.uint8, device=gpu)
    wb.whale_proj_qkv_bwd(dm, tHw, tHs, norm, 1e-5, *tg, sq, skv, tWq, tWk, None, to_dev(dQ, dtype, gpu),
                          to_dev(dK, dtype, gpu), None, None, dHw, dHs, dWq, dWk, None, *dgb, ws)
    torch.cuda.synchronize()
    assert_close("Q", Q, Q_ref, dtype)
    assert_close("K", K, K_ref, dtype)
    assert_close("dH_w", dHw, ref["dH_w"], dtype)
    assert_close("dH_s", dHs, ref["dH_s"], dtype)
    assert_close("dW_Q", dWq, ref["dW_Q"], dtype)
    assert_close("dW_K", dWk, ref["dW_K"], dtype)
    if norm != O.NORM_NONE:
        assert_close("dg_kv", dgb[2], ref["dg_kv"], dtype)
    if norm == O.NORM_LAYER:
        assert_close("db_kv", dgb[3], ref["db_kv"], dtype)


# Serving form: a different number of candidates per request (zero included).
# The first case runs the ping-pong kernel (largest C_b * n_q >= 1024) with
# requests whose query count is not a multiple of its 512-query blocks; the
# others run the general kernel.
VARC_CASES = [
    ("bf16", 256, 4, 32, [64, 0, 17, 40, 1], [900, 50, 0, 1300, 257]),
    ("bf16", 128, 4, 16, [16, 3, 0, 9], [300, 1, 65, 0]),
    ("f32", 64, 2, 8, [3, 0, 5, 1], [100, 7, 0, 65]),
]


@pytest.mark.parametrize("case", VARC_CASES, ids=lambda c: f"{c[0]}-d{c[1]}h{c[2]}-nq{c[3]}-B{len(c[4])}")
def test_xattn_fwd_varc(gpu, case):
    dtype, d, h, n_q, C_b, L = case
    print(f"\n[xattn_fwd_varc] {case}", flush=True)
    B = len(L)
    coff, off = offsets(C_b), offsets(L)
    M, T = n_q * int(coff[-1]), int(off[-1])
    Q, K, V = draw(91, (M, d), dtype), draw(92, (T, d), dtype), draw(93, (T, d), dtype)
    A_ref, lse_ref = O.xattn_fwd(Q, K, V, off, None, n_q, h, cand_offsets=coff)
    dm = wb.dims(B, max(C_b), n_q, d, h, max(L), T)
    tQ, tK, tV = (to_dev(x, dtype, gpu) for x in (Q, K, V))
    A, lse = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    wb.whale_jagged_xattn_fwd_varc(dm, tQ, tK, tV, i64_dev(off, gpu), i64_dev(coff, gpu), 0.0, A, lse)
    torch.cuda.synchronize()
    assert_close("A", A, A_ref, dtype)
    fin = np.isfinite(lse_ref)
    got = host(lse)
    assert np.array_equal(np.isfinite(got), fin)
    assert_close("lse", got[fin], lse_ref[fin], "f32" if dtype == "f32" else "bf16")


def test_xattn_fwd_varc_equal_counts_match_fixed_call_bitwise(gpu):
    """With every C_b = C the serving form runs the same arithmetic as the
    fixed-count call: identical bits."""
    d, h, n_q, C, L = 256, 4, 32, 48, [700, 1, 333]
    B = len(L)
    off = offsets(L)
    M, T = B * C * n_q, int(off[-1])
    Q, K, V = draw(94, (M, d), "bf16"), draw(95, (T, d), "bf16"), draw(96, (T, d), "bf16")
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tQ, tK, tV = (to_dev(x, "bf16", gpu) for x in (Q, K, V))
    toff = i64_dev(off, gpu)
    A0, l0 = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    A1, l1 = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, tQ, tK, tV, toff, 0.0, A0, l0)
    wb.whale_jagged_xattn_fwd_varc(dm, tQ, tK, tV, toff, i64_dev(offsets([C] * B), gpu), 0.0, A1, l1)
    torch.cuda.synchronize()
    assert torch.equal(A0, A1) and torch.equal(l0, l1)


# The two schedules of the attention backward: the hybrid (Q-parallel dQ
# kernel + KV-parallel dK/dV kernel) and the KV-parallel one (one kernel forms
# dK, dV and dQ; dQ block partials summed in a fixed order when a history
# spans several 128-row blocks).  WHALE_XATTN_BWD_SCHEDULE forces one.  Both
# against the oracle; dK and dV bit for bit equal across the schedules (same
# accumulation code, same D).
KV_SCHED_CASES = [
    # dtype, d, h, C, n_q, lengths, tied
    ("bf16", 256, 4, 64, 32, [100, 128, 1, 0, 64], False),      # one block per history: the automatic choice
    ("bf16", 128, 4, 16, 16, [1000, 333, 129, 0], False),       # several blocks: dQ partials
    ("f32", 128, 2, 3, 5, [0, 1, 63, 64, 65, 257], False),      # query splits, partials
    ("bf16", 256, 2, 20, 15, [130, 1, 700, 64], False),         # d_h = 128
    ("bf16", 128, 4, 8, 16, [120, 5, 77], False),               # d_h = 32
    ("bf16", 256, 4, 16, 32, [100, 7, 0, 128], True),           # shared key-value form
]


@pytest.mark.parametrize("case", KV_SCHED_CASES, ids=lambda c: f"{c[0]}-d{c[1]}h{c[2]}-C{c[3]}nq{c[4]}-L{c[5]}-t{c[6]}")
def test_xattn_bwd_kv_schedule(gpu, case, monkeypatch):
    dtype, d, h, C, n_q, L, tied = case
    print(f"\n[xattn_bwd schedules] {case}", flush=True)
    B = len(L)
    M, off = B * C * n_q, offsets(L)
    T = int(off[-1])
    Q, K, dA = draw(81, (M, d), dtype), draw(82, (T, d), dtype), draw(84, (M, d), dtype)
    V = K if tied else draw(83, (T, d), dtype)
    dQ_ref, dK_ref, dV_ref = O.xattn_bwd(Q, K, V, off, C, n_q, h, None, dA)
    if tied:
        dK_ref, dV_ref = dK_ref + dV_ref, None
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tQ, tK, tdA = (to_dev(x, dtype, gpu) for x in (Q, K, dA))
    tV = tK if tied else to_dev(V, dtype, gpu)
    toff = i64_dev(off, gpu)
    A, lse = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, tQ, tK, tV, toff, 0.0, A, lse)
    res = {}
    for sched in ("q", "kv"):
        monkeypatch.setenv("WHALE_XATTN_BWD_SCHEDULE", sched)
        dQ, dK = torch.full_like(tQ, float("nan")), torch.full_like(tK, float("nan"))
        dV = None if tied else torch.full_like(tV, float("nan"))
        ws = torch.empty(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb._dtype_code(tQ)), dtype=torch.uint8,
                         device=gpu)
        wb.whale_jagged_xattn_bwd(dm, tQ, tK, tV, toff, 0.0, A, lse, tdA, dQ, dK, dV, ws)
        torch.cuda.synchronize()
        res[sched] = (dQ, dK, dV)
        print(f"  schedule {sched}:", flush=True)
        assert_close("dQ", dQ, dQ_ref, dtype)
        assert_close("dK", dK, dK_ref, dtype)
        if not tied:
            assert_close("dV", dV, dV_ref, dtype)
    assert torch.equal(res["q"][1], res["kv"][1])
    if not tied:
        assert torch.equal(res["q"][2], res["kv"][2])


# Jagged batches of up to 256 requests run longest history first (each
# workgroup ranks the requests; the dQ kernel leaves the order in the
# workspace for the dK/dV kernel); larger batches keep the index order.
# Both sides of the bound, with the ping-pong forward (C n_q = 1024) and the
# Q-parallel backward, checked on sampled requests (each request's outputs
# depend on its own rows only): the longest, an empty one, short ones.
@pytest.mark.parametrize("B", [256, 257])
def test_xattn_many_jagged_requests(gpu, B):
    dtype, d, h, C, n_q = "bf16", 128, 2, 32, 32
    # 129 ... 328 rows (past 128: the Q-parallel schedule of the backward),
    # plus an empty and a one-row history
    L = [129 + (37 * b + 11) % 200 for b in range(B)]
    L[3], L[5] = 0, 1
    print(f"\n[xattn many jagged] B={B} max_L={max(L)}", flush=True)
    QR = C * n_q
    M, off = B * QR, offsets(L)
    T = int(off[-1])
    Q, K, V, dA = draw(41, (M, d), dtype), draw(42, (T, d), dtype), draw(43, (T, d), dtype), draw(44, (M, d), dtype)
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tQ, tK, tV, tdA = (to_dev(x, dtype, gpu) for x in (Q, K, V, dA))
    toff = i64_dev(off, gpu)
    A, lse = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, tQ, tK, tV, toff, 0.0, A, lse)
    dQ, dK, dV = torch.empty_like(tQ), torch.empty_like(tK), torch.empty_like(tV)
    ws = torch.empty(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb._dtype_code(tQ)), dtype=torch.uint8, device=gpu)
    wb.whale_jagged_xattn_bwd(dm, tQ, tK, tV, toff, 0.0, A, lse, tdA, dQ, dK, dV, ws)
    torch.cuda.synchronize()
    sample = sorted({int(np.argmax(L)), L.index(0), L.index(1), B // 2, B - 1})
    for b in sample:
        q, k = slice(b * QR, (b + 1) * QR), slice(int(off[b]), int(off[b + 1]))
        o1 = np.array([0, L[b]])
        A_ref, lse_ref = O.xattn_fwd(Q[q], K[k], V[k], o1, C, n_q, h)
        dQ_ref, dK_ref, dV_ref = O.xattn_bwd(Q[q], K[k], V[k], o1, C, n_q, h, None, dA[q])
        assert_close(f"A[{b}]", A[q], A_ref, dtype)
        assert_close(f"dQ[{b}]", dQ[q], dQ_ref, dtype)
        if L[b] > 0:
            assert_close(f"dK[{b}]", dK[k], dK_ref, dtype)
            assert_close(f"dV[{b}]", dV[k], dV_ref, dtype)


def test_xattn_order_changes_no_bit(gpu):
    """The same 256 jagged requests run longest history first (alone) and in
    index order (with a 257th request appended): every output of the 256,
    forward and backward, is the same bit for bit."""
    dtype, d, h, C, n_q = "bf16", 128, 2, 32, 32
    # histories past 128 rows (the Q-parallel backward, one query split for
    # both batch sizes); the appended request is shorter than the longest, so
    # the shape hints other than B and total_L are the same
    L = [130 + (29 * b + 7) % 150 for b in range(256)]
    QR = C * n_q

    def run(lengths):
        B = len(lengths)
        M, off = B * QR, offsets(lengths)
        T = int(off[-1])
        Q, K, V, dA = draw(51, (M, d), dtype), draw(52, (T, d), dtype), draw(53, (T, d), dtype), draw(54, (M, d), dtype)
        dm = wb.dims(B, C, n_q, d, h, max(lengths), T)
        tQ, tK, tV, tdA = (to_dev(x, dtype, gpu) for x in (Q, K, V, dA))
        toff = i64_dev(off, gpu)
        A, lse = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
        wb.whale_jagged_xattn_fwd(dm, tQ, tK, tV, toff, 0.0, A, lse)
        dQ, dK, dV = torch.empty_like(tQ), torch.empty_like(tK), torch.empty_like(tV)
        ws = torch.empty(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb._dtype_code(tQ)), dtype=torch.uint8,
                         device=gpu)
        wb.whale_jagged_xattn_bwd(dm, tQ, tK, tV, toff, 0.0, A, lse, tdA, dQ, dK, dV, ws)
        torch.cuda.synchronize()
        return A, lse, dQ, dK, dV

    # the appended request's rows come last in every tensor, so the first
    # 256 requests' inputs (drawn row-major from the same seeds) are identical
    ranked = run(L)
    indexed = run(L + [5])
    M, T = 256 * QR, int(offsets(L)[-1])
    for name, a, b_, n in zip(("A", "lse", "dQ", "dK", "dV"), ranked, indexed, (M, M, M, T, T)):
        assert torch.equal(a[:n], b_[:n]), name
