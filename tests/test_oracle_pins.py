"""Pins of the fp64 oracle against things other than itself.

Each test fixes one part of the oracle by a library routine that computes the
same quantity independently (torch's fp64 CPU attention, layer norm, RMS norm,
SiLU and autograd), a closed form, an invariant, a hand-derived worked example
or brute force on tiny inputs.  Together they are chosen so that a dropped
term, a wrong sign or index, or a transposed operand anywhere in the oracle
fails at least one of them (the mutation tests at the end check a few such
mistakes explicitly).  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import whale_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def small_case(seed=0, B=3, C=2, n_q=3, d=16, h=2, lengths=(5, 1, 7)):
    L = np.asarray(lengths)
    off = np.concatenate([[0], np.cumsum(L)])
    M, T = B * C * n_q, int(off[-1])
    return dict(B=B, C=C, n_q=n_q, d=d, h=h, off=off,
                Q=rnd(seed, M, d), K=rnd(seed + 1, T, d), V=rnd(seed + 2, T, d))


def t64(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


# ------------------------------------------------------------ worked examples

def test_golden_worked_examples():
    g = json.load(open(GOLDEN))
    e = g["attention_two_keys"]
    A, lse = O.xattn_fwd(e["q"], e["k"], e["v"], [0, 2], C=1, n_q=1, h=1, scale=e["scale"])
    np.testing.assert_allclose(A, e["A"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], e["lse"], rtol=0, atol=1e-14)
    e = g["fusion_mlp_select"]
    F, _ = O.fusion_mlp(e["A"], e["H_w"], e["W_F"], O.ACT_NONE)
    np.testing.assert_array_equal(F, e["F_none"])
    F, _ = O.fusion_mlp(e["A"], e["H_w"], e["W_F"], O.ACT_SILU)
    np.testing.assert_allclose(F, e["F_silu"], rtol=0, atol=1e-15)
    e = g["swiglu_tied_scalar"]
    Y, _ = O.swiglu_ffn(e["F"], O.NORM_NONE, 0.0, [1.0], [0.0], e["W_U"], O.GATE_SHARED, e["W_D"])
    np.testing.assert_allclose(Y, e["Y"], rtol=1e-15)


# ------------------------------------------------------------ attention (a3)

def test_attention_matches_torch_sdpa():
    c = small_case()
    A, lse = O.xattn_fwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    dh = c["d"] // c["h"]
    for b in range(c["B"]):
        rows = slice(b * c["C"] * c["n_q"], (b + 1) * c["C"] * c["n_q"])
        lo, hi = c["off"][b], c["off"][b + 1]
        for j in range(c["h"]):
            cols = slice(j * dh, (j + 1) * dh)
            q, k, v = t64(c["Q"][rows, cols]), t64(c["K"][lo:hi, cols]), t64(c["V"][lo:hi, cols])
            ref = TF.scaled_dot_product_attention(q[None], k[None], v[None])[0].numpy()
            np.testing.assert_allclose(A[rows, cols], ref, rtol=1e-12, atol=1e-13)
            s = (q @ k.T).numpy() / math.sqrt(dh)
            np.testing.assert_allclose(lse[rows, j], torch.logsumexp(torch.tensor(s), 1).numpy(),
                                       rtol=1e-13, atol=1e-13)


def test_attention_brute_force_fsum():
    c = small_case(seed=3, B=2, C=2, n_q=2, d=4, h=2, lengths=(3, 4))
    A, lse = O.xattn_fwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    dh = 2
    for b in range(2):
        for m in range(b * 4, (b + 1) * 4):
            for j in range(2):
                keys = range(c["off"][b], c["off"][b + 1])
                sc = [math.fsum(c["Q"][m, j * dh + e] * c["K"][l, j * dh + e] for e in range(dh))
                      / math.sqrt(dh) for l in keys]
                w = [math.exp(x) for x in sc]
                z = math.fsum(w)
                assert abs(lse[m, j] - math.log(z)) < 1e-13
                for e in range(dh):
                    a = math.fsum(w[i] * c["V"][l, j * dh + e] for i, l in enumerate(keys)) / z
                    assert abs(A[m, j * dh + e] - a) < 1e-13


def test_attention_weights_sum_to_one():
    c = small_case(seed=5)
    ones = np.ones_like(c["V"])
    A, _ = O.xattn_fwd(c["Q"], c["K"], ones, c["off"], c["C"], c["n_q"], c["h"])
    np.testing.assert_allclose(A, 1.0, rtol=0, atol=1e-14)


def test_single_key_returns_value_row_exactly():
    c = small_case(seed=7, lengths=(1, 1, 1))
    A, lse = O.xattn_fwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    per = c["C"] * c["n_q"]
    for b in range(c["B"]):
        np.testing.assert_array_equal(A[b * per:(b + 1) * per], np.repeat(c["V"][b:b + 1], per, 0))


def test_uniform_scores_give_average_pooling():
    # Q = 0 makes every score equal: the attention reduces to the mean of the
    # history's values, the average-pooling ablation of Table 1.
    c = small_case(seed=9)
    A, lse = O.xattn_fwd(np.zeros_like(c["Q"]), c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    per = c["C"] * c["n_q"]
    for b in range(c["B"]):
        lo, hi = c["off"][b], c["off"][b + 1]
        np.testing.assert_allclose(A[b * per:(b + 1) * per], np.repeat(c["V"][lo:hi].mean(0, keepdims=True), per, 0),
                                   rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse[b * per:(b + 1) * per], math.log(hi - lo), rtol=1e-14)


def test_one_hot_saturated_scores_pick_one_row():
    c = small_case(seed=11, B=1, C=1, n_q=2, d=4, h=1, lengths=(9,))
    K = np.zeros((9, 4))
    K[6] = [2000.0, 0, 0, 0]      # score gap 1000: exp(-1000) underflows to 0 in fp64
    Q = np.array([[1.0, 0, 0, 0], [1.0, 0, 0, 0]])
    A, lse = O.xattn_fwd(Q, K, c["V"], c["off"], 1, 2, 1)
    np.testing.assert_array_equal(A, np.repeat(c["V"][6:7], 2, 0))


def test_history_permutation_invariance():
    c = small_case(seed=13)
    A, lse = O.xattn_fwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    perm = np.concatenate([c["off"][b] + np.random.default_rng(b).permutation(c["off"][b + 1] - c["off"][b])
                           for b in range(c["B"])])
    A2, lse2 = O.xattn_fwd(c["Q"], c["K"][perm], c["V"][perm], c["off"], c["C"], c["n_q"], c["h"])
    np.testing.assert_allclose(A2, A, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13, atol=1e-14)


def test_candidate_independence():
    # Sharing K/V across the C candidates equals attending per candidate.
    c = small_case(seed=17)
    A, _ = O.xattn_fwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    n_q, C = c["n_q"], c["C"]
    for b in range(c["B"]):
        lo, hi = c["off"][b], c["off"][b + 1]
        for cc in range(C):
            rows = slice((b * C + cc) * n_q, (b * C + cc + 1) * n_q)
            A1, _ = O.xattn_fwd(c["Q"][rows], c["K"][lo:hi], c["V"][lo:hi], [0, hi - lo], 1, n_q, c["h"])
            np.testing.assert_allclose(A1, A[rows], rtol=1e-13, atol=1e-14)


def test_variable_candidates_match_sdpa_per_request():
    """Serving form (a different candidate count per request, zero included):
    every query row against torch's attention over its own request's history,
    and the whole against per-request calls with a fixed count."""
    n_q, d, h = 3, 8, 2
    C_b = [2, 0, 5, 1]
    L = [4, 6, 1, 3]
    coff = np.concatenate([[0], np.cumsum(C_b)])
    off = np.concatenate([[0], np.cumsum(L)])
    M, T = n_q * int(coff[-1]), int(off[-1])
    Q, K, V = rnd(41, M, d), rnd(42, T, d), rnd(43, T, d)
    A, lse = O.xattn_fwd(Q, K, V, off, None, n_q, h, cand_offsets=coff)
    dh = d // h
    for b in range(len(C_b)):
        rows = slice(n_q * coff[b], n_q * coff[b + 1])
        lo, hi = off[b], off[b + 1]
        for j in range(h):
            cols = slice(j * dh, (j + 1) * dh)
            q, k, v = t64(Q[rows, cols]), t64(K[lo:hi, cols]), t64(V[lo:hi, cols])
            ref = TF.scaled_dot_product_attention(q[None], k[None], v[None])[0].numpy()
            np.testing.assert_allclose(A[rows, cols], ref, rtol=1e-12, atol=1e-13)
            s = (q @ k.T).numpy() / math.sqrt(dh)
            np.testing.assert_allclose(lse[rows, j], torch.logsumexp(torch.tensor(s), 1).numpy(),
                                       rtol=1e-13, atol=1e-13)
        if C_b[b]:
            A1, l1 = O.xattn_fwd(Q[rows], K[lo:hi], V[lo:hi], [0, hi - lo], C_b[b], n_q, h)
            np.testing.assert_array_equal(A1, A[rows])
            np.testing.assert_array_equal(l1, lse[rows])


def test_variable_candidates_layer_is_per_request_layers():
    """A layer with a different candidate count per request equals the same
    layer run request by request with that request's fixed count."""
    C_b, L = [3, 1, 0, 2], [4, 2, 3, 5]
    coff = np.concatenate([[0], np.cumsum(C_b)])
    x, p, _, kw = _layer_case(43, lengths=L)
    n_q, h, off = kw["n_q"], kw["h"], kw["offsets"]
    r = np.random.default_rng(44)
    H_w = r.standard_normal((n_q * int(coff[-1]), x["H_w"].shape[1]))
    Y = O.layer_fwd(H_w, x["H_s"], off, None, n_q, h, p, cand_offsets=coff)["Y"]
    for b in range(len(C_b)):
        if C_b[b] == 0:
            continue
        rows = slice(n_q * coff[b], n_q * coff[b + 1])
        Y1 = O.layer_fwd(H_w[rows], x["H_s"][off[b]:off[b + 1]], [0, L[b]], C_b[b], n_q, h, p)["Y"]
        np.testing.assert_allclose(Y[rows], Y1, rtol=1e-12, atol=1e-12)


def test_empty_history():
    c = small_case(seed=19, lengths=(4, 0, 3))
    A, lse = O.xattn_fwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    per = c["C"] * c["n_q"]
    assert np.all(A[per:2 * per] == 0) and np.all(np.isneginf(lse[per:2 * per]))
    dA = rnd(1, *A.shape)
    dQ, dK, dV = O.xattn_bwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"], None, dA)
    assert np.all(dQ[per:2 * per] == 0)


# ------------------------------------------------------------ norms, act

@pytest.mark.parametrize("kind", [O.NORM_LAYER, O.NORM_RMS, O.NORM_NONE])
def test_norm_matches_torch(kind):
    x, g, b = rnd(1, 6, 16) * 3 + 1, rnd(2, 16), rnd(3, 16)
    y, xhat, rstd = O.norm_fwd(x, kind, g, b, 1e-5)
    if kind == O.NORM_LAYER:
        ref = TF.layer_norm(t64(x), (16,), t64(g), t64(b), 1e-5).numpy()
        np.testing.assert_allclose(xhat.mean(1), 0, atol=1e-14)
        np.testing.assert_allclose(xhat.var(1), 1, rtol=1e-5)
    elif kind == O.NORM_RMS:
        ref = TF.rms_norm(t64(x), (16,), t64(g), 1e-5).numpy()
        np.testing.assert_allclose(np.sqrt((xhat ** 2).mean(1)), 1, rtol=1e-5)
    else:
        ref = x
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_silu_and_derivative_match_torch():
    z = t64(np.linspace(-30, 30, 601)).requires_grad_()
    s = TF.silu(z)
    s.sum().backward()
    np.testing.assert_allclose(O.silu(z.detach().numpy()), s.detach().numpy(), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(O.dsilu(z.detach().numpy()), z.grad.numpy(), rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------ a1, a2, a4, a5

def test_identity_projection():
    Hw, Hs = rnd(1, 6, 8), rnd(2, 5, 8)
    I = np.eye(8)
    Q, K, V = O.proj_qkv(Hw, Hs, O.NORM_NONE, 0.0, None, None, None, None, I, I, I)
    np.testing.assert_array_equal(Q, Hw)
    np.testing.assert_array_equal(K, Hs)
    np.testing.assert_array_equal(V, Hs)


def test_projection_matches_torch_linear():
    Hw, Hs = rnd(1, 6, 8), rnd(2, 5, 8)
    Wq, Wk, Wv = rnd(3, 8, 8), rnd(4, 8, 8), rnd(5, 8, 8)
    g, b = rnd(6, 8), rnd(7, 8)
    Q, K, V = O.proj_qkv(Hw, Hs, O.NORM_LAYER, 1e-5, g, b, g, b, Wq, Wk, Wv)
    Xq = TF.layer_norm(t64(Hw), (8,), t64(g), t64(b), 1e-5)
    Xs = TF.layer_norm(t64(Hs), (8,), t64(g), t64(b), 1e-5)
    np.testing.assert_allclose(Q, TF.linear(Xq, t64(Wq)).numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(K, TF.linear(Xs, t64(Wk)).numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(V, TF.linear(Xs, t64(Wv)).numpy(), rtol=1e-13, atol=1e-13)


def test_fusion_mlp_closed_forms():
    A, Hw = rnd(1, 5, 4), rnd(2, 5, 4)
    I, Z0 = np.eye(4), np.zeros((4, 4))
    F, _ = O.fusion_mlp(A, Hw, np.zeros((4, 8)), O.ACT_SILU)
    np.testing.assert_array_equal(F, Hw)                       # SiLU(0) = 0
    F, _ = O.fusion_mlp(A, Hw, np.hstack([I, Z0]), O.ACT_NONE)
    np.testing.assert_array_equal(F, Hw + A)                   # attended half first
    F, _ = O.fusion_mlp(A, Hw, np.hstack([Z0, I]), O.ACT_NONE)
    np.testing.assert_array_equal(F, 2 * Hw)                   # Wukong half second
    W = rnd(3, 4, 8)
    F, Z = O.fusion_mlp(A, Hw, W, O.ACT_SILU)
    ref = t64(Hw) + TF.silu(TF.linear(torch.cat([t64(A), t64(Hw)], 1), t64(W)))
    np.testing.assert_allclose(F, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_swiglu_closed_forms():
    Fm = rnd(1, 6, 4)
    d, H = 4, 4
    Wu, Wd = rnd(2, H, d), rnd(3, d, H)
    Y, U = O.swiglu_ffn(Fm, O.NORM_NONE, 0.0, None, None, Wu, O.GATE_SHARED, np.zeros((d, H)))
    np.testing.assert_array_equal(Y, Fm)                         # W_D = 0
    Y, U = O.swiglu_ffn(Fm, O.NORM_NONE, 0.0, None, None, np.eye(4), O.GATE_SHARED, np.eye(4))
    sig = 1 / (1 + np.exp(-Fm))
    np.testing.assert_allclose(Y, Fm + Fm * Fm * sig, rtol=1e-14)   # G = U^2 sigma(U)
    # separate gate with W_G = W_U equals the tied gate
    g, b = rnd(4, d), rnd(5, d)
    Yt, _ = O.swiglu_ffn(Fm, O.NORM_LAYER, 1e-5, g, b, Wu, O.GATE_SHARED, Wd)
    Ys, _ = O.swiglu_ffn(Fm, O.NORM_LAYER, 1e-5, g, b, np.vstack([Wu, Wu]), O.GATE_SEPARATE, Wd)
    np.testing.assert_allclose(Ys, Yt, rtol=1e-14, atol=1e-14)
    # separate gate against torch with distinct W_G, W_U
    Wg = rnd(6, H, d)
    Ys, _ = O.swiglu_ffn(Fm, O.NORM_LAYER, 1e-5, g, b, np.vstack([Wg, Wu]), O.GATE_SEPARATE, Wd)
    X = TF.layer_norm(t64(Fm), (d,), t64(g), t64(b), 1e-5)
    ref = t64(Fm) + TF.linear(TF.silu(TF.linear(X, t64(Wg))) * TF.linear(X, t64(Wu)), t64(Wd))
    np.testing.assert_allclose(Ys, ref.numpy(), rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ backward

def _layer_case(seed, lengths=(3, 1, 0), norm=O.NORM_LAYER, gate=O.GATE_SHARED, ffn=True, act=O.ACT_SILU):
    B, C, n_q, d, h, H = len(lengths), 2, 2, 8, 2, 12
    off = np.concatenate([[0], np.cumsum(lengths)])
    r = np.random.default_rng(seed)
    p = {k: r.standard_normal((d, d)) * 0.4 for k in ("W_Q", "W_K", "W_V")}
    p["W_F"] = r.standard_normal((d, 2 * d)) * 0.3
    p["W_U"] = r.standard_normal(((2 if gate == O.GATE_SEPARATE else 1) * H, d)) * 0.3
    p["W_D"] = r.standard_normal((d, H)) * 0.3
    for k in ("g_q", "g_kv", "g_f"):
        p[k] = 1 + 0.3 * r.standard_normal(d)
    for k in ("b_q", "b_kv", "b_f"):
        p[k] = 0.3 * r.standard_normal(d)
    x = dict(H_w=r.standard_normal((B * C * n_q, d)), H_s=r.standard_normal((int(off[-1]), d)))
    dY = r.standard_normal((B * C * n_q, d))
    kw = dict(offsets=off, C=C, n_q=n_q, h=h, norm=norm, gate=gate, ffn=ffn, act=act)
    return x, p, dY, kw


GRAD_OF = {"H_w": "dH_w", "H_s": "dH_s", "W_Q": "dW_Q", "W_K": "dW_K", "W_V": "dW_V",
           "W_F": "dW_F", "W_U": "dW_U", "W_D": "dW_D", "g_q": "dg_q", "b_q": "db_q",
           "g_kv": "dg_kv", "b_kv": "db_kv", "g_f": "dg_f", "b_f": "db_f"}


# Every branch of the oracle's backward: the three norms, both gates, both
# fusion activations, with and without the FFN.
FD_CASES = [(O.NORM_LAYER, O.GATE_SHARED, True, O.ACT_SILU),
            (O.NORM_RMS, O.GATE_SEPARATE, True, O.ACT_SILU),
            (O.NORM_LAYER, O.GATE_SHARED, False, O.ACT_SILU),
            (O.NORM_LAYER, O.GATE_SEPARATE, True, O.ACT_NONE),
            (O.NORM_NONE, O.GATE_SHARED, True, O.ACT_NONE),
            (O.NORM_NONE, O.GATE_SEPARATE, True, O.ACT_SILU),
            (O.NORM_RMS, O.GATE_SHARED, False, O.ACT_NONE)]


@pytest.mark.parametrize("norm,gate,ffn,act", FD_CASES)
def test_layer_gradients_match_finite_differences(norm, gate, ffn, act):
    x, p, dY, kw = _layer_case(21, norm=norm, gate=gate, ffn=ffn, act=act)

    def loss():
        out = O.layer_fwd(x["H_w"], x["H_s"], p=p, **kw)
        return float((out["Y"] * dY).sum())

    g = O.layer_bwd(x["H_w"], x["H_s"], p=p, dY=dY, **kw)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if not ffn and name in ("W_U", "W_D", "g_f", "b_f"):
            continue
        if (norm == O.NORM_RMS and name in ("b_q", "b_kv", "b_f")) or (norm == O.NORM_NONE and name[:2] in ("g_", "b_")):
            # parameters the norm does not use: exactly zero gradient
            np.testing.assert_array_equal(g[gname], 0)
            continue
        arr = x[name] if name in x else p[name]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss()
            arr[idx] = old - eps
            lm = loss()
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=1e-6, atol=1e-7, err_msg=name)


def _torch_norm(x, kind, g, b):
    d = x.shape[1]
    if kind == O.NORM_LAYER:
        return TF.layer_norm(x, (d,), g, b, 1e-5)
    if kind == O.NORM_RMS:
        return TF.rms_norm(x, (d,), g, 1e-5)
    return x


def _torch_layer(T, kw, tied=False):
    """The fusion layer written with torch fp64 ops (SDPA per request and
    head), independent of the oracle, for autograd."""
    C, n_q, h, off = kw["C"], kw["n_q"], kw["h"], kw["offsets"]
    norm, gate, act, ffn = kw["norm"], kw["gate"], kw["act"], kw["ffn"]
    d = T["H_w"].shape[1]
    Xq = _torch_norm(T["H_w"], norm, T["g_q"], T["b_q"])
    Xs = _torch_norm(T["H_s"], norm, T["g_kv"], T["b_kv"])
    Q, K = Xq @ T["W_Q"].T, Xs @ T["W_K"].T
    V = K if tied else Xs @ T["W_V"].T
    dh = d // h
    A_rows = []
    for b in range(len(off) - 1):
        q = Q[b * C * n_q:(b + 1) * C * n_q].reshape(-1, h, dh).transpose(0, 1)
        k = K[off[b]:off[b + 1]].reshape(-1, h, dh).transpose(0, 1)
        v = V[off[b]:off[b + 1]].reshape(-1, h, dh).transpose(0, 1)
        if k.shape[1] == 0:
            A_rows.append(torch.zeros(C * n_q, d, dtype=torch.float64))
            continue
        A_rows.append(TF.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(-1, d))
    A = torch.cat(A_rows)
    Z = torch.cat([A, T["H_w"]], 1) @ T["W_F"].T
    F = T["H_w"] + (TF.silu(Z) if act == O.ACT_SILU else Z)
    if not ffn:
        return F
    U = _torch_norm(F, norm, T["g_f"], T["b_f"]) @ T["W_U"].T
    if gate == O.GATE_SHARED:
        G = TF.silu(U) * U
    else:
        Hh = U.shape[1] // 2
        G = TF.silu(U[:, :Hh]) * U[:, Hh:]
    return F + G @ T["W_D"].T


@pytest.mark.parametrize("norm,gate,ffn,act", FD_CASES)
def test_gradients_match_torch_autograd(norm, gate, ffn, act):
    x, p, dY, kw = _layer_case(23, lengths=(6, 2, 5), norm=norm, gate=gate, ffn=ffn, act=act)
    g = O.layer_bwd(x["H_w"], x["H_s"], p=p, dY=dY, **kw)
    T = {k: t64(v).requires_grad_() for k, v in {**x, **p}.items()}
    Y = _torch_layer(T, kw)
    (Y * t64(dY)).sum().backward()
    for name, gname in GRAD_OF.items():
        if not ffn and name in ("W_U", "W_D", "g_f", "b_f"):
            continue
        want = T[name].grad
        want = np.zeros(T[name].shape) if want is None else want.numpy()   # unused by this norm kind
        np.testing.assert_allclose(g[gname], want, rtol=1e-10, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("act", [O.ACT_SILU, O.ACT_NONE])
def test_fusion_mlp_bwd_matches_autograd(act):
    """fusion_mlp_bwd on its own, for both activations (the calls the GPU
    tests compare against)."""
    r = np.random.default_rng(71)
    M, d = 9, 6
    A, Hw, Wf, dF = r.standard_normal((M, d)), r.standard_normal((M, d)), r.standard_normal((d, 2 * d)), \
        r.standard_normal((M, d))
    dA, dHw, dWf = O.fusion_mlp_bwd(A, Hw, Wf, act, dF)
    tA, tH, tW = (t64(v).requires_grad_() for v in (A, Hw, Wf))
    Z = torch.cat([tA, tH], 1) @ tW.T
    F = tH + (TF.silu(Z) if act == O.ACT_SILU else Z)
    (F * t64(dF)).sum().backward()
    for got, want in ((dA, tA.grad), (dHw, tH.grad), (dWf, tW.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kind", [O.NORM_LAYER, O.NORM_RMS, O.NORM_NONE])
def test_norm_bwd_matches_autograd(kind):
    r = np.random.default_rng(73)
    x, g, b, dy = r.standard_normal((7, 10)) * 2 + 0.5, 1 + 0.3 * r.standard_normal(10), r.standard_normal(10), \
        r.standard_normal((7, 10))
    dx, dg, db = O.norm_bwd(x, kind, g, 1e-5, dy)
    tx, tg, tb = (t64(v).requires_grad_() for v in (x, g, b))
    (_torch_norm(tx, kind, tg, tb) * t64(dy)).sum().backward()
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dg, np.zeros(10) if tg.grad is None else tg.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db, np.zeros(10) if tb.grad is None else tb.grad.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("norm", [O.NORM_LAYER, O.NORM_RMS, O.NORM_NONE])
@pytest.mark.parametrize("gate", [O.GATE_SHARED, O.GATE_SEPARATE])
def test_swiglu_ffn_bwd_matches_autograd(norm, gate):
    r = np.random.default_rng(79)
    M, d, H = 8, 6, 10
    F, dY = r.standard_normal((M, d)), r.standard_normal((M, d))
    g, b = 1 + 0.3 * r.standard_normal(d), 0.3 * r.standard_normal(d)
    Wu = r.standard_normal(((2 if gate == O.GATE_SEPARATE else 1) * H, d)) * 0.5
    Wd = r.standard_normal((d, H)) * 0.5
    out = O.swiglu_ffn_bwd(F, norm, 1e-5, g, b, Wu, gate, Wd, dY)
    tF, tg, tb, tU, tD = (t64(v).requires_grad_() for v in (F, g, b, Wu, Wd))
    U = _torch_norm(tF, norm, tg, tb) @ tU.T
    G = TF.silu(U) * U if gate == O.GATE_SHARED else TF.silu(U[:, :H]) * U[:, H:]
    ((tF + G @ tD.T) * t64(dY)).sum().backward()
    for k, t in (("dF", tF), ("dW_U", tU), ("dW_D", tD), ("dg_f", tg), ("db_f", tb)):
        want = np.zeros(t.shape) if t.grad is None else t.grad.numpy()
        np.testing.assert_allclose(out[k], want, rtol=1e-11, atol=1e-12, err_msg=k)


@pytest.mark.parametrize("norm", [O.NORM_LAYER, O.NORM_RMS, O.NORM_NONE])
@pytest.mark.parametrize("tied", [False, True])
def test_proj_qkv_bwd_matches_autograd(norm, tied):
    r = np.random.default_rng(83)
    M, T, d = 7, 9, 8
    Hw, Hs = r.standard_normal((M, d)), r.standard_normal((T, d))
    gq, bq, gk, bk = (1 + 0.3 * r.standard_normal(d) if i % 2 == 0 else 0.3 * r.standard_normal(d) for i in range(4))
    Wq, Wk, Wv = (r.standard_normal((d, d)) * 0.4 for _ in range(3))
    dQ, dK, dV = r.standard_normal((M, d)), r.standard_normal((T, d)), r.standard_normal((T, d))
    out = O.proj_qkv_bwd(Hw, Hs, norm, 1e-5, gq, bq, gk, bk, Wq, Wk, None if tied else Wv, dQ, dK,
                         None if tied else dV)
    t = {k: t64(v).requires_grad_() for k, v in dict(H_w=Hw, H_s=Hs, g_q=gq, b_q=bq, g_kv=gk, b_kv=bk, W_Q=Wq,
                                                      W_K=Wk, W_V=Wv).items()}
    Q = _torch_norm(t["H_w"], norm, t["g_q"], t["b_q"]) @ t["W_Q"].T
    Xs = _torch_norm(t["H_s"], norm, t["g_kv"], t["b_kv"])
    K = Xs @ t["W_K"].T
    loss = (Q * t64(dQ)).sum() + (K * t64(dK)).sum()
    if not tied:
        loss = loss + ((Xs @ t["W_V"].T) * t64(dV)).sum()
    loss.backward()
    names = ["H_w", "H_s", "W_Q", "W_K", "g_q", "b_q", "g_kv", "b_kv"] + ([] if tied else ["W_V"])
    for n in names:
        want = np.zeros(t[n].shape) if t[n].grad is None else t[n].grad.numpy()
        np.testing.assert_allclose(out[GRAD_OF[n]], want, rtol=1e-11, atol=1e-12, err_msg=n)
    assert tied == ("dW_V" not in out)


def test_shared_kv_layer_matches_finite_differences_and_autograd():
    """Shared key-value form (one tensor as keys and values, no W_V): every
    gradient against central differences, and against torch autograd through
    a model that feeds the same tensor to both roles of the attention."""
    x, p, dY, kw = _layer_case(37, lengths=(4, 1, 3))
    del p["W_V"]

    def loss():
        return float((O.layer_fwd(x["H_w"], x["H_s"], p=p, **kw)["Y"] * dY).sum())

    g = O.layer_bwd(x["H_w"], x["H_s"], p=p, dY=dY, **kw)
    assert "dW_V" not in g and g["dV"] is None
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if name == "W_V":
            continue
        arr = x[name] if name in x else p[name]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss()
            arr[idx] = old - eps
            lm = loss()
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], num, rtol=1e-6, atol=1e-7, err_msg=name)

    T = {k: t64(v).requires_grad_() for k, v in {**x, **p}.items()}
    C, n_q, h, off = kw["C"], kw["n_q"], kw["h"], kw["offsets"]
    d = T["H_w"].shape[1]
    Xq = TF.layer_norm(T["H_w"], (d,), T["g_q"], T["b_q"], 1e-5)
    Xs = TF.layer_norm(T["H_s"], (d,), T["g_kv"], T["b_kv"], 1e-5)
    Q, K = Xq @ T["W_Q"].T, Xs @ T["W_K"].T
    dh = d // h
    A_rows = []
    for b in range(len(off) - 1):
        q = Q[b * C * n_q:(b + 1) * C * n_q].reshape(-1, h, dh).transpose(0, 1)
        k = K[off[b]:off[b + 1]].reshape(-1, h, dh).transpose(0, 1)
        if k.shape[1] == 0:
            A_rows.append(torch.zeros(C * n_q, d, dtype=torch.float64))
            continue
        A_rows.append(TF.scaled_dot_product_attention(q, k, k).transpose(0, 1).reshape(-1, d))
    A = torch.cat(A_rows)
    F = T["H_w"] + TF.silu(torch.cat([A, T["H_w"]], 1) @ T["W_F"].T)
    U = TF.layer_norm(F, (d,), T["g_f"], T["b_f"], 1e-5) @ T["W_U"].T
    Y = F + (TF.silu(U) * U) @ T["W_D"].T
    (Y * t64(dY)).sum().backward()
    for name, gname in GRAD_OF.items():
        if name != "W_V":
            np.testing.assert_allclose(g[gname], T[name].grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_single_key_backward_closed_form():
    c = small_case(seed=29, lengths=(1, 1, 1))
    dA = rnd(31, *c["Q"].shape)
    dQ, dK, dV = O.xattn_bwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"], None, dA)
    per = c["C"] * c["n_q"]
    np.testing.assert_allclose(dQ, 0, atol=1e-14)
    np.testing.assert_allclose(dK, 0, atol=1e-13)
    for b in range(c["B"]):
        np.testing.assert_allclose(dV[b], dA[b * per:(b + 1) * per].sum(0), rtol=1e-13)


def test_kv_gradient_sums_over_candidates():
    # dK, dV of the shared K/V = the sum over candidates of each candidate's own.
    c = small_case(seed=37)
    dA = rnd(41, *c["Q"].shape)
    _, dK, dV = O.xattn_bwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"], None, dA)
    n_q, C = c["n_q"], c["C"]
    for b in range(c["B"]):
        lo, hi = c["off"][b], c["off"][b + 1]
        sk, sv = np.zeros((hi - lo, c["d"])), np.zeros((hi - lo, c["d"]))
        for cc in range(C):
            rows = slice((b * C + cc) * n_q, (b * C + cc + 1) * n_q)
            _, k1, v1 = O.xattn_bwd(c["Q"][rows], c["K"][lo:hi], c["V"][lo:hi], [0, hi - lo], 1, n_q,
                                    c["h"], None, dA[rows])
            sk += k1
            sv += v1
        np.testing.assert_allclose(dK[lo:hi], sk, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dV[lo:hi], sv, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ planted mistakes

def _mutant_xattn(kind):
    """A copy of the oracle's attention with one plausible mistake planted."""
    def f(Q, K, V, offsets, C, n_q, h, scale=None):
        Q, K, V = np.asarray(Q, float), np.asarray(K, float), np.asarray(V, float)
        M, d = Q.shape
        dh = d // h
        sc = 1 / np.sqrt(dh) if kind != "no_scale" else 1.0
        A = np.zeros((M, d))
        for b in range(len(offsets) - 1):
            rows = slice(b * C * n_q, (b + 1) * C * n_q)
            if kind == "row_by_request_only":
                rows = slice(b * n_q, (b + 1) * n_q) if b * n_q < M else slice(0, 0)
            lo, hi = offsets[b], offsets[b + 1]
            if kind == "drop_last_key":
                hi = max(lo + 1, hi - 1)
            for j in range(h):
                cols = slice(j * dh, (j + 1) * dh)
                s = sc * Q[rows, cols] @ K[lo:hi, cols].T
                e = np.exp(s - s.max(1, keepdims=True))
                p = e / e.sum(1, keepdims=True)
                if kind == "transposed_head":
                    A[rows, cols] = p @ V[lo:hi, (slice((h - 1 - j) * dh, (h - j) * dh))]
                else:
                    A[rows, cols] = p @ V[lo:hi, cols]
        return A
    return f


@pytest.mark.parametrize("kind", ["no_scale", "row_by_request_only", "drop_last_key", "transposed_head"])
def test_pins_catch_planted_attention_mistakes(kind):
    c = small_case(seed=43, lengths=(5, 4, 7))
    mut = _mutant_xattn(kind)(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    ok, _ = O.xattn_fwd(c["Q"], c["K"], c["V"], c["off"], c["C"], c["n_q"], c["h"])
    dh = c["d"] // c["h"]
    ref = np.zeros_like(ok)
    for b in range(c["B"]):
        rows = slice(b * c["C"] * c["n_q"], (b + 1) * c["C"] * c["n_q"])
        lo, hi = c["off"][b], c["off"][b + 1]
        for j in range(c["h"]):
            cols = slice(j * dh, (j + 1) * dh)
            ref[rows, cols] = TF.scaled_dot_product_attention(
                t64(c["Q"][rows, cols])[None], t64(c["K"][lo:hi, cols])[None], t64(c["V"][lo:hi, cols])[None])[0].numpy()
    np.testing.assert_allclose(ok, ref, rtol=1e-12, atol=1e-13)
    assert not np.allclose(mut, ref, rtol=1e-6, atol=1e-8)
