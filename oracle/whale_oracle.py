"""Plain fp64 CPU oracle of the WHALE attention-fusion module, forward and backward.

TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only code that may import this module.  It imports
nothing from the HIP package and the HIP package imports nothing from it.  It
is slow on purpose: every function writes out the plain definition of one step
in float64 with numpy, one request and one head at a time, with a matrix
product as the only library primitive.  None of the GPU path's tiling,
online-softmax rescaling, sharing of K/V across candidates, or query split
appears here, because none of them changes the result.

Sources (web pages about arXiv 2607.17017, "WHALE: A Scalable Unified Model for
Recommendation with Wukong-HSTU Architecture"):
  [GS 2.1]  gist.science explainer, Technical Summary §2.1 (Core Architecture,
            "Attention-Based Fusion Module")
  [GS 2.2]  gist.science explainer, Technical Summary §2.2 (Efficiency
            Optimizations: shared key-value, shared-gate SwiGLU, mixed
            precision)
  [PD 2]    paper-daily.com deep reading of WHALE, §2 (method details)
  [PV km]   pith.science verdict record, pith_extraction.key_machinery
  [PV ref]  pith.science verdict record, referee_report: minor comments on
            Eq. (4) and Eq. (5), major comment on §5.1/Footnote 1
  [PR arg]  pith.science review page, "What carries the argument"

What the pages fix:
  * Queries come from the normalised Wukong tokens H_w through W_Q; keys and
    values come from the normalised HSTU states H_s through W_K and W_V
    [PV km], [PD 2], [GS 2.1].
  * Softmax dot-product attention gives one history-derived vector per
    interaction token, Eq. (4) [PV km], [PD 2].
  * K/V projections are computed per request and shared by all of its
    candidates (M-FALCON amortisation, Footnote 1) [PV ref].  Here this only
    means that K and V carry no candidate index.
  * The attended vector is concatenated with the Wukong representation,
    projected by one linear layer, and a residual is added, Eq. (5)
    [GS 2.1], [PV ref minor comment on Eq. (5)], [PV km].
  * A pre-norm SwiGLU FFN follows, whose gate and up projections are tied,
    so it costs two matrix products instead of three [GS 2.1], [GS 2.2], [PD 2].

Readings taken where the pages are silent (each one is listed with its
reason in the design notes of the repository):
  R1  "normalised" = LayerNorm with biased variance, eps inside the square
      root, affine gamma/beta; RMSNorm and no norm are also provided.
  R2  residuals add the un-normalised stream (H_w for the fusion MLP, F for
      the FFN): the usual pre-norm residual stream.
  R3  softmax scale 1/sqrt(d_h) unless given.
  R4  h heads split d into contiguous slices of width d_h = d/h; there is no
      output projection besides W_F.
  R5  no biases in the linear layers.
  R6  no causal/time mask and no relative bias in the fusion attention; only
      the jagged history length bounds each request.
  R7  concatenation order [A, H_w]; activation SiLU (or none).
  R8  tied gate: G = SiLU(U) * U with U = X_f W_U^T.  Separate gate (merged
      GEMM with [W_G; W_U]): G = SiLU(U_g) * U_u.
  R9  an empty history (L_b = 0) gives A = 0, lse = -inf, zero gradients.
  R10 shared key-value (K = V, [GS 2.2]) means one projection, through W_K,
      whose output serves as both keys and values; the layer then has no
      W_V, and the gradient of that one tensor is the sum of its gradients
      in the two roles.  A layer whose parameters hold no W_V is tied.
  R11 serving with a different number of candidates per request: request b
      has C_b >= 0 candidates, given as prefix sums cand_offsets [B+1], and
      owns query rows n_q*cand_offsets[b] .. n_q*cand_offsets[b+1]-1.  Each
      of them attends the history of request b exactly as in Eq. (4); the
      K/V of a request are the same whichever candidates query them
      (Footnote 1, [PV ref]).
  R12 HSTU self-attention (NEXT f4, the producer of H_s): causal pointwise
      SiLU attention normalised by the history length, with a relative
      position bias and a log2-bucketed time bias shared by all heads (the
      pages name rab(p, t) without defining it; see hstu_attn_fwd).

Layouts (row-vector convention y = x W^T, weights stored [out, in]):
  H_w, Q, A, F, Y : [M, d] with M = B*C*n_q, row m = (b*C + c)*n_q + i
  H_s, K, V       : [T, d], request b owns rows offsets[b] .. offsets[b+1]-1
  lse             : [M, h], natural logarithm
"""
import numpy as np

NORM_LAYER, NORM_RMS, NORM_NONE = 0, 1, 2
ACT_SILU, ACT_NONE = 0, 1
GATE_SHARED, GATE_SEPARATE = 0, 1


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- norms (R1)

def norm_fwd(x, kind, gamma, beta, eps):
    """Row-wise normalisation before the Q, K/V and FFN projections [PV km],
    [GS 2.1 "pre-norm"].  Returns (y, xhat, rstd)."""
    x = _f64(x)
    if kind == NORM_NONE:
        return x.copy(), x.copy(), np.ones(x.shape[0])
    if kind == NORM_LAYER:
        mean = x.mean(axis=1, keepdims=True)
        var = ((x - mean) ** 2).mean(axis=1, keepdims=True)
        rstd = 1.0 / np.sqrt(var + eps)
        xhat = (x - mean) * rstd
        y = xhat * _f64(gamma) + _f64(beta)
    elif kind == NORM_RMS:
        ms = (x ** 2).mean(axis=1, keepdims=True)
        rstd = 1.0 / np.sqrt(ms + eps)
        xhat = x * rstd
        y = xhat * _f64(gamma)
    else:
        raise ValueError("unknown norm kind")
    return y, xhat, rstd[:, 0]


def norm_bwd(x, kind, gamma, eps, dy):
    """Chain rule through norm_fwd: returns (dx, dgamma, dbeta)."""
    x, dy = _f64(x), _f64(dy)
    n = x.shape[1]
    if kind == NORM_NONE:
        return dy.copy(), np.zeros(n), np.zeros(n)
    _, xhat, rstd = norm_fwd(x, kind, np.ones(n), np.zeros(n), eps)
    g = _f64(gamma)
    dgamma = (dy * xhat).sum(axis=0)
    dbeta = dy.sum(axis=0) if kind == NORM_LAYER else np.zeros(n)
    dxhat = dy * g
    r = rstd[:, None]
    if kind == NORM_LAYER:
        # xhat = (x - mean(x)) * r,  r = (var + eps)^(-1/2)
        dx = r * (dxhat - dxhat.mean(axis=1, keepdims=True)
                  - xhat * (dxhat * xhat).mean(axis=1, keepdims=True))
    else:
        # xhat = x * r,  r = (mean(x^2) + eps)^(-1/2)
        dx = r * (dxhat - xhat * (dxhat * xhat).mean(axis=1, keepdims=True))
    return dx, dgamma, dbeta


# ---------------------------------------------------------------- activations

def sigmoid(z):
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = _f64(z)
    return z * sigmoid(z)


def dsilu(z):
    s = sigmoid(z)
    return s * (1.0 + _f64(z) * (1.0 - s))


# ---------------------------------------------------------------- a1, a2

def proj_qkv(H_w, H_s, norm, eps, g_q, b_q, g_kv, b_kv, W_Q, W_K, W_V):
    """Q = Norm_q(H_w) W_Q^T ; K = Norm_kv(H_s) W_K^T ; V = Norm_kv(H_s) W_V^T.

    Queries from the normalised Wukong output, shared keys and values from the
    normalised HSTU output [PV km], [PD 2].  K and V are computed once per
    history row: no candidate index appears (Footnote 1, [PV ref]).
    W_V = None is the shared key-value form (R10): V is K itself."""
    X_q, _, _ = norm_fwd(H_w, norm, g_q, b_q, eps)
    X_s, _, _ = norm_fwd(H_s, norm, g_kv, b_kv, eps)
    K = X_s @ _f64(W_K).T
    return X_q @ _f64(W_Q).T, K, (K if W_V is None else X_s @ _f64(W_V).T)


def proj_qkv_bwd(H_w, H_s, norm, eps, g_q, b_q, g_kv, b_kv, W_Q, W_K, W_V, dQ, dK, dV):
    """Chain rule through proj_qkv.  Returns a dict with dH_w (the Q-path part
    only), dH_s, dW_Q, dW_K, dW_V, dg_q, db_q, dg_kv, db_kv.  In the shared
    key-value form (W_V and dV None, R10) dK is the gradient of the one
    tensor and there is no dW_V."""
    dQ, dK = _f64(dQ), _f64(dK)
    X_q, _, _ = norm_fwd(H_w, norm, g_q, b_q, eps)
    X_s, _, _ = norm_fwd(H_s, norm, g_kv, b_kv, eps)
    out = {"dW_Q": dQ.T @ X_q, "dW_K": dK.T @ X_s}
    dX_q = dQ @ _f64(W_Q)
    dX_s = dK @ _f64(W_K)
    if W_V is not None:
        dV = _f64(dV)
        out["dW_V"] = dV.T @ X_s
        dX_s = dX_s + dV @ _f64(W_V)
    out["dH_w"], out["dg_q"], out["db_q"] = norm_bwd(H_w, norm, g_q, eps, dX_q)
    out["dH_s"], out["dg_kv"], out["db_kv"] = norm_bwd(H_s, norm, g_kv, eps, dX_s)
    return out


# ---------------------------------------------------------------- a3

def _request_rows(b, C, n_q, cand_offsets=None):
    if cand_offsets is not None:                       # R11
        return slice(n_q * int(cand_offsets[b]), n_q * int(cand_offsets[b + 1]))
    return slice(b * C * n_q, (b + 1) * C * n_q)


def xattn_fwd(Q, K, V, offsets, C, n_q, h, scale=None, cand_offsets=None):
    """Eq. (4): every interaction token of every candidate of request b
    attends, with an unmasked softmax over dot products, to the whole history
    of request b [PV km], [PD 2], [GS 2.1].  Returns (A [M,d], lse [M,h]).
    cand_offsets [B+1] (R11) gives each request its own number of candidates;
    C is then unused."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    offsets = np.asarray(offsets, dtype=np.int64)
    B = len(offsets) - 1
    M, d = Q.shape
    dh = d // h
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(dh)
    A = np.zeros((M, d))
    lse = np.full((M, h), -np.inf)
    for b in range(B):
        rows = _request_rows(b, C, n_q, cand_offsets)
        lo, hi = offsets[b], offsets[b + 1]
        if hi == lo:
            continue                                   # R9
        for j in range(h):
            cols = slice(j * dh, (j + 1) * dh)
            s = scale * (Q[rows, cols] @ K[lo:hi, cols].T)   # [C*n_q, L_b]
            mu = s.max(axis=1, keepdims=True)
            e = np.exp(s - mu)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            A[rows, cols] = p @ V[lo:hi, cols]
            lse[rows, j] = (mu + np.log(z))[:, 0]
    return A, lse


def xattn_bwd(Q, K, V, offsets, C, n_q, h, scale, dA):
    """Exact chain rule of xattn_fwd.  The softmax Jacobian is applied in its
    textbook form dS = P * (dP - <P, dP>); dK and dV sum over all C*n_q
    queries of the request, which is what sharing K/V across candidates
    means for the gradient.  Returns (dQ, dK, dV)."""
    Q, K, V, dA = _f64(Q), _f64(K), _f64(V), _f64(dA)
    offsets = np.asarray(offsets, dtype=np.int64)
    B = len(offsets) - 1
    M, d = Q.shape
    dh = d // h
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(dh)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        rows = _request_rows(b, C, n_q)
        lo, hi = offsets[b], offsets[b + 1]
        if hi == lo:
            continue
        for j in range(h):
            cols = slice(j * dh, (j + 1) * dh)
            q, k, v, da = Q[rows, cols], K[lo:hi, cols], V[lo:hi, cols], dA[rows, cols]
            s = scale * (q @ k.T)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            dV[lo:hi, cols] = p.T @ da
            dp = da @ v.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dQ[rows, cols] = scale * (ds @ k)
            dK[lo:hi, cols] = scale * (ds.T @ q)
    return dQ, dK, dV


# ---------------------------------------------------------------- a4

def fusion_mlp(A, H_w, W_F, act=ACT_SILU):
    """Eq. (5): F = H_w + phi([A, H_w] W_F^T), one linear layer from 2d to d
    on the concatenation of the attended vector and the Wukong representation,
    plus a residual [GS 2.1], [PV ref minor comment on Eq. (5)], [PV km].
    Returns (F, Z) with Z the pre-activation."""
    X = np.concatenate([_f64(A), _f64(H_w)], axis=1)
    Z = X @ _f64(W_F).T
    phi = silu(Z) if act == ACT_SILU else Z
    return _f64(H_w) + phi, Z


def fusion_mlp_bwd(A, H_w, W_F, act, dF):
    """Chain rule of fusion_mlp.  Returns (dA, dH_w, dW_F); dH_w holds the
    residual term plus the H_w half of the concatenation."""
    A, H_w, W_F, dF = _f64(A), _f64(H_w), _f64(W_F), _f64(dF)
    d = A.shape[1]
    X = np.concatenate([A, H_w], axis=1)
    Z = X @ W_F.T
    dZ = dF * (dsilu(Z) if act == ACT_SILU else 1.0)
    dX = dZ @ W_F
    dW_F = dZ.T @ X
    return dX[:, :d], dF + dX[:, d:], dW_F


# ---------------------------------------------------------------- a5

def swiglu_ffn(F, norm, eps, g_f, b_f, W_U, gate, W_D):
    """Pre-norm SwiGLU FFN with the residual on F [GS 2.1], [PV km].
    Shared gate (W_gate = W_up): G = SiLU(U) * U, two matrix products
    [GS 2.2], [PD 2].  Separate gate: W_U holds [W_G; W_U] stacked (2H rows)
    and G = SiLU(U_g) * U_u.  Returns (Y, U) with U = X_f W_U^T."""
    X_f, _, _ = norm_fwd(F, norm, g_f, b_f, eps)
    U = X_f @ _f64(W_U).T
    if gate == GATE_SHARED:
        G = silu(U) * U
    else:
        H = U.shape[1] // 2
        G = silu(U[:, :H]) * U[:, H:]
    return _f64(F) + G @ _f64(W_D).T, U


def swiglu_ffn_bwd(F, norm, eps, g_f, b_f, W_U, gate, W_D, dY):
    """Chain rule of swiglu_ffn.  Returns dict dF, dW_U, dW_D, dg_f, db_f."""
    F, W_U, W_D, dY = _f64(F), _f64(W_U), _f64(W_D), _f64(dY)
    X_f, _, _ = norm_fwd(F, norm, g_f, b_f, eps)
    U = X_f @ W_U.T
    if gate == GATE_SHARED:
        G = silu(U) * U
    else:
        H = U.shape[1] // 2
        G = silu(U[:, :H]) * U[:, H:]
    dG = dY @ W_D
    if gate == GATE_SHARED:
        # d/du [silu(u) u] = silu'(u) u + silu(u)
        dU = dG * (dsilu(U) * U + silu(U))
    else:
        Ug, Uu = U[:, :H], U[:, H:]
        dU = np.concatenate([dG * Uu * dsilu(Ug), dG * silu(Ug)], axis=1)
    out = {"dW_D": dY.T @ G, "dW_U": dU.T @ X_f}
    dX_f = dU @ W_U
    dxn, out["dg_f"], out["db_f"] = norm_bwd(F, norm, g_f, eps, dX_f)
    out["dF"] = dY + dxn
    return out


# ---------------------------------------------------------------- whole layer

def layer_fwd(H_w, H_s, offsets, C, n_q, h, p, norm=NORM_LAYER, eps=1e-5,
              act=ACT_SILU, gate=GATE_SHARED, ffn=True, scale=None, cand_offsets=None):
    """One fusion layer: a1..a5 in order [GS 2.1].  `p` holds W_Q, W_K, W_V,
    W_F, W_U, W_D and the norm parameters g_q, b_q, g_kv, b_kv, g_f, b_f;
    without W_V the layer shares one tensor as keys and values (R10), and
    with cand_offsets each request has its own number of candidates (R11).
    Returns a dict with every intermediate; 'Y' is the layer output (F when
    ffn is False)."""
    Q, K, V = proj_qkv(H_w, H_s, norm, eps, p["g_q"], p["b_q"], p["g_kv"], p["b_kv"],
                       p["W_Q"], p["W_K"], p.get("W_V"))
    A, lse = xattn_fwd(Q, K, V, offsets, C, n_q, h, scale, cand_offsets)
    F, Z = fusion_mlp(A, H_w, p["W_F"], act)
    out = {"Q": Q, "K": K, "V": V, "A": A, "lse": lse, "F": F, "Z": Z}
    if ffn:
        out["Y"], out["U"] = swiglu_ffn(F, norm, eps, p["g_f"], p["b_f"], p["W_U"], gate, p["W_D"])
    else:
        out["Y"] = F
    return out


def layer_bwd(H_w, H_s, offsets, C, n_q, h, p, dY, norm=NORM_LAYER, eps=1e-5,
              act=ACT_SILU, gate=GATE_SHARED, ffn=True, scale=None):
    """Exact chain rule of layer_fwd, step by step in reverse order.  Returns a
    dict of input gradients (dH_w, dH_s) and parameter gradients."""
    fw = layer_fwd(H_w, H_s, offsets, C, n_q, h, p, norm, eps, act, gate, ffn, scale)
    g = {}
    if ffn:
        fb = swiglu_ffn_bwd(fw["F"], norm, eps, p["g_f"], p["b_f"], p["W_U"], gate, p["W_D"], dY)
        dF = fb["dF"]
        g.update(dW_U=fb["dW_U"], dW_D=fb["dW_D"], dg_f=fb["dg_f"], db_f=fb["db_f"])
    else:
        dF = _f64(dY)
    dA, dH_w_mlp, g["dW_F"] = fusion_mlp_bwd(fw["A"], H_w, p["W_F"], act, dF)
    dQ, dK, dV = xattn_bwd(fw["Q"], fw["K"], fw["V"], offsets, C, n_q, h, scale, dA)
    W_V = p.get("W_V")
    if W_V is None:
        # One tensor in both roles: its gradient is the sum of the two (R10).
        dK, dV = dK + dV, None
    pb = proj_qkv_bwd(H_w, H_s, norm, eps, p["g_q"], p["b_q"], p["g_kv"], p["b_kv"],
                      p["W_Q"], p["W_K"], W_V, dQ, dK, dV)
    for k in ("dW_Q", "dW_K", "dW_V"):
        if k in pb:
            g[k] = pb[k]
    g["dH_w"] = dH_w_mlp + pb["dH_w"]
    g["dH_s"] = pb["dH_s"]
    g.update(dg_q=pb["dg_q"], db_q=pb["db_q"], dg_kv=pb["dg_kv"], db_kv=pb["db_kv"])
    g.update(dA=dA, dQ=dQ, dK=dK, dV=dV, dF=dF)
    return g


# ---------------------------------------------------------------- HSTU (NEXT f4)
#
# The pages describe the HSTU module, the producer of H_s, as sequential
# attention with relative position-and-time biases [PV km], [GS 2.1], but do
# not define the bias rab(p, t) (pith.science review page, referee minor
# comment 2 on Eq. (2), which points to the HSTU paper, reference [34]).
# Reading R12, the plainest one the pages and that reference support:
#   * per request b, history rows i, j in [0, L_b), per head: causal
#     (j <= i) pointwise attention, SiLU of the biased score in place of a
#     softmax, normalised by the request's length:
#       A_i = (1 / L_b) * sum_{j <= i} SiLU(scale * <q_i, k_j> + rab(i, j)) v_j
#   * rab(i, j) = w_pos[min(i - j, NP - 1)] + w_time[bucket(tau_i - tau_j)],
#     one position table [NP] and one time table [NT] shared by all heads;
#   * bucket(delta) = min(floor(log2(max(delta, 1))), NT - 1) on the integer
#     time difference (timestamps are int64; delta <= 1 gives bucket 0).

def time_bucket(delta, n_time):
    """floor(log2(max(delta, 1))) clipped to n_time - 1.  Below 2^53 the
    difference is exact in float64 and frexp's exponent e (x = m 2^e with
    0.5 <= m < 1) gives floor(log2 x) = e - 1 exactly; larger values take
    Python's integer bit length."""
    d = np.maximum(np.asarray(delta, dtype=np.int64), 1)
    _, e = np.frexp(d.astype(np.float64))
    out = e.astype(np.int64) - 1
    big = d >= 2 ** 53
    if big.any():
        out[big] = [int(v).bit_length() - 1 for v in d[big].tolist()]
    return np.minimum(out, n_time - 1)


def hstu_rab(ts, w_pos, w_time):
    """rab(i, j) of one request: [L, L] (entries with j > i are unused)."""
    ts = np.asarray(ts, dtype=np.int64)
    L = len(ts)
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    p = np.minimum(np.maximum(i - j, 0), len(w_pos) - 1)
    t = time_bucket(ts[:, None] - ts[None, :], len(w_time))
    return _f64(w_pos)[p] + _f64(w_time)[t]


def hstu_attn_fwd(Q, K, V, offsets, h, timestamps, w_pos, w_time, scale=None):
    """R12: causal pointwise (SiLU) jagged self-attention with relative
    position-and-time bias, per request and head.  Q, K, V [T, d]; returns
    A [T, d]."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    offsets = np.asarray(offsets, dtype=np.int64)
    T, d = Q.shape
    dh = d // h
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(dh)
    A = np.zeros((T, d))
    for b in range(len(offsets) - 1):
        lo, hi = offsets[b], offsets[b + 1]
        L = hi - lo
        if L == 0:
            continue
        rab = hstu_rab(np.asarray(timestamps)[lo:hi], w_pos, w_time)
        causal = np.tril(np.ones((L, L)))
        for j in range(h):
            cols = slice(j * dh, (j + 1) * dh)
            s = scale * (Q[lo:hi, cols] @ K[lo:hi, cols].T) + rab
            A[lo:hi, cols] = ((silu(s) * causal) @ V[lo:hi, cols]) / L
    return A
