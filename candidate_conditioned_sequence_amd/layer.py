"""One WHALE fusion layer driven through the C ABI.

This only allocates buffers with torch and calls the libwhalefuse entry points
in the order of the module (gist.science Technical Summary §2.1): projections,
jagged cross-attention, fusion MLP, shared-gate SwiGLU FFN, and their
backward in reverse order.  No arithmetic of the module happens here.
"""
import torch

from . import binding as wb


def _empty(shape, dtype, dev):
    return torch.empty(shape, dtype=dtype, device=dev)


def _ws(nbytes, dev):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


class FusionLayer:
    """Weights are torch device tensors in the layer's dtype (W_Q, W_K, W_V,
    W_F, W_U, W_D); norm parameters are fp32 (g_q, b_q, g_kv, b_kv, g_f, b_f).
    Without W_V (absent or None) the layer shares one tensor as keys and
    values (gist.science Technical Summary §2.2, shared key-value)."""

    def __init__(self, params, C, n_q, h, norm=wb.NORM_LAYER, eps=1e-5, act=wb.ACT_SILU, gate=wb.GATE_SHARED,
                 ffn=True, scale=0.0):
        self.p = params
        self.C, self.n_q, self.h = C, n_q, h
        self.norm, self.eps, self.act, self.gate, self.ffn = norm, eps, act, gate, ffn
        self.scale = scale
        self.d = params["W_Q"].shape[0]
        self.H = params["W_D"].shape[1]
        self.tied_kv = params.get("W_V") is None
        self.ctx = None

    def dims(self, H_w, max_L, total_L):
        B = H_w.shape[0] // (self.C * self.n_q)
        return wb.dims(B, self.C, self.n_q, self.d, self.h, max_L, total_L)

    def forward(self, H_w, H_s, offsets, max_L, save=True, stream=None, cand_offsets=None, max_C=None):
        """cand_offsets (device int64 [B+1]) with its host hint max_C: the
        serving form, request b having cand_offsets[b+1] - cand_offsets[b]
        candidates (forward only).  The row-wise calls then see the query
        rows as one batch and only the attention call sees the requests."""
        p, dev, dt = self.p, H_w.device, H_w.dtype
        M, T, d = H_w.shape[0], H_s.shape[0], self.d
        # Host-side shape checks only (nothing is read from the device): the
        # kernels index H_w, H_s and the offsets by these sizes.
        if H_w.dim() != 2 or H_s.dim() != 2 or H_w.shape[1] != d or H_s.shape[1] != d:
            raise ValueError(f"H_w and H_s must be [rows, {d}]")
        for name, o in (("offsets", offsets), ("cand_offsets", cand_offsets)):
            if o is not None and (o.dtype != torch.int64 or o.dim() != 1 or not o.is_contiguous()
                                  or o.device != dev):
                raise ValueError(f"{name} must be a contiguous int64 vector on {dev}")
        if not 0 <= int(max_L) <= T:
            raise ValueError(f"max_L = {max_L} must lie in [0, {T}] (T = rows of H_s)")
        if cand_offsets is None:
            per = self.C * self.n_q
            if M == 0 or M % per != 0:
                raise ValueError(f"H_w has {M} rows, not a positive multiple of C*n_q = {per}")
            if offsets.shape[0] != M // per + 1:
                raise ValueError(f"offsets has {offsets.shape[0]} entries for B = {M // per} requests "
                                 f"(B + 1 expected)")
        if cand_offsets is not None:
            if save:
                raise ValueError("the form with candidate offsets is forward only (save=False)")
            if max_C is None or M % self.n_q != 0 or cand_offsets.shape != offsets.shape:
                raise ValueError("candidate offsets need max_C, n_q rows per candidate and one entry per "
                                 "history offset")
            B = offsets.shape[0] - 1
            dm = wb.dims(1, M // self.n_q, self.n_q, d, self.h, T, T)
            dm_att = wb.dims(B, max_C, self.n_q, d, self.h, max_L, T)
        else:
            dm = dm_att = self.dims(H_w, max_L, T)
        nn = self.norm != wb.NORM_NONE
        Q, K = _empty((M, d), dt, dev), _empty((T, d), dt, dev)
        V = None if self.tied_kv else _empty((T, d), dt, dev)
        sq = _empty((M, 2), torch.float32, dev) if nn else None
        skv = _empty((T, 2), torch.float32, dev) if nn else None
        # For the backward the normalised inputs are written once (the
        # projections then read them and the backward reuses them).  A
        # forward-only call does not keep them: the projections normalise on
        # the fly and write only the row statistics.
        Xq = _empty((M, d), dt, dev) if (nn and save) else None
        Xs = _empty((T, d), dt, dev) if (nn and save) else None
        wb.whale_proj_qkv(dm, H_w, H_s, self.norm, self.eps, p["g_q"], p["b_q"], p["g_kv"], p["b_kv"], p["W_Q"],
                          p["W_K"], p.get("W_V"), Q, K, V, sq, skv, Xq, Xs, stream)
        if self.tied_kv:
            V = K
        A, lse = _empty((M, d), dt, dev), _empty((M, self.h), torch.float32, dev)
        if cand_offsets is not None:
            wb.whale_jagged_xattn_fwd_varc(dm_att, Q, K, V, offsets, cand_offsets, self.scale, A, lse, stream)
        else:
            wb.whale_jagged_xattn_fwd(dm, Q, K, V, offsets, self.scale, A, lse, stream)
        F = _empty((M, d), dt, dev)
        Z = _empty((M, d), dt, dev) if (save and self.act == wb.ACT_SILU) else None
        wb.whale_fusion_mlp(dm, A, H_w, p["W_F"], self.act, F, Z, stream)
        out = dict(Q=Q, K=K, V=V, A=A, lse=lse, F=F, Z=Z, stats_q=sq, stats_kv=skv, X_q=Xq, X_s=Xs)
        if self.ffn:
            H = self.H
            Hu = 2 * H if self.gate == wb.GATE_SEPARATE else H
            Y = _empty((M, d), dt, dev)
            U = _empty((M, Hu), dt, dev) if save else None
            sf = _empty((M, 2), torch.float32, dev) if nn else None
            Xf = _empty((M, d), dt, dev) if (save and nn) else None
            ws = _ws(wb.whale_swiglu_ffn_workspace_size(dm, wb._dtype_code(F), self.gate, H), dev)
            wb.whale_swiglu_ffn(dm, F, self.norm, self.eps, p["g_f"], p["b_f"], p["W_U"], self.gate, H, p["W_D"], Y, U,
                                sf, ws, stream, X_f=Xf)
            out.update(Y=Y, U=U, stats_f=sf, X_f=Xf)
        else:
            out["Y"] = F
        if save:
            self.ctx = dict(out, H_w=H_w, H_s=H_s, offsets=offsets, dims=dm)
        return out

    def backward(self, dY, stream=None):
        c, p = self.ctx, self.p
        if c is None:
            raise RuntimeError("forward(save=True) must run before backward")
        dm, dev, dt = c["dims"], dY.device, dY.dtype
        code = wb._dtype_code(dY)
        M, d = dY.shape
        T = c["H_s"].shape[0]
        g = {}
        if self.ffn:
            dF = _empty((M, d), dt, dev)
            g["dW_U"] = _empty(tuple(p["W_U"].shape), torch.float32, dev)
            g["dW_D"] = _empty(tuple(p["W_D"].shape), torch.float32, dev)
            g["dg_f"], g["db_f"] = _empty((d,), torch.float32, dev), _empty((d,), torch.float32, dev)
            ws = _ws(wb.whale_swiglu_ffn_bwd_workspace_size(dm, code, self.gate, self.H), dev)
            wb.whale_swiglu_ffn_bwd(dm, c["F"], self.norm, self.eps, p["g_f"], p["b_f"], c["stats_f"], p["W_U"],
                                    self.gate, self.H, p["W_D"], c["U"], dY, dF, g["dW_U"], g["dW_D"], g["dg_f"],
                                    g["db_f"], ws, stream, X_f=c.get("X_f"))
        else:
            dF = dY
        dA, dHw_mlp = _empty((M, d), dt, dev), _empty((M, d), dt, dev)
        g["dW_F"] = _empty(tuple(p["W_F"].shape), torch.float32, dev)
        ws = _ws(wb.whale_fusion_mlp_bwd_workspace_size(dm, code), dev)
        wb.whale_fusion_mlp_bwd(dm, c["A"], c["H_w"], p["W_F"], self.act, c["Z"], dF, dA, dHw_mlp, g["dW_F"], ws,
                                stream)
        dQ, dK = _empty((M, d), dt, dev), _empty((T, d), dt, dev)
        dV = None if self.tied_kv else _empty((T, d), dt, dev)
        ws = _ws(wb.whale_jagged_xattn_bwd_workspace_size(dm, code), dev)
        wb.whale_jagged_xattn_bwd(dm, c["Q"], c["K"], c["V"], c["offsets"], self.scale, c["A"], c["lse"], dA, dQ, dK,
                                  dV, ws, stream)
        g["dH_w"], g["dH_s"] = _empty((M, d), dt, dev), _empty((T, d), dt, dev)
        for k in ("dW_Q", "dW_K") + (() if self.tied_kv else ("dW_V",)):
            g[k] = _empty((d, d), torch.float32, dev)
        for k in ("dg_q", "db_q", "dg_kv", "db_kv"):
            g[k] = _empty((d,), torch.float32, dev)
        ws = _ws(wb.whale_proj_qkv_bwd_workspace_size(dm, code), dev)
        wb.whale_proj_qkv_bwd(dm, c["H_w"], c["H_s"], self.norm, self.eps, p["g_q"], p["b_q"], p["g_kv"], p["b_kv"],
                              c["stats_q"], c["stats_kv"], p["W_Q"], p["W_K"], p.get("W_V"), dQ, dK, dV, dHw_mlp,
                              g["dH_w"], g["dH_s"], g["dW_Q"], g["dW_K"], g.get("dW_V"), g["dg_q"], g["db_q"], g["dg_kv"],
                              g["db_kv"], ws, c.get("X_q"), c.get("X_s"), stream)
        g.update(dA=dA, dQ=dQ, dK=dK, dV=dV, dF=dF)
        return g
