"""ctypes binding of libwhalefuse: the C-ABI calls under the same names.

Argument marshalling only.  Tensors are torch device tensors owned by the
caller (torch provides device memory and the stream); every step of the path
runs in the library's HIP kernels.  There is no fallback: if the library is
missing, or a call returns an error status, this module raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwhalefuse.so")

F32, BF16 = 0, 1
NORM_LAYER, NORM_RMS, NORM_NONE = 0, 1, 2
ACT_SILU, ACT_NONE = 0, 1
GATE_SHARED, GATE_SEPARATE = 0, 1
STATUS = ["WHALE_OK", "WHALE_ERR_NULL", "WHALE_ERR_SHAPE", "WHALE_ERR_DTYPE", "WHALE_ERR_UNSUPPORTED",
          "WHALE_ERR_WORKSPACE", "WHALE_ERR_LAUNCH"]

# Every symbol declared in include/whalefuse.h.
EXPORTS = [
    "whale_status_string", "whale_version",
    "whale_proj_qkv", "whale_jagged_xattn_fwd", "whale_jagged_xattn_fwd_varc", "whale_fusion_mlp",
    "whale_swiglu_ffn_workspace_size", "whale_swiglu_ffn",
    "whale_jagged_xattn_bwd_workspace_size", "whale_jagged_xattn_bwd",
    "whale_fusion_mlp_bwd_workspace_size", "whale_fusion_mlp_bwd",
    "whale_swiglu_ffn_bwd_workspace_size", "whale_swiglu_ffn_bwd",
    "whale_proj_qkv_bwd_workspace_size", "whale_proj_qkv_bwd",
    "whale_mfma_peak_probe",
    "whale_validate_offsets", "whale_validate_timestamps", "whale_debug_checks", "whale_debug_status",
    "whale_jagged_xattn_bwd_noalloc",
    "whale_hstu_attn_fwd",
]
BAD_FIRST, BAD_ORDER, BAD_MAX_L, BAD_TOTAL, BAD_CAND_FIRST, BAD_CAND_ORDER, BAD_MAX_C = 1, 2, 4, 8, 16, 32, 64
BAD_TIME = 128


class WhaleDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("C", ctypes.c_int32), ("n_q", ctypes.c_int32), ("d", ctypes.c_int32),
                ("h", ctypes.c_int32), ("max_L", ctypes.c_int32), ("total_L", ctypes.c_int64)]


class WhaleError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed: {msg}")
        self.code = code


_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_D = ctypes.POINTER(WhaleDims)
_SIGS = {
    "whale_status_string": (ctypes.c_char_p, [_I]),
    "whale_version": (ctypes.c_char_p, []),
    "whale_proj_qkv": (_I, [_D, _I, _P, _P, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "whale_jagged_xattn_fwd": (_I, [_D, _I, _P, _P, _P, _P, _F, _P, _P, _P]),
    "whale_jagged_xattn_fwd_varc": (_I, [_D, _I, _P, _P, _P, _P, _P, _F, _P, _P, _P]),
    "whale_mfma_peak_probe": (_I, [_P, ctypes.c_int32, ctypes.c_int32, _P]),
    "whale_validate_offsets": (_I, [_D, _P, _P, _P, _P]),
    "whale_validate_timestamps": (_I, [_D, _P, _P, _P, _P]),
    "whale_hstu_attn_fwd": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, _F, _P, _P]),
    "whale_jagged_xattn_bwd_noalloc": (_I, [_D, _I, _P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _P, _P]),
    "whale_debug_checks": (ctypes.c_int32, [ctypes.c_int32]),
    "whale_debug_status": (_I, [_P, ctypes.c_int32, _P]),
    "whale_fusion_mlp": (_I, [_D, _I, _P, _P, _P, _I, _P, _P, _P]),
    "whale_swiglu_ffn_workspace_size": (_S, [_D, _I, _I, ctypes.c_int32]),
    "whale_swiglu_ffn": (_I, [_D, _I, _P, _I, _F, _P, _P, _P, _I, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _S, _P]),
    "whale_jagged_xattn_bwd_workspace_size": (_S, [_D, _I]),
    "whale_jagged_xattn_bwd": (_I, [_D, _I, _P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
    "whale_fusion_mlp_bwd_workspace_size": (_S, [_D, _I]),
    "whale_fusion_mlp_bwd": (_I, [_D, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _S, _P]),
    "whale_swiglu_ffn_bwd_workspace_size": (_S, [_D, _I, _I, ctypes.c_int32]),
    "whale_swiglu_ffn_bwd": (_I, [_D, _I, _P, _I, _F, _P, _P, _P, _P, _I, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P, _S, _P]),
    "whale_proj_qkv_bwd_workspace_size": (_S, [_D, _I]),
    "whale_proj_qkv_bwd": (_I, [_D, _I, _P, _P, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
}

_lib = None


def load():
    """Load libwhalefuse.so (built in-tree by __graft_entry__.build()).  Raises
    if it is missing: there is no other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def dims(B, C, n_q, d, h, max_L, total_L):
    return WhaleDims(int(B), int(C), int(n_q), int(d), int(h), int(max_L), int(total_L))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("libwhalefuse takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libwhalefuse takes contiguous tensors")
    return t.data_ptr()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(name, rc):
    if rc != 0:
        msg = load().whale_status_string(rc).decode()
        raise WhaleError(name, rc, msg)


def version():
    return load().whale_version().decode()


def status_string(code):
    return load().whale_status_string(code).decode()


def whale_proj_qkv(d_, H_w, H_s, norm, eps, g_q, b_q, g_kv, b_kv, W_Q, W_K, W_V, Q, K, V, stats_q, stats_kv,
                   X_q=None, X_s=None, stream=None):
    rc = load().whale_proj_qkv(ctypes.byref(d_), _dtype_code(H_w), _ptr(H_w), _ptr(H_s), norm, eps, _ptr(g_q),
                               _ptr(b_q), _ptr(g_kv), _ptr(b_kv), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(Q), _ptr(K),
                               _ptr(V), _ptr(stats_q), _ptr(stats_kv), _ptr(X_q), _ptr(X_s), _stream(stream))
    _check("whale_proj_qkv", rc)


def whale_jagged_xattn_fwd(d_, Q, K, V, offsets, scale, A, lse, stream=None):
    rc = load().whale_jagged_xattn_fwd(ctypes.byref(d_), _dtype_code(Q), _ptr(Q), _ptr(K), _ptr(V), _ptr(offsets),
                                       float(scale), _ptr(A), _ptr(lse), _stream(stream))
    _check("whale_jagged_xattn_fwd", rc)


def whale_jagged_xattn_fwd_varc(d_, Q, K, V, offsets, cand_offsets, scale, A, lse, stream=None):
    rc = load().whale_jagged_xattn_fwd_varc(ctypes.byref(d_), _dtype_code(Q), _ptr(Q), _ptr(K), _ptr(V),
                                            _ptr(offsets), _ptr(cand_offsets), float(scale), _ptr(A), _ptr(lse),
                                            _stream(stream))
    _check("whale_jagged_xattn_fwd_varc", rc)


def whale_mfma_peak_probe(out, iters, blocks, stream=None):
    """Launch the matrix-core rate probe (out: fp32 device tensor of blocks*256)."""
    if out.numel() < blocks * 256:
        raise ValueError("out needs blocks * 256 floats")
    rc = load().whale_mfma_peak_probe(_ptr(out), int(iters), int(blocks), _stream(stream))
    _check("whale_mfma_peak_probe", rc)


def whale_fusion_mlp(d_, A, H_w, W_F, act, F, Z_saved, stream=None):
    rc = load().whale_fusion_mlp(ctypes.byref(d_), _dtype_code(A), _ptr(A), _ptr(H_w), _ptr(W_F), act, _ptr(F),
                                 _ptr(Z_saved), _stream(stream))
    _check("whale_fusion_mlp", rc)


def whale_swiglu_ffn_workspace_size(d_, dtype_code, gate, H):
    return load().whale_swiglu_ffn_workspace_size(ctypes.byref(d_), dtype_code, gate, H)


def whale_swiglu_ffn(d_, F, norm, eps, g_f, b_f, W_U, gate, H, W_D, Y, U_saved, stats_f, workspace, stream=None,
                     X_f=None):
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().whale_swiglu_ffn(ctypes.byref(d_), _dtype_code(F), _ptr(F), norm, eps, _ptr(g_f), _ptr(b_f),
                                 _ptr(W_U), gate, H, _ptr(W_D), _ptr(Y), _ptr(U_saved), _ptr(stats_f), _ptr(X_f),
                                 _ptr(workspace), ws, _stream(stream))
    _check("whale_swiglu_ffn", rc)


def whale_jagged_xattn_bwd_workspace_size(d_, dtype_code):
    return load().whale_jagged_xattn_bwd_workspace_size(ctypes.byref(d_), dtype_code)


def whale_jagged_xattn_bwd(d_, Q, K, V, offsets, scale, A, lse, dA, dQ, dK, dV, workspace, stream=None):
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().whale_jagged_xattn_bwd(ctypes.byref(d_), _dtype_code(Q), _ptr(Q), _ptr(K), _ptr(V), _ptr(offsets),
                                       float(scale), _ptr(A), _ptr(lse), _ptr(dA), _ptr(dQ), _ptr(dK), _ptr(dV),
                                       _ptr(workspace), ws, _stream(stream))
    _check("whale_jagged_xattn_bwd", rc)


def whale_fusion_mlp_bwd_workspace_size(d_, dtype_code):
    return load().whale_fusion_mlp_bwd_workspace_size(ctypes.byref(d_), dtype_code)


def whale_fusion_mlp_bwd(d_, A, H_w, W_F, act, Z_saved, dF, dA, dH_w, dW_F, workspace, stream=None):
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().whale_fusion_mlp_bwd(ctypes.byref(d_), _dtype_code(A), _ptr(A), _ptr(H_w), _ptr(W_F), act,
                                     _ptr(Z_saved), _ptr(dF), _ptr(dA), _ptr(dH_w), _ptr(dW_F), _ptr(workspace), ws,
                                     _stream(stream))
    _check("whale_fusion_mlp_bwd", rc)


def whale_swiglu_ffn_bwd_workspace_size(d_, dtype_code, gate, H):
    return load().whale_swiglu_ffn_bwd_workspace_size(ctypes.byref(d_), dtype_code, gate, H)


def whale_swiglu_ffn_bwd(d_, F, norm, eps, g_f, b_f, stats_f, W_U, gate, H, W_D, U_saved, dY, dF, dW_U, dW_D, dg_f,
                         db_f, workspace, stream=None, X_f=None):
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().whale_swiglu_ffn_bwd(ctypes.byref(d_), _dtype_code(F), _ptr(F), norm, eps, _ptr(g_f), _ptr(b_f),
                                     _ptr(stats_f), _ptr(W_U), gate, H, _ptr(W_D), _ptr(U_saved), _ptr(X_f), _ptr(dY),
                                     _ptr(dF),
                                     _ptr(dW_U), _ptr(dW_D), _ptr(dg_f), _ptr(db_f), _ptr(workspace), ws,
                                     _stream(stream))
    _check("whale_swiglu_ffn_bwd", rc)


def whale_proj_qkv_bwd_workspace_size(d_, dtype_code):
    return load().whale_proj_qkv_bwd_workspace_size(ctypes.byref(d_), dtype_code)


def whale_proj_qkv_bwd(d_, H_w, H_s, norm, eps, g_q, b_q, g_kv, b_kv, stats_q, stats_kv, W_Q, W_K, W_V, dQ, dK, dV,
                       dH_w_in, dH_w, dH_s, dW_Q, dW_K, dW_V, dg_q, db_q, dg_kv, db_kv, workspace, X_q=None, X_s=None,
                       stream=None):
    ws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().whale_proj_qkv_bwd(ctypes.byref(d_), _dtype_code(H_w), _ptr(H_w), _ptr(H_s), norm, eps, _ptr(g_q),
                                   _ptr(b_q), _ptr(g_kv), _ptr(b_kv), _ptr(stats_q), _ptr(stats_kv), _ptr(X_q),
                                   _ptr(X_s), _ptr(W_Q),
                                   _ptr(W_K), _ptr(W_V), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dH_w_in), _ptr(dH_w),
                                   _ptr(dH_s), _ptr(dW_Q), _ptr(dW_K), _ptr(dW_V), _ptr(dg_q), _ptr(db_q),
                                   _ptr(dg_kv), _ptr(db_kv), _ptr(workspace), ws, _stream(stream))
    _check("whale_proj_qkv_bwd", rc)


def whale_validate_offsets(d_, offsets, cand_offsets, flag, stream=None):
    """flag: int32 device tensor with at least one element (receives the bitmask)."""
    if flag.dtype != torch.int32:
        raise TypeError("flag must be an int32 tensor")
    rc = load().whale_validate_offsets(ctypes.byref(d_), _ptr(offsets), _ptr(cand_offsets), _ptr(flag),
                                       _stream(stream))
    _check("whale_validate_offsets", rc)


def whale_validate_timestamps(d_, offsets, timestamps, flag, stream=None):
    """flag: int32 device tensor with at least one element (receives the bitmask)."""
    if flag.dtype != torch.int32:
        raise TypeError("flag must be an int32 tensor")
    rc = load().whale_validate_timestamps(ctypes.byref(d_), _ptr(offsets), _ptr(timestamps), _ptr(flag),
                                          _stream(stream))
    _check("whale_validate_timestamps", rc)


def whale_debug_checks(enable):
    """Turn debug mode on or off; returns the previous setting (0 / 1)."""
    return int(load().whale_debug_checks(1 if enable else 0))


def whale_debug_status(flag, reset=False, stream=None):
    if flag.dtype != torch.int32:
        raise TypeError("flag must be an int32 tensor")
    rc = load().whale_debug_status(_ptr(flag), 1 if reset else 0, _stream(stream))
    _check("whale_debug_status", rc)


def whale_jagged_xattn_bwd_noalloc(d_, Q, K, V, offsets, scale, A, lse, dA, dQ, dK, dV, stream=None):
    rc = load().whale_jagged_xattn_bwd_noalloc(ctypes.byref(d_), _dtype_code(Q), _ptr(Q), _ptr(K), _ptr(V),
                                               _ptr(offsets), float(scale), _ptr(A), _ptr(lse), _ptr(dA), _ptr(dQ),
                                               _ptr(dK), _ptr(dV), _stream(stream))
    _check("whale_jagged_xattn_bwd_noalloc", rc)


NOALLOC_SCRATCH_BYTES = 32 << 20   # the static scratch of whale_jagged_xattn_bwd_noalloc, per GPU


def whale_hstu_attn_fwd(d_, Q, K, V, offsets, timestamps, w_pos, w_time, scale, A, stream=None):
    """w_pos, w_time: fp32 device tensors (their lengths are n_pos, n_time)."""
    rc = load().whale_hstu_attn_fwd(ctypes.byref(d_), _dtype_code(Q), _ptr(Q), _ptr(K), _ptr(V), _ptr(offsets),
                                    _ptr(timestamps), _ptr(w_pos), int(w_pos.numel()), _ptr(w_time),
                                    int(w_time.numel()), float(scale), _ptr(A), _stream(stream))
    _check("whale_hstu_attn_fwd", rc)
