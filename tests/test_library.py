"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before enqueueing anything."""
import ctypes
import os
import re

import pytest

from candidate_conditioned_sequence_amd import binding as wb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "whalefuse.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(whale_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert header_functions() == sorted(wb.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = wb.load()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert wb.version().count(".") == 2


def test_status_strings():
    for code, name in enumerate(wb.STATUS):
        assert wb.status_string(code).startswith(name)


def _dims(**kw):
    base = dict(B=2, C=4, n_q=8, d=128, h=2, max_L=100, total_L=150)
    base.update(kw)
    return wb.dims(**base)


def test_host_validation_rejects_before_launch():
    lib = wb.load()
    fake = ctypes.c_void_p(256)      # never dereferenced: validation fails first
    d = _dims()
    # NULL dims, bad dtype
    assert lib.whale_jagged_xattn_fwd(None, 1, fake, fake, fake, fake, 0.0, fake, None, None) == 1
    assert lib.whale_jagged_xattn_fwd(ctypes.byref(d), 7, fake, fake, fake, fake, 0.0, fake, None, None) == 3
    # NULL required pointer
    assert lib.whale_jagged_xattn_fwd(ctypes.byref(d), 1, None, fake, fake, fake, 0.0, fake, None, None) == 1
    # d % h != 0, shape hints inconsistent, negative scale
    for bad in (_dims(h=3), _dims(max_L=200, total_L=150), _dims(max_L=10, total_L=150), _dims(B=0)):
        assert lib.whale_jagged_xattn_fwd(ctypes.byref(bad), 1, fake, fake, fake, fake, 0.0, fake, None, None) == 2
    assert lib.whale_jagged_xattn_fwd(ctypes.byref(d), 1, fake, fake, fake, fake, -1.0, fake, None, None) == 2
    # unsupported head widths (d_h = 16, 256) and width above 512
    for bad in (_dims(d=64, h=4), _dims(d=512, h=2), _dims(d=1024, h=16)):
        assert lib.whale_jagged_xattn_fwd(ctypes.byref(bad), 1, fake, fake, fake, fake, 0.0, fake, None, None) == 4
    # d_h = 128 passes the host checks (it fails on the NULL output instead)
    assert lib.whale_jagged_xattn_fwd(ctypes.byref(_dims(d=256, h=2)), 1, fake, fake, fake, fake, 0.0, None, None,
                                      None) == 1
    # FFN hidden width not a multiple of 64, workspace too small
    assert lib.whale_swiglu_ffn(ctypes.byref(d), 1, fake, 0, 1e-5, fake, fake, fake, 0, 100, fake, fake, None, fake,
                                None, fake, 1 << 30, None) == 4
    assert lib.whale_swiglu_ffn(ctypes.byref(d), 1, fake, 0, 1e-5, fake, fake, fake, 0, 512, fake, fake, None, fake,
                                None, fake, 16, None) == 5
    # LayerNorm without its statistics buffer
    assert lib.whale_proj_qkv(ctypes.byref(d), 1, fake, fake, 0, 1e-5, fake, fake, fake, fake, fake, fake, fake, fake,
                              fake, fake, None, fake, None, None, None) == 1
    # Matrix-core probe: NULL output, no iterations or no workgroups
    assert lib.whale_mfma_peak_probe(None, 10, 1, None) == 1
    assert lib.whale_mfma_peak_probe(fake, 0, 1, None) == 2
    assert lib.whale_mfma_peak_probe(fake, 10, 0, None) == 2
    # Shared key-value form: W_V and V must be NULL together; a NULL dV needs V == K
    assert lib.whale_proj_qkv(ctypes.byref(d), 1, fake, fake, 2, 1e-5, None, None, None, None, fake, fake, None, fake,
                              fake, fake, None, None, None, None, None) == 1
    other = ctypes.c_void_p(512)
    assert lib.whale_jagged_xattn_bwd(ctypes.byref(d), 1, fake, fake, other, fake, 0.0, fake, fake, fake, fake, fake,
                                      None, fake, 1 << 30, None) == 2
    assert lib.whale_proj_qkv_bwd(ctypes.byref(d), 1, fake, fake, 2, 1e-5, None, None, None, None, None, None, None,
                                  None, fake, fake, None, fake, fake, fake, None, fake, fake, fake, fake, None, None,
                                  None, None, None, fake, 1 << 30, None) == 1


def test_workspace_sizes_are_host_only_and_monotone():
    lib = wb.load()
    small, big = _dims(), _dims(B=8, total_L=600)
    for fn in ("whale_jagged_xattn_bwd_workspace_size", "whale_fusion_mlp_bwd_workspace_size",
               "whale_proj_qkv_bwd_workspace_size"):
        f = getattr(lib, fn)
        a, b = f(ctypes.byref(small), 1), f(ctypes.byref(big), 1)
        assert 0 < a <= b, fn
    assert lib.whale_swiglu_ffn_bwd_workspace_size(ctypes.byref(small), 1, 0, 512) > 0
    assert lib.whale_swiglu_ffn_workspace_size(ctypes.byref(small), 1, 1, 512) == \
        lib.whale_swiglu_ffn_workspace_size(ctypes.byref(small), 1, 0, 512)


def test_validator_host_checks():
    lib = wb.load()
    fake = ctypes.c_void_p(256)
    d = _dims()
    assert lib.whale_validate_offsets(None, fake, None, fake, None) == 1
    assert lib.whale_validate_offsets(ctypes.byref(d), None, None, fake, None) == 1
    assert lib.whale_validate_offsets(ctypes.byref(d), fake, None, None, None) == 1
    for bad in (_dims(B=0), _dims(C=0), _dims(max_L=-1)):
        assert lib.whale_validate_offsets(ctypes.byref(bad), fake, None, fake, None) == 2
    # the timestamps check: every pointer required (no device work is reached)
    assert lib.whale_validate_timestamps(None, fake, fake, fake, None) == 1
    assert lib.whale_validate_timestamps(ctypes.byref(d), None, fake, fake, None) == 1
    assert lib.whale_validate_timestamps(ctypes.byref(d), fake, None, fake, None) == 1
    assert lib.whale_validate_timestamps(ctypes.byref(d), fake, fake, None, None) == 1
    for bad in (_dims(B=0), _dims(C=0), _dims(max_L=-1), _dims(total_L=-1)):
        assert lib.whale_validate_timestamps(ctypes.byref(bad), fake, fake, fake, None) == 2
    assert lib.whale_debug_status(None, 0, None) == 1


def test_debug_switch_round_trip():
    prev = wb.whale_debug_checks(True)
    try:
        assert wb.whale_debug_checks(False) == 1
        assert wb.whale_debug_checks(False) == 0
    finally:
        wb.whale_debug_checks(prev)


def test_layer_rejects_inconsistent_shapes_on_the_host():
    """FusionLayer.forward checks sizes on the host before any call (CPU
    tensors suffice: the checks run first)."""
    import torch
    from candidate_conditioned_sequence_amd.layer import FusionLayer
    d, C, n_q = 64, 2, 3
    p = {k: torch.zeros(d, d) for k in ("W_Q", "W_K", "W_V")}
    p.update(W_F=torch.zeros(d, 2 * d), W_U=torch.zeros(4 * d, d), W_D=torch.zeros(d, 4 * d))
    lay = FusionLayer(p, C, n_q, 2)
    Hw, Hs = torch.zeros(2 * C * n_q, d), torch.zeros(10, d)
    off = torch.tensor([0, 4, 10])
    with pytest.raises(ValueError, match="multiple of C\\*n_q"):
        lay.forward(Hw[:-1], Hs, off, 6)
    with pytest.raises(ValueError, match="B \\+ 1 expected"):
        lay.forward(Hw, Hs, off[:2], 6)
    with pytest.raises(ValueError, match="int64"):
        lay.forward(Hw, Hs, off.to(torch.int32), 6)
    with pytest.raises(ValueError, match="max_L"):
        lay.forward(Hw, Hs, off, 11)
    with pytest.raises(ValueError, match="rows"):
        lay.forward(Hw[:, :32], Hs, off, 6)


def test_noalloc_backward_rejects_shapes_beyond_its_scratch():
    """The no-alloc backward decides on the host, from the dims alone, that a
    workspace larger than its static scratch does not fit."""
    lib = wb.load()
    fake = ctypes.c_void_p(256)
    big = _dims(B=2048, C=64, n_q=32, d=256, h=4, max_L=100, total_L=1000)     # M*h*4 = 64 MiB
    assert lib.whale_jagged_xattn_bwd_workspace_size(ctypes.byref(big), 1) > wb.NOALLOC_SCRATCH_BYTES
    assert lib.whale_jagged_xattn_bwd_noalloc(ctypes.byref(big), 1, fake, fake, fake, fake, 0.0, fake, fake, fake,
                                              fake, fake, fake, None) == 5
    assert lib.whale_jagged_xattn_bwd_noalloc(ctypes.byref(_dims()), 1, None, fake, fake, fake, 0.0, fake, fake,
                                              fake, fake, fake, fake, None) == 1
