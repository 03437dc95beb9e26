"""whale_jagged_xattn_bwd_noalloc (the attention backward whose workspace is
the library's static device scratch) against whale_jagged_xattn_bwd with a
caller workspace, through the C ABI: bit for bit, and both against the fp64
oracle, on calls in a row whose sizes shrink (the scratch keeps the previous
call's contents)."""
import numpy as np
import pytest
import torch

from candidate_conditioned_sequence_amd import binding as wb
from candidate_conditioned_sequence_amd import synth
from oracle import whale_oracle as O
from tests.util import assert_close, i64_dev, to_dev

pytestmark = pytest.mark.gpu


def _draw(seed, shape):
    return synth.round_bf16(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


def _one(gpu, L, C, n_q, d, h, seed, tied=False):
    B = len(L)
    M, off = B * C * n_q, synth.offsets_of(L)
    T = int(off[-1])
    Q, K, dA = _draw(seed, (M, d)), _draw(seed + 1, (T, d)), _draw(seed + 3, (M, d))
    V = K if tied else _draw(seed + 2, (T, d))
    dm = wb.dims(B, C, n_q, d, h, max(L), T)
    tQ, tK, tdA = (to_dev(x, "bf16", gpu) for x in (Q, K, dA))
    tV = tK if tied else to_dev(V, "bf16", gpu)
    toff = i64_dev(off, gpu)
    A, lse = torch.empty_like(tQ), torch.empty((M, h), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, tQ, tK, tV, toff, 0.0, A, lse)

    def outs():
        return torch.full_like(tQ, float("nan")), torch.full_like(tK, float("nan")), \
            (None if tied else torch.full_like(tV, float("nan")))

    rQ, rK, rV = outs()
    ws = torch.empty(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb.BF16), dtype=torch.uint8, device=gpu)
    wb.whale_jagged_xattn_bwd(dm, tQ, tK, tV, toff, 0.0, A, lse, tdA, rQ, rK, rV, ws)
    gQ, gK, gV = outs()
    wb.whale_jagged_xattn_bwd_noalloc(dm, tQ, tK, tV, toff, 0.0, A, lse, tdA, gQ, gK, gV)
    torch.cuda.synchronize()
    assert torch.equal(gQ, rQ) and torch.equal(gK, rK)
    if not tied:
        assert torch.equal(gV, rV)
    dQ_ref, dK_ref, dV_ref = O.xattn_bwd(Q, K, V, off, C, n_q, h, None, dA)
    assert_close("dQ", gQ, dQ_ref, "bf16")
    assert_close("dK" if not tied else "dK+dV", gK, dK_ref if not tied else dK_ref + dV_ref, "bf16")
    if not tied:
        assert_close("dV", gV, dV_ref, "bf16")


def test_noalloc_matches_workspace_call_on_shrinking_calls(gpu):
    # 1: split query ranges (fp32 partials in the scratch), ragged and empty
    #    histories; 2: a smaller shape, no split; 3: smaller still, shared K = V.
    for i, (L, C, n_q, d, h, tied) in enumerate([([130, 1, 700, 64, 0], 20, 15, 256, 4, False),
                                                 ([97, 40], 8, 16, 128, 4, False),
                                                 ([33, 5], 4, 8, 128, 2, True)]):
        print(f"\n[noalloc] call {i}: L={L} C={C} n_q={n_q} d={d} h={h} tied={tied}", flush=True)
        _one(gpu, L, C, n_q, d, h, seed=100 + 10 * i, tied=tied)
