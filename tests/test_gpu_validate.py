"""Device-side validation of the jagged offsets against the host shape hints
(whale_validate_offsets) and of the HSTU call's timestamps
(whale_validate_timestamps), and debug mode, in which the attention calls
run those checks first and skip their kernels when they fail.

Bad offsets are only ever handed to the validator itself.  The one test that
runs attention kernels in debug mode with failing offsets uses offsets whose
rows all lie inside the buffers (offsets[B] below the total_L hint): the
kernels would stay in bounds even if they ran."""
import numpy as np
import pytest
import torch

from candidate_conditioned_sequence_amd import binding as wb
from tests.util import i64_dev

pytestmark = pytest.mark.gpu


def check(gpu, off, max_L, total_L, C=4, coff=None):
    flag = torch.full((1,), -1, dtype=torch.int32, device=gpu)
    B = len(off) - 1
    dm = wb.dims(B, C, 2, 64, 2, max_L, total_L)
    wb.whale_validate_offsets(dm, i64_dev(off, gpu), None if coff is None else i64_dev(coff, gpu), flag)
    torch.cuda.synchronize()
    return int(flag.item())


def test_valid_offsets_give_zero(gpu):
    print("\n[validate] valid offsets", flush=True)
    assert check(gpu, [0, 5, 5, 12], 7, 12) == 0
    assert check(gpu, [0, 5, 5, 12], 7, 12, C=3, coff=[0, 3, 3, 5]) == 0
    assert check(gpu, [0, 0], 0, 0) == 0


@pytest.mark.parametrize("off,max_L,total_L,coff,C,want", [
    ([1, 5, 12], 7, 12, None, 4, wb.BAD_FIRST),
    ([0, 5, 4, 12], 8, 12, None, 4, wb.BAD_ORDER),
    ([0, 5, 13], 7, 13, None, 4, wb.BAD_MAX_L),
    ([0, 5, 12], 7, 11, None, 4, wb.BAD_TOTAL),
    ([0, 5, 12], 7, 12, [1, 2, 4], 4, wb.BAD_CAND_FIRST),
    ([0, 5, 12], 7, 12, [0, 3, 2], 4, wb.BAD_CAND_ORDER),
    ([0, 5, 12], 7, 12, [0, 5, 6], 4, wb.BAD_MAX_C),
    ([2, 1, 20], 7, 19, [0, 9, 8], 4, wb.BAD_FIRST | wb.BAD_ORDER | wb.BAD_MAX_L | wb.BAD_TOTAL | wb.BAD_MAX_C
     | wb.BAD_CAND_ORDER),
])
def test_each_violation_sets_its_bit(gpu, off, max_L, total_L, coff, C, want):
    print(f"\n[validate] off={off} max_L={max_L} total_L={total_L} coff={coff} C={C}", flush=True)
    assert check(gpu, off, max_L, total_L, C=C, coff=coff) == want


def test_violation_far_into_a_long_batch(gpu):
    """B = 1000 requests (four waves, several per thread): one bad request
    near the end, in another wave than thread 0's."""
    print("\n[validate] B=1000", flush=True)
    L = np.full(1000, 3)
    off = np.concatenate([[0], np.cumsum(L)])
    assert check(gpu, off, 3, int(off[-1])) == 0
    bad = off.copy()
    bad[778:] += 2                        # request 777 has L = 5 > max_L = 3
    assert check(gpu, bad, 3, int(bad[-1])) == wb.BAD_MAX_L


def _attn_inputs(gpu, L, T_alloc, d=128, h=2, C=3, n_q=5):
    r = np.random.default_rng(5)
    M = len(L) * C * n_q
    Q = torch.from_numpy(r.standard_normal((M, d)).astype(np.float32)).to(gpu).to(torch.bfloat16)
    K = torch.from_numpy(r.standard_normal((T_alloc, d)).astype(np.float32)).to(gpu).to(torch.bfloat16)
    V = torch.from_numpy(r.standard_normal((T_alloc, d)).astype(np.float32)).to(gpu).to(torch.bfloat16)
    dA = torch.from_numpy(r.standard_normal((M, d)).astype(np.float32)).to(gpu).to(torch.bfloat16)
    return Q, K, V, dA, C, n_q, d, h


def _run_attention(gpu, dm, Q, K, V, dA, toff, h):
    M = Q.shape[0]
    A = torch.full_like(Q, float("nan"))
    lse = torch.full((M, h), float("nan"), device=gpu)
    wb.whale_jagged_xattn_fwd(dm, Q, K, V, toff, 0.0, A, lse)
    dQ, dK, dV = (torch.full_like(x, float("nan")) for x in (Q, K, V))
    ws = torch.empty(wb.whale_jagged_xattn_bwd_workspace_size(dm, wb.BF16), dtype=torch.uint8, device=gpu)
    wb.whale_jagged_xattn_bwd(dm, Q, K, V, toff, 0.0, A, lse, dA, dQ, dK, dV, ws)
    torch.cuda.synchronize()
    return A, lse, dQ, dK, dV


def test_debug_mode_valid_offsets_same_bits(gpu):
    """Debug mode with consistent offsets: the same bits as without it, and
    a clean flag."""
    L = [70, 0, 129]
    off = np.concatenate([[0], np.cumsum(L)])
    T = int(off[-1])
    Q, K, V, dA, C, n_q, d, h = _attn_inputs(gpu, L, T)
    dm = wb.dims(len(L), C, n_q, d, h, max(L), T)
    toff = i64_dev(off, gpu)
    print("\n[debug mode] valid offsets", flush=True)
    ref = _run_attention(gpu, dm, Q, K, V, dA, toff, h)
    flag = torch.full((1,), -1, dtype=torch.int32, device=gpu)
    prev = wb.whale_debug_checks(True)
    try:
        wb.whale_debug_status(flag, reset=True)
        got = _run_attention(gpu, dm, Q, K, V, dA, toff, h)
        wb.whale_debug_status(flag)
        torch.cuda.synchronize()
    finally:
        wb.whale_debug_checks(prev)
    assert int(flag.item()) == 0
    for a, b in zip(got, ref):
        assert torch.equal(torch.nan_to_num(a, nan=7.0), torch.nan_to_num(b, nan=7.0))


def test_debug_mode_skips_kernels_on_failed_check(gpu):
    """offsets[B] = 10 below the total_L hint 12 (every row the kernels could
    touch lies inside the 12-row buffers): debug mode flags it and the
    attention kernels leave their outputs untouched."""
    L = [5, 5]
    off = np.array([0, 5, 10])
    Q, K, V, dA, C, n_q, d, h = _attn_inputs(gpu, L, 12)
    dm = wb.dims(2, C, n_q, d, h, 6, 12)
    toff = i64_dev(off, gpu)
    flag = torch.full((1,), -1, dtype=torch.int32, device=gpu)
    print("\n[debug mode] offsets[B] != total_L", flush=True)
    prev = wb.whale_debug_checks(True)
    try:
        wb.whale_debug_status(flag, reset=True)
        A, lse, dQ, dK, dV = _run_attention(gpu, dm, Q, K, V, dA, toff, h)
        wb.whale_debug_status(flag, reset=True)
        torch.cuda.synchronize()
        assert int(flag.item()) == wb.BAD_TOTAL
        for t in (A, lse, dQ, dK, dV):
            assert torch.isnan(t.float()).all()
        wb.whale_debug_status(flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0          # cleared by the reset
    finally:
        wb.whale_debug_checks(prev)


# ---------------------------------------------------------------- timestamps
# whale_validate_timestamps: the offsets check plus the HSTU call's contract
# (every timestamp of a request within 2^30 of the request's first).

def check_ts(gpu, off, ts, max_L, total_L):
    flag = torch.full((1,), -1, dtype=torch.int32, device=gpu)
    dm = wb.dims(len(off) - 1, 1, 1, 64, 1, max_L, total_L)
    wb.whale_validate_timestamps(dm, i64_dev(off, gpu), i64_dev(np.asarray(ts, dtype=np.int64), gpu), flag)
    torch.cuda.synchronize()
    return int(flag.item())


def test_timestamp_contract_boundaries(gpu):
    """Differences of 2^30 - 1 either way pass; 2^30 either way is flagged;
    int64 extremes are flagged without overflow; an empty request reads
    nothing."""
    print("\n[validate ts] boundaries", flush=True)
    t0, lim = 1_700_000_000, 2 ** 30
    off = [0, 3, 3, 6]
    ok = [t0, t0 + lim - 1, t0 - (lim - 1), 5, 5 + lim - 1, 5]
    assert check_ts(gpu, off, ok, 3, 6) == 0
    assert check_ts(gpu, off, [t0, t0 + lim, t0, 5, 5, 5], 3, 6) == wb.BAD_TIME
    assert check_ts(gpu, off, [t0, t0, t0, 5, 5 - lim, 5], 3, 6) == wb.BAD_TIME
    i64 = np.iinfo(np.int64)
    assert check_ts(gpu, off, [i64.max, i64.min, i64.max, 0, 0, 0], 3, 6) == wb.BAD_TIME
    assert check_ts(gpu, [0, 2], [i64.min, i64.min + lim - 1], 2, 2) == 0


def test_timestamp_violation_deep_in_a_long_batch(gpu):
    """B = 1000 requests of 300 rows (several rows per thread): one bad row
    in request 777."""
    print("\n[validate ts] B=1000", flush=True)
    L = np.full(1000, 300)
    off = np.concatenate([[0], np.cumsum(L)])
    ts = np.repeat(np.arange(1000, dtype=np.int64) * 10 ** 12, 300) + np.tile(np.arange(300), 1000)
    assert check_ts(gpu, off, ts, 300, int(off[-1])) == 0
    ts[777 * 300 + 211] += 2 ** 30
    assert check_ts(gpu, off, ts, 300, int(off[-1])) == wb.BAD_TIME


def test_timestamp_check_reads_no_row_past_total_L(gpu):
    """offsets[B] above the total_L hint (and a decreasing pair): the offsets
    bits are set, and the rows past total_L (not allocated) are not read:
    the last request is skipped, so no timestamp bit either."""
    print("\n[validate ts] bad offsets", flush=True)
    assert check_ts(gpu, [0, 4, 9], np.arange(8), 5, 8) == wb.BAD_TOTAL
    assert check_ts(gpu, [0, 5, 3, 8], np.arange(8), 5, 8) == wb.BAD_ORDER


def _hstu(gpu, dm, Q, K, V, toff, tts, wp, wt):
    A = torch.full_like(Q, float("nan"))
    wb.whale_hstu_attn_fwd(dm, Q, K, V, toff, tts, wp, wt, 0.0, A)
    torch.cuda.synchronize()
    return A


def test_debug_mode_hstu_timestamps(gpu):
    """Debug mode on the HSTU call: valid timestamps give the same bits as
    without it and a clean flag; a timestamp 2^30 past its request's first
    is flagged and the kernel leaves its output untouched."""
    print("\n[debug mode] hstu timestamps", flush=True)
    L, d, h = [70, 0, 129], 128, 2
    off = np.concatenate([[0], np.cumsum(L)])
    T = int(off[-1])
    r = np.random.default_rng(8)
    Q, K, V = (torch.from_numpy(r.standard_normal((T, d)).astype(np.float32)).to(gpu).to(torch.bfloat16)
               for _ in range(3))
    ts = np.concatenate([1_700_000_000 + np.cumsum(r.integers(0, 5000, n)) for n in L]).astype(np.int64)
    wp = torch.from_numpy(0.3 * r.standard_normal(100).astype(np.float32)).to(gpu)
    wt = torch.from_numpy(0.3 * r.standard_normal(20).astype(np.float32)).to(gpu)
    dm = wb.dims(len(L), 1, 1, d, h, max(L), T)
    toff, tts = i64_dev(off, gpu), i64_dev(ts, gpu)
    ref = _hstu(gpu, dm, Q, K, V, toff, tts, wp, wt)
    flag = torch.full((1,), -1, dtype=torch.int32, device=gpu)
    bad = ts.copy()
    bad[off[2] + 100] = bad[off[2]] + 2 ** 30
    prev = wb.whale_debug_checks(True)
    try:
        wb.whale_debug_status(flag, reset=True)
        got = _hstu(gpu, dm, Q, K, V, toff, tts, wp, wt)
        wb.whale_debug_status(flag, reset=True)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        assert torch.equal(got, ref)
        A = _hstu(gpu, dm, Q, K, V, toff, i64_dev(bad, gpu), wp, wt)
        wb.whale_debug_status(flag, reset=True)
        torch.cuda.synchronize()
        assert int(flag.item()) == wb.BAD_TIME
        assert torch.isnan(A.float()).all()
    finally:
        wb.whale_debug_checks(prev)
