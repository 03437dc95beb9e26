"""Pins of the oracle's HSTU self-attention (reading R12: causal pointwise
SiLU attention with a relative position bias and a log2-bucketed time bias,
normalised by the history length) against things other than itself: a
hand-derived bucket table and a loop definition of the bucket, an
independent torch fp64 formulation (float log2 for the buckets), brute force
with math.fsum, closed forms (prefix sums, the bias read back through an
identity V), causality, and planted mistakes.  CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import whale_oracle as O


def _case(seed, lengths=(7, 1, 0, 12), d=16, h=2, n_pos=6, n_time=8):
    r = np.random.default_rng(seed)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    Q, K, V = (r.standard_normal((T, d)) for _ in range(3))
    ts = np.zeros(T, np.int64)
    for b in range(len(lengths)):
        gaps = r.integers(0, 400, lengths[b])
        ts[off[b]:off[b + 1]] = 1_700_000_000 + np.cumsum(gaps)
    w_pos, w_time = 0.3 * r.standard_normal(n_pos), 0.3 * r.standard_normal(n_time)
    return dict(Q=Q, K=K, V=V, off=off, ts=ts, w_pos=w_pos, w_time=w_time, h=h, d=d)


def test_time_bucket_hand_table_and_loop_definition():
    # floor(log2(max(delta, 1))) clipped to NT - 1, derived by hand
    table = {-5: 0, 0: 0, 1: 0, 2: 1, 3: 1, 4: 2, 7: 2, 8: 3, 1000: 9, 1023: 9, 1024: 10, 2 ** 40: 31}
    got = O.time_bucket(np.array(list(table)), 32)
    assert got.tolist() == list(table.values())
    # the largest b with 2^b <= max(delta, 1), by a loop
    r = np.random.default_rng(3)
    deltas = np.concatenate([np.arange(-3, 4100), r.integers(0, 2 ** 45, 500)])
    for nt in (5, 64):
        want = []
        for dv in deltas.tolist():
            x, b = max(dv, 1), 0
            while 2 ** (b + 1) <= x:
                b += 1
            want.append(min(b, nt - 1))
        np.testing.assert_array_equal(O.time_bucket(deltas, nt), want)


def _torch_hstu(c, scale=None):
    """Independent torch fp64 formulation (buckets through float log2)."""
    Q, K, V = (torch.as_tensor(c[k], dtype=torch.float64) for k in ("Q", "K", "V"))
    off, ts, h, d = c["off"], torch.as_tensor(c["ts"]), c["h"], c["d"]
    wp, wt = torch.as_tensor(c["w_pos"]), torch.as_tensor(c["w_time"])
    dh = d // h
    scale = 1 / math.sqrt(dh) if scale is None else scale
    out = torch.zeros_like(Q)
    for b in range(len(off) - 1):
        lo, hi = int(off[b]), int(off[b + 1])
        L = hi - lo
        if L == 0:
            continue
        idx = torch.arange(L)
        rel = (idx[:, None] - idx[None, :]).clamp(0, len(wp) - 1)
        dt = (ts[lo:hi, None] - ts[None, lo:hi]).clamp(min=1).double()
        bucket = torch.floor(torch.log2(dt)).long().clamp(max=len(wt) - 1)
        rab = wp[rel] + wt[bucket]
        mask = torch.tril(torch.ones(L, L, dtype=torch.float64))
        for j in range(h):
            cs = slice(j * dh, (j + 1) * dh)
            s = scale * Q[lo:hi, cs] @ K[lo:hi, cs].T + rab
            out[lo:hi, cs] = (TF.silu(s) * mask) @ V[lo:hi, cs] / L
    return out.numpy()


@pytest.mark.parametrize("seed", [1, 2])
def test_hstu_matches_torch_formulation(seed):
    c = _case(seed)
    A = O.hstu_attn_fwd(c["Q"], c["K"], c["V"], c["off"], c["h"], c["ts"], c["w_pos"], c["w_time"])
    np.testing.assert_allclose(A, _torch_hstu(c), rtol=1e-12, atol=1e-13)


def test_hstu_brute_force_fsum():
    c = _case(5, lengths=(5, 3), d=4, h=2)
    A = O.hstu_attn_fwd(c["Q"], c["K"], c["V"], c["off"], c["h"], c["ts"], c["w_pos"], c["w_time"])
    dh = 2
    for b in range(2):
        lo, L = int(c["off"][b]), int(c["off"][b + 1] - c["off"][b])
        for i in range(L):
            for hd in range(2):
                for e in range(dh):
                    terms = []
                    for j in range(i + 1):
                        s = sum(c["Q"][lo + i, hd * dh + u] * c["K"][lo + j, hd * dh + u] for u in range(dh))
                        s = s / math.sqrt(dh)
                        dt = max(int(c["ts"][lo + i] - c["ts"][lo + j]), 1)
                        bk = min(dt.bit_length() - 1, len(c["w_time"]) - 1)
                        s += c["w_pos"][min(i - j, len(c["w_pos"]) - 1)] + c["w_time"][bk]
                        terms.append(s / (1 + math.exp(-s)) * c["V"][lo + j, hd * dh + e])
                    assert abs(A[lo + i, hd * dh + e] - math.fsum(terms) / L) < 1e-13


def test_hstu_is_causal():
    c = _case(7, lengths=(9,))
    A = O.hstu_attn_fwd(c["Q"], c["K"], c["V"], c["off"], c["h"], c["ts"], c["w_pos"], c["w_time"])
    c2 = dict(c)
    for k in ("K", "V", "Q"):
        c2[k] = c[k].copy()
        c2[k][6:] = 100.0
    ts2 = c["ts"].copy()
    ts2[6:] += 10 ** 9
    A2 = O.hstu_attn_fwd(c2["Q"], c2["K"], c2["V"], c["off"], c["h"], ts2, c["w_pos"], c["w_time"])
    np.testing.assert_array_equal(A[:6], A2[:6])
    assert not np.allclose(A[6:], A2[6:])


def test_hstu_constant_bias_gives_prefix_sums():
    # Q = 0, time table 0, position table constant c: A_i = SiLU(c)/L * sum_{j<=i} v_j
    c = _case(9, lengths=(6, 4))
    cval = 0.7
    A = O.hstu_attn_fwd(np.zeros_like(c["Q"]), c["K"], c["V"], c["off"], c["h"], c["ts"],
                        np.full(6, cval), np.zeros(8))
    sil = cval / (1 + math.exp(-cval))
    for b in range(2):
        lo, hi = c["off"][b], c["off"][b + 1]
        np.testing.assert_allclose(A[lo:hi], sil * np.cumsum(c["V"][lo:hi], axis=0) / (hi - lo), rtol=1e-13)


def test_hstu_bias_read_back_through_identity_values():
    # Q = 0 and V = I: A_i[e] = SiLU(rab(i, e)) / L for e <= i, 0 above.  The
    # tables hold distinct values, so a swapped table, a reversed position
    # or a bucket off by one changes the result.
    L = 8
    ts = 1000 + np.array([0, 1, 3, 4, 20, 21, 300, 5000], np.int64)
    w_pos = np.array([0.0, 0.1, 0.2, 0.3, 0.4])
    w_time = np.array([1.0, 1.5, 2.0, 2.5, 3.0, 3.5, 4.0, 4.5, 5.0, 5.5, 6.0, 6.5, 7.0])
    A = O.hstu_attn_fwd(np.zeros((L, L)), np.zeros((L, L)), np.eye(L), [0, L], 1, ts, w_pos, w_time)
    for i in range(L):
        for e in range(L):
            if e > i:
                assert A[i, e] == 0
                continue
            dt = int(ts[i] - ts[e])
            bk = 0
            while 2 ** (bk + 1) <= max(dt, 1):
                bk += 1
            r = w_pos[min(i - e, 4)] + w_time[min(bk, 12)]
            assert abs(A[i, e] - r / (1 + math.exp(-r)) / L) < 1e-15


def _mutant(kind):
    def f(Q, K, V, off, h, ts, wp, wt):
        Q, K, V = np.asarray(Q, float), np.asarray(K, float), np.asarray(V, float)
        T, d = Q.shape
        dh = d // h
        A = np.zeros((T, d))
        for b in range(len(off) - 1):
            lo, hi = off[b], off[b + 1]
            L = hi - lo
            if L == 0:
                continue
            i, j = np.arange(L)[:, None], np.arange(L)[None, :]
            rel = np.minimum(np.maximum((j - i) if kind == "sign" else (i - j), 0), len(wp) - 1)
            bk = O.time_bucket(ts[lo:hi][:, None] - ts[lo:hi][None, :], len(wt))
            if kind == "bucket_plus_one":
                bk = np.minimum(bk + 1, len(wt) - 1)
            rab = np.asarray(wp)[rel] + np.asarray(wt)[bk]
            mask = np.tril(np.ones((L, L))) if kind != "not_causal" else np.ones((L, L))
            for hd in range(h):
                cs = slice(hd * dh, (hd + 1) * dh)
                s = Q[lo:hi, cs] @ K[lo:hi, cs].T / np.sqrt(dh) + rab
                norm = L if kind != "no_norm" else 1
                A[lo:hi, cs] = (O.silu(s) * mask) @ V[lo:hi, cs] / norm
        return A
    return f


@pytest.mark.parametrize("kind", ["sign", "bucket_plus_one", "not_causal", "no_norm"])
def test_hstu_pins_catch_planted_mistakes(kind):
    c = _case(11)
    mut = _mutant(kind)(c["Q"], c["K"], c["V"], c["off"], c["h"], c["ts"], c["w_pos"], c["w_time"])
    ref = _torch_hstu(c)
    assert not np.allclose(mut, ref, rtol=1e-6, atol=1e-8)
