"""The seeded input generator: bf16 rounding, determinism, per-request slicing."""
import numpy as np
import torch

from candidate_conditioned_sequence_amd import synth


def test_round_bf16_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.round_bf16(x), ref)


def test_lengths_follow_config_ranges():
    for key in ("c2", "c3", "c4", "c5"):
        cfg = synth.CONFIGS[key]
        L = synth.lengths(cfg)
        lo, hi = cfg.lengths[-2:]
        assert L.shape == (cfg.B,) and L.min() >= lo and L.max() <= hi
    assert np.all(synth.lengths(synth.CONFIGS["c3L10k"]) == 10000)
    assert synth.lengths(synth.CONFIGS["c1"]).tolist() == [256]


def test_subset_rows_equal_full_rows():
    cfg = synth.scaled(synth.CONFIGS["c2"], B=5, C=2, n_q=3, d=16, h=2,
                       lengths=("list", [4, 0, 7, 1, 3]))
    Hw, Hs, off = synth.inputs(cfg)
    Hw2, Hs2, off2 = synth.inputs(cfg, requests=[2, 4])
    per = cfg.C * cfg.n_q
    np.testing.assert_array_equal(Hw2, np.concatenate([Hw[2 * per:3 * per], Hw[4 * per:5 * per]]))
    np.testing.assert_array_equal(Hs2, np.concatenate([Hs[off[2]:off[3]], Hs[off[4]:off[5]]]))
    assert off2.tolist() == [0, 7, 10]
    # deterministic
    Hw3, _, _ = synth.inputs(cfg)
    np.testing.assert_array_equal(Hw, Hw3)
    p = synth.layer_params(cfg)
    assert np.all(synth.round_bf16(p["W_F"]) == p["W_F"])
    a = np.sqrt(6 / (3 * cfg.d))
    assert np.abs(p["W_F"]).max() <= a
