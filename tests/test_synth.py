"""Seeded synthetic inputs: determinism and the shapes / ranges of each workload."""
import numpy as np

from hstu_sequential_transduction_jagged_amd import synth


def test_round_bf16_ties_to_even_and_exactness():
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.1415926],
                 np.float32)
    r = synth.round_bf16(a)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert r[1] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6
    assert r[2] == np.float32(1.0 + 2 ** -6)
    assert r[3] == 1.0
    assert r[4] == -2.5
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    assert np.all(synth.round_bf16(r) == r)


def test_attn_small_recipe_and_determinism():
    a = synth.attn_small()
    b = synth.attn_small()
    assert np.array_equal(a.q, b.q) and np.array_equal(a.offsets, b.offsets)
    n = np.diff(a.offsets)
    assert a.B == 4 and a.H == 2 and a.dqk == 32 and a.dtype == "f32"
    assert np.all((n >= 16) & (n <= 128))
    assert a.alpha == 1.0 / 128
    assert a.bias.w_pos.shape == (128,) and a.bias.w_time.shape == (32,)
    for bb in range(a.B):
        t = a.ts[a.offsets[bb]:a.offsets[bb + 1]]
        assert np.all(np.diff(t) >= 0)


def test_attn_long_lengths():
    a = synth.attn_long()
    n = np.diff(a.offsets)
    assert a.B == 16 and np.all((n >= 256) & (n <= 8192))
    assert a.dtype == "bf16"
    assert np.all((a.q.view(np.uint32) & 0xFFFF) == 0)
    assert a.bias.w_pos.shape == (256,) and a.alpha == 1.0 / 8192
    # median of the lognormal draw is 2048: over many draws about half fall below
    rng = np.random.default_rng(0)
    draws = synth.lognormal_lengths(rng, 20000)
    assert 1900 < np.median(draws) < 2200


def test_layer_small_and_stack8():
    a = synth.layer_small()
    n = np.diff(a.offsets)
    assert np.all((n >= 8) & (n <= 1024)) and a.B == 32
    L = a.layers[0]
    assert L.w1.shape == (1024, 256) and L.w2.shape == (256, 256)
    bound = np.sqrt(6.0 / (256 + 1024))
    assert np.abs(L.w1).max() <= bound * (1 + 2 ** -8)
    s = synth.stack8(B=64, n_layers=2)
    n = np.diff(s.offsets)
    assert np.all((n >= 1) & (n <= 4096)) and len(s.layers) == 2 and s.residual
    # stochastic length: sequences above the cap are either whole or exactly the cap
    assert len(s.ts) == s.T


def test_genrank_small():
    g = synth.genrank(B=3, lo=16, hi=32, n_items=1000)
    assert g.item_table.shape == (1000, 512) and g.action_table.shape == (4, 512)
    assert g.item_ids.min() >= 0 and g.item_ids.max() < 1000
    assert g.action_ids.min() >= 0 and g.action_ids.max() < 4
    assert g.layers[0].bias.kind == synth.BIAS_ALIBI
    # Zipf(1.1): rank 1 is the most frequent id
    ids = synth.truncated_zipf(np.random.default_rng(0), 100000, 1.1, 1000)
    counts = np.bincount(ids, minlength=1000)
    assert counts[0] == counts.max() and counts[0] > 5 * counts[10]
