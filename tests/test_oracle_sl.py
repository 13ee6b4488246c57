"""Pins of the Stochastic Length oracle ("Actions Speak Louder than Words" reading notes §3.3).

  * the target length N_c^(alpha/2) against the page's worked figure (4096 -> 776 at alpha =
    1.6) and the no-SL baseline alpha = 2 (tests/golden/sl.txt);
  * sequences no longer than the target are kept whatever the draws;
  * the keep-or-subsample decision sits exactly at probability 1 - N_c^alpha / n^2 (draws just
    below / above the threshold);
  * the subsequence is the target number of smallest keys (brute force over (key, index)),
    in order; the output offsets are the prefix sums of the new lengths;
  * statistically, with uniform draws, each event survives subsampling with probability L / n
    and users are subsampled with frequency 1 - N_c^alpha / n^2.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sl.txt")


def _rows():
    out = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            n, a, L = line.split()
            out.append((int(n), float(a), int(L)))
    return out


@pytest.mark.parametrize("row", _rows())
def test_target_length_golden(row):
    N_c, alpha, L = row
    assert oracle.sl_length(N_c, alpha) == L


def test_short_sequences_are_kept():
    lengths = [1, 5, 20, 20]
    offs = np.concatenate([[0], np.cumsum(lengths)])
    L = oracle.sl_length(400, 1.0)  # 20
    assert L == 20
    out, src = oracle.stochastic_length(offs, 400, 1.0, np.zeros(4, np.float32),
                                        np.random.default_rng(0).random(46).astype(np.float32))
    np.testing.assert_array_equal(out, offs)
    np.testing.assert_array_equal(src, np.arange(46))


def test_decision_threshold():
    N_c, alpha = 1000, 1.5
    L = oracle.sl_length(N_c, alpha)  # 177
    n = 400
    p = 1.0 - float(N_c) ** alpha / (n * n)
    below = np.nextafter(np.float32(p), np.float32(0))
    above = np.nextafter(np.float32(p), np.float32(1))
    assert float(below) < p <= float(above)
    offs = np.array([0, n, 2 * n])
    keys = np.random.default_rng(1).random(2 * n).astype(np.float32)
    out, src = oracle.stochastic_length(offs, N_c, alpha, np.array([below, above], np.float32), keys)
    assert out[1] - out[0] == L           # u < p: subsampled
    assert out[2] - out[1] == n           # u >= p: kept whole


def test_subsequence_is_smallest_keys_in_order():
    rng = np.random.default_rng(2)
    lengths = [300, 50, 1000, 0, 601]
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    keys = rng.integers(0, 50, size=T).astype(np.float32) / 50  # many ties
    N_c, alpha = 1000, 1.4
    L = oracle.sl_length(N_c, alpha)
    out, src = oracle.stochastic_length(offs, N_c, alpha, np.zeros(5, np.float32), keys)
    for b, n in enumerate(lengths):
        got = src[out[b]:out[b + 1]]
        s = int(offs[b])
        if n <= L:
            np.testing.assert_array_equal(got, np.arange(s, s + n))
            continue
        pairs = sorted((float(keys[s + i]), i) for i in range(n))[:L]
        np.testing.assert_array_equal(got, s + np.array(sorted(i for _, i in pairs)))
        assert np.all(np.diff(got) > 0)
    np.testing.assert_array_equal(np.diff(out), [min(n, L) if n > L else n for n in lengths])


def test_statistics():
    rng = np.random.default_rng(3)
    N_c, alpha = 100, 1.0
    L = oracle.sl_length(N_c, alpha)  # 10
    n = 40
    trials = 3000
    offs = np.arange(0, n * trials + 1, n)
    out, src = oracle.stochastic_length(offs, N_c, alpha, rng.random(trials).astype(np.float32),
                                        rng.random(n * trials).astype(np.float32))
    lens = np.diff(out)
    p_sub = 1.0 - N_c ** alpha / n ** 2
    frac = np.mean(lens == L)
    assert abs(frac - p_sub) < 4 * np.sqrt(p_sub * (1 - p_sub) / trials)
    # among subsampled users each position survives with probability L / n
    counts = np.zeros(n)
    for b in np.nonzero(lens == L)[0]:
        counts[src[out[b]:out[b + 1]] - b * n] += 1
    m = (lens == L).sum()
    pk = L / n
    assert np.all(np.abs(counts / m - pk) < 5 * np.sqrt(pk * (1 - pk) / m))
