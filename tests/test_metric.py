"""The parity metric itself (CPU)."""
import numpy as np
import torch

from tests.hstu_testutil import err_rms, err_stored


def test_exact_result_rounded_to_bf16_scores_zero():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(200000) * np.exp(rng.standard_normal(200000))
    y = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert err_rms(y, ref) > 0.01          # the storage rounding alone
    assert err_stored(y, ref, "bf16") <= 1e-7


def test_metric_sees_errors_beyond_the_rounding():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal(1000)
    rms = np.sqrt(np.mean(ref ** 2))
    y = ref.copy()
    y[17] += 0.05 * rms
    assert abs(err_stored(y, ref, "bf16") - (0.05 - 2 ** -8 * abs(ref[17]) / rms)) < 1e-12
    assert abs(err_stored(y, ref, "f32") - 0.05) < 1e-12
    assert err_stored(ref, ref, "f32") == 0.0
