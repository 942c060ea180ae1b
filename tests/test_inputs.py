"""The seeded input generator: deterministic draws and bfloat16 rounding equal to torch's."""
import numpy as np
import torch

from synth import CONFIGS, bf16_round, make_inputs


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-40, 38, 200000)).astype(np.float32)
    x[:9] = [np.inf, -np.inf, 0.0, -0.0, 3.3895e38, -3.3895e38, 1e-40, -1e-40, 1.00390625]
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf16_round(x), ref)
    assert np.isnan(bf16_round(np.array([np.nan], dtype=np.float32)))[0]


def test_inputs_deterministic_and_rounded():
    wl = CONFIGS[3].with_(B=2, N=20)
    a, b = make_inputs(wl), make_inputs(wl)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    for key in ("q", "k", "v", "u", "g1", "gh"):
        np.testing.assert_array_equal(bf16_round(a[key]), a[key])
    assert a["q"].shape == (2, 3, 20, 64) and a["mu"].shape == (3, 64) and a["g1"].shape == (2, 3, 20)
    assert np.all(a["tau"] == 0)
    t = make_inputs(CONFIGS[2].with_(B=1, N=4))["tau"]
    assert np.all(np.abs(t) <= 1) and np.any(t != 0)
