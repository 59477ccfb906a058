"""CPU checks of the comparison helpers the GPU parity tests rely on."""

import numpy as np
import torch

from tests import parity as PT


def test_half_ulp_matches_torch_rounding():
    rng = np.random.default_rng(0)
    # start from float32 values: the GPU rounds f32 results into the storage type
    v = (rng.standard_normal(20000) * np.exp(rng.standard_normal(20000) * 4)).astype(np.float32).astype(np.float64)
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)):
        r = torch.from_numpy(v).to(tdt).to(torch.float64).numpy()
        ok = np.isfinite(r)
        err = np.abs(r - v)[ok]
        # round-to-nearest never moves a value by more than half an ulp
        assert np.all(err <= PT.half_ulp(np.maximum(np.abs(r), np.abs(v))[ok], dt) * (1 + 1e-12))
    assert PT.half_ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -8
    assert PT.half_ulp(np.array([1.0]), "f16")[0] == 2.0 ** -11


def test_check_close_flags_a_real_error():
    ref = np.linspace(-1, 1, 1000)
    got = ref.copy()
    got[10] += 0.05
    try:
        PT.check_close("x", got, ref, 2e-2, "bf16")
    except AssertionError:
        return
    raise AssertionError("a 0.05 error on an RMS-0.58 tensor passed")
