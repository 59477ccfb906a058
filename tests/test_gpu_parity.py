"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle
on the same seeded inputs, element by element.  Small shapes span several
128-row tiles and ragged tails; the bench workload runs at full size."""

import numpy as np
import pytest
import torch

import moe_inputs as MI
from tests import parity as PT

pytestmark = pytest.mark.gpu

W = MI.Workload

# Sparse-expert cases (few tokens per expert) run in f16 and in bf16; bf16
# layers are checked against the oracle with bf16 storage rounding (see
# tests/parity.py).
SMALL = [
    W("t300_d128_e4k2_i128_f32", T=300, d=128, E=4, k=2, I=128, dtype="f32"),
    W("t300_d128_e4k2_i128_bf16", T=300, d=128, E=4, k=2, I=128, dtype="bf16"),
    W("t300_d128_e4k2_i128_f16_norenorm", T=300, d=128, E=4, k=2, I=128, dtype="f16", renorm=False),
    # k = E: the router gradient is a difference of expert outputs (cancellation), run in f16
    W("t257_d256_e2k2_i128_f16_shared1", T=257, d=256, E=2, k=2, I=128, n_shared=1, I_shared=256, dtype="f16"),
    W("t4096_d256_e8k2_i256_bf16_shared1", T=4096, d=256, E=8, k=2, I=256, n_shared=1, I_shared=256),
    W("t1000_d256_e64k6_i128_f16_shared2", T=1000, d=256, E=64, k=6, I=128, n_shared=2, I_shared=128,
      dtype="f16"),
    W("t777_d128_e128k8_i128_zipf_f16", T=777, d=128, E=128, k=8, I=128, zipf_s=1.1, dtype="f16"),
    W("t64_d128_e1k1_i256_bf16", T=64, d=128, E=1, k=1, I=256),
    W("t2100_d384_e8k1_i256_f16_noaux", T=2100, d=384, E=8, k=1, I=256, dtype="f16", aux_coef=0.0),
    W("t513_d256_e16k4_i384_f32_shared1", T=513, d=256, E=16, k=4, I=384, n_shared=1, I_shared=128, dtype="f32"),
    W("t1500_d256_e200k3_i128_f16", T=1500, d=256, E=200, k=3, I=128, dtype="f16"),
    W("t1000_d256_e64k6_i128_bf16_shared2", T=1000, d=256, E=64, k=6, I=128, n_shared=2, I_shared=128),
    W("t777_d128_e128k8_i128_zipf_bf16", T=777, d=128, E=128, k=8, I=128, zipf_s=1.1),
    W("t1500_d256_e200k3_i128_bf16", T=1500, d=256, E=200, k=3, I=128),
    W("t257_d256_e2k2_i128_bf16_shared1", T=257, d=256, E=2, k=2, I=128, n_shared=1, I_shared=256),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_workloads_match_oracle(wl):
    PT.full_parity(wl)


# Every GEMM tile engine (128 x 128 with 4 waves, 128 x 256 with 4 waves for
# the row GEMMs, 256 x 256 with 8 waves) on shapes that all divide, with
# ragged row tails and several tiles per expert.
TILED = [
    W("t3000_d512_e8k2_i512_bf16_shared1", T=3000, d=512, E=8, k=2, I=512, n_shared=1, I_shared=256),
    W("t2500_d256_e4k2_i768_f16", T=2500, d=256, E=4, k=2, I=768, dtype="f16"),
]


@pytest.mark.parametrize("tile", ["128", "256", "128x256"])
@pytest.mark.parametrize("wl", TILED, ids=[w.name for w in TILED])
def test_tile_engines_match_oracle(wl, tile, monkeypatch):
    monkeypatch.setenv("MOE_ROW_TILE", tile)
    monkeypatch.setenv("MOE_WGRAD_TILE", tile if tile != "128x256" else "128")
    PT.full_parity(wl)


# Weight gradients split over tokens (f32 partials, summed in order), including
# experts with fewer tokens than splits (empty splits write zero partials).
SPLIT = [
    W("t4096_d256_e8k2_i256_bf16_shared1", T=4096, d=256, E=8, k=2, I=256, n_shared=1, I_shared=256),
    W("t1000_d256_e64k6_i128_f16_shared2", T=1000, d=256, E=64, k=6, I=128, n_shared=2, I_shared=128,
      dtype="f16"),
]


@pytest.mark.parametrize("splits", [2, 3])
@pytest.mark.parametrize("wl", SPLIT, ids=[w.name for w in SPLIT])
def test_split_weight_gradients_match_oracle(wl, splits, monkeypatch):
    monkeypatch.setenv("MOE_WGRAD_SPLITS", str(splits))
    PT.full_parity(wl)


def test_tiny_reference_workload():
    PT.full_parity(MI.WORKLOADS[MI.TINY])


def test_forced_empty_experts_write_zero_gradients():
    wl = W("t600_d128_e8k2_i128_bf16_bias", T=600, d=128, E=8, k=2, I=128)
    inp = MI.make_inputs(wl)
    b = torch.zeros(8, dtype=torch.float32)
    b[[1, 5]] = -1e4          # experts 1 and 5 never chosen
    inp["bias"] = b
    gpu, fwd, _, st = PT.full_parity(wl, inp)
    assert fwd["counts"][1] == 0 and fwd["counts"][5] == 0
    assert st["n_unused"] == 2


def test_zero_router_ties_break_to_lower_index():
    wl = W("t256_d128_e8k3_i128_f16_zero_router", T=256, d=128, E=8, k=3, I=128, dtype="f16")
    inp = MI.make_inputs(wl)
    inp["w_router"] = torch.zeros_like(inp["w_router"])
    gpu, fwd, _, st = PT.full_parity(wl, inp)
    assert (gpu["topk_idx"] == np.array([0, 1, 2])).all()
    assert abs(gpu["aux"]["aux"] - 1.0) < 1e-6


def test_two_runs_are_bitwise_identical():
    wl = W("t1000_d256_e64k6_i128_bf16_shared2", T=1000, d=256, E=64, k=6, I=128, n_shared=2, I_shared=128)
    inp = MI.make_inputs(wl)
    a = PT.gpu_run(wl, inp)
    b = PT.gpu_run(wl, inp)
    for key, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[key]), key


def test_empty_batch():
    wl = W("t0_d128_e4k2_i128_bf16_shared1", T=0, d=128, E=4, k=2, I=128, n_shared=1, I_shared=128)
    inp = MI.make_inputs(wl)
    gpu = PT.gpu_run(wl, inp)
    assert gpu["counts"].sum() == 0 and np.all(gpu["offsets"] == 0)
    for key in ("dw_router", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"):
        assert not np.any(gpu[key]), key


def test_bench_workload_full_size():
    PT.full_parity(MI.WORKLOADS[MI.BENCH])


# The two other full-size 16-bit workloads (the MX-fp8 one is in
# test_gpu_mx.py): element by element against the oracle, which takes about a
# minute of host time each.
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["t32768_d1536_e4k2_i3072_s1x3072_f16", "t16384_d2048_e128k8_i768_zipf_bf16"])
def test_large_workloads_full_size(name):
    PT.full_parity(MI.WORKLOADS[name])
