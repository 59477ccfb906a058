"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle
on the same seeded inputs, element by element.  Small shapes span several
128-row tiles and ragged tails; the bench workload runs at full size."""

import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from tests import parity as PT

pytestmark = pytest.mark.gpu

W = MI.Workload

# Sparse-expert cases (few tokens per expert) run in f16 and in bf16; every
# layer is checked against the exact fp64 oracle (see tests/parity.py).
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
# the row GEMMs, 256 x 256 with 8 waves, and the 256 x 256 ping-pong row
# GEMMs) on shapes that all divide, with ragged row tails and several tiles
# per expert.
TILED = [
    W("t3000_d512_e8k2_i512_bf16_shared1", T=3000, d=512, E=8, k=2, I=512, n_shared=1, I_shared=256),
    W("t2500_d256_e4k2_i768_f16", T=2500, d=256, E=4, k=2, I=768, dtype="f16"),
]


@pytest.mark.parametrize("tile", ["128", "256", "128x256", "256pp"])
@pytest.mark.parametrize("wl", TILED, ids=[w.name for w in TILED])
def test_tile_engines_match_oracle(wl, tile, monkeypatch):
    monkeypatch.setenv("MOE_ROW_TILE", tile)
    monkeypatch.setenv("MOE_WGRAD_TILE", tile if tile in ("128", "256") else "128")
    PT.full_parity(wl)


# bf16 plans whose experts see few rows (fewer than 128 on average) add the
# products of the operands' rounding remainders to the expert weight
# gradients: forced on here for every row tile of the down dgrad (whose
# epilogue writes the remainders) and both weight-gradient tiles.
@pytest.mark.parametrize("tile", ["128", "128x256", "256", "256pp"])
def test_remainder_weight_gradients_on_every_tile(tile, monkeypatch):
    wl = W("t3000_d512_e8k2_i512_bf16_shared1", T=3000, d=512, E=8, k=2, I=512, n_shared=1, I_shared=256)
    monkeypatch.setenv("MOE_WGRAD_COMP", "1")
    monkeypatch.setenv("MOE_ROW_TILE", tile)
    monkeypatch.setenv("MOE_WGRAD_TILE", tile if tile in ("128", "256", "256pp") else "128")
    PT.full_parity(wl)


def test_down_dgrad_remainders_and_wh_rows():
    """The down dgrad's extra outputs against the oracle at 200 experts of
    about 22 rows each: w H (the routing weight times H = silu(G) U) rounded
    to bf16 once, and the bf16 rounding remainders of w H and of [dG | dU],
    each at most half an ulp of the rounded value and, added to it, within
    f32 arithmetic of the exact value."""
    wl = W("t1500_d256_e200k3_i128_bf16", T=1500, d=256, E=200, k=3, I=128)
    inp = MI.make_inputs(wl)
    f64 = PT.oracle_inputs(inp)
    gpu = PT.gpu_run(wl, inp, intermediates=True, extra=("wh", "dgu_lo", "wh_lo"))
    fwd, bwd, _ = PT.oracle_run(wl, f64)
    assert PT.compare_routing(wl, gpu, fwd)
    PT.compare_dispatch(gpu, fwd)
    inv, off, w = fwd["inv"], fwd["offsets"], fwd["w"]
    wsorted = np.zeros(wl.T * wl.k)
    wsorted[inv.reshape(-1)] = w.reshape(-1)
    dy = f64["dy"]
    dy_rows = np.zeros((wl.T * wl.k, wl.d))
    dy_rows[inv.reshape(-1)] = np.repeat(dy, wl.k, axis=0)
    # bf16 layers: dY_perm holds plain copies of dy's rows
    assert np.array_equal(gpu["dy_perm"], dy_rows)
    wh_exact = wsorted[:, None] * fwd["h"]
    dgu_exact = np.zeros_like(gpu["dgu"])
    for e in range(wl.E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            dgu_exact[r0:r1], _ = O.expert_down_backward_step(bwd["dy_perm"][r0:r1], fwd["g"][r0:r1],
                                                             fwd["u"][r0:r1], fwd["h"][r0:r1], f64["w_down"][e],
                                                             None, lambda a, kind: a)
    for name, hi, lo, exact in [("wH", gpu["wh"], gpu["wh_lo"], wh_exact),
                                ("dGU", gpu["dgu"], gpu["dgu_lo"], dgu_exact)]:
        assert np.all(np.abs(lo) <= PT.half_ulp(hi, "bf16")), f"{name}: remainder above half an ulp"
        e_hi = float(np.linalg.norm(hi - exact))
        e_pair = float(np.linalg.norm(hi + lo - exact))
        PT.say(f"{name}: |hi - exact| {e_hi:.3e}, |hi + lo - exact| {e_pair:.3e}")
        assert e_pair <= 2e-2 * e_hi, name


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
# test_gpu_mx.py): element by element against the exact oracle, which takes
# about a minute of host time each.
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["t32768_d1536_e4k2_i3072_s1x3072_f16", "t16384_d2048_e128k8_i768_zipf_bf16"])
def test_large_workloads_full_size(name):
    PT.full_parity(MI.WORKLOADS[name])
