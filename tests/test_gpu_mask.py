"""GPU parity of the balancing statistic over real (non-filler) tokens.

The spark-gpt README's MoE paragraph computes the statistic over real tokens
only.  Fillers are still routed and run through the experts; only the
statistic, its metrics and its gradient (through P_e, on real tokens) leave
them out.  Compared with the oracle given the same mask, on both router
backward engines; an all-real mask must reproduce the unmasked layer bit for
bit, and an all-filler mask must zero the statistic and its gradient."""

import numpy as np
import pytest

import moe_inputs as MI
from tests import parity as PT

pytestmark = pytest.mark.gpu
W = MI.Workload

# aux_coef large enough that the balancing gradient is visible in dx and dW_r
MASKED = [
    W("t3000_d256_e8k2_i128_bf16_masked", T=3000, d=256, E=8, k=2, I=128, aux_coef=0.5),        # few experts
    W("t2000_d256_e64k6_i128_f16_masked", T=2000, d=256, E=64, k=6, I=128, dtype="f16", aux_coef=0.5),
    W("t700_d128_e4k2_i128_f32_norenorm_masked", T=700, d=128, E=4, k=2, I=128, dtype="f32", renorm=False,
      aux_coef=0.5),
]


@pytest.mark.parametrize("wl", MASKED, ids=[w.name for w in MASKED])
def test_masked_statistic_matches_oracle(wl):
    mask = MI.real_token_mask(wl.T)
    gpu, _, _, st = PT.full_parity(wl, mask=mask)
    PT.say(f"[mask] {wl.name}: {int(mask.sum())} of {wl.T} tokens real; aux {gpu['aux']['aux']:.6f} "
           f"(oracle {st['aux']:.6f})")


def test_all_real_mask_is_bitwise_the_unmasked_layer():
    wl = MASKED[0]
    inp = MI.make_inputs(wl)
    a = PT.gpu_run(wl, inp)
    b = PT.gpu_run(wl, inp, mask=np.ones(wl.T, dtype=np.int32))
    for n in ("dx", "dw_router", "dbias", "f", "p_mean", "dw_gate_up", "dw_down"):
        assert np.array_equal(a[n], b[n]), n
    assert a["aux"] == b["aux"]
    assert b["real_counts"].tolist() == a["counts"].tolist() + [wl.T]


def test_all_filler_mask_zeroes_the_statistic_and_its_gradient():
    wl = MASKED[0]
    inp = MI.make_inputs(wl)
    none = PT.gpu_run(wl, inp, mask=np.zeros(wl.T, dtype=np.int32))
    assert none["real_counts"].tolist() == [0] * (wl.E + 1)
    assert np.all(none["f"] == 0) and np.all(none["p_mean"] == 0)
    assert none["aux"]["aux"] == 0.0 and none["aux"]["entropy_mean"] == 0.0
    # the layer's gradients are then those of aux_coef = 0
    ref = PT.gpu_run(wl.with_(aux_coef=0.0), inp)
    for n in ("dx", "dw_router", "dbias"):
        assert np.array_equal(none[n], ref[n]), n


@pytest.mark.parametrize("wl", MASKED[:2], ids=[w.name for w in MASKED[:2]])
def test_masked_statistic_gradient_alone(wl):
    # dy = 0 leaves the balancing term as the only source of gradient: the
    # router gradients then come from the masked statistic alone, and filler
    # tokens must get exactly none.  The coefficient is large so that dz stays
    # in f16's normal range (its hi/lo pair in f16 has no relative precision
    # below 2^-14; with a real loss the routing term keeps dz far above that)
    wl = wl.with_(aux_coef=1000.0)
    inp = MI.make_inputs(wl)
    inp["dy"] = inp["dy"] * 0
    mask = MI.real_token_mask(wl.T, seed=5)
    gpu, _, bwd, _ = PT.full_parity(wl, inp=inp, mask=mask)
    assert np.all(gpu["dx"][mask == 0] == 0.0)
    assert np.abs(gpu["dx"][mask == 1]).max() > 0 and np.abs(bwd["dw_router"]).max() > 0
