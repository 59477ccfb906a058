"""The dense SwiGLU MLP through the same grouped GEMM: one expert, top-1.

With E = 1 and k = 1 the softmax is 1, every token takes expert 0 with weight
1, the permutation is the identity and the layer is the dense SwiGLU block
(spark-gpt README: dense mode remains the default beside the optional MoE
layers).  The oracle pins that reduction on the CPU
(test_single_expert_top1_is_dense_swiglu_mlp); here the whole GPU chain runs
it, forward and backward, against the oracle."""

import numpy as np
import pytest

import moe_inputs as MI
from tests import parity as PT

pytestmark = pytest.mark.gpu
W = MI.Workload

DENSE = [
    W("t3000_d256_e1k1_i512_bf16_dense", T=3000, d=256, E=1, k=1, I=512),
    W("t2048_d512_e1k1_i256_f16_shared1_dense", T=2048, d=512, E=1, k=1, I=256, n_shared=1, I_shared=256,
      dtype="f16"),
    W("t700_d128_e1k1_i128_f32_dense", T=700, d=128, E=1, k=1, I=128, dtype="f32"),
]


@pytest.mark.parametrize("wl", DENSE, ids=[w.name for w in DENSE])
def test_dense_swiglu_mlp_matches_oracle(wl):
    gpu, fwd, bwd, _ = PT.full_parity(wl)
    # the structure the reduction implies, on the device's own outputs
    assert np.all(gpu["topk_idx"] == 0) and np.all(gpu["probs"] == 1.0) and np.all(gpu["topk_w"] == 1.0)
    assert np.array_equal(gpu["perm_token"], np.arange(wl.T)) and gpu["counts"].tolist() == [wl.T]
    # a single expert's softmax has no gradient: the router gradient vanishes
    assert np.all(gpu["dw_router"] == 0.0)
