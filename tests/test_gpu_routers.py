"""GPU parity of the router variants against the oracle (KohakUwULLM README,
"Key features": Sinkhorn, expert-choice and ReLU routers beside the default;
the readings are the oracle's).

Sinkhorn router: the column scales within SINKHORN_B_RTOL of the oracle's
(computed in fp64 from the oracle's own probabilities), the routing bit-exact
except near-ties of ln(p b), the weights within 1e-6, on every router engine
(4, 8, 64, 128 and 256 experts; f32, f16, bf16; with and without renorm and
logit bias) and for 1 to 30 rounds; then the whole layer routed this way
against the exact oracle layer.

ReLU router: the whole layer against the exact oracle (see RELU below)."""

import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from tests import parity as PT

pytestmark = pytest.mark.gpu

W = MI.Workload

ROUTE_CASES = [
    (W("t1000_d256_e4k2_i128_bf16", T=1000, d=256, E=4, k=2, I=128), 8),
    (W("t300_d128_e8k2_i128_f32_norenorm", T=300, d=128, E=8, k=2, I=128, dtype="f32", renorm=False), 3),
    (W("t777_d128_e64k6_i128_f16", T=777, d=128, E=64, k=6, I=128, dtype="f16"), 1),
    (W("t1536_d256_e128k8_i128_zipf_bf16", T=1536, d=256, E=128, k=8, I=128, zipf_s=1.1), 30),
    (W("t513_d128_e256k4_i128_zipf_f16", T=513, d=128, E=256, k=4, I=128, zipf_s=1.1, dtype="f16"), 10),
]


@pytest.mark.parametrize("wl,n_iter", ROUTE_CASES, ids=[f"{w.name}_it{n}" for w, n in ROUTE_CASES])
def test_sinkhorn_route_matches_oracle(wl, n_iter):
    from mixture_experts_ffn_wave_amd import moe_route_sinkhorn
    inp = MI.make_inputs(wl)
    f64 = PT.oracle_inputs(inp)
    b = inp.get("bias")
    plan = PT.plan_for(wl, b is not None)
    dev = "cuda"
    probs = torch.empty(wl.T, wl.E, dtype=torch.float32, device=dev)
    idx = torch.empty(wl.T, wl.k, dtype=torch.int32, device=dev)
    w = torch.empty(wl.T, wl.k, dtype=torch.float32, device=dev)
    cs = torch.empty(wl.E, dtype=torch.float32, device=dev)
    ws = torch.empty(max(plan.workspace_bytes(), 256), dtype=torch.uint8, device=dev)
    moe_route_sinkhorn(plan, inp["x"].cuda(), inp["w_router"].cuda(), b.float().cuda() if b is not None else None,
                       n_iter, probs, idx, w, cs, ws)
    torch.cuda.synchronize()
    gpu = {"probs": PT.to_np(probs), "topk_idx": PT.to_np(idx), "topk_w": PT.to_np(w),
           "sinkhorn_b": PT.to_np(cs)}
    z = O.router_logits(f64["x"], f64["w_router"], f64.get("bias"))
    p = O.softmax_rows(z)
    bref = O.sinkhorn_column_scales(p, n_iter)
    idx_ref = O.topk_select(O.sinkhorn_selection_scores(p, bref), wl.k)
    fwd = {"z": z, "p": p, "idx": idx_ref, "w": O.gate_weights(p, idx_ref, wl.renorm), "sinkhorn_b": bref}
    same = PT.compare_routing(wl, gpu, fwd)
    PT.say(f"[sinkhorn] {wl.name} rounds={n_iter}: routing identical={same}, max b rel err "
           f"{np.max(np.abs(gpu['sinkhorn_b'] - bref) / bref):.2e}")


def test_sinkhorn_layer_matches_oracle():
    wl = W("t1536_d256_e64k6_i128_zipf_bf16_shared1", T=1536, d=256, E=64, k=6, I=128, zipf_s=1.1, n_shared=1,
           I_shared=128)
    gpu, fwd, _, _ = PT.full_parity(wl, sinkhorn=8)
    counts = fwd["counts"]
    plain = np.bincount(O.topk_select(fwd["z"], wl.k).ravel(), minlength=wl.E)
    # the Sinkhorn choice spreads the skewed router's load
    assert counts.std() < 0.5 * plain.std(), (counts.std(), plain.std())


# ReLU router (moe_config.router = MOE_ROUTER_RELU): gates max(z, 0), the k
# largest positive logits per token, empty slots -1; the whole layer against
# the exact oracle on the router engines of 4, 8, 64 and 128 experts.  A
# constant logit bias falling from hi to lo over the experts makes some tokens
# have fewer than k (or no) positive logits.
RELU = [
    (W("t1000_d256_e8k2_i128_bf16_relu", T=1000, d=256, E=8, k=2, I=128, renorm=False, router="relu"), (0.1, -0.3)),
    (W("t777_d128_e4k2_i256_f16_relu_shared1", T=777, d=128, E=4, k=2, I=256, renorm=False, router="relu",
       n_shared=1, I_shared=128, dtype="f16"), (0.1, -0.3)),
    (W("t513_d128_e64k6_i128_f32_relu", T=513, d=128, E=64, k=6, I=128, renorm=False, router="relu", dtype="f32"),
     (0.0, -1.0)),
    (W("t1200_d256_e128k8_i128_bf16_relu", T=1200, d=256, E=128, k=8, I=128, renorm=False, router="relu"),
     (0.1, -2.0)),
]


@pytest.mark.parametrize("wl,bias", RELU, ids=[w.name for w, _ in RELU])
def test_relu_router_layer_matches_oracle(wl, bias):
    inp = MI.make_inputs(wl)
    inp["bias"] = torch.linspace(bias[0], bias[1], wl.E, dtype=torch.float32)
    gpu, fwd, _, _ = PT.full_parity(wl, inp)
    empty = int((fwd["idx"] < 0).sum())
    PT.say(f"[relu] {wl.name}: {empty} empty slots of {wl.T * wl.k}, {int(fwd['offsets'][-1])} rows")
    assert empty > 0                                 # the case of fewer than k positive logits is exercised


# Expert-choice router (MOE_ROUTER_EXPERT_CHOICE, moe_route_expert_choice):
# every expert takes its C = T k / E tokens of largest probability; [T, E]
# slots; the whole layer against the exact oracle on both router-backward
# engines (E <= 16: the fused per-block kernel; 64: dz kernel + MFMA products).
EXPERT_CHOICE = [
    W("t1000_d256_e4k2_i128_bf16_ec", T=1000, d=256, E=4, k=2, I=128, renorm=False, router="expert_choice"),
    W("t777_d128_e8k2_i256_f16_ec_shared1", T=777, d=128, E=8, k=2, I=256, renorm=False, router="expert_choice",
      n_shared=1, I_shared=128, dtype="f16"),
    # (uniform router: with a Zipf-skewed one some tokens are taken by up to
    # 17 experts, y's largest elements sit 16 RMS out, and the bf16 rounding
    # of H alone, the down GEMM's operand, puts y 0.030 RMS past the bar)
    W("t1536_d256_e64k4_i128_bf16_ec", T=1536, d=256, E=64, k=4, I=128, renorm=False, router="expert_choice"),
    W("t513_d128_e16k3_i128_f32_ec", T=513, d=128, E=16, k=3, I=128, renorm=False, router="expert_choice",
      dtype="f32"),
]


@pytest.mark.parametrize("wl", EXPERT_CHOICE, ids=[w.name for w in EXPERT_CHOICE])
def test_expert_choice_layer_matches_oracle(wl):
    gpu, fwd, _, _ = PT.full_parity(wl)
    per_token = (fwd["idx"] >= 0).sum(axis=1)
    PT.say(f"[expert-choice] {wl.name}: C={(wl.T * wl.k) // wl.E}, experts per token "
           f"{per_token.min()}..{per_token.max()}, tokens with none {int((per_token == 0).sum())}")
    assert np.array_equal(fwd["counts"], np.full(wl.E, (wl.T * wl.k) // wl.E))
