"""GPU parity of the aux-loss-free balancing router variant against the oracle.

Experts are ranked on probability + a per-expert selection bias, weighted by
the unbiased probabilities, and the bias moves by gamma * sign(mean load -
load) after a step (KohakUwULLM README, "Key features": DeepSeekMoE with
aux-loss-free load balancing; the rule is the published method's).  The whole
layer is compared with the oracle layer given the same bias; the bias update
is bit-exact; and repeated updates even out a Zipf-skewed router on the
device."""

import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from tests import parity as PT

pytestmark = pytest.mark.gpu
W = MI.Workload

# router engines: one-wave K-split (E <= 32 and <= 64) and multi-wave (128)
BALANCED = [
    (W("t1000_d256_e8k2_i128_f32_bal", T=1000, d=256, E=8, k=2, I=128, dtype="f32"), 0.05),
    (W("t1536_d256_e64k6_i128_bf16_shared1_bal", T=1536, d=256, E=64, k=6, I=128, n_shared=1, I_shared=128),
     0.01),
    (W("t1200_d256_e128k8_i128_zipf_bf16_bal", T=1200, d=256, E=128, k=8, I=128, zipf_s=1.1), 0.005),
    (W("t900_d128_e4k2_i256_f16_norenorm_bal", T=900, d=128, E=4, k=2, I=256, dtype="f16", renorm=False), 0.1),
]


@pytest.mark.parametrize("wl,scale", BALANCED, ids=[w.name for w, _ in BALANCED])
def test_balanced_layer_matches_oracle(wl, scale):
    sb = MI.selection_bias(wl.E, scale)
    gpu, fwd, _, _ = PT.full_parity(wl, sel_bias=sb)
    # the bias changed the choice of experts for a good share of the tokens
    plain = O.topk_select(fwd["z"], wl.k)
    changed = np.any(np.sort(plain, axis=1) != np.sort(fwd["idx"], axis=1), axis=1).mean()
    PT.say(f"[balance] {wl.name}: selection bias changed the expert set of {changed:.1%} of tokens")
    assert changed > 0.02


def test_balance_update_is_bit_exact():
    from mixture_experts_ffn_wave_amd import Plan, moe_balance_update
    T, E, k = 3000, 64, 6                   # mean load 281.25: never an integer
    plan = Plan(T, 256, E, k, 128)
    rng = np.random.default_rng(3)
    counts = rng.integers(150, 420, size=E).astype(np.int32)
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    for gamma in (1e-3, 2.0 ** -20, 0.0):
        cd, bd = torch.from_numpy(counts).cuda(), torch.from_numpy(b).cuda()
        moe_balance_update(plan, cd, bd, gamma)
        torch.cuda.synchronize()
        ref = O.balance_bias_update(b, counts, T, k, gamma)
        assert np.array_equal(bd.cpu().numpy(), ref), gamma
    # an integer mean load gives sign 0 exactly where count == mean
    plan2 = Plan(64, 256, 8, 2, 128)
    c2 = np.array([16, 15, 17, 16, 0, 32, 16, 16], dtype=np.int32)
    b2 = np.zeros(8, dtype=np.float32)
    bd = torch.from_numpy(b2).cuda()
    moe_balance_update(plan2, torch.from_numpy(c2).cuda(), bd, 0.5)
    assert bd.cpu().numpy().tolist() == [0.0, 0.5, -0.5, 0.0, 0.5, -0.5, 0.0, 0.0]
    plan.close(); plan2.close()


def test_balancing_evens_out_a_skewed_router():
    # route + permute (for the loads) + update, many steps on fixed inputs with
    # a strongly skewed router; then the last step's whole layer against the
    # oracle given the bias the device arrived at
    from mixture_experts_ffn_wave_amd import MoELayer, moe_permute
    wl = W("t4096_d256_e16k2_i128_zipf_bf16_bal", T=4096, d=256, E=16, k=2, I=128, zipf_s=1.2)
    inp = MI.make_inputs(wl)
    plan = PT.plan_for(wl, True)
    layer = MoELayer(plan)
    dev = {n: (v.cuda() if v is not None else None) for n, v in inp.items()}
    layer.set_params(dev["x"], dev["w_router"], dev["w_gate_up"], dev["w_down"], bias=dev["bias"].float())
    layer.enable_balancing()
    cv = []
    for it in range(300):
        layer.route()
        moe_permute(plan, layer.topk_idx, dev["x"], layer.counts, layer.offsets, layer.perm_token,
                    layer.inv_perm, layer.x_perm, layer.ws)
        if it % 25 == 0 or it == 299:
            c = layer.counts.cpu().numpy().astype(np.float64)
            cv.append(c.std() / c.mean())
        layer.update_balance(2e-3)
    torch.cuda.synchronize()
    PT.say(f"[balance] load CV every 25 steps: " + " ".join(f"{v:.3f}" for v in cv))
    assert cv[0] > 0.8 and cv[-1] < 0.25 * cv[0]
    sb = layer.sel_bias.cpu().numpy()
    plan.close()
    PT.full_parity(wl, inp=inp, sel_bias=sb)


def test_balanced_route_full_size_zipf():
    # the skewed workload at full size: router outputs against the oracle router
    from mixture_experts_ffn_wave_amd import moe_route_balanced
    wl = MI.WORKLOADS["t16384_d2048_e128k8_i768_zipf_bf16"]
    inp = MI.make_inputs(wl)
    sb = MI.selection_bias(wl.E, 0.003)
    plan = PT.plan_for(wl, True)
    x, wr, b = inp["x"].cuda(), inp["w_router"].cuda(), inp["bias"].float().cuda()
    probs = torch.empty(wl.T, wl.E, dtype=torch.float32, device="cuda")
    idx = torch.empty(wl.T, wl.k, dtype=torch.int32, device="cuda")
    w = torch.empty(wl.T, wl.k, dtype=torch.float32, device="cuda")
    moe_route_balanced(plan, x, wr, b, torch.from_numpy(sb).cuda(), probs, idx, w)
    torch.cuda.synchronize()
    f64 = PT.oracle_inputs(inp)
    z = O.router_logits(f64["x"], f64["w_router"], f64["bias"])
    p = O.softmax_rows(z)
    sel = O.topk_select(O.balanced_selection_scores(p, sb.astype(np.float64)), wl.k)
    fwd = {"z": z, "p": p, "idx": sel, "w": O.gate_weights(p, sel, wl.renorm), "sel_bias": sb.astype(np.float64)}
    gpu = {"probs": PT.to_np(probs), "topk_idx": PT.to_np(idx), "topk_w": PT.to_np(w)}
    same = PT.compare_routing(wl, gpu, fwd)
    PT.say(f"[balance] full-size skewed router: identical routing for every token: {same}")
    plan.close()
