"""GPU parity of the MX-fp8 expert path: the quantiser bit for bit against
the oracle's MX rule, and the layer with MX experts against the oracle's
layer that MX-quantises the same expert GEMM operands, at the MX tolerance
(6e-2 x RMS), with the distance from the unquantised layer printed
alongside."""

import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from tests import parity as PT

pytestmark = pytest.mark.gpu

W = MI.Workload


def e4m3_value(code):
    """Value of an OCP e4m3 byte, from the format's definition (bias 7,
    3 mantissa bits, subnormals m * 2^-9)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 15
    m = code & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    assert not np.any((code & 0x7F) == 0x7F), "NaN code"
    return sign * mag


def test_mx_quantiser_matches_the_oracle_bit_for_bit():
    from mixture_experts_ffn_wave_amd import mx_quantize_rows
    rng = np.random.default_rng(3)
    R, K = 64, 512
    mag = np.exp2(rng.integers(-40, 40, size=(R, K // 32, 1)))          # a magnitude per block
    v = (rng.standard_normal((R, K // 32, 32)) * mag).reshape(R, K)
    v[0, :32] = 0.0                                                       # all-zero block
    v[1, :32] = 0.0; v[1, 5] = -3.0                                       # single value
    v[2, :32] = 448.0; v[2, 7] = -448.0                                   # amax exactly 448
    v[3, :32] = np.linspace(-1, 1, 32) * 1e-3                             # small values, subnormal codes
    v[4, :32] = 1.0 + np.arange(32) / 8.0                                 # e4m3 grid points and ties
    v[5, 32:64] = np.exp2(-np.arange(32, dtype=np.float64))               # a wide range in one block
    x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    xc = x.cuda()
    pay = torch.empty(R, K, dtype=torch.uint8, device="cuda")
    sc = torch.empty(R, K // 32, dtype=torch.uint8, device="cuda")
    mx_quantize_rows(xc, pay, sc)
    torch.cuda.synchronize()
    xv = x.to(torch.float64).numpy().reshape(R, K // 32, 32)
    ex = O.mx_block_scale(np.abs(xv).max(axis=-1))
    assert np.array_equal(sc.cpu().numpy().astype(np.int64) - 127, ex), "scale exponents"
    ref = O.e4m3_round(xv / np.exp2(ex)[..., None]).reshape(R, K)
    got = e4m3_value(pay.cpu().numpy())
    assert np.array_equal(got, ref), f"payload differs at {np.argwhere(got != ref)[:5]}"


SMALL_MX = [
    W("t1200_d256_e8k2_i256_mx", T=1200, d=256, E=8, k=2, I=256, expert_dtype="mxfp8"),
    # skewed segments (Zipf bias): one expert far above the mean, several below 32 tokens
    W("t1536_d256_e32k4_i128_zipf_mx", T=1536, d=256, E=32, k=4, I=128, zipf_s=1.1, expert_dtype="mxfp8"),
    W("t900_d256_e16k4_i384_s2x128_mx", T=900, d=256, E=16, k=4, I=384, n_shared=2, I_shared=128,
      expert_dtype="mxfp8"),
    W("t2049_d512_e4k2_i512_s1x256_mx", T=2049, d=512, E=4, k=2, I=512, n_shared=1, I_shared=256,
      expert_dtype="mxfp8"),
]


@pytest.mark.parametrize("wl", SMALL_MX, ids=[w.name for w in SMALL_MX])
def test_mx_layer_matches_oracle(wl):
    PT.full_parity(wl)


# The 256 x 256 MX tiles (8 waves) of the forward GEMMs, the gate/up dgrad
# and the weight gradients (those whose two sides are multiples of 256),
# forced on shapes that span several tiles with ragged and skewed segments
# (the large workload takes them by default)
MX_256 = [SMALL_MX[0], SMALL_MX[1], SMALL_MX[3]]


@pytest.mark.parametrize("wl", MX_256, ids=[w.name for w in MX_256])
def test_mx_256_tiles_match_oracle(wl, monkeypatch):
    monkeypatch.setenv("MOE_ROW_TILE", "256")
    monkeypatch.setenv("MOE_WGRAD_TILE", "256")
    PT.full_parity(wl)


def test_mx_forced_empty_experts_write_zero_gradients():
    wl = W("t700_d256_e8k2_i256_mx_bias", T=700, d=256, E=8, k=2, I=256, n_shared=1, I_shared=128,
           expert_dtype="mxfp8")
    inp = MI.make_inputs(wl)
    b = torch.zeros(8, dtype=torch.float32)
    b[[2, 6]] = -1e4          # experts 2 and 6 never chosen
    inp["bias"] = b
    gpu, fwd, _, st = PT.full_parity(wl, inp)
    assert fwd["counts"][2] == 0 and fwd["counts"][6] == 0
    for e in (2, 6):
        assert not np.any(gpu["dw_gate_up"][e]) and not np.any(gpu["dw_down"][e])


def test_mx_empty_batch():
    wl = W("t0_d256_e4k2_i128_mx_shared1", T=0, d=256, E=4, k=2, I=128, n_shared=1, I_shared=128,
           expert_dtype="mxfp8")
    gpu = PT.gpu_run(wl, MI.make_inputs(wl))
    assert gpu["counts"].sum() == 0
    for key in ("dw_router", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"):
        assert not np.any(gpu[key]), key


def test_mx_empty_batch_fused_plan():
    """A fused-only plan with no tokens: every weight gradient written as zeros."""
    wl = W("t0_d256_e4k2_i128_mx_shared1_fused", T=0, d=256, E=4, k=2, I=128, n_shared=1, I_shared=128,
           expert_dtype="mxfp8")
    out = _mx_step(wl, MI.make_inputs(wl), True, store_h=False, fused=True)
    for key in ("dw_router", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"):
        assert not bool(out[key].any()), key


def test_mx_two_runs_are_bitwise_identical():
    wl = W("t900_d256_e16k4_i384_s2x128_mx_det", T=900, d=256, E=16, k=4, I=384, n_shared=2, I_shared=128,
           expert_dtype="mxfp8")
    inp = MI.make_inputs(wl)
    a = PT.gpu_run(wl, inp, intermediates=True)
    b = PT.gpu_run(wl, inp, intermediates=True)
    for key, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[key]), key


def test_mx_backward_without_kept_dgu():
    """By default an MX backward stores [dG | dU] and dY_perm only as their MX
    operands (dY_perm's token-axis codes from dy's rows gathered by
    perm_token and scaled by the routing weight): the act-dtype "dgu",
    "dgu_shared" and "dy_perm" regions keep what was there, and every gradient
    and every MX operand is bitwise what a backward that also stores them
    (moe_keep_intermediates) gives."""
    wl = W("t700_d256_e8k2_i256_s1x128_mx_nodgu", T=700, d=256, E=8, k=2, I=256, n_shared=1, I_shared=128,
           expert_dtype="mxfp8")
    inp = MI.make_inputs(wl)
    from mixture_experts_ffn_wave_amd import MoELayer, workspace_region
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    runs = []
    for keep in (False, True):
        layer = MoELayer(PT.plan_for(wl, inp.get("bias") is not None))
        layer.write_x_perm = True
        layer.set_params(dev["x"], dev["w_router"], dev["w_gate_up"], dev["w_down"],
                         ws_gate_up=dev.get("ws_gate_up"), ws_down=dev.get("ws_down"))
        if keep:
            layer.keep_intermediates()
        layer.forward()
        assert layer.mx_gather                   # the backward gets perm_token
        for n in ("dgu", "dgu_shared", "dy_perm"):
            layer.backward_intermediate(n).fill_(7.0)
        layer.backward(dev["dy"])
        torch.cuda.synchronize()
        off, nb = workspace_region(layer.plan, "mx_pad")
        end = int(layer.ws[off:off + nb].view(torch.int32)[-1])         # padded token axis in use
        A, I = wl.T * wl.k, wl.I
        mx = {}
        NI = wl.n_shared * wl.I_shared
        for n, rows in (("mx_dguq", A), ("mx_dgut", 2 * I), ("mx_sdguq", wl.T), ("mx_sdgut", 2 * NI),
                        ("mx_dyq", A), ("mx_dyt", wl.d)):
            for r in (n, n + ".scales"):
                off, nb = workspace_region(layer.plan, r)
                v = PT.to_np(layer.ws[off:off + nb]).reshape(rows, -1)
                # the routed token axis has headroom past the last segment, never written
                tok = n in ("mx_dgut", "mx_dyt")
                mx[r] = v[:, :end // (32 if r.endswith(".scales") else 1)] if tok else v
        runs.append((layer, {n: PT.to_np(t) for n, t in layer.grads.items()}, mx))
    (quiet, g0, m0), (kept, g1, m1) = runs
    for n in ("dgu", "dgu_shared", "dy_perm"):
        assert bool((quiet.backward_intermediate(n) == 7.0).all()), n
        assert not bool((kept.backward_intermediate(n) == 7.0).all()), n
    for n in g0:
        assert np.array_equal(g0[n], g1[n]), n
    for n in m0:
        assert np.array_equal(m0[n], m1[n]), n


def _mx_step(wl, inp, save, store_h=True, fused=False):
    from mixture_experts_ffn_wave_amd import MoELayer, Plan
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    if fused:                                   # a fused-only plan (smaller workspace)
        plan = Plan(wl.T, wl.d, wl.E, wl.k, wl.I, n_shared=wl.n_shared, d_ff_shared=wl.I_shared,
                    renorm=wl.renorm, has_router_bias=inp.get("bias") is not None, dtype=wl.torch_dtype,
                    aux_coef=wl.aux_coef, expert_dtype="mxfp8", router=wl.router, mx_fused=True)
    else:
        plan = PT.plan_for(wl, inp.get("bias") is not None)
    layer = MoELayer(plan)
    layer.mx_save = save
    layer.store_h = store_h
    b = dev.get("bias")
    layer.set_params(dev["x"], dev["w_router"], dev["w_gate_up"], dev["w_down"],
                     bias=(b.float() if b is not None else None),
                     ws_gate_up=dev.get("ws_gate_up"), ws_down=dev.get("ws_down"))
    layer.forward()
    layer.backward(dev["dy"])
    torch.cuda.synchronize()
    out = {n: getattr(layer, n).clone() for n in (("gu", "h", "y_perm", "y") if store_h else ("gu", "y_perm", "y"))}
    out.update({n: t.clone() for n, t in layer.grads.items() if t is not None})
    return out


SAVED_CASES = [(SMALL_MX[2], None), (SMALL_MX[3], None), (SMALL_MX[1], "256"), (SMALL_MX[3], "256")]


@pytest.mark.parametrize("wl,tile", SAVED_CASES, ids=[f"{w.name}-{t or 'auto'}" for w, t in SAVED_CASES])
def test_mx_saved_codes_change_nothing(wl, tile, monkeypatch):
    """The forward's saved codes (the weights along the backward's reduction
    axes, from the pass that makes the forward's row-wise codes; H along each
    expert's tokens, from the gate/up epilogue) are the codes the backward
    makes itself without them: every output and gradient is bitwise the same
    either way, on 128 x 128 and 256 x 256 gate/up tiles, and also when the
    forward then keeps H only as its codes (h = NULL)."""
    if tile:
        monkeypatch.setenv("MOE_ROW_TILE", tile)
    inp = MI.make_inputs(wl)
    a, b = _mx_step(wl, inp, True), _mx_step(wl, inp, False)
    for n in a:
        assert torch.equal(a[n], b[n]), n
    c = _mx_step(wl, inp, True, store_h=False)
    for n in c:
        assert torch.equal(a[n], c[n]), n
    f = _mx_step(wl, inp, True, store_h=False, fused=True)    # the fused-only plan
    for n in f:
        assert torch.equal(a[n], f[n]), n


def test_mx_gather_on_load_equals_the_x_perm_path():
    """The gate/up GEMM reading x's codes through perm_token, and the weight
    gradient gathering x's rows, quantise the same values as the x_perm path
    (x_perm[r] = x[perm_token[r]]), so every output is bitwise the same."""
    wl = W("t700_d256_e8k3_i256_s1x128_mx_gather", T=700, d=256, E=8, k=3, I=256, n_shared=1, I_shared=128,
           expert_dtype="mxfp8")
    inp = MI.make_inputs(wl)
    from mixture_experts_ffn_wave_amd import MoELayer
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    outs = []
    for gather in (True, False):
        layer = MoELayer(PT.plan_for(wl, inp.get("bias") is not None))
        layer.mx_gather = gather
        layer.store_h = True
        layer.set_params(dev["x"], dev["w_router"], dev["w_gate_up"], dev["w_down"],
                         bias=(dev["bias"].float() if inp.get("bias") is not None else None),
                         ws_gate_up=dev.get("ws_gate_up"), ws_down=dev.get("ws_down"))
        layer.forward()
        layer.backward(dev["dy"])
        torch.cuda.synchronize()
        o = {n: getattr(layer, n).clone() for n in ("gu", "h", "y_perm", "y", "gu_shared", "h_shared", "y_shared")}
        o.update({n: t.clone() for n, t in layer.grads.items() if t is not None})
        outs.append(o)
    for key, v in outs[0].items():
        assert torch.equal(v, outs[1][key]), key


@pytest.mark.timeout(900)
def test_mx_workload_full_size():
    PT.full_parity(MI.WORKLOADS["t16384_d2048_e64k6_i1408_s2x1408_mxfp8"], mx_diagnostic=False)


def test_mx_workload_full_size_default_path_is_the_checked_one():
    """At the full MX workload the fused-only plan the benchmark runs (saved
    codes, H kept only as codes, [dG | dU] and dY_perm not stored, the smaller
    workspace) gives bitwise the outputs and gradients of the path the parity
    tests check (no saved codes, H stored): it adds no arithmetic of its own."""
    wl = MI.WORKLOADS["t16384_d2048_e64k6_i1408_s2x1408_mxfp8"]
    inp = MI.make_inputs(wl)
    a = _mx_step(wl, inp, True, store_h=False, fused=True)
    b = _mx_step(wl, inp, False)
    for n in a:
        assert torch.equal(a[n], b[n]), n
