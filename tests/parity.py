"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the fp64 oracle on the same seeded inputs, compare.

Reference.  f32, f16 and bf16 layers are compared with the exact fp64 oracle
(no rounding anywhere in it).  The fp64 oracle run with the layer's storage
rounding (``store``) is printed beside it as a diagnostic only.

Tolerances, per output matrix and element (each expert's weight gradient is
its own matrix, as each expert is a separate parameter, with its RMS floored
at the RMS of the whole stacked gradient):
  |gpu - oracle| <= c * RMS(oracle tensor) + ulp(value) / 2
  with c = 2e-2 for bf16 / f16 storage (the layer's stated bar) and c = 1e-4
  for f32 storage (f32 MFMA products, f32 intermediates).  The half-ulp term
  is the rounding of the result into its storage dtype, which no
  implementation that returns that dtype can avoid: for bf16 it alone reaches
  2^-8 of an element just above a power of two, i.e. about 2.2% of the RMS at
  the largest elements of these tensors.  The raw max|err|/RMS and the excess
  over the half ulp are reported too.  Router probabilities and
  routing weights within 1e-6 absolute; routing indices, counts, offsets,
  permutation and inverse permutation bit-exact, except tokens whose oracle
  logits tie within 1e-5 (set or slot order), whose GPU choice must only be a
  valid top-k within that margin.

MX-fp8 experts (KohakUwULLM README, "Key features"): see full_parity.
"""

import sys

import numpy as np
import torch

import moe_inputs as MI
import oracle as O

TIE_EPS = 1e-5
PROB_ATOL = 1e-6
# Sinkhorn router: ties are judged on ln(p_te b_e); the GPU's column scales
# carry f32 rounding of T-term sums over several rounds (measured under 5e-7 relative)
SINKHORN_TIE_EPS = 5e-5
SINKHORN_B_RTOL = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_tol(wl):
    if wl.expert_dtype == "mxfp8":
        return 6e-2
    return 1e-4 if wl.dtype == "f32" else 2e-2


# MX-fp8 layers.  Step-wise: every GEMM step of the oracle run on the inputs
# the GPU step received (quantised by the oracle from the GPU's stored
# values, which the bit-exact code tests show the GPU quantises identically),
# so only f32 against fp64 accumulation separates the two.
MX_STEP_TOL = 2e-3
# End to end against the oracle's whole MX layer (bf16 storage, no GPU value
# in it): a stored value one bf16 ulp away from the oracle's (f32 against fp64
# accumulation) lands on a neighbouring e4m3 code now and then, and at a
# block's largest value moves the block's scale, so single elements can
# differ by a code step; the criterion is on the bulk of the tensor:
# relative Frobenius distance <= MX_E2E_FRO and the 99.9th percentile of
# (|err| - ulp/2) <= MX_E2E_P999 x RMS.
MX_E2E_FRO = 2e-2
MX_E2E_P999 = 6e-2


def gu_dtype(wl):
    """Storage of the saved [G | U] (include/moe.h, moe_ffn_args)."""
    if wl.expert_dtype == "mxfp8":
        return "bf16"
    return "f32" if wl.dtype == "bf16" else wl.dtype


def y_perm_dtype(wl):
    if wl.expert_dtype == "mxfp8":
        return "bf16"
    return "f32" if wl.dtype == "bf16" else wl.dtype


def plan_for(wl, has_bias):
    from mixture_experts_ffn_wave_amd import Plan
    return Plan(wl.T, wl.d, wl.E, wl.k, wl.I, n_shared=wl.n_shared, d_ff_shared=wl.I_shared,
                renorm=wl.renorm, has_router_bias=has_bias, dtype=wl.torch_dtype, aux_coef=wl.aux_coef,
                expert_dtype=wl.expert_dtype or None, router=wl.router)


def to_np(t):
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype in (torch.int32, torch.int64):
        return t.to(torch.int64).numpy()
    return t.to(torch.float64).numpy()


def gpu_run(wl, inp, routing=None, intermediates=False, sel_bias=None, mask=None, extra=(), sinkhorn=None):
    """One fwd+bwd step on cuda:0.  ``routing`` (probs, idx, w as numpy) replaces
    the router's outputs when given (then moe_route is not called).
    ``intermediates`` also returns what the backward left in the workspace
    (dy_perm, dgu, dx_perm and, with shared experts, dgu_shared, dx_shared).
    ``sel_bias`` (numpy [E]) routes with aux-loss-free balancing; ``mask``
    (numpy [T], 0 = filler) takes the balancing statistic over real tokens.
    ``extra`` names further workspace intermediates to return ("wh",
    "dgu_lo", "wh_lo").  ``sinkhorn`` (rounds) routes with the Sinkhorn
    router."""
    from mixture_experts_ffn_wave_amd import MoELayer, decode_aux
    b = inp.get("bias")
    plan = plan_for(wl, b is not None)
    layer = MoELayer(plan)
    layer.write_x_perm = True                  # compared with the oracle's gather
    layer.store_h = True                       # (MX layers keep H only as codes otherwise)
    if intermediates:
        layer.keep_intermediates()             # MX plans: also store [dG | dU] in the act dtype
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    layer.set_params(dev["x"], dev["w_router"], dev["w_gate_up"], dev["w_down"],
                     bias=(dev["bias"].float() if b is not None else None),
                     ws_gate_up=dev.get("ws_gate_up"), ws_down=dev.get("ws_down"))
    if sel_bias is not None:
        layer.enable_balancing(torch.from_numpy(np.asarray(sel_bias, dtype=np.float32)).cuda())
    if sinkhorn is not None:
        layer.enable_sinkhorn(sinkhorn)
    if mask is not None:
        layer.set_real_mask(torch.from_numpy(np.asarray(mask, dtype=np.int32)).cuda())
    if routing is None:
        layer.forward()
    else:
        layer.probs.copy_(torch.from_numpy(routing["p"]).to(torch.float32))
        layer.topk_idx.copy_(torch.from_numpy(routing["idx"]).to(torch.int32))
        layer.topk_w.copy_(torch.from_numpy(routing["w"]).to(torch.float32))
        layer.dispatch_and_experts()
    if mask is not None:
        layer.aux_stats()                   # the masked backward needs the real tokens' counts
        layer.backward(dev["dy"])
    else:
        layer.backward(dev["dy"])
        layer.aux_stats()
    torch.cuda.synchronize()
    out = {n: to_np(getattr(layer, n)) for n in
           ["probs", "topk_idx", "topk_w", "counts", "offsets", "perm_token", "inv_perm", "x_perm", "gu",
            "h", "y_perm", "y", "gu_shared", "h_shared", "y_shared", "f", "p_mean"]}
    for n, t in layer.grads.items():
        out[n] = to_np(t)
    out["aux"] = decode_aux(layer.aux_out)
    if sinkhorn is not None and routing is None:
        out["sinkhorn_b"] = to_np(layer.sinkhorn_b)
    if mask is not None:
        out["real_counts"] = to_np(layer.real_counts)
    if intermediates:
        names = ["dy_perm", "dgu", "dx_perm"] + (["dgu_shared", "dx_shared"] if wl.n_shared else []) + list(extra)
        for n in names:
            out[n] = to_np(layer.backward_intermediate(n))
    return out


def oracle_inputs(inp):
    return {k: MI.to_f64(v) for k, v in inp.items()}


def storage_rounding(wl):
    """The ``store`` rounding of a layer whose values are kept in wl.dtype
    (kind "f32": the router's dz and Y_perm stay in f32; an MX layer keeps
    Y_perm in bf16, whose half-ulp rounding its comparisons allow)."""
    return lambda a, kind: O.round_to_format(a, "f32" if kind == "f32" else wl.dtype)


def oracle_run(wl, f64, store=None, quant=None, sel_bias=None, mask=None, sinkhorn=None):
    b = f64.get("bias")
    fwd = O.layer_forward(f64["x"], f64["w_router"], f64["w_gate_up"], f64["w_down"], top_k=wl.k,
                          renorm=wl.renorm, bias=b, ws_gate_up=f64.get("ws_gate_up"),
                          ws_down=f64.get("ws_down"), store=store, quant=quant,
                          sel_bias=None if sel_bias is None else np.asarray(sel_bias, dtype=np.float64),
                          sinkhorn_iters=sinkhorn, router=wl.router)
    bwd = O.layer_backward(fwd, f64["dy"], aux_coef=wl.aux_coef, quant=quant, mask=mask)
    if mask is None:
        st = O.aux_statistics(fwd["p"], fwd["counts"], wl.k)
    else:
        rc, tr = O.real_token_counts(fwd["idx"], mask, wl.E)
        st = O.aux_statistics(fwd["p"], rc, wl.k, mask)
        st["real_counts"] = np.concatenate([rc, [tr]])
    return fwd, bwd, st


MANTISSA_BITS = {"f32": 23, "f16": 10, "bf16": 7}
MIN_EXP = {"f32": -126, "f16": -14, "bf16": -126}


def half_ulp(v, dtype):
    """Half a unit in the last place of |v| in ``dtype`` (normal and subnormal range)."""
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex - 1, MIN_EXP[dtype])
    return np.ldexp(0.5, e - MANTISSA_BITS[dtype])


REPORT = []


STRICT = [True]


def check_close(name, got, ref, c, dtype="f32", ulps=0.5, rms_floor=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:
        return 0.0, 0.0
    diff = np.abs(got - ref)
    rms = max(float(np.sqrt(np.mean(ref * ref))), rms_floor)
    excess = diff - 2.0 * ulps * half_ulp(np.maximum(np.abs(got), np.abs(ref)), dtype)
    err = float(diff.max())
    worst = float(excess.max())
    REPORT.append((name, err / rms if rms > 0 else 0.0, worst / rms if rms > 0 else 0.0))
    if not STRICT[0]:
        return err, rms
    assert worst <= c * rms + 1e-30, (f"{name}: max(|err| - ulp/2) {worst:.3e} > {c:g} x RMS {rms:.3e} "
                                      f"(raw max|err| {err:.3e} = {err / max(rms, 1e-300):.4f} RMS)")
    return err, rms


def compare_routing(wl, gpu, fwd):
    """Returns True when the GPU chose exactly the oracle's routing for every
    token; asserts that any difference is an allowed near-tie.  The ranked
    values are the logits, or probability + selection bias when balancing."""
    eps = TIE_EPS
    if wl.router == "relu":
        return _compare_relu_routing(wl, gpu, fwd)
    if wl.router == "expert_choice":
        return _compare_expert_choice_routing(wl, gpu, fwd)
    if fwd.get("sinkhorn_b") is not None:
        # Sinkhorn router: scales first, then ranks on ln(p b)
        if "sinkhorn_b" in gpu:
            b_ref = fwd["sinkhorn_b"]
            rel = np.max(np.abs(gpu["sinkhorn_b"] - b_ref) / np.abs(b_ref))
            assert rel <= SINKHORN_B_RTOL, f"Sinkhorn column scales: max relative error {rel:.3e}"
        z = np.log(O.sinkhorn_selection_scores(fwd["p"], fwd["sinkhorn_b"]))
        eps = SINKHORN_TIE_EPS
    else:
        z = fwd["z"] if fwd.get("sel_bias") is None else O.balanced_selection_scores(fwd["p"], fwd["sel_bias"])
    k, E = wl.k, wl.E
    assert np.max(np.abs(gpu["probs"] - fwd["p"])) <= PROB_ATOL, "router probabilities"
    gi = gpu["topk_idx"]
    same = np.all(gi == fwd["idx"], axis=1)
    set_tie, order_tie = O.near_tie_tokens(z, k, eps)
    bad = ~same & ~(set_tie | order_tie)
    assert not bad.any(), f"routing differs on {int(bad.sum())} non-tied tokens, e.g. {np.where(bad)[0][:5]}"
    for t in np.where(~same)[0]:
        sel = gi[t]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < E
        zs = z[t, sel]
        assert np.all(np.diff(zs) <= eps), f"token {t}: slot order not descending"
        rest = np.setdiff1d(np.arange(E), sel)
        if rest.size:
            assert zs.min() >= z[t, rest].max() - eps, f"token {t}: not a top-k"
    if same.any():
        assert np.max(np.abs(gpu["topk_w"][same] - fwd["w"][same])) <= PROB_ATOL, "routing weights"
    return bool(same.all())


RELU_ATOL = 1e-5      # gates are f32 logits (f32 accumulation over d): relative to max(1, |gate|)


def _compare_relu_routing(wl, gpu, fwd):
    """The ReLU router: gates max(z, 0) against the oracle's, and the choice
    (the k largest positive logits, -1 past them) bit-exact except tokens
    whose choice a near-tie decides: the k-th and (k+1)-th logits within
    TIE_EPS, or a logit within TIE_EPS of zero (its sign decides whether it
    may be chosen); those must hold a valid choice within that margin."""
    z, k, E = fwd["z"], wl.k, wl.E
    g_ref = fwd["p"]
    assert np.max(np.abs(gpu["probs"] - g_ref) / np.maximum(1.0, np.abs(g_ref))) <= RELU_ATOL, "ReLU gates"
    gi = gpu["topk_idx"]
    same = np.all(gi == fwd["idx"], axis=1)
    set_tie, order_tie = O.near_tie_tokens(z, k, TIE_EPS)
    tie = set_tie | order_tie | (np.abs(z) < TIE_EPS).any(axis=1)
    bad = ~same & ~tie
    assert not bad.any(), f"ReLU routing differs on {int(bad.sum())} non-tied tokens, e.g. {np.where(bad)[0][:5]}"
    for t in np.where(~same)[0]:
        sel = gi[t][gi[t] >= 0]
        assert np.all(gi[t][len(sel):] == -1), f"token {t}: empty slots not last"
        assert len(set(sel.tolist())) == len(sel) and (sel.size == 0 or sel.max() < E)
        zs = z[t, sel]
        assert np.all(zs > -TIE_EPS) and np.all(np.diff(zs) <= TIE_EPS), f"token {t}: not positive / descending"
        rest = np.setdiff1d(np.arange(E), sel)
        bound = zs.min() if len(sel) == k else 0.0
        if rest.size:
            assert z[t, rest].max() <= bound + TIE_EPS, f"token {t}: a larger positive logit left out"
    if same.any():
        w = fwd["w"][same]
        assert np.max(np.abs(gpu["topk_w"][same] - w) / np.maximum(1.0, np.abs(w))) <= RELU_ATOL, "ReLU weights"
    return bool(same.all())


def _compare_expert_choice_routing(wl, gpu, fwd):
    """Expert choice: probabilities within PROB_ATOL; every expert takes
    exactly C tokens; the [T, E] slots bit-exact except tokens whose
    probability for some expert lies within TIE_EPS of that expert's C-th
    largest (the expert's choice is decided by a near-tie there): their
    slots must still be a valid choice within that margin."""
    p, T, E = fwd["p"], wl.T, wl.E
    C = (T * wl.k) // E
    assert np.max(np.abs(gpu["probs"] - p)) <= PROB_ATOL, "router probabilities"
    gi = gpu["topk_idx"]
    assert gi.shape == (T, E)
    assert np.all((gi == np.arange(E)[None, :]) | (gi == -1)), "slot e holds e or -1"
    assert np.all((gi >= 0).sum(axis=0) == C), "every expert takes C tokens"
    same = np.all(gi == fwd["idx"], axis=1)
    srt = -np.sort(-p, axis=0)
    thr = srt[C - 1] if C > 0 else np.full(E, np.inf)
    tie = (np.abs(p - thr[None, :]) < TIE_EPS).any(axis=1)
    bad = ~same & ~tie
    assert not bad.any(), f"expert choice differs on {int(bad.sum())} non-tied tokens, e.g. {np.where(bad)[0][:5]}"
    taken = gi >= 0
    assert np.all(p[taken] >= np.broadcast_to(thr, p.shape)[taken] - TIE_EPS), "a taken token below the C-th"
    assert np.all(p[~taken] <= np.broadcast_to(thr, p.shape)[~taken] + TIE_EPS), "a left token above the C-th"
    if same.any():
        assert np.max(np.abs(gpu["topk_w"][same] - fwd["w"][same])) <= PROB_ATOL, "routing weights"
    return bool(same.all())


def compare_dispatch(gpu, fwd):
    """Integer work and the gather: bit-exact (over the offsets[E] real rows:
    the ReLU router's empty slots are no assignment)."""
    n = int(fwd["offsets"][-1])
    assert np.array_equal(gpu["counts"], fwd["counts"]), "counts"
    assert np.array_equal(gpu["offsets"], fwd["offsets"]), "offsets"
    assert np.array_equal(gpu["perm_token"][:n], fwd["perm_token"]), "perm_token"
    assert np.array_equal(gpu["inv_perm"], fwd["inv"]), "inv_perm"
    assert np.array_equal(gpu["x_perm"][:n], fwd["x_perm"]), "x_perm is a pure copy"


def compare_stats(gpu, st, p_atol=PROB_ATOL):
    """Balancing statistic and router metrics (and, over real tokens, their
    counts: integers, bit-exact).  ``p_atol``: of the mean probability (the
    ReLU router's mean gate: relative to max(1, value))."""
    if "real_counts" in st:
        assert np.array_equal(gpu["real_counts"], st["real_counts"]), "real-token counts"
    assert np.allclose(gpu["f"], st["f"], rtol=1e-6, atol=0), "f"
    assert np.max(np.abs(gpu["p_mean"] - st["p_mean"]) / np.maximum(1.0, np.abs(st["p_mean"]))) <= p_atol, "p_mean"
    a = gpu["aux"]
    assert abs(a["aux"] - st["aux"]) <= 1e-5 * max(1.0, abs(st["aux"])), ("aux", a["aux"], st["aux"])
    assert abs(a["aux_raw"] - st["aux_raw"]) <= 1e-5 * max(1.0, abs(st["aux_raw"]))
    assert abs(a["entropy_mean"] - st["entropy_mean"]) <= 1e-5 * max(1.0, abs(st["entropy_mean"]))
    assert abs(a["count_cv"] - st["count_cv"]) <= 1e-5 * max(1.0, abs(st["count_cv"]))
    assert a["count_min"] == st["count_min"] and a["count_max"] == st["count_max"]
    assert a["n_unused"] == st["n_unused"]


def compare_downstream(wl, gpu, fwd, bwd, st, rounded=False):
    """``rounded``: the reference holds its stored intermediates rounded to
    the storage format too; both sides of those comparisons then carry up to
    half an ulp of rounding, so they are allowed one ulp."""
    c = rel_tol(wl)
    dt = wl.dtype
    gdt, ydt = gu_dtype(wl), y_perm_dtype(wl)
    ku = 1.0 if rounded else 0.5
    compare_dispatch(gpu, fwd)
    inter = wl.I
    n = int(fwd["offsets"][-1])                     # real rows
    check_close("G", gpu["gu"][:n, :inter], fwd["g"], c, gdt, ku)
    check_close("U", gpu["gu"][:n, inter:], fwd["u"], c, gdt, ku)
    check_close("H", gpu["h"][:n], fwd["h"], c, dt, ku)
    check_close("Y_perm", gpu["y_perm"][:n], fwd["y_perm"], c, ydt, ku)
    if wl.n_shared:
        Is = wl.I_shared
        for s, (gs, us, hs) in enumerate(fwd["shared"]):
            check_close(f"G_shared[{s}]", gpu["gu_shared"][:, 2 * s * Is:2 * s * Is + Is], gs, c, gdt, ku)
            check_close(f"U_shared[{s}]", gpu["gu_shared"][:, 2 * s * Is + Is:2 * (s + 1) * Is], us, c, gdt, ku)
            check_close(f"H_shared[{s}]", gpu["h_shared"][:, s * Is:(s + 1) * Is], hs, c, dt, ku)
        check_close("Y_shared", gpu["y_shared"], fwd["y_shared"], c, dt, ku)
    check_close("y", gpu["y"], fwd["y"], c, dt)
    check_close("dx", gpu["dx"], bwd["dx"], c, dt)
    check_close("dW_router", gpu["dw_router"], bwd["dw_router"], c, dt)
    check_close("dbias", gpu["dbias"], bwd["dbias"], c, "f32")
    # each expert's weight is its own parameter matrix: compared at the scale
    # of its own gradient, but never at a finer scale than the whole stacked
    # output's (an expert that saw a handful of tokens has a gradient far
    # below that scale, made of a few rank-1 terms)
    fl_gu = float(np.sqrt(np.mean(bwd["dw_gate_up"] ** 2)))
    fl_d = float(np.sqrt(np.mean(bwd["dw_down"] ** 2)))
    for e in range(wl.E):
        check_close(f"dW_gate_up[{e}]", gpu["dw_gate_up"][e], bwd["dw_gate_up"][e], c, dt, rms_floor=fl_gu)
        check_close(f"dW_down[{e}]", gpu["dw_down"][e], bwd["dw_down"][e], c, dt, rms_floor=fl_d)
    empty = np.where(fwd["counts"] == 0)[0]
    for e in empty:
        assert not np.any(gpu["dw_gate_up"][e]) and not np.any(gpu["dw_down"][e]), f"empty expert {e} grads"
    if wl.n_shared:
        for s_ in range(wl.n_shared):
            check_close(f"dWs_gate_up[{s_}]", gpu["dws_gate_up"][s_], bwd["dws_gate_up"][s_], c, dt)
            check_close(f"dWs_down[{s_}]", gpu["dws_down"][s_], bwd["dws_down"][s_], c, dt)
    compare_stats(gpu, st, RELU_ATOL if wl.router == "relu" else PROB_ATOL)


def compare_mx_stepwise(wl, gpu, fwd, f64, st):
    """An MX layer, one GEMM step at a time.  MX quantisation turns each
    stored value into a code, and a value one storage ulp away from the
    oracle's can land on the next code (or, at a block's largest value, on
    the next block scale); such a step is correct for its own input, yet
    the change travels down the chain.  So every step after the first is
    checked on the inputs the GPU step received: the oracle's step function
    runs on the GPU's stored G, U, H, Y_perm, dY_perm, [dG | dU], dX_perm
    (and the shared experts' counterparts), quantising them itself."""
    c = MX_STEP_TOL
    dt = wl.dtype
    q = O.mx_fake_quant
    sr = storage_rounding(wl)
    I, E, k, d = wl.I, wl.E, wl.k, wl.d
    off = fwd["offsets"]
    inv = fwd["inv"]
    compare_dispatch(gpu, fwd)
    G, U, H = gpu["gu"][:, :I], gpu["gu"][:, I:], gpu["h"]
    # gate/up: its inputs (x_perm, the weights) are the oracle's own
    check_close("G", G, fwd["g"], c, dt, 1.0)
    check_close("U", U, fwd["u"], c, dt, 1.0)
    check_close("H", H, fwd["h"], c, dt, 1.0)
    y_perm = np.zeros_like(gpu["y_perm"])
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            y_perm[r0:r1] = sr(O.expert_down_step(H[r0:r1], f64["w_down"][e], q), "f32")
    check_close("Y_perm", gpu["y_perm"], y_perm, c, y_perm_dtype(wl), 1.0)
    y_shared = None
    if wl.n_shared:
        Is = wl.I_shared
        y_shared = np.zeros((wl.T, d))
        for s_, (gs, us, hs) in enumerate(fwd["shared"]):
            Gs = gpu["gu_shared"][:, 2 * s_ * Is:2 * s_ * Is + Is]
            Us = gpu["gu_shared"][:, 2 * s_ * Is + Is:2 * (s_ + 1) * Is]
            Hs = gpu["h_shared"][:, s_ * Is:(s_ + 1) * Is]
            check_close(f"G_shared[{s_}]", Gs, gs, c, dt, 1.0)
            check_close(f"U_shared[{s_}]", Us, us, c, dt, 1.0)
            check_close(f"H_shared[{s_}]", Hs, hs, c, dt, 1.0)
            y_shared += O.expert_down_step(Hs, f64["ws_down"][s_], q)
        check_close("Y_shared", gpu["y_shared"], sr(y_shared, "act"), c, dt, 1.0)
    w = gpu["topk_w"]
    check_close("y", gpu["y"], O.combine(gpu["y_perm"], inv, w, gpu.get("y_shared")), c, dt)

    # backward
    dy = f64["dy"]
    dy_perm = np.zeros_like(gpu["dy_perm"])
    dy_perm[inv.reshape(-1)] = sr((w[:, :, None] * dy[:, None, :]).reshape(-1, d), "act")
    check_close("dY_perm", gpu["dy_perm"], dy_perm, c, dt, 1.0)
    dgu = np.zeros_like(gpu["dgu"])
    dx_perm = np.zeros_like(gpu["dx_perm"])
    ref_dwgu = np.zeros_like(gpu["dw_gate_up"])
    ref_dwd = np.zeros_like(gpu["dw_down"])
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        dgu[r0:r1], ref_dwd[e] = O.expert_down_backward_step(gpu["dy_perm"][r0:r1], G[r0:r1], U[r0:r1],
                                                             H[r0:r1], f64["w_down"][e], q, sr)
        dxe, ref_dwgu[e] = O.expert_gate_up_backward_step(gpu["dgu"][r0:r1], gpu["x_perm"][r0:r1],
                                                          f64["w_gate_up"][e], q)
        dx_perm[r0:r1] = sr(dxe, "act")
    check_close("dGU", gpu["dgu"], dgu, c, dt, 1.0)
    check_close("dX_perm", gpu["dx_perm"], dx_perm, c, dt, 1.0)
    fl_gu = float(np.sqrt(np.mean(ref_dwgu ** 2)))
    fl_d = float(np.sqrt(np.mean(ref_dwd ** 2)))
    for e in range(E):
        check_close(f"dW_gate_up[{e}]", gpu["dw_gate_up"][e], ref_dwgu[e], c, dt, rms_floor=fl_gu)
        check_close(f"dW_down[{e}]", gpu["dw_down"][e], ref_dwd[e], c, dt, rms_floor=fl_d)
    for e in np.where(fwd["counts"] == 0)[0]:
        assert not np.any(gpu["dw_gate_up"][e]) and not np.any(gpu["dw_down"][e]), f"empty expert {e} grads"
    dx = np.zeros((wl.T, d))
    for j in range(k):
        dx += gpu["dx_perm"][inv[:, j]]
    if wl.n_shared:
        Is = wl.I_shared
        dxs = np.zeros((wl.T, d))
        for s_ in range(wl.n_shared):
            Gs = gpu["gu_shared"][:, 2 * s_ * Is:2 * s_ * Is + Is]
            Us = gpu["gu_shared"][:, 2 * s_ * Is + Is:2 * (s_ + 1) * Is]
            Hs = gpu["h_shared"][:, s_ * Is:(s_ + 1) * Is]
            dgs, dwsd = O.expert_down_backward_step(dy, Gs, Us, Hs, f64["ws_down"][s_], q, sr)
            check_close(f"dGU_shared[{s_}]", gpu["dgu_shared"][:, 2 * s_ * Is:2 * (s_ + 1) * Is], dgs, c, dt, 1.0)
            check_close(f"dWs_down[{s_}]", gpu["dws_down"][s_], dwsd, c, dt)
            dxs_s, dwsgu = O.expert_gate_up_backward_step(gpu["dgu_shared"][:, 2 * s_ * Is:2 * (s_ + 1) * Is],
                                                          f64["x"], f64["ws_gate_up"][s_], q)
            check_close(f"dWs_gate_up[{s_}]", gpu["dws_gate_up"][s_], dwsgu, c, dt)
            dxs += dxs_s
        check_close("dX_shared", gpu["dx_shared"], sr(dxs, "act"), c, dt, 1.0)
        dx += gpu["dx_shared"]
    # router: from the GPU's probabilities, weights and expert output rows
    _, dz = O.router_backward(dy, gpu["y_perm"], inv, gpu["probs"], fwd["idx"], w, wl.renorm,
                              fwd["counts"], wl.aux_coef, sr)
    check_close("dW_router", gpu["dw_router"], dz.T @ f64["x"], c, dt)
    check_close("dbias", gpu["dbias"], dz.sum(axis=0), c, "f32")
    check_close("dx", gpu["dx"], dx + dz @ f64["w_router"], c, dt)
    compare_stats(gpu, st)


def compare_mx_end_to_end(wl, gpu, fwd, bwd):
    """An MX layer against the oracle's whole MX layer (bf16 storage; no GPU
    value enters it): the MX_E2E_* criterion on every stored intermediate and
    every output."""
    dt = wl.dtype
    pairs = [("G", gpu["gu"][:, :wl.I], fwd["g"], dt), ("U", gpu["gu"][:, wl.I:], fwd["u"], dt),
             ("H", gpu["h"], fwd["h"], dt), ("Y_perm", gpu["y_perm"], fwd["y_perm"], y_perm_dtype(wl)),
             ("y", gpu["y"], fwd["y"], dt), ("dx", gpu["dx"], bwd["dx"], dt),
             ("dW_router", gpu["dw_router"], bwd["dw_router"], dt), ("dbias", gpu["dbias"], bwd["dbias"], "f32"),
             ("dW_gate_up", gpu["dw_gate_up"], bwd["dw_gate_up"], dt), ("dW_down", gpu["dw_down"], bwd["dw_down"], dt)]
    if wl.n_shared:
        pairs += [("Y_shared", gpu["y_shared"], fwd["y_shared"], dt),
                  ("dWs_gate_up", gpu["dws_gate_up"], bwd["dws_gate_up"], dt),
                  ("dWs_down", gpu["dws_down"], bwd["dws_down"], dt)]
    out = {}
    for name, got, ref, sdt in pairs:
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape and np.all(np.isfinite(got)), name
        if ref.size == 0:
            continue
        rms = float(np.sqrt(np.mean(ref * ref)))
        fro = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
        exc = np.abs(got - ref) - half_ulp(np.maximum(np.abs(got), np.abs(ref)), sdt)
        p999 = float(np.quantile(exc, 0.999)) / max(rms, 1e-300)
        out[name] = (fro, p999)
        assert fro <= MX_E2E_FRO and p999 <= MX_E2E_P999, (
            f"{name}: relative Frobenius {fro:.4f} (bar {MX_E2E_FRO}), 99.9th percentile {p999:.4f} x RMS "
            f"(bar {MX_E2E_P999}) against the oracle's MX layer")
    return out


def _report(wl, tag):
    worst = {}
    for n, r, e in REPORT:
        key = n.split("[")[0]
        a = worst.get(key, (0.0, 0.0))
        worst[key] = (max(a[0], r), max(a[1], e))
    say(f"[parity] {wl.name}: {tag}, max|err|/RMS raw/excess " +
        " ".join(f"{n}={r:.4f}/{e:.4f}" for n, (r, e) in worst.items()))


def _diagnostic(fn):
    """Run a comparison without asserting (it fills REPORT)."""
    REPORT.clear()
    STRICT[0] = False
    try:
        fn()
    finally:
        STRICT[0] = True


def full_parity(wl, inp=None, mx_diagnostic=True, sel_bias=None, mask=None, sinkhorn=None):
    """The whole chain on the GPU against the oracle.  When a near-tie made
    the GPU pick a different (valid) routing, the downstream calls are run a
    second time from the oracle's routing so every later tensor is compared
    on identical assignments.

    f32 / f16 / bf16 experts: every tensor against the exact fp64 oracle
    (compare_downstream, asserted); for bf16 the oracle with the layer's
    storage rounding is printed beside it.

    MX-fp8 experts: (1) one GEMM step at a time (compare_mx_stepwise, at
    MX_STEP_TOL) against the oracle's MX-quantised steps on the inputs the
    GPU step received, (2) end to end against the oracle's whole MX layer
    (compare_mx_end_to_end, the MX_E2E_* criterion); ``mx_diagnostic`` also
    prints the distance from the exact, unquantised layer, which the method
    itself does not come within 6e-2 x RMS of (tests/golden
    mx_method_distance)."""
    if inp is None:
        inp = MI.make_inputs(wl)
    f64 = oracle_inputs(inp)
    say(f"[parity] {wl.name}: {MI.describe(wl)} -- GPU chain")
    mx = wl.expert_dtype == "mxfp8"
    gpu = gpu_run(wl, inp, intermediates=mx, sel_bias=sel_bias, mask=mask, sinkhorn=sinkhorn)
    say(f"[parity] {wl.name}: oracle" + (" (MX-quantised expert GEMM operands, bf16 storage)" if mx else " (exact)"))
    fwd, bwd, st = oracle_run(wl, f64, storage_rounding(wl) if mx else None,
                              quant=O.mx_fake_quant if mx else None, sel_bias=sel_bias, mask=mask,
                              sinkhorn=sinkhorn)
    identical = compare_routing(wl, gpu, fwd)
    if not identical:
        say(f"[parity] {wl.name}: near-tie routing differs; rerunning downstream from the oracle routing")
        gpu = gpu_run(wl, inp, routing={"p": fwd["p"], "idx": fwd["idx"], "w": fwd["w"]}, intermediates=mx,
                      mask=mask)
    REPORT.clear()
    if mx:
        compare_mx_stepwise(wl, gpu, fwd, f64, st)
        _report(wl, "MX step-wise")
        e2e = compare_mx_end_to_end(wl, gpu, fwd, bwd)
        say(f"[parity] {wl.name}: vs the whole MX oracle layer, relative Frobenius / p99.9 excess " +
            " ".join(f"{n}={a:.4f}/{b:.4f}" for n, (a, b) in e2e.items()))
        if mx_diagnostic:
            xf, xb, xs = oracle_run(wl, f64, sel_bias=sel_bias, mask=mask)
            _diagnostic(lambda: compare_downstream(wl, gpu, xf, xb, xs))
            _report(wl, "vs exact (unquantised) oracle, not asserted")
    else:
        compare_downstream(wl, gpu, fwd, bwd, st)
        _report(wl, "vs exact oracle")
        if wl.dtype == "bf16" and mx_diagnostic:
            rf, rb, rs = oracle_run(wl, f64, storage_rounding(wl), sel_bias=sel_bias, mask=mask,
                                    sinkhorn=sinkhorn)
            _diagnostic(lambda: compare_downstream(wl, gpu, rf, rb, rs, rounded=True))
            _report(wl, "vs storage-rounded oracle, not asserted")
    return gpu, fwd, bwd, st
