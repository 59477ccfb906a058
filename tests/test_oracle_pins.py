"""Pins of the fp64 oracle against things other than itself.

Each test fixes a part of the oracle by brute force (pure-Python loops with
math.exp), by a closed form, by an invariant the mathematics forces, by a
special case that reduces to a library routine (torch float64), by finite
differences, or by a figure the pages print.  A plausible slip anywhere in the
oracle (dropped term, wrong sign or index, transposed operand, wrong tie rule)
breaks at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(T=8, d=16, E=4, k=2, inter=8, n_shared=0, inter_s=8, seed=0, wscale=0.3, bias=False):
    rng = np.random.default_rng(seed)
    L = dict(
        x=rng.standard_normal((T, d)),
        w_router=wscale * rng.standard_normal((E, d)),
        w_gate_up=wscale * rng.standard_normal((E, 2 * inter, d)),
        w_down=wscale * rng.standard_normal((E, d, inter)),
        ws_gate_up=wscale * rng.standard_normal((n_shared, 2 * inter_s, d)) if n_shared else None,
        ws_down=wscale * rng.standard_normal((n_shared, d, inter_s)) if n_shared else None,
        bias=rng.standard_normal(E) if bias else None,
        dy=rng.standard_normal((T, d)),
    )
    return L


def fwd_of(L, k, renorm=True, quant=None):
    return O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=k,
                           renorm=renorm, bias=L["bias"], ws_gate_up=L["ws_gate_up"],
                           ws_down=L["ws_down"], quant=quant)


# ------------------------------------------------------------------ softmax

def test_softmax_rows_sum_to_one():
    z = np.random.default_rng(1).standard_normal((64, 13)) * 5
    p = O.softmax_rows(z)
    assert np.all(p > 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-12


def test_softmax_two_experts_is_logistic():
    # closed form: with two logits, p0 = 1 / (1 + exp(z1 - z0))
    z = np.random.default_rng(2).standard_normal((50, 2)) * 4
    p = O.softmax_rows(z)
    for t in range(50):
        ref = 1.0 / (1.0 + math.exp(z[t, 1] - z[t, 0]))
        assert abs(p[t, 0] - ref) < 1e-14


def test_softmax_shift_invariant_and_large_logits():
    z = np.array([[1000.0, 999.0, -1000.0]])
    p = O.softmax_rows(z)
    e = math.exp(-1.0)
    assert abs(p[0, 0] - 1 / (1 + e)) < 1e-14 and abs(p[0, 1] - e / (1 + e)) < 1e-14
    assert p[0, 2] == 0.0


# ------------------------------------------------------------------- top-k

def _brute_topk(row, k):
    # selection by repeated scanning: largest value, lowest index on ties
    chosen = []
    for _ in range(k):
        best = None
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best is None or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (8, 2), (8, 8), (16, 6), (128, 8)])
def test_topk_matches_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 31 + k)
    z = rng.integers(-3, 4, size=(40, E)).astype(np.float64)   # many exact ties
    idx = O.topk_select(z, k)
    for t in range(40):
        assert list(idx[t]) == _brute_topk(list(z[t]), k)


def test_topk_zero_router_picks_lowest_indices():
    L = rand_layer(T=16, E=8)
    z = O.router_logits(L["x"], np.zeros_like(L["w_router"]))
    idx = O.topk_select(z, 3)
    assert (idx == np.array([0, 1, 2])).all()


def test_router_bias_shifts_selection():
    x = np.zeros((3, 4))
    z = O.router_logits(x, np.zeros((5, 4)), bias=np.array([0.0, 2.0, 1.0, 3.0, -1.0]))
    assert list(O.topk_select(z, 3)[0]) == [3, 1, 2]


# ----------------------------------------------------------------- renorm

def test_renorm_rows_sum_to_one_and_match_softmax_over_selected():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((100, 16)) * 2
    p = O.softmax_rows(z)
    idx = O.topk_select(z, 4)
    w = O.gate_weights(p, idx, renorm=True)
    assert np.max(np.abs(w.sum(axis=1) - 1)) < 1e-12
    # identity: renormalised top-k probabilities == softmax over the selected logits
    for t in range(100):
        sel = [z[t, e] for e in idx[t]]
        m = max(sel)
        ex = [math.exp(v - m) for v in sel]
        s = sum(ex)
        for j in range(4):
            assert abs(w[t, j] - ex[j] / s) < 1e-14
    # without renorm the weights are the raw probabilities of the selected experts
    w0 = O.gate_weights(p, idx, renorm=False)
    assert np.array_equal(w0, np.take_along_axis(p, idx, axis=1))
    assert np.all(w0.sum(axis=1) < 1.0)


def test_k_equals_E_renorm_gives_full_softmax():
    z = np.random.default_rng(4).standard_normal((20, 6))
    p = O.softmax_rows(z)
    idx = O.topk_select(z, 6)
    w = O.gate_weights(p, idx, renorm=True)
    assert np.max(np.abs(w - np.take_along_axis(p, idx, axis=1))) < 1e-15


def test_near_tie_detection():
    z = np.array([[3.0, 2.0, 2.0 + 5e-6, 0.0],      # set tie between slot 2 and 3 for k=2
                  [3.0, 3.0 - 1e-6, 1.0, 0.0],      # order tie inside the set
                  [3.0, 2.0, 1.0, 0.0]])
    st, ot = O.near_tie_tokens(z, 2)
    assert list(st) == [True, False, False]
    assert list(ot) == [False, True, False]


# ------------------------------------------------------------ permutation

@pytest.mark.parametrize("E,k", [(4, 2), (8, 2), (16, 3), (5, 5)])
def test_permutation_properties(E, k):
    rng = np.random.default_rng(E + 7 * k)
    T = 37
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    counts, offsets, perm_token, inv = O.expert_permutation(idx, E)
    # counts by explicit tally
    tally = [0] * E
    for t in range(T):
        for j in range(k):
            tally[idx[t, j]] += 1
    assert list(counts) == tally
    assert offsets[0] == 0 and offsets[E] == T * k and np.all(np.diff(offsets) >= 0)
    # bijection, inverse and stability
    assert sorted(inv.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            r = inv[t, j]
            assert perm_token[r] == t
            e = idx[t, j]
            assert offsets[e] <= r < offsets[e + 1]
    for e in range(E):
        seg = perm_token[offsets[e]:offsets[e + 1]]
        assert all(seg[i] < seg[i + 1] for i in range(len(seg) - 1))
    x = rng.standard_normal((T, 5))
    xp = x[perm_token]
    for t in range(T):
        for j in range(k):
            assert np.array_equal(xp[inv[t, j]], x[t])


# ----------------------------------------------------- forward brute force

def _py_forward(L, k, renorm, sel_bias=None):
    """The whole forward with Python loops and math.exp, no numpy algebra.
    With sel_bias the experts are chosen on probability + bias (aux-loss-free
    balancing) and weighted by the unbiased probabilities."""
    x, Wr, Wgu, Wd = L["x"].tolist(), L["w_router"].tolist(), L["w_gate_up"].tolist(), L["w_down"].tolist()
    T, d, E, inter = len(x), len(x[0]), len(Wr), len(Wd[0][0])
    b = L["bias"].tolist() if L["bias"] is not None else [0.0] * E

    def dot(a, c):
        return sum(ai * ci for ai, ci in zip(a, c))

    def expert(xt, wgu, wd, I):
        h = []
        for i in range(I):
            gv = dot(xt, wgu[i])
            uv = dot(xt, wgu[I + i])
            h.append(gv / (1 + math.exp(-gv)) * uv)
        return [dot(h, wd[o]) for o in range(d)]

    ys = []
    for t in range(T):
        z = [dot(x[t], Wr[e]) + b[e] for e in range(E)]
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        s = sum(ex)
        p = [v / s for v in ex]
        sel = _brute_topk(z if sel_bias is None else [p[e] + sel_bias[e] for e in range(E)], k)
        wts = [p[e] for e in sel]
        if renorm:
            sw = sum(wts)
            wts = [v / sw for v in wts]
        y = [0.0] * d
        for e, wv in zip(sel, wts):
            ye = expert(x[t], Wgu[e], Wd[e], inter)
            y = [a + wv * c for a, c in zip(y, ye)]
        if L["ws_gate_up"] is not None:
            for s_ in range(len(L["ws_gate_up"])):
                ye = expert(x[t], L["ws_gate_up"][s_].tolist(), L["ws_down"][s_].tolist(),
                            L["ws_down"].shape[2])
                y = [a + c for a, c in zip(y, ye)]
        ys.append(y)
    return np.array(ys)


@pytest.mark.parametrize("k,renorm,n_shared,bias", [(2, True, 0, False), (2, False, 0, True),
                                                    (1, True, 1, False), (3, True, 2, True)])
def test_forward_matches_python_loops(k, renorm, n_shared, bias):
    L = rand_layer(T=6, d=8, E=4, k=k, inter=5, n_shared=n_shared, inter_s=3, seed=11 + k, bias=bias)
    fwd = fwd_of(L, k, renorm)
    ref = _py_forward(L, k, renorm)
    assert np.max(np.abs(fwd["y"] - ref)) < 1e-12 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("k,renorm", [(2, True), (3, False)])
def test_balanced_forward_matches_python_loops(k, renorm):
    L = rand_layer(T=6, d=8, E=5, k=k, inter=5, seed=40 + k)
    sb = [0.3, -0.2, 0.05, 0.0, -0.4]
    fwd = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=k, renorm=renorm,
                          sel_bias=np.array(sb))
    ref = _py_forward(L, k, renorm, sel_bias=sb)
    assert np.max(np.abs(fwd["y"] - ref)) < 1e-12 * max(1.0, np.abs(ref).max())


def test_zero_selection_bias_is_the_plain_router():
    # ranking probabilities ranks the logits (softmax is monotone per row)
    L = rand_layer(T=64, E=8, seed=5)
    z = O.router_logits(L["x"], L["w_router"])
    p = O.softmax_rows(z)
    assert (O.topk_select(O.balanced_selection_scores(p, np.zeros(8)), 3) == O.topk_select(z, 3)).all()


def test_large_selection_bias_forces_the_choice_not_the_weights():
    # probabilities lie in (0, 1), so a bias of 2 puts expert 5 first for every
    # token; its weight is still its own probability over the chosen ones
    L = rand_layer(T=32, E=8, seed=6)
    sb = np.zeros(8)
    sb[5] = 2.0
    fwd = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=2, renorm=True, sel_bias=sb)
    assert (fwd["idx"][:, 0] == 5).all()
    p = fwd["p"]
    for t in range(32):
        e1 = fwd["idx"][t, 1]
        assert e1 == max((e for e in range(8) if e != 5), key=lambda e: (p[t, e], -e))
        assert abs(fwd["w"][t, 0] - p[t, 5] / (p[t, 5] + p[t, e1])) < 1e-15


def test_balance_bias_update_hand_values():
    # T k = 30 over E = 3 experts: mean load 10; loads 12, 10, 8
    out = O.balance_bias_update([0.5, 0.0, -0.75], [12, 10, 8], T=10, top_k=3, gamma=0.25)
    assert out.dtype == np.float32 and list(out) == [0.25, 0.0, -0.5]
    # the bias is f32: 1 + 2^-30 rounds back to 1 (an f64 sum would not)
    assert O.balance_bias_update([1.0, 1.0], [0, 4], T=2, top_k=2, gamma=2.0 ** -30)[0] == np.float32(1.0)
    # a mean load that is not an integer: T k / E = 7 / 2
    assert list(O.balance_bias_update([0.0, 0.0], [4, 3], T=7, top_k=1, gamma=1.0)) == [-1.0, 1.0]


def test_bias_updates_balance_a_skewed_router():
    # the purpose of the method: with fixed, strongly skewed logits, repeated
    # updates drive the per-expert loads toward the mean without touching the
    # gate weights' source (the unbiased probabilities)
    rng = np.random.default_rng(7)
    T, E, k = 2048, 8, 2
    z = rng.standard_normal((T, E)) + np.log(1.0 / np.arange(1, E + 1) ** 1.2)[None, :]
    p = O.softmax_rows(z)
    b = np.zeros(E, dtype=np.float32)
    cv = []
    for _ in range(400):
        idx = O.topk_select(O.balanced_selection_scores(p, b), k)
        counts = np.bincount(idx.ravel(), minlength=E)
        cv.append(counts.std() / counts.mean())
        b = O.balance_bias_update(b, counts, T, k, gamma=1e-3)
    assert cv[0] > 0.5 and max(cv[-50:]) < 0.1 * cv[0]


def test_single_expert_top1_is_dense_swiglu_mlp():
    # E = 1, k = 1 reduces to a dense SwiGLU MLP: down(silu(gate x) * up x), here via torch float64
    L = rand_layer(T=32, d=24, E=1, k=1, inter=40, seed=5)
    fwd = fwd_of(L, 1)
    x = torch.from_numpy(L["x"])
    wg = torch.from_numpy(L["w_gate_up"][0, :40])
    wu = torch.from_numpy(L["w_gate_up"][0, 40:])
    wd = torch.from_numpy(L["w_down"][0])
    ref = F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd).numpy()
    assert np.max(np.abs(fwd["y"] - ref)) < 1e-13


def test_two_shared_experts_equal_one_of_double_width():
    L = rand_layer(T=10, d=12, E=4, k=2, inter=6, n_shared=2, inter_s=5, seed=8)
    y2, _ = O.shared_experts_forward(L["x"], L["ws_gate_up"], L["ws_down"])
    gu, dn = L["ws_gate_up"], L["ws_down"]
    wide_gu = np.concatenate([gu[0, :5], gu[1, :5], gu[0, 5:], gu[1, 5:]], axis=0)[None]
    wide_d = np.concatenate([dn[0], dn[1]], axis=1)[None]
    y1, _ = O.shared_experts_forward(L["x"], wide_gu, wide_d)
    assert np.max(np.abs(y1 - y2)) < 1e-13


def test_k_equals_E_is_dense_soft_mixture():
    L = rand_layer(T=9, d=10, E=3, k=3, inter=4, seed=9)
    fwd = fwd_of(L, 3, renorm=True)
    x = torch.from_numpy(L["x"])
    p = torch.softmax(x @ torch.from_numpy(L["w_router"]).T, dim=1)
    y = torch.zeros_like(x)
    for e in range(3):
        wg = torch.from_numpy(L["w_gate_up"][e, :4])
        wu = torch.from_numpy(L["w_gate_up"][e, 4:])
        wd = torch.from_numpy(L["w_down"][e])
        y += p[:, e:e + 1] * F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd)
    assert np.max(np.abs(fwd["y"] - y.numpy())) < 1e-13


def test_empty_expert_contributes_nothing():
    L = rand_layer(T=12, d=8, E=4, k=1, inter=4, seed=3)
    L["bias"] = np.array([0.0, 0.0, -1e9, 0.0])      # expert 2 never chosen
    fwd = fwd_of(L, 1)
    assert fwd["counts"][2] == 0
    bwd = O.layer_backward(fwd, L["dy"], aux_coef=0.01)
    assert np.all(bwd["dw_gate_up"][2] == 0) and np.all(bwd["dw_down"][2] == 0)


# --------------------------------------------------------------------- aux

def test_aux_zero_router_is_one():
    L = rand_layer(T=20, d=8, E=5, k=2, seed=4)
    L["w_router"] = np.zeros_like(L["w_router"])
    st = O.aux_statistics(fwd_of(L, 2)["p"], fwd_of(L, 2)["counts"], 2)
    assert abs(st["aux"] - 1.0) < 1e-14          # P_e = 1/E for all e, sum f = 1
    assert abs(st["entropy_mean"] - math.log(5)) < 1e-13


def test_aux_fully_concentrated_is_E_over_k():
    T, E, k = 16, 8, 2
    L = rand_layer(T=T, d=4, E=E, k=k, seed=6)
    L["w_router"] = np.zeros_like(L["w_router"])
    L["bias"] = np.array([0, 60.0, 0, 60.0, 0, 0, 0, 0])
    fwd = fwd_of(L, k)
    st = O.aux_statistics(fwd["p"], fwd["counts"], k)
    assert abs(st["aux"] - E / k) < 1e-12
    assert st["n_unused"] == E - k and st["count_min"] == 0 and st["count_max"] == T


def test_aux_balanced_counts_uniform_p():
    T, E, k = 8, 4, 2
    p = np.full((T, E), 1.0 / E)
    counts = np.array([4, 4, 4, 4])
    st = O.aux_statistics(p, counts, k)
    assert abs(st["aux"] - 1.0) < 1e-15 and st["count_cv"] == 0.0
    counts = np.array([8, 0, 4, 4])
    st = O.aux_statistics(p, counts, k)
    # coefficient of variation by hand: mean 4, population std sqrt((16+16+0+0)/4)
    assert abs(st["count_cv"] - math.sqrt(8.0) / 4.0) < 1e-15 and st["n_unused"] == 1


# ---------------------------------------------------------------- backward

def _min_gap(L, k):
    z = O.router_logits(L["x"], L["w_router"], L["bias"])
    s = -np.sort(-z, axis=1)
    gaps = [s[:, j] - s[:, j + 1] for j in range(min(k, s.shape[1] - 1))]
    return np.min(gaps)


def _fd_case(renorm, aux_coef, n_shared, seed):
    k = 2
    for sd in range(seed, seed + 200):
        L = rand_layer(T=8, d=16, E=4, k=k, inter=8, n_shared=n_shared, inter_s=8, seed=sd, wscale=0.3)
        if _min_gap(L, k) >= 1e-3:
            return L
    raise RuntimeError("no seed with separated logits")


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("aux_coef", [0.0, 0.5])
@pytest.mark.parametrize("n_shared", [0, 1])
def test_backward_matches_central_differences(renorm, aux_coef, n_shared):
    k = 2
    L = _fd_case(renorm, aux_coef, n_shared, seed=100 * n_shared + 17)
    fwd = fwd_of(L, k, renorm)
    g = O.layer_backward(fwd, L["dy"], aux_coef=aux_coef)
    names = {"x": "dx", "w_router": "dw_router", "w_gate_up": "dw_gate_up", "w_down": "dw_down"}
    if n_shared:
        names.update({"ws_gate_up": "dws_gate_up", "ws_down": "dws_down"})
    rng = np.random.default_rng(0)
    h = 1e-6
    for pname, gname in names.items():
        arr = L[pname]
        flat_idx = rng.choice(arr.size, size=min(arr.size, 48), replace=False)
        for fi in flat_idx:
            pos = np.unravel_index(fi, arr.shape)
            orig = arr[pos]
            arr[pos] = orig + h
            lp = O.layer_loss(fwd_of(L, k, renorm), L["dy"], aux_coef)
            arr[pos] = orig - h
            lm = O.layer_loss(fwd_of(L, k, renorm), L["dy"], aux_coef)
            arr[pos] = orig
            fd = (lp - lm) / (2 * h)
            an = g[gname][pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (pname, pos, fd, an)


@pytest.mark.parametrize("renorm", [True, False])
def test_masked_statistic_gradient_matches_central_differences(renorm):
    # the balancing statistic over the real tokens only: its gradient (only
    # real tokens' probabilities get the term) against finite differences of
    # the masked loss
    k, aux_coef = 2, 0.5
    L = _fd_case(renorm, aux_coef, 0, seed=23)
    T = L["x"].shape[0]
    mask = np.ones(T, dtype=np.int64)
    mask[1::3] = 0
    fwd = fwd_of(L, k, renorm)
    g = O.layer_backward(fwd, L["dy"], aux_coef=aux_coef, mask=mask)
    rng = np.random.default_rng(1)
    h = 1e-6
    for pname, gname in {"x": "dx", "w_router": "dw_router"}.items():
        arr = L[pname]
        for fi in rng.choice(arr.size, size=min(arr.size, 48), replace=False):
            pos = np.unravel_index(fi, arr.shape)
            orig = arr[pos]
            arr[pos] = orig + h
            lp = O.layer_loss(fwd_of(L, k, renorm), L["dy"], aux_coef, mask)
            arr[pos] = orig - h
            lm = O.layer_loss(fwd_of(L, k, renorm), L["dy"], aux_coef, mask)
            arr[pos] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[gname][pos]) <= 1e-6 * max(1.0, abs(g[gname][pos])), (pname, pos)


def test_masked_statistic_ignores_fillers():
    # fillers change nothing: the statistic of real tokens plus arbitrary
    # fillers under the mask equals the plain statistic of the real tokens
    rng = np.random.default_rng(9)
    T, E, k = 40, 6, 2
    p = O.softmax_rows(rng.standard_normal((T, E)) * 2)
    idx = O.topk_select(np.log(p), k)
    mask = (rng.random(T) < 0.6).astype(np.int64)
    rc, Tr = O.real_token_counts(idx, mask, E)
    assert Tr == mask.sum() and rc.sum() == Tr * k
    ref = O.aux_statistics(p[mask == 1], np.bincount(idx[mask == 1].ravel(), minlength=E), k)
    got = O.aux_statistics(p, rc, k, mask)
    for key in ("aux", "aux_raw", "entropy_mean", "count_cv", "count_min", "count_max", "n_unused"):
        assert abs(got[key] - ref[key]) < 1e-14, key
    assert np.allclose(got["f"], ref["f"], rtol=0, atol=1e-15) and np.allclose(got["p_mean"], ref["p_mean"],
                                                                                rtol=0, atol=1e-15)
    # all real: the unmasked statistic; none real: all zero
    full = O.aux_statistics(p, np.bincount(idx.ravel(), minlength=E), k)
    allm = O.aux_statistics(p, O.real_token_counts(idx, np.ones(T), E)[0], k, np.ones(T))
    assert abs(full["aux"] - allm["aux"]) < 1e-15
    none = O.aux_statistics(p, np.zeros(E), k, np.zeros(T))
    assert none["aux"] == 0.0 and none["entropy_mean"] == 0.0 and none["count_cv"] == 0.0


def test_masked_statistic_hand_values():
    # T = 4 tokens, 2 real (tokens 0 and 2), E = 2, k = 1
    p = np.array([[0.75, 0.25], [0.5, 0.5], [0.25, 0.75], [1.0, 0.0]])
    idx = np.array([[0], [0], [1], [0]])
    mask = np.array([1, 0, 1, 0])
    rc, Tr = O.real_token_counts(idx, mask, 2)
    assert rc.tolist() == [1, 1] and Tr == 2
    st = O.aux_statistics(p, rc, 1, mask)
    # f = (1/2, 1/2), P = ((0.75+0.25)/2, (0.25+0.75)/2) = (1/2, 1/2): aux_raw = 1/2, aux = 1
    assert st["aux_raw"] == 0.5 and st["aux"] == 1.0
    # gradient term only on real rows: aux_coef * E * f_e / T_r = 1 * 2 * 0.5 / 2 = 0.5
    _, dz = O.router_backward(np.zeros((4, 1)), np.zeros((4, 1)), np.arange(4).reshape(4, 1), p, idx,
                              np.ones((4, 1)), False, rc, aux_coef=1.0, mask=mask)
    # dp = 0.5 on both experts of a real row: dz = p * (dp - <p, dp>) = 0 there; 0 on fillers
    assert np.all(dz == 0.0)
    rc2 = np.array([2, 0])
    _, dz = O.router_backward(np.zeros((4, 1)), np.zeros((4, 1)), np.arange(4).reshape(4, 1), p, idx,
                              np.ones((4, 1)), False, rc2, aux_coef=1.0, mask=mask)
    # dp = (1, 0) on real rows: dz = p * ((1, 0) - p_0) -> token 0: (0.75 * 0.25, -0.25 * 0.75)
    assert np.allclose(dz[0], [0.1875, -0.1875], rtol=0, atol=1e-15) and np.all(dz[1] == 0) and np.all(dz[3] == 0)


def test_router_gradient_invariants():
    L = _fd_case(True, 0.0, 0, seed=300)
    fwd = fwd_of(L, 2, True)
    g0 = O.layer_backward(fwd, L["dy"], aux_coef=0.0)
    dz = g0["dz"]
    # rows of a softmax Jacobian product sum to zero
    assert np.max(np.abs(dz.sum(axis=1))) < 1e-14
    # with renormalisation and no aux term, unselected experts get no gradient
    mask = np.ones_like(dz, dtype=bool)
    np.put_along_axis(mask, fwd["idx"], False, axis=1)
    assert np.max(np.abs(dz[mask])) < 1e-15
    # without renormalisation they do
    fwd_n = fwd_of(L, 2, False)
    dzn = O.layer_backward(fwd_n, L["dy"], aux_coef=0.0)["dz"]
    assert np.max(np.abs(dzn[mask])) > 1e-6
    # gradients are linear in dy (aux off)
    g2 = O.layer_backward(fwd, 2.5 * L["dy"], aux_coef=0.0)
    for key in ("dx", "dw_router", "dw_gate_up", "dw_down"):
        assert np.max(np.abs(g2[key] - 2.5 * g0[key])) < 1e-12 * max(1, np.abs(g0[key]).max())


# ---------------------------------------------------------------------- MX

def test_e4m3_rounding_hand_vectors():
    v = np.array([0.0, 1.0, 1.0625, 1.125, 1.1875, 448.0, 460.0, 1000.0, 2.0 ** -9, 2.0 ** -10,
                  3 * 2.0 ** -10, 248.0, 240.0, -17.0, 2.0 ** -6 + 2.0 ** -10, 2.0 ** -6 + 3 * 2.0 ** -10])
    q = O.e4m3_round(v)
    # 1.0625 is halfway between 1.0 and 1.125 -> even mantissa 1.0; 1.1875 halfway 1.125/1.25 -> 1.25;
    # 2^-6 + 2^-10 is halfway in the first normal binade (spacing 2^-9) -> 2^-6, 2^-6 + 3*2^-10 -> up
    exp = [0.0, 1.0, 1.0, 1.125, 1.25, 448.0, 448.0, 448.0, 2.0 ** -9, 0.0,
           2 * 2.0 ** -9, 256.0, 240.0, -16.0, 2.0 ** -6, 2.0 ** -6 + 2 * 2.0 ** -9]
    assert list(q) == exp


def test_mx_block_scale_hand_vectors():
    # block of ones -> scale 2^-8 (1/2^-8 = 256 <= 448, 1/2^-9 = 512 > 448), exact
    a = np.ones((1, 32))
    assert O.mx_block_scale(np.array([1.0]))[0] == -8
    assert np.array_equal(O.mx_fake_quant(a, 1), a)
    # amax 1.9 -> scale 2^-7; 1.9 * 128 = 243.2 -> 240 -> 1.875
    b = np.full((1, 32), 0.1)
    b[0, 3] = 1.9
    qb = O.mx_fake_quant(b, 1)
    assert qb[0, 3] == 1.875
    # exactly 448 * 2^e sits on the boundary -> that e
    assert O.mx_block_scale(np.array([448.0]))[0] == 0
    assert O.mx_block_scale(np.array([448.0 * 2 ** -20]))[0] == -20
    assert O.mx_block_scale(np.array([np.nextafter(448.0, 1e9)]))[0] == 1
    assert O.mx_block_scale(np.array([0.0]))[0] == -127


def test_mx_fake_quant_properties():
    rng = np.random.default_rng(12)
    a = rng.standard_normal((7, 100)) * np.exp(rng.standard_normal((7, 1)) * 3)
    q = O.mx_fake_quant(a, 1)
    assert np.array_equal(O.mx_fake_quant(q, 1), q)          # idempotent
    # per-block scale is a power of two and no element overflows 448 * scale
    for r in range(7):
        for b0 in range(0, 100, 32):
            blk = a[r, b0:b0 + 32]
            e = O.mx_block_scale(np.array([np.abs(blk).max()]))[0]
            assert np.abs(blk).max() <= 448 * 2.0 ** e
            rel = np.abs(q[r, b0:b0 + 32] - blk) / np.abs(blk)
            normal = np.abs(blk) >= 2.0 ** (e - 6)
            assert np.all(rel[normal] <= 2.0 ** -4 + 1e-15)
    # blocks run along the requested axis
    qt = O.mx_fake_quant(a.T.copy(), 0)
    assert np.array_equal(qt, q.T)


# ------------------------------------------------------ printed parameter counts

def test_expert_shape_matches_printed_parameter_counts():
    """spark-gpt prints ~164M total / 50.7M active for its default 50M shape
    with 8 SwiGLU experts, top-2, width 768.  With the oracle's expert weights
    (packed gate/up [2I, d] plus down [d, I], i.e. 3 d I per expert) and the
    page's attention shape, the totals come out at those figures."""
    with open(os.path.join(GOLDEN, "spark_gpt_moe_param_counts.json")) as f:
        gold = json.load(f)
    s = gold["shape"]
    L = rand_layer(T=2, d=s["d_model"] // 64, E=s["experts"], k=s["top_k"], inter=s["expert_inter"] // 64)
    per_expert_small = L["w_gate_up"][0].size + L["w_down"][0].size
    d, inter = s["d_model"], s["expert_inter"]
    per_expert = per_expert_small * 64 * 64               # both dims scale by 64
    assert per_expert == 3 * d * inter
    hd = s["head_dim"]
    attn = d * s["q_heads"] * hd * 2 + d * s["kv_heads"] * hd * 2
    norms = 2 * d + 2 * hd
    router = s["experts"] * d
    emb = s["vocab"] * d * (2 if s["untied_embeddings"] else 1)
    nl = s["layers"]
    total = nl * (s["experts"] * per_expert + attn + norms + router) + d + emb
    active = nl * (s["top_k"] * per_expert + attn + norms + router) + d + emb
    assert round(total / 1e6) == gold["printed_total_params_millions"]
    assert abs(active / 1e6 - gold["printed_active_params_millions"]) < 0.05


# ------------------------------------------------------ storage-format rounding

@pytest.mark.parametrize("fmt,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_round_to_format_matches_library_conversion(fmt, tdt):
    """Every float32 value, across normal, subnormal and overflowing
    magnitudes, rounds as the library's float32 -> fmt conversion (nearest,
    ties to even)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-110, 25, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(tdt).to(torch.float64).numpy()
    got = O.round_to_format(x.astype(np.float64), fmt)
    assert np.array_equal(ref, got)


def test_round_to_format_hand_values():
    r = O.round_to_format
    # bf16 keeps 8 significant bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1)
    assert r(1.0 + 2.0 ** -8, "bf16") == 1.0
    assert r(1.0 + 3 * 2.0 ** -8, "bf16") == 1.0 + 2.0 ** -6       # tie -> even mantissa
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -20, "bf16") == 1.0 + 2.0 ** -7
    # f16: largest finite 65504; 65520 is the tie with 65536 -> overflows to inf
    assert r(65504.0, "f16") == 65504.0 and r(65519.0, "f16") == 65504.0
    assert np.isinf(r(65520.0, "f16"))
    # f16 subnormals are multiples of 2^-24
    assert r(3 * 2.0 ** -26, "f16") == 2.0 ** -24
    assert r(2.0 ** -25, "f16") == 0.0                               # tie -> even (0)
    assert r(0.0, "bf16") == 0.0 and r(-2.5, "f32") == -2.5


def test_storage_rounding_lands_on_the_stated_values_only():
    """With a bf16 store, the kept intermediates are bf16 numbers (Y_perm and
    dz f32 numbers); an identity store reproduces the exact layer bit for bit."""
    L = rand_layer(T=16, d=16, E=4, k=2, inter=8, n_shared=1)
    bf = lambda a, kind: O.round_to_format(a, "f32" if kind == "f32" else "bf16")
    rep = lambda a, fmt: np.array_equal(O.round_to_format(a, fmt), a)
    fwd = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=2, bias=None,
                          ws_gate_up=L["ws_gate_up"], ws_down=L["ws_down"], store=bf)
    bwd = O.layer_backward(fwd, L["dy"], aux_coef=0.01)
    for n in ["g", "u", "h"]:
        assert rep(fwd[n], "bf16"), n
    assert rep(fwd["y_perm"], "f32") and rep(fwd["y_shared"], "bf16")
    assert rep(bwd["dy_perm"], "bf16") and rep(bwd["dx_perm"], "bf16") and rep(bwd["dz"], "f32")
    assert not rep(fwd["y"], "bf16")                                  # outputs are not rounded
    ident = lambda a, kind: a
    f0 = fwd_of(L, 2)
    b0 = O.layer_backward(f0, L["dy"], aux_coef=0.01)
    f1 = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=2, bias=None,
                         ws_gate_up=L["ws_gate_up"], ws_down=L["ws_down"], store=ident)
    b1 = O.layer_backward(f1, L["dy"], aux_coef=0.01)
    assert np.array_equal(f0["y"], f1["y"])
    for n in ["dx", "dw_router", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"]:
        assert np.array_equal(b0[n], b1[n]), n


def test_expert_steps_match_torch_autograd():
    """The per-expert steps against torch autograd of the dense SwiGLU MLP
    y = (silu(x Wg^T) * x Wu^T) Wd^T in float64 (a textbook routine)."""
    rng = np.random.default_rng(11)
    n, d, inter = 7, 12, 5
    x = rng.standard_normal((n, d))
    w_gu = rng.standard_normal((2 * inter, d)) * 0.3
    w_d = rng.standard_normal((d, inter)) * 0.3
    dy = rng.standard_normal((n, d))
    G, U, H = O.expert_gate_up_step(x, w_gu)
    Y = O.expert_down_step(H, w_d)
    dgu, dw_d = O.expert_down_backward_step(dy, G, U, H, w_d)
    dx, dw_gu = O.expert_gate_up_backward_step(dgu, x, w_gu)

    tx = torch.tensor(x, requires_grad=True)
    tgu = torch.tensor(w_gu, requires_grad=True)
    td = torch.tensor(w_d, requires_grad=True)
    g = tx @ tgu[:inter].T
    u = tx @ tgu[inter:].T
    g.retain_grad(); u.retain_grad()
    y = (torch.nn.functional.silu(g) * u) @ td.T
    (torch.tensor(dy) * y).sum().backward()
    assert np.allclose(Y, y.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dgu[:, :inter], g.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dgu[:, inter:], u.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dw_d, td.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dw_gu, tgu.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("aux_coef", [0.0, 0.7])
def test_router_backward_matches_torch_autograd(renorm, aux_coef):
    """dz of router_backward against torch autograd of
    L = sum_tj w_tj(z) <dy_t, Y_perm[inv_tj]> + aux_coef * E * sum_e f_e P_e(z)
    with the selection and the counts held fixed (f carries no gradient)."""
    rng = np.random.default_rng(12)
    T, E, k, d = 9, 6, 2, 4
    z = rng.standard_normal((T, E))
    idx = O.topk_select(z, k)
    counts, _, _, inv = O.expert_permutation(idx, E)
    y_perm = rng.standard_normal((T * k, d))
    dy = rng.standard_normal((T, d))
    p = O.softmax_rows(z)
    w = O.gate_weights(p, idx, renorm)
    _, dz = O.router_backward(dy, y_perm, inv, p, idx, w, renorm, counts, aux_coef)

    tz = torch.tensor(z, requires_grad=True)
    tp = torch.softmax(tz, dim=1)
    sel = torch.gather(tp, 1, torch.tensor(idx))
    tw = sel / sel.sum(dim=1, keepdim=True) if renorm else sel
    gsc = np.einsum("td,tjd->tj", dy, y_perm[inv])
    f = torch.tensor(counts / (T * k))
    loss = (tw * torch.tensor(gsc)).sum() + aux_coef * E * (f * tp.mean(dim=0)).sum()
    loss.backward()
    assert np.allclose(dz, tz.grad.numpy(), rtol=1e-10, atol=1e-13)
