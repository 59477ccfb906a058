"""Pins of the oracle's router variants (KohakUwULLM README, "Key features":
Sinkhorn, expert-choice and ReLU routers registered beside the default; the
pages give no rules, so each follows its published method, as stated in the
oracle's docstrings).

Sinkhorn router: hand-computed scalings of a 2 x 2 matrix, a pure-Python loop
implementation, the marginals the iteration converges to, a matrix already
balanced (the scales are then constant and the choice is the plain top-k),
the balancing effect on a skewed router, and finite differences of the whole
layer with Sinkhorn routing (the selection is piecewise constant, so the
gradient is that of the default router's weights).
"""

import numpy as np
import pytest

import oracle as O
from tests.test_oracle_pins import rand_layer


# ----------------------------------------------------------------- Sinkhorn

def test_sinkhorn_two_by_two_by_hand():
    p = np.array([[0.9, 0.1], [0.6, 0.4]])
    # first Sinkhorn round, from b = 1: a = (1/2) / [1, 1]; column sums [0.75, 0.25]; b = (1/2) / them
    assert np.allclose(O.sinkhorn_column_scales(p, 1), [2.0 / 3.0, 2.0], rtol=0, atol=1e-15)
    # second Sinkhorn round: p b = [0.8, 1.2], a = [5/8, 5/12]; column sums [13/16, 11/48]
    assert np.allclose(O.sinkhorn_column_scales(p, 2), [8.0 / 13.0, 24.0 / 11.0], rtol=0, atol=1e-15)
    assert np.array_equal(O.sinkhorn_column_scales(p, 0), [1.0, 1.0])


def _loop_sinkhorn(p, n_iter):
    T, E = len(p), len(p[0])
    b = [1.0] * E
    for _ in range(n_iter):
        a = []
        for t in range(T):
            s = 0.0
            for e in range(E):
                s += p[t][e] * b[e]
            a.append((1.0 / T) / s)
        for e in range(E):
            s = 0.0
            for t in range(T):
                s += p[t][e] * a[t]
            b[e] = (1.0 / E) / s
    return b


def test_sinkhorn_matches_a_loop_implementation():
    rng = np.random.default_rng(3)
    p = O.softmax_rows(rng.standard_normal((7, 3)) * 2)
    for n in (1, 2, 5):
        assert np.allclose(O.sinkhorn_column_scales(p, n), _loop_sinkhorn(p.tolist(), n), rtol=1e-14, atol=0)


def test_sinkhorn_converges_to_uniform_marginals():
    rng = np.random.default_rng(4)
    T, E = 40, 6
    p = O.softmax_rows(rng.standard_normal((T, E)) * 1.5 + np.log(np.arange(1, E + 1.0))[None, :])
    b = O.sinkhorn_column_scales(p, 3000)
    a = (1.0 / T) / (p @ b)
    m = a[:, None] * p * b[None, :]
    assert np.max(np.abs(m.sum(axis=1) - 1.0 / T)) < 1e-12
    assert np.max(np.abs(m.sum(axis=0) - 1.0 / E)) < 1e-10


def test_sinkhorn_on_a_balanced_matrix_is_the_plain_top_k():
    # a circulant matrix: every column has the same sum, so the scales stay
    # equal and the ranking is that of p itself
    E = 5
    row = np.array([0.4, 0.25, 0.15, 0.12, 0.08])
    p = np.stack([np.roll(row, s) for s in range(E)] * 3)
    b = O.sinkhorn_column_scales(p, 7)
    assert np.allclose(b, b[0], rtol=1e-14, atol=0)
    s = O.sinkhorn_selection_scores(p, b)
    assert np.array_equal(O.topk_select(s, 2), O.topk_select(p, 2))


def test_sinkhorn_selection_balances_a_skewed_router():
    rng = np.random.default_rng(5)
    T, E, k = 2048, 16, 2
    zipf = np.log((np.arange(E) + 1.0) ** -1.2)
    p = O.softmax_rows(rng.standard_normal((T, E)) + 2.0 * zipf[None, :])
    plain = np.bincount(O.topk_select(p, k).ravel(), minlength=E)
    b = O.sinkhorn_column_scales(p, 20)
    sk = np.bincount(O.topk_select(O.sinkhorn_selection_scores(p, b), k).ravel(), minlength=E)
    cv = lambda c: c.std() / c.mean()
    assert cv(sk) < 0.25 * cv(plain), (cv(sk), cv(plain))
    assert sk.sum() == plain.sum() == T * k


def test_layer_with_sinkhorn_routing_chooses_and_weights_as_stated():
    L = rand_layer(T=24, d=16, E=6, k=2, inter=8, seed=7, bias=True)
    fwd = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=2, bias=L["bias"],
                          sinkhorn_iters=4)
    b = O.sinkhorn_column_scales(fwd["p"], 4)
    assert np.array_equal(fwd["sinkhorn_b"], b)
    assert np.array_equal(fwd["idx"], O.topk_select(fwd["p"] * b[None, :], 2))
    assert np.array_equal(fwd["w"], O.gate_weights(fwd["p"], fwd["idx"], True))


def _sk_fwd(L, k, renorm, n_iter):
    return O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=k, renorm=renorm,
                           bias=L["bias"], sinkhorn_iters=n_iter)


def _sk_gap(L, k, n_iter):
    fwd = _sk_fwd(L, k, True, n_iter)
    s = -np.sort(-np.log(O.sinkhorn_selection_scores(fwd["p"], fwd["sinkhorn_b"])), axis=1)
    return np.min(s[:, k - 1] - s[:, k])


@pytest.mark.parametrize("renorm", [True, False])
def test_sinkhorn_layer_gradient_matches_central_differences(renorm):
    k, n_iter, aux_coef = 2, 6, 0.3
    for sd in range(50, 250):
        L = rand_layer(T=10, d=12, E=5, k=k, inter=8, seed=sd, wscale=0.3)
        if _sk_gap(L, k, n_iter) >= 1e-3:
            break
    fwd = _sk_fwd(L, k, renorm, n_iter)
    g = O.layer_backward(fwd, L["dy"], aux_coef=aux_coef)
    rng = np.random.default_rng(2)
    h = 1e-6
    for pname, gname in {"x": "dx", "w_router": "dw_router", "w_down": "dw_down"}.items():
        arr = L[pname]
        for fi in rng.choice(arr.size, size=min(arr.size, 30), replace=False):
            pos = np.unravel_index(fi, arr.shape)
            orig = arr[pos]
            arr[pos] = orig + h
            lp = O.layer_loss(_sk_fwd(L, k, renorm, n_iter), L["dy"], aux_coef)
            arr[pos] = orig - h
            lm = O.layer_loss(_sk_fwd(L, k, renorm, n_iter), L["dy"], aux_coef)
            arr[pos] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[gname][pos]) <= 1e-6 * max(1.0, abs(g[gname][pos])), (pname, pos)


# --------------------------------------------------------------------- ReLU

def _brute_relu_select(z, k):
    out = []
    for row in z.tolist():
        pos = [(v, e) for e, v in enumerate(row) if v > 0]
        pos.sort(key=lambda ve: (-ve[0], ve[1]))        # value descending, lower index on ties
        sel = [e for _, e in pos[:k]]
        out.append(sel + [-1] * (k - len(sel)))
    return np.array(out)


def test_relu_select_by_brute_force():
    rng = np.random.default_rng(8)
    z = np.round(rng.standard_normal((60, 7)), 1)         # ties and zeros on purpose
    z[3] = -1.0                                           # a token with no positive logit
    z[4] = 0.0                                            # zero is not positive
    for k in (1, 3, 7):
        assert np.array_equal(O.relu_select(z, k), _brute_relu_select(z, k))
    idx = O.relu_select(z, 3)
    w = O.relu_gate_weights(O.relu_gates(z), idx)
    for t in range(60):
        for j in range(3):
            assert w[t, j] == (z[t, idx[t, j]] if idx[t, j] >= 0 else 0.0)
    assert np.all(idx[3] == -1) and np.all(idx[4] == -1)


def test_permutation_with_empty_slots_by_brute_force():
    idx = np.array([[2, -1], [0, 2], [-1, -1], [2, 1], [1, -1]])
    counts, offsets, perm, inv = O.expert_permutation(idx, 3)
    assert counts.tolist() == [1, 2, 3] and offsets.tolist() == [0, 1, 3, 6]
    assert perm.tolist() == [1, 3, 4, 0, 1, 3]            # expert ascending, then token ascending
    assert inv.tolist() == [[3, -1], [0, 4], [-1, -1], [5, 1], [2, -1]]


def test_relu_layer_with_every_expert_active_is_the_gate_weighted_sum():
    # all logits positive and k = E: y_t = sum_e relu(z_te) SwiGLU_e(x_t)
    L = rand_layer(T=9, d=12, E=4, k=4, inter=8, seed=11)
    bias = np.full(4, 5.0)
    fwd = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=4, renorm=False, bias=bias,
                          router="relu")
    z = O.router_logits(L["x"], L["w_router"], bias)
    assert np.all(z > 0)
    y = np.zeros_like(L["x"])
    for e in range(4):
        y += z[:, e:e + 1] * O.swiglu_rows(L["x"], L["w_gate_up"][e], L["w_down"][e])[3]
    assert np.allclose(fwd["y"], y, rtol=1e-13, atol=1e-13)


def _relu_fwd(L, k, bias):
    return O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=k, renorm=False, bias=bias,
                           ws_gate_up=L["ws_gate_up"], ws_down=L["ws_down"], router="relu")


@pytest.mark.parametrize("n_shared", [0, 1])
def test_relu_layer_gradient_matches_central_differences(n_shared):
    k, aux_coef = 2, 0.4
    bias = np.array([0.2, -0.1, 0.0, 0.1, -0.2])
    for sd in range(300, 600):
        L = rand_layer(T=10, d=12, E=5, k=k, inter=8, n_shared=n_shared, inter_s=8, seed=sd, wscale=0.3)
        z = O.router_logits(L["x"], L["w_router"], bias)
        srt = -np.sort(-z, axis=1)
        # away from every kink: no logit near 0, the k-th and (k+1)-th apart,
        # and some tokens with fewer than k positive logits
        if np.min(np.abs(z)) > 1e-3 and np.min(srt[:, k - 1] - srt[:, k]) > 1e-3 and (srt[:, k - 1] < 0).any():
            break
    fwd = _relu_fwd(L, k, bias)
    assert (fwd["idx"] == -1).any()
    g = O.layer_backward(fwd, L["dy"], aux_coef=aux_coef)
    names = {"x": "dx", "w_router": "dw_router", "w_gate_up": "dw_gate_up", "w_down": "dw_down"}
    if n_shared:
        names.update({"ws_gate_up": "dws_gate_up"})
    rng = np.random.default_rng(3)
    h = 1e-6
    for pname, gname in names.items():
        arr = L[pname]
        for fi in rng.choice(arr.size, size=min(arr.size, 30), replace=False):
            pos = np.unravel_index(fi, arr.shape)
            orig = arr[pos]
            arr[pos] = orig + h
            lp = O.layer_loss(_relu_fwd(L, k, bias), L["dy"], aux_coef)
            arr[pos] = orig - h
            lm = O.layer_loss(_relu_fwd(L, k, bias), L["dy"], aux_coef)
            arr[pos] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[gname][pos]) <= 1e-6 * max(1.0, abs(g[gname][pos])), (pname, pos)


# ------------------------------------------------------------ expert choice

def _brute_expert_choice(p, C):
    T, E = len(p), len(p[0])
    idx = [[-1] * E for _ in range(T)]
    for e in range(E):
        col = sorted(range(T), key=lambda t: (-p[t][e], t))   # probability descending, lower token on ties
        for t in col[:C]:
            idx[t][e] = e
    return np.array(idx)


def test_expert_choice_by_brute_force():
    rng = np.random.default_rng(12)
    p = O.softmax_rows(np.round(rng.standard_normal((37, 5)), 1))   # ties on purpose
    for C in (0, 1, 7, 37):
        got = O.expert_choice_select(p, C)
        assert np.array_equal(got, _brute_expert_choice(p.tolist(), C))
        assert np.all((got >= 0).sum(axis=0) == C)                  # every expert takes exactly C tokens
        assert np.all((got == np.arange(5)[None, :]) | (got == -1))  # slot e is expert e's


def test_expert_choice_at_full_capacity_is_the_soft_mixture():
    # k = E: C = T, every expert takes every token: y_t = sum_e p_te SwiGLU_e(x_t)
    L = rand_layer(T=9, d=12, E=4, k=4, inter=8, seed=13)
    fwd = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=4, renorm=False,
                          router="expert_choice")
    p = O.softmax_rows(O.router_logits(L["x"], L["w_router"]))
    assert np.all(fwd["idx"] == np.arange(4)[None, :]) and np.array_equal(fwd["counts"], [9] * 4)
    y = np.zeros_like(L["x"])
    for e in range(4):
        y += p[:, e:e + 1] * O.swiglu_rows(L["x"], L["w_gate_up"][e], L["w_down"][e])[3]
    assert np.allclose(fwd["y"], y, rtol=1e-13, atol=1e-13)


def _ec_fwd(L, k):
    return O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=k, renorm=False,
                           ws_gate_up=L["ws_gate_up"], ws_down=L["ws_down"], router="expert_choice")


@pytest.mark.parametrize("n_shared", [0, 1])
def test_expert_choice_layer_gradient_matches_central_differences(n_shared):
    k, aux_coef = 2, 0.4
    for sd in range(600, 900):
        L = rand_layer(T=10, d=12, E=5, k=k, inter=8, n_shared=n_shared, inter_s=8, seed=sd, wscale=0.3)
        p = O.softmax_rows(O.router_logits(L["x"], L["w_router"]))
        C = (10 * k) // 5
        srt = -np.sort(-p, axis=0)
        if np.min(srt[C - 1] - srt[C]) > 1e-4:                      # each expert's C-th and (C+1)-th apart
            break
    fwd = _ec_fwd(L, k)
    assert (fwd["idx"] < 0).any() and ((fwd["idx"] >= 0).sum(axis=1) != k).any()   # uneven tokens
    g = O.layer_backward(fwd, L["dy"], aux_coef=aux_coef)
    names = {"x": "dx", "w_router": "dw_router", "w_gate_up": "dw_gate_up", "w_down": "dw_down"}
    if n_shared:
        names.update({"ws_down": "dws_down"})
    rng = np.random.default_rng(4)
    h = 1e-6
    for pname, gname in names.items():
        arr = L[pname]
        for fi in rng.choice(arr.size, size=min(arr.size, 30), replace=False):
            pos = np.unravel_index(fi, arr.shape)
            orig = arr[pos]
            arr[pos] = orig + h
            lp = O.layer_loss(_ec_fwd(L, k), L["dy"], aux_coef)
            arr[pos] = orig - h
            lm = O.layer_loss(_ec_fwd(L, k), L["dy"], aux_coef)
            arr[pos] = orig
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[gname][pos]) <= 1e-6 * max(1.0, abs(g[gname][pos])), (pname, pos)
