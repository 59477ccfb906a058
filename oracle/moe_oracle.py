"""Plain float64 definition of the routed MoE SwiGLU FFN layer, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What the layer computes is taken from three descriptions of it:
  * KochiLLM v1.0 model card, "Architecture": each token goes through one
    always-on expert and through 2 of 4 routed experts whose two weights are
    rescaled to sum to one; the loss gains 0.01 times the layer mean of the
    balancing term 4 * sum_i f_i * p_i (a single layer here).
  * KochiLLM v1.0 model card, "Configuration": experts are SwiGLU blocks.
  * spark-gpt README, feature list (optional Qwen3-MoE layers): a router
    without bias, a softmax taken in fp32, top-k choice, SwiGLU experts whose
    gate and up weights live in one tensor, and rescaling of the chosen
    probabilities; and its MoE paragraph: the rescaling can be turned off, the
    balancing statistic combines integer counts (no gradient) with a
    differentiable mean of probabilities, and the logged router metrics are
    the smallest and largest per-expert count, their coefficient of variation,
    the mean routing entropy and the number of experts that got no token.

Readings where the pages are silent (each is also listed in the design notes):
  * top-k is taken on the logits (after any constant router bias), ordered by
    logit descending and, on equal logits, by lower expert index;
  * aux-loss-free balancing (KohakUwULLM README, "Key features": DeepSeekMoE
    with aux-loss-free load balancing, no rule given) follows the published
    method: top-k on probability + per-expert selection bias, weights from the
    unbiased probabilities, bias += gamma * sign(mean load - load) per step;
  * the Sinkhorn router (KohakUwULLM README, "Key features": named, no rule)
    follows the published Sinkhorn-Knopp balancing: a fixed number of
    alternating row / column scalings of the batch's probability matrix,
    top-k on the column-scaled probabilities, weights from the unscaled ones;
  * f_e = count_e / (T * k), P_e = mean over all T tokens of the full softmax,
    aux = E * sum_e f_e * P_e (equals 1 at perfect balance; E = 4 gives the
    model card's "4 * sum");
  * f_e is a hard count and carries no gradient; P_e does;
  * shared experts have weight 1 and no gate;
  * packed gate/up layout: W_gu[e] rows 0..I-1 are the gate rows, rows
    I..2I-1 the up rows, each row of length d; W_d[e] is [d, I].

All arrays are numpy float64 (int64 for indices).  Loops over experts are plain
Python; every contraction is a numpy matmul (a library primitive).
"""

import numpy as np


# ---------------------------------------------------------------- routing ---

def router_logits(x, w_router, bias=None):
    """z = x W_r^T (+ b).  spark-gpt README, Qwen3-MoE feature: the router is a
    bias-free linear map; ``bias`` is the constant per-expert offset used only
    to skew expert popularity in a stress workload, never trained."""
    z = x @ w_router.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    return z


def softmax_rows(z):
    """Row softmax, max-subtracted.  spark-gpt README: fp32-softmax routing
    (computed here in float64)."""
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=1, keepdims=True)


def topk_select(z, k):
    """Indices [T, k] of the k largest logits per row, in slot order: logit
    descending, lower expert index first on equal logits (a stable sort of -z).
    KochiLLM "Architecture" (top-2 of 4) and spark-gpt Qwen3-MoE feature (top-k)."""
    order = np.argsort(-z, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def gate_weights(p, idx, renorm):
    """Weights of the selected experts.  With ``renorm`` the selected
    probabilities are divided by their sum (KochiLLM "Architecture": the two
    chosen weights are rescaled; spark-gpt MoE paragraph: the default, with a
    flag that disables it)."""
    sel = np.take_along_axis(p, idx, axis=1)
    if renorm:
        return sel / sel.sum(axis=1, keepdims=True)
    return sel


def balanced_selection_scores(p, sel_bias):
    """Scores the aux-loss-free balancing router ranks for top-k: the routing
    probabilities plus a per-expert selection bias.  KohakUwULLM README, "Key
    features", names DeepSeekMoE with aux-loss-free load balancing and gives
    no rule; the reading taken is the published method (a bias added to each
    expert's routing score for the choice of experts only, the gate weights
    still taken from the unbiased probabilities).  Rank with topk_select;
    weights with gate_weights on the unbiased ``p``."""
    return p + np.asarray(sel_bias, dtype=np.float64)[None, :]


def sinkhorn_column_scales(p, n_iter):
    """Column scales b [E] of the Sinkhorn router.  KohakUwULLM README, "Key
    features", names Sinkhorn routers beside the default one and gives no
    rule; the reading taken is the published Sinkhorn-Knopp balancing of the
    batch's [T, E] routing-probability matrix toward equal row sums (1/T,
    every token routed) and equal column sums (1/E, every expert equally
    loaded): starting from b = 1, ``n_iter`` times
        a_t = (1/T) / sum_e p_te b_e,   then   b_e = (1/E) / sum_t p_te a_t.
    A fixed number of rounds (no convergence test) keeps the layer free of
    host synchronisation."""
    p = np.asarray(p, dtype=np.float64)
    T, E = p.shape
    b = np.ones(E)
    for _ in range(int(n_iter)):
        a = (1.0 / T) / (p @ b)
        b = (1.0 / E) / (p.T @ a)
    return b


def sinkhorn_selection_scores(p, b):
    """Scores the Sinkhorn router ranks for top-k: the balanced matrix
    a_t p_te b_e of one token, without its row scale a_t (common to the
    token's experts, so it does not change the ranking).  Rank with
    topk_select; the gate weights stay the unscaled probabilities of the
    chosen experts (gate_weights on ``p``), so the selection carries no
    gradient."""
    return np.asarray(p, dtype=np.float64) * np.asarray(b, dtype=np.float64)[None, :]


def relu_gates(z):
    """Gates of the ReLU router: g_te = max(z_te, 0), no softmax.  KohakUwULLM
    README, "Key features", names ReLU routers and gives no rule; the reading
    taken is the published ReLU routing (ReMoE): a token uses every expert
    whose gate is positive, weighted by the gate itself, and the gates take
    the place of the probabilities everywhere else, so the layer's balancing
    statistic E sum_e f_e mean_t g_te is the published load-balanced L1 term
    on the gates.  Here at most ``top_k`` experts per token (relu_select)."""
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


def relu_select(z, k):
    """The ReLU router's choice: the token's k largest logits that are
    positive (descending, lower index first on equal logits); slots past the
    token's positive logits hold -1 (no expert)."""
    idx = topk_select(z, k)
    zs = np.take_along_axis(z, idx, axis=1)
    return np.where(zs > 0, idx, -1)


def relu_gate_weights(g, idx):
    """Weights of the slots of the ReLU and expert-choice routers: the gate
    (or probability) of the slot's expert, 0 for an empty slot (no
    renormalisation)."""
    sel = np.take_along_axis(g, np.maximum(idx, 0), axis=1)
    return np.where(idx >= 0, sel, 0.0)


def expert_choice_select(p, capacity):
    """Expert-choice routing.  KohakUwULLM README, "Key features", names
    expert-choice routers and gives no rule; the reading taken is the
    published method: every expert takes the ``capacity`` tokens with the
    largest routing probability p_te (lower token index first on equal
    probabilities), C = T k / E rounded down with k the average number of
    experts per token, so a token is taken by any number of experts (0 to E)
    and every expert by exactly C tokens.  Returns idx [T, E]: idx[t, e] = e
    when expert e took token t, else -1 (slot e belongs to expert e)."""
    p = np.asarray(p, dtype=np.float64)
    T, E = p.shape
    idx = np.full((T, E), -1, dtype=np.int64)
    for e in range(E):
        taken = np.argsort(-p[:, e], kind="stable")[:capacity]
        idx[taken, e] = e
    return idx


def balance_bias_update(sel_bias, counts, T, top_k, gamma):
    """One update of the selection bias after a step: b_e += gamma * sign(mean
    load - count_e), mean load = T k / E, so overloaded experts lose and
    underloaded ones gain a fixed step (the published aux-loss-free rule; see
    balanced_selection_scores).  The bias is an f32 vector, so the addition
    is rounded to f32 once; the sign is decided exactly in integers
    (T k - E count_e)."""
    b = np.asarray(sel_bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    E = b.shape[0]
    sgn = np.sign(int(T) * int(top_k) - E * c).astype(np.float32)
    return (b + np.float32(gamma) * sgn).astype(np.float32)


def near_tie_tokens(z, k, eps=1e-5):
    """Tokens whose routing is decided by a near-tie of the logits.

    Returns (set_tie, order_tie), boolean [T] masks:
      set_tie   -- the k-th and (k+1)-th largest logits differ by less than eps
                   (the selected *set* is ambiguous at that precision);
      order_tie -- two adjacent selected logits differ by less than eps (the
                   *slot order* inside the set is ambiguous).
    """
    srt = -np.sort(-z, axis=1)
    E = z.shape[1]
    if k < E:
        set_tie = (srt[:, k - 1] - srt[:, k]) < eps
    else:
        set_tie = np.zeros(z.shape[0], dtype=bool)
    if k > 1:
        order_tie = ((srt[:, : k - 1] - srt[:, 1:k]) < eps).any(axis=1)
    else:
        order_tie = np.zeros(z.shape[0], dtype=bool)
    return set_tie, order_tie


# ------------------------------------------------------------ permutation ---

def expert_permutation(idx, n_experts):
    """Group the T*k assignments by expert.

    counts[e]      number of assignments (t, j) with idx[t, j] == e
    offsets        exclusive prefix sum of counts, length E+1
    perm_token[r]  token of the r-th row of the expert-sorted order, the order
                   being (expert ascending, token ascending)
    inv[t, j]      row r at which assignment (t, j) sits in that order
    A slot holding -1 (no expert: the ReLU router) is no assignment: it gets
    no row and inv -1, and perm_token covers the offsets[E] real rows.
    """
    T, k = idx.shape
    flat = idx.reshape(-1)
    real = flat >= 0
    counts = np.bincount(flat[real], minlength=n_experts).astype(np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    pos = np.nonzero(real)[0]                        # flat positions f = t*k + j of real slots
    order = pos[np.argsort(flat[real], kind="stable")]
    perm_token = (order // k).astype(np.int64)
    inv = np.full(T * k, -1, dtype=np.int64)
    inv[order] = np.arange(order.size, dtype=np.int64)
    return counts, offsets, perm_token, inv.reshape(T, k)


# ----------------------------------------------------------------- experts ---

def silu(a):
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a))."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def _sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def swiglu_rows(rows, w_gate_up_e, w_down_e):
    """One SwiGLU expert on a block of rows: G = X Wg^T, U = X Wu^T,
    H = silu(G) * U, Y = H Wd^T (no biases).  KochiLLM "Configuration"
    (SwiGLU experts) and spark-gpt (packed SwiGLU experts: gate and up stacked
    in one [2I, d] weight)."""
    inter = w_down_e.shape[1]
    g = rows @ w_gate_up_e[:inter].T
    u = rows @ w_gate_up_e[inter:].T
    h = silu(g) * u
    return g, u, h, h @ w_down_e.T


def shared_experts_forward(x, ws_gate_up, ws_down):
    """Sum of the always-on shared experts, each applied to every token with
    weight 1 and no gate (KochiLLM "Architecture")."""
    y = np.zeros((x.shape[0], ws_down.shape[1]))
    parts = []
    for s in range(ws_gate_up.shape[0]):
        g, u, h, ys = swiglu_rows(x, ws_gate_up[s], ws_down[s])
        parts.append((g, u, h))
        y += ys
    return y, parts


def combine(y_perm, inv, w, y_shared=None):
    """y_t = sum_j w_tj * Y_perm[inv[t, j]] (+ shared output); slots with
    inv -1 (no expert) add nothing."""
    rows = np.where((inv >= 0)[:, :, None], y_perm[np.maximum(inv, 0)], 0.0)
    y = np.einsum("tj,tjd->td", w, rows)
    if y_shared is not None:
        y = y + y_shared
    return y


# ---------------------------------------------------------- aux statistics ---

def real_token_counts(idx, mask, n_experts):
    """Assignments per expert among the real tokens (mask 1) only, and the
    number of real tokens."""
    m = np.asarray(mask, dtype=np.int64)
    sel = idx[m != 0].ravel()
    return np.bincount(sel[sel >= 0], minlength=n_experts).astype(np.int64), int(m.sum())


def aux_statistics(p, counts, top_k, mask=None):
    """Load-balancing statistic and router metrics.

    KochiLLM "Architecture": the term 4 * sum_i f_i * p_i for its 4 experts;
    spark-gpt MoE paragraph: the raw balancing value plus count extremes,
    count spread (coefficient of variation), mean routing entropy and the
    number of idle experts.  f_e = count_e / (T k), P_e = mean_t p_te,
    aux_raw = sum_e f_e P_e, aux = E * aux_raw.

    ``mask`` ([T], 1 = real token, 0 = filler): the spark-gpt MoE paragraph
    computes the statistic over real (non-filler) tokens only; then T is the
    number of real tokens, ``counts`` must be their assignments
    (real_token_counts), P_e averages p over the real tokens and every
    metric is taken over them.  No real token: every value is 0.
    """
    T, E = p.shape
    if mask is not None:
        m = np.asarray(mask, dtype=np.float64)
        p = p[m != 0]
        T = p.shape[0]
    counts = np.asarray(counts, dtype=np.float64)
    f = counts / (T * top_k) if T > 0 else np.zeros(E)
    p_mean = p.mean(axis=0) if T > 0 else np.zeros(E)
    aux_raw = float((f * p_mean).sum())
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    entropy = float((-plogp.sum(axis=1)).mean()) if T > 0 else 0.0
    mean_c = counts.mean()
    cv = float(counts.std() / mean_c) if mean_c > 0 else 0.0
    return {
        "f": f,
        "p_mean": p_mean,
        "aux_raw": aux_raw,
        "aux": E * aux_raw,
        "entropy_mean": entropy,
        "count_min": int(counts.min()),
        "count_max": int(counts.max()),
        "count_cv": cv,
        "n_unused": int((counts == 0).sum()),
    }


# ------------------------------------------------------------ layer passes ---

def _no_store(a, kind):
    return a


def _ident_quant(a, axis):
    return a


def expert_gate_up_step(rows, w_gate_up_e, quant=None, store=None):
    """G, U and H = silu(G) * U of one expert on a block of rows, each as
    stored (``store`` kind "act"); H is formed from the unrounded G and U.
    ``quant`` is applied to both GEMM operands along the contraction (d)."""
    q = quant or _ident_quant
    st = store or _no_store
    inter = w_gate_up_e.shape[0] // 2
    xr = q(rows, 1)
    wgu = q(w_gate_up_e, 1)
    g = xr @ wgu[:inter].T
    u = xr @ wgu[inter:].T
    return st(g, "act"), st(u, "act"), st(silu(g) * u, "act")


def expert_down_step(h, w_down_e, quant=None):
    """H W_d^T of one expert (unrounded), both operands quantised along I."""
    q = quant or _ident_quant
    return q(h, 1) @ q(w_down_e, 1).T


def layer_forward(x, w_router, w_gate_up, w_down, *, top_k, renorm=True, bias=None,
                  ws_gate_up=None, ws_down=None, quant=None, store=None, sel_bias=None,
                  sinkhorn_iters=None, router="softmax"):
    """Full forward pass.  Returns a dict of every intermediate.

    ``sel_bias`` (aux-loss-free balancing) moves the choice of experts to
    balanced_selection_scores(p, sel_bias); the weights stay the unbiased
    probabilities of the chosen experts.  ``sinkhorn_iters`` (the Sinkhorn
    router) moves it to sinkhorn_selection_scores(p, b) with b =
    sinkhorn_column_scales(p, sinkhorn_iters), returned as "sinkhorn_b".
    ``router="expert_choice"``: idx = expert_choice_select(p, T top_k // E)
    ([T, E] slots, -1 where the expert did not take the token), weights the
    probabilities of the taken slots (no renormalisation: renorm must be
    False).
    ``router="relu"`` (the ReLU router) replaces the probabilities by the
    gates relu_gates(z) (returned as "p"), the choice by relu_select and the
    weights by relu_gate_weights (no renormalisation: renorm must be False).

    ``quant``, if given, is applied to each operand of each expert GEMM as
    quant(array, axis) with ``axis`` the contraction axis of that GEMM (the MX
    fake-quant mode); the router, softmax and combine are never quantised.

    ``store``, if given, is store(array, kind) and rounds the values the layer
    keeps between its steps to their storage format: kind "act" for the gate
    and up pre-activations G, U, the activation H and the shared experts'
    output (the activation dtype), kind "f32" for the routed experts' output
    rows Y_perm.  The layer is trained in that dtype (spark-gpt README:
    BF16 grouped GEMM; KochiLLM model card: fp16 training), so this is the
    layer those pages run; with store=None the exact layer is computed.
    Products and sums are exact either way.
    """
    st = store if store is not None else _no_store
    T, d = x.shape
    E = w_router.shape[0]
    z = router_logits(x, w_router, bias)
    relu = router == "relu"
    ec = router == "expert_choice"
    if relu or ec:
        assert not renorm and sel_bias is None and sinkhorn_iters is None, "no renormalisation for this router"
    p = relu_gates(z) if relu else softmax_rows(z)
    sk_b = None
    if relu:
        idx = relu_select(z, top_k)
    elif ec:
        idx = expert_choice_select(p, (T * top_k) // E)
    elif sinkhorn_iters is not None:
        sk_b = sinkhorn_column_scales(p, sinkhorn_iters) if T > 0 else np.ones(E)
        idx = topk_select(sinkhorn_selection_scores(p, sk_b), top_k)
    else:
        idx = topk_select(z if sel_bias is None else balanced_selection_scores(p, sel_bias), top_k)
    w = relu_gate_weights(p, idx) if (relu or ec) else gate_weights(p, idx, renorm)
    counts, offsets, perm_token, inv = expert_permutation(idx, E)
    x_perm = x[perm_token]
    inter = w_down.shape[2]
    A = int(offsets[-1])                            # real rows (T k unless slots are empty)
    g = np.zeros((A, inter)); u = np.zeros((A, inter)); h = np.zeros((A, inter))
    y_perm = np.zeros((A, d))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        g[r0:r1], u[r0:r1], h[r0:r1] = expert_gate_up_step(x_perm[r0:r1], w_gate_up[e], quant, store)
        y_perm[r0:r1] = st(expert_down_step(h[r0:r1], w_down[e], quant), "f32")
    y_shared = None
    shared = []
    if ws_gate_up is not None and ws_gate_up.shape[0] > 0:
        y_shared = np.zeros((T, d))
        for s in range(ws_gate_up.shape[0]):
            gs, us, hs = expert_gate_up_step(x, ws_gate_up[s], quant, store)
            y_shared += expert_down_step(hs, ws_down[s], quant)
            shared.append((gs, us, hs))
        y_shared = st(y_shared, "act")
    y = combine(y_perm, inv, w, y_shared)
    return dict(z=z, p=p, idx=idx, w=w, counts=counts, offsets=offsets,
                perm_token=perm_token, inv=inv, x_perm=x_perm, g=g, u=u, h=h,
                y_perm=y_perm, y_shared=y_shared, shared=shared, y=y,
                x=x, w_router=w_router, w_gate_up=w_gate_up, w_down=w_down,
                ws_gate_up=ws_gate_up, ws_down=ws_down, top_k=top_k,
                renorm=renorm, bias=bias, store=store, sel_bias=sel_bias, sinkhorn_b=sk_b, router=router)


def expert_down_backward_step(dy_rows, g, u, h, w_down_e, quant=None, store=None):
    """Backward of one expert's down projection and SwiGLU on a block of rows.
    dH = dY W_d (operands quantised along d), dW_d = dY^T H (along the rows),
    then dG = dH * U * s * (1 + G (1 - s)) with s = sigmoid(G), dU = dH *
    silu(G).  Returns ([dG | dU] as stored, kind "act"; dW_d unrounded)."""
    q = quant or _ident_quant
    st = store or _no_store
    dh = q(dy_rows, 1) @ q(w_down_e, 0)
    dw_down = q(dy_rows, 0).T @ q(h, 0)
    sg = _sigmoid(g)
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))
    du = dh * silu(g)
    return st(np.concatenate([dg, du], axis=1), "act"), dw_down


def expert_gate_up_backward_step(dgu, rows, w_gate_up_e, quant=None):
    """Backward of one expert's packed gate/up projection: dX = [dG | dU] W_gu
    (operands quantised along 2I) and dW_gu = [dG | dU]^T X (along the rows),
    both unrounded."""
    q = quant or _ident_quant
    return q(dgu, 1) @ q(w_gate_up_e, 0), q(dgu, 0).T @ q(rows, 0)


def router_backward(dy, y_perm, inv, p, idx, w, renorm, counts, aux_coef=0.0, store=None, mask=None,
                    router="softmax"):
    """Gradient of L = <dy, y> + aux_coef * aux with respect to the router
    logits, given the expert output rows Y_perm the combine weighted.

    g_tj = <dy_t, Y_perm[inv_tj]> reaches the routing weight of slot j; with
    renormalisation w = p_sel / S, so dL/dp_sel = (g - <w, g>) / S; the
    balancing term adds aux_coef * E * f_e / T to every p_te (f_e is a count,
    no gradient); the softmax Jacobian then gives dz = p * (dp - <p, dp>).
    With ``mask`` the statistic covers the real tokens only (aux_statistics):
    ``counts`` are theirs, T is their number, and only real tokens' p_te get
    the balancing term.
    ``router="relu"``: ``p`` holds the gates max(z, 0), which are the weights
    themselves, so dL/dg of a slot is g_tj, the balancing term is added the
    same way, and dz = dp where z > 0 (g > 0), 0 elsewhere; slots with idx -1
    carry nothing.
    Returns (g [T, k], dz [T, E] as stored, kind "f32")."""
    st = store or _no_store
    T, E = p.shape
    k = idx.shape[1]
    real = inv >= 0
    gsc = np.where(real, np.einsum("td,tjd->tj", dy, y_perm[np.maximum(inv, 0)]), 0.0)
    if router == "relu":
        dp = np.zeros_like(p)
        for j in range(k):
            t = np.nonzero(idx[:, j] >= 0)[0]
            dp[t, idx[t, j]] += gsc[t, j]
        if aux_coef != 0.0:
            if mask is None:
                dp = dp + aux_coef * E * (np.asarray(counts, dtype=np.float64) / (T * k))[None, :] / T
            else:
                m = np.asarray(mask, dtype=np.float64)
                Tr = float(m.sum())
                if Tr > 0:
                    f = np.asarray(counts, dtype=np.float64) / (Tr * k)
                    dp = dp + m[:, None] * (aux_coef * E * f[None, :] / Tr)
        return gsc, st(np.where(p > 0, dp, 0.0), "f32")
    p_sel = np.take_along_axis(p, idx, axis=1)
    if renorm:
        S = p_sel.sum(axis=1, keepdims=True)
        dp_sel = (gsc - (w * gsc).sum(axis=1, keepdims=True)) / S
    else:
        dp_sel = gsc
    dp = np.zeros_like(p)
    np.put_along_axis(dp, idx, dp_sel, axis=1)
    if aux_coef != 0.0:
        if mask is None:
            f = np.asarray(counts, dtype=np.float64) / (T * k)
            dp = dp + aux_coef * E * f[None, :] / T
        else:
            m = np.asarray(mask, dtype=np.float64)
            Tr = float(m.sum())
            if Tr > 0:
                f = np.asarray(counts, dtype=np.float64) / (Tr * k)
                dp = dp + m[:, None] * (aux_coef * E * f[None, :] / Tr)
    return gsc, st(p * (dp - (p * dp).sum(axis=1, keepdims=True)), "f32")


def layer_backward(fwd, dy, *, aux_coef=0.0, quant=None, mask=None):
    """Gradients of L = <dy, y> + aux_coef * aux with respect to x and every
    weight, by the chain rule through the forward of ``layer_forward``.

    f_e is an integer count and carries no gradient; P_e does (spark-gpt MoE
    paragraph: counts without gradient, a differentiable stand-in).

    With the forward's ``store`` rounding, the gradients the layer keeps
    between its steps are rounded too: dY_perm, [dG | dU] and dX_perm of the
    routed experts and the shared experts' [dG | dU] and input gradient (kind
    "act"); the router's logit gradient dz (kind "f32").  Final outputs are
    not rounded.
    """
    st = fwd.get("store") or _no_store
    x, w_r = fwd["x"], fwd["w_router"]
    w_gate_up, w_down = fwd["w_gate_up"], fwd["w_down"]
    p, idx, w, inv = fwd["p"], fwd["idx"], fwd["w"], fwd["inv"]
    offsets, counts = fwd["offsets"], fwd["counts"]
    T, d = x.shape
    E = w_r.shape[0]
    k = fwd["top_k"]

    # combine: y_t = sum_j w_tj Y_perm[inv_tj]  ->  dY_perm rows w_tj dy_t
    dy_perm = np.zeros_like(fwd["y_perm"])
    realf = inv.reshape(-1) >= 0
    dy_perm[inv.reshape(-1)[realf]] = st((w[:, :, None] * dy[:, None, :]).reshape(-1, d)[realf], "act")

    dw_gate_up = np.zeros_like(w_gate_up)
    dw_down = np.zeros_like(w_down)
    dx_perm = np.zeros((int(offsets[-1]), d))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        dgu, dw_down[e] = expert_down_backward_step(dy_perm[r0:r1], fwd["g"][r0:r1], fwd["u"][r0:r1],
                                                    fwd["h"][r0:r1], w_down[e], quant, st)
        dxe, dw_gate_up[e] = expert_gate_up_backward_step(dgu, fwd["x_perm"][r0:r1], w_gate_up[e], quant)
        dx_perm[r0:r1] = st(dxe, "act")

    dx = np.zeros((T, d))
    for j in range(inv.shape[1]):                   # slots (E of them for expert choice)
        t = np.nonzero(inv[:, j] >= 0)[0]
        dx[t] += dx_perm[inv[t, j]]

    grads = {"dw_gate_up": dw_gate_up, "dw_down": dw_down}
    if fwd["ws_gate_up"] is not None and fwd["ws_gate_up"].shape[0] > 0:
        ws_gu, ws_d = fwd["ws_gate_up"], fwd["ws_down"]
        dws_gu = np.zeros_like(ws_gu)
        dws_d = np.zeros_like(ws_d)
        for s, (G, U, H) in enumerate(fwd["shared"]):
            dgu, dws_d[s] = expert_down_backward_step(dy, G, U, H, ws_d[s], quant, st)
            dx_s, dws_gu[s] = expert_gate_up_backward_step(dgu, x, ws_gu[s], quant)
            dx_shared = dx_s if s == 0 else dx_shared + dx_s
        dx += st(dx_shared, "act")
        grads["dws_gate_up"] = dws_gu
        grads["dws_down"] = dws_d

    # router (the balancing statistic over the real tokens when masked)
    if mask is not None:
        counts, _ = real_token_counts(idx, mask, E)
    gsc, dz = router_backward(dy, fwd["y_perm"], inv, p, idx, w, fwd["renorm"], counts, aux_coef, st, mask,
                              fwd.get("router", "softmax"))
    grads["dw_router"] = dz.T @ x
    grads["dbias"] = dz.sum(axis=0)
    dx += dz @ w_r
    grads["dx"] = dx
    grads["dz"] = dz
    grads["g"] = gsc
    grads["dy_perm"] = dy_perm
    grads["dx_perm"] = dx_perm
    return grads


def layer_loss(fwd, dy, aux_coef=0.0, mask=None):
    """L = <dy, y> + aux_coef * aux  (the scalar whose gradient layer_backward
    returns; used by the finite-difference pins)."""
    if mask is None:
        st = aux_statistics(fwd["p"], fwd["counts"], fwd["top_k"])
    else:
        rc, _ = real_token_counts(fwd["idx"], mask, fwd["p"].shape[1])
        st = aux_statistics(fwd["p"], rc, fwd["top_k"], mask)
    return float((dy * fwd["y"]).sum()) + aux_coef * st["aux"]
