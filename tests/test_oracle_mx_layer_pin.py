"""Pin of the oracle's MX-fp8 layer mode by brute force.

The oracle's MX mode (``layer_forward`` / ``layer_backward`` with
``quant=mx_fake_quant``) quantises each operand of each expert GEMM along that
GEMM's contraction axis (KohakUwULLM README, "Key features": e4m3 values with
one power-of-two UE8M0 scale per 32 elements, on the experts' matmuls).  Here
the same layer is written out with Python loops and nothing from ``oracle``
but the routing of the tokens (pinned on its own elsewhere):

  * the e4m3 grid is enumerated from the format's definition (OCP 8-bit
    floating point, E4M3: bias 7, three mantissa bits, subnormals m/8 * 2^-6,
    largest finite 448, no infinities) and a value is rounded to the nearest
    grid point, ties to the even code;
  * a block's scale exponent is found by counting up from -127 to the first x
    with max|v| <= 448 * 2^x (the no-overflow reading of the UE8M0 scale);
  * every GEMM is a triple loop over explicitly quantised operand blocks:
      gate/up   G, U = X W_g^T, X W_u^T   both operands blocked along d
      down      Y = H W_d^T               blocked along I
      dgrad     dH = dY W_d               blocked along d
                dX = [dG | dU] W_gu       blocked along 2I
      wgrad     dW_d = dY^T H             blocked along the expert's tokens
                dW_gu = [dG | dU]^T X     blocked along the expert's tokens
    where the token blocks restart at every expert segment and a short last
    block is padded with zeros;
  * the router, softmax, combine and routing gradient are not quantised.

The shape has an expert segment longer than 32 rows and not a multiple of 32,
so the segment-restarting token blocks differ from blocks over all rows, and
d = I = 64 (two blocks per row) with unequal operand axes, so a wrong blocking
axis changes the result.  A one-token-block-over-all-rows variant and an
every-axis-swapped variant of the oracle are checked to differ.
"""

import bisect
import math

import numpy as np
import pytest

import oracle as O

# ---------------------------------------------------------------- e4m3 grid

def _e4m3_positive_grid():
    """(value, code) of every finite non-negative e4m3 number, ascending."""
    out = []
    for ef in range(16):
        for m in range(8):
            if ef == 15 and m == 7:                 # the NaN code
                continue
            v = (m / 8.0) * 2.0 ** -6 if ef == 0 else (1.0 + m / 8.0) * 2.0 ** (ef - 7)
            out.append((v, ef * 8 + m))
    out.sort()
    return out


_GRID = _e4m3_positive_grid()
_GRID_V = [v for v, _ in _GRID]


def e4m3_nearest(v):
    """Nearest e4m3 value to v (ties to the even code), clamped to +-448."""
    a = abs(v)
    if a >= _GRID_V[-1]:
        q = _GRID_V[-1]
    else:
        i = bisect.bisect_left(_GRID_V, a)
        if _GRID_V[i] == a:
            q = a
        else:
            lo, hi = _GRID[i - 1], _GRID[i]
            dl, dh = a - lo[0], hi[0] - a
            if dl < dh:
                q = lo[0]
            elif dh < dl:
                q = hi[0]
            else:
                q = lo[0] if lo[1] % 2 == 0 else hi[0]
    return math.copysign(q, v) if v != 0 else 0.0


def block_exponent(amax):
    x = -127
    while x < 127 and amax > 448.0 * 2.0 ** x:
        x += 1
    return x


def quant_vector(vals):
    """Quantise-dequantise a list in consecutive blocks of 32 (zero padded)."""
    out = []
    for b0 in range(0, len(vals), 32):
        blk = list(vals[b0:b0 + 32])
        amax = max(abs(v) for v in blk) if blk else 0.0
        sc = 2.0 ** block_exponent(amax)
        out.extend(e4m3_nearest(v / sc) * sc for v in blk)
    return out


def quant_rows(M):
    """Each row blocked along its length."""
    return [quant_vector(r) for r in M]


def quant_cols(M):
    """Each column blocked along the rows (M a list of rows); returns rows."""
    nr, nc = len(M), len(M[0]) if M else 0
    cols = [quant_vector([M[r][c] for r in range(nr)]) for c in range(nc)]
    return [[cols[c][r] for c in range(nc)] for r in range(nr)]


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def matmul_nt(A, B):
    """A [m][k] times B [n][k] transposed -> [m][n]."""
    return [[dot(a, b) for b in B] for a in A]


def transpose(M):
    return [list(r) for r in zip(*M)] if M else []


def sig(a):
    return 1.0 / (1.0 + math.exp(-a))


# ----------------------------------------------------------- the MX layer

def brute_mx_layer(L, idx, w, perm_token, offsets, aux_coef, restart_segments=True):
    """Forward and backward of the MX layer with explicit loops, from the
    routing (idx, w, perm, offsets).  restart_segments=False blocks the
    weight gradients' token axis over all rows at once (a wrong reading, used
    only to show that this shape tells the two apart)."""
    x = L["x"].tolist()
    T, d = len(x), len(x[0])
    E, inter = L["w_gate_up"].shape[0], L["w_down"].shape[2]
    k = idx.shape[1]
    A = T * k
    dy = L["dy"].tolist()
    Wr = L["w_router"].tolist()
    # sorted row r -> (t, j)
    slot = {}
    for t in range(T):
        for j in range(k):
            slot[(int(idx[t, j]), t)] = j
    rows_tj = [(int(perm_token[r]), slot[(e, int(perm_token[r]))])
               for e in range(E) for r in range(offsets[e], offsets[e + 1])]

    def expert_fwd(X, wgu, wd):
        I2 = len(wgu) // 2
        GU = matmul_nt(quant_rows(X), quant_rows(wgu))                 # blocks along d
        G = [r[:I2] for r in GU]
        U = [r[I2:] for r in GU]
        H = [[g * sig(g) * u for g, u in zip(gr, ur)] for gr, ur in zip(G, U)]
        Y = matmul_nt(quant_rows(H), quant_rows(wd))                   # blocks along I
        return G, U, H, Y

    def token_blocks(M, seg_bounds):
        """Quantise the columns of M (rows = tokens) along the tokens, in
        blocks restarting at each segment start."""
        out = [None] * len(M)
        for s0, s1 in seg_bounds:
            if s1 > s0:
                q = quant_cols(M[s0:s1])
                out[s0:s1] = q
        return out

    def expert_bwd(dY, G, U, wgu, wd):
        # dH = dY W_d: dY rows along d, W_d [d][I] columns along d
        dH = matmul_nt(quant_rows(dY), transpose(quant_cols(wd)))
        dGU = []
        for r in range(len(dY)):
            dg = [dh * u * sig(g) * (1.0 + g * (1.0 - sig(g))) for dh, g, u in zip(dH[r], G[r], U[r])]
            du = [dh * g * sig(g) for dh, g in zip(dH[r], G[r])]
            dGU.append(dg + du)
        # dX = [dG | dU] W_gu: rows along 2I, W_gu [2I][d] columns along 2I
        dX = matmul_nt(quant_rows(dGU), transpose(quant_cols(wgu)))
        return dGU, dX

    # ---- routed experts
    x_perm = [x[t] for t, _ in rows_tj]
    Gp, Up, Hp, Yp = [None] * A, [None] * A, [None] * A, [None] * A
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        G, U, H, Y = expert_fwd(x_perm[r0:r1], L["w_gate_up"][e].tolist(), L["w_down"][e].tolist())
        Gp[r0:r1], Up[r0:r1], Hp[r0:r1], Yp[r0:r1] = G, U, H, Y
    # ---- shared experts (each applied to every token, weight 1)
    ns = 0 if L["ws_gate_up"] is None else L["ws_gate_up"].shape[0]
    shared = [expert_fwd(x, L["ws_gate_up"][s].tolist(), L["ws_down"][s].tolist()) for s in range(ns)]
    y = []
    for t in range(T):
        row = [0.0] * d
        for j in range(k):
            r = next(rr for rr, tj in enumerate(rows_tj) if tj == (t, j))
            row = [a + w[t, j] * b for a, b in zip(row, Yp[r])]
        for s in range(ns):
            row = [a + b for a, b in zip(row, shared[s][3][t])]
        y.append(row)

    # ---- backward of the experts
    dYp = [[w[t, j] * v for v in dy[t]] for t, j in rows_tj]
    dWgu = np.zeros(L["w_gate_up"].shape)
    dWd = np.zeros(L["w_down"].shape)
    dXp, dGUp = [None] * A, [None] * A
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            dGUp[r0:r1], dXp[r0:r1] = expert_bwd(dYp[r0:r1], Gp[r0:r1], Up[r0:r1], L["w_gate_up"][e].tolist(),
                                                 L["w_down"][e].tolist())
    # weight gradients: contraction over the tokens of each segment, blocks
    # restarting at its first row (or, restart_segments=False, blocks of 32
    # counted from row 0 of all A rows)
    segs = [(offsets[e], offsets[e + 1]) for e in range(E)] if restart_segments else [(0, A)]
    qdY, qH, qdGU, qX = (token_blocks(M, segs) for M in (dYp, Hp, dGUp, x_perm))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        for c in range(d):
            for i in range(inter):
                dWd[e, c, i] = sum(qdY[r][c] * qH[r][i] for r in range(r0, r1))
        for m in range(2 * inter):
            for c in range(d):
                dWgu[e, m, c] = sum(qdGU[r][m] * qX[r][c] for r in range(r0, r1))
    dx = [[0.0] * d for _ in range(T)]
    for r, (t, j) in enumerate(rows_tj):
        dx[t] = [a + b for a, b in zip(dx[t], dXp[r])]
    dWs_gu = np.zeros(L["ws_gate_up"].shape) if ns else None
    dWs_d = np.zeros(L["ws_down"].shape) if ns else None
    for s in range(ns):
        G, U, H, _ = shared[s]
        dGU, dX = expert_bwd(dy, G, U, L["ws_gate_up"][s].tolist(), L["ws_down"][s].tolist())
        qdY, qH, qdGU, qX = (token_blocks(M, [(0, T)]) for M in (dy, H, dGU, x))
        Is = len(G[0])
        for c in range(d):
            for i in range(Is):
                dWs_d[s, c, i] = sum(qdY[r][c] * qH[r][i] for r in range(T))
        for m in range(2 * Is):
            for c in range(d):
                dWs_gu[s, m, c] = sum(qdGU[r][m] * qX[r][c] for r in range(T))
        dx = [[a + b for a, b in zip(dx[t], dX[t])] for t in range(T)]

    # ---- router (never quantised)
    bias = L["bias"].tolist() if L["bias"] is not None else [0.0] * E
    p = []
    for t in range(T):
        z = [dot(x[t], Wr[e]) + bias[e] for e in range(E)]
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        sm = sum(ex)
        p.append([v / sm for v in ex])
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            counts[int(idx[t, j])] += 1
    dz = []
    for t in range(T):
        g = []
        for j in range(k):
            r = next(rr for rr, tj in enumerate(rows_tj) if tj == (t, j))
            g.append(dot(dy[t], Yp[r]))
        sel = [int(e) for e in idx[t]]
        S = sum(p[t][e] for e in sel)
        wg = sum(w[t, j] * g[j] for j in range(k))
        dp = [0.0] * E
        for j, e in enumerate(sel):
            dp[e] = (g[j] - wg) / S
        for e in range(E):
            dp[e] += aux_coef * E * (counts[e] / (T * k)) / T
        pdp = dot(p[t], dp)
        dz.append([p[t][e] * (dp[e] - pdp) for e in range(E)])
    dWr = [[sum(dz[t][e] * x[t][c] for t in range(T)) for c in range(d)] for e in range(E)]
    for t in range(T):
        dx[t] = [a + sum(dz[t][e] * Wr[e][c] for e in range(E)) for c, a in enumerate(dx[t])]
    out = dict(g=np.array(Gp), u=np.array(Up), h=np.array(Hp), y_perm=np.array(Yp), y=np.array(y),
               dx=np.array(dx), dw_router=np.array(dWr), dbias=np.array(dz).sum(axis=0),
               dw_gate_up=dWgu, dw_down=dWd)
    if ns:
        out["dws_gate_up"] = dWs_gu
        out["dws_down"] = dWs_d
    return out


# ------------------------------------------------------------------- tests

def _layer(seed, T=40, d=64, E=3, k=2, inter=64, n_shared=1, inter_s=64):
    rng = np.random.default_rng(seed)
    row_scale = np.exp(rng.standard_normal((T, 1)))              # blocks of unequal scale
    return dict(
        x=rng.standard_normal((T, d)) * row_scale,
        w_router=0.3 * rng.standard_normal((E, d)),
        w_gate_up=0.2 * rng.standard_normal((E, 2 * inter, d)) * np.exp(rng.standard_normal((E, 2 * inter, 1))),
        w_down=0.2 * rng.standard_normal((E, d, inter)) * np.exp(rng.standard_normal((E, 1, inter))),
        ws_gate_up=0.2 * rng.standard_normal((n_shared, 2 * inter_s, d)) if n_shared else None,
        ws_down=0.2 * rng.standard_normal((n_shared, d, inter_s)) if n_shared else None,
        bias=np.array([1.5, 0.0, -0.5])[:E],
        dy=rng.standard_normal((T, d)),
    )


def _oracle(L, k, renorm, aux_coef, quant):
    fwd = O.layer_forward(L["x"], L["w_router"], L["w_gate_up"], L["w_down"], top_k=k, renorm=renorm,
                          bias=L["bias"], ws_gate_up=L["ws_gate_up"], ws_down=L["ws_down"], quant=quant)
    bwd = O.layer_backward(fwd, L["dy"], aux_coef=aux_coef, quant=quant)
    return fwd, bwd


def _max_rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300))


KEYS_FWD = ["g", "u", "h", "y_perm", "y"]
KEYS_BWD = ["dx", "dw_router", "dbias", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"]


@pytest.fixture(scope="module")
def mx_case():
    k, aux = 2, 0.01
    L = _layer(seed=5)
    fwd, bwd = _oracle(L, k, True, aux, O.mx_fake_quant)
    counts = fwd["counts"]
    # the shape this pin needs: a segment longer than one token block and not a multiple of 32
    assert any(c > 32 and c % 32 for c in counts), counts
    ref = brute_mx_layer(L, fwd["idx"], fwd["w"], fwd["perm_token"], fwd["offsets"], aux)
    return L, k, aux, fwd, bwd, ref


def test_brute_force_e4m3_grid_and_scale():
    # the enumerated grid: 126 finite positive values plus zero, largest 448, smallest 2^-9
    assert len(_GRID) == 127 and _GRID_V[-1] == 448.0 and _GRID_V[1] == 2.0 ** -9
    # it agrees with the oracle's e4m3 rounding on a dense sweep, ties included
    v = np.concatenate([np.linspace(-500, 500, 20001), np.array(_GRID_V) * 1.0000001,
                        0.5 * (np.array(_GRID_V[1:]) + np.array(_GRID_V[:-1]))])
    assert np.array_equal(O.e4m3_round(v), np.array([e4m3_nearest(a) for a in v]))
    for amax in [0.0, 1e-40, 1.0, 448.0, 448.0000001, 3.7e5, 2.0 ** -100]:
        assert O.mx_block_scale(np.array([amax]))[0] == block_exponent(amax)


def test_mx_layer_forward_matches_brute_force(mx_case):
    L, k, aux, fwd, bwd, ref = mx_case
    for key in KEYS_FWD:
        assert _max_rel(fwd[key], ref[key]) < 1e-12, key
    # the shared experts' sum enters y; check it on its own too
    assert _max_rel(fwd["y_shared"], ref["y"] - O.combine(fwd["y_perm"], fwd["inv"], fwd["w"])) < 1e-12


def test_mx_layer_backward_matches_brute_force(mx_case):
    L, k, aux, fwd, bwd, ref = mx_case
    for key in KEYS_BWD:
        assert _max_rel(bwd[key], ref[key]) < 1e-12, key


def test_mx_layer_quantisation_is_not_a_no_op(mx_case):
    """The MX layer is measurably different from the exact one on this shape
    (every quantised step is exercised)."""
    L, k, aux, fwd, bwd, ref = mx_case
    efwd, ebwd = _oracle(L, k, True, aux, None)
    for key in ["h", "y", "dx", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"]:
        src = fwd if key in fwd else bwd
        dst = efwd if key in efwd else ebwd
        assert _max_rel(src[key], dst[key]) > 1e-4, key


def test_wrong_readings_are_told_apart(mx_case):
    """Token blocks over all rows instead of per segment, or every operand
    blocked along the other axis, move the result far beyond the pin's bar."""
    L, k, aux, fwd, bwd, ref = mx_case
    glob = brute_mx_layer(L, fwd["idx"], fwd["w"], fwd["perm_token"], fwd["offsets"], aux,
                          restart_segments=False)
    assert max(_max_rel(bwd[key], glob[key]) for key in ["dw_gate_up", "dw_down"]) > 1e-6
    swapped = lambda a, axis: O.mx_fake_quant(a, 1 - axis)
    sfwd, sbwd = _oracle(L, k, True, aux, swapped)
    assert _max_rel(sfwd["y"], ref["y"]) > 1e-4
    assert _max_rel(sbwd["dx"], ref["dx"]) > 1e-4
