"""Distance from the exact layer of a bf16 layer that keeps some of its
intermediates in bf16 -- the figures behind the library's choice of which
intermediates a bf16 layer keeps in f32.

spark-gpt README, feature list: the experts are BF16 grouped GEMMs, so their
operands (x, the weights, H, dY_perm, [dG | dU]) are bf16.  Which of the
values the layer keeps between its steps are *also* rounded is an
implementation choice; this script measures, at the skewed 128-expert top-8
workload (16384 tokens, d_model 2048), how far each choice lands from the
exact fp64 oracle, in the measure the parity tests apply:
max(|err| - half an ulp of the bf16 output) / RMS per tensor (per expert,
floored at the stacked RMS, for the weight gradients), with the outputs
rounded to bf16 as a layer returning bf16 must.

Configurations (everything not named is computed exactly in fp64 here):
  library       GEMM operands bf16; [G | U], Y_perm and dX_perm kept in f32;
                the down projection's input gradient formed from dy's own
                rows with the routing weight applied after the product, the
                routing-weight gradient g = <dy W_d, H> from f32 G, U, and
                the down weight gradient from dy's own rows and bf16(w H)
                with H in f32
  [G | U] bf16  as library, the saved pre-activations rounded to bf16 (the
                SwiGLU backward and the routing-weight gradient read them)
  Y_perm bf16   as library, Y_perm rounded to bf16
  dX_perm bf16  as library, dX_perm rounded to bf16
  dW_down from bf16(w dy), bf16(H)
                as library, the down weight gradient's operands rounded
                separately (two roundings per product instead of one)
  all bf16      [G | U], dX_perm rounded to bf16, g = <dy, Y_perm> from the
                bf16-H down product, the down dgrad reading bf16(w dy), and
                the down weight gradient from bf16(w dy), bf16(H)

The exact reference is ``oracle.layer_forward`` / ``layer_backward``; the
variants re-run the same chain in fp64 with the stated roundings
(``oracle.round_to_format``).  No GPU value enters.

    python tests/golden/bf16_storage_distance.py    # writes bf16_storage_distance.json beside it
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import moe_inputs as MI  # noqa: E402
import oracle as O  # noqa: E402

WORKLOAD = "t16384_d2048_e128k8_i768_zipf_bf16"
CONFIGS = {"library": set(), "[G | U] bf16": {"GU"}, "Y_perm bf16": {"Y"}, "dX_perm bf16": {"dXp"},
           "dW_down from bf16(w dy), bf16(H)": {"wgH"},
           "all bf16": {"GU", "gH", "dXp", "dYw", "wgH"}}


def half_ulp_bf16(v):
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    return np.ldexp(0.5, np.maximum(ex - 1, -126) - 7)


def excess(got, ref, floor=0.0):
    rms = max(float(np.sqrt(np.mean(ref * ref))), floor)
    e = np.abs(got - ref) - half_ulp_bf16(np.maximum(np.abs(got), np.abs(ref)))
    return float(e.max()) / rms


def variant(wl, f, xf, xb, flags):
    R = lambda a: O.round_to_format(a, "bf16")
    x, Wr, Wgu, Wd, dy = f["x"], f["w_router"], f["w_gate_up"], f["w_down"], f["dy"]
    idx, w, inv, off, perm, p = xf["idx"], xf["w"], xf["inv"], xf["offsets"], xf["perm_token"], xf["p"]
    E, k, T, d, I = wl.E, wl.k, wl.T, wl.d, wl.I
    A = T * k
    slot = np.empty(A, dtype=np.int64)
    for j in range(k):
        slot[inv[:, j]] = j
    wr = w[perm, slot]
    y = np.zeros((T, d)); dx = np.zeros((T, d)); g = np.zeros(A)
    dwgu = np.zeros_like(Wgu); dwd = np.zeros_like(Wd)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        X = x[perm[r0:r1]]
        G, U = X @ Wgu[e, :I].T, X @ Wgu[e, I:].T
        Hx = O.silu(G) * U
        Hb = R(Hx)                                       # operand of the down GEMM
        Yp = Hb @ Wd[e].T
        np.add.at(y, perm[r0:r1], wr[r0:r1, None] * (R(Yp) if "Y" in flags else Yp))
        dyr = dy[perm[r0:r1]]
        Gs, Us = (R(G), R(U)) if "GU" in flags else (G, U)   # the saved pre-activations
        Hs = O.silu(Gs) * Us                                  # H as the backward forms it
        g[r0:r1] = (dyr * Yp).sum(1) if "gH" in flags else (dyr * (Hs @ Wd[e].T)).sum(1)
        dYw = R(wr[r0:r1, None] * dyr)
        dH = dYw @ Wd[e] if "dYw" in flags else wr[r0:r1, None] * (dyr @ Wd[e])
        sg = 1.0 / (1.0 + np.exp(-Gs))
        dGU = R(np.concatenate([dH * Us * sg * (1 + Gs * (1 - sg)), dH * Gs * sg], 1))   # operand
        dwd[e] = dYw.T @ Hb if "wgH" in flags else dyr.T @ R(wr[r0:r1, None] * Hs)
        dwgu[e] = dGU.T @ X
        dX = dGU @ Wgu[e]
        np.add.at(dx, perm[r0:r1], R(dX) if "dXp" in flags else dX)
    gs = np.stack([g[inv[:, j]] for j in range(k)], 1)
    psel = np.take_along_axis(p, idx, 1)
    S = psel.sum(1, keepdims=True)
    dps = (gs - (w * gs).sum(1, keepdims=True)) / S if wl.renorm else gs
    dp = np.zeros_like(p)
    np.put_along_axis(dp, idx, dps, 1)
    dp += wl.aux_coef * E * (xf["counts"] / (T * k))[None, :] / T
    dz = p * (dp - (p * dp).sum(1, keepdims=True))
    dwr = dz.T @ x
    dx += dz @ Wr
    fl_gu = float(np.sqrt(np.mean(xb["dw_gate_up"] ** 2)))
    fl_d = float(np.sqrt(np.mean(xb["dw_down"] ** 2)))
    return {"y": excess(R(y), xf["y"]), "dx": excess(R(dx), xb["dx"]),
            "dW_router": excess(R(dwr), xb["dw_router"]),
            "dW_gate_up": max(excess(R(dwgu[e]), xb["dw_gate_up"][e], fl_gu) for e in range(E)),
            "dW_down": max(excess(R(dwd[e]), xb["dw_down"][e], fl_d) for e in range(E))}


def main():
    wl = MI.WORKLOADS[WORKLOAD]
    f = {k: MI.to_f64(v) for k, v in MI.make_inputs(wl).items()}
    xf = O.layer_forward(f["x"], f["w_router"], f["w_gate_up"], f["w_down"], top_k=wl.k, renorm=wl.renorm,
                         bias=f["bias"])
    xb = O.layer_backward(xf, f["dy"], aux_coef=wl.aux_coef)
    res = {"workload": WORKLOAD, "describe": MI.describe(wl), "bar": 2e-2,
           "measure": "max(|err| - ulp/2) / RMS against the exact fp64 oracle, outputs rounded to bf16",
           "configs": {name: variant(wl, f, xf, xb, flags) for name, flags in CONFIGS.items()}}
    path = os.path.join(HERE, "bf16_storage_distance.json")
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
    print(path)


if __name__ == "__main__":
    main()
