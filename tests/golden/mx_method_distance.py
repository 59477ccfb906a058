"""Distance of the MX-fp8 layer (the method itself, computed exactly) from the
unquantised layer, at the fine-grained MX workload.

KohakUwULLM README, "Key features": the experts' matmuls run on e4m3 values
with one power-of-two scale per 32 elements.  This script runs the fp64
oracle twice on the same seeded inputs -- once exactly, once with every
expert GEMM operand MX-quantised (``quant=mx_fake_quant``, no other rounding)
-- and records, per tensor, max|MX - exact| / RMS(exact) and the relative
Frobenius distance.  It calls only ``oracle`` and the seeded input generator;
no GPU value enters it.  The figures say how far the method itself lands from
the unquantised layer, which bounds what any MX implementation can reach
against the exact oracle.

    python tests/golden/mx_method_distance.py   # writes mx_method_distance.json beside it
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import moe_inputs as MI  # noqa: E402
import oracle as O  # noqa: E402

WORKLOAD = "t16384_d2048_e64k6_i1408_s2x1408_mxfp8"


def run(wl, f, quant):
    fwd = O.layer_forward(f["x"], f["w_router"], f["w_gate_up"], f["w_down"], top_k=wl.k, renorm=wl.renorm,
                          bias=f.get("bias"), ws_gate_up=f.get("ws_gate_up"), ws_down=f.get("ws_down"), quant=quant)
    bwd = O.layer_backward(fwd, f["dy"], aux_coef=wl.aux_coef, quant=quant)
    keep = {"y": fwd["y"], "h": fwd["h"], "y_perm": fwd["y_perm"]}
    keep.update({k: bwd[k] for k in ("dx", "dw_router", "dbias", "dw_gate_up", "dw_down", "dws_gate_up",
                                     "dws_down")})
    return keep


def distances(wl):
    inp = MI.make_inputs(wl)
    f = {k: MI.to_f64(v) for k, v in inp.items()}
    exact = run(wl, f, None)
    mx = run(wl, f, O.mx_fake_quant)
    out = {}
    for k, ref in exact.items():
        got = mx[k]
        rms = float(np.sqrt(np.mean(ref * ref)))
        out[k] = {"max_abs_over_rms": float(np.abs(got - ref).max()) / rms,
                  "relative_frobenius": float(np.linalg.norm(got - ref) / np.linalg.norm(ref))}
    return out


def main():
    wl = MI.WORKLOADS[WORKLOAD]
    res = {"workload": WORKLOAD, "describe": MI.describe(wl),
           "what": "fp64 oracle with every expert GEMM operand MX-fp8 quantised, against the exact fp64 oracle",
           "tensors": distances(wl)}
    path = os.path.join(HERE, "mx_method_distance.json")
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
    print(path)


if __name__ == "__main__":
    main()
