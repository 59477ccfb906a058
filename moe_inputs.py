"""Seeded synthetic inputs for the MoE SwiGLU FFN layer.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the layer's arithmetic.  It is the only code that both the fp64 oracle
and the HIP path consume (the tests and the benchmark pass its tensors to both).

Recipe (one numpy PCG64 generator per workload, ``default_rng(seed)``), drawn
in float32 in this order: x ~ N(0,1) [T,d]; W_r ~ N(0, 0.02^2) [E,d];
W_gu ~ N(0, 0.02^2) [E,2I,d] (gate rows first, then up rows); W_d ~ N(0,
0.02^2) [E,d,I]; shared W_gu [Ns,2Is,d]; shared W_d [Ns,d,Is]; dy ~ N(0,1)
[T,d].  Each array is then rounded to nearest-even into the storage dtype.
The skewed workload adds a constant router bias b_e = ln(pi_e) with
pi_e proportional to (e+1)^-s (Zipf popularity, expert 0 most popular).
"""

from dataclasses import dataclass, replace
import numpy as np
import torch

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    n_shared: int = 0
    I_shared: int = 0
    renorm: bool = True
    dtype: str = "bf16"          # activations, router weight, expert weights (storage)
    expert_dtype: str = ""       # "" = same as dtype; "mxfp8" = MX e4m3 expert GEMMs
    zipf_s: float = 0.0          # > 0: constant router bias ln(pi_e), pi_e ~ (e+1)^-s
    aux_coef: float = 0.01
    seed: int = 0
    router: str = "softmax"      # "softmax" or "relu" (the ReLU router)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]

    @property
    def assignments(self):
        return self.T * self.k

    def with_(self, **kw):
        return replace(self, **kw)


# The five workloads, named by their shapes.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("t512_d256_e8k2_i128_f32", T=512, d=256, E=8, k=2, I=128, dtype="f32"),
        Workload("t16384_d512_e8k2_i768_bf16", T=16384, d=512, E=8, k=2, I=768, dtype="bf16"),
        Workload("t32768_d1536_e4k2_i3072_s1x3072_f16", T=32768, d=1536, E=4, k=2, I=3072,
                 n_shared=1, I_shared=3072, dtype="f16"),
        Workload("t16384_d2048_e128k8_i768_zipf_bf16", T=16384, d=2048, E=128, k=8, I=768,
                 dtype="bf16", zipf_s=1.1),
        Workload("t16384_d2048_e64k6_i1408_s2x1408_mxfp8", T=16384, d=2048, E=64, k=6, I=1408,
                 n_shared=2, I_shared=1408, dtype="bf16", expert_dtype="mxfp8"),
    ]
}

TINY = "t512_d256_e8k2_i128_f32"
BENCH = "t16384_d512_e8k2_i768_bf16"                 # the small bf16 workload (full-size parity case)
LARGEST = "t32768_d1536_e4k2_i3072_s1x3072_f16"      # the largest single-GPU workload: the benchmark's default


def zipf_bias(E, s):
    """ln(pi_e) with pi_e = (e+1)^-s / sum_e' (e'+1)^-s, as float32."""
    w = np.array([(e + 1.0) ** (-s) for e in range(E)], dtype=np.float64)
    return np.log(w / w.sum()).astype(np.float32)


def make_inputs(wl: Workload, seed=None, device="cpu"):
    """Draw every input of one fwd+bwd step of ``wl``.  Returns a dict of torch
    tensors in the storage dtype (bias in float32) on ``device``."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    dt = wl.torch_dtype

    def draw(shape, scale):
        a = rng.standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        return torch.from_numpy(a).to(dt)

    out = {}
    out["x"] = draw((wl.T, wl.d), 1.0)
    out["w_router"] = draw((wl.E, wl.d), 0.02)
    out["w_gate_up"] = draw((wl.E, 2 * wl.I, wl.d), 0.02)
    out["w_down"] = draw((wl.E, wl.d, wl.I), 0.02)
    if wl.n_shared > 0:
        out["ws_gate_up"] = draw((wl.n_shared, 2 * wl.I_shared, wl.d), 0.02)
        out["ws_down"] = draw((wl.n_shared, wl.d, wl.I_shared), 0.02)
    out["dy"] = draw((wl.T, wl.d), 1.0)
    out["bias"] = torch.from_numpy(zipf_bias(wl.E, wl.zipf_s)) if wl.zipf_s > 0 else None
    if device != "cpu":
        out = {k: (v.to(device) if v is not None else None) for k, v in out.items()}
    return out


def selection_bias(E, scale, seed=1):
    """A seeded per-expert selection bias (float32 numpy [E]) for the
    aux-loss-free balancing router: normal draws times ``scale``, a size
    comparable to the gaps between routing probabilities (about 1/E)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(E, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def real_token_mask(T, filler_frac=0.3, seed=2):
    """A seeded real-token mask (int32 numpy [T], 0 = filler): runs of filler
    tokens of random length, as padding between packed documents leaves
    them, covering about ``filler_frac`` of the batch, plus a filler tail."""
    rng = np.random.default_rng(seed)
    m = np.ones(T, dtype=np.int32)
    t = 0
    while t < T:
        t += int(rng.integers(16, 128))                 # a document
        n = int(rng.integers(1, 48))                    # then its padding
        if rng.random() < filler_frac * 2:
            m[t:t + n] = 0
        t += n
    m[T - T // 16:] = 0                                 # padded tail
    return m


def to_f64(t):
    """Exact upcast of a stored tensor to a float64 numpy array (None passes)."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()


def describe(wl: Workload):
    ed = wl.expert_dtype or wl.dtype
    return (f"T={wl.T} d={wl.d} E={wl.E} k={wl.k} I={wl.I} shared={wl.n_shared}x{wl.I_shared} "
            f"renorm={wl.renorm} dtype={wl.dtype} experts={ed} zipf={wl.zipf_s}" +
            (f" router={wl.router}" if wl.router != "softmax" else ""))

