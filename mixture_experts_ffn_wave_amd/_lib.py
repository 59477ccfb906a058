"""ctypes binding of libmoe.so.

Argument marshalling only: every function below checks tensor shapes, dtypes,
devices and contiguity, passes ``data_ptr()`` values and the current HIP
stream to the C ABI in ``include/moe.h``, and raises on a non-zero status.
All arithmetic runs in the library's kernels; there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_F16, MOE_BF16, MOE_MXFP8_E4M3 = 0, 1, 2, 3
MOE_ERR_SCRATCH = -6
ROUTER_KINDS = {"softmax": 0, "relu": 1, "expert_choice": 2}
_DTYPE_CODE = {torch.float32: MOE_F32, torch.float16: MOE_F16, torch.bfloat16: MOE_BF16}

c_int32, c_int64, c_float, c_void_p, c_size_t = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                                   ctypes.c_void_p, ctypes.c_size_t)


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", c_int64), ("d_model", c_int32), ("n_experts", c_int32), ("top_k", c_int32),
                ("d_ff", c_int32), ("n_shared", c_int32), ("d_ff_shared", c_int32),
                ("renorm", c_int32), ("has_router_bias", c_int32), ("act_dtype", c_int32),
                ("expert_dtype", c_int32), ("aux_coef", c_float), ("router", c_int32), ("mx_fused", c_int32)]


_FFN_FIELDS = ["x_perm", "offsets", "w_gate_up", "w_down", "gu", "h", "y_perm", "x", "ws_gate_up",
               "ws_down", "gu_shared", "h_shared", "y_shared", "perm_token", "mx_saved"]
_SAVED_FIELDS = ["x", "w_router", "probs", "topk_idx", "topk_w", "counts", "offsets", "inv_perm",
                 "x_perm", "gu", "h", "y_perm", "w_gate_up", "w_down", "ws_gate_up", "ws_down",
                 "gu_shared", "h_shared", "real_mask", "real_counts", "perm_token", "mx_saved"]
_GRAD_FIELDS = ["dx", "dw_router", "dbias", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down"]


class MoeFfnArgs(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in _FFN_FIELDS]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in _SAVED_FIELDS]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in _GRAD_FIELDS]


class MoeAuxScalars(ctypes.Structure):
    _fields_ = [("aux", c_float), ("aux_raw", c_float), ("entropy_mean", c_float),
                ("count_cv", c_float), ("count_min", c_int32), ("count_max", c_int32),
                ("n_unused", c_int32), ("reserved", c_int32)]


# Every symbol include/moe.h declares, with its ctypes signature.
SIGNATURES = {
    "moe_plan_create": (c_int32, [ctypes.POINTER(MoeConfig), ctypes.POINTER(c_void_p)]),
    "moe_plan_destroy": (None, [c_void_p]),
    "moe_workspace_bytes": (c_size_t, [c_void_p]),
    "moe_mx_saved_bytes": (c_size_t, [c_void_p]),
    "moe_status_string": (ctypes.c_char_p, [c_int32]),
    "moe_version": (ctypes.c_char_p, []),
    "moe_route": (c_int32, [c_void_p] * 8),
    "moe_route_balanced": (c_int32, [c_void_p] * 9),
    "moe_route_sinkhorn": (c_int32, [c_void_p] * 4 + [c_int32] + [c_void_p] * 5 + [c_size_t, c_void_p]),
    "moe_route_expert_choice": (c_int32, [c_void_p] * 8 + [c_size_t, c_void_p]),
    "moe_balance_update": (c_int32, [c_void_p, c_void_p, c_void_p, c_float, c_void_p]),
    "moe_permute": (c_int32, [c_void_p] * 9 + [c_size_t, c_void_p]),
    "moe_permute_noalloc": (c_int32, [c_void_p] * 9),
    "moe_expert_ffn": (c_int32, [c_void_p, ctypes.POINTER(MoeFfnArgs), c_void_p, c_size_t, c_void_p]),
    "moe_combine": (c_int32, [c_void_p] * 7),
    "moe_backward": (c_int32, [c_void_p, ctypes.POINTER(MoeSaved), c_void_p, ctypes.POINTER(MoeGrads),
                               c_void_p, c_size_t, c_void_p]),
    "moe_aux_stats": (c_int32, [c_void_p] * 7 + [c_size_t, c_void_p]),
    "moe_aux_stats_masked": (c_int32, [c_void_p] * 9 + [c_size_t, c_void_p]),
    "moe_probe_enable": (c_int32, [c_void_p, ctypes.c_char_p, c_int32]),
    "moe_probe_read": (c_int32, [c_void_p, ctypes.POINTER(c_float), ctypes.POINTER(c_int32)]),
    "moe_kernel_names": (ctypes.c_char_p, []),
    "moe_mx_quantize_rows": (c_int32, [c_void_p, c_int32, c_int64, c_int32, c_void_p, c_void_p, c_void_p]),
    "moe_keep_intermediates": (c_int32, [c_void_p, c_int32]),
    "moe_mx_saved_region": (c_int32, [c_void_p, ctypes.c_char_p, ctypes.POINTER(c_size_t),
                                      ctypes.POINTER(c_size_t)]),
    "moe_workspace_region": (c_int32, [c_void_p, ctypes.c_char_p, ctypes.POINTER(c_size_t),
                                       ctypes.POINTER(c_size_t)]),
}

_lib = None


def lib():
    """Load libmoe.so once.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with `python -m mixture_experts_ffn_wave_amd.build` "
                "(or __graft_entry__.build()).  The MoE layer has no non-HIP implementation.")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


class MoeError(RuntimeError):
    def __init__(self, call, status):
        self.status = status
        msg = lib().moe_status_string(status).decode()
        super().__init__(f"{call} failed with status {status}: {msg}")


def _check(call, st):
    if st != 0:
        raise MoeError(call, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, shape, dtype, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


class Plan:
    """An immutable layer plan (moe_plan_create).  Host-only; safe to build
    without a GPU."""

    def __init__(self, T, d_model, n_experts, top_k, d_ff, n_shared=0, d_ff_shared=0, renorm=True,
                 has_router_bias=False, dtype=torch.bfloat16, aux_coef=0.01, expert_dtype=None, router="softmax",
                 mx_fused=False):
        if dtype not in _DTYPE_CODE:
            raise ValueError(f"unsupported activation dtype {dtype}")
        code = _DTYPE_CODE[dtype]
        if expert_dtype is None:
            ecode = code
        elif expert_dtype == "mxfp8":
            ecode = MOE_MXFP8_E4M3
        else:
            ecode = expert_dtype
        if router not in ROUTER_KINDS:
            raise ValueError(f"unknown router {router!r}")
        self.cfg = MoeConfig(T, d_model, n_experts, top_k, d_ff, n_shared, d_ff_shared, int(renorm),
                             int(has_router_bias), code, ecode, aux_coef, ROUTER_KINDS[router], int(mx_fused))
        self.mx_fused = bool(mx_fused)                     # MX: the fused path only (smaller workspace)
        self.router = router
        # routing slots per token (topk_idx, topk_w, inv_perm are [T, slots]):
        # top_k, or one per expert for expert choice
        self.slots = n_experts if router == "expert_choice" else top_k
        self.dtype = dtype
        self.mx = ecode == MOE_MXFP8_E4M3                  # MX-fp8 experts
        self.T, self.d, self.E, self.k, self.I = T, d_model, n_experts, top_k, d_ff
        self.Ns, self.Is = n_shared, (d_ff_shared if n_shared else 0)
        self.renorm, self.has_bias, self.aux_coef = bool(renorm), bool(has_router_bias), aux_coef
        # storage of the saved [G | U], of Y_perm and of the experts' input
        # gradient rows (include/moe.h): f32 in a bf16 layer with bf16 experts
        if self.mx:
            self.gu_dtype = self.y_perm_dtype = self.dx_rows_dtype = dtype            # bf16
        else:
            wide = torch.float32 if dtype == torch.bfloat16 else dtype
            self.gu_dtype = self.y_perm_dtype = self.dx_rows_dtype = wide
        h = c_void_p()
        _check("moe_plan_create", lib().moe_plan_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def workspace_bytes(self):
        return int(lib().moe_workspace_bytes(self._h))

    def mx_saved_bytes(self):
        """Bytes of the optional MX-fp8 saved-codes buffer (0 unless MX)."""
        return int(lib().moe_mx_saved_bytes(self._h))

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().moe_plan_destroy(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------ the six calls --

def moe_route(plan, x, w_router, bias, probs, topk_idx, topk_w, stream=None):
    T, d, E, k, dt = plan.T, plan.d, plan.E, plan.k, plan.dtype
    _need(x, "x", (T, d), dt); _need(w_router, "w_router", (E, d), dt)
    _need(probs, "probs", (T, E), torch.float32)
    _need(topk_idx, "topk_idx", (T, plan.slots), torch.int32); _need(topk_w, "topk_w", (T, plan.slots), torch.float32)
    if plan.has_bias:
        _need(bias, "bias", (E,), torch.float32)
    st = lib().moe_route(plan.handle, _ptr(x), _ptr(w_router), _ptr(bias) if plan.has_bias else None,
                         _ptr(probs), _ptr(topk_idx), _ptr(topk_w), _stream(stream))
    _check("moe_route", st)


def moe_route_balanced(plan, x, w_router, bias, sel_bias, probs, topk_idx, topk_w, stream=None):
    T, d, E, k, dt = plan.T, plan.d, plan.E, plan.k, plan.dtype
    _need(x, "x", (T, d), dt); _need(w_router, "w_router", (E, d), dt)
    _need(sel_bias, "sel_bias", (E,), torch.float32)
    _need(probs, "probs", (T, E), torch.float32)
    _need(topk_idx, "topk_idx", (T, plan.slots), torch.int32); _need(topk_w, "topk_w", (T, plan.slots), torch.float32)
    if plan.has_bias:
        _need(bias, "bias", (E,), torch.float32)
    st = lib().moe_route_balanced(plan.handle, _ptr(x), _ptr(w_router), _ptr(bias) if plan.has_bias else None,
                                  _ptr(sel_bias), _ptr(probs), _ptr(topk_idx), _ptr(topk_w), _stream(stream))
    _check("moe_route_balanced", st)


def moe_route_sinkhorn(plan, x, w_router, bias, n_iter, probs, topk_idx, topk_w, col_scale, ws, stream=None):
    T, d, E, k, dt = plan.T, plan.d, plan.E, plan.k, plan.dtype
    _need(x, "x", (T, d), dt); _need(w_router, "w_router", (E, d), dt)
    _need(probs, "probs", (T, E), torch.float32)
    _need(topk_idx, "topk_idx", (T, plan.slots), torch.int32); _need(topk_w, "topk_w", (T, plan.slots), torch.float32)
    _need(col_scale, "col_scale", (E,), torch.float32)
    if plan.has_bias:
        _need(bias, "bias", (E,), torch.float32)
    st = lib().moe_route_sinkhorn(plan.handle, _ptr(x), _ptr(w_router), _ptr(bias) if plan.has_bias else None,
                                  int(n_iter), _ptr(probs), _ptr(topk_idx), _ptr(topk_w), _ptr(col_scale),
                                  _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_route_sinkhorn", st)


def moe_route_expert_choice(plan, x, w_router, bias, probs, topk_idx, topk_w, ws, stream=None):
    T, d, E, dt = plan.T, plan.d, plan.E, plan.dtype
    _need(x, "x", (T, d), dt); _need(w_router, "w_router", (E, d), dt)
    _need(probs, "probs", (T, E), torch.float32)
    _need(topk_idx, "topk_idx", (T, plan.slots), torch.int32)
    _need(topk_w, "topk_w", (T, plan.slots), torch.float32)
    if plan.has_bias:
        _need(bias, "bias", (E,), torch.float32)
    st = lib().moe_route_expert_choice(plan.handle, _ptr(x), _ptr(w_router), _ptr(bias) if plan.has_bias else None,
                                       _ptr(probs), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(),
                                       _stream(stream))
    _check("moe_route_expert_choice", st)


def moe_balance_update(plan, counts, sel_bias, gamma, stream=None):
    _need(counts, "counts", (plan.E,), torch.int32); _need(sel_bias, "sel_bias", (plan.E,), torch.float32)
    st = lib().moe_balance_update(plan.handle, _ptr(counts), _ptr(sel_bias), c_float(gamma), _stream(stream))
    _check("moe_balance_update", st)


def moe_permute(plan, topk_idx, x, counts, offsets, perm_token, inv_perm, x_perm, ws, stream=None):
    T, d, E, k, dt = plan.T, plan.d, plan.E, plan.k, plan.dtype
    _need(topk_idx, "topk_idx", (T, plan.slots), torch.int32); _need(x, "x", (T, d), dt)
    _need(counts, "counts", (E,), torch.int32); _need(offsets, "offsets", (E + 1,), torch.int32)
    _need(perm_token, "perm_token", (T * k,), torch.int32); _need(inv_perm, "inv_perm", (T, plan.slots), torch.int32)
    if x_perm is not None:                     # None: indices only (MX experts gathering on load)
        _need(x_perm, "x_perm", (T * k, d), dt)
    st = lib().moe_permute(plan.handle, _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
                           _ptr(perm_token), _ptr(inv_perm), _ptr(x_perm), _ptr(ws), ws.numel(),
                           _stream(stream))
    _check("moe_permute", st)


def moe_permute_noalloc(plan, topk_idx, x, counts, offsets, perm_token, inv_perm, x_perm, stream=None):
    """moe_permute with its scratch in the library's fixed device array (no workspace)."""
    T, d, E, k, dt = plan.T, plan.d, plan.E, plan.k, plan.dtype
    _need(topk_idx, "topk_idx", (T, plan.slots), torch.int32); _need(x, "x", (T, d), dt)
    _need(counts, "counts", (E,), torch.int32); _need(offsets, "offsets", (E + 1,), torch.int32)
    _need(perm_token, "perm_token", (T * k,), torch.int32); _need(inv_perm, "inv_perm", (T, plan.slots), torch.int32)
    if x_perm is not None:
        _need(x_perm, "x_perm", (T * k, d), dt)
    st = lib().moe_permute_noalloc(plan.handle, _ptr(topk_idx), _ptr(x), _ptr(counts), _ptr(offsets),
                                   _ptr(perm_token), _ptr(inv_perm), _ptr(x_perm), _stream(stream))
    _check("moe_permute_noalloc", st)


def moe_expert_ffn(plan, x_perm, offsets, w_gate_up, w_down, gu, h, y_perm, x=None, ws_gate_up=None,
                   ws_down=None, gu_shared=None, h_shared=None, y_shared=None, ws=None, stream=None,
                   perm_token=None, mx_saved=None):
    T, d, E, k, I, dt = plan.T, plan.d, plan.E, plan.k, plan.I, plan.dtype
    A = T * k
    if x_perm is not None or perm_token is None:   # x_perm may be omitted when MX experts gather on load
        _need(x_perm, "x_perm", (A, d), dt)
    _need(offsets, "offsets", (E + 1,), torch.int32)
    _need(w_gate_up, "w_gate_up", (E, 2 * I, d), dt); _need(w_down, "w_down", (E, d, I), dt)
    _need(gu, "gu", (A, 2 * I), plan.gu_dtype)
    if h is not None or mx_saved is None:            # H may be omitted when MX experts save their codes
        _need(h, "h", (A, I), dt)
    _need(y_perm, "y_perm", (A, d), plan.y_perm_dtype)
    args = MoeFfnArgs(*[None] * len(_FFN_FIELDS))
    for n, t in [("x_perm", x_perm), ("offsets", offsets), ("w_gate_up", w_gate_up), ("w_down", w_down),
                 ("gu", gu), ("h", h), ("y_perm", y_perm)]:
        setattr(args, n, t.data_ptr() if t is not None else None)
    if plan.Ns > 0:
        Ns, Is = plan.Ns, plan.Is
        _need(x, "x", (T, d), dt); _need(ws_gate_up, "ws_gate_up", (Ns, 2 * Is, d), dt)
        _need(ws_down, "ws_down", (Ns, d, Is), dt)
        _need(gu_shared, "gu_shared", (T, 2 * Ns * Is), plan.gu_dtype)
        if h_shared is not None or mx_saved is None:
            _need(h_shared, "h_shared", (T, Ns * Is), dt)
        _need(y_shared, "y_shared", (T, d), dt)
        for n, t in [("x", x), ("ws_gate_up", ws_gate_up), ("ws_down", ws_down), ("gu_shared", gu_shared),
                     ("h_shared", h_shared), ("y_shared", y_shared)]:
            setattr(args, n, t.data_ptr() if t is not None else None)
    if perm_token is not None:
        _need(perm_token, "perm_token", (A,), torch.int32)
        _need(x, "x", (T, d), dt)
        args.perm_token = perm_token.data_ptr()
        args.x = x.data_ptr()
    if mx_saved is not None:
        _need(mx_saved, "mx_saved", (plan.mx_saved_bytes(),), torch.uint8)
        args.mx_saved = mx_saved.data_ptr()
    st = lib().moe_expert_ffn(plan.handle, ctypes.byref(args), _ptr(ws), ws.numel() if ws is not None else 0,
                              _stream(stream))
    _check("moe_expert_ffn", st)


def moe_combine(plan, y_perm, inv_perm, topk_w, y_shared, y, stream=None):
    T, d, k, dt = plan.T, plan.d, plan.k, plan.dtype
    _need(y_perm, "y_perm", (T * k, d), plan.y_perm_dtype); _need(inv_perm, "inv_perm", (T, plan.slots), torch.int32)
    _need(topk_w, "topk_w", (T, plan.slots), torch.float32); _need(y, "y", (T, d), dt)
    if y_shared is not None:
        _need(y_shared, "y_shared", (T, d), dt)
    st = lib().moe_combine(plan.handle, _ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(y_shared), _ptr(y),
                           _stream(stream))
    _check("moe_combine", st)


def moe_backward(plan, saved, dy, grads, ws, stream=None):
    """``saved`` and ``grads`` are dicts keyed like the moe_saved / moe_grads
    fields; absent or None entries are passed as NULL."""
    T, d, E, I, dt = plan.T, plan.d, plan.E, plan.I, plan.dtype
    _need(dy, "dy", (T, d), dt)
    _need(grads["dx"], "dx", (T, d), dt); _need(grads["dw_router"], "dw_router", (E, d), dt)
    _need(grads["dw_gate_up"], "dw_gate_up", (E, 2 * I, d), dt); _need(grads["dw_down"], "dw_down", (E, d, I), dt)
    if grads.get("dbias") is not None:
        _need(grads["dbias"], "dbias", (E,), torch.float32)
    if plan.Ns > 0:
        _need(grads["dws_gate_up"], "dws_gate_up", (plan.Ns, 2 * plan.Is, d), dt)
        _need(grads["dws_down"], "dws_down", (plan.Ns, d, plan.Is), dt)
    for key in _SAVED_FIELDS:
        t = saved.get(key)
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"saved[{key}] must be a contiguous GPU tensor")
    sv = MoeSaved(*[(saved[n].data_ptr() if saved.get(n) is not None else None) for n in _SAVED_FIELDS])
    gr = MoeGrads(*[(grads[n].data_ptr() if grads.get(n) is not None else None) for n in _GRAD_FIELDS])
    st = lib().moe_backward(plan.handle, ctypes.byref(sv), _ptr(dy), ctypes.byref(gr), _ptr(ws), ws.numel(),
                            _stream(stream))
    _check("moe_backward", st)


def moe_aux_stats(plan, probs, counts, f, p_mean, out, ws, stream=None):
    """``out`` is a 32-byte uint8 GPU tensor that receives one moe_aux_scalars."""
    T, E = plan.T, plan.E
    _need(probs, "probs", (T, E), torch.float32); _need(counts, "counts", (E,), torch.int32)
    _need(f, "f", (E,), torch.float32); _need(p_mean, "p_mean", (E,), torch.float32)
    _need(out, "out", (ctypes.sizeof(MoeAuxScalars),), torch.uint8)
    st = lib().moe_aux_stats(plan.handle, _ptr(probs), _ptr(counts), _ptr(f), _ptr(p_mean), _ptr(out),
                             _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_aux_stats", st)


def moe_aux_stats_masked(plan, probs, topk_idx, real_mask, f, p_mean, real_counts, out, ws, stream=None):
    """The statistic over real tokens (real_mask [T] int32, 0 = filler);
    real_counts [E+1] int32 receives their counts and their number."""
    T, E, k = plan.T, plan.E, plan.k
    _need(probs, "probs", (T, E), torch.float32); _need(topk_idx, "topk_idx", (T, plan.slots), torch.int32)
    _need(real_mask, "real_mask", (T,), torch.int32)
    _need(f, "f", (E,), torch.float32); _need(p_mean, "p_mean", (E,), torch.float32)
    _need(real_counts, "real_counts", (E + 1,), torch.int32)
    _need(out, "out", (ctypes.sizeof(MoeAuxScalars),), torch.uint8)
    st = lib().moe_aux_stats_masked(plan.handle, _ptr(probs), _ptr(topk_idx), _ptr(real_mask), _ptr(f),
                                    _ptr(p_mean), _ptr(real_counts), _ptr(out), _ptr(ws), ws.numel(),
                                    _stream(stream))
    _check("moe_aux_stats_masked", st)


def decode_aux(out_tensor):
    """Copy a device moe_aux_scalars (uint8 tensor) to a Python dict."""
    raw = bytes(out_tensor.cpu().numpy().tobytes())
    s = MoeAuxScalars.from_buffer_copy(raw)
    return {n: getattr(s, n) for n, _ in MoeAuxScalars._fields_ if n != "reserved"}


def probe_enable(plan, kernel, max_launches):
    _check("moe_probe_enable", lib().moe_probe_enable(plan.handle, kernel.encode(), int(max_launches)))


def probe_read(plan):
    ms, n = c_float(), c_int32()
    _check("moe_probe_read", lib().moe_probe_read(plan.handle, ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def workspace_region(plan, name):
    """(byte offset, bytes) of a backward intermediate in the workspace
    (moe_workspace_region)."""
    off, nb = c_size_t(), c_size_t()
    _check("moe_workspace_region", lib().moe_workspace_region(plan.handle, name.encode(), ctypes.byref(off),
                                                              ctypes.byref(nb)))
    return int(off.value), int(nb.value)


def mx_saved_region(plan, name):
    """(byte offset, bytes) of an operand in the MX saved-codes buffer
    (moe_mx_saved_region)."""
    off, nb = c_size_t(), c_size_t()
    _check("moe_mx_saved_region", lib().moe_mx_saved_region(plan.handle, name.encode(), ctypes.byref(off),
                                                            ctypes.byref(nb)))
    return int(off.value), int(nb.value)


def keep_intermediates(plan, keep=True):
    """MX-fp8 plans: make moe_backward also store the act-dtype [dG | dU]
    ("dgu", "dgu_shared"), which it otherwise reads only as MX operands."""
    _check("moe_keep_intermediates", lib().moe_keep_intermediates(plan.handle, int(bool(keep))))


def kernel_names():
    return lib().moe_kernel_names().decode().split(",")


def mx_quantize_rows(x, payload, scales, stream=None):
    """MX-fp8 quantisation of the rows of x [R, K] (bf16 or f16) into payload
    [R, K] uint8 and scales [R, K/32] uint8 (moe_mx_quantize_rows)."""
    if x.dim() != 2 or x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("x must be a 2-D bf16 or f16 tensor")
    R, K = x.shape
    _need(x, "x", (R, K), x.dtype)
    _need(payload, "payload", (R, K), torch.uint8)
    _need(scales, "scales", (R, K // 32), torch.uint8)
    _check("moe_mx_quantize_rows", lib().moe_mx_quantize_rows(
        _ptr(x), _DTYPE_CODE[x.dtype], R, K, _ptr(payload), _ptr(scales), _stream(stream)))
