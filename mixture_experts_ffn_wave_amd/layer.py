"""A plan plus the device buffers one fwd+bwd step of the layer needs.

Allocation only (torch is the device allocator here): every step of the
computation is one of the six C-ABI calls, issued in order on one stream with
no host synchronisation in between.
"""

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, plan: L.Plan, device="cuda"):
        self.plan = p = plan
        dev = torch.device(device)
        dt = p.dtype
        T, d, E, k, I, A = p.T, p.d, p.E, p.k, p.I, p.T * p.k
        z = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=dev)
        self.probs = z(T, E, dtype=torch.float32)
        self.topk_idx = z(T, p.slots, dtype=torch.int32)      # [T, slots]: slots = E for expert choice
        self.topk_w = z(T, p.slots, dtype=torch.float32)
        self.counts = z(E, dtype=torch.int32)
        self.offsets = z(E + 1, dtype=torch.int32)
        self.perm_token = z(A, dtype=torch.int32)
        # MX experts: the gate/up GEMM and its weight gradient gather x's rows
        # by perm_token instead of reading x_perm (False: the x_perm path);
        # the gather addresses x with 32-bit offsets
        self.mx_gather = plan.mx and T * d < 2 ** 31
        # x_perm is written only when something reads it: the non-MX experts,
        # the x_perm path, or a caller that inspects it (write_x_perm = True);
        # on the gather path it is allocated on first use
        self.write_x_perm = False
        self.inv_perm = z(T, p.slots, dtype=torch.int32)
        self._x_perm = None if self.mx_gather else z(A, d)
        self.gu = z(A, 2 * I, dtype=p.gu_dtype)
        # H: MX experts keep it only as codes unless store_h (allocated on first use)
        self._h = None if p.mx else z(A, I)
        self.y_perm = z(A, d, dtype=p.y_perm_dtype)
        self.y = z(T, d)
        if p.Ns > 0:
            NI = p.Ns * p.Is
            self.gu_shared = z(T, 2 * NI, dtype=p.gu_dtype)
            self._h_shared = None if p.mx else z(T, NI)
            self.y_shared = z(T, d)
        else:
            self.gu_shared = self._h_shared = self.y_shared = None
        self.grads = {
            "dx": z(T, d),
            "dw_router": z(E, d),
            "dbias": z(E, dtype=torch.float32),
            "dw_gate_up": z(E, 2 * I, d),
            "dw_down": z(E, d, I),
            "dws_gate_up": z(p.Ns, 2 * p.Is, d) if p.Ns else None,
            "dws_down": z(p.Ns, d, p.Is) if p.Ns else None,
        }
        self.f = z(E, dtype=torch.float32)
        self.p_mean = z(E, dtype=torch.float32)
        self.aux_out = torch.zeros(L.ctypes.sizeof(L.MoeAuxScalars), dtype=torch.uint8, device=dev)
        self.ws = torch.empty(max(p.workspace_bytes(), 256), dtype=torch.uint8, device=dev)
        # MX-fp8 experts: the forward saves the weights' and H's backward codes
        # for the backward (moe_ffn_args.mx_saved); False: the backward makes them
        self.mx_save = p.mx
        self.mx_saved = torch.empty(p.mx_saved_bytes(), dtype=torch.uint8, device=dev) if p.mx else None
        # with saved codes the MX layer needs H only as codes: store_h = True
        # also writes the act-dtype H (self.h, self.h_shared)
        self.store_h = not p.mx
        self.params = None
        self.sel_bias = None      # aux-loss-free balancing: set by enable_balancing()
        self.balance_gamma = 0.0
        self.sinkhorn_iters = 0   # Sinkhorn router: set by enable_sinkhorn()
        self.sinkhorn_b = None
        self.real_mask = None     # statistic over real tokens only: set by set_real_mask()
        self.real_counts = None

    @property
    def h(self):
        if self._h is None:
            p = self.plan
            self._h = torch.empty(p.T * p.k, p.I, dtype=p.dtype, device=self.probs.device)
        return self._h

    @property
    def h_shared(self):
        p = self.plan
        if self._h_shared is None and p.Ns > 0:
            self._h_shared = torch.empty(p.T, p.Ns * p.Is, dtype=p.dtype, device=self.probs.device)
        return self._h_shared

    @property
    def x_perm(self):
        if self._x_perm is None:
            p = self.plan
            self._x_perm = torch.empty(p.T * p.k, p.d, dtype=p.dtype, device=self.probs.device)
        return self._x_perm

    def set_real_mask(self, mask):
        """Compute the balancing statistic (and its gradient) over the tokens
        whose mask is non-zero only: mask [T] int32 device tensor, or None."""
        self.real_mask = mask
        self.real_counts = (torch.empty(self.plan.E + 1, dtype=torch.int32, device=self.probs.device)
                            if mask is not None else None)

    def enable_balancing(self, sel_bias=None, gamma=0.0):
        """Route with a per-expert selection bias (aux-loss-free balancing):
        zeros, or the given [E] f32 device tensor, which the layer then owns.
        With gamma > 0, step() ends with the bias update from the step's loads."""
        E = self.plan.E
        self.sel_bias = sel_bias if sel_bias is not None else torch.zeros(E, dtype=torch.float32,
                                                                          device=self.probs.device)
        self.balance_gamma = float(gamma)

    def enable_sinkhorn(self, n_iter):
        """Route with the Sinkhorn router (n_iter balancing rounds); the
        column scales of the last route call land in self.sinkhorn_b."""
        self.sinkhorn_iters = int(n_iter)
        self.sinkhorn_b = torch.empty(self.plan.E, dtype=torch.float32, device=self.probs.device)

    def update_balance(self, gamma, stream=None):
        """Step-end update of the selection bias from this step's counts."""
        L.moe_balance_update(self.plan, self.counts, self.sel_bias, gamma, stream)

    # -------------------------------------------------------------- forward
    def set_params(self, x, w_router, w_gate_up, w_down, bias=None, ws_gate_up=None, ws_down=None):
        self.params = dict(x=x, w_router=w_router, w_gate_up=w_gate_up, w_down=w_down, bias=bias,
                           ws_gate_up=ws_gate_up, ws_down=ws_down)

    def route(self, stream=None):
        q = self.params
        if self.plan.router == "expert_choice":
            L.moe_route_expert_choice(self.plan, q["x"], q["w_router"], q["bias"], self.probs, self.topk_idx,
                                      self.topk_w, self.ws, stream)
        elif self.sinkhorn_iters > 0:
            L.moe_route_sinkhorn(self.plan, q["x"], q["w_router"], q["bias"], self.sinkhorn_iters, self.probs,
                                 self.topk_idx, self.topk_w, self.sinkhorn_b, self.ws, stream)
        elif self.sel_bias is not None:
            L.moe_route_balanced(self.plan, q["x"], q["w_router"], q["bias"], self.sel_bias, self.probs,
                                 self.topk_idx, self.topk_w, stream)
        else:
            L.moe_route(self.plan, q["x"], q["w_router"], q["bias"], self.probs, self.topk_idx, self.topk_w,
                        stream)

    def dispatch_and_experts(self, stream=None):
        q = self.params
        xp = self.x_perm if (self.write_x_perm or not self.mx_gather) else None
        L.moe_permute(self.plan, self.topk_idx, q["x"], self.counts, self.offsets, self.perm_token,
                      self.inv_perm, xp, self.ws, stream)
        h = self.h if (self.store_h or not self.mx_save) else None
        hs = self.h_shared if h is not None else None
        L.moe_expert_ffn(self.plan, xp, self.offsets, q["w_gate_up"], q["w_down"], self.gu,
                         h, self.y_perm, q["x"], q["ws_gate_up"], q["ws_down"], self.gu_shared,
                         hs, self.y_shared, self.ws, stream,
                         perm_token=self.perm_token if self.mx_gather else None,
                         mx_saved=self.mx_saved if self.mx_save else None)
        L.moe_combine(self.plan, self.y_perm, self.inv_perm, self.topk_w, self.y_shared, self.y, stream)

    def forward(self, stream=None):
        self.route(stream)
        self.dispatch_and_experts(stream)
        return self.y

    # ------------------------------------------------------------- backward
    def saved(self):
        q = self.params
        # perm_token: the down dgrad of 16-bit / f32 experts gathers dy by it,
        # and MX experts on the gather path read x's rows through it
        return dict(x=q["x"], w_router=q["w_router"], probs=self.probs, topk_idx=self.topk_idx,
                    topk_w=self.topk_w, counts=self.counts, offsets=self.offsets, inv_perm=self.inv_perm,
                    x_perm=None if self.mx_gather else self._x_perm, gu=self.gu, h=self._h,
                    y_perm=self.y_perm, w_gate_up=q["w_gate_up"], w_down=q["w_down"],
                    ws_gate_up=q["ws_gate_up"], ws_down=q["ws_down"], gu_shared=self.gu_shared,
                    h_shared=self._h_shared, real_mask=self.real_mask, real_counts=self.real_counts,
                    perm_token=self.perm_token if (self.mx_gather or not self.plan.mx) else None,
                    mx_saved=self.mx_saved if self.mx_save else None)

    def backward(self, dy, stream=None):
        L.moe_backward(self.plan, self.saved(), dy, self.grads, self.ws, stream)
        return self.grads

    def keep_intermediates(self, keep=True):
        """MX-fp8 experts: let later backwards also store "dgu" and
        "dgu_shared" (by default they exist only as MX operands)."""
        L.keep_intermediates(self.plan, keep)

    def backward_intermediate(self, name):
        """View of an intermediate the last backward left in the workspace
        ("dy_perm", "dgu", "dx_perm", "dgu_shared", "dx_shared"; bf16 and f32
        experts also "wh", the w H rows of the down weight gradient; bf16
        plans with few rows per expert also "dgu_lo", "wh_lo", the rounding
        remainders)."""
        p = self.plan
        A, NI = p.T * p.k, p.Ns * p.Is
        shape = {"dy_perm": (A, p.d), "dgu": (A, 2 * p.I), "dx_perm": (A, p.d),
                 "dgu_shared": (p.T, 2 * NI), "dx_shared": (p.T, p.d), "wh": (A, p.I),
                 "dgu_lo": (A, 2 * p.I), "wh_lo": (A, p.I)}[name]
        off, nb = L.workspace_region(p, name)
        dt = p.dx_rows_dtype if name in ("dx_perm", "dx_shared") else p.dtype
        return self.ws[off:off + nb].view(dt).view(*shape)

    def aux_stats(self, stream=None):
        if self.real_mask is not None:
            L.moe_aux_stats_masked(self.plan, self.probs, self.topk_idx, self.real_mask, self.f, self.p_mean,
                                   self.real_counts, self.aux_out, self.ws, stream)
        else:
            L.moe_aux_stats(self.plan, self.probs, self.counts, self.f, self.p_mean, self.aux_out, self.ws,
                            stream)

    def step(self, dy, stream=None):
        """One full pass: route, permute, experts, combine, backward, aux
        statistics (and the balancing bias update when enabled with gamma > 0).
        With a real-token mask the statistic runs before the backward, whose
        balancing gradient needs the real tokens' counts."""
        self.forward(stream)
        if self.real_mask is not None:
            self.aux_stats(stream)
            self.backward(dy, stream)
        else:
            self.backward(dy, stream)
            self.aux_stats(stream)
        if self.sel_bias is not None and self.balance_gamma > 0.0:
            self.update_balance(self.balance_gamma, stream)
