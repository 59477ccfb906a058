"""Every MX-fp8 operand the expert GEMMs read, bit for bit against the oracle's
MX rule applied to the stored 16-bit values.

KohakUwULLM README, "Key features": the experts' matmuls run on e4m3 values
with one power-of-two (UE8M0) scale per 32 elements.  Each GEMM's operands are
blocked along that GEMM's contraction: the row operands along their rows
(x or x_perm, H, dY_perm, [dG | dU], the shared experts' counterparts, the
weights along d or along I / 2I), the weight gradients' operands along the
tokens of each expert segment, with blocks restarting at the segment start and
the short last block padded with zeros.  Some of these codes come from
quantiser passes, others from the epilogues of the kernels that produce the
tensor (H: gate/up epilogue; dY_perm and dY: combine backward; [dG | dU]:
SwiGLU-backward epilogue).  Here each buffer is read back from the workspace
and compared with ``O.mx_block_scale`` / ``O.e4m3_round`` of the values the
layer stored: scale bytes exactly, payload codes decoded exactly.

Covered: skewed segments (Zipf router bias: one expert far above the mean,
several under 32 tokens), forced-empty experts, shared experts, both the
gather-on-load and the x_perm path, and the full-size MX workload on sampled
rows of every buffer.
"""

import numpy as np
import pytest
import torch

import moe_inputs as MI
import oracle as O
from tests import parity as PT

pytestmark = pytest.mark.gpu

W = MI.Workload


def e4m3_value(code):
    """Value of an OCP e4m3 byte from the format's definition (bias 7, three
    mantissa bits, subnormals m * 2^-9); 0x7F / 0xFF (NaN) must not occur."""
    code = np.asarray(code, dtype=np.int64)
    assert not np.any((code & 0x7F) == 0x7F), "NaN code"
    sign = np.where(code & 0x80, -1.0, 1.0)
    e = (code >> 3) & 15
    m = code & 7
    return sign * np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))


def expect_codes(vals):
    """(scale exponents [R, K/32], e4m3 values [R, K]) of vals [R, K] under the
    oracle's rule, blocks of 32 along K."""
    R, K = vals.shape
    blk = vals.reshape(R, K // 32, 32)
    ex = O.mx_block_scale(np.abs(blk).max(axis=-1))
    q = O.e4m3_round(blk / np.exp2(ex)[..., None]).reshape(R, K)
    return ex, q


def check_codes(name, pay, sc, vals):
    """pay [R, K] uint8, sc [R, K/32] uint8 (numpy), vals [R, K] float64."""
    assert pay.shape == vals.shape and sc.shape == (vals.shape[0], vals.shape[1] // 32), name
    ex, q = expect_codes(vals)
    got_ex = sc.astype(np.int64) - 127
    bad = np.argwhere(got_ex != ex)
    assert bad.size == 0, f"{name}: scale bytes differ at {bad[:4].tolist()} ({got_ex[tuple(bad[0])]} vs {ex[tuple(bad[0])]})"
    got = e4m3_value(pay)
    bad = np.argwhere(got != q)
    assert bad.size == 0, f"{name}: payload differs at {bad[:4].tolist()} ({got[tuple(bad[0])]} vs {q[tuple(bad[0])]})"


SAVED = ("mx_wdt", "mx_wgut", "mx_ht", "mx_swdt", "mx_swgut", "mx_sht")


class Regions:
    """Reads MX buffers (payload, scales) of a layer's workspace, or of its
    saved-codes buffer for the operands the forward saved there."""

    def __init__(self, layer):
        from mixture_experts_ffn_wave_amd._lib import workspace_region, mx_saved_region
        self.layer, self.wr, self.sr = layer, workspace_region, mx_saved_region

    def raw(self, name, rows, K, sel=None):
        saved = self.layer.mx_save and name in SAVED
        ws = self.layer.mx_saved if saved else self.layer.ws
        where = self.sr if saved else self.wr
        off, nb = where(self.layer.plan, name)
        assert nb == rows * K, (name, nb, rows, K)
        pay = ws[off:off + nb].view(rows, K)
        off, nb = where(self.layer.plan, name + ".scales")
        assert nb == rows * (K // 32), (name, nb)
        sc = ws[off:off + nb].view(rows, K // 32)
        if sel is not None:
            s = torch.as_tensor(sel, device=ws.device)
            pay, sc = pay.index_select(0, s), sc.index_select(0, s)
        return pay.cpu().numpy(), sc.cpu().numpy()

    def pad(self, E):
        off, nb = self.wr(self.layer.plan, "mx_pad")
        return self.layer.ws[off:off + nb].view(torch.int32).cpu().numpy().astype(np.int64)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_layer(wl, inp, gather, save=True):
    """``save``: the forward writes the weights' and H's backward codes into
    the saved-codes buffer (else the backward quantises them itself)."""
    from mixture_experts_ffn_wave_amd import MoELayer
    b = inp.get("bias")
    layer = MoELayer(PT.plan_for(wl, b is not None))
    layer.mx_gather = gather
    layer.mx_save = save
    layer.store_h = True                       # the bf16 H its codes are checked against
    layer.write_x_perm = True
    layer.keep_intermediates()                 # the bf16 [dG | dU] the codes are checked against
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    layer.set_params(dev["x"], dev["w_router"], dev["w_gate_up"], dev["w_down"],
                     bias=(dev["bias"].float() if b is not None else None),
                     ws_gate_up=dev.get("ws_gate_up"), ws_down=dev.get("ws_down"))
    layer.forward()
    layer.backward(dev["dy"])
    torch.cuda.synchronize()
    return layer, dev


def token_axis(vals, off, pad, Kpad):
    """The [C][Kpad] operand of a weight gradient: segment g's tokens (rows
    off[g]..off[g+1] of vals [tokens][C]) at K positions pad[g].., zeros up to
    pad[g+1]."""
    C = vals.shape[1]
    out = np.zeros((C, Kpad))
    for g in range(len(off) - 1):
        n = off[g + 1] - off[g]
        out[:, pad[g]:pad[g] + n] = vals[off[g]:off[g + 1]].T
    return out


def check_all(wl, layer, dev, gather, rows=None):
    """Compare every MX buffer; ``rows`` = number of sampled rows per buffer
    (None: all rows)."""
    rg = Regions(layer)
    T, d, E, k, I, A = wl.T, wl.d, wl.E, wl.k, wl.I, wl.T * wl.k
    rng = np.random.default_rng(7)

    def pick(R):
        if rows is None or R <= rows:
            return None
        s = np.sort(rng.choice(R, size=rows, replace=False))
        return s

    def cmp(name, vals_fn, R, K, Kuse=None):
        """Rows (all or sampled) of buffer `name` [R][K], its first Kuse columns."""
        sel = pick(R)
        pay, sc = rg.raw(name, R, K, sel)
        Kuse = K if Kuse is None else Kuse
        check_codes(name, pay[:, :Kuse], sc[:, :Kuse // 32], vals_fn(sel))

    def rows_of(t):
        def fn(sel):
            a = t if sel is None else t.index_select(0, torch.as_tensor(sel, device=t.device))
            return f64(a)
        return fn

    off = layer.offsets.cpu().numpy().astype(np.int64)
    pad = rg.pad(E)
    counts = np.diff(off)
    assert pad[0] == 0 and np.array_equal(np.diff(pad), (counts + 127) // 128 * 128), "padded offsets"
    Apad = int(rg.wr(layer.plan, "mx_dyt")[1] // d)

    def cols(t, sel):
        """t [tokens][C] restricted to the columns `sel` (all when None), float64."""
        return f64(t if sel is None else t.index_select(1, torch.as_tensor(sel, device=t.device)))

    def tok(t):
        return lambda sel: token_axis(cols(t, sel), off, pad, int(pad[E]))

    def tok_single(t, Tpad):
        def fn(sel):
            c = cols(t, sel)
            v = np.zeros((c.shape[1], Tpad))
            v[:, :T] = c.T
            return v
        return fn

    dy_perm = layer.backward_intermediate("dy_perm")
    dgu = layer.backward_intermediate("dgu")
    wgu2 = dev["w_gate_up"].reshape(E * 2 * I, d)
    wd2 = dev["w_down"].reshape(E * d, I)
    # routed experts, row operands
    if gather and not wl.n_shared:
        # gather path: x's T rows, quantised once per token, lead the buffer
        pay, sc = rg.raw("mx_xq", A, d)
        check_codes("mx_xq (x rows)", pay[:T], sc[:T], f64(dev["x"]))
    elif not gather:
        cmp("mx_xq", rows_of(layer.x_perm), A, d)
    cmp("mx_hq", rows_of(layer.h), A, I)
    cmp("mx_dyq", rows_of(dy_perm), A, d)
    cmp("mx_dguq", rows_of(dgu), A, 2 * I)
    cmp("mx_wgu", rows_of(wgu2), E * 2 * I, d)
    cmp("mx_wd", rows_of(wd2), E * d, I)
    cmp("mx_wdt", lambda sel: cols(wd2, sel).T, I, E * d)
    cmp("mx_wgut", lambda sel: cols(wgu2, sel).T, d, E * 2 * I)
    # routed experts, token-axis operands of the weight gradients
    Kr = int(pad[E])                      # past the last padded segment the buffer is not written
    cmp("mx_dyt", tok(dy_perm), d, Apad, Kr)
    cmp("mx_ht", tok(layer.h), I, Apad, Kr)
    cmp("mx_dgut", tok(dgu), 2 * I, Apad, Kr)
    cmp("mx_xt", tok(layer.x_perm), d, Apad, Kr)
    if wl.n_shared:
        Ns, Is = wl.n_shared, wl.I_shared
        NI = Ns * Is
        Tpad = (T + 127) // 128 * 128
        dgs = layer.backward_intermediate("dgu_shared")
        swgu2 = dev["ws_gate_up"].reshape(2 * NI, d)
        swd = torch.cat([dev["ws_down"][s] for s in range(Ns)], dim=1)          # [d][NI]
        cmp("mx_sxq", rows_of(dev["x"]), T, d)
        cmp("mx_shq", rows_of(layer.h_shared), T, NI)
        cmp("mx_sdyq", rows_of(dev["dy"]), T, d)
        cmp("mx_sdguq", rows_of(dgs), T, 2 * NI)
        cmp("mx_swgu", rows_of(swgu2), 2 * NI, d)
        cmp("mx_swd", rows_of(swd), d, NI)
        cmp("mx_swdt", lambda sel: cols(swd, sel).T, NI, d)
        cmp("mx_swgut", lambda sel: cols(swgu2, sel).T, d, 2 * NI)
        cmp("mx_sdyt", tok_single(dev["dy"], Tpad), d, Tpad)
        cmp("mx_sht", tok_single(layer.h_shared, Tpad), NI, Tpad)
        cmp("mx_sdgut", tok_single(dgs, Tpad), 2 * NI, Tpad)
        cmp("mx_sxt", tok_single(dev["x"], Tpad), d, Tpad)
    return counts


CASES = [
    (W("t1536_d256_e32k4_i128_zipf_mx", T=1536, d=256, E=32, k=4, I=128, zipf_s=1.1, expert_dtype="mxfp8"), True),
    (W("t1536_d256_e32k4_i128_zipf_mx", T=1536, d=256, E=32, k=4, I=128, zipf_s=1.1, expert_dtype="mxfp8"), False),
    (W("t2049_d512_e4k2_i512_s1x256_mx", T=2049, d=512, E=4, k=2, I=512, n_shared=1, I_shared=256,
       expert_dtype="mxfp8"), True),
    (W("t900_d256_e16k4_i384_s2x128_mx", T=900, d=256, E=16, k=4, I=384, n_shared=2, I_shared=128,
       expert_dtype="mxfp8"), False),
]


@pytest.mark.parametrize("wl,gather", CASES, ids=[f"{w.name}-{'gather' if g else 'xperm'}" for w, g in CASES])
def test_every_mx_operand_is_bit_exact(wl, gather):
    PT.say(f"[mx-codes] {wl.name} gather={gather}")
    inp = MI.make_inputs(wl)
    layer, dev = run_layer(wl, inp, gather)
    counts = check_all(wl, layer, dev, gather)
    if wl.zipf_s:
        assert counts.max() > 4 * counts.mean() and (counts[counts > 0] < 32).any(), counts


# Without the saved-codes buffer the backward quantises the weights along its
# reduction axes and H along the tokens itself (the transposing quantiser)
@pytest.mark.parametrize("wl,gather", [CASES[1], CASES[3]], ids=["zipf-xperm", "shared2-xperm"])
def test_every_mx_operand_is_bit_exact_without_saved_codes(wl, gather):
    PT.say(f"[mx-codes] {wl.name} gather={gather} no saved codes")
    inp = MI.make_inputs(wl)
    layer, dev = run_layer(wl, inp, gather, save=False)
    check_all(wl, layer, dev, gather)


# The 256 x 256 tiles (8 waves) of the forward GEMMs and the gate/up dgrad:
# H's row-wise codes come from the 256-wide gate/up epilogue
@pytest.mark.parametrize("wl,gather", [CASES[0], CASES[2]], ids=["zipf-gather", "shared1-gather"])
def test_every_mx_operand_is_bit_exact_with_256_tiles(wl, gather, monkeypatch):
    monkeypatch.setenv("MOE_ROW_TILE", "256")
    PT.say(f"[mx-codes] {wl.name} gather={gather} row tiles 256 x 256")
    inp = MI.make_inputs(wl)
    layer, dev = run_layer(wl, inp, gather)
    check_all(wl, layer, dev, gather)


def test_mx_codes_with_empty_experts():
    wl = W("t700_d256_e8k2_i256_s1x128_mx_empty", T=700, d=256, E=8, k=2, I=256, n_shared=1, I_shared=128,
           expert_dtype="mxfp8")
    inp = MI.make_inputs(wl)
    b = torch.zeros(8, dtype=torch.float32)
    b[[0, 5]] = -1e4                      # experts 0 and 5 never chosen
    inp["bias"] = b
    for gather in (True, False):
        layer, dev = run_layer(wl, inp, gather)
        counts = check_all(wl, layer, dev, gather)
        assert counts[0] == 0 and counts[5] == 0


@pytest.mark.timeout(600)
def test_mx_codes_full_size_sampled_rows():
    wl = MI.WORKLOADS["t16384_d2048_e64k6_i1408_s2x1408_mxfp8"]
    PT.say(f"[mx-codes] {wl.name} (48 sampled rows per buffer)")
    inp = MI.make_inputs(wl)
    layer, dev = run_layer(wl, inp, True)
    check_all(wl, layer, dev, True, rows=48)
