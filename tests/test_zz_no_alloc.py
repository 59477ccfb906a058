"""moe_permute_noalloc (the permute without a workspace, its scratch in the
library's fixed device array) against moe_permute (the caller's workspace):
counts, offsets, perm_token, inv_perm and x_perm bit for bit, on two calls in
a row, the second with fewer tokens, so the second call reads the array the
first one left behind.  (Its refusal of a plan beyond the array is a host
test in test_abi_host.py.)"""

import numpy as np
import pytest
import torch

from mixture_experts_ffn_wave_amd import _lib as L

pytestmark = pytest.mark.gpu


def routing(T, E, k, seed):
    """Valid top-k indices: k distinct experts per token, skewed popularity."""
    rng = np.random.default_rng(seed)
    pop = np.exp(rng.standard_normal(E) * 1.5)
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        idx[t] = rng.choice(E, size=k, replace=False, p=pop / pop.sum())
    return torch.from_numpy(idx).cuda()


def run_both(T, d, E, k, seed):
    plan = L.Plan(T, d, E, k, 128, dtype=torch.bfloat16)
    idx = routing(T, E, k, seed)
    x = torch.randn(T, d, device="cuda").to(torch.bfloat16)
    ws = torch.empty(max(plan.workspace_bytes(), 256), dtype=torch.uint8, device="cuda")
    outs = []
    for noalloc in (False, True):
        # outputs start from different garbage each time
        fill = 0x5A if noalloc else 0x00
        counts = torch.full((E,), fill, dtype=torch.int32, device="cuda")
        offsets = torch.full((E + 1,), fill, dtype=torch.int32, device="cuda")
        perm = torch.full((T * k,), fill, dtype=torch.int32, device="cuda")
        inv = torch.full((T, k), fill, dtype=torch.int32, device="cuda")
        xp = torch.full((T * k, d), float(fill), dtype=torch.bfloat16, device="cuda")
        if noalloc:
            L.moe_permute_noalloc(plan, idx, x, counts, offsets, perm, inv, xp)
        else:
            L.moe_permute(plan, idx, x, counts, offsets, perm, inv, xp, ws)
        torch.cuda.synchronize()
        outs.append([counts.cpu(), offsets.cpu(), perm.cpu(), inv.cpu(), xp.cpu()])
    return outs, idx.cpu().numpy()


def test_permute_noalloc_equals_permute_on_two_calls():
    # first call: 5000 tokens, 64 experts (20 token blocks); second: fewer
    # tokens and experts, so it reads only part of what the first call left
    for T, d, E, k, seed in [(5000, 256, 64, 6, 1), (777, 128, 16, 2, 2)]:
        (ref, got), idx = run_both(T, d, E, k, seed)
        for name, a, b in zip(["counts", "offsets", "perm_token", "inv_perm", "x_perm"], ref, got):
            assert torch.equal(a, b), f"T={T}: {name} differs"
        counts = np.bincount(idx.reshape(-1), minlength=E)
        assert np.array_equal(ref[0].numpy(), counts)
