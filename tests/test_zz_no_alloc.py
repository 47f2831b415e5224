"""kda_chunk_fwd_noalloc (no workspace argument; the library's own per-GPU segment workspace)
against kda_chunk_fwd with a caller-given workspace, through the C ABI.

The two entry points run the same kernels on the same plan, so their outputs must be
bit-identical; both are also held to the float64 oracle's bf16 bar (relative Frobenius
<= 1.5e-2).  Two calls in a row on one GPU, the second smaller, so the second reads a
workspace that still holds the first call's values.
"""
import ctypes
import sys

import numpy as np
import pytest

import kda_synth as ks
import oracle

pytestmark = pytest.mark.gpu

TOL_BF16 = 1.5e-2
WORKSPACE_ERR = 6
NOALLOC_SCRATCH_BYTES = 64 << 20          # KDA_NOALLOC_SCRATCH_BYTES in include/kda.h


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def g():
    import torch
    assert torch.cuda.is_available()
    import gated_delta_rule_107_amd as g
    return g


def _dev(x, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def _inputs(r):
    import torch
    x = ks.make_prefill(r)
    d = {n: _dev(x[n], torch.bfloat16) for n in ("q", "k", "v")}
    d["log_alpha"] = _dev(x["log_alpha"], torch.float32)
    d["beta"] = _dev(x["beta"], torch.float32)
    d["S0"] = None if x["S0"] is None else _dev(x["S0"], torch.float32)
    return x, d


def _noalloc(g, d, r, plan):
    """One kda_chunk_fwd_noalloc call through ctypes; returns (status, o, S_T)."""
    import torch
    o = torch.full((r.B, r.T, r.H, r.dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    S_T = torch.full((r.B, r.H, r.dk, r.dv), float("nan"), dtype=torch.float32, device="cuda")
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = g.lib().kda_chunk_fwd_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["log_alpha"]), p(d["beta"]),
                                       p(d["S0"]), p(o), p(S_T), r.B, r.T, r.H, r.dk, r.dv, r.chunk, 1,
                                       ctypes.byref(plan) if plan is not None else None,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, o, S_T


def _case(g, r, plan, what):
    import torch
    _say(f"case: {what}: B{r.B} T{r.T} H{r.H} {r.dk}/{r.dv} chunk {r.chunk}, plan {plan}")
    x, d = _inputs(r)
    resolved = plan if plan is not None else g.default_plan(r.B, r.T, r.H, r.dk, r.dv, r.chunk)
    nws = g.workspace_bytes(r.B, r.T, r.H, r.dk, r.dv, r.chunk, torch.bfloat16, resolved)
    assert resolved.n_segments > 1 and 0 < nws <= NOALLOC_SCRATCH_BYTES, (resolved, nws)
    st, o, S = _noalloc(g, d, r, plan)
    assert st == 0, g.lib().kda_last_error().decode()
    o_ws, S_ws = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=r.chunk, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(S, S_ws), "noalloc differs from the workspace entry point"
    o_ref, S_ref = oracle.kda_chunked(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["S0"], chunk=r.chunk)
    eo = oracle.rel_fro(o.float().cpu().numpy(), o_ref)
    es = oracle.rel_fro(S.cpu().numpy(), S_ref)
    _say(f"{what}: bit-identical to kda_chunk_fwd; rel_fro vs oracle o={eo:.3e} S_T={es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_noalloc_matches_workspace_entry_point(g):
    # 1) the B=1 T=4096 H=16 prefill in its default plan (16 segments, 48 MiB of workspace)
    _case(g, ks.WORKLOADS[1], None, "first call, default plan")
    # 2) a smaller call right after: 3 segments over a ragged last chunk; the library's
    #    workspace still holds the first call's values
    r2 = ks.Recipe("noalloc2", B=1, T=500, H=2, dk=128, dv=128, chunk=64, dtype="bf16", s0_std=0.1,
                   tag=ks.TAG_BASE + 500)
    _case(g, r2, g.Plan(3, 128), "second call, smaller")


def test_noalloc_rejects_plans_beyond_its_workspace(g):
    """64 heads x 16 segments need 192 MiB of segment workspace: rejected before any launch."""
    import torch
    plan = g.Plan(16, 128)
    nws = g.workspace_bytes(1, 1 << 16, 64, 128, 128, 64, torch.bfloat16, plan)
    assert nws > NOALLOC_SCRATCH_BYTES
    e = torch.empty(1, 1 << 16, 64, 128, dtype=torch.bfloat16, device="cuda")
    ef = torch.empty(1, 1 << 16, 64, 128, dtype=torch.float32, device="cuda")
    beta = torch.empty(1, 1 << 16, 64, dtype=torch.float32, device="cuda")
    o = torch.empty_like(e)
    S_T = torch.empty(1, 64, 128, 128, dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = g.lib().kda_chunk_fwd_noalloc(p(e), p(e), p(e), p(ef), p(beta), None, p(o), p(S_T), 1, 1 << 16, 64,
                                       128, 128, 64, 1, ctypes.byref(plan), None)
    assert st == WORKSPACE_ERR
    assert "workspace" in g.lib().kda_last_error().decode()
