"""kdn_scan_fwd_static, the allocation-free scan entry (the library's own
static scratch instead of a caller workspace), called through the C ABI: its
outputs equal those of kdn_scan_fwd with a workspace, bit for bit, and meet the
oracle's bar, on consecutive calls whose second input is smaller (the scratch
keeps the first call's contents), for the delta write with scores and the
diagonal Kalman write."""
import ctypes

import numpy as np
import pytest

import workloads
from _util import TOL_BF16, TOL_F32, assert_close, dev_tensor, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kdn():
    import torch
    import delta_rule_scans_amd as k
    assert torch.cuda.is_available()
    return k


def _static_call(kdn, t, o, m, S, cov_out, cov_in, mode, qvar, dims, chunk=64):
    import torch
    B, H, L, dk, dv = dims
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())  # noqa: E731
    st = kdn.lib.kdn_scan_fwd_static(
        p(t["q"]), p(t["k"]), p(t["v"]), kdn.BF16, p(t["alpha"]), p(t["beta"]), p(t.get("r")),
        p(cov_in), p(cov_out), ctypes.c_float(qvar), None, p(S), p(o), kdn.F32, p(m), 0,
        B, H, L, dk, dv, chunk, kdn.MODES[mode], 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, kdn.kdn_status_string(st)


@pytest.mark.parametrize("mode", ["delta", "diag"])
def test_static_scratch_matches_workspace_entry(kdn, orc, mode):
    import torch
    diag = mode == "diag"
    qvar = 1.0 if diag else 0.0
    for i, (B, H, L) in enumerate(((2, 4, 1000), (1, 3, 300))):
        d = 128
        log(f"static scratch {mode}: call {i}, B={B} H={H} L={L}")
        inp = workloads.scan_inputs(B, H, L, d, d, seed=130 + i, dtype="bf16", with_r=diag)
        t = {n: dev_tensor(inp[n], "bf16") for n in ("q", "k", "v")}
        t["alpha"], t["beta"] = dev_tensor(inp["alpha"]), dev_tensor(inp["beta"])
        if diag:
            t["r"] = dev_tensor(inp["r"])
        cov0 = torch.ones((B, H, d), device="cuda") if diag else None
        need = kdn.kdn_scan_workspace_size(B, H, L, d, d, 64, mode, kdn.BF16, with_scores=not diag)
        assert 0 < need <= kdn.STATIC_SCRATCH_BYTES
        # the ordinary entry with a caller workspace
        o1 = torch.empty((B, H, L, d), device="cuda")
        S1 = torch.empty((B, H, d, d), device="cuda")
        c1 = torch.empty_like(cov0) if diag else None
        m1 = None if diag else torch.empty((B, H, L), device="cuda")
        res = kdn.kdn_scan_fwd(t["q"], t["k"], t["v"], alpha=t["alpha"], beta=t["beta"],
                               r=t.get("r"), cov_in=cov0, cov_out=c1, q_noise_var=qvar,
                               state_out=S1, o=o1, mode=mode, m=m1)
        # the static entry
        o2 = torch.full_like(o1, float("nan"))
        S2 = torch.full_like(S1, float("nan"))
        c2 = torch.full_like(cov0, float("nan")) if diag else None
        m2 = None if diag else torch.full_like(m1, float("nan"))
        _static_call(kdn, t, o2, m2, S2, c2, cov0, mode, qvar, (B, H, L, d, d))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), "o differs from the workspace entry"
        assert torch.equal(S1, S2), "state differs from the workspace entry"
        if diag:
            assert torch.equal(c1, c2), "covariance differs from the workspace entry"
        else:
            assert torch.equal(m1, m2), "scores differ from the workspace entry"
        ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"],
                       r=inp["r"], cov0=np.ones((B, H, d), np.float32) if diag else None,
                       q_noise_var=qvar, mode=mode)
        assert_close(host(o2), ref["o"], TOL_BF16, f"static {mode} o call {i}")
        assert_close(host(S2), ref["S"], TOL_BF16, f"static {mode} S call {i}")
        if diag:
            assert_close(host(c2), ref["cov"], TOL_F32, f"static {mode} p call {i}")
        else:
            assert_close(host(m2), ref["m"], TOL_BF16, f"static {mode} m call {i}")
        del res


def test_static_scratch_limit_is_an_error(kdn):
    """A call that needs more than the static scratch is rejected with
    KDN_ERR_SCRATCH_LIMIT before anything runs (outputs untouched)."""
    import torch
    B, H, L, d = 4, 16, 4096, 128
    q = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    a = torch.ones((B, H, L), device="cuda")
    o = torch.full((B, H, L, d), 7.0, device="cuda")
    cov = torch.ones((B, H, d), device="cuda")
    with pytest.raises(kdn.KdnError) as ei:
        kdn.kdn_scan_fwd_static(q, q, q, o, alpha=a, r=a, cov_in=cov, mode="diag")
    assert ei.value.status == -10
    torch.cuda.synchronize()
    assert bool(torch.all(o == 7.0))
