"""GPU parity of kdn_scan_bwd (gradients of the delta-write scan) against the
fp64 oracle's adjoint, which the CPU suite pins by finite differences."""
import numpy as np
import pytest

import workloads
from _util import TOL_F32, assert_close, dev_tensor, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kdn():
    import torch
    import delta_rule_scans_amd as k
    assert torch.cuda.is_available()
    return k


def _case(kdn, orc, B, H, L, dk, dv, resid, seed, heads=None, tol=TOL_F32):
    import torch
    inp = workloads.scan_inputs(B, H, L, dk, dv, seed=seed, dtype="f32")
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.1).astype(np.float32)
    d_o = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    dS = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    g = kdn.kdn_scan_bwd(*(dev_tensor(inp[n]) for n in ("q", "k", "v", "alpha", "beta")),
                         dev_tensor(d_o), state_in=dev_tensor(S0), dstate_out=dev_tensor(dS),
                         resid=resid)
    torch.cuda.synchronize()
    got = {n: host(x) for n, x in g.items()}
    sel = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    bs = np.array([s[0] for s in sel])
    hs = np.array([s[1] for s in sel])
    sub = lambda x: np.ascontiguousarray(x[bs, hs][None])  # noqa: E731
    ref = orc.scan_bwd(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), alpha=sub(inp["alpha"]),
                       beta=sub(inp["beta"]), S0=sub(S0), d_o=sub(d_o), dS=sub(dS), resid=resid)
    for n in ("dq", "dk", "dv", "dalpha", "dbeta"):
        assert_close(got[n][bs, hs], ref[n][0], tol, f"{resid} {n}")
    assert_close(got["dstate_in"][bs, hs], ref["dS0"][0], tol, f"{resid} dS0")


@pytest.mark.parametrize("resid", ["gated", "plain", "noerase"])
def test_backward_small(kdn, orc, resid):
    log(f"backward {resid}")
    _case(kdn, orc, 1, 2, 150, 64, 64, resid, seed=401)


def test_backward_odd_shapes(kdn, orc):
    _case(kdn, orc, 2, 1, 70, 40, 24, "gated", seed=402)
    # several value tiles, the last one partial (100 = 3 x 32 + 4), full d_k
    _case(kdn, orc, 1, 1, 200, 128, 100, "plain", seed=405)


def test_backward_full_size(kdn, orc):
    """The gated workload's shape (B=4, H=16, L=4096, d=128) in float32, checked
    on sampled heads."""
    log("backward full size")
    _case(kdn, orc, 4, 16, 4096, 128, 128, "gated", seed=403, heads=[(0, 0), (3, 15)])


def test_backward_defaults(kdn, orc):
    """No decay array (alpha = 1), no initial state and no final-state gradient;
    one token, and one full chunk plus one token, with d_k != d_v."""
    import torch
    for L, dk, dv in ((1, 128, 64), (65, 64, 128)):
        log(f"backward defaults L {L} dk {dk} dv {dv}")
        inp = workloads.scan_inputs(1, 2, L, dk, dv, seed=404, dtype="f32")
        rng = np.random.Generator(np.random.PCG64([404, L]))
        d_o = rng.standard_normal((1, 2, L, dv)).astype(np.float32)
        g = kdn.kdn_scan_bwd(dev_tensor(inp["q"]), dev_tensor(inp["k"]), dev_tensor(inp["v"]), None,
                             dev_tensor(inp["beta"]), dev_tensor(d_o))
        torch.cuda.synchronize()
        assert g["dalpha"] is None
        ref = orc.scan_bwd(inp["q"], inp["k"], inp["v"], alpha=None, beta=inp["beta"], d_o=d_o)
        for n in ("dq", "dk", "dv", "dbeta"):
            assert_close(host(g[n]), ref[n], TOL_F32, f"defaults {n}")
        assert_close(host(g["dstate_in"]), ref["dS0"], TOL_F32, "defaults dS0")
