"""GPU parity of kdn_scan_bwd (gradients of the delta-write scan) against the
fp64 oracle's adjoint, which the CPU suite pins by finite differences."""
import numpy as np
import pytest

import workloads
from _util import TOL_F32, assert_close, dev_tensor, extreme_alpha, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kdn():
    import torch
    import delta_rule_scans_amd as k
    assert torch.cuda.is_available()
    return k


def _case(kdn, orc, B, H, L, dk, dv, resid, seed, heads=None, tol=TOL_F32, alpha=None,
          dlog_alpha=False):
    import torch
    inp = workloads.scan_inputs(B, H, L, dk, dv, seed=seed, dtype="f32")
    if alpha is not None:
        inp["alpha"] = alpha
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
        g_, r_ = got[n][bs, hs], ref[n][0]
        if n == "dalpha" and dlog_alpha:
            # the gradient with respect to log alpha: alpha dL/dalpha
            a_ = inp["alpha"][bs, hs].astype(np.float64)
            g_, r_, n = g_ * a_, r_ * a_, "alpha dalpha"
        assert_close(g_, r_, tol, f"{resid} {n}")
    assert_close(got["dstate_in"][bs, hs], ref["dS0"][0], tol, f"{resid} dS0")


@pytest.mark.parametrize("resid", ["gated", "plain", "noerase"])
def test_backward_small(kdn, orc, resid):
    log(f"backward {resid}")
    _case(kdn, orc, 1, 2, 150, 64, 64, resid, seed=401)


@pytest.mark.parametrize("resid", ["gated", "noerase"])
def test_backward_extreme_decay(kdn, orc, resid):
    """Decays from exactly 1 down to 1e-8 inside 64-token chunks, with abrupt
    switches and a ragged tail (the scan tests' extreme-decay pattern): the
    decay ratios are differences of log-decay prefixes near -1000. The decay's
    gradient is checked as alpha dL/dalpha, the gradient with respect to log
    alpha: at alpha = 1e-8, dL/dalpha is that gradient times 1e8, so its
    float32 rounding, relative to the other tokens' entries, grows by the same
    factor (measured: 12.6 of RMS(dL/dalpha) against 1e-4)."""
    log(f"backward extreme decay {resid}")
    _case(kdn, orc, 1, 2, 357, 64, 64, resid, seed=406, alpha=extreme_alpha(1, 2, 357, 406),
          dlog_alpha=True)


def test_backward_odd_shapes(kdn, orc):
    _case(kdn, orc, 2, 1, 70, 40, 24, "gated", seed=402)
    # several value tiles, the last one partial (100 = 3 x 32 + 4), full d_k
    _case(kdn, orc, 1, 1, 200, 128, 100, "plain", seed=405)


def test_backward_full_size(kdn, orc):
    """The gated workload's shape (B=4, H=16, L=4096, d=128) in float32, checked
    on 16 heads spread over the batch and the heads."""
    log("backward full size")
    heads = [(b, h) for b in range(4) for h in (0, 5, 10, 15)]
    _case(kdn, orc, 4, 16, 4096, 128, 128, "gated", seed=403, heads=heads)


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


def _kalman_case(kdn, orc, B, H, L, dk, dv, mode, dtype, seed, heads=None, qvar=0.7):
    """kdn_scan_bwd_ex for a Kalman write against the oracle's adjoint: every
    gradient (q, k, v, alpha, r, the prior covariance, the initial state) for a
    loss with dL/do, dL/dS_L and dL/dcov_L all given."""
    import torch
    inp = workloads.scan_inputs(B, H, L, dk, dv, seed=seed, dtype=dtype, with_r=True)
    rng = np.random.Generator(np.random.PCG64([seed, 8]))
    inp["k"] = inp["k"] * rng.uniform(0.5, 1.5, (B, H, L, 1)).astype(np.float32)
    d_o = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    if dtype == "bf16":
        inp["k"] = workloads.bf16_round(inp["k"])
        d_o = workloads.bf16_round(d_o)
    cshape = (B, H, dk) if mode == "diag" else (B, H)
    cov0 = rng.uniform(0.5, 2.0, cshape).astype(np.float32)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.1).astype(np.float32)
    dS = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    dcov = rng.standard_normal(cshape).astype(np.float32)
    g = kdn.kdn_scan_bwd_ex(*(dev_tensor(inp[n], dtype) for n in ("q", "k", "v")),
                            dev_tensor(d_o, dtype), alpha=dev_tensor(inp["alpha"]),
                            r=dev_tensor(inp["r"]), cov_in=dev_tensor(cov0), q_noise_var=qvar,
                            state_in=dev_tensor(S0), dstate_out=dev_tensor(dS),
                            dcov_out=dev_tensor(dcov), mode=mode)
    torch.cuda.synchronize()
    got = {n: host(x) for n, x in g.items() if x is not None}
    sel = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    bs = np.array([s[0] for s in sel])
    hs = np.array([s[1] for s in sel])
    sub = lambda x: np.ascontiguousarray(x[bs, hs][None])  # noqa: E731
    ref = orc.scan_bwd_kalman(sub(inp["q"]), sub(inp["k"]), sub(inp["v"]), alpha=sub(inp["alpha"]),
                              r=sub(inp["r"]), cov0=sub(cov0), q_noise_var=qvar, S0=sub(S0),
                              d_o=sub(d_o), dS=sub(dS), dcov=sub(dcov), mode=mode)
    for n in ("dq", "dk", "dv", "dalpha", "dr", "dS0", "dcov0"):
        gn = {"dS0": "dstate_in", "dcov0": "dcov_in"}.get(n, n)
        assert_close(got[gn][bs, hs], ref[n][0], TOL_F32, f"{mode} {dtype} {n}")


@pytest.mark.parametrize("mode", ["diag", "iso"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kalman_backward_small(kdn, orc, mode, dtype):
    log(f"kalman backward {mode} {dtype}")
    _kalman_case(kdn, orc, 1, 2, 150, 64, 64, mode, dtype, seed=406)


def test_kalman_backward_shapes(kdn, orc):
    """d_k = 128 (two coordinates per lane in the covariance adjoint), d_v not
    a multiple of 32, no process noise, a ragged last chunk."""
    _kalman_case(kdn, orc, 2, 1, 77, 128, 40, "diag", "f32", seed=407, qvar=0.0)
    _kalman_case(kdn, orc, 1, 3, 130, 40, 24, "iso", "f32", seed=408)


def test_kalman_backward_many_chunks(kdn, orc):
    """131 adjoint chunks of 64 tokens: the carry of dp over chunks takes them
    64 at a time from the end, the first block ragged."""
    _kalman_case(kdn, orc, 1, 1, 64 * 130 + 17, 64, 32, "diag", "f32", seed=410)
    _kalman_case(kdn, orc, 1, 1, 64 * 130 + 17, 64, 32, "iso", "f32", seed=411)


def test_delta_backward_bf16_inputs(kdn, orc):
    """The delta write's gradients from bf16 inputs through kdn_scan_bwd_ex: the
    oracle on the same bf16 values, float32 bar (the backward runs in float32)."""
    import torch
    B, H, L, d = 1, 2, 150, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=409, dtype="bf16")
    rng = np.random.Generator(np.random.PCG64(409))
    d_o = workloads.bf16_round(rng.standard_normal((B, H, L, d)).astype(np.float32))
    dS = rng.standard_normal((B, H, d, d)).astype(np.float32)
    g = kdn.kdn_scan_bwd_ex(*(dev_tensor(inp[n], "bf16") for n in ("q", "k", "v")),
                            dev_tensor(d_o, "bf16"), alpha=dev_tensor(inp["alpha"]),
                            beta=dev_tensor(inp["beta"]), dstate_out=dev_tensor(dS), mode="delta")
    torch.cuda.synchronize()
    ref = orc.scan_bwd(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], d_o=d_o,
                       dS=dS)
    for n in ("dq", "dk", "dv", "dalpha", "dbeta"):
        assert_close(host(g[n]), ref[n], TOL_F32, f"bf16 delta {n}")
    assert_close(host(g["dstate_in"]), ref["dS0"], TOL_F32, "bf16 delta dS0")


def test_kalman_backward_full_size(kdn, orc):
    """The diagonal Kalman workload's shape (B=4, H=16, L=4096, d=128, bf16
    inputs), checked on 16 heads spread over the batch and the heads."""
    log("kalman backward full size")
    heads = [(b, h) for b in range(4) for h in (0, 5, 10, 15)]
    _kalman_case(kdn, orc, 4, 16, 4096, 128, 128, "diag", "bf16", seed=410, heads=heads, qvar=1.0)
