"""The chunkwise-parallel (WY / UT-transform) form of the gated delta write,
restated in numpy and checked against the sequential fp64 oracle.

The pages give only the sequential recurrence ("A Hippocampus for Linear
Attention", sec. 3.3 eq. (5), sec. 3.5) and call the Kalman variants
scan-compatible ("Kalman Delta Networks", abstract). The HIP kernels compute
the same recurrence chunk by chunk; this test pins that derivation. For a chunk
of C tokens with incoming state S0, general write vectors b_t (beta_t k_t for
the delta rule, the Kalman gain otherwise) and chunk-local decay
g_i = prod_{l<=i} alpha_l:
    A  = strict_lower((K B^T) * G),  G_il = g_i / g_l
    T  = (I + A)^-1
    U  = T (V - diag(g) K S0)          (U equals the per-token residuals e_t)
    O  = diag(g) Q S0 + lower_incl((Q B^T) * G) U
    S  = g_C S0 + (diag(g_C / g) B)^T U
"""
import numpy as np
import pytest

import workloads


def chunked_scan(q, k, v, alpha, bvec, S0, C):
    L, dk = k.shape
    S = S0.copy()
    O = np.zeros((L, v.shape[1]))
    U_all = np.zeros_like(O)
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        K, Q, V, Bm = k[sl], q[sl], v[sl], bvec[sl]
        n = K.shape[0]
        lg = np.cumsum(np.log(alpha[sl]))
        G = np.exp(lg[:, None] - lg[None, :])
        g = np.exp(lg)
        A = np.tril((K @ Bm.T) * G, -1)
        T = np.linalg.inv(np.eye(n) + A)
        U = T @ (V - g[:, None] * (K @ S))
        O[sl] = g[:, None] * (Q @ S) + np.tril((Q @ Bm.T) * G) @ U
        S = g[-1] * S + (Bm * (g[-1] / g)[:, None]).T @ U
        U_all[sl] = U
    return O, S, U_all


@pytest.mark.parametrize("C", [1, 7, 16, 64])
def test_chunk_form_matches_sequential_delta(orc, C):
    inp = workloads.scan_inputs(1, 2, 200, 16, 12, seed=31, dtype="f32")
    S0 = np.random.Generator(np.random.PCG64(31)).standard_normal((1, 2, 16, 12))
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], S0=S0)
    for h in range(2):
        k = inp["k"][0, h].astype(np.float64)
        b = inp["beta"][0, h].astype(np.float64)[:, None] * k
        O, S, U = chunked_scan(inp["q"][0, h].astype(np.float64), k, inp["v"][0, h].astype(np.float64),
                               inp["alpha"][0, h].astype(np.float64), b, S0[0, h], C)
        np.testing.assert_allclose(O, ref["o"][0, h], atol=1e-12 * np.abs(ref["o"]).max())
        np.testing.assert_allclose(S, ref["S"][0, h], atol=1e-12 * np.abs(ref["S"]).max())
        # the WY residuals are the per-token residuals: beta ||u_t|| is the write score
        np.testing.assert_allclose(inp["beta"][0, h] * np.linalg.norm(U, axis=1), ref["m"][0, h],
                                   rtol=1e-10)


@pytest.mark.parametrize("C", [16, 64])
def test_chunk_form_matches_sequential_kalman_gain(orc, C):
    """Same chunk form with the Kalman gains as write vectors: the gains do not
    depend on S, so they can be computed first and fed to the chunked scan."""
    inp = workloads.scan_inputs(1, 1, 150, 8, 6, seed=32, dtype="f32", with_r=True)
    p0 = np.ones((1, 1, 8))
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=1.0, mode="diag")
    # gains from the covariance recursion alone (the oracle's one-token steps give them)
    k = inp["k"][0, 0].astype(np.float64)
    a = inp["alpha"][0, 0].astype(np.float64)
    r = inp["r"][0, 0].astype(np.float64)
    p = p0[0, 0].copy()
    gains = np.zeros_like(k)
    for t in range(k.shape[0]):
        pm = a[t] ** 2 * p + (1 - a[t] ** 2)
        gains[t] = pm * k[t] / (np.sum(pm * k[t] ** 2) + r[t])
        p = pm * r[t] / (r[t] + pm * k[t] ** 2)
    O, S, _ = chunked_scan(inp["q"][0, 0].astype(np.float64), k, inp["v"][0, 0].astype(np.float64),
                           a, gains, np.zeros((8, 6)), C)
    np.testing.assert_allclose(O, ref["o"][0, 0], atol=1e-12 * np.abs(ref["o"]).max())
    np.testing.assert_allclose(S, ref["S"][0, 0], atol=1e-12 * np.abs(ref["S"]).max())
