"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test names the passage that fixes the fact (page title, section/equation).
None of them re-types the oracle's per-token recursion: they use closed forms
(ridge / weighted ridge / batch Gaussian conditioning), special cases with
exact answers (orthonormal keys, no-op writes, k = 0, one-hot keys), library
routines (numpy.linalg, torch's scaled-dot-product attention and rms_norm),
brute-force sorting, and numbers printed on the pages.
"""
import math
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(x):
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


# ---------------------------------------------------------------------------
# Full-covariance (RLS / Kalman) write
# ---------------------------------------------------------------------------

def test_rls_equals_ridge_every_prefix(orc):
    """DeltaNet-PC, eqs. (6)-(7) and the ridge energy before them: with S_0 = 0,
    P_0 = eps^-1 I, unit noise and no decay, the recursive update reproduces the
    ridge-regression minimiser over every prefix:
    S_t = (K_t^T K_t + eps I)^-1 K_t^T V_t, and P_t = (K_t^T K_t + eps I)^-1."""
    inp = workloads.named_scan_inputs("tiny")
    eps = 1e-2
    q, k, v = inp["q"], inp["k"], inp["v"]
    L, dk = q.shape[2], q.shape[3]
    cov0 = np.eye(dk)[None, None] / eps
    res = orc.scan(q, k, v, cov0=cov0, mode="full")
    K = k[0, 0].astype(np.float64)
    V = v[0, 0].astype(np.float64)
    Q = q[0, 0].astype(np.float64)
    worst = 0.0
    for t in range(1, L + 1):
        St = np.linalg.solve(K[:t].T @ K[:t] + eps * np.eye(dk), K[:t].T @ V[:t])
        ot = St.T @ Q[t - 1]
        worst = max(worst, np.max(np.abs(res["o"][0, 0, t - 1] - ot)) / np.max(np.abs(ot)))
    assert worst < 1e-11
    SL = np.linalg.solve(K.T @ K + eps * np.eye(dk), K.T @ V)
    np.testing.assert_allclose(res["S"][0, 0], SL, rtol=0, atol=1e-11 * np.abs(SL).max())
    PL = np.linalg.inv(K.T @ K + eps * np.eye(dk))
    np.testing.assert_allclose(res["cov"][0, 0], PL, rtol=0, atol=1e-11 * np.abs(PL).max())
    # a shorter prefix, checked on the whole state
    t = 23
    res_t = orc.scan(q[:, :, :t], k[:, :, :t], v[:, :, :t], cov0=cov0, mode="full")
    St = np.linalg.solve(K[:t].T @ K[:t] + eps * np.eye(dk), K[:t].T @ V[:t])
    np.testing.assert_allclose(res_t["S"][0, 0], St, rtol=0, atol=1e-11 * np.abs(St).max())


def test_kalman_decay_noise_weighted_ridge(orc):
    """Kalman Delta Networks, abstract (memory as a linear-Gaussian state-space
    model whose transition propagates the state and its uncertainty): with
    decay alpha, per-token noise r and no process noise, the filtered mean is a
    weighted ridge solution. With G_t = prod_{l<=t} alpha_l and c_j = G_j / G_t:
    P_t^-1 = P_0^-1 / G_t^2 + sum_j c_j^2 k_j k_j^T / r_j,
    S_t = P_t (G_t^-1 P_0^-1 S_0 + sum_j c_j k_j v_j^T / r_j)."""
    rng = _rng(11)
    B, H, L, dk, dv = 1, 2, 40, 6, 5
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    k = _unit(rng.standard_normal((B, H, L, dk)))
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    a = rng.uniform(0.8, 1.0, (B, H, L)).astype(np.float32)
    r = rng.uniform(0.2, 2.0, (B, H, L)).astype(np.float32)
    A0 = rng.standard_normal((B, H, dk, dk))
    P0 = np.einsum("bhij,bhkj->bhik", A0, A0) + 0.5 * np.eye(dk)
    S0 = rng.standard_normal((B, H, dk, dv))
    res = orc.scan(q, k, v, alpha=a, r=r, cov0=P0, q_noise_var=0.0, S0=S0, mode="full")
    for h in range(H):
        K, V, Qm = (x[0, h].astype(np.float64) for x in (k, v, q))
        al, rr = a[0, h].astype(np.float64), r[0, h].astype(np.float64)
        P0i = np.linalg.inv(P0[0, h])
        for t in (1, 7, L):
            G = np.cumprod(al[:t])
            Gt = G[-1]
            c = G / Gt
            prec = P0i / Gt ** 2 + np.einsum("j,ji,jk->ik", c ** 2 / rr[:t], K[:t], K[:t])
            rhs = P0i @ S0[0, h] / Gt + np.einsum("j,ji,jk->ik", c / rr[:t], K[:t], V[:t])
            St = np.linalg.solve(prec, rhs)
            if t == L:
                np.testing.assert_allclose(res["S"][0, h], St, atol=1e-10 * np.abs(St).max())
                np.testing.assert_allclose(res["cov"][0, h], np.linalg.inv(prec),
                                           atol=1e-10 * np.abs(np.linalg.inv(prec)).max())
            np.testing.assert_allclose(res["o"][0, h, t - 1], St.T @ Qm[t - 1],
                                       atol=1e-10 * np.abs(St).max())


def _batch_gaussian_filter(K, V, alpha, r, P0, S0, qvar):
    """Exact filtering posterior of the linear-Gaussian memory model by batch
    Gaussian conditioning (no recursion): latent z = [S_0, w_1..w_L] with prior
    N([S0,0..], blockdiag(P0, Q_1 I, .., Q_L I)); S_t = M_t z; v_t = S_t^T k_t + n_t.
    Returns the posterior mean and covariance of S_L given v_1..v_L."""
    L, dk = K.shape
    Qs = (1.0 - alpha ** 2) * qvar
    n = dk * (L + 1)
    prior_cov = np.zeros((n, n))
    prior_cov[:dk, :dk] = P0
    for t in range(L):
        prior_cov[dk * (t + 1):dk * (t + 2), dk * (t + 1):dk * (t + 2)] = Qs[t] * np.eye(dk)
    prior_mean = np.zeros((n, S0.shape[1]))
    prior_mean[:dk] = S0
    Ms = []
    M = np.zeros((dk, n))
    M[:, :dk] = np.eye(dk)
    for t in range(L):
        M = alpha[t] * M
        M[:, dk * (t + 1):dk * (t + 2)] += np.eye(dk)
        Ms.append(M.copy())
    Hm = np.stack([K[t] @ Ms[t] for t in range(L)])          # [L, n]
    Sy = Hm @ prior_cov @ Hm.T + np.diag(r)
    gain = prior_cov @ Hm.T @ np.linalg.inv(Sy)
    post_mean = prior_mean + gain @ (V - Hm @ prior_mean)
    post_cov = prior_cov - gain @ Hm @ prior_cov
    ML = Ms[-1]
    return ML @ post_mean, ML @ post_cov @ ML.T


def test_kalman_with_process_noise_batch_conditioning(orc):
    """Kalman Delta Networks, abstract: the Kalman filter is the optimal
    recursive estimator of the linear-Gaussian memory. Its output must equal the
    filtering posterior computed in one shot by Gaussian conditioning, here with
    decay, per-token noise and stationary process noise Q_t = (1 - alpha_t^2) sigma^2."""
    rng = _rng(12)
    L, dk, dv = 12, 4, 3
    q = rng.standard_normal((1, 1, L, dk)).astype(np.float32)
    k = _unit(rng.standard_normal((1, 1, L, dk)))
    v = rng.standard_normal((1, 1, L, dv)).astype(np.float32)
    a = rng.uniform(0.6, 1.0, (1, 1, L)).astype(np.float32)
    r = rng.uniform(0.3, 1.5, (1, 1, L)).astype(np.float32)
    A0 = rng.standard_normal((dk, dk))
    P0 = A0 @ A0.T + 0.3 * np.eye(dk)
    S0 = rng.standard_normal((dk, dv))
    sig2 = 0.7
    res = orc.scan(q, k, v, alpha=a, r=r, cov0=P0[None, None], q_noise_var=sig2,
                   S0=S0[None, None], mode="full")
    for t in (1, 5, L):
        mean, cov = _batch_gaussian_filter(k[0, 0, :t].astype(np.float64),
                                           v[0, 0, :t].astype(np.float64),
                                           a[0, 0, :t].astype(np.float64),
                                           r[0, 0, :t].astype(np.float64), P0, S0, sig2)
        o_t = mean.T @ q[0, 0, t - 1].astype(np.float64)
        np.testing.assert_allclose(res["o"][0, 0, t - 1], o_t, atol=1e-10)
    np.testing.assert_allclose(res["S"][0, 0], mean, atol=1e-10)
    np.testing.assert_allclose(res["cov"][0, 0], cov, atol=1e-10)


def test_full_covariance_is_symmetrised(orc):
    """The full covariance is a covariance matrix (Kalman Delta Networks,
    abstract): symmetric. A prior with a last-bit asymmetry comes out exactly
    symmetric, and close to the run from the symmetrised prior."""
    rng = _rng(23)
    dk, L = 6, 12
    inp = workloads.scan_inputs(1, 1, L, dk, 3, seed=23, dtype="f32", with_r=True)
    A = rng.standard_normal((dk, dk))
    P0 = A @ A.T / dk + np.eye(dk)
    P0a = P0.copy()
    P0a[0, 1] = np.nextafter(P0a[0, 1], np.inf)
    out = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"],
                   cov0=P0a[None, None], q_noise_var=0.3, mode="full")
    P = out["cov"][0, 0]
    np.testing.assert_array_equal(P, P.T)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"],
                   cov0=P0[None, None], q_noise_var=0.3, mode="full")
    np.testing.assert_allclose(P, ref["cov"][0, 0], rtol=1e-12, atol=1e-14)


def test_rls_capacity_recall(orc):
    """DeltaNet-PC, summary (empirical results): sequences are recalled with
    perfect accuracy when L <= D. For generic keys with L <= d_k and a vanishing
    ridge term the recursive-least-squares memory interpolates every pair."""
    rng = _rng(13)
    L, dk, dv = 12, 16, 8
    k = _unit(rng.standard_normal((1, 1, L, dk)))
    v = rng.standard_normal((1, 1, L, dv)).astype(np.float32)
    q = k.copy()
    for eps in (1e-4, 1e-6):
        res = orc.scan(q, k, v, cov0=np.eye(dk)[None, None] / eps, mode="full")
        recall = np.einsum("ij,tj->ti", res["S"][0, 0].T, k[0, 0].astype(np.float64))
        err = np.max(np.abs(recall - v[0, 0]))
        assert err < 200 * eps


# ---------------------------------------------------------------------------
# Diagonal-covariance (mean-field) write
# ---------------------------------------------------------------------------

def test_diag_one_step_is_meanfield_projection_of_exact_posterior(orc):
    """Kalman Delta Networks, abstract: diagonal KDN projects each one-step
    posterior onto the diagonal Gaussian family by mean-field inference. From a
    diagonal prior, one exact step (FULL branch, pinned above) gives a dense
    posterior; the mean-field (KL(q||p)) projection keeps its mean and the
    diagonal of its precision matrix. The DIAG branch must agree with that for
    general keys, decays, noises and process noise."""
    rng = _rng(14)
    B, H, dk, dv = 2, 3, 8, 5
    for trial in range(3):
        q = rng.standard_normal((B, H, 1, dk)).astype(np.float32)
        k = _unit(rng.standard_normal((B, H, 1, dk)))
        v = rng.standard_normal((B, H, 1, dv)).astype(np.float32)
        a = rng.uniform(0.5, 1.0, (B, H, 1)).astype(np.float32)
        r = rng.uniform(0.1, 2.0, (B, H, 1)).astype(np.float32)
        p0 = rng.uniform(0.2, 3.0, (B, H, dk))
        S0 = rng.standard_normal((B, H, dk, dv))
        sig2 = [0.0, 1.0, 0.3][trial]
        full = orc.scan(q, k, v, alpha=a, r=r, cov0=np.einsum("bhi,ij->bhij", p0, np.eye(dk)),
                        q_noise_var=sig2, S0=S0, mode="full")
        diag = orc.scan(q, k, v, alpha=a, r=r, cov0=p0, q_noise_var=sig2, S0=S0, mode="diag")
        np.testing.assert_allclose(diag["S"], full["S"], atol=1e-12)
        np.testing.assert_allclose(diag["o"], full["o"], atol=1e-12)
        prec_diag = np.einsum("bhii->bhi", np.linalg.inv(full["cov"]))
        np.testing.assert_allclose(1.0 / diag["cov"], prec_diag, rtol=1e-11)


def test_diag_precision_affine_without_process_noise(orc):
    """Kalman Delta Networks, abstract (diagonal projection; Moebius uncertainty
    maps): with no process noise the diagonal precision is affine in time,
    1/p_t = (1/p_0)/G_t^2 + sum_j (G_j/G_t)^2 k_j^2 / r_j."""
    inp = workloads.scan_inputs(2, 2, 50, 8, 4, seed=15, dtype="f32", with_r=True)
    p0 = _rng(15).uniform(0.5, 2.0, (2, 2, 8))
    res = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=0.0, mode="diag")
    a = inp["alpha"].astype(np.float64)
    G = np.cumprod(a, axis=-1)
    Gt = G[..., -1:]
    c2 = (G / Gt) ** 2 / inp["r"].astype(np.float64)
    prec = (1.0 / p0) / Gt ** 2 + np.einsum("bht,bhti->bhi", c2, inp["k"].astype(np.float64) ** 2)
    np.testing.assert_allclose(1.0 / res["cov"], prec, rtol=1e-11)


def test_diag_zero_keys_and_fixed_point(orc):
    """Kalman Delta Networks, abstract (uncertainty recurrences are Moebius maps).
    k = 0: nothing is observed, so p_t = sigma^2 + G_t^2 (p_0 - sigma^2) and the
    state only decays, S_t = G_t S_0. Constant (alpha, k_i, r): p converges to the
    positive root of k^2 a^2 p^2 + (r (1 - a^2) + k^2 Q) p - r Q = 0."""
    rng = _rng(16)
    L, dk, dv, sig2 = 30, 4, 3, 0.8
    a = rng.uniform(0.7, 1.0, (1, 1, L)).astype(np.float32)
    z = np.zeros((1, 1, L, dk), np.float32)
    v = rng.standard_normal((1, 1, L, dv)).astype(np.float32)
    S0 = rng.standard_normal((1, 1, dk, dv))
    p0 = np.array([[[0.1, 1.0, 2.0, 5.0]]])
    res = orc.scan(z, z, v, alpha=a, r=np.ones((1, 1, L), np.float32), cov0=p0,
                   q_noise_var=sig2, S0=S0, mode="diag")
    G = np.prod(a.astype(np.float64))
    np.testing.assert_allclose(res["cov"][0, 0], sig2 + G ** 2 * (p0[0, 0] - sig2), rtol=1e-12)
    np.testing.assert_allclose(res["S"][0, 0], G * S0[0, 0], rtol=1e-12)

    L = 4000
    al, rr = np.float32(0.9), np.float32(0.5)
    kk = np.full((1, 1, L, dk), np.float32(0.5))
    res = orc.scan(kk, kk, np.zeros((1, 1, L, 1), np.float32), alpha=np.full((1, 1, L), al),
                   r=np.full((1, 1, L), rr), cov0=np.ones((1, 1, dk)), q_noise_var=sig2,
                   mode="diag")
    a2, k2, Q, r = float(al) ** 2, 0.25, (1 - float(al) ** 2) * sig2, float(rr)
    root = max(np.roots([k2 * a2, r * (1 - a2) + k2 * Q, -r * Q]).real)
    np.testing.assert_allclose(res["cov"][0, 0], root, rtol=1e-12)


def test_diag_equals_full_for_one_hot_keys(orc):
    """Kalman Delta Networks, abstract: the diagonal family is closed under
    updates with (scaled) one-hot keys, so there the projection is exact and the
    diagonal write must equal the full-covariance write over a whole sequence."""
    rng = _rng(17)
    B, H, L, dk, dv = 1, 2, 60, 6, 4
    idx = rng.integers(0, dk, (B, H, L))
    k = (np.eye(dk)[idx] * rng.uniform(0.5, 1.5, (B, H, L, 1))).astype(np.float32)
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    a = rng.uniform(0.8, 1.0, (B, H, L)).astype(np.float32)
    r = rng.uniform(0.2, 1.0, (B, H, L)).astype(np.float32)
    p0 = rng.uniform(0.5, 2.0, (B, H, dk))
    for sig2 in (0.0, 1.0):
        diag = orc.scan(q, k, v, alpha=a, r=r, cov0=p0, q_noise_var=sig2, mode="diag")
        full = orc.scan(q, k, v, alpha=a, r=r, cov0=np.einsum("bhi,ij->bhij", p0, np.eye(dk)),
                        q_noise_var=sig2, mode="full")
        np.testing.assert_allclose(diag["o"], full["o"], atol=1e-12)
        np.testing.assert_allclose(diag["cov"], np.einsum("bhii->bhi", full["cov"]), rtol=1e-12)


def test_delta_is_covariance_reset_kalman(orc):
    """Kalman Delta Networks, abstract, and Memory by Design, abstract: the
    delta rule is the Kalman write with a token-wise isotropic covariance
    surrogate and no covariance tracking (a covariance reset). Resetting the
    predicted covariance to c I before every token and choosing
    r_t = c (1/beta_t - ||k_t||^2) gives gain beta_t k_t, i.e. the delta rule."""
    rng = _rng(18)
    B, H, L, dk, dv = 1, 2, 25, 16, 8
    # keys with entries +-1/4 are exactly unit-norm in binary floating point
    k = (rng.choice([-0.25, 0.25], (B, H, L, dk))).astype(np.float32)
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, (B, H, L)).astype(np.float32)
    for gated in (False, True):
        a = (rng.uniform(0.7, 1.0, (B, H, L)) if gated else np.ones((B, H, L))).astype(np.float32)
        ref = orc.scan(q, k, v, alpha=a, beta=beta, mode="delta")
        c = 2.0
        S = np.zeros((B, H, dk, dv))
        outs, ms = [], []
        for t in range(L):
            r_t = (c * (1.0 / beta[..., t].astype(np.float64) - 1.0))
            # prior before the predict step is c / alpha^2 so that P- = c I (no process noise)
            p_in = np.repeat((c / a[..., t].astype(np.float64) ** 2)[..., None], dk, axis=-1)
            res = orc.scan(q[:, :, t:t + 1], k[:, :, t:t + 1], v[:, :, t:t + 1],
                           alpha=a[..., t:t + 1], r=r_t[..., None].astype(np.float32),
                           cov0=p_in, q_noise_var=0.0, S0=S, mode="diag")
            S = res["S"]
            outs.append(res["o"][:, :, 0])
            ms.append(res["m"][:, :, 0])
        # r is float32 in the interface: rounding it changes the gain at ~1e-7
        np.testing.assert_allclose(np.stack(outs, 2), ref["o"], atol=2e-6 * np.abs(ref["o"]).max())
        np.testing.assert_allclose(S, ref["S"], atol=2e-6 * np.abs(ref["S"]).max())
        np.testing.assert_allclose(np.stack(ms, 2), ref["m"], rtol=2e-6)


# ---------------------------------------------------------------------------
# Isotropic-covariance write (one variance per head)
# ---------------------------------------------------------------------------

def test_iso_one_step_is_isotropic_projection_of_exact_posterior(orc):
    """Kalman Delta Networks, abstract (the isotropic variant keeps a single
    uncertainty scalar per head): from the prior p I one exact step (FULL
    branch, pinned above) gives the posterior mean and a dense posterior
    precision (1/p-) I + k k^T / r. The KL(q||p) projection onto covariances
    c I keeps the mean and sets 1/c to the average diagonal entry of that
    precision, trace / d_k. The ISO branch must agree for general keys (not
    unit-norm), decays, noises and process noise."""
    rng = _rng(31)
    B, H, dk, dv = 2, 3, 8, 5
    for trial in range(3):
        q = rng.standard_normal((B, H, 1, dk)).astype(np.float32)
        k = rng.standard_normal((B, H, 1, dk)).astype(np.float32)
        v = rng.standard_normal((B, H, 1, dv)).astype(np.float32)
        a = rng.uniform(0.5, 1.0, (B, H, 1)).astype(np.float32)
        r = rng.uniform(0.1, 2.0, (B, H, 1)).astype(np.float32)
        p0 = rng.uniform(0.2, 3.0, (B, H))
        S0 = rng.standard_normal((B, H, dk, dv))
        sig2 = [0.0, 1.0, 0.3][trial]
        full = orc.scan(q, k, v, alpha=a, r=r, cov0=p0[..., None, None] * np.eye(dk),
                        q_noise_var=sig2, S0=S0, mode="full")
        iso = orc.scan(q, k, v, alpha=a, r=r, cov0=p0, q_noise_var=sig2, S0=S0, mode="iso")
        np.testing.assert_allclose(iso["S"], full["S"], atol=1e-12)
        np.testing.assert_allclose(iso["o"], full["o"], atol=1e-12)
        np.testing.assert_allclose(iso["m"], full["m"], rtol=1e-12)
        prec_mean = np.einsum("bhii->bh", np.linalg.inv(full["cov"])) / dk
        np.testing.assert_allclose(1.0 / iso["cov"], prec_mean, rtol=1e-11)


def test_iso_precision_affine_without_process_noise(orc):
    """Kalman Delta Networks, abstract (Moebius uncertainty maps): with no
    process noise the isotropic precision is affine in time,
    1/p_t = (1/p_0)/G_t^2 + sum_j (G_j/G_t)^2 ||k_j||^2 / (d_k r_j)."""
    inp = workloads.scan_inputs(2, 2, 50, 8, 4, seed=32, dtype="f32", with_r=True)
    k = inp["k"] * _rng(32).uniform(0.5, 2.0, (2, 2, 50, 1)).astype(np.float32)
    p0 = _rng(33).uniform(0.5, 2.0, (2, 2))
    res = orc.scan(inp["q"], k, inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=0.0, mode="iso")
    G = np.cumprod(inp["alpha"].astype(np.float64), axis=-1)
    Gt = G[..., -1]
    kk = np.sum(k.astype(np.float64) ** 2, axis=-1)
    prec = (1.0 / p0) / Gt ** 2 + np.sum((G / Gt[..., None]) ** 2 * kk / (8 * inp["r"]), axis=-1)
    np.testing.assert_allclose(1.0 / res["cov"], prec, rtol=1e-11)


def test_iso_zero_keys_and_fixed_point(orc):
    """Kalman Delta Networks, abstract (Moebius maps). k = 0: p_t = sigma^2 +
    G_t^2 (p_0 - sigma^2) and S_t = G_t S_0. Constant (alpha, ||k||^2, r): with
    c = ||k||^2 / (d_k r), p converges to the positive root of
    c a^2 p^2 + (1 + c Q - a^2) p - Q = 0."""
    rng = _rng(34)
    L, dk, dv, sig2 = 30, 4, 3, 0.8
    a = rng.uniform(0.7, 1.0, (1, 1, L)).astype(np.float32)
    z = np.zeros((1, 1, L, dk), np.float32)
    v = rng.standard_normal((1, 1, L, dv)).astype(np.float32)
    S0 = rng.standard_normal((1, 1, dk, dv))
    p0 = np.array([[3.0]])
    res = orc.scan(z, z, v, alpha=a, r=np.ones((1, 1, L), np.float32), cov0=p0,
                   q_noise_var=sig2, S0=S0, mode="iso")
    G = np.prod(a.astype(np.float64))
    np.testing.assert_allclose(res["cov"], sig2 + G ** 2 * (p0 - sig2), rtol=1e-12)
    np.testing.assert_allclose(res["S"][0, 0], G * S0[0, 0], rtol=1e-12)

    L = 4000
    al, rr = np.float32(0.9), np.float32(0.5)
    kk = np.full((1, 1, L, dk), np.float32(0.75))
    res = orc.scan(kk, kk, np.zeros((1, 1, L, 1), np.float32), alpha=np.full((1, 1, L), al),
                   r=np.full((1, 1, L), rr), cov0=np.ones((1, 1)), q_noise_var=sig2, mode="iso")
    a2, Q = float(al) ** 2, (1 - float(al) ** 2) * sig2
    c = dk * 0.75 ** 2 / (dk * float(rr))
    root = max(np.roots([c * a2, 1 + c * Q - a2, -Q]).real)
    np.testing.assert_allclose(res["cov"][0, 0], root, rtol=1e-12)


def test_iso_equals_diag_for_one_dimensional_keys(orc):
    """With d_k = 1 a single variance per head and a diagonal covariance are the
    same family, so the isotropic and the diagonal writes must agree exactly
    over a whole sequence (any decay, noise and process noise)."""
    rng = _rng(35)
    B, H, L, dv = 2, 2, 70, 5
    q = rng.standard_normal((B, H, L, 1)).astype(np.float32)
    k = rng.standard_normal((B, H, L, 1)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    a = rng.uniform(0.7, 1.0, (B, H, L)).astype(np.float32)
    r = rng.uniform(0.2, 2.0, (B, H, L)).astype(np.float32)
    p0 = rng.uniform(0.5, 2.0, (B, H))
    for sig2 in (0.0, 1.0):
        iso = orc.scan(q, k, v, alpha=a, r=r, cov0=p0, q_noise_var=sig2, mode="iso")
        diag = orc.scan(q, k, v, alpha=a, r=r, cov0=p0[..., None], q_noise_var=sig2, mode="diag")
        np.testing.assert_allclose(iso["o"], diag["o"], rtol=0, atol=1e-13 * np.abs(diag["o"]).max())
        np.testing.assert_allclose(iso["cov"], diag["cov"][..., 0], rtol=1e-13)
        np.testing.assert_allclose(iso["m"], diag["m"], rtol=1e-12)


# ---------------------------------------------------------------------------
# Delta write (gated and plain forms)
# ---------------------------------------------------------------------------

def _orthonormal_basis(rng, d):
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return Qm


def test_delta_orthonormal_keys_closed_form(orc):
    """A Hippocampus for Linear Attention, sec. 3.3 eq. (5) and sec. 3.5: with keys
    drawn (with repeats) from an orthonormal basis u_1..u_d, the write only
    touches the direction of the current key, so x_i = S^T u_i follows a scalar
    recursion: for the written key x <- alpha (1 - beta) x + beta v (gated
    residual e = v - alpha S^T k), for every other key x <- alpha x. The read-out
    is o_t = sum_i (q_t . u_i) x_i after the write. Signed permutations of the
    standard basis make the keys exact in float32."""
    rng = _rng(19)
    B, H, L, d, dv = 1, 2, 80, 8, 5
    for kind in ("perm", "qr"):
        U = np.eye(d)[rng.permutation(d)] * rng.choice([-1.0, 1.0], d)[:, None] if kind == "perm" \
            else _orthonormal_basis(rng, d)
        U = U.astype(np.float32)
        idx = rng.integers(0, d, (B, H, L))
        k = U[idx]
        q = rng.standard_normal((B, H, L, d)).astype(np.float32)
        v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
        a = rng.uniform(0.6, 1.0, (B, H, L)).astype(np.float32)
        beta = rng.uniform(0.0, 1.0, (B, H, L)).astype(np.float32)
        S0 = rng.standard_normal((B, H, d, dv))
        tol = 1e-12 if kind == "perm" else 1e-6
        for resid in ("gated", "plain"):
            res = orc.scan(q, k, v, alpha=a, beta=beta, S0=S0, mode="delta", resid=resid)
            U64 = U.astype(np.float64)
            v64 = v.astype(np.float64)
            for h in range(H):
                x = U64 @ S0[0, h]                      # rows: x_i = S^T u_i
                for t in range(L):
                    i = idx[0, h, t]
                    al, be = float(a[0, h, t]), float(beta[0, h, t])
                    xi_old = x[i].copy()
                    x *= al
                    if resid == "gated":
                        x[i] = al * (1 - be) * xi_old + be * v64[0, h, t]
                    else:
                        x[i] = (al - be) * xi_old + be * v64[0, h, t]
                    o_t = (U64 @ q[0, h, t].astype(np.float64)) @ x
                    np.testing.assert_allclose(res["o"][0, h, t], o_t, atol=tol * 10)
                np.testing.assert_allclose(U64 @ res["S"][0, h], x, atol=tol * 10)


def test_delta_exact_recall_unit_beta(orc):
    """A Hippocampus for Linear Attention, sec. 3.3 (the delta rule is the
    Widrow-Hoff/LMS rule): beta = 1 with orthonormal keys stores each value
    exactly; under decay S_n^T k_j = (prod_{i>j} alpha_i) v_j."""
    rng = _rng(20)
    d, dv, n = 16, 6, 16
    perm = rng.permutation(d)
    k = np.eye(d, dtype=np.float32)[perm][None, None]
    v = rng.standard_normal((1, 1, n, dv)).astype(np.float32)
    q = k.copy()
    for gated in (False, True):
        a = (rng.uniform(0.5, 1.0, (1, 1, n)) if gated else np.ones((1, 1, n))).astype(np.float32)
        res = orc.scan(q, k, v, alpha=a, beta=np.ones((1, 1, n), np.float32))
        recall = k[0, 0].astype(np.float64) @ res["S"][0, 0]
        decay = np.array([np.prod(a[0, 0, j + 1:].astype(np.float64)) for j in range(n)])
        np.testing.assert_allclose(recall, decay[:, None] * v[0, 0], rtol=1e-15, atol=0)
        # o_t reads the just-written value back exactly
        np.testing.assert_allclose(res["o"][0, 0], v[0, 0], rtol=1e-15, atol=0)


@pytest.mark.parametrize("mode,resid", [("delta", "gated"), ("delta", "plain"), ("diag", "gated"),
                                        ("iso", "gated"), ("full", "gated")])
def test_split_scan_resumes_exactly(orc, mode, resid):
    """The write is a first-order recursion in the memory S (and, for the
    Kalman forms, its covariance): each token's update uses only the state
    left by the token before (A Hippocampus for Linear Attention, eq. (5);
    Kalman Delta Networks, abstract: a linear-Gaussian state-space model
    filtered token by token). So a scan over
    [0, L) equals a scan over [0, L1) followed by one over [L1, L) started from
    the state and covariance the first returns, exactly: a returned state or
    covariance taken before the last token's update fails this."""
    B, H, L, L1, dk, dv = 1, 2, 23, 9, 6, 5
    kal = mode != "delta"
    inp = workloads.scan_inputs(B, H, L, dk, dv, seed=31, dtype="f32", with_r=kal)
    rng = _rng(31)
    cov0 = {"diag": rng.uniform(0.5, 2.0, (B, H, dk)),
            "iso": rng.uniform(0.5, 2.0, (B, H)),
            "full": np.eye(dk)[None, None] * rng.uniform(0.5, 2.0, (B, H, 1, 1))}.get(mode)
    S0 = rng.standard_normal((B, H, dk, dv))
    kw = dict(mode=mode, resid=resid, q_noise_var=0.3 if kal else 0.0)

    def part(a, b, S, cov):
        sl = {n: (x[:, :, a:b] if x is not None else None) for n, x in inp.items()}
        return orc.scan(sl["q"], sl["k"], sl["v"], alpha=sl["alpha"],
                        beta=None if kal else sl["beta"], r=sl["r"], cov0=cov, S0=S, **kw)

    whole = part(0, L, S0, cov0)
    first = part(0, L1, S0, cov0)
    second = part(L1, L, first["S"], first["cov"])
    np.testing.assert_array_equal(np.concatenate([first["o"], second["o"]], 2), whole["o"])
    np.testing.assert_array_equal(second["S"], whole["S"])
    np.testing.assert_array_equal(np.concatenate([first["m"], second["m"]], 2), whole["m"])
    if kal:
        np.testing.assert_array_equal(second["cov"], whole["cov"])


def test_delta_noop_write(orc):
    """alpha = 1, beta = 0: the write Delta_t = beta k e^T (A Hippocampus for
    Linear Attention, eq. (5)) vanishes, S stays S_0 and o_t = S_0^T q_t."""
    inp = workloads.scan_inputs(2, 3, 33, 8, 7, seed=21, dtype="f32")
    S0 = _rng(21).standard_normal((2, 3, 8, 7))
    res = orc.scan(inp["q"], inp["k"], inp["v"], alpha=np.ones((2, 3, 33), np.float32),
                   beta=np.zeros((2, 3, 33), np.float32), S0=S0)
    np.testing.assert_array_equal(res["S"], S0)
    np.testing.assert_allclose(res["o"], np.einsum("bhtk,bhkv->bhtv", inp["q"].astype(np.float64), S0),
                               rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(res["m"], 0.0)


@pytest.mark.parametrize("drop", [None, 1e-6, 1e-8])
def test_plain_residual_is_reparameterised_gated(orc, drop):
    """The plain residual e = v - S^T k with decay alpha equals the gated form of
    sec. 3.5 (A Hippocampus for Linear Attention) under (beta, v) -> (beta/alpha,
    alpha v): the rank-1 write, hence the score, is unchanged. Also with single
    tokens whose decay drops to 1e-6 or 1e-8 (alpha in (0, 1], sec. 3.5)."""
    inp = workloads.scan_inputs(1, 2, 40, 8, 6, seed=22, dtype="f32")
    a = inp["alpha"]
    if drop is not None:
        a[:, :, [3, 17, 18, 31]] = drop
    plain = orc.scan(inp["q"], inp["k"], inp["v"], alpha=a, beta=inp["beta"], resid="plain")
    gated = orc.scan(inp["q"], inp["k"], (inp["v"].astype(np.float64) * a[..., None]),
                     alpha=a, beta=(inp["beta"].astype(np.float64) / a), resid="gated")
    # the reparameterised inputs are rounded to float32 at the interface
    np.testing.assert_allclose(plain["o"], gated["o"], atol=1e-6 * np.abs(plain["o"]).max())
    np.testing.assert_allclose(plain["m"], gated["m"], rtol=1e-6)


def test_score_is_frobenius_norm_of_write(orc):
    """A Hippocampus for Linear Attention, eq. (6): m_t = ||Delta_t||_F, with
    Delta_t = S_t - alpha_t S_{t-1} the token's whole effect on the state, and
    for unit keys m_t = beta_t ||e_t||. Checked by differencing whole states
    (brute force), in the delta and in the Kalman modes."""
    rng = _rng(23)
    d, dv, L = 16, 9, 12
    k = rng.choice([-0.25, 0.25], (1, 1, L, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, L, dv)).astype(np.float32)
    a = rng.uniform(0.7, 1.0, (1, 1, L)).astype(np.float32)
    beta = rng.uniform(0.1, 1.0, (1, 1, L)).astype(np.float32)
    r = rng.uniform(0.5, 1.0, (1, 1, L)).astype(np.float32)
    for mode in ("delta", "diag", "full"):
        cov0 = np.ones((1, 1, d)) if mode == "diag" else (np.eye(d)[None, None] if mode == "full" else None)
        full = orc.scan(q, k, v, alpha=a, beta=beta, r=r, cov0=cov0, q_noise_var=0.5, mode=mode)
        prev = np.zeros((d, dv))
        for t in range(1, L + 1):
            res = orc.scan(q[:, :, :t], k[:, :, :t], v[:, :, :t], alpha=a[..., :t],
                           beta=beta[..., :t], r=r[..., :t], cov0=cov0, q_noise_var=0.5, mode=mode)
            delta = res["S"][0, 0] - float(a[0, 0, t - 1]) * prev
            np.testing.assert_allclose(full["m"][0, 0, t - 1], np.linalg.norm(delta), rtol=1e-12)
            prev = res["S"][0, 0]


def test_delta_state_stays_bounded(orc):
    """A Hippocampus for Linear Attention, sec. 3.4: unit keys keep the
    eigenvalues of I - beta k k^T in [0, 1], so with alpha <= 1 and beta in [0, 1]
    the state cannot blow up over a long sequence."""
    inp = workloads.scan_inputs(1, 4, 3000, 32, 32, seed=24, dtype="f32", alpha="one")
    res = orc.scan(inp["q"], inp["k"], inp["v"], beta=inp["beta"])
    vmax = np.abs(inp["v"]).max()
    assert np.all(np.isfinite(res["S"]))
    assert np.linalg.norm(res["S"], axis=(-2, -1)).max() < 3000 * vmax


# ---------------------------------------------------------------------------
# HOLA exact cache
# ---------------------------------------------------------------------------

def test_cache_membership_equals_sorted_topw(orc):
    """A Hippocampus for Linear Attention, sec. 3.3: the cache holds the w
    tokens with the largest score seen so far; because a token's score is fixed
    when it is written, online maintenance equals selecting the top-w of the whole
    history (ties: the earlier token wins). Brute force by sorting at every step."""
    rng = _rng(25)
    B, H, dk, dv, w, T = 2, 3, 4, 3, 8, 60
    cache = orc.HolaCache(B, H, dk, dv, w)
    hist = []
    for t in range(T):
        q = rng.standard_normal((B, H, dk)).astype(np.float32)
        k = rng.standard_normal((B, H, dk)).astype(np.float32)
        v = rng.standard_normal((B, H, dv)).astype(np.float32)
        # coarse scores force many exact ties
        m = np.round(rng.uniform(0, 4, (B, H)) * 2) / 2
        hist.append(m.astype(np.float32))
        cache.step(q, k, v, m, t)
        scores = np.stack(hist, -1)
        for b in range(B):
            for h in range(H):
                order = sorted(range(t + 1), key=lambda j: (-scores[b, h, j], j))[:w]
                n = cache.count[b, h]
                assert n == min(t + 1, w)
                assert sorted(cache.pos[b, h, :n].tolist()) == sorted(order)


def test_cache_membership_nan_scores_rank_last(orc):
    """The pages never meet a NaN score; the reading taken is that a NaN score
    ranks below every other score (as -infinity). With it the online cache
    still equals the top-w of the whole history, one token at a time and a
    whole prompt in blocks. Brute force: sort with NaN mapped to -infinity."""
    rng = _rng(26)
    B, H, dk, dv, w, T = 1, 3, 4, 3, 6, 50
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    m = np.round(rng.uniform(0, 3, (B, H, T)) * 2) / 2
    m[rng.uniform(size=(B, H, T)) < 0.3] = np.nan
    m[0, 0, :4] = np.nan          # NaN slots in a cache that then fills up
    key = lambda s, j: (-(s[j] if s[j] == s[j] else -np.inf), j)  # noqa: E731
    cache = orc.HolaCache(B, H, dk, dv, w)
    for t in range(T):
        cache.step(q[:, :, t], k[:, :, t], v[:, :, t], m[:, :, t], t)
        for h in range(H):
            s = m[0, h, :t + 1].astype(np.float32)
            order = sorted(range(t + 1), key=lambda j: key(s, j))[:w]
            assert sorted(cache.pos[0, h, :cache.count[0, h]].tolist()) == sorted(order)
    for block in (1, 7, 64):
        c = orc.HolaCache(B, H, dk, dv, w)
        c.prefill(q, k, v, m, 0, block)
        for h in range(H):
            s = m[0, h].astype(np.float32)
            order = sorted(range(T), key=lambda j: key(s, j))[:w]
            np.testing.assert_array_equal(c.pos[0, h], np.array(order))


def _rmsnorm(x, eps):
    import torch
    return torch.nn.functional.rms_norm(x, (x.shape[-1],), eps=eps)


def test_cache_read_is_softmax_attention_when_nothing_evicted(orc):
    """A Hippocampus for Linear Attention, sec. 3.2 eq. (4) and sec. 3.4 eq. (7):
    while nothing has been evicted (w >= t) the cache read over the visible set is
    exact causal softmax attention on RMS-normalised q, k at scale 1/sqrt(d).
    Reference: torch's rms_norm and scaled_dot_product_attention (CPU, float64).
    At t = 0 the only visible token is the current one, so o = v_0 exactly."""
    import torch
    rng = _rng(26)
    B, H, dk, dv, T, eps = 2, 2, 16, 8, 20, 1e-6
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    for use_sink in (False, True):
        cache = orc.HolaCache(B, H, dk, dv, T)
        outs = []
        for t in range(T):
            outs.append(cache.step(q[:, :, t], k[:, :, t], v[:, :, t], np.ones((B, H)), t,
                                   sink_logit=sink if use_sink else None, rms_eps=eps))
        got = np.stack(outs, 2)
        qt = _rmsnorm(torch.from_numpy(q).double(), eps)
        kt = _rmsnorm(torch.from_numpy(k).double(), eps)
        vt = torch.from_numpy(v).double()
        if not use_sink:
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
            np.testing.assert_array_equal(got[:, :, 0], v[:, :, 0].astype(np.float64))
        else:
            # one extra key whose logit is set through the additive mask; its value is 0
            kz = torch.cat([kt, torch.zeros(B, H, 1, dk, dtype=torch.float64)], 2)
            vz = torch.cat([vt, torch.zeros(B, H, 1, dv, dtype=torch.float64)], 2)
            mask = torch.full((T, T + 1), float("-inf"), dtype=torch.float64)
            mask[:, :T] = torch.triu(torch.full((T, T), float("-inf"), dtype=torch.float64), 1)
            mask = mask.expand(B, H, T, T + 1).clone()
            mask[..., T] = torch.from_numpy(sink.astype(np.float64))[None, :, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kz, vz, attn_mask=mask)
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, val = line.split("=")
                vals[key.strip()] = float(val)
    return vals


def test_cache_read_sharpness_numbers_from_the_page(orc):
    """A Hippocampus for Linear Attention, sec. 3.4: among w = 64 entries, a
    perfectly matching key whose logit is ~0.83 (others orthogonal, logit 0) gets
    only ~3.5% of the mass; with RMS-normalised q, k of norm sqrt(d) the logit is
    ~sqrt(d) cos (~11 cos for d = 128) and the read becomes near-argmax."""
    g = _read_golden("hola_read_sharpness.txt")
    d, w = 128, int(g["w"])
    basis = np.eye(d, dtype=np.float32)
    for target_logit, expect, tol in ((g["unit_logit"], g["unit_mass"], g["unit_mass_tol"]),
                                      (math.sqrt(d), None, None)):
        cache = orc.HolaCache(1, 1, d, w, w)
        # w - 1 cached keys along e_1..e_{w-1}; one-hot values expose the softmax weights
        for j in range(w - 1):
            vj = np.zeros((1, 1, w), np.float32)
            vj[0, 0, j] = 1
            cache.step(np.zeros((1, 1, d), np.float32) + basis[0], basis[j + 1][None, None], vj,
                       np.ones((1, 1)), j, rms_eps=0.0)
        # the current token: key e_0; query with cos(q, e_0) = target / sqrt(d)
        cos = target_logit / math.sqrt(d)
        qv = (cos * basis[0]).astype(np.float32)
        qv[w] = math.sqrt(max(0.0, 1 - cos ** 2))   # e_w is orthogonal to every key present
        v_cur = np.zeros((1, 1, w), np.float32)
        v_cur[0, 0, w - 1] = 1
        o = cache.step(qv[None, None], basis[0][None, None], v_cur, np.ones((1, 1)), w - 1, rms_eps=0.0)
        mass = o[0, 0, w - 1]
        analytic = math.exp(target_logit) / (math.exp(target_logit) + (w - 1))
        np.testing.assert_allclose(mass, analytic, rtol=1e-6)
        if expect is not None:
            assert abs(mass - expect) <= tol
        else:
            assert mass > g["sharp_mass_min"]


# ---------------------------------------------------------------------------
# HOLA cache over a whole prompt (block by block)
# ---------------------------------------------------------------------------

def test_prefill_with_unit_blocks_is_the_decode_step(orc):
    """A Hippocampus for Linear Attention, sec. 3.4 eq. (7): the visible set of
    a token is the cache, the causal tokens of its block and the sink. With
    blocks of one token that is the decode step's read-then-insert, so the
    prompt routine must reproduce a sequence of decode steps exactly, starting
    from a non-empty cache."""
    rng = _rng(40)
    B, H, dk, dv, w, L = 2, 2, 8, 5, 6, 40
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    m = np.round(rng.uniform(0, 3, (B, H, L)) * 4) / 4   # many exact ties
    sink = rng.standard_normal(H).astype(np.float32)
    a = orc.HolaCache(B, H, dk, dv, w)
    for t in range(4):                                    # a cache from earlier tokens
        a.step(q[:, :, t], k[:, :, t], v[:, :, t], m[:, :, t] + 1.0, t - 10)
    b = orc.HolaCache(B, H, dk, dv, w)
    for f in ("k", "v", "m", "pos", "count"):
        setattr(b, f, getattr(a, f).copy())
    steps = np.stack([a.step(q[:, :, t], k[:, :, t], v[:, :, t], m[:, :, t], t + 100, sink)
                      for t in range(L)], 2)
    pre = b.prefill(q, k, v, m, 100, 1, sink)
    np.testing.assert_allclose(pre, steps, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(b.count, a.count)
    for bb in range(B):
        for h in range(H):
            n = a.count[bb, h]
            sa = sorted(zip(a.pos[bb, h, :n], a.m[bb, h, :n]))
            sb = sorted(zip(b.pos[bb, h, :n], b.m[bb, h, :n]))
            assert sa == sb
            ia, ib = np.argsort(a.pos[bb, h, :n]), np.argsort(b.pos[bb, h, :n])
            np.testing.assert_array_equal(a.k[bb, h, ia], b.k[bb, h, ib])
            np.testing.assert_array_equal(a.v[bb, h, ia], b.v[bb, h, ib])


def test_prefill_without_eviction_is_causal_attention(orc):
    """A Hippocampus for Linear Attention, sec. 3.2 eq. (4), sec. 3.4 eq. (7):
    when nothing is evicted (w >= cached + L) every token sees every earlier
    token (from the cache or from its own block) and itself, for any block
    size: exact causal softmax attention on RMS-normalised q, k at 1/sqrt(d),
    here against torch's rms_norm and scaled_dot_product_attention in float64,
    with the cached tokens as an always-visible prefix and the sink as an extra
    key through the additive mask."""
    import torch
    rng = _rng(41)
    B, H, dk, dv, L, P, eps = 1, 2, 16, 8, 45, 3, 1e-6
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, P + L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, P + L, dv)).astype(np.float32)
    sink = rng.standard_normal(H).astype(np.float32)
    qt = _rmsnorm(torch.from_numpy(q).double(), eps)
    kt = _rmsnorm(torch.from_numpy(k).double(), eps)
    vt = torch.from_numpy(v).double()
    kz = torch.cat([kt, torch.zeros(B, H, 1, dk, dtype=torch.float64)], 2)
    vz = torch.cat([vt, torch.zeros(B, H, 1, dv, dtype=torch.float64)], 2)
    for use_sink in (False, True):
        mask = torch.full((L, P + L + 1), float("-inf"), dtype=torch.float64)
        mask[:, :P] = 0.0
        mask[:, P:P + L] = torch.triu(torch.full((L, L), float("-inf"), dtype=torch.float64), 1)
        mask = mask.expand(B, H, L, P + L + 1).clone()
        if use_sink:
            mask[..., P + L] = torch.from_numpy(sink.astype(np.float64))[None, :, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kz, vz, attn_mask=mask).numpy()
        for block in (1, 7, 16, 64):
            c = orc.HolaCache(B, H, dk, dv, P + L)
            for t in range(P):
                c.step(q[:, :, 0], k[:, :, t], v[:, :, t], np.ones((B, H)), t - P)
            got = c.prefill(q, k[:, :, P:], v[:, :, P:], rng.uniform(0, 1, (B, H, L)), 0, block,
                            sink if use_sink else None, eps)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_prefill_final_cache_is_sorted_topw(orc):
    """A Hippocampus for Linear Attention, sec. 3.3: the cache is the top-w of
    the whole history by score (ties: the earlier token), whatever the block
    size; the prompt routine leaves it in that order. Brute force by sorting."""
    rng = _rng(42)
    B, H, dk, dv, w, L = 1, 3, 4, 3, 10, 77
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    m = np.round(rng.uniform(0, 3, (B, H, L)) * 3) / 3
    m32 = m.astype(np.float32)
    for block in (1, 5, 32, 200):
        c = orc.HolaCache(B, H, dk, dv, w)
        c.prefill(q, k, v, m, 1000, block)
        for h in range(H):
            order = sorted(range(L), key=lambda j: (-m32[0, h, j], j))[:w]
            assert c.count[0, h] == w
            np.testing.assert_array_equal(c.pos[0, h], np.array(order) + 1000)
            np.testing.assert_array_equal(c.m[0, h], m32[0, h, order])
            np.testing.assert_array_equal(c.k[0, h], k[0, h, order])
            np.testing.assert_array_equal(c.v[0, h], v[0, h, order])


# ---------------------------------------------------------------------------
# Ablation switches: no-erase write, score variants, recency eviction
# ---------------------------------------------------------------------------

def test_noerase_is_decayed_linear_attention(orc):
    """A Hippocampus for Linear Attention, sec. 3.5 (the gated delta rule adds an
    erase term to the decayed outer-product write): without it,
    S_t = sum_{j<=t} (prod_{j<i<=t} alpha_i) beta_j k_j v_j^T and o_t = S_t^T q_t,
    written out here directly."""
    inp = workloads.scan_inputs(2, 2, 60, 8, 5, seed=50, dtype="f32")
    res = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"],
                   resid="noerase")
    a, b = inp["alpha"].astype(np.float64), inp["beta"].astype(np.float64)
    K, V, Q = (inp[n].astype(np.float64) for n in ("k", "v", "q"))
    L = a.shape[-1]
    for t in (0, 17, L - 1):
        w = np.array([np.prod(a[..., j + 1:t + 1], axis=-1) for j in range(t + 1)])  # [t+1,B,H]
        S = np.einsum("jbh,bhj,bhjd,bhje->bhde", w, b[..., :t + 1], K[:, :, :t + 1], V[:, :, :t + 1])
        np.testing.assert_allclose(res["o"][:, :, t], np.einsum("bhde,bhd->bhe", S, Q[:, :, t]),
                                   rtol=0, atol=1e-12)
        if t == L - 1:
            np.testing.assert_allclose(res["S"], S, rtol=0, atol=1e-12)
    # its write score is beta ||v||
    np.testing.assert_allclose(res["m"], b * np.linalg.norm(V, axis=-1), rtol=1e-12)


def test_score_variants(orc):
    """A Hippocampus for Linear Attention, sec. 3.3 ("versus recency") and sec.
    4.5: the ablation scores are the residual alone, ||e_t||, and the write
    strength alone, beta_t ||v_t||. ||e_t|| is recomputed from the states of
    the prefix scans (brute force); beta ||v|| from the inputs."""
    inp = workloads.scan_inputs(1, 2, 25, 8, 6, seed=51, dtype="f32")
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    resid = orc.scan(q, k, v, alpha=a, beta=b, score="resid")["m"]
    value = orc.scan(q, k, v, alpha=a, beta=b, score="value")["m"]
    np.testing.assert_allclose(value, b.astype(np.float64) * np.linalg.norm(v.astype(np.float64), axis=-1),
                               rtol=1e-12)
    prev = np.zeros((1, 2, 8, 6))
    for t in range(25):
        e = v[:, :, t].astype(np.float64) - a[:, :, t, None] * np.einsum("bhde,bhd->bhe", prev, k[:, :, t])
        np.testing.assert_allclose(resid[:, :, t], np.linalg.norm(e, axis=-1), rtol=1e-11)
        prev = orc.scan(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1], alpha=a[..., :t + 1],
                        beta=b[..., :t + 1])["S"]
    # Kalman writes: the write strength is the gain's norm
    r = np.ones_like(a)
    p0 = np.ones((1, 2, 8))
    wr = orc.scan(q, k, v, alpha=a, r=r, cov0=p0, mode="diag", score="write")["m"]
    rs = orc.scan(q, k, v, alpha=a, r=r, cov0=p0, mode="diag", score="resid")["m"]
    va = orc.scan(q, k, v, alpha=a, r=r, cov0=p0, mode="diag", score="value")["m"]
    np.testing.assert_allclose(va, wr / rs * np.linalg.norm(v.astype(np.float64), axis=-1), rtol=1e-11)


def test_recency_eviction_keeps_the_last_w(orc):
    """A Hippocampus for Linear Attention, sec. 4.5 (the matched control keeps the
    most recent w tokens): decode-step and prompt versions, against brute force,
    and the prompt version with unit blocks against the decode steps."""
    rng = _rng(52)
    B, H, dk, dv, w, L = 1, 2, 4, 3, 7, 40
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    m = rng.uniform(0, 1, (B, H, L))
    a = orc.HolaCache(B, H, dk, dv, w, policy="recency")
    outs = []
    for t in range(L):
        outs.append(a.step(q[:, :, t], k[:, :, t], v[:, :, t], m[:, :, t], t))
        n = a.count[0, 0]
        assert sorted(a.pos[0, 0, :n].tolist()) == list(range(max(0, t + 1 - w), t + 1))
    for block in (1, 6, 64):
        c = orc.HolaCache(B, H, dk, dv, w, policy="recency")
        o = c.prefill(q, k, v, m, 0, block)
        np.testing.assert_array_equal(c.pos[0, 0], np.arange(L - 1, L - 1 - w, -1))
        np.testing.assert_array_equal(c.k[0, 1], k[0, 1, L - 1:L - 1 - w:-1])
        if block == 1:
            np.testing.assert_allclose(o, np.stack(outs, 2), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Backward pass of the delta-write scan
# ---------------------------------------------------------------------------

def _fd_loss(orc, inp, S0, d_o, dS, resid):
    r = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], S0=S0,
                 resid=resid, want_m=False)
    return float(np.sum(r["o"] * d_o) + np.sum(r["S"] * dS))


@pytest.mark.parametrize("resid,L,dk,dv", [("gated", 9, 4, 3), ("plain", 9, 4, 3),
                                           ("noerase", 9, 4, 3), ("gated", 150, 4, 3),
                                           ("gated", 9, 3, 5)])
def test_backward_matches_finite_differences(orc, resid, L, dk, dv):
    """The gradients of the scan (the pages give none; the adjoint recurrence is
    derived for this library) against central finite differences of the forward
    oracle, for every input including the initial state, on a loss
    sum(d_o * o) + sum(dS * S_L). Inputs are float32, so the steps are powers
    of two that keep the perturbed inputs exact; L = 150 crosses the backward's
    64-token recomputation checkpoints (sampled elements); d_v > d_k once."""
    rng = _rng(60 + L)
    B, H = 1, 2
    inp = workloads.scan_inputs(B, H, L, dk, dv, seed=61, dtype="f32")
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    d_o = rng.standard_normal((B, H, L, dv))
    dS = rng.standard_normal((B, H, dk, dv))
    g = orc.scan_bwd(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], S0=S0,
                     d_o=d_o, dS=dS, resid=resid)
    h = 2.0 ** -12
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta"}
    for name, gname in names.items():
        x = inp[name]
        idx = list(np.ndindex(x.shape))
        if L > 20:
            idx = [idx[i] for i in rng.choice(len(idx), 25, replace=False)]
        for ix in idx:
            xp = {**inp, name: x.copy()}
            xm = {**inp, name: x.copy()}
            xp[name][ix] += np.float32(h)
            xm[name][ix] -= np.float32(h)
            fd = (_fd_loss(orc, xp, S0, d_o, dS, resid) - _fd_loss(orc, xm, S0, d_o, dS, resid)) / (2 * h)
            assert abs(fd - g[gname][ix]) <= 1e-6 * (1 + abs(fd)), (name, ix, fd, g[gname][ix])
    for ix in np.ndindex(S0.shape):
        sp, sm = S0.copy(), S0.copy()
        sp[ix] += h
        sm[ix] -= h
        fd = (_fd_loss(orc, inp, sp, d_o, dS, resid) - _fd_loss(orc, inp, sm, d_o, dS, resid)) / (2 * h)
        assert abs(fd - g["dS0"][ix]) <= 1e-6 * (1 + abs(fd)), ("S0", ix, fd, g["dS0"][ix])


def _fd_loss_kalman(orc, inp, cov0, S0, d_o, dS, dcov, mode, qvar):
    out = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=cov0,
                   q_noise_var=qvar, S0=S0, mode=mode, want_m=False)
    return float(np.sum(d_o * out["o"]) + np.sum(dS * out["S"]) + np.sum(dcov * out["cov"]))


@pytest.mark.parametrize("mode,L,dk,dv,qvar", [("diag", 9, 4, 3, 0.7), ("iso", 9, 4, 3, 0.7),
                                               ("diag", 150, 4, 3, 1.0), ("iso", 150, 3, 5, 0.0),
                                               ("diag", 9, 3, 5, 0.0)])
def test_kalman_backward_matches_finite_differences(orc, mode, L, dk, dv, qvar):
    """The gradients of the Kalman writes (Kalman Delta Networks, abstract: the
    diagonal and isotropic covariance forms; the pages give no backward pass)
    against central finite differences of the forward oracle, for q, k, v,
    alpha, r, the prior covariance and the initial state, on a loss
    sum(d_o * o) + sum(dS * S_L) + sum(dcov * cov_L), with and without process
    noise. Keys of varying norm; L = 150 crosses the 64-token checkpoints
    (sampled elements)."""
    rng = _rng(70 + L + dk)
    B, H = 1, 2
    inp = workloads.scan_inputs(B, H, L, dk, dv, seed=71, dtype="f32", with_r=True)
    inp["k"] = (inp["k"] * rng.uniform(0.5, 1.5, (B, H, L, 1))).astype(np.float32)
    cshape = (B, H, dk) if mode == "diag" else (B, H)
    cov0 = rng.uniform(0.5, 2.0, cshape)
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    d_o = rng.standard_normal((B, H, L, dv))
    dS = rng.standard_normal((B, H, dk, dv))
    dcov = rng.standard_normal(cshape)
    g = orc.scan_bwd_kalman(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"],
                            cov0=cov0, q_noise_var=qvar, S0=S0, d_o=d_o, dS=dS, dcov=dcov, mode=mode)
    loss = lambda x, c0, s0: _fd_loss_kalman(orc, x, c0, s0, d_o, dS, dcov, mode, qvar)  # noqa: E731
    h = 2.0 ** -12
    names = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "r": "dr"}
    for name, gname in names.items():
        x = inp[name]
        idx = list(np.ndindex(x.shape))
        if L > 20:
            idx = [idx[i] for i in rng.choice(len(idx), 25, replace=False)]
        for ix in idx:
            xp = {**inp, name: x.copy()}
            xm = {**inp, name: x.copy()}
            xp[name][ix] += np.float32(h)
            xm[name][ix] -= np.float32(h)
            fd = (loss(xp, cov0, S0) - loss(xm, cov0, S0)) / (2 * h)
            assert abs(fd - g[gname][ix]) <= 1e-6 * (1 + abs(fd)), (name, ix, fd, g[gname][ix])
    for ix in np.ndindex(cov0.shape):
        cp, cm = cov0.copy(), cov0.copy()
        cp[ix] += h
        cm[ix] -= h
        fd = (loss(inp, cp, S0) - loss(inp, cm, S0)) / (2 * h)
        assert abs(fd - g["dcov0"][ix]) <= 1e-6 * (1 + abs(fd)), ("cov0", ix, fd, g["dcov0"][ix])
    sidx = list(np.ndindex(S0.shape))
    for ix in [sidx[i] for i in rng.choice(len(sidx), min(len(sidx), 12), replace=False)]:
        sp, sm = S0.copy(), S0.copy()
        sp[ix] += h
        sm[ix] -= h
        fd = (loss(inp, cov0, sp) - loss(inp, cov0, sm)) / (2 * h)
        assert abs(fd - g["dS0"][ix]) <= 1e-6 * (1 + abs(fd)), ("S0", ix, fd, g["dS0"][ix])
