"""Helpers shared by the GPU parity tests: tensor upload, the tolerance check
and the extreme-decay pattern of the scan and backward tests.

The bar: err = max |x_gpu - x_oracle| <= tol * RMS(x_oracle), with tol = 1e-4
for float32 workloads and 2e-2 for bf16 inputs with float32 state.
"""
import sys

import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(x, dtype="f32"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
    return t.cuda()


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return err / rms if rms > 0 else err


def assert_close(got, ref, tol, what=""):
    """err = max|got - ref| / RMS(ref) <= tol; the measured ratio is printed
    (with -s, or in the captured output of a failing test) so margins show."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    e = rel_err(got, ref)
    log(f"  {what}: max|diff|/RMS = {e:.3e} (tol {tol:.0e}, margin {tol / max(e, 1e-300):.1f}x)")
    assert e <= tol, f"{what}: max|diff| / RMS = {e:.3e} > {tol:.1e}"
    return e


def extreme_alpha(B, H, L, seed):
    """Decays that stress the chunk form's factored decay ratios (alpha in
    (0, 1], A Hippocampus for Linear Attention, sec. 3.5), in 64-token chunks:
    0: alpha = 1 exactly; 1: alpha = 1e-3 on the first half (a 16-token span
    of log2 decay ~160, past the factored ratios' range); 2: alpha = 1 on the
    first half and 1e-4 on the second (an abrupt switch); 3: the gated
    distribution with single-token drops to 1e-6 and 1e-8; 4: alpha = 1e-8
    on every token; 5 (ragged tail): alternating 1 and 1e-3, the last token
    0.3 (so the state carried out of a chunk sees a decay other than 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = np.exp(-np.logaddexp(0.0, rng.standard_normal((B, H, L))) * 0.1)
    a[..., 0:64] = 1.0
    a[..., 64:96] = 1e-3
    a[..., 128:160] = 1.0
    a[..., 160:192] = 1e-4
    a[..., [197, 203, 230, 231, 250]] = [1e-6, 1e-8, 1e-8, 1e-6, 1e-8]
    a[..., 256:320] = 1e-8
    a[..., 320::2] = 1.0
    a[..., 321::2] = 1e-3
    a[..., -1] = 0.3
    return a.astype(np.float32)
