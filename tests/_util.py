"""Helpers shared by the GPU parity tests: tensor upload and the tolerance check.

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
