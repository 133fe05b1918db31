"""fp64 CPU oracle for the delta-rule / Kalman-Delta scans and the HOLA cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; never by the product package.
It shares no code with the HIP library. The arithmetic lives in
``kdn_oracle.c`` (plain sequential C in double precision, built with gcc).

Sources are cited per function in ``kdn_oracle.c``:
"A Hippocampus for Linear Attention" (part 2/3, secs. 3.2-3.5, eqs. 4-7),
"Kalman Delta Networks: Uncertainty-aware Associative Memory" (abstract),
"Memory by Design: Probabilistic Sequence Layers" (abstract),
"DeltaNet-PC: Test-Time Memory Without Backpropagation Through Time" (eqs. 6-7).

Parity unpinned: the diagonal-covariance write with stationary process noise
and general keys (no closed form exists; pinned only through its special
cases k = 0, one-hot keys, covariance reset and the Moebius fixed point).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kdn_oracle.c")
_LIB = os.path.join(_HERE, "libkdn_oracle.so")

MODES = {"delta": 0, "diag": 1, "full": 2, "iso": 3}
RESIDS = {"gated": 0, "plain": 1, "noerase": 2}
SCORES = {"write": 0, "resid": 1, "value": 2}
POLICIES = {"score": 0, "recency": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        d = ctypes.c_double
        lib.oracle_scan.argtypes = [i, i, i, i, i, P, P, P, P, P, P, P, d, P, i, i, i, P, P]
        lib.oracle_scan.restype = i
        lib.oracle_hola_step.argtypes = [i, i, i, i, i, P, P, P, P, i, P, P, P, P, P, P, d, i, P]
        lib.oracle_hola_step.restype = i
        lib.oracle_hola_prefill.argtypes = [i, i, i, i, i, i, i, P, P, P, P, i, P, P, P, P, P, P,
                                            d, i, P]
        lib.oracle_hola_prefill.restype = i
        lib.oracle_scan_bwd.argtypes = [i, i, i, i, i, P, P, P, P, P, P, P, P, i, P, P, P, P, P, P]
        lib.oracle_scan_bwd.restype = i
        lib.oracle_scan_bwd_kalman.argtypes = [i, i, i, i, i, P, P, P, P, P, P, d, P, P, P, P, i,
                                               P, P, P, P, P, P, P]
        lib.oracle_scan_bwd_kalman.restype = i
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def _f32(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float32)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def scan(q, k, v, alpha=None, beta=None, r=None, cov0=None, q_noise_var: float = 0.0,
         S0=None, mode: str = "delta", resid: str = "gated", want_m: bool = True,
         score: str = "write") -> dict:
    """Sequential fp64 scan. q, k: [B,H,L,dk]; v: [B,H,L,dv]; alpha/beta/r: [B,H,L].
    cov0: [B,H,dk] (diag), [B,H,dk,dk] (full) or [B,H] (iso). S0: [B,H,dk,dv] (default zeros).
    Returns dict(o [B,H,L,dv], S [B,H,dk,dv], cov, m [B,H,L]) in float64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, L, dk) and v.shape == (B, H, L, dv)
    alpha, beta, r = _f32(alpha), _f32(beta), _f32(r)
    for x in (alpha, beta, r):
        assert x is None or x.shape == (B, H, L)
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, order="C")
    assert S.shape == (B, H, dk, dv)
    cov = None
    if mode == "diag":
        cov = np.array(cov0, dtype=np.float64, order="C").reshape(B, H, dk)
    elif mode == "full":
        cov = np.array(cov0, dtype=np.float64, order="C").reshape(B, H, dk, dk)
    elif mode == "iso":
        cov = np.array(cov0, dtype=np.float64, order="C").reshape(B, H)
    o = np.zeros((B, H, L, dv))
    m = np.zeros((B, H, L)) if want_m else None
    rc = _load().oracle_scan(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(beta), _ptr(r), _ptr(cov), float(q_noise_var), _ptr(S),
                             MODES[mode], RESIDS[resid], SCORES[score], _ptr(o), _ptr(m))
    if rc != 0:
        raise ValueError(f"oracle_scan rejected the arguments (status {rc})")
    return dict(o=o, S=S, cov=cov, m=m)


def scan_bwd(q, k, v, alpha=None, beta=None, S0=None, d_o=None, dS=None,
             resid: str = "gated") -> dict:
    """Gradients of the delta-write scan (fp64 adjoint, see kdn_oracle.c) for the
    loss sum(d_o * o) + sum(dS * S_L). Returns dict(dq, dk, dv, dalpha, dbeta, dS0)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    alpha, beta = _f32(alpha), _f32(beta)
    S0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    d_o = np.ascontiguousarray(d_o, dtype=np.float64)
    assert d_o.shape == (B, H, L, dv)
    dS = None if dS is None else np.ascontiguousarray(dS, dtype=np.float64)
    out = dict(dq=np.zeros((B, H, L, dk)), dk=np.zeros((B, H, L, dk)), dv=np.zeros((B, H, L, dv)),
               dalpha=np.zeros((B, H, L)), dbeta=np.zeros((B, H, L)), dS0=np.zeros((B, H, dk, dv)))
    rc = _load().oracle_scan_bwd(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                 _ptr(beta), _ptr(S0), _ptr(d_o), _ptr(dS), RESIDS[resid],
                                 _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                 _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dS0"]))
    if rc != 0:
        raise ValueError(f"oracle_scan_bwd rejected the arguments (status {rc})")
    return out


def scan_bwd_kalman(q, k, v, alpha=None, r=None, cov0=None, q_noise_var: float = 0.0, S0=None,
                    d_o=None, dS=None, dcov=None, mode: str = "diag") -> dict:
    """Gradients of the Kalman writes (mode "diag": cov [B,H,dk]; "iso": cov [B,H];
    gated residual) for the loss sum(d_o * o) + sum(dS * S_L) + sum(dcov * cov_L)
    (fp64 adjoint, see kdn_oracle.c). Returns dict(dq, dk, dv, dalpha, dr, dcov0, dS0)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    alpha, r = _f32(alpha), _f32(r)
    cshape = (B, H, dk) if mode == "diag" else (B, H)
    cov0 = np.ascontiguousarray(np.broadcast_to(cov0, cshape), dtype=np.float64)
    S0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    d_o = np.ascontiguousarray(d_o, dtype=np.float64)
    assert d_o.shape == (B, H, L, dv)
    dS = None if dS is None else np.ascontiguousarray(dS, dtype=np.float64)
    dcov = None if dcov is None else np.ascontiguousarray(np.broadcast_to(dcov, cshape),
                                                          dtype=np.float64)
    out = dict(dq=np.zeros((B, H, L, dk)), dk=np.zeros((B, H, L, dk)), dv=np.zeros((B, H, L, dv)),
               dalpha=np.zeros((B, H, L)), dr=np.zeros((B, H, L)), dcov0=np.zeros(cshape),
               dS0=np.zeros((B, H, dk, dv)))
    rc = _load().oracle_scan_bwd_kalman(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                        _ptr(r), _ptr(cov0), float(q_noise_var), _ptr(S0),
                                        _ptr(d_o), _ptr(dS), _ptr(dcov), MODES[mode],
                                        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                        _ptr(out["dalpha"]), _ptr(out["dr"]), _ptr(out["dcov0"]),
                                        _ptr(out["dS0"]))
    if rc != 0:
        raise ValueError(f"oracle_scan_bwd_kalman rejected the arguments (status {rc})")
    return out


class HolaCache:
    """Oracle-side HOLA cache state for [B, H] heads with capacity w."""

    def __init__(self, B: int, H: int, dk: int, dv: int, w: int, policy: str = "score"):
        self.B, self.H, self.dk, self.dv, self.w = B, H, dk, dv, w
        self.policy = POLICIES[policy]
        self.k = np.zeros((B, H, w, dk), np.float32)
        self.v = np.zeros((B, H, w, dv), np.float32)
        self.m = np.zeros((B, H, w), np.float32)
        self.pos = np.full((B, H, w), -1, np.int32)
        self.count = np.zeros((B, H), np.int32)

    def step(self, q, k, v, m, t: int, sink_logit=None, rms_eps: float = 1e-6):
        """Read over cache + current token (+ sink), then insert token t with score m.
        Returns o_cache [B,H,dv] float64."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        m = np.ascontiguousarray(m, dtype=np.float64)
        sink = _f32(sink_logit)
        o = np.zeros((self.B, self.H, self.dv))
        _load().oracle_hola_step(self.B, self.H, self.dk, self.dv, self.w, _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(m), int(t), _ptr(self.k), _ptr(self.v),
                                 _ptr(self.m), _ptr(self.pos), _ptr(self.count), _ptr(sink),
                                 float(rms_eps), self.policy, _ptr(o))
        return o


    def prefill(self, q, k, v, m, t0: int, block: int, sink_logit=None, rms_eps: float = 1e-6):
        """A whole prompt of L tokens (q, k: [B,H,L,dk]; v: [B,H,L,dv]; m: [B,H,L]) in
        blocks of ``block``: each token reads the cache as it stood before its block
        plus the block's tokens up to itself (+ sink); then the block is inserted.
        Returns o_cache [B,H,L,dv] float64; the cache ends sorted by (m desc, pos asc)."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        B, H, L, dk = q.shape
        assert (B, H, dk) == (self.B, self.H, self.dk) and v.shape == (B, H, L, self.dv)
        m = np.ascontiguousarray(m, dtype=np.float64)
        assert m.shape == (B, H, L)
        sink = _f32(sink_logit)
        o = np.zeros((B, H, L, self.dv))
        rc = _load().oracle_hola_prefill(B, H, L, dk, self.dv, self.w, int(block), _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(m), int(t0), _ptr(self.k), _ptr(self.v),
                                         _ptr(self.m), _ptr(self.pos), _ptr(self.count), _ptr(sink),
                                         float(rms_eps), self.policy, _ptr(o))
        if rc != 0:
            raise ValueError(f"oracle_hola_prefill rejected the arguments (status {rc})")
        return o


def decode_run(steps_inputs, B: int, H: int, dk: int, dv: int, w: int, mode: str = "delta",
               resid: str = "gated", S0=None, cov0=None, r_steps=None, q_noise_var: float = 0.0,
               sink_logit=None, rms_eps: float = 1e-6, t0: int = 0, cache: HolaCache = None,
               score: str = "write", policy: str = "score"):
    """Decode a sequence of single tokens: per step, the recurrence (one token of
    ``scan``) then the HOLA cache read/insert with that token's score.
    ``steps_inputs`` yields dicts with q, k, v ([B,H,d]) and alpha, beta ([B,H]).
    Returns (list of o, list of o_cache, list of m, final S, final cov, cache)."""
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    cov = None if cov0 is None else np.array(cov0, dtype=np.float64)
    cache = cache or HolaCache(B, H, dk, dv, w, policy)
    outs, couts, ms = [], [], []
    for i, inp in enumerate(steps_inputs):
        rr = None if r_steps is None else r_steps[i][..., None]
        res = scan(inp["q"][:, :, None], inp["k"][:, :, None], inp["v"][:, :, None],
                   alpha=inp["alpha"][..., None], beta=inp["beta"][..., None], r=rr,
                   cov0=cov, q_noise_var=q_noise_var, S0=S, mode=mode, resid=resid, score=score)
        S, cov = res["S"], res["cov"]
        m = res["m"][..., 0]
        oc = cache.step(inp["q"], inp["k"], inp["v"], m, t0 + i, sink_logit, rms_eps)
        outs.append(res["o"][:, :, 0])
        couts.append(oc)
        ms.append(m)
    return outs, couts, ms, S, cov, cache
