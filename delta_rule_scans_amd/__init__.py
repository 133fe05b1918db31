"""MI355X-native delta-rule / Kalman-Delta scans and the HOLA exact cache.

A thin ctypes binding over ``libkdn.so`` (built from ``csrc/`` by
``delta_rule_scans_amd.build``); its C ABI is declared in ``include/kdn.h``.
This module only marshals arguments: it checks devices, dtypes and shapes,
allocates outputs and workspace through torch (device memory and streams
only), and passes raw pointers and the current HIP stream. Every step of the
computation runs in the HIP kernels. There is no CPU fallback: importing the
package fails if the library has not been built.

Functions carry the C names:
  kdn_scan_fwd       chunkwise scan over whole sequences
  kdn_step_decode    one token per head, state updated in place
  hola_cache_update  HOLA cache read + top-w insert for one token per head
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "lib", "KdnError", "kdn_scan_fwd", "kdn_step_decode", "hola_cache_update",
    "kdn_scan_workspace_size", "kdn_status_string", "HolaCache", "LIB_PATH",
    "hola_prefill", "hola_prefill_workspace_size", "kdn_scan_bwd",
    "F32", "BF16", "MODES", "RESIDS", "PHASES", "kdn_scan_fwd_static", "STATIC_SCRATCH_BYTES",
    "kdn_scan_bwd_ex",
]

STATIC_SCRATCH_BYTES = 64 << 20  # KDN_STATIC_SCRATCH_BYTES in include/kdn.h

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkdn.so")

F32, BF16 = 0, 1
MODES = {"delta": 0, "diag": 1, "full": 2, "iso": 3}
RESIDS = {"gated": 0, "plain": 1, "noerase": 2}
SCORES = {"write": 0, "resid": 1, "value": 2}
POLICIES = {"score": 0, "recency": 1}
PHASES = {"all": 0, "prepare": 1, "state": 2}


class KdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {kdn_status_string(status)}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m delta_rule_scans_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.kdn_status_string.argtypes = [I]
    L.kdn_status_string.restype = ctypes.c_char_p
    L.kdn_version.argtypes = []
    L.kdn_version.restype = I
    L.kdn_scan_workspace_size.argtypes = [I, I, I, I, I, I, I, I, I]
    L.kdn_scan_workspace_size.restype = SZ
    L.kdn_scan_fwd.argtypes = [P, P, P, I, P, P, P, P, P, F, P, P, P, I, P, I,
                               I, I, I, I, I, I, I, I, P, SZ, P]
    L.kdn_scan_fwd.restype = I
    L.kdn_scan_fwd_phase.argtypes = [I] + L.kdn_scan_fwd.argtypes
    L.kdn_scan_fwd_phase.restype = I
    L.kdn_scan_fwd_static.argtypes = L.kdn_scan_fwd.argtypes[:-3] + [P]
    L.kdn_scan_fwd_static.restype = I
    L.kdn_step_decode.argtypes = [P, P, P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, P]
    L.kdn_step_decode.restype = I
    L.hola_cache_update.argtypes = [P, P, P, P, ctypes.c_int32, P, P, P, P, P, P, P, F,
                                    I, I, I, I, I, I, P]
    L.hola_cache_update.restype = I
    L.kdn_scan_bwd_workspace_size.argtypes = [I, I, I, I, I]
    L.kdn_scan_bwd_workspace_size.restype = SZ
    L.kdn_scan_bwd.argtypes = [P] * 14 + [I] * 6 + [P, SZ, P]
    L.kdn_scan_bwd.restype = I
    L.kdn_scan_bwd_ex_workspace_size.argtypes = [I, I, I, I, I, I, I]
    L.kdn_scan_bwd_ex_workspace_size.restype = SZ
    L.kdn_scan_bwd_ex.argtypes = [P, P, P, P, I, P, P, P, P, F] + [P] * 11 + [I] * 7 + [P, SZ, P]
    L.kdn_scan_bwd_ex.restype = I
    L.hola_prefill_workspace_size.argtypes = [I, I, I, I, I, I, I]
    L.hola_prefill_workspace_size.restype = SZ
    L.hola_prefill.argtypes = [P, P, P, I, P, ctypes.c_int32, I, P, P, P, P, P, P, P, F,
                               I, I, I, I, I, I, I, P, SZ, P]
    L.hola_prefill.restype = I
    return L


lib = _load()


def kdn_status_string(status: int) -> str:
    return lib.kdn_status_string(int(status)).decode()


def kdn_scan_workspace_size(B, H, L, d_k, d_v, chunk, mode="delta", in_dtype=BF16,
                            with_scores: bool = False) -> int:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return int(lib.kdn_scan_workspace_size(B, H, L, d_k, d_v, chunk, m, in_dtype,
                                           1 if with_scores else 0))


# ----------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise ValueError(f"unsupported element type {dt}")


# ----------------------------------------------------------------- scan

def kdn_scan_fwd(q, k, v, alpha=None, beta=None, r=None, cov_in=None, cov_out=None,
                 q_noise_var: float = 0.0, state_in=None, state_out=None, o=None, out_dtype=None,
                 chunk: int = 64, mode: str = "delta", resid: str = "gated", workspace=None,
                 stream=None, phase: str = "all", m=None, score: str = "write"):
    """Chunkwise scan. q, k: [B,H,L,d_k]; v: [B,H,L,d_v] (bf16 or float32, same dtype);
    alpha/beta/r: [B,H,L] float32; cov_in/cov_out: [B,H,d_k] (diag), [B,H,d_k,d_k]
    (full) or [B,H] (iso) float32; state_in/state_out: [B,H,d_k,d_v] float32. Returns o [B,H,L,d_v]
    (float32 unless ``out_dtype`` or ``o`` says otherwise). ``phase`` "prepare" /
    "state" runs one half of the call (kdn_scan_fwd_phase); both halves must see
    the same ``workspace`` tensor. ``m`` ([B,H,L] float32 tensor, or True to
    allocate one) receives the write scores of kind ``score`` ("write", "resid",
    "value"); the call then returns (o, m)."""
    torch = _torch()
    _check(q, "q", (torch.bfloat16, torch.float32))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", q.dtype, (B, H, L, dk), dev)
    _check(v, "v", q.dtype, (B, H, L, dv), dev)
    for name, t in (("alpha", alpha), ("beta", beta), ("r", r)):
        _check(t, name, torch.float32, (B, H, L), dev)
    cshape = {"diag": (B, H, dk), "iso": (B, H)}.get(mode, (B, H, dk, dk))
    _check(cov_in, "cov_in", torch.float32, cshape, dev)
    _check(cov_out, "cov_out", torch.float32, cshape, dev)
    _check(state_in, "state_in", torch.float32, (B, H, dk, dv), dev)
    _check(state_out, "state_out", torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=out_dtype or torch.float32, device=dev)
    _check(o, "o", (torch.bfloat16, torch.float32), (B, H, L, dv), dev)
    in_code = _dtype_code(q.dtype)
    mcode, rcode = MODES[mode], RESIDS[resid]
    want_m = m is not None and m is not False
    if m is True:
        m = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    if want_m:
        _check(m, "m", torch.float32, (B, H, L), dev)
    need = int(lib.kdn_scan_workspace_size(B, H, L, dk, dv, chunk, mcode, in_code,
                                           1 if want_m else 0))
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if phase != "all" and need > 0 and wbytes < need:
        raise ValueError("a split scan needs the caller's workspace tensor")
    st = lib.kdn_scan_fwd_phase(PHASES[phase], _ptr(q), _ptr(k), _ptr(v), in_code, _ptr(alpha),
                                _ptr(beta), _ptr(r), _ptr(cov_in), _ptr(cov_out),
                                float(q_noise_var), _ptr(state_in), _ptr(state_out), _ptr(o),
                                _dtype_code(o.dtype), _ptr(m) if want_m else None, SCORES[score],
                                B, H, L, dk, dv, int(chunk), mcode, rcode, _ptr(workspace), wbytes,
                                _stream(stream))
    if st != 0:
        raise KdnError(st, "kdn_scan_fwd")
    return (o, m) if want_m else o


def kdn_scan_fwd_static(q, k, v, o, alpha=None, beta=None, r=None, cov_in=None, cov_out=None,
                        q_noise_var: float = 0.0, state_in=None, state_out=None, m=None,
                        chunk: int = 64, mode: str = "delta", resid: str = "gated", stream=None,
                        score: str = "write"):
    """kdn_scan_fwd on the library's static scratch (no workspace, nothing
    allocated here or in the library): every output, ``o`` and optionally
    ``m`` ([B,H,L] float32), ``state_out`` and ``cov_out``, is the caller's
    tensor. Same shapes and meaning as kdn_scan_fwd; calls on one GPU must not
    overlap (they share its scratch)."""
    torch = _torch()
    _check(q, "q", (torch.bfloat16, torch.float32))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", q.dtype, (B, H, L, dk), dev)
    _check(v, "v", q.dtype, (B, H, L, dv), dev)
    for name, t in (("alpha", alpha), ("beta", beta), ("r", r)):
        _check(t, name, torch.float32, (B, H, L), dev)
    cshape = {"diag": (B, H, dk), "iso": (B, H)}.get(mode, (B, H, dk, dk))
    _check(cov_in, "cov_in", torch.float32, cshape, dev)
    _check(cov_out, "cov_out", torch.float32, cshape, dev)
    _check(state_in, "state_in", torch.float32, (B, H, dk, dv), dev)
    _check(state_out, "state_out", torch.float32, (B, H, dk, dv), dev)
    _check(o, "o", (torch.bfloat16, torch.float32), (B, H, L, dv), dev)
    _check(m, "m", torch.float32, (B, H, L), dev)
    st = lib.kdn_scan_fwd_static(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(alpha),
                                 _ptr(beta), _ptr(r), _ptr(cov_in), _ptr(cov_out),
                                 float(q_noise_var), _ptr(state_in), _ptr(state_out), _ptr(o),
                                 _dtype_code(o.dtype), _ptr(m), SCORES[score], B, H, L, dk, dv,
                                 int(chunk), MODES[mode], RESIDS[resid], _stream(stream))
    if st != 0:
        raise KdnError(st, "kdn_scan_fwd_static")
    return o


# ----------------------------------------------------------------- decode

def kdn_step_decode(q, k, v, alpha, beta, state, o=None, m=None, r=None, cov=None,
                    q_noise_var: float = 0.0, mode: str = "delta", resid: str = "gated",
                    stream=None, score: str = "write"):
    """One token per head. q, k: [B,H,d_k]; v: [B,H,d_v]; alpha, beta, r: [B,H];
    state [B,H,d_k,d_v] and cov [B,H,d_k] (diag) or [B,H] (iso) are updated in place.
    Returns (o [B,H,d_v], m [B,H])."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    f = torch.float32
    _check(q, "q", f)
    _check(k, "k", f, (B, H, dk), dev)
    _check(v, "v", f, (B, H, dv), dev)
    _check(alpha, "alpha", f, (B, H), dev)
    _check(beta, "beta", f, (B, H), dev)
    _check(r, "r", f, (B, H), dev)
    _check(cov, "cov", f, (B, H) if mode == "iso" else (B, H, dk), dev)
    _check(state, "state", f, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=f, device=dev)
    if m is None:
        m = torch.empty((B, H), dtype=f, device=dev)
    _check(o, "o", f, (B, H, dv), dev)
    _check(m, "m", f, (B, H), dev)
    st = lib.kdn_step_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(r),
                             _ptr(cov), float(q_noise_var), _ptr(state), _ptr(o), _ptr(m),
                             SCORES[score], B, H, dk, dv, MODES[mode], RESIDS[resid],
                             _stream(stream))
    if st != 0:
        raise KdnError(st, "kdn_step_decode")
    return o, m


# ----------------------------------------------------------------- HOLA cache

class HolaCache:
    """Device tensors of a HOLA exact cache for [B, H] heads with capacity w."""

    def __init__(self, B: int, H: int, d_k: int, d_v: int, w: int = 64, device="cuda",
                 policy: str = "score"):
        torch = _torch()
        self.B, self.H, self.d_k, self.d_v, self.w = B, H, d_k, d_v, w
        self.policy = POLICIES[policy]
        self.k = torch.zeros((B, H, w, d_k), dtype=torch.float32, device=device)
        self.v = torch.zeros((B, H, w, d_v), dtype=torch.float32, device=device)
        self.m = torch.zeros((B, H, w), dtype=torch.float32, device=device)
        self.pos = torch.full((B, H, w), -1, dtype=torch.int32, device=device)
        self.count = torch.zeros((B, H), dtype=torch.int32, device=device)


def hola_cache_update(q, k, v, m, t: int, cache: HolaCache, sink_logit=None, o_cache=None,
                      rms_eps: float = 1e-6, stream=None):
    """Read over cache + current token (+ sink), then insert token t with score m.
    q, k: [B,H,d_k]; v: [B,H,d_v]; m: [B,H]; sink_logit: [H] or None.
    Returns o_cache [B,H,d_v]."""
    torch = _torch()
    B, H, dk, dv, w = cache.B, cache.H, cache.d_k, cache.d_v, cache.w
    f = torch.float32
    dev = cache.k.device
    _check(q, "q", f, (B, H, dk), dev)
    _check(k, "k", f, (B, H, dk), dev)
    _check(v, "v", f, (B, H, dv), dev)
    _check(m, "m", f, (B, H), dev)
    _check(sink_logit, "sink_logit", f, (H,), dev)
    if o_cache is None:
        o_cache = torch.empty((B, H, dv), dtype=f, device=dev)
    _check(o_cache, "o_cache", f, (B, H, dv), dev)
    st = lib.hola_cache_update(_ptr(q), _ptr(k), _ptr(v), _ptr(m), int(t), _ptr(cache.k),
                               _ptr(cache.v), _ptr(cache.m), _ptr(cache.pos), _ptr(cache.count),
                               _ptr(sink_logit), _ptr(o_cache), float(rms_eps), B, H, dk, dv, w,
                               cache.policy, _stream(stream))
    if st != 0:
        raise KdnError(st, "hola_cache_update")
    return o_cache


def hola_prefill(q, k, v, m, t0: int, cache: HolaCache, block: int = 256, sink_logit=None,
                 o_cache=None, rms_eps: float = 1e-6, workspace=None, stream=None):
    """The HOLA cache over a whole prompt in blocks of ``block`` tokens: each
    token reads the cache as it stood before its block, its block's tokens up to
    itself and the sink; then the block is inserted. q, k: [B,H,L,d_k]; v:
    [B,H,L,d_v] (bf16 or float32); m: [B,H,L] float32 scores; t0: position of
    token 0. Updates ``cache`` in place; returns o_cache [B,H,L,d_v] float32."""
    torch = _torch()
    B, H, dk, dv, w = cache.B, cache.H, cache.d_k, cache.d_v, cache.w
    dev = cache.k.device
    _check(q, "q", (torch.bfloat16, torch.float32))
    L = q.shape[2]
    _check(q, "q", q.dtype, (B, H, L, dk), dev)
    _check(k, "k", q.dtype, (B, H, L, dk), dev)
    _check(v, "v", q.dtype, (B, H, L, dv), dev)
    _check(m, "m", torch.float32, (B, H, L), dev)
    _check(sink_logit, "sink_logit", torch.float32, (H,), dev)
    if o_cache is None:
        o_cache = torch.empty((B, H, L, dv), dtype=torch.float32, device=dev)
    _check(o_cache, "o_cache", torch.float32, (B, H, L, dv), dev)
    need = int(lib.hola_prefill_workspace_size(B, H, max(L, 1), dk, dv, w, int(block)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.hola_prefill(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), _ptr(m), int(t0),
                          int(block), _ptr(cache.k), _ptr(cache.v), _ptr(cache.m),
                          _ptr(cache.pos), _ptr(cache.count), _ptr(sink_logit), _ptr(o_cache),
                          float(rms_eps), B, H, L, dk, dv, w, cache.policy, _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise KdnError(st, "hola_prefill")
    return o_cache


def hola_prefill_workspace_size(B, H, L, d_k, d_v, w, block) -> int:
    return int(lib.hola_prefill_workspace_size(B, H, L, d_k, d_v, w, block))


def kdn_scan_bwd(q, k, v, alpha, beta, d_o, state_in=None, dstate_out=None, resid: str = "gated",
                 workspace=None, stream=None, want_dstate: bool = True) -> dict:
    """Gradients of the delta-write scan for dL/do = d_o and dL/dS_L = dstate_out
    (float32 tensors, shapes as kdn_scan_fwd). Returns dict(dq, dk, dv, dalpha,
    dbeta, dstate_in)."""
    torch = _torch()
    f = torch.float32
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(q, "q", f, (B, H, L, dk), dev)
    _check(k, "k", f, (B, H, L, dk), dev)
    _check(v, "v", f, (B, H, L, dv), dev)
    _check(alpha, "alpha", f, (B, H, L), dev)
    _check(beta, "beta", f, (B, H, L), dev)
    _check(d_o, "d_o", f, (B, H, L, dv), dev)
    _check(state_in, "state_in", f, (B, H, dk, dv), dev)
    _check(dstate_out, "dstate_out", f, (B, H, dk, dv), dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dalpha=torch.empty((B, H, L), dtype=f, device=dev) if alpha is not None else None,
               dbeta=torch.empty((B, H, L), dtype=f, device=dev),
               dstate_in=torch.empty((B, H, dk, dv), dtype=f, device=dev) if want_dstate else None)
    need = int(lib.kdn_scan_bwd_workspace_size(B, H, max(L, 1), dk, dv))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.kdn_scan_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in),
                          _ptr(d_o), _ptr(dstate_out), _ptr(out["dq"]), _ptr(out["dk"]),
                          _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]),
                          _ptr(out["dstate_in"]), B, H, L, dk, dv, RESIDS[resid],
                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                          _stream(stream))
    if st != 0:
        raise KdnError(st, "kdn_scan_bwd")
    return out


def kdn_scan_bwd_ex(q, k, v, d_o, alpha=None, beta=None, r=None, cov_in=None,
                    q_noise_var: float = 0.0, state_in=None, dstate_out=None, dcov_out=None,
                    mode: str = "delta", resid: str = "gated", workspace=None, stream=None,
                    want_dstate: bool = True, want_dcov: bool = True) -> dict:
    """Gradients of the scan for every write mode but the full covariance
    (kdn_scan_bwd_ex): q, k, v, d_o float32 or bf16 (one dtype), the forward
    call's alpha, beta (delta), r, cov_in (Kalman) and state_in, and the
    gradients of the loss w.r.t. o (d_o), the final state and the final
    covariance. Returns float32 dict(dq, dk, dv, dalpha, dbeta, dr, dcov_in,
    dstate_in) (None where the mode has no such input)."""
    torch = _torch()
    f = torch.float32
    _check(q, "q", (torch.bfloat16, f))
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _check(k, "k", q.dtype, (B, H, L, dk), dev)
    _check(v, "v", q.dtype, (B, H, L, dv), dev)
    _check(d_o, "d_o", q.dtype, (B, H, L, dv), dev)
    for name, t in (("alpha", alpha), ("beta", beta), ("r", r)):
        _check(t, name, f, (B, H, L), dev)
    kalman = mode in ("diag", "iso")
    cshape = {"diag": (B, H, dk), "iso": (B, H)}.get(mode)
    if kalman:
        _check(cov_in, "cov_in", f, cshape, dev)
        _check(dcov_out, "dcov_out", f, cshape, dev)
    _check(state_in, "state_in", f, (B, H, dk, dv), dev)
    _check(dstate_out, "dstate_out", f, (B, H, dk, dv), dev)
    e = lambda shape: torch.empty(shape, dtype=f, device=dev)  # noqa: E731
    out = dict(dq=e((B, H, L, dk)), dk=e((B, H, L, dk)), dv=e((B, H, L, dv)),
               dalpha=e((B, H, L)) if alpha is not None else None,
               dbeta=e((B, H, L)) if mode == "delta" else None,
               dr=e((B, H, L)) if kalman and r is not None else None,
               dcov_in=e(cshape) if kalman and want_dcov else None,
               dstate_in=e((B, H, dk, dv)) if want_dstate else None)
    code = _dtype_code(q.dtype)
    need = int(lib.kdn_scan_bwd_ex_workspace_size(B, H, max(L, 1), dk, dv, MODES[mode], code))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.kdn_scan_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(d_o), code, _ptr(alpha), _ptr(beta),
                             _ptr(r), _ptr(cov_in), float(q_noise_var), _ptr(state_in),
                             _ptr(dstate_out), _ptr(dcov_out), _ptr(out["dq"]), _ptr(out["dk"]),
                             _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]),
                             _ptr(out["dr"]), _ptr(out["dcov_in"]), _ptr(out["dstate_in"]),
                             B, H, L, dk, dv, MODES[mode], RESIDS[resid], _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise KdnError(st, "kdn_scan_bwd_ex")
    return out
