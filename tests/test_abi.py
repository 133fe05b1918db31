"""The C-ABI library loads, exports exactly what include/kdn.h declares, and
rejects bad arguments with the documented status codes before touching a
device (these calls run on a machine without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdn.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def _header_constants():
    vals = {}
    for name, val in re.findall(r"#define\s+(KDN_[A-Z0-9_]+)\s+\(?(-?\d+)\)?", open(HEADER).read()):
        vals[name] = int(val)
    return vals


@pytest.fixture(scope="module")
def kdn():
    import delta_rule_scans_amd as k
    return k


def test_exports_match_header(kdn):
    declared = _header_functions()
    assert declared == sorted(["hola_cache_update", "hola_prefill", "hola_prefill_workspace_size",
                               "kdn_scan_bwd", "kdn_scan_bwd_workspace_size", "kdn_scan_bwd_ex",
                               "kdn_scan_bwd_ex_workspace_size", "kdn_scan_fwd",
                               "kdn_scan_fwd_phase", "kdn_scan_fwd_static", "kdn_scan_workspace_size",
                               "kdn_status_string", "kdn_step_decode", "kdn_version"])
    out = subprocess.run(["nm", "-D", "--defined-only", kdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines()
                      if " T " in line and not line.split()[-1].startswith("_"))
    assert exported == declared
    for name in declared:
        assert hasattr(kdn.lib, name)


def test_status_strings_and_constants(kdn):
    c = _header_constants()
    assert c["KDN_OK"] == 0
    codes = [v for k, v in c.items() if k.startswith("KDN_ERR_")]
    assert len(codes) == len(set(codes)) and all(v < 0 for v in codes)
    for v in codes:
        s = kdn.kdn_status_string(v)
        assert s and s != "unknown status"
    assert kdn.kdn_status_string(0) == "ok"
    assert kdn.lib.kdn_version() >= 100
    assert (c["KDN_GAIN_DELTA"], c["KDN_GAIN_DIAG"], c["KDN_GAIN_FULL"], c["KDN_GAIN_ISO"]) == (0, 1, 2, 3)
    assert [kdn.MODES[m] for m in ("delta", "diag", "full", "iso")] == [0, 1, 2, 3]


def test_workspace_size(kdn):
    assert kdn.kdn_scan_workspace_size(4, 16, 4096, 128, 128, 64, "delta", kdn.F32) == 0
    assert kdn.kdn_scan_workspace_size(4, 16, 4096, 128, 128, 32, "delta", kdn.BF16) == 0
    # matrix-core path, one record per (head, chunk): the three nonzero 32 x 32
    # fp16 blocks of (I + A)^-1 and three float4 scalars per token
    tinv = 4 * 16 * 64 * (3 * 32 * 32 * 2 + 64 * 48)
    assert kdn.kdn_scan_workspace_size(4, 16, 4096, 128, 128, 64, "delta", kdn.BF16) == tinv
    ws = kdn.kdn_scan_workspace_size(4, 16, 4096, 128, 128, 64, "diag", kdn.BF16)
    gains = 4 * 16 * 4096 * 128 * 2
    maps = 4 * 16 * 64 * 128 * 16
    assert ws >= gains + maps + tinv
    # isotropic write: per-token write strengths and key norms, one map per chunk
    iso = kdn.kdn_scan_workspace_size(4, 16, 4096, 128, 128, 64, "iso", kdn.BF16)
    assert iso == 4 * 16 * 64 * 16 + 2 * 4 * 16 * 4096 * 4 + tinv
    assert kdn.kdn_scan_workspace_size(1, 1, 64, 16, 16, 16, "full", kdn.F32) >= 64 * 16 * 4
    assert kdn.kdn_scan_workspace_size(1, 1, 64, 16, 16, 17, "full", kdn.F32) == 0


# Fake (never dereferenced) device addresses: every call below must be rejected
# by the host-side checks before any launch.
P = 0x10000


def _scan(kdn, **kw):
    a = dict(q=P, k=P, v=P, in_dtype=1, alpha=P, beta=P, r=None, cov_in=None, cov_out=None,
             qvar=0.0, state_in=None, state_out=None, o=P, out_dtype=1, m=None, sk=0, B=1, H=1, L=64, dk=128,
             dv=128, chunk=64, mode=0, resid=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return kdn.lib.kdn_scan_fwd(a["q"], a["k"], a["v"], a["in_dtype"], a["alpha"], a["beta"],
                                a["r"], a["cov_in"], a["cov_out"], a["qvar"], a["state_in"],
                                a["state_out"], a["o"], a["out_dtype"], a["m"], a["sk"], a["B"], a["H"], a["L"],
                                a["dk"], a["dv"], a["chunk"], a["mode"], a["resid"], a["ws"],
                                a["wsb"], a["stream"])


def test_scan_rejections(kdn):
    c = _header_constants()
    assert _scan(kdn, q=None) == c["KDN_ERR_NULL_POINTER"]
    assert _scan(kdn, o=None) == c["KDN_ERR_NULL_POINTER"]
    assert _scan(kdn, beta=None) == c["KDN_ERR_NULL_POINTER"]
    assert _scan(kdn, mode=1) == c["KDN_ERR_NULL_POINTER"]            # DIAG without cov_in
    assert _scan(kdn, in_dtype=7) == c["KDN_ERR_BAD_DTYPE"]
    assert _scan(kdn, out_dtype=-1) == c["KDN_ERR_BAD_DTYPE"]
    assert _scan(kdn, mode=3) == c["KDN_ERR_NULL_POINTER"]            # ISO without cov_in
    assert _scan(kdn, mode=4) == c["KDN_ERR_BAD_MODE"]
    assert _scan(kdn, mode=3, resid=1, cov_in=P) == c["KDN_ERR_BAD_MODE"]
    assert _scan(kdn, mode=3, cov_in=P) == c["KDN_ERR_WORKSPACE"]
    assert _scan(kdn, mode=1, resid=1, cov_in=P) == c["KDN_ERR_BAD_MODE"]
    for bad in (dict(B=0), dict(H=-1), dict(L=-1), dict(dk=0), dict(dv=129), dict(dk=256)):
        assert _scan(kdn, **bad) == c["KDN_ERR_BAD_SHAPE"], bad
    assert _scan(kdn, qvar=-1.0) == c["KDN_ERR_BAD_SHAPE"]
    assert _scan(kdn, qvar=float("nan")) == c["KDN_ERR_BAD_SHAPE"]
    for ch in (0, 8, 17, 96, 256):
        assert _scan(kdn, chunk=ch) == c["KDN_ERR_BAD_CHUNK"], ch
    # chunk 128 is taken, and runs as 64-token chunks: the same workspace
    for mode in ("delta", "diag", "iso"):
        for dt in (kdn.F32, kdn.BF16):
            assert kdn.kdn_scan_workspace_size(2, 3, 1000, 128, 128, 128, mode, dt, True) == \
                kdn.kdn_scan_workspace_size(2, 3, 1000, 128, 128, 64, mode, dt, True)
    assert _scan(kdn, mode=2, cov_in=P, dk=128) == c["KDN_ERR_UNSUPPORTED"]
    assert _scan(kdn, mode=2, cov_in=P, dk=64) == c["KDN_ERR_WORKSPACE"]
    # an unknown phase is rejected like an unknown mode
    assert kdn.lib.kdn_scan_fwd_phase(3, P, P, P, 1, P, P, None, None, None, 0.0, None, None, P, 1,
                                      None, 0, 1, 1, 64, 128, 128, 64, 0, 0, None, 0, None) == c["KDN_ERR_BAD_MODE"]
    # residual forms other than the gated one take the delta write only; scores 0..2
    assert _scan(kdn, resid=3) == c["KDN_ERR_BAD_MODE"]
    assert _scan(kdn, resid=2, mode=1, cov_in=P) == c["KDN_ERR_BAD_MODE"]
    assert _scan(kdn, m=P, sk=3) == c["KDN_ERR_BAD_MODE"]
    # scores need the larger workspace
    base = kdn.kdn_scan_workspace_size(1, 1, 64, 128, 128, 64, "delta", kdn.BF16)
    big = kdn.kdn_scan_workspace_size(1, 1, 64, 128, 128, 64, "delta", kdn.BF16, with_scores=True)
    assert big >= base + 64 * 128 * 2
    assert _scan(kdn, m=P, ws=P, wsb=base) == c["KDN_ERR_WORKSPACE"]
    need = kdn.kdn_scan_workspace_size(1, 1, 64, 128, 128, 64, "diag", kdn.BF16)
    assert _scan(kdn, mode=1, cov_in=P, ws=P, wsb=need - 1) == c["KDN_ERR_WORKSPACE"]
    assert _scan(kdn, mode=1, cov_in=P, ws=P + 4, wsb=need) == c["KDN_ERR_WORKSPACE"]


def _decode(kdn, **kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, r=None, cov=None, qvar=0.0, state=P, o=P, m=P, sk=0,
             B=2, H=2, dk=128, dv=128, mode=0, resid=0, stream=None)
    a.update(kw)
    return kdn.lib.kdn_step_decode(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["r"],
                                   a["cov"], a["qvar"], a["state"], a["o"], a["m"], a["sk"],
                                   a["B"], a["H"], a["dk"], a["dv"], a["mode"], a["resid"],
                                   a["stream"])


def test_decode_rejections(kdn):
    c = _header_constants()
    assert _decode(kdn, state=None) == c["KDN_ERR_NULL_POINTER"]
    assert _decode(kdn, beta=None) == c["KDN_ERR_NULL_POINTER"]
    assert _decode(kdn, mode=1) == c["KDN_ERR_NULL_POINTER"]
    assert _decode(kdn, mode=2) == c["KDN_ERR_UNSUPPORTED"]
    assert _decode(kdn, mode=3) == c["KDN_ERR_NULL_POINTER"]
    assert _decode(kdn, mode=3, resid=1, cov=P) == c["KDN_ERR_BAD_MODE"]
    assert _decode(kdn, mode=5) == c["KDN_ERR_BAD_MODE"]
    assert _decode(kdn, sk=5) == c["KDN_ERR_BAD_MODE"]
    assert _decode(kdn, resid=2, mode=3, cov=P) == c["KDN_ERR_BAD_MODE"]
    assert _decode(kdn, mode=1, resid=1, cov=P) == c["KDN_ERR_BAD_MODE"]
    assert _decode(kdn, dk=0) == c["KDN_ERR_BAD_SHAPE"]
    assert _decode(kdn, dv=200) == c["KDN_ERR_BAD_SHAPE"]
    assert _decode(kdn, B=0) == c["KDN_ERR_BAD_SHAPE"]


def _hola(kdn, **kw):
    a = dict(q=P, k=P, v=P, m=P, t=0, ck=P, cv=P, cm=P, cp=P, cc=P, sink=None, oc=P, eps=1e-6,
             B=1, H=1, dk=128, dv=128, w=64, policy=0, stream=None)
    a.update(kw)
    return kdn.lib.hola_cache_update(a["q"], a["k"], a["v"], a["m"], a["t"], a["ck"], a["cv"],
                                     a["cm"], a["cp"], a["cc"], a["sink"], a["oc"], a["eps"],
                                     a["B"], a["H"], a["dk"], a["dv"], a["w"], a["policy"],
                                     a["stream"])


def test_hola_rejections(kdn):
    c = _header_constants()
    for w in (0, -3, 257, 1024):
        assert _hola(kdn, w=w) == c["KDN_ERR_BAD_CAPACITY"]
    assert _hola(kdn, cc=None) == c["KDN_ERR_NULL_POINTER"]
    assert _hola(kdn, m=None) == c["KDN_ERR_NULL_POINTER"]
    assert _hola(kdn, dk=129) == c["KDN_ERR_BAD_SHAPE"]
    assert _hola(kdn, eps=-1.0) == c["KDN_ERR_BAD_SHAPE"]
    assert _hola(kdn, eps=float("nan")) == c["KDN_ERR_BAD_SHAPE"]
    assert _hola(kdn, policy=2) == c["KDN_ERR_BAD_MODE"]


def test_product_package_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "delta_rule_scans_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def _prefill(kdn, **kw):
    a = dict(q=P, k=P, v=P, dt=1, m=P, t0=0, block=256, ck=P, cv=P, cm=P, cp=P, cc=P, sink=None,
             oc=P, eps=1e-6, B=1, H=1, L=512, dk=128, dv=128, w=64, policy=0, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return kdn.lib.hola_prefill(a["q"], a["k"], a["v"], a["dt"], a["m"], a["t0"], a["block"],
                                a["ck"], a["cv"], a["cm"], a["cp"], a["cc"], a["sink"], a["oc"],
                                a["eps"], a["B"], a["H"], a["L"], a["dk"], a["dv"], a["w"],
                                a["policy"], a["ws"], a["wsb"], a["stream"])


def test_prefill_rejections(kdn):
    c = _header_constants()
    need = kdn.hola_prefill_workspace_size(1, 1, 512, 128, 128, 64, 256)
    # members per block, final cache and a staging copy of the final rows
    assert need >= 2 * 64 * 4 + 64 * 256 * 4
    assert kdn.hola_prefill_workspace_size(1, 1, 512, 128, 128, 0, 256) == 0
    assert _prefill(kdn, dt=3) == c["KDN_ERR_BAD_DTYPE"]
    for w in (0, 257):
        assert _prefill(kdn, w=w) == c["KDN_ERR_BAD_CAPACITY"]
    for bad in (dict(block=0), dict(block=1025), dict(L=-1), dict(dk=129), dict(B=0),
                dict(eps=-1.0), dict(t0=2 ** 31 - 100)):
        assert _prefill(kdn, **bad) == c["KDN_ERR_BAD_SHAPE"], bad
    assert _prefill(kdn, policy=-1) == c["KDN_ERR_BAD_MODE"]
    assert _prefill(kdn, cc=None) == c["KDN_ERR_NULL_POINTER"]
    assert _prefill(kdn, m=None) == c["KDN_ERR_NULL_POINTER"]
    assert _prefill(kdn, L=0, m=None) == c["KDN_OK"]          # nothing to do, nothing touched
    assert _prefill(kdn) == c["KDN_ERR_WORKSPACE"]
    assert _prefill(kdn, ws=P, wsb=need - 1) == c["KDN_ERR_WORKSPACE"]
    assert _prefill(kdn, ws=P + 8, wsb=need) == c["KDN_ERR_WORKSPACE"]


def _bwd(kdn, **kw):
    a = dict(q=P, k=P, v=P, alpha=P, beta=P, s0=None, do=P, dso=None, dq=P, dk=P, dv=P, da=P, db=P,
             ds0=None, B=1, H=1, L=64, dk_=128, dv_=128, resid=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return kdn.lib.kdn_scan_bwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["s0"], a["do"],
                                a["dso"], a["dq"], a["dk"], a["dv"], a["da"], a["db"], a["ds0"],
                                a["B"], a["H"], a["L"], a["dk_"], a["dv_"], a["resid"], a["ws"],
                                a["wsb"], a["stream"])


def test_backward_rejections(kdn):
    c = _header_constants()
    need = kdn.lib.kdn_scan_bwd_workspace_size(1, 1, 64, 128, 128)
    # one 64-token chunk: its start state and end-state gradient, residuals and
    # their gradients, three [64, d_k] contractions, five 64 x 64 chunk matrices
    assert need >= 4 * (2 * 128 * 128 + 2 * 64 * 128 + 3 * 64 * 128 + 5 * 64 * 64)
    assert _bwd(kdn, resid=3) == c["KDN_ERR_BAD_MODE"]
    assert _bwd(kdn, dk_=129) == c["KDN_ERR_BAD_SHAPE"]
    assert _bwd(kdn, L=-1) == c["KDN_ERR_BAD_SHAPE"]
    # one workgroup row per 64-token chunk: at most 65535 chunks
    assert _bwd(kdn, L=65536 * 64) == c["KDN_ERR_BAD_SHAPE"]
    assert _bwd(kdn, L=65535 * 64) == c["KDN_ERR_WORKSPACE"]  # passes the shape checks
    assert _bwd(kdn, do=None) == c["KDN_ERR_NULL_POINTER"]
    assert _bwd(kdn, da=None) == c["KDN_ERR_NULL_POINTER"]
    assert _bwd(kdn) == c["KDN_ERR_WORKSPACE"]
    assert _bwd(kdn, ws=P, wsb=need - 1) == c["KDN_ERR_WORKSPACE"]


def test_static_scratch_entry_rejects_before_any_hip_call(kdn):
    """kdn_scan_fwd_static (the allocation-free scan) checks its arguments and
    its scratch limit before any HIP call, so on a machine without a GPU it
    returns the documented codes: a null pointer, a bad chunk, and a call that
    needs more workspace than KDN_STATIC_SCRATCH_BYTES."""
    c = _header_constants()
    assert kdn.STATIC_SCRATCH_BYTES == 64 << 20
    fake = ctypes.c_void_p(1 << 40)      # never dereferenced: every call is rejected first
    lib = kdn.lib

    def call(q, B, H, L, chunk=64, mode=0, m=None, beta=fake):
        return lib.kdn_scan_fwd_static(q, fake, fake, kdn.BF16, None, beta, None, fake, None,
                                       0.0, None, None, fake, kdn.F32, m, 0, B, H, L, 128, 128,
                                       chunk, mode, 0, None)

    assert call(None, 1, 1, 64) == c["KDN_ERR_NULL_POINTER"]
    assert call(fake, 1, 1, 64, chunk=48) == c["KDN_ERR_BAD_CHUNK"]
    assert call(fake, 1, 1, 64, beta=None) == c["KDN_ERR_NULL_POINTER"]
    # B*H = 64, L = 4096 (the gated workload): the delta write fits, with scores or as
    # the diagonal Kalman write it does not
    fits = kdn.kdn_scan_workspace_size(4, 16, 4096, 128, 128, 64, "delta", kdn.BF16)
    assert 0 < fits <= kdn.STATIC_SCRATCH_BYTES
    assert kdn.kdn_scan_workspace_size(4, 16, 4096, 128, 128, 64, "diag", kdn.BF16) > kdn.STATIC_SCRATCH_BYTES
    assert call(fake, 4, 16, 4096, mode=1) == c["KDN_ERR_SCRATCH_LIMIT"]
    assert call(fake, 4, 16, 4096, m=fake) == c["KDN_ERR_SCRATCH_LIMIT"]
    assert call(fake, 8, 16, 4096) == c["KDN_ERR_SCRATCH_LIMIT"]
