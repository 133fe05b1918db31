"""GPU parity of kdn_scan_fwd against the fp64 oracle (element by element).

Small cases span several chunks and a ragged tail; the full-size workloads are
run exactly as the benchmark launches them and checked on sampled heads, each
of which the oracle recomputes over the whole sequence.
"""
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


def _scan_gpu(kdn, inp, dtype, chunk, mode="delta", resid="gated", cov0=None, qvar=0.0, S0=None,
              out_dtype=None, want_state=True):
    import torch
    q, k, v = (dev_tensor(inp[n], dtype) for n in ("q", "k", "v"))
    B, H, L, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    alpha = dev_tensor(inp["alpha"])
    beta = dev_tensor(inp["beta"])
    r = dev_tensor(inp["r"]) if inp.get("r") is not None else None
    cov_in = dev_tensor(cov0) if cov0 is not None else None
    cov_out = torch.empty_like(cov_in) if cov0 is not None else None
    s_in = dev_tensor(S0) if S0 is not None else None
    s_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda") if want_state else None
    od = {"f32": torch.float32, "bf16": torch.bfloat16, None: None}[out_dtype]
    o = kdn.kdn_scan_fwd(q, k, v, alpha=alpha, beta=beta, r=r, cov_in=cov_in, cov_out=cov_out,
                         q_noise_var=qvar, state_in=s_in, state_out=s_out, out_dtype=od,
                         chunk=chunk, mode=mode, resid=resid)
    torch.cuda.synchronize()
    return dict(o=host(o), S=host(s_out) if want_state else None,
                cov=host(cov_out) if cov_out is not None else None)


def test_tiny_fp32_delta_and_rls(kdn, orc):
    """The tiny float32 workload: delta rule and full-covariance RLS (eps = 1e-2),
    the latter also against the closed-form ridge solution (DeltaNet-PC, eqs. 6-7)."""
    inp = workloads.named_scan_inputs("tiny")
    log("tiny f32 delta")
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    for chunk in (16, 32, 64):
        got = _scan_gpu(kdn, inp, "f32", chunk)
        assert_close(got["o"], ref["o"], TOL_F32, f"delta o chunk {chunk}")
        assert_close(got["S"], ref["S"], TOL_F32, f"delta S chunk {chunk}")
    log("tiny f32 rls")
    eps = 1e-2
    dk = inp["q"].shape[-1]
    P0 = (np.eye(dk) / eps)[None, None].astype(np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], cov0=P0, mode="full")
    got = _scan_gpu(kdn, inp, "f32", 16, mode="full", cov0=P0)
    assert_close(got["o"], ref["o"], TOL_F32, "rls o")
    assert_close(got["S"], ref["S"], TOL_F32, "rls S")
    assert_close(got["cov"], ref["cov"], TOL_F32, "rls P")
    K = inp["k"][0, 0].astype(np.float64)
    V = inp["v"][0, 0].astype(np.float64)
    ridge = np.linalg.solve(K.T @ K + eps * np.eye(dk), K.T @ V)
    assert_close(got["S"][0, 0], ridge, TOL_F32, "rls S vs ridge")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_delta_small(kdn, orc, dtype):
    inp = workloads.scan_inputs(2, 3, 300, 128, 128, seed=101, dtype=dtype)
    S0 = np.random.Generator(np.random.PCG64(101)).standard_normal((2, 3, 128, 128)).astype(np.float32) * 0.1
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], S0=S0)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for chunk in (16, 32, 64):
        log(f"gated {dtype} chunk {chunk}")
        got = _scan_gpu(kdn, inp, dtype, chunk, S0=S0)
        assert_close(got["o"], ref["o"], tol, f"o chunk {chunk}")
        assert_close(got["S"], ref["S"], tol, f"S chunk {chunk}")
    # bf16 output: exactly the float32 result rounded to nearest even
    f32 = _scan_gpu(kdn, inp, dtype, 64, S0=S0, out_dtype="f32", want_state=False)
    b16 = _scan_gpu(kdn, inp, dtype, 64, S0=S0, out_dtype="bf16", want_state=False)
    np.testing.assert_array_equal(b16["o"], workloads.bf16_round(f32["o"].astype(np.float32)))


def test_odd_shapes_fp32(kdn, orc):
    inp = workloads.scan_inputs(1, 2, 77, 24, 40, seed=102, dtype="f32")
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    for chunk in (16, 64):
        got = _scan_gpu(kdn, inp, "f32", chunk)
        assert_close(got["o"], ref["o"], TOL_F32, f"o chunk {chunk}")
        assert_close(got["S"], ref["S"], TOL_F32, f"S chunk {chunk}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plain_residual(kdn, orc, dtype):
    inp = workloads.scan_inputs(1, 2, 200, 128, 64, seed=103, dtype=dtype)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], resid="plain")
    got = _scan_gpu(kdn, inp, dtype, 64, resid="plain")
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_close(got["o"], ref["o"], tol, "plain o")
    assert_close(got["S"], ref["S"], tol, "plain S")


def test_short_sequences(kdn, orc):
    """Lengths of one token, a partial chunk, exactly one and two chunks and one
    past them, on the matrix-core path with B*H = 8 (the XCD-aware block order),
    with and without a final state."""
    for L in (1, 5, 63, 64, 65, 128, 129):
        log(f"short L {L}")
        inp = workloads.scan_inputs(2, 4, L, 128, 128, seed=110 + L, dtype="bf16")
        ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
        got = _scan_gpu(kdn, inp, "bf16", 64, want_state=L % 2 == 1)
        assert_close(got["o"], ref["o"], TOL_BF16, f"o L {L}")
        if got["S"] is not None:
            assert_close(got["S"], ref["S"], TOL_BF16, f"S L {L}")


@pytest.mark.parametrize("mode", ["delta", "diag"])
def test_grouped_prepare(kdn, orc, mode):
    """Enough (head, chunk) pairs that the prepare step hands each workgroup
    several consecutive chunks (here 4), with a chunk count the group size does
    not divide and a ragged last chunk: B=2, H=32, L=4100 is 65 chunks, the
    last of 4 tokens. The delta write and the diagonal Kalman write (which also
    stages Q and the gains); the oracle on sampled heads."""
    B, H, L, d = 2, 32, 4100, 128
    diag = mode == "diag"
    inp = workloads.scan_inputs(B, H, L, d, d, seed=111, dtype="bf16", with_r=diag)
    cov0 = np.ones((B, H, d), np.float32) if diag else None
    got = _scan_gpu(kdn, inp, "bf16", 64, mode=mode, cov0=cov0, qvar=1.0 if diag else 0.0)
    for (b, h) in [(0, 0), (1, 17), (1, 31)]:
        log(f"grouped prepare {mode}: oracle on head ({b}, {h})")
        sub = {n: (x[b:b + 1, h:h + 1] if x is not None else None) for n, x in inp.items()}
        ref = orc.scan(sub["q"], sub["k"], sub["v"], alpha=sub["alpha"], beta=sub["beta"],
                       r=sub["r"], cov0=None if cov0 is None else cov0[b:b + 1, h:h + 1],
                       q_noise_var=1.0 if diag else 0.0, mode=mode, want_m=False)
        assert_close(got["o"][b:b + 1, h:h + 1], ref["o"], TOL_BF16, f"{mode} o head {(b, h)}")
        assert_close(got["S"][b:b + 1, h:h + 1], ref["S"], TOL_BF16, f"{mode} S head {(b, h)}")
        if diag:
            assert_close(got["cov"][b:b + 1, h:h + 1], ref["cov"], TOL_F32, f"p head {(b, h)}")


@pytest.mark.parametrize("dv", [32, 96])
def test_value_slices(kdn, orc, dv):
    """d_v of one and of three 32-column slices on the matrix-core path, with
    B*H = 16 (the XCD-aware block order with a slice count other than 4)."""
    inp = workloads.scan_inputs(2, 8, 200, 128, dv, seed=113 + dv, dtype="bf16")
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    got = _scan_gpu(kdn, inp, "bf16", 64)
    assert_close(got["o"], ref["o"], TOL_BF16, f"o d_v {dv}")
    assert_close(got["S"], ref["S"], TOL_BF16, f"S d_v {dv}")


def test_misaligned_buffers(kdn, orc):
    """bf16 q, k, v and the output as views at a one-element offset (2 bytes:
    not 16-byte aligned): the matrix-core kernels need 16-byte rows, so these
    run on the general float32 kernel. Same oracle bar, and the output agrees
    with the aligned run to the bf16 tolerance."""
    import torch
    B, H, L, d = 1, 2, 130, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=112, dtype="bf16")
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        view = buf[1:].view(t.shape)
        view.copy_(t)
        return view

    q, k, v = (shifted(dev_tensor(inp[n], "bf16")) for n in ("q", "k", "v"))
    o = shifted(torch.zeros((B, H, L, d), dtype=torch.float32, device="cuda"))
    assert all(t.data_ptr() % 16 != 0 for t in (q, k, v, o))
    S = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                     state_out=S, o=o)
    torch.cuda.synchronize()
    assert_close(host(o), ref["o"], TOL_BF16, "misaligned o")
    assert_close(host(S), ref["S"], TOL_BF16, "misaligned S")
    aligned = _scan_gpu(kdn, inp, "bf16", 64)
    assert_close(host(o), aligned["o"], TOL_BF16, "misaligned vs aligned o")


@pytest.mark.parametrize("mode", ["diag", "iso"])
def test_split_sequence_resume_kalman(kdn, orc, mode):
    """The Kalman writes resumed from the returned state and covariance: [0, L)
    against [0, L1) then [L1, L), both split points inside a chunk."""
    B, H, L, L1, d = 1, 2, 333, 130, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=105, dtype="bf16", with_r=True)
    cov0 = np.ones((B, H, d) if mode == "diag" else (B, H), np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=cov0,
                   q_noise_var=1.0, mode=mode)
    first = {n: (x[:, :, :L1] if x is not None else None) for n, x in inp.items()}
    second = {n: (x[:, :, L1:] if x is not None else None) for n, x in inp.items()}
    a = _scan_gpu(kdn, first, "bf16", 64, mode=mode, cov0=cov0, qvar=1.0)
    b = _scan_gpu(kdn, second, "bf16", 64, mode=mode, cov0=a["cov"].astype(np.float32), qvar=1.0,
                  S0=a["S"].astype(np.float32))
    assert_close(np.concatenate([a["o"], b["o"]], 2), ref["o"], TOL_BF16, f"{mode} resumed o")
    assert_close(b["S"], ref["S"], TOL_BF16, f"{mode} resumed S")
    assert_close(b["cov"], ref["cov"], TOL_F32, f"{mode} resumed p")


@pytest.mark.parametrize("mode", ["delta", "diag"])
def test_phases_on_two_streams(kdn, mode):
    """kdn_scan_fwd_phase: the state-independent part enqueued on a second
    stream, the state scan on the first after an event, one caller workspace:
    the same outputs, state and covariance as one kdn_scan_fwd call, bit for bit."""
    import torch
    B, H, L, d = 2, 4, 300, 128
    diag = mode == "diag"
    inp = workloads.scan_inputs(B, H, L, d, d, seed=114, dtype="bf16", with_r=diag)
    q, k, v = (dev_tensor(inp[n], "bf16") for n in ("q", "k", "v"))
    alpha, beta = dev_tensor(inp["alpha"]), dev_tensor(inp["beta"])
    r = dev_tensor(inp["r"]) if diag else None
    kw = dict(alpha=alpha, beta=beta, r=r, mode=mode, q_noise_var=1.0 if diag else 0.0)
    cov0 = torch.ones((B, H, d), device="cuda") if diag else None

    def fresh():
        return (torch.empty((B, H, d, d), device="cuda"),
                torch.empty_like(cov0) if diag else None)

    S1, c1 = fresh()
    o1 = kdn.kdn_scan_fwd(q, k, v, state_out=S1, cov_in=cov0, cov_out=c1, **kw)
    need = kdn.kdn_scan_workspace_size(B, H, L, d, d, 64, mode=mode)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    S2, c2 = fresh()
    o2 = torch.empty_like(o1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    done = torch.cuda.Event()
    with torch.cuda.stream(side):
        kdn.kdn_scan_fwd(q, k, v, state_out=S2, cov_in=cov0, cov_out=c2, o=o2, workspace=ws,
                         phase="prepare", stream=side, **kw)
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    kdn.kdn_scan_fwd(q, k, v, state_out=S2, cov_in=cov0, cov_out=c2, o=o2, workspace=ws,
                     phase="state", **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(S1, S2)
    if diag:
        assert torch.equal(c1, c2)


def test_split_sequence_resume(kdn, orc):
    """Scanning [0, L) equals scanning [0, L1) and resuming [L1, L) from the
    returned state."""
    inp = workloads.scan_inputs(1, 2, 333, 128, 128, seed=104, dtype="bf16")
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    L1 = 130
    first = {n: (x[:, :, :L1] if x is not None else None) for n, x in inp.items()}
    second = {n: (x[:, :, L1:] if x is not None else None) for n, x in inp.items()}
    a = _scan_gpu(kdn, first, "bf16", 64)
    b = _scan_gpu(kdn, second, "bf16", 64, S0=a["S"].astype(np.float32))
    assert_close(np.concatenate([a["o"], b["o"]], 2), ref["o"], TOL_BF16, "resumed o")
    assert_close(b["S"], ref["S"], TOL_BF16, "resumed S")


def test_exact_recall_standard_basis_bitexact(kdn):
    """beta = 1, alpha = 1, distinct standard-basis keys: each write stores v_t
    exactly and a query equal to a stored key reads it back exactly (the
    delta rule's exact-recall case; A Hippocampus for Linear Attention, sec. 3.3)."""
    import torch
    d, L = 128, 128
    rng = np.random.Generator(np.random.PCG64(105))
    perm = rng.permutation(d)
    k = np.eye(d, dtype=np.float32)[perm][None, None]
    v = workloads.bf16_round(rng.standard_normal((1, 1, L, d)).astype(np.float32))
    inp = dict(q=k.copy(), k=k, v=v, alpha=np.ones((1, 1, L), np.float32),
               beta=np.ones((1, 1, L), np.float32))
    for dtype in ("bf16", "f32"):
        got = _scan_gpu(kdn, inp, dtype, 64, out_dtype="f32")
        np.testing.assert_array_equal(got["o"], v.astype(np.float64))
        recall = k[0, 0].astype(np.float64) @ got["S"][0, 0]
        np.testing.assert_array_equal(recall, v[0, 0].astype(np.float64))


def test_noop_write_keeps_state(kdn, orc):
    inp = workloads.scan_inputs(1, 2, 100, 128, 128, seed=106, dtype="bf16")
    inp["alpha"] = np.ones_like(inp["alpha"])
    inp["beta"] = np.zeros_like(inp["beta"])
    S0 = np.random.Generator(np.random.PCG64(106)).standard_normal((1, 2, 128, 128)).astype(np.float32)
    got = _scan_gpu(kdn, inp, "bf16", 64, S0=S0)
    np.testing.assert_array_equal(got["S"], S0.astype(np.float64))
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], S0=S0)
    assert_close(got["o"], ref["o"], TOL_BF16, "no-op o")


def test_zero_length(kdn):
    import torch
    S0 = torch.randn(2, 2, 128, 64, device="cuda")
    Sout = torch.empty_like(S0)
    q = torch.empty(2, 2, 0, 128, device="cuda", dtype=torch.bfloat16)
    v = torch.empty(2, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    a = torch.empty(2, 2, 0, device="cuda")
    kdn.kdn_scan_fwd(q, q, v, alpha=a, beta=a, state_in=S0, state_out=Sout)
    torch.cuda.synchronize()
    assert torch.equal(S0, Sout)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_diag_kalman_small(kdn, orc, dtype):
    inp = workloads.scan_inputs(2, 2, 260, 128, 128, seed=107, dtype=dtype, with_r=True)
    p0 = np.full((2, 2, 128), 1.0, np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=1.0, mode="diag")
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for chunk in (32, 64):
        log(f"diag {dtype} chunk {chunk}")
        got = _scan_gpu(kdn, inp, dtype, chunk, mode="diag", cov0=p0, qvar=1.0)
        assert_close(got["o"], ref["o"], tol, "diag o")
        assert_close(got["S"], ref["S"], tol, "diag S")
        assert_close(got["cov"], ref["cov"], TOL_F32, "diag p")
    # bf16 output (the Kalman form of the output stores): exactly the float32
    # result rounded to nearest even
    f32 = _scan_gpu(kdn, inp, dtype, 64, mode="diag", cov0=p0, qvar=1.0, out_dtype="f32", want_state=False)
    b16 = _scan_gpu(kdn, inp, dtype, 64, mode="diag", cov0=p0, qvar=1.0, out_dtype="bf16", want_state=False)
    np.testing.assert_array_equal(b16["o"], workloads.bf16_round(f32["o"].astype(np.float32)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_iso_kalman_small(kdn, orc, dtype):
    """Isotropic Kalman write (one variance per head), keys of varying norm."""
    inp = workloads.scan_inputs(2, 2, 260, 128, 128, seed=109, dtype=dtype, with_r=True)
    scale = np.random.Generator(np.random.PCG64(109)).uniform(0.5, 1.5, (2, 2, 260, 1))
    inp["k"] = inp["k"] * scale.astype(np.float32)
    if dtype == "bf16":
        inp["k"] = workloads.bf16_round(inp["k"])
    p0 = np.array([[0.5, 1.0], [2.0, 1.0]], np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=1.0, mode="iso")
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for chunk in (16, 64):
        log(f"iso {dtype} chunk {chunk}")
        got = _scan_gpu(kdn, inp, dtype, chunk, mode="iso", cov0=p0, qvar=1.0)
        assert_close(got["o"], ref["o"], tol, "iso o")
        assert_close(got["S"], ref["S"], tol, "iso S")
        assert_close(got["cov"], ref["cov"], TOL_F32, "iso p")


def test_full_kalman_small(kdn, orc):
    inp = workloads.scan_inputs(1, 2, 150, 32, 48, seed=108, dtype="f32", with_r=True)
    rng = np.random.Generator(np.random.PCG64(108))
    A = rng.standard_normal((1, 2, 32, 32))
    P0 = (np.einsum("bhij,bhkj->bhik", A, A) / 32 + np.eye(32)).astype(np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=P0,
                   q_noise_var=0.5, mode="full")
    got = _scan_gpu(kdn, inp, "f32", 32, mode="full", cov0=P0, qvar=0.5)
    assert_close(got["o"], ref["o"], TOL_F32, "full o")
    assert_close(got["S"], ref["S"], TOL_F32, "full S")
    assert_close(got["cov"], ref["cov"], TOL_F32, "full P")


def test_full_kalman_largest_dk(kdn, orc):
    """Full covariance at the largest d_k it takes (64), bf16 inputs, chunk 64,
    a random positive-definite initial covariance."""
    inp = workloads.scan_inputs(1, 2, 130, 64, 64, seed=109, dtype="bf16", with_r=True)
    rng = np.random.Generator(np.random.PCG64(109))
    A = rng.standard_normal((1, 2, 64, 64))
    P0 = (np.einsum("bhij,bhkj->bhik", A, A) / 64 + np.eye(64)).astype(np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=P0,
                   q_noise_var=0.5, mode="full")
    got = _scan_gpu(kdn, inp, "bf16", 64, mode="full", cov0=P0, qvar=0.5)
    assert_close(got["o"], ref["o"], TOL_BF16, "full o")
    assert_close(got["S"], ref["S"], TOL_BF16, "full S")
    assert_close(got["cov"], ref["cov"], TOL_F32, "full P")


@pytest.mark.parametrize("mode,resid,dtype,dk", [("delta", "gated", "bf16", 128),
                                                 ("delta", "gated", "f32", 128),
                                                 ("delta", "plain", "bf16", 128),
                                                 ("diag", "gated", "bf16", 128),
                                                 ("iso", "gated", "f32", 64),
                                                 ("full", "gated", "f32", 32)])
def test_write_scores(kdn, orc, mode, resid, dtype, dk):
    """Per-token write scores m_t = ||b_t e_t^T||_F (A Hippocampus for Linear
    Attention, sec. 3.3 eq. (6)) emitted by the scan, against the oracle's."""
    import torch
    inp = workloads.scan_inputs(2, 2, 200, dk, 64, seed=110, dtype=dtype, with_r=True)
    cov0 = {"diag": np.ones((2, 2, dk), np.float32), "iso": np.ones((2, 2), np.float32),
            "full": np.broadcast_to(np.eye(dk, dtype=np.float32), (2, 2, dk, dk)).copy()}.get(mode)
    qvar = 0.5 if mode != "delta" else 0.0
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"],
                   r=inp["r"] if mode != "delta" else None, cov0=cov0, q_noise_var=qvar,
                   mode=mode, resid=resid)
    q, k, v = (dev_tensor(inp[n], dtype) for n in ("q", "k", "v"))
    cin = dev_tensor(cov0) if cov0 is not None else None
    cout = torch.empty_like(cin) if cin is not None else None
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for chunk in ((64,) if dtype == "bf16" else (32, 64)):
        log(f"scores {mode}/{resid} {dtype} chunk {chunk}")
        o, m = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                                r=dev_tensor(inp["r"]) if mode != "delta" else None, cov_in=cin,
                                cov_out=cout, q_noise_var=qvar, chunk=chunk, mode=mode,
                                resid=resid, m=True)
        torch.cuda.synchronize()
        assert_close(host(m), ref["m"], tol, f"m {mode}")
        assert_close(host(o), ref["o"], tol, f"o {mode}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noerase_write(kdn, orc, dtype):
    """Decayed linear attention (the write without its erase term), with scores."""
    import torch
    inp = workloads.scan_inputs(2, 2, 230, 128, 64, seed=111, dtype=dtype)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"],
                   resid="noerase")
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for chunk in (16, 64):
        got = _scan_gpu(kdn, inp, dtype, chunk, resid="noerase")
        assert_close(got["o"], ref["o"], tol, f"noerase o chunk {chunk}")
        assert_close(got["S"], ref["S"], tol, f"noerase S chunk {chunk}")
    q, k, v = (dev_tensor(inp[n], dtype) for n in ("q", "k", "v"))
    _, m = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                            resid="noerase", m=True)
    torch.cuda.synchronize()
    assert_close(host(m), ref["m"], tol, "noerase m")


@pytest.mark.parametrize("score,mode,resid,dtype", [("resid", "delta", "gated", "bf16"),
                                                    ("value", "delta", "gated", "bf16"),
                                                    ("resid", "delta", "plain", "f32"),
                                                    ("value", "delta", "plain", "bf16"),
                                                    ("value", "diag", "gated", "f32"),
                                                    ("resid", "iso", "gated", "bf16")])
def test_score_variants(kdn, orc, score, mode, resid, dtype):
    """The ablation scores (A Hippocampus for Linear Attention, sec. 3.3 "versus
    recency", sec. 4.5): the residual alone and the write strength alone."""
    import torch
    inp = workloads.scan_inputs(1, 2, 150, 128, 64, seed=112, dtype=dtype, with_r=True)
    cov0 = {"diag": np.ones((1, 2, 128), np.float32), "iso": np.ones((1, 2), np.float32)}.get(mode)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"],
                   r=inp["r"] if mode != "delta" else None, cov0=cov0, q_noise_var=0.5,
                   mode=mode, resid=resid, score=score)
    q, k, v = (dev_tensor(inp[n], dtype) for n in ("q", "k", "v"))
    cin = dev_tensor(cov0) if cov0 is not None else None
    _, m = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                            r=dev_tensor(inp["r"]) if mode != "delta" else None, cov_in=cin,
                            cov_out=torch.empty_like(cin) if cin is not None else None,
                            q_noise_var=0.5, mode=mode, resid=resid, m=True, score=score)
    torch.cuda.synchronize()
    assert_close(host(m), ref["m"], TOL_BF16 if dtype == "bf16" else TOL_F32, f"m {score}")


# --------------------------------------------------------------- full-size workloads

def _sampled_check(kdn, orc, name, heads, mode="delta", check_state=True):
    cfg = workloads.WORKLOADS[name]
    inp = workloads.named_scan_inputs(name)
    log(f"{name}: full-size GPU run")
    cshape = {"diag": (cfg["B"], cfg["H"], cfg["dk"]), "iso": (cfg["B"], cfg["H"])}.get(mode)
    cov0 = np.full(cshape, cfg.get("cov_init", 1.0), np.float32) if cshape else None
    got = _scan_gpu(kdn, inp, cfg["dtype"], cfg["chunk"], mode=mode, cov0=cov0,
                    qvar=cfg.get("q_noise_var", 0.0))
    assert np.all(np.isfinite(got["o"]))
    for (b, h) in heads:
        log(f"{name}: oracle on head ({b}, {h})")
        sub = {n: (x[b:b + 1, h:h + 1] if x is not None else None) for n, x in inp.items()}
        ref = orc.scan(sub["q"], sub["k"], sub["v"], alpha=sub["alpha"], beta=sub["beta"],
                       r=sub["r"], cov0=None if cov0 is None else cov0[b:b + 1, h:h + 1],
                       q_noise_var=cfg.get("q_noise_var", 0.0), mode=mode, want_m=False)
        assert_close(got["o"][b:b + 1, h:h + 1], ref["o"], TOL_BF16, f"{name} o head {(b, h)}")
        if check_state:
            assert_close(got["S"][b:b + 1, h:h + 1], ref["S"], TOL_BF16, f"{name} S head {(b, h)}")
        if cov0 is not None:
            assert_close(got["cov"][b:b + 1, h:h + 1], ref["cov"], TOL_F32, f"{name} p head {(b, h)}")


def test_full_size_gated(kdn, orc):
    _sampled_check(kdn, orc, "gated", [(0, 0), (1, 7), (3, 15)])


def test_full_size_kdn_diag(kdn, orc):
    _sampled_check(kdn, orc, "kdn_diag", [(0, 3), (2, 9), (3, 15)], mode="diag")


def test_full_size_kdn_iso(kdn, orc):
    """The Kalman workload's inputs with one variance per head instead of a diagonal."""
    _sampled_check(kdn, orc, "kdn_diag", [(0, 3), (3, 15)], mode="iso")


def test_full_size_long(kdn, orc):
    _sampled_check(kdn, orc, "long", [(0, 0), (0, 31)])
