"""GPU parity of kdn_scan_fwd against the fp64 oracle (element by element).

Small cases span several chunks and a ragged tail; the full-size workloads are
run exactly as the benchmark launches them and checked on every head, each of
which the oracle recomputes over the whole sequence.
"""
import numpy as np
import pytest

import workloads
from _util import (TOL_BF16, TOL_F32, assert_close, dev_tensor, extreme_alpha as _extreme_alpha,
                   host, log, rel_err)

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
    alpha, beta, r = (dev_tensor(inp[n]) if inp.get(n) is not None else None
                      for n in ("alpha", "beta", "r"))
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
    for chunk in (16, 32, 64, 128):
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
    """Enough (head, chunk) pairs (more than 16384) that the prepare step hands
    each workgroup two consecutive chunks, the second one's inputs loading
    while the first is computed, with a chunk count the group size does not
    divide and a ragged last chunk: B=2, H=64, L=8196 is 129 chunks per head,
    the last of 4 tokens, 16512 in all. The delta write and the diagonal
    Kalman write (which also stages Q, carries each coordinate's variance
    through the chunk and writes the gains); the oracle on sampled heads."""
    B, H, L, d = 2, 64, 8196, 128
    diag = mode == "diag"
    inp = workloads.scan_inputs(B, H, L, d, d, seed=111, dtype="bf16", with_r=diag)
    cov0 = np.ones((B, H, d), np.float32) if diag else None
    got = _scan_gpu(kdn, inp, "bf16", 64, mode=mode, cov0=cov0, qvar=1.0 if diag else 0.0)
    for (b, h) in [(0, 0), (1, 17), (1, 63)]:
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


@pytest.mark.parametrize("case", ["delta_bf16", "diag_bf16", "tiny_f32", "tiny_rls"])
def test_graph_replay_matches_eager(kdn, case):
    """One kdn_scan_fwd call captured into a HIP graph and replayed three times,
    with eager scans of other inputs and synchronisations between the replays:
    every replay gives the eager call's outputs, state and covariance bit for
    bit (the library enqueues kernels only: no allocation, copy or fill)."""
    import torch
    if case.startswith("tiny"):
        inp = workloads.named_scan_inputs("tiny")
        dtype, chunk, d = "f32", 16, inp["q"].shape[-1]
        mode = "full" if case == "tiny_rls" else "delta"
    else:
        d, dtype, chunk = 128, "bf16", 64
        mode = "diag" if case == "diag_bf16" else "delta"
        inp = workloads.scan_inputs(2, 3, 200, d, d, seed=131, dtype="bf16", with_r=mode == "diag")
    B, H, L, _ = inp["q"].shape
    q, k, v = (dev_tensor(inp[n], dtype) for n in ("q", "k", "v"))
    alpha = dev_tensor(inp["alpha"])
    beta = dev_tensor(inp["beta"]) if mode == "delta" else None
    r = dev_tensor(inp["r"]) if mode == "diag" else None
    cov_in = {"diag": lambda: torch.ones((B, H, d), device="cuda"),
              "full": lambda: (100.0 * torch.eye(d, device="cuda")).expand(B, H, d, d).contiguous(),
              "delta": lambda: None}[mode]()
    S0 = dev_tensor(np.random.default_rng(5).standard_normal((B, H, d, d)).astype(np.float32) * 0.1)
    need = kdn.kdn_scan_workspace_size(B, H, L, d, d, chunk, mode=mode,
                                       in_dtype=kdn.F32 if dtype == "f32" else kdn.BF16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, L, d), device="cuda")
    S = torch.empty((B, H, d, d), device="cuda")
    cov = torch.empty_like(cov_in) if cov_in is not None else None
    kw = dict(alpha=alpha, beta=beta, r=r, cov_in=cov_in, cov_out=cov, state_in=S0, state_out=S,
              o=o, chunk=chunk, mode=mode, q_noise_var=1.0 if mode == "diag" else 0.0,
              workspace=ws)
    kdn.kdn_scan_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    want = [t.clone() for t in (o, S, cov) if t is not None]
    # eager work between replays: the same call on reversed inputs
    other = [x.flip(2).contiguous() for x in (q, k, v)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kdn.kdn_scan_fwd(q, k, v, **kw)
    for rep in range(3):
        for t in (o, S, cov):
            if t is not None:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, S, cov) if t is not None]
        for g, w in zip(got, want):
            assert torch.equal(g, w), f"{case}: replay {rep} differs from the eager call"
        kdn.kdn_scan_fwd(*other, **{**kw, "o": torch.empty_like(o), "state_out": torch.empty_like(S),
                                    "cov_out": torch.empty_like(cov) if cov is not None else None,
                                    "workspace": None})
        torch.cuda.synchronize()
    log(f"graph replay {case}: 3 replays equal to the eager call")


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


@pytest.mark.parametrize("given,L", [(False, 200), (True, 230), (True, 192)])
def test_diag_kalman_spread_variances(kdn, orc, given, L):
    """Diagonal Kalman write on the matrix-core path from starting variances
    that differ per coordinate (0.05 .. 20, log-uniform), so that a coordinate
    taken for another where the chunk-start variances reach the gains would
    show; alpha and r left out (alpha = 1, r = 1: no process noise) or given.
    B=1 H=3; the last chunk holds 8 tokens (inside its first 32-token half),
    38 (inside its second half) or 64; o, S and the final variances against
    the oracle."""
    B, H, d = 1, 3, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=131, dtype="bf16", with_r=True)
    if not given:
        inp["alpha"] = None
        inp["r"] = None
    rng = np.random.Generator(np.random.PCG64(131))
    p0 = np.exp(rng.uniform(np.log(0.05), np.log(20.0), (B, H, d))).astype(np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=0.5, mode="diag")
    got = _scan_gpu(kdn, inp, "bf16", 64, mode="diag", cov0=p0, qvar=0.5)
    assert_close(got["o"], ref["o"], TOL_BF16, "diag o")
    assert_close(got["S"], ref["S"], TOL_BF16, "diag S")
    assert_close(got["cov"], ref["cov"], TOL_F32, "diag p")


def test_diag_kalman_wide_variance_range(kdn, orc):
    """Diagonal Kalman write on the matrix-core path with starting variances
    spread over six decades (1e-3 .. 1e3, log-uniform per coordinate) and a
    small observation noise (r = 0.01): gains that range widely within a
    token, and variances that fall by orders of magnitude over the sequence
    (the float32 recursion of the prepare kernel and the chunk-start scan).
    B=1 H=2 L=300, o, S and the final variances against the oracle."""
    B, H, L, d = 1, 2, 300, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=142, dtype="bf16", with_r=True)
    inp["r"] = np.full((B, H, L), 0.01, np.float32)
    rng = np.random.Generator(np.random.PCG64(142))
    p0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e3), (B, H, d))).astype(np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=0.2, mode="diag")
    got = _scan_gpu(kdn, inp, "bf16", 64, mode="diag", cov0=p0, qvar=0.2)
    assert_close(got["o"], ref["o"], TOL_BF16, "diag o")
    assert_close(got["S"], ref["S"], TOL_BF16, "diag S")
    assert_close(got["cov"], ref["cov"], TOL_F32, "diag p")


@pytest.mark.parametrize("dk", [40, 64])
def test_diag_kalman_other_key_widths(kdn, orc, dk):
    """Diagonal Kalman write on the float32 path with d_k = 40 (the chunk-start
    scan with lanes as chunks) and d_k = 64 (the scan with one group of 64
    coordinates as lanes), L = 300 (five chunks of 64, the last ragged), from
    starting variances that differ per coordinate."""
    B, H, L, dv = 1, 2, 300, 48
    inp = workloads.scan_inputs(B, H, L, dk, dv, seed=140 + dk, dtype="f32", with_r=True)
    rng = np.random.Generator(np.random.PCG64(140 + dk))
    p0 = np.exp(rng.uniform(np.log(0.1), np.log(10.0), (B, H, dk))).astype(np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=0.7, mode="diag")
    got = _scan_gpu(kdn, inp, "f32", 64, mode="diag", cov0=p0, qvar=0.7)
    assert_close(got["o"], ref["o"], TOL_F32, f"diag o d_k {dk}")
    assert_close(got["S"], ref["S"], TOL_F32, f"diag S d_k {dk}")
    assert_close(got["cov"], ref["cov"], TOL_F32, f"diag p d_k {dk}")


def test_diag_kalman_without_final_variances(kdn):
    """The matrix-core diagonal write with no cov_out: the same o and state as
    the call that asks for the final variances (they are only dropped)."""
    import torch
    inp = workloads.scan_inputs(1, 2, 230, 128, 128, seed=141, dtype="bf16", with_r=True)
    p0 = np.ones((1, 2, 128), np.float32)
    full = _scan_gpu(kdn, inp, "bf16", 64, mode="diag", cov0=p0, qvar=1.0)
    q, k, v = (dev_tensor(inp[n], "bf16") for n in ("q", "k", "v"))
    S = torch.empty((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    o = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), r=dev_tensor(inp["r"]),
                         cov_in=dev_tensor(p0), q_noise_var=1.0, state_out=S, mode="diag")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o), full["o"])
    np.testing.assert_array_equal(host(S), full["S"])


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


@pytest.mark.parametrize("mode", ["diag", "iso"])
def test_kalman_prefix_many_chunks(kdn, orc, mode):
    """More chunks than the prefix scan takes at once (64): 151 chunks of 64 on
    the matrix cores and 603 of 16 on the float32 path, the last block and the
    last chunk ragged; o, S and the final variance against the oracle."""
    B, H, L, d = 1, 2, 9637, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=131, dtype="bf16", with_r=True)
    p0 = (np.full((B, H, d), 1.0, np.float32) if mode == "diag"
          else np.array([[0.7, 1.3]], np.float32))
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=p0,
                   q_noise_var=1.0, mode=mode, want_m=False)
    for chunk in (64, 16):
        log(f"{mode} prefix scan, L {L} chunk {chunk}")
        got = _scan_gpu(kdn, inp, "bf16", chunk, mode=mode, cov0=p0, qvar=1.0)
        assert_close(got["o"], ref["o"], TOL_BF16, f"{mode} o chunk {chunk}")
        assert_close(got["S"], ref["S"], TOL_BF16, f"{mode} S chunk {chunk}")
        assert_close(got["cov"], ref["cov"], TOL_F32, f"{mode} p chunk {chunk}")


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


@pytest.mark.parametrize("dk,dv,L", [(13, 7, 70), (1, 5, 65), (61, 17, 129)])
def test_full_kalman_odd_sizes(kdn, orc, dk, dv, L):
    """Full covariance with key widths that are not multiples of the four lanes
    that share a row of P k, one key coordinate, and lengths one past a
    64-token input tile."""
    inp = workloads.scan_inputs(2, 1, L, dk, dv, seed=150 + dk, dtype="f32", with_r=True)
    rng = np.random.Generator(np.random.PCG64(150 + dk))
    A = rng.standard_normal((2, 1, dk, dk))
    P0 = (np.einsum("bhij,bhkj->bhik", A, A) / dk + np.eye(dk)).astype(np.float32)
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], r=inp["r"], cov0=P0,
                   q_noise_var=0.5, mode="full")
    got = _scan_gpu(kdn, inp, "f32", 16, mode="full", cov0=P0, qvar=0.5)
    assert_close(got["o"], ref["o"], TOL_F32, f"full d_k {dk} o")
    assert_close(got["S"], ref["S"], TOL_F32, f"full d_k {dk} S")
    assert_close(got["cov"], ref["cov"], TOL_F32, f"full d_k {dk} P")


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


@pytest.mark.parametrize("mode,resid,dtype", [("delta", "gated", "bf16"), ("delta", "plain", "bf16"),
                                              ("delta", "noerase", "bf16"),
                                              ("diag", "gated", "bf16"), ("iso", "gated", "bf16"),
                                              ("delta", "plain", "f32"), ("delta", "gated", "f32"),
                                              ("delta", "noerase", "f32")])
def test_extreme_decay(kdn, orc, mode, resid, dtype):
    """Very fast decay, alpha = 1 exactly and abrupt switches (see _extreme_alpha),
    on the matrix-core path (bf16, d_k = 128, chunk 64) and the float32 path,
    with a nonzero initial state; o, S (and p) against the oracle."""
    B, H, L, d = 1, 3, 357, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=120, dtype=dtype, with_r=mode != "delta")
    inp["alpha"] = _extreme_alpha(B, H, L, 120)
    S0 = np.random.Generator(np.random.PCG64(121)).standard_normal((B, H, d, d)).astype(np.float32) * 0.1
    cov0 = {"diag": np.ones((B, H, d), np.float32), "iso": np.ones((B, H), np.float32)}.get(mode)
    qvar = 1.0 if mode != "delta" else 0.0
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], r=inp["r"],
                   cov0=cov0, q_noise_var=qvar, S0=S0, mode=mode, resid=resid)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for chunk in ((64,) if dtype == "bf16" else (16, 64)):
        log(f"extreme decay {mode}/{resid} {dtype} chunk {chunk}")
        got = _scan_gpu(kdn, inp, dtype, chunk, mode=mode, resid=resid, cov0=cov0, qvar=qvar, S0=S0)
        assert_close(got["o"], ref["o"], tol, f"extreme {mode}/{resid} o")
        assert_close(got["S"], ref["S"], tol, f"extreme {mode}/{resid} S")
        if cov0 is not None:
            assert_close(got["cov"], ref["cov"], TOL_F32, f"extreme {mode} p")


def test_extreme_decay_scores(kdn, orc):
    """Write scores under the extreme decays, matrix-core path, plain and gated."""
    import torch
    B, H, L, d = 1, 2, 357, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=122, dtype="bf16")
    inp["alpha"] = _extreme_alpha(B, H, L, 122)
    q, k, v = (dev_tensor(inp[n], "bf16") for n in ("q", "k", "v"))
    for resid in ("gated", "plain"):
        ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], resid=resid)
        o, m = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                                resid=resid, m=True)
        torch.cuda.synchronize()
        assert_close(host(m), ref["m"], TOL_BF16, f"extreme {resid} m")
        assert_close(host(o), ref["o"], TOL_BF16, f"extreme {resid} o")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nonfinite_inputs_propagate(kdn, orc, dtype):
    """NaN and Inf inputs are not checked; they propagate. Head 0 is clean, head
    1 has a NaN in one value entry (token 100, column 5), head 2 a NaN in one key
    component (token 130), head 3 an Inf value entry (token 70, column 9).
    Every output the oracle makes non-finite is non-finite; outputs before the
    start of the 64-token chunk that holds the first non-finite input are
    bit-identical to a clean run (the chunk form mixes a chunk's tokens, so on
    the matrix-core path the earlier tokens of that chunk may turn non-finite
    too); value columns the bad entry never reaches match the oracle; clean
    heads are bit-identical to the clean run."""
    B, H, L, d = 1, 4, 200, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=123, dtype=dtype)
    clean = _scan_gpu(kdn, inp, dtype, 64)
    bad = {n: (x.copy() if x is not None else None) for n, x in inp.items()}
    bad["v"][0, 1, 100, 5] = np.nan
    bad["k"][0, 2, 130, 17] = np.nan
    bad["v"][0, 3, 70, 9] = np.inf
    got = _scan_gpu(kdn, bad, dtype, 64)
    ref = orc.scan(bad["q"], bad["k"], bad["v"], alpha=bad["alpha"], beta=bad["beta"])
    np.testing.assert_array_equal(got["o"][0, 0], clean["o"][0, 0])
    np.testing.assert_array_equal(got["S"][0, 0], clean["S"][0, 0])
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for h, t0 in ((1, 100), (2, 130), (3, 70)):
        c0 = t0 // 64 * 64
        np.testing.assert_array_equal(got["o"][0, h, :c0], clean["o"][0, h, :c0])
        bad_ref = ~np.isfinite(ref["o"][0, h])
        assert bad_ref.any()
        assert np.all(~np.isfinite(got["o"][0, h][bad_ref])), f"head {h}: a non-finite output came out finite"
        assert np.all(~np.isfinite(got["S"][0, h][~np.isfinite(ref["S"][0, h])]))
    for h, col in ((1, 5), (3, 9)):
        keep = np.arange(d) != col
        assert_close(got["o"][0, h][:, keep], ref["o"][0, h][:, keep], tol, f"head {h} untouched columns")
        assert np.all(~np.isfinite(got["o"][0, h, (70 if h == 3 else 100):, col]))


@pytest.mark.parametrize("mode", ["delta", "diag"])
def test_fp16_range_large_values(kdn, orc, mode):
    """Values far beyond the fp16 range of the matrix-core operands (bf16 allows
    them): the state, values and residuals are carried scaled by exact powers
    of two. Head 0: |v| up to ~1e5 in chunks 1 and 2, ordinary values around
    them (the scale must come back); head 1: values ~5000 (the state grows
    past 2^12 and is rescaled on its own); head 2: an initial state of ~1e5
    with ordinary values. o, S (and p) against the oracle at the bf16 bar."""
    B, H, L, d = 1, 3, 330, 128
    diag = mode == "diag"
    inp = workloads.scan_inputs(B, H, L, d, d, seed=124, dtype="bf16", with_r=diag)
    v = inp["v"].copy()
    v[0, 0, 64:192] *= 4.0e4
    v[0, 1] *= 2.5e3
    inp["v"] = workloads.bf16_round(v)
    rng = np.random.Generator(np.random.PCG64(124))
    S0 = (rng.standard_normal((B, H, d, d)) * 0.1).astype(np.float32)
    S0[0, 2] *= 1.0e6
    inp["alpha"][0, 2] = 1.0   # the large initial state lasts to the final state
    cov0 = np.ones((B, H, d), np.float32) if diag else None
    qvar = 1.0 if diag else 0.0
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"], r=inp["r"],
                   cov0=cov0, q_noise_var=qvar, S0=S0, mode=mode)
    assert np.abs(ref["o"][0, :2]).max() > 65504 and np.abs(ref["S"][0, 2]).max() > 65504
    got = _scan_gpu(kdn, inp, "bf16", 64, mode=mode, cov0=cov0, qvar=qvar, S0=S0)
    for h in range(H):
        assert_close(got["o"][0, h], ref["o"][0, h], TOL_BF16, f"range {mode} o head {h}")
        assert_close(got["S"][0, h], ref["S"][0, h], TOL_BF16, f"range {mode} S head {h}")
    # the ordinary chunks after the large ones, on their own scale
    assert_close(got["o"][0, 0, 192:], ref["o"][0, 0, 192:], TOL_BF16, f"range {mode} o after")
    if diag:
        assert_close(got["cov"], ref["cov"], TOL_F32, "range diag p")


def test_fp16_range_scores(kdn, orc):
    """Write scores from the matrix-core path's fp16 residual copies when those
    residuals are carried scaled (values ~5000)."""
    import torch
    inp = workloads.scan_inputs(1, 2, 200, 128, 128, seed=125, dtype="bf16")
    inp["v"] = workloads.bf16_round(inp["v"] * 5.0e3)
    q, k, v = (dev_tensor(inp[n], "bf16") for n in ("q", "k", "v"))
    o, m = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                            m=True)
    torch.cuda.synchronize()
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    assert_close(host(m), ref["m"], TOL_BF16, "range scores m")
    assert_close(host(o), ref["o"], TOL_BF16, "range scores o")


def test_fp16_range_tiny_components(kdn, orc):
    """Key and query components below 2^-14 (fp16 subnormals once staged):
    keys whose mass sits on a few coordinates with the rest ~1e-6, queries
    with small entries; the bar relative to RMS(o) holds."""
    B, H, L, d = 1, 2, 200, 128
    inp = workloads.scan_inputs(B, H, L, d, d, seed=126, dtype="f32")
    rng = np.random.Generator(np.random.PCG64(126))
    k = inp["k"].copy()
    small = rng.uniform(size=k.shape) < 0.8
    k[small] *= 1.0e-5
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = inp["q"].copy()
    q[rng.uniform(size=q.shape) < 0.5] *= 3.0e-5
    inp["k"], inp["q"] = workloads.bf16_round(k), workloads.bf16_round(q)
    inp["v"] = workloads.bf16_round(inp["v"])
    assert np.sum((np.abs(inp["k"]) < 2.0 ** -14) & (inp["k"] != 0)) > 1000
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    got = _scan_gpu(kdn, inp, "bf16", 64)
    assert_close(got["o"], ref["o"], TOL_BF16, "tiny components o")
    assert_close(got["S"], ref["S"], TOL_BF16, "tiny components S")


# --------------------------------------------------------------- full-size workloads

def _full_check(kdn, orc, name, mode="delta", resid="gated"):
    """The named workload at full size, launched as the benchmark launches it,
    against the oracle on every head: o, the final state and (Kalman) the final
    covariance, each to its bar over all heads at once and per head."""
    cfg = workloads.WORKLOADS[name]
    inp = workloads.named_scan_inputs(name)
    log(f"{name}/{mode}/{resid}: full-size GPU run")
    cshape = {"diag": (cfg["B"], cfg["H"], cfg["dk"]), "iso": (cfg["B"], cfg["H"])}.get(mode)
    cov0 = np.full(cshape, cfg.get("cov_init", 1.0), np.float32) if cshape else None
    got = _scan_gpu(kdn, inp, cfg["dtype"], cfg["chunk"], mode=mode, cov0=cov0,
                    qvar=cfg.get("q_noise_var", 0.0), resid=resid)
    log(f"{name}/{mode}/{resid}: oracle on all {cfg['B'] * cfg['H']} heads")
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"],
                   r=inp["r"], cov0=cov0, q_noise_var=cfg.get("q_noise_var", 0.0), mode=mode,
                   resid=resid, want_m=False)
    assert_close(got["o"], ref["o"], TOL_BF16, f"{name} o (all heads)")
    assert_close(got["S"], ref["S"], TOL_BF16, f"{name} S (all heads)")
    if cov0 is not None:
        assert_close(got["cov"], ref["cov"], TOL_F32, f"{name} p (all heads)")
    worst = max(rel_err(got["o"][b, h], ref["o"][b, h])
                for b in range(cfg["B"]) for h in range(cfg["H"]))
    log(f"  {name}: worst single-head max|diff|/RMS(head) of o = {worst:.3e}")
    assert worst <= TOL_BF16


def test_full_size_gated(kdn, orc):
    _full_check(kdn, orc, "gated")


def test_full_size_noerase(kdn, orc):
    """The gated workload's inputs with the write's erase term dropped (decayed
    linear attention) on the matrix cores: the same chunk form with A = 0."""
    _full_check(kdn, orc, "gated", resid="noerase")


def test_full_size_kdn_diag(kdn, orc):
    _full_check(kdn, orc, "kdn_diag", mode="diag")


def test_full_size_kdn_iso(kdn, orc):
    """The Kalman workload's inputs with one variance per head instead of a diagonal."""
    _full_check(kdn, orc, "kdn_diag", mode="iso")


def test_full_size_long(kdn, orc):
    _full_check(kdn, orc, "long")


@pytest.mark.parametrize("cols", ["16", "32"])
def test_state_tilings(kdn, orc, cols, monkeypatch):
    """The delta write's two state-kernel tilings -- 32-column slices, and the
    16-column slices taken when the heads are too few to fill the device --
    each forced in turn through KDN_STATE_COLS, on the cases that reach every
    branch of the chain (initial state, bf16 output, plain and no-erase
    residuals, short and ragged lengths, extreme decay, the fp16 range)."""
    monkeypatch.setenv("KDN_STATE_COLS", cols)
    log(f"state tiling: {cols}-column slices")
    test_gated_delta_small(kdn, orc, "bf16")
    test_plain_residual(kdn, orc, "bf16")
    test_noerase_write(kdn, orc, "bf16")
    test_short_sequences(kdn, orc)
    test_extreme_decay(kdn, orc, "delta", "gated", "bf16")
    test_fp16_range_large_values(kdn, orc, "delta")
    test_fp16_range_tiny_components(kdn, orc)
