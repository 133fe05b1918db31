"""GPU parity of kdn_step_decode and hola_cache_update against the fp64 oracle.

Cache membership is compared exactly as sets of token positions. The decision
is taken on float32 scores on both sides; where the GPU's and the oracle's
float32 score of a token differ (rounding) and that token sits at the
eviction boundary, the two memberships may legitimately differ: such a case is
accepted only if the GPU cache is exactly the top-w of the GPU's own score
history and the scores involved agree to 1e-5 relative.
"""
import numpy as np
import pytest

import workloads
from _util import TOL_F32, assert_close, dev_tensor, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kdn():
    import torch
    import delta_rule_scans_amd as k
    assert torch.cuda.is_available()
    return k


def _steps(n, B, H, dk, dv, seed, diag=False):
    out = []
    for s in range(n):
        inp = workloads.decode_step_inputs(s, B, H, dk, dv, seed=seed)
        if diag:
            rng = np.random.Generator(np.random.PCG64([seed, s, 7]))
            inp["r"] = np.logaddexp(0.0, rng.standard_normal((B, H))).astype(np.float32)
        out.append(inp)
    return out


def _membership(hist, w):
    """Cache content after each step for one head, as a boolean matrix
    member[t, j]: token j is among the top-w of the float32 scores hist[0..t]
    by (score desc, position asc). Token j's rank at step t counts the tokens
    i <= t ordered before it."""
    s = np.asarray(hist, np.float32)
    T = len(s)
    idx = np.arange(T)
    before = (s[:, None] > s[None, :]) | ((s[:, None] == s[None, :]) & (idx[:, None] < idx[None, :]))
    rank = np.cumsum(before, axis=0)          # rank[t, j] = #{i <= t : i before j}
    return (idx[None, :] <= idx[:, None]) & (rank < w)


def _run_decode(kdn, orc, B, H, dk, dv, w, steps, seed, mode="delta", resid="gated",
                sink=False, qvar=0.0, sample=None):
    import torch
    kalman = mode in ("diag", "iso")
    inputs = _steps(steps, B, H, dk, dv, seed, diag=kalman)
    state = torch.zeros((B, H, dk, dv), device="cuda")
    cshape = {"diag": (B, H, dk), "iso": (B, H)}.get(mode)
    cov = torch.ones(cshape, device="cuda") if kalman else None
    cache = kdn.HolaCache(B, H, dk, dv, w)
    rng = np.random.Generator(np.random.PCG64([seed, 99]))
    sink_np = rng.standard_normal(H).astype(np.float32) if sink else None
    sink_t = dev_tensor(sink_np) if sink else None
    sel = sample if sample is not None else [(b, h) for b in range(B) for h in range(H)]
    bs = np.array([s[0] for s in sel])
    hs = np.array([s[1] for s in sel])
    outs, couts, ms = [], [], []
    for t, inp in enumerate(inputs):
        d = {n: dev_tensor(x) for n, x in inp.items()}
        o, m = kdn.kdn_step_decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], state,
                                   r=d.get("r"), cov=cov, q_noise_var=qvar, mode=mode, resid=resid)
        oc = kdn.hola_cache_update(d["q"], d["k"], d["v"], m, t, cache, sink_logit=sink_t)
        outs.append(host(o)[bs, hs])
        couts.append(host(oc)[bs, hs])
        ms.append(host(m)[bs, hs])
    torch.cuda.synchronize()
    # oracle on the sampled heads only (B' = 1, H' = len(sample))
    sub_inputs = [{n: x[bs, hs][None] for n, x in inp.items()} for inp in inputs]
    r_steps = [s["r"] for s in sub_inputs] if kalman else None
    o_ref, oc_ref, m_ref, S_ref, cov_ref, ocache = orc.decode_run(
        sub_inputs, 1, len(sel), dk, dv, w, mode=mode, resid=resid,
        cov0=np.ones((1, len(sel)) + ((dk,) if mode == "diag" else ())) if kalman else None,
        r_steps=r_steps,
        q_noise_var=qvar, sink_logit=None if sink_np is None else sink_np[hs],
        rms_eps=1e-6)
    got = dict(o=np.stack(outs), oc=np.stack(couts), m=np.stack(ms), S=host(state)[bs, hs],
               cov=None if cov is None else host(cov)[bs, hs], pos=host(cache.pos)[bs, hs].astype(np.int64),
               count=host(cache.count)[bs, hs].astype(np.int64))
    ref = dict(o=np.stack(o_ref)[:, 0], oc=np.stack(oc_ref)[:, 0], m=np.stack(m_ref)[:, 0],
               S=S_ref[0], cov=None if cov_ref is None else cov_ref[0], pos=ocache.pos[0],
               count=ocache.count[0])
    return got, ref


def _compare(got, ref, w, what):
    assert_close(got["o"], ref["o"], TOL_F32, f"{what} o")
    assert_close(got["m"], ref["m"], TOL_F32, f"{what} m")
    assert_close(got["S"], ref["S"], TOL_F32, f"{what} S")
    if got["cov"] is not None:
        assert_close(got["cov"], ref["cov"], TOL_F32, f"{what} cov")
    steps, nh = got["m"].shape
    tie_steps = 0
    ok = np.zeros((steps, nh), bool)   # steps whose read saw the same cache on both sides
    for i in range(nh):
        oh = ref["m"][:, i].astype(np.float32)
        gm = _membership(got["m"][:, i], w)
        om = _membership(oh, w)
        # the GPU cache is exactly the top-w of the GPU's own scores (ties: earlier token)
        n = int(got["count"][i])
        assert n == int(ref["count"][i]) == min(steps, w)
        assert sorted(got["pos"][i][:n].tolist()) == np.flatnonzero(gm[-1]).tolist(), \
            f"{what}: head {i} cache content"
        assert sorted(ref["pos"][i][:n].tolist()) == np.flatnonzero(om[-1]).tolist()
        same = np.ones(steps, bool)
        same[1:] = np.all(gm[:-1] == om[:-1], axis=1)
        ok[:, i] = same
        for t in np.flatnonzero(~same):
            # only a float32 rounding difference at the eviction boundary may cause this
            tie_steps += 1
            kth = np.sort(oh[:t])[::-1][w - 1]
            for j in np.flatnonzero(gm[t - 1] != om[t - 1]):
                assert abs(oh[j] - kth) <= 1e-5 * abs(kth), f"{what}: head {i} token {j} not at a tie"
    # o_cache of every (step, head) whose read saw the same cache: per-vector bar
    rms = np.sqrt(np.mean(ref["oc"] ** 2, axis=-1))
    err = np.max(np.abs(got["oc"] - ref["oc"]), axis=-1) / np.where(rms > 0, rms, 1.0)
    assert np.all(np.isfinite(got["oc"]))
    worst = float(np.max(err[ok])) if ok.any() else 0.0
    log(f"  {what} o_cache: worst per-step max|diff|/RMS = {worst:.3e} over {int(ok.sum())} "
        f"(step, head) reads; steps whose cache differs only by a rounding tie: {tie_steps}")
    assert worst <= TOL_F32


@pytest.mark.parametrize("mode,resid,sink", [("delta", "gated", False), ("delta", "plain", True),
                                             ("diag", "gated", False), ("iso", "gated", True)])
def test_decode_hola_small(kdn, orc, mode, resid, sink):
    log(f"decode {mode} {resid} sink={sink}")
    got, ref = _run_decode(kdn, orc, 3, 4, 128, 128, 16, 60, seed=201, mode=mode, resid=resid,
                           sink=sink, qvar=1.0 if mode in ("diag", "iso") else 0.0)
    _compare(got, ref, 16, f"decode {mode}/{resid}")


def test_decode_odd_shapes(kdn, orc):
    got, ref = _run_decode(kdn, orc, 2, 3, 40, 24, 5, 30, seed=202)
    _compare(got, ref, 5, "decode odd shapes")


def test_decode_equals_scan(kdn):
    """L decode steps from S = 0 give the same outputs and state as one scan of L
    tokens (float32 paths)."""
    import torch
    B, H, L, d = 2, 3, 70, 64
    inp = workloads.scan_inputs(B, H, L, d, d, seed=203, dtype="f32")
    q, k, v = (dev_tensor(inp[n]) for n in ("q", "k", "v"))
    a, b = dev_tensor(inp["alpha"]), dev_tensor(inp["beta"])
    S = torch.zeros((B, H, d, d), device="cuda")
    o_scan = kdn.kdn_scan_fwd(q, k, v, alpha=a, beta=b, state_out=S, chunk=32)
    Sd = torch.zeros_like(S)
    outs = []
    for t in range(L):
        o, _ = kdn.kdn_step_decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                   v[:, :, t].contiguous(), a[:, :, t].contiguous(),
                                   b[:, :, t].contiguous(), Sd)
        outs.append(o)
    torch.cuda.synchronize()
    assert_close(host(torch.stack(outs, 2)), host(o_scan), TOL_F32, "decode vs scan o")
    assert_close(host(Sd), host(S), TOL_F32, "decode vs scan S")


def test_diag_with_covariance_reset_is_delta(kdn):
    """Kalman Delta Networks, abstract: resetting the predicted covariance to c I
    before every token, with r_t = c (1 - beta_t) / beta_t and unit keys, turns
    the Kalman write into the delta write with beta_t."""
    import torch
    B, H, d, T, c = 2, 2, 128, 25, 2.0
    rng = np.random.Generator(np.random.PCG64(204))
    S1 = torch.zeros((B, H, d, d), device="cuda")
    S2 = torch.zeros_like(S1)
    for t in range(T):
        k = dev_tensor(rng.choice([-1.0, 1.0], (B, H, d)).astype(np.float32) / np.sqrt(d).astype(np.float32))
        q = dev_tensor(rng.standard_normal((B, H, d)).astype(np.float32))
        v = dev_tensor(rng.standard_normal((B, H, d)).astype(np.float32))
        beta_np = rng.uniform(0.1, 0.9, (B, H)).astype(np.float32)
        ones = torch.ones((B, H), device="cuda")
        o1, m1 = kdn.kdn_step_decode(q, k, v, ones, dev_tensor(beta_np), S1)
        cov = torch.full((B, H, d), c, device="cuda")
        r = dev_tensor((c * (1.0 - beta_np.astype(np.float64)) / beta_np).astype(np.float32))
        o2, m2 = kdn.kdn_step_decode(q, k, v, ones, ones, S2, r=r, cov=cov, mode="diag")
        torch.cuda.synchronize()
        assert_close(host(o2), host(o1), 1e-5, "reset o")
        assert_close(host(m2), host(m1), 1e-5, "reset m")
    assert_close(host(S2), host(S1), 1e-5, "reset S")


@pytest.mark.parametrize("B,H,dk,dv,w,steps,sink", [
    (48, 32, 128, 128, 12, 30, True),   # many heads, with a sink
    (2, 3, 64, 64, 80, 100, False),     # w > 64: more slots than a wavefront, evicting
    (1, 2, 64, 64, 256, 300, True),     # the largest capacity: four slots per lane
    (2, 3, 30, 18, 6, 20, True),        # rows that are not whole 16-byte quads (scalar loads)
])
def test_cache_kernel_forms(kdn, orc, B, H, dk, dv, w, steps, sink):
    """The cache kernel against the oracle on the shapes its code paths split
    on: 16-byte rows or not, and capacities above one slot per lane of the
    wavefront that chooses the eviction."""
    log(f"cache kernel B={B} H={H} dk={dk} dv={dv} w={w} steps={steps} sink={sink}")
    sample = None if B * H <= 16 else [(0, 0), (5, 7), (23, 31), (47, 30), (47, 31)]
    got, ref = _run_decode(kdn, orc, B, H, dk, dv, w, steps, seed=207, sink=sink, sample=sample)
    _compare(got, ref, w, f"cache kernel w={w} dk={dk}")


def test_full_size_decode_hola(kdn, orc):
    """The decode workload at full size (B=256, H=32, d=128, 512 steps, w=64),
    checked over every step on 297 heads spread over the whole batch and every
    eighth... head index (b = 0, 8, ..., 248, 255; h = 0, 4, ..., 28, 31)."""
    cfg = workloads.WORKLOADS["decode"]
    bs = list(range(0, 256, 8)) + [255]
    hs = list(range(0, 32, 4)) + [31]
    sample = [(b, h) for b in bs for h in hs]
    got, ref = _run_decode(kdn, orc, cfg["B"], cfg["H"], cfg["dk"], cfg["dv"], cfg["w"],
                           cfg["steps"], seed=workloads.DECODE_SEED, sample=sample)
    _compare(got, ref, cfg["w"], "decode full size")


@pytest.mark.parametrize("resid,score", [("noerase", "write"), ("gated", "resid"),
                                         ("plain", "resid"), ("plain", "value")])
def test_decode_switches(kdn, orc, resid, score):
    """No-erase write and the ablation scores in the decode step."""
    import torch
    B, H, d, T = 2, 3, 64, 30
    inputs = _steps(T, B, H, d, d, seed=205)
    state = torch.zeros((B, H, d, d), device="cuda")
    ms, outs = [], []
    for inp in inputs:
        g = {n: dev_tensor(x) for n, x in inp.items()}
        o, m = kdn.kdn_step_decode(g["q"], g["k"], g["v"], g["alpha"], g["beta"], state,
                                   resid=resid, score=score)
        outs.append(host(o))
        ms.append(host(m))
    torch.cuda.synchronize()
    o_ref, _, m_ref, S_ref, _, _ = orc.decode_run(inputs, B, H, d, d, 4, resid=resid, score=score)
    assert_close(np.stack(outs), np.stack(o_ref), TOL_F32, f"{resid} o")
    assert_close(np.stack(ms), np.stack(m_ref), TOL_F32, f"{score} m")
    assert_close(host(state), S_ref, TOL_F32, f"{resid} S")


def test_recency_cache(kdn, orc):
    """The recency control (A Hippocampus for Linear Attention, sec. 4.5): the
    cache keeps the w most recent tokens; reads against the oracle."""
    import torch
    B, H, d, w, T = 2, 2, 128, 8, 40
    inputs = _steps(T, B, H, d, d, seed=206)
    cache = kdn.HolaCache(B, H, d, d, w, policy="recency")
    ocache = orc.HolaCache(B, H, d, d, w, policy="recency")
    for t, inp in enumerate(inputs):
        g = {n: dev_tensor(x) for n, x in inp.items()}
        m = torch.rand((B, H), device="cuda")
        oc = kdn.hola_cache_update(g["q"], g["k"], g["v"], m, t, cache)
        ref = ocache.step(inp["q"], inp["k"], inp["v"], host(m), t)
        assert_close(host(oc), ref, TOL_F32, f"recency o_cache t={t}")
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            assert sorted(host(cache.pos)[b, h].astype(int).tolist()) == list(range(T - w, T))


def test_decode_graph_replays(kdn):
    """Three decode + cache steps captured in one HIP graph: every replay, with
    eager work and synchronisation between replays, matches the same steps run
    eagerly on a copy of the state and cache (bit for bit: same kernels, same
    inputs)."""
    import torch
    B, H, d, w = 2, 3, 128, 4
    steps = [workloads.decode_step_inputs(s, B, H, d, d) for s in range(3)]
    x = [{n: dev_tensor(a) for n, a in st.items()} for st in steps]

    def new_state():
        return torch.zeros((B, H, d, d), device="cuda"), kdn.HolaCache(B, H, d, d, w)

    def run(state, cache, o, m, oc, base):
        for i, xi in enumerate(x):
            kdn.kdn_step_decode(xi["q"], xi["k"], xi["v"], xi["alpha"], xi["beta"], state, o=o, m=m)
            kdn.hola_cache_update(xi["q"], xi["k"], xi["v"], m, base + i, cache, o_cache=oc)

    outs = lambda: (torch.empty((B, H, d), device="cuda"), torch.empty((B, H), device="cuda"),
                    torch.empty((B, H, d), device="cuda"))
    se, ce = new_state()
    oe, me, oce = outs()
    sg, cg = new_state()
    og, mg, ocg = outs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(sg, cg, og, mg, ocg, 0)
    for rep in range(3):
        log(f"graph replay {rep}")
        run(se, ce, oe, me, oce, 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b, name in ((sg, se, "state"), (og, oe, "o"), (mg, me, "m"), (ocg, oce, "o_cache"),
                           (cg.k, ce.k, "cache k"), (cg.v, ce.v, "cache v"), (cg.m, ce.m, "cache m"),
                           (cg.pos, ce.pos, "cache pos"), (cg.count, ce.count, "cache count")):
            assert torch.equal(a, b), f"replay {rep}: {name}"



def test_nan_scores_same_rule_decode_and_prompt(kdn, orc):
    """A NaN write score ranks below every other score (the reading both the
    oracle and the kernels take; the pages are silent): the decode-step cache
    and the prompt cache hold the same members as the oracle, token by token
    and block by block, with NaN scores in the cache before it fills and after."""
    import torch
    rng = np.random.Generator(np.random.PCG64(208))
    B, H, d, w, T = 1, 4, 64, 6, 40
    q, k, v = (rng.standard_normal((B, H, T, d)).astype(np.float32) for _ in range(3))
    m = (np.round(rng.uniform(0, 3, (B, H, T)) * 2) / 2).astype(np.float32)
    m[rng.uniform(size=(B, H, T)) < 0.3] = np.nan
    m[0, 0, :4] = np.nan
    cache = kdn.HolaCache(B, H, d, d, w)
    ocache = orc.HolaCache(B, H, d, d, w)
    for t in range(T):
        qt, kt, vt = (dev_tensor(np.ascontiguousarray(x[:, :, t])) for x in (q, k, v))
        oc = kdn.hola_cache_update(qt, kt, vt, dev_tensor(np.ascontiguousarray(m[:, :, t])), t, cache)
        ref = ocache.step(q[:, :, t], k[:, :, t], v[:, :, t], m[:, :, t].astype(np.float64), t)
        assert_close(host(oc), ref, TOL_F32, f"nan-score decode o_cache t={t}")
        torch.cuda.synchronize()
        for h in range(H):
            n = int(host(cache.count)[0, h])
            assert n == int(ocache.count[0, h])
            assert sorted(host(cache.pos)[0, h, :n].astype(int).tolist()) == \
                sorted(ocache.pos[0, h, :n].tolist()), f"decode head {h} t={t}"
    for block in (1, 7, 64):
        pc = kdn.HolaCache(B, H, d, d, w)
        oc = kdn.hola_prefill(dev_tensor(q), dev_tensor(k), dev_tensor(v), dev_tensor(m), 0, pc,
                              block=block)
        torch.cuda.synchronize()
        oref = orc.HolaCache(B, H, d, d, w)
        ref = oref.prefill(q, k, v, m.astype(np.float64), 0, block)
        assert_close(host(oc), ref, TOL_F32, f"nan-score prompt o_cache block {block}")
        np.testing.assert_array_equal(host(pc.pos).astype(np.int64), oref.pos.astype(np.int64))
        np.testing.assert_array_equal(host(pc.count).astype(np.int64), oref.count.astype(np.int64))
        # the decode cache, token by token, holds the same set as the prompt cache
        for h in range(H):
            assert sorted(host(pc.pos)[0, h].astype(int).tolist()) == \
                sorted(host(cache.pos)[0, h].astype(int).tolist())


def test_decode_nonfinite_inputs_propagate(kdn, orc):
    """A NaN value entry in one head's token makes that head's value column
    non-finite from then on (output and state); other heads are bit-identical to
    a clean run, and other columns of the head match the oracle."""
    import torch
    B, H, d, T = 2, 3, 128, 12
    inputs = _steps(T, B, H, d, d, seed=209)
    bad = [{n: x.copy() for n, x in st.items()} for st in inputs]
    bad[5]["v"][1, 2, 7] = np.nan

    def run(steps):
        state = torch.zeros((B, H, d, d), device="cuda")
        outs = []
        for st in steps:
            g = {n: dev_tensor(x) for n, x in st.items()}
            o, _ = kdn.kdn_step_decode(g["q"], g["k"], g["v"], g["alpha"], g["beta"], state)
            outs.append(host(o))
        torch.cuda.synchronize()
        return np.stack(outs), host(state)

    o_clean, s_clean = run(inputs)
    o_bad, s_bad = run(bad)
    o_ref, _, _, S_ref, _, _ = orc.decode_run(bad, B, H, d, d, 4)
    o_ref = np.stack(o_ref)
    clean_heads = [(b, h) for b in range(B) for h in range(H) if (b, h) != (1, 2)]
    for (b, h) in clean_heads:
        np.testing.assert_array_equal(o_bad[:, b, h], o_clean[:, b, h])
        np.testing.assert_array_equal(s_bad[b, h], s_clean[b, h])
    np.testing.assert_array_equal(o_bad[:5, 1, 2], o_clean[:5, 1, 2])
    assert np.all(~np.isfinite(o_bad[5:, 1, 2, 7])) and np.all(~np.isfinite(s_bad[1, 2, :, 7]))
    keep = np.arange(d) != 7
    assert_close(o_bad[:, 1, 2][:, keep], o_ref[:, 1, 2][:, keep], TOL_F32, "decode untouched columns")
    assert np.all(~np.isfinite(o_ref[5:, 1, 2, 7]))
