"""GPU parity of hola_prefill (the HOLA cache over a whole prompt, block by
block) and of the scan's write scores feeding it, against the fp64 oracle.

The oracle is run on the scores the GPU emitted (the cache decision is taken
on float32 scores on both sides), so membership must match exactly: same
count, same positions in the same rank order, bit-identical scores, keys and
values. The read is float32 arithmetic on the exact input values, so o_cache
is held to the float32 tolerance for bf16 inputs too.
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


def _prefill_case(kdn, orc, q, k, v, m, t0, block, w, dtype, sink=None, init=None, heads=None,
                  policy="score"):
    """Run hola_prefill on the GPU and the oracle (on `heads`, default all) and compare."""
    import torch
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    cache = kdn.HolaCache(B, H, dk, dv, w, policy=policy)
    ocache = orc.HolaCache(B, H, dk, dv, w, policy=policy)
    if init is not None:
        n0, rng = init
        for f, shape in (("k", (B, H, w, dk)), ("v", (B, H, w, dv))):
            x = rng.standard_normal(shape).astype(np.float32)
            getattr(cache, f).copy_(torch.from_numpy(x))
            setattr(ocache, f, x.copy())
        cm = rng.uniform(0, 3, (B, H, w)).astype(np.float32)
        cp = np.broadcast_to(np.arange(w, dtype=np.int32) - w - 5, (B, H, w)).copy()
        cache.m.copy_(torch.from_numpy(cm))
        cache.pos.copy_(torch.from_numpy(cp))
        cache.count.fill_(n0)
        ocache.m, ocache.pos = cm.copy(), cp.copy()
        ocache.count = np.full((B, H), n0, np.int32)
    dq, dk_, dvv = (dev_tensor(x, dtype) for x in (q, k, v))
    sink_t = dev_tensor(sink) if sink is not None else None
    oc = kdn.hola_prefill(dq, dk_, dvv, dev_tensor(m), t0, cache, block=block, sink_logit=sink_t)
    torch.cuda.synchronize()
    got = dict(o=host(oc), k=host(cache.k), v=host(cache.v), m=host(cache.m),
               pos=host(cache.pos).astype(np.int64), count=host(cache.count).astype(np.int64))
    sel = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    bs = np.array([s[0] for s in sel])
    hs = np.array([s[1] for s in sel])
    sub = orc.HolaCache(1, len(sel), dk, dv, w, policy=policy)
    for f in ("k", "v", "m", "pos"):
        setattr(sub, f, np.ascontiguousarray(getattr(ocache, f)[bs, hs][None]))
    sub.count = np.ascontiguousarray(ocache.count[bs, hs][None])
    qq, kk, vv = (workloads.bf16_round(x) if dtype == "bf16" else x for x in (q, k, v))
    ref_o = sub.prefill(qq[bs, hs][None], kk[bs, hs][None], vv[bs, hs][None],
                        m[bs, hs][None].astype(np.float64), t0, block,
                        None if sink is None else sink[hs])
    assert_close(got["o"][bs, hs], ref_o[0], TOL_F32, f"o_cache block {block}")
    n = got["count"][bs, hs]
    np.testing.assert_array_equal(n, sub.count[0])
    for i in range(len(sel)):
        c = int(n[i])
        np.testing.assert_array_equal(got["pos"][bs[i], hs[i], :c], sub.pos[0, i, :c])
        np.testing.assert_array_equal(got["m"][bs[i], hs[i], :c], sub.m[0, i, :c])
        np.testing.assert_array_equal(got["k"][bs[i], hs[i], :c], sub.k[0, i, :c])
        np.testing.assert_array_equal(got["v"][bs[i], hs[i], :c], sub.v[0, i, :c])
    return got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_small(kdn, orc, dtype):
    rng = np.random.Generator(np.random.PCG64(301))
    B, H, L, d, w = 2, 3, 300, 128, 16
    q = rng.standard_normal((B, H, L, d)).astype(np.float32)
    k = rng.standard_normal((B, H, L, d)).astype(np.float32)
    v = rng.standard_normal((B, H, L, d)).astype(np.float32)
    m = (np.round(rng.uniform(0, 3, (B, H, L)) * 8) / 8).astype(np.float32)  # exact ties
    sink = rng.standard_normal(H).astype(np.float32)
    for block, use_sink, init in ((64, False, None), (1, True, None), (17, True, 5),
                                  (256, False, 16), (1000, True, 9)):
        log(f"prefill {dtype} block {block} sink {use_sink} init {init}")
        _prefill_case(kdn, orc, q, k, v, m, 40, block, w, dtype, sink if use_sink else None,
                      None if init is None else (init, rng))


def test_prefill_max_capacity(kdn, orc):
    """The largest capacity the library takes (w = 256): a cache partly full
    (200) and a full one, blocks of 128 and 300, with exact score ties."""
    rng = np.random.Generator(np.random.PCG64(304))
    B, H, L, d, w = 1, 2, 600, 64, 256
    q = rng.standard_normal((B, H, L, d)).astype(np.float32)
    k = rng.standard_normal((B, H, L, d)).astype(np.float32)
    v = rng.standard_normal((B, H, L, d)).astype(np.float32)
    m = (np.round(rng.uniform(0, 3, (B, H, L)) * 8) / 8).astype(np.float32)
    for block, init in ((128, 200), (300, 256)):
        log(f"prefill w {w} block {block} init {init}")
        _prefill_case(kdn, orc, q, k, v, m, 7, block, w, "f32", None, (init, rng))


def test_prefill_recency(kdn, orc):
    """The recency control (A Hippocampus for Linear Attention, sec. 4.5) over a prompt."""
    rng = np.random.Generator(np.random.PCG64(304))
    B, H, L, d, w = 1, 3, 200, 64, 12
    q, k, v = (rng.standard_normal((B, H, L, d)).astype(np.float32) for _ in range(3))
    m = rng.uniform(0, 1, (B, H, L)).astype(np.float32)
    for block, init in ((1, None), (32, 6), (128, None)):
        got = _prefill_case(kdn, orc, q, k, v, m, 50, block, w, "f32",
                            init=None if init is None else (init, rng), policy="recency")
        np.testing.assert_array_equal(got["pos"][0, 0], np.arange(50 + L - 1, 50 + L - 1 - w, -1))


def test_prefill_odd_shapes(kdn, orc):
    rng = np.random.Generator(np.random.PCG64(302))
    B, H, L, dk, dv, w = 1, 2, 70, 40, 24, 5
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    m = rng.uniform(0, 1, (B, H, L)).astype(np.float32)
    _prefill_case(kdn, orc, q, k, v, m, 0, 9, w, "f32", rng.standard_normal(H).astype(np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_unaligned_rows(kdn, orc, dtype):
    """Key and value widths that are not multiples of 4 (the element-wise
    gather), and d_k > 64 (two contraction passes for the logits)."""
    rng = np.random.Generator(np.random.PCG64(305))
    B, H, L, dk, dv, w = 1, 2, 150, 66, 18, 7
    q = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, L, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, L, dv)).astype(np.float32)
    m = rng.uniform(0, 1, (B, H, L)).astype(np.float32)
    for block, init in ((32, None), (100, 4)):
        _prefill_case(kdn, orc, q, k, v, m, 3, block, w, dtype,
                      rng.standard_normal(H).astype(np.float32),
                      init=None if init is None else (init, rng))


def test_prefill_value_range(kdn, orc):
    """Value rows from 1e-20 to 1e30 (far outside fp16 range, where the read's
    split products scale each key tile by a power of two) and one whole block
    of tiny values: every query's output against the oracle, relative to that
    query's own output size."""
    import torch
    rng = np.random.Generator(np.random.PCG64(306))
    B, H, L, d, w = 1, 2, 260, 64, 12
    q = rng.standard_normal((B, H, L, d)).astype(np.float32)
    k = rng.standard_normal((B, H, L, d)).astype(np.float32)
    mag = 10.0 ** rng.uniform(-20, 30, (B, H, L, 1))
    mag[:, :, 64:128] = 1e-25  # the second block: tiny values only
    v = (rng.standard_normal((B, H, L, d)) * mag).astype(np.float32)
    m = rng.uniform(0, 1, (B, H, L)).astype(np.float32)
    cache = kdn.HolaCache(B, H, d, d, w)
    oc = kdn.hola_prefill(dev_tensor(q), dev_tensor(k), dev_tensor(v), dev_tensor(m), 0, cache, block=64)
    torch.cuda.synchronize()
    got = host(oc).astype(np.float64)
    ref = orc.HolaCache(B, H, d, d, w).prefill(q, k, v, m.astype(np.float64), 0, 64, None)
    assert np.all(np.isfinite(got))
    scale = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    err = np.max(np.abs(got - ref) / scale)
    log(f"  value range 1e-20..1e30: worst per-query max|diff|/RMS = {err:.3e} (tol {TOL_F32:.0e})")
    assert err <= TOL_F32


def test_scan_scores_then_prefill(kdn, orc):
    """The scan's scores feed the cache: gated delta scan with scores, then the
    prompt cache, both checked against the oracle (scores to the bf16 bar,
    membership exactly on the GPU's own scores)."""
    import torch
    inp = workloads.scan_inputs(2, 2, 520, 128, 128, seed=303, dtype="bf16")
    q, k, v = (dev_tensor(inp[n], "bf16") for n in ("q", "k", "v"))
    o, m = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                            m=True)
    torch.cuda.synchronize()
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    assert_close(host(m), ref["m"], TOL_BF16, "scan m")
    m_gpu = host(m).astype(np.float32)
    _prefill_case(kdn, orc, inp["q"], inp["k"], inp["v"], m_gpu, 0, 256, 64, "bf16")


def test_full_size_gated_prefill(kdn, orc):
    """The gated workload (B=4, H=16, L=4096, d=128, bf16): scan with scores, then
    the prompt cache with blocks of 256 and w = 64; the scores checked on every
    head, the cache (membership, order, contents, o_cache) on every head."""
    import torch
    cfg = workloads.WORKLOADS["gated"]
    inp = workloads.named_scan_inputs("gated")
    q, k, v = (dev_tensor(inp[n], "bf16") for n in ("q", "k", "v"))
    log("gated: scan with scores")
    o, m = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]),
                            m=True)
    torch.cuda.synchronize()
    m_host = host(m)
    log("gated: oracle scores on every head")
    ref = orc.scan(inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"])
    assert_close(m_host, ref["m"], TOL_BF16, "m (all heads)")
    del ref
    log("gated: prompt cache, every head")
    _prefill_case(kdn, orc, inp["q"], inp["k"], inp["v"], m_host.astype(np.float32), 0, 256, 64,
                  "bf16")
