"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop models
behind the roofline fields, the digest that keeps the committed counter record
tied to the kernel source it was taken on, and the refusal of more than one
GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_scan_bytes_headline():
    """Gated workload B=4 H=16 L=4096 d=128, the roofline's unit: bf16 q, k, v
    read once (768 B per token and head), float32 alpha and beta (8 B), bf16 o
    written once (256 B): 1032 B, plus the float32 final state of every head;
    with the float32 output the library writes by default, 1288 B."""
    B, H, L, d = 4, 16, 4096, 128
    tokens = B * H * L
    expect = tokens * (3 * d * 2 + 8 + d * 2) + B * H * d * d * 4
    assert bench.scan_bytes(B, H, L, d, d) == expect == 274_726_912
    assert bench.scan_bytes(B, H, L, d, d, state_out=False) == tokens * 1032
    assert bench.scan_bytes(B, H, L, d, d, out_bytes=4) == 341_835_776
    assert bench.scan_bytes(B, H, L, d, d, out_bytes=4, state_out=False) == tokens * 1288


def test_scan_flops_per_token_head():
    """The algorithmic flop count the MFMA fractions use: 1.406e5 per token and
    head at C = 64, d_k = d_v = 128 (triangles counted once). Its state
    products (K S, Q S, B^T U: 2 d_k d_v each) do not depend on the chunk, the
    intra-chunk terms grow linearly in C except the triangular inverse
    (C^3 / 3 per chunk, C^2 / 3 per token)."""
    f = bench.scan_flops_per_token_head
    assert f(64, 128, 128) == pytest.approx(1.406e5, rel=1e-3)
    assert f(1, 0, 0) == pytest.approx(1 / 3)  # the inverse alone
    state = f(0, 128, 128)
    assert state == 6 * 128 * 128
    # linear part: f(C) - state - C^2/3 is proportional to C
    lin = lambda C: f(C, 128, 128) - state - C * C / 3  # noqa: E731
    assert lin(64) == pytest.approx(2 * lin(32)) == pytest.approx(4 * lin(16))


def test_decode_bytes_per_head():
    """One decode + cache step per head at d = 128, w = 64: the float32 state
    read and written (131072 B), the cache's keys and values read (65536 B),
    its scores and positions read (512 B), the token's q, k, v, alpha, beta
    (1544 B), o and o_cache written with the score written and read back
    (1032 B), and the insert: key and value rows, score and position, the
    fill count read and written (1040 B): 200736 B."""
    assert bench.DECODE_BYTES_PER_HEAD == 131072 + 65536 + 512 + 1544 + 1032 + 1040 == 200_736


def test_code_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("// header\nint f(int x)\n{\n\treturn x+1;\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.code_digest(str(a)) == bench.code_digest(str(b))
    assert bench.code_digest(str(a)) != bench.code_digest(str(c))


def test_counter_record_fields():
    """The committed record names its kernel source, and its byte counts are
    the scaled counter values of one launch (positive, and not below the
    algorithmic bytes of the kernel by more than the record allows)."""
    import json
    path = os.path.join(ROOT, "profiles", "scan_gated_B4H16L4096_traffic.json")
    rec = json.load(open(path))
    for key in ("kernel", "hbm_read_bytes", "hbm_write_bytes", "source", "code_sha256",
                "fetch_scale", "write_scale", "mfma_executed_flops", "mfma_busy_frac"):
        assert key in rec, key
    assert os.path.exists(os.path.join(ROOT, rec["source"]))
    assert rec["hbm_read_bytes"] > 0 and rec["hbm_write_bytes"] > 0
    # o (float32) and the final state are written at least once
    assert rec["hbm_write_bytes"] >= 4 * 16 * 4096 * 128 * 4
    assert 0.0 < rec["mfma_busy_frac"] < 1.0


def test_gpus_above_one_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
