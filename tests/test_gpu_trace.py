"""Launch tracing: with KDN_TRACE=1 the library writes one stderr line per
kernel launch (kernel, grid, workgroup, LDS bytes, stream) and one per scan
call naming the path it took; without it, nothing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch, workloads
import delta_rule_scans_amd as kdn
from _util import dev_tensor
inp = workloads.scan_inputs(1, 2, 200, 128, 64, seed=7, dtype="bf16")
q, k, v = (dev_tensor(inp[n], "bf16") for n in ("q", "k", "v"))
o = kdn.kdn_scan_fwd(q, k, v, alpha=dev_tensor(inp["alpha"]), beta=dev_tensor(inp["beta"]))
torch.cuda.synchronize()
print("done", float(o.float().abs().sum()) > 0)
"""


def _run(trace):
    env = dict(os.environ)
    env.pop("KDN_TRACE", None)
    if trace:
        env["KDN_TRACE"] = "1"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, os.path.join(ROOT, "tests")])
    return subprocess.run([sys.executable, "-c", _CHILD, ROOT], capture_output=True, text=True,
                          timeout=240, env=env)


@pytest.mark.gpu
def test_trace_logs_launches():
    r = _run(True)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "done True" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("kdn: ")]
    call = [l for l in lines if "kdn_scan_fwd" in l]
    assert call and "matrix-core path" in call[0] and "L 200" in call[0], lines
    launches = [l for l in lines if l.startswith("kdn: launch ")]
    names = " ".join(launches)
    assert "prep_kernel" in names and "state_kernel" in names, lines
    state = [l for l in launches if "state_kernel" in l][0]
    # two heads of 64 value columns: two 32-column slices each, or four
    # 16-column ones when the 32-column tiling would fill at most half the
    # device (as here); one LDS-resident workgroup per CU either way
    grid = "grid (8,1,1)" if "(16 columns)" in state else "grid (4,1,1)"
    assert grid in state and " lds " in state, state
    assert int(state.split(" lds ")[1].split()[0]) > 64 * 1024, state


@pytest.mark.gpu
def test_no_trace_without_the_variable():
    r = _run(False)
    assert r.returncode == 0, r.stderr[-2000:]
    assert not [l for l in r.stderr.splitlines() if l.startswith("kdn: ")]
