"""The debug build (Q4DEC_DEBUG=1): every kernel checks its launch contract
on the device (staging capacity, full plans, grid coverage of rows, tiles
and K slices) and records failures for q4dec_debug_status(). One child
python loads libq4dec_debug.so, calls every kernel family over the model
shapes and ragged ones, and reports: no check may fail, the build must still
compute the GEMV within its bar, and the self-test's deliberate failure must
be reported (bit 31) and then cleared."""
import json
import os
import subprocess
import sys

import pytest

from int4_weight_only_block_amd import build as q4build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not os.path.exists(q4build.DEBUG_LIB_PATH),
                                 reason="libq4dec_debug.so not built (build(debug=True))")]


def test_debug_build_checks_pass_and_report():
    env = dict(os.environ, Q4DEC_LIB=q4build.DEBUG_LIB_PATH,
               PYTHONPATH=os.pathsep.join(p for p in (ROOT, os.environ.get("PYTHONPATH")) if p))
    res = subprocess.run([sys.executable, "-u", os.path.join(HERE, "gpu_debug_child.py")], env=env,
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-3000:]
    out = json.loads(res.stdout.strip().splitlines()[-1])
    assert out["lib"] == q4build.DEBUG_LIB_PATH
    assert out["start"] == [0, 0]
    assert out["after_calls"] == [0, 0], f"launch-contract bits set: {out['after_calls'][1]:#x}"
    assert out["gemv_within_bar"]
    assert out["selftest"] == [0, 0, 1 << 31]
    assert out["cleared"] == [0, 0]
