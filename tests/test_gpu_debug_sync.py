"""CSA2_DEBUG_SYNC=1: every library call synchronises its stream and reports
runtime errors; the Full-layer decode of the tiny workload still matches the
oracle in that mode.  The variable is read once per process, so the check runs
in a child process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_full_layer_decode_under_debug_sync():
    pytest.importorskip("kv_cache_decode_mxfp4_amd")
    env = dict(os.environ, CSA2_DEBUG_SYNC="1")
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.smoke()"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "smoke ok" in r.stdout
