"""Host-side behaviour of the entry points that needs no GPU: the benchmark
refuses several GPUs, and the package does not import without its native
library (there is no fallback path)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable] + args, cwd=ROOT, env=e, capture_output=True,
                          text=True, timeout=300)


def test_bench_refuses_several_gpus():
    r = _run(["bench.py", "--gpus", "2"])
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for an unmeasured run


def test_package_needs_native_library():
    r = _run(["-c", "import kv_cache_compression_hkv_amd"],
             env={"HKV_LIBRARY": os.path.join(ROOT, "no_such_dir", "libhkv.so")})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr
