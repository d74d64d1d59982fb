"""Host-side checks that need no GPU.

* The work-list rules of the grouped GEMMs (csrc/worklist.h: row tiles per
  expert, the tail decision, the item order, the XCD order, the K split of
  the last round) are re-run by a hipcc-built host program over thousands of
  random expert-count vectors, which checks that the items cover every
  (sorted row, column tile) pair exactly once and that K parts tile [0, nk).
  The device builder (dispatch.hip) calls the same functions.
* The CPU oracle is rebuilt with AddressSanitizer and UBSan and its pin
  tests run against that build (any report aborts the run).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_02_amd", "csrc")
HERE = os.path.dirname(os.path.abspath(__file__))


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def test_worklist_rules_cover_every_row_once(tmp_path):
    exe = str(tmp_path / "worklist_check")
    cmd = [_hipcc(), "-O2", "-std=c++17", "--offload-arch=gfx950", "-I", CSRC,
           os.path.join(HERE, "worklist_check.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    for seed in (1, 2):
        r = subprocess.run([exe, "1500", str(seed)], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and r.stdout.startswith("worklist ok"), r.stdout + r.stderr


_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import oracle
# a call through the sanitized build, and proof that it is the one mapped
x = np.ones((3, 4), np.float32)
r = oracle.forward(x, np.ones((2, 4), np.float32), np.ones((2, 6, 4), np.float32),
                   np.ones((2, 4, 3), np.float32), top_k=1)
assert r["out"].shape == (3, 4)
maps = open("/proc/self/maps").read()
assert {lib!r} in maps, "sanitized oracle not loaded"
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", {pins!r}, {routing!r}]))
"""


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the gcc ASan runtime is not installed")
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "libmoe_oracle_san.so"))
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", MOE_ORACLE_LIB=lib)
    code = _CHILD.format(root=ROOT, lib=lib, pins=os.path.join(HERE, "test_oracle_pins.py"),
                         routing=os.path.join(HERE, "test_oracle_routing_pins.py"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    assert "passed" in r.stdout
