"""The host ABI tests (tests/test_abi_host.py) against a build whose host-side argument checks
(api.cpp) run under AddressSanitizer and UndefinedBehaviorSanitizer: every rejection path is
exercised with the sanitizers watching for out-of-bounds accesses, overflow and other undefined
behaviour. CPU only: no call here reaches the GPU."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not available")


def test_host_abi_checks_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from block_sparse_attention_query_amd import build as b
    lib = b.build_host_sanitized(os.path.join(ROOT, "_build", "hostsan"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the ABI checks are not instrumented"
    env = dict(os.environ)
    env.update({
        "SA_LIB_PATH": lib,
        "LD_PRELOAD": b.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                        "-p", "no:cacheprovider", "-x"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    import re
    m = re.search(r"(\d+) passed", r.stdout)
    assert m and int(m.group(1)) >= 100 and "skipped" not in r.stdout, tail
