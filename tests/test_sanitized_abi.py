"""The C-ABI tests again, against the library built with AddressSanitizer and
UndefinedBehaviorSanitizer in its host code (argument validation, size and
workspace arithmetic, the thread-local error text).  No GPU is used: every
call in tests/test_abi.py either returns before any device work or is a pure
host query.  The sanitized build comes from
``python -m attention_pass_cascaded_amd.build --sanitize`` (build() in
__graft_entry__ makes it too); clang's ASan runtime is preloaded into a child
Python that runs the ABI tests, so a sanitizer report fails this test."""
import glob
import os
import subprocess
import sys

import pytest

from attention_pass_cascaded_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime():
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


@pytest.mark.skipif(not os.path.exists(B.SANITIZED_LIB), reason="sanitized build absent (build.py --sanitize)")
@pytest.mark.skipif(asan_runtime() is None, reason="clang ASan runtime not found")
def test_abi_under_asan_and_ubsan(tmp_path):
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan_runtime(), RF_ATTN_LIB=B.SANITIZED_LIB,
               ASAN_OPTIONS=f"detect_leaks=0:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={tmp_path}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(f"{tmp_path}/*san*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], r.stderr[-3000:], reports[:5000])
    assert " passed" in r.stdout
