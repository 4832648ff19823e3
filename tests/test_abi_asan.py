"""The C ABI tests again, against a build of the library whose host code runs
under AddressSanitizer (argument checks, planning, the thread-local error
text): any out-of-bounds access or use after free on the host side aborts the
run.  CPU only; the GPU code is built as usual and never launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_address_sanitizer(tmp_path):
    from token_verify_attention_amd import build
    runtime = build.asan_runtime()
    if runtime is None or not os.path.exists(build.HIPCC):
        pytest.skip("no AddressSanitizer runtime or hipcc")
    lib = build.build(out_dir=str(tmp_path / "lib"), obj_dir=str(tmp_path / "obj"), asan=True,
                      jobs=8)
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               TVA_LIB=lib, LD_LIBRARY_PATH=os.path.dirname(runtime))
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                          "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:]
    assert "AddressSanitizer" not in res.stdout
    assert " passed" in res.stdout
