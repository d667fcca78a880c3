"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The C ABI layer (mamba_ssd_chunked_fwd_amd/csrc/ssd_api.cpp) is built with
  g++ against stand-in launchers (tests/sanitize/stub_launchers.cpp) and
  driven through every entry point's checks and dispatch
  (tests/sanitize/abi_driver.cpp).
* The fp64 oracle is built instrumented (oracle.build(sanitize=True)) and
  its pin tests run in a child process with the sanitizer runtimes
  preloaded.

Either run stops at the first memory or undefined-behaviour error.  The
same commands by hand:

    g++ -std=c++17 -O1 -fsanitize=address,undefined -fno-sanitize-recover=undefined \\
        -fno-omit-frame-pointer -g -I include -I mamba_ssd_chunked_fwd_amd/csrc \\
        -I tests/sanitize tests/sanitize/abi_driver.cpp tests/sanitize/stub_launchers.cpp \\
        mamba_ssd_chunked_fwd_amd/csrc/ssd_api.cpp -o /tmp/abi_driver && /tmp/abi_driver
    python -c "import oracle; oracle.build(force=True, sanitize=True)"
    env SSD_ORACLE_SANITIZE=1 ASAN_OPTIONS=detect_leaks=0 \\
        LD_PRELOAD=$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so) \\
        python -m pytest tests -m "not gpu" -q
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _have_sanitizers() -> bool:
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        return False
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    return p.returncode == 0 and os.path.isabs(p.stdout.strip())


pytestmark = pytest.mark.skipif(not _have_sanitizers(), reason="gcc sanitizer runtimes missing")


def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "mamba_ssd_chunked_fwd_amd", "csrc"), "-I", SAN,
           os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "stub_launchers.cpp"),
           os.path.join(ROOT, "mamba_ssd_chunked_fwd_amd", "csrc", "ssd_api.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_oracle_pins_under_sanitizers():
    sys.path.insert(0, ROOT)
    import oracle
    oracle.build(force=True, sanitize=True)
    env = oracle.sanitizer_env()
    mods = ["tests/test_oracle_pins.py", "tests/test_oracle_conv_pins.py",
            "tests/test_oracle_gdn_pins.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *mods], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
