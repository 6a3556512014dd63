"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the fp64 oracle and a host-only copy of the C-ABI layer (gdn_api.cpp linked with
launchers that report no device, tests/sanitize/stub_launch.cpp) with gcc/g++
-fsanitize=address,undefined, then reruns the oracle pins and the C-ABI tests against those
builds in a child process that preloads the ASan runtime. Any sanitizer report aborts the
child and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "gated_deltanet_recurrent_02_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1", "-fPIC", "-shared"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(path):
        pytest.skip("gcc has no shared ASan runtime")
    return path


def _build_oracle(src, out):
    subprocess.run(["gcc", *SAN, "-std=c99", "-ffp-contract=off", "-o", out, src, "-lm"],
                   check=True)


def _build_abi(out):
    subprocess.run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-o", out,
                    os.path.join(CSRC, "gdn_api.cpp"), os.path.join(HERE, "sanitize", "stub_launch.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)


def _run_child(lib_oracle, lib_gdn, files):
    env = dict(os.environ, LD_PRELOAD=_runtime(), GDN_SAN_ORACLE=lib_oracle, GDN_SAN_LIBGDN=lib_gdn,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=os.pathsep.join([os.path.join(HERE, "sanitize"), HERE, ROOT]))
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "sanitize_plugin", "-m", "not gpu",
           "-p", "no:cacheprovider", *(os.path.join(HERE, f) for f in files)]
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)


def test_oracle_and_abi_under_asan_ubsan(tmp_path):
    lib_oracle = str(tmp_path / "liboracle_san.so")
    lib_gdn = str(tmp_path / "libgdn_san.so")
    _build_oracle(os.path.join(ROOT, "oracle", "gdn_oracle.c"), lib_oracle)
    _build_abi(lib_gdn)
    r = _run_child(lib_oracle, lib_gdn, ["test_oracle_pins.py", "test_abi.py"])
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-40:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail


def test_planted_overflow_is_reported(tmp_path):
    # The harness itself: an oracle copy that clears one row past its scratch state must make
    # the sanitized child abort with an AddressSanitizer report.
    with open(os.path.join(ROOT, "oracle", "gdn_oracle.c")) as f:
        src = f.read()
    old = "for (int32_t i = 0; i < dv; ++i)\n        for (int32_t j = 0; j < dk; ++j) S[(size_t)i * dk + j] = 0.0;"
    assert src.count(old) == 1
    bad = tmp_path / "gdn_oracle_overflow.c"
    bad.write_text(src.replace(old, old.replace("i < dv", "i <= dv")))
    lib_oracle = str(tmp_path / "liboracle_bad.so")
    lib_gdn = str(tmp_path / "libgdn_san.so")
    _build_oracle(str(bad), lib_oracle)
    _build_abi(lib_gdn)
    r = _run_child(lib_oracle, lib_gdn, ["test_oracle_pins.py"])
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr
