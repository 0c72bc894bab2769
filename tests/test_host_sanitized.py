"""The host path of libfx on the CPU, under the address and undefined-behaviour
sanitizers: csrc/fx_api.cpp (plan creation, argument validation, workspace layout and
every entry point) built with g++ against stand-ins for the device calls
(tests/host/dev_stub.cpp), driven by tests/host/host_check.cpp, which forces every
fx_status code and checks the plan layouts and the workspace split."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "block_sparse_decode_summary_amd", "csrc")


@pytest.fixture(scope="module")
def host_check(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("host") / "host_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-Wall", "-Wextra", "-Werror",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{HOST}",
           os.path.join(HOST, "host_check.cpp"), os.path.join(HOST, "dev_stub.cpp"),
           os.path.join(CSRC, "fx_api.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_host_path_under_sanitizers(host_check):
    # verify_asan_link_order=0: another preloaded library may come before the ASan runtime.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([host_check], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
