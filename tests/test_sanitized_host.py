"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

kvq_api.cpp is compiled with g++ and the sanitizers into a host-only library whose kernel
launchers are stubs that return an error (no GPU code is built), and the ABI tests
(validation, plane sizes, the host-side permutation, dynamic codebook and bit allocation,
refusals) plus the fast-division check run against it in a child process with the ASan
runtime preloaded.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

from tests.conftest import ROOT
from tests.test_fastdiv import HEADER, PROGRAM

CSRC = os.path.join(ROOT, "rotate_then_bit_amd", "csrc")

STUBS = r"""
#include "kvq_internal.h"
namespace kvq {
#define KVQ_STUB(NAME) int NAME(int, int, int, const CodecArgs&, void*) { return 98; }
KVQ_STUB(launch_encode_f16_d128) KVQ_STUB(launch_encode_f16_d256) KVQ_STUB(launch_encode_bf16_d128)
KVQ_STUB(launch_encode_bf16_d256) KVQ_STUB(launch_encode_f32_d128) KVQ_STUB(launch_encode_f32_d256)
KVQ_STUB(launch_decode_f16_d128) KVQ_STUB(launch_decode_f16_d256) KVQ_STUB(launch_decode_bf16_d128)
KVQ_STUB(launch_decode_bf16_d256) KVQ_STUB(launch_decode_f32_d128) KVQ_STUB(launch_decode_f32_d256)
const char* device_error_string(int) { return "host-only build: no device"; }
int launch_attend(int, int, const AttendArgs&, void*) { return 98; }
int launch_encode_dense(int, int, int, const CodecArgs&, void*) { return 98; }
int launch_decode_dense(int, int, int, const CodecArgs&, void*) { return 98; }
int launch_attend_gen_d128_k2(int, int, const AttendArgs&, void*) { return 98; }
int launch_attend_gen_d128_k3(int, int, const AttendArgs&, void*) { return 98; }
int launch_attend_gen_d128_k4(int, int, const AttendArgs&, void*) { return 98; }
int launch_attend_gen_d256_k2(int, int, const AttendArgs&, void*) { return 98; }
int launch_attend_gen_d256_k3(int, int, const AttendArgs&, void*) { return 98; }
int launch_attend_gen_d256_k4(int, int, const AttendArgs&, void*) { return 98; }
int attend_scratch(void**) { return 98; }
int launch_channel_stats(const CalibArgs&, void*) { return 98; }
int launch_detect_sinks(const CalibArgs&, void*) { return 98; }
int launch_rotated_moments(const CalibArgs&, void*) { return 98; }
int launch_entropy(const EntropyArgs&, void*) { return 98; }
}
"""

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime")
    stub = tmp_path / "stubs.cpp"
    stub.write_text(STUBS)
    lib = tmp_path / "libkvq_host_san.so"
    subprocess.run(["g++", "-std=c++17", "-g", "-O1", "-fPIC", "-shared", *SAN, f"-I{CSRC}",
                    os.path.join(CSRC, "kvq_api.cpp"), str(stub), "-o", str(lib)], check=True)
    fd_src = tmp_path / "fastdiv.cpp"
    fd_src.write_text(PROGRAM % HEADER)
    fd = tmp_path / "fastdiv"
    subprocess.run(["g++", "-std=c++17", "-O1", *SAN, str(fd_src), "-o", str(fd)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([str(fd)], capture_output=True, text=True, env=env, timeout=600)
    assert out.returncode == 0 and "runtime error" not in out.stderr and "ERROR: AddressSanitizer" not in out.stderr, \
        out.stderr[-3000:]
    env = dict(env, LD_PRELOAD=asan, KVQ_TEST_LIBRARY=str(lib), PYTHONDONTWRITEBYTECODE="1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-k", "not single_hip_runtime"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = p.stdout + p.stderr
    assert "ERROR: AddressSanitizer" not in log and "runtime error:" not in log, log[-4000:]
    assert p.returncode == 0, log[-4000:]
    assert " passed" in p.stdout
