"""Host logic of the KV block pool and pooled sessions (prefix sharing, publishing, copy on
write, eviction), checked on the CPU: tests/native/kv_pool_check.cpp drives the library's own
header (dense_gqa_decoder_amd/csrc/kv_pool.h) through random operations against a brute-force
model of every block's contents, built with g++ and AddressSanitizer + UBSan."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_kv_pool_randomised_against_brute_force(tmp_path):
    exe = tmp_path / "kv_pool_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "dense_gqa_decoder_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "kv_pool_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe), "200000"], capture_output=True, text=True, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("ok")
