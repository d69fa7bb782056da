"""The library's host code (encoder, section views, validator, table builder)
under sanitizers: tests/native/host_stress.cpp is compiled with g++ together
with the host sources (no HIP code) and run under AddressSanitizer + UBSan and
under ThreadSanitizer (the encoder is multithreaded)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "huffman_decode_block_amd", "csrc")
HOST_SOURCES = [os.path.join(CSRC, f) for f in ("df11_encode.cpp", "df11_capi.cpp", "df11_tables.cpp")]
DRIVER = os.path.join(ROOT, "tests", "native", "host_stress.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
@pytest.mark.parametrize("sanitizers,blocks", [("address,undefined", 40), ("thread", 16)])
def test_host_code_under_sanitizers(tmp_path, sanitizers, blocks):
    exe = str(tmp_path / "host_stress")
    cmd = ["g++", "-O1", "-g", "-std=c++17", f"-fsanitize={sanitizers}", "-fno-omit-frame-pointer", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, DRIVER, *HOST_SOURCES, "-o", exe]
    if "undefined" in sanitizers:
        cmd.insert(4, "-fno-sanitize-recover=undefined")
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe, str(blocks)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 problems" in r.stdout, r.stdout
