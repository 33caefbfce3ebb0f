"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle (oracle/oracle.c) and libbq's host packer (bq_pack.cpp) are each built
into a small driver program with gcc / g++ -fsanitize=address,undefined and
run; any report aborts the driver.  Host code only: no GPU code is built."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _have_asan(tmp_path) -> bool:
    src = tmp_path / "probe.c"
    src.write_text("int main(void) { return 0; }\n")
    r = subprocess.run(["gcc", *SAN, str(src), "-o", str(tmp_path / "probe")], capture_output=True)
    return r.returncode == 0


def _run(cmd_build, exe):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout[-2000:], r.stderr[-4000:])


@pytest.fixture(scope="module")
def asan_ok(tmp_path_factory):
    if not shutil.which("gcc") or not _have_asan(tmp_path_factory.mktemp("probe")):
        pytest.skip("gcc has no AddressSanitizer runtime here")


def test_oracle_under_sanitizers(asan_ok, tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-lpthread", "-o", exe], exe)


def test_packer_under_sanitizers(asan_ok, tmp_path):
    exe = str(tmp_path / "pack_asan")
    _run(["g++", *SAN, "-std=c++17", os.path.join(ROOT, "ternary_quantized_gemv_amd", "csrc", "bq_pack.cpp"),
          os.path.join(HERE, "pack_driver.cpp"), "-o", exe], exe)
