"""CPU builds under AddressSanitizer and UBSan (no GPU).

Three programs under tests/host/ are compiled with gcc / g++ and
``-fsanitize=address,undefined -fno-sanitize-recover=all`` and run:

* ``oracle_check``: the CPU oracle over random and edge-case inputs;
* ``api_check``: the C ABI's host code (argument checks, create / destroy
  error paths, workspace layout, chunking, launch sequence) against recording
  stand-ins for the HIP runtime and the kernel launchers;
* ``index_check``: the index arithmetic the kernels share with the host code
  (tile plan, dense-tile map, sample-run starts, LDS sizes, the staged
  select's prefix) over every tile length and a spread of vocab sizes.

Each prints one ``... ok`` line and exits 0, or names its failed checks.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "decode_token_sampling_row_amd", "csrc")
ROCM_INC = "/opt/rocm/include"

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
CXX = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INC,
       "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + SAN


def _build_run(tmp_path, cmd, exe, expect):
    subprocess.run(cmd + ["-o", str(exe)], check=True, capture_output=True, text=True,
                   timeout=240)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-6000:])
    assert expect in r.stdout, r.stdout


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    cmd = ["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math"] + SAN + [
        os.path.join(HOST, "oracle_check.c"), os.path.join(ROOT, "oracle", "sampler_oracle.c"),
        "-lm"]
    # the link line puts -lm last, after the sources
    _build_run(tmp_path, cmd, tmp_path / "oracle_check", "oracle checks ok")


def test_host_api_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.isdir(os.path.join(ROCM_INC, "hip")):
        pytest.skip("HIP headers not found")
    cmd = CXX + [os.path.join(HOST, "api_check.cpp"), os.path.join(CSRC, "sampler_api.cpp")]
    _build_run(tmp_path, cmd, tmp_path / "api_check", "api checks ok")


def test_index_arithmetic_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.isdir(os.path.join(ROCM_INC, "hip")):
        pytest.skip("HIP headers not found")
    cmd = CXX + [os.path.join(HOST, "index_check.cpp")]
    _build_run(tmp_path, cmd, tmp_path / "index_check", "index checks ok")
