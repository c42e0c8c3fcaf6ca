"""Sanitizer builds of the host code, run on the CPU.

- The C-ABI front end (csrc/api.cpp: validation, launch planning, workspace
  carving, the plan log) is built with g++ under AddressSanitizer and
  UndefinedBehaviorSanitizer, with the HIP runtime calls and the kernel
  launchers replaced by host stubs (tests/native/abi_host_check.cpp). The stubs
  write every byte of workspace a kernel would write into an allocation of
  exactly the queried size, over sweeps of shapes, compute-unit counts and
  planner overrides.
- The oracle (oracle/attention.c) is built under ASan + UBSan and under
  ThreadSanitizer (tests/native/oracle_host_check.c).
- FA_LOG=1 prints one plan line per call.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "flashattention_forward_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
ROCM_INCLUDE = "/opt/rocm/include"

SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not installed")


def _run(cmd, timeout, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    return r


def _build(cmd):
    r = _run(cmd, 300)
    assert r.returncode == 0, f"build failed: {' '.join(cmd)}\n{r.stderr}"


@pytest.fixture(scope="module")
def abi_check(tmp_path_factory):
    _need("g++")
    if not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("HIP runtime headers not found")
    exe = str(tmp_path_factory.mktemp("abi") / "abi_host_check")
    _build(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            f"-I{ROCM_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"] + SAN +
           [os.path.join(CSRC, "api.cpp"), os.path.join(NATIVE, "abi_host_check.cpp"),
            "-o", exe])
    return exe


def test_front_end_under_asan_ubsan(abi_check):
    env = {k: v for k, v in ENV.items() if not k.startswith("FA_")}
    r = _run([abi_check, "sweep"], 240, env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert "ERROR" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-6000:]
    n = int(r.stdout.split("checked")[1].split()[0])
    assert n > 100000


def test_plan_log(abi_check):
    env = {k: v for k, v in ENV.items() if not k.startswith("FA_")}
    quiet = _run([abi_check, "log"], 60, env)
    assert quiet.returncode == 0 and "fa_log" not in quiet.stderr
    env["FA_LOG"] = "1"
    env["FA_NUM_CUS"] = "256"
    r = _run([abi_check, "log"], 60, env)
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("fa_log ")]
    assert len(lines) == 2, r.stderr
    pf = dict(kv.split("=") for kv in lines[0].split()[2:])
    assert lines[0].split()[1] == "prefill"
    # 512 queries x 32 heads (groups of 4) over 16384 keys: 8-wave workgroups
    # in head packs of 4, 8 query tiles of 64 rows; 32 one-head tiles of 256
    # rows leave the 256 CUs short, so the keys are split 4 ways.
    assert pf["cus"] == "256" and pf["waves"] == "8" and pf["pack"] == "4"
    assert pf["qtiles"] == "8" and pf["splits"] == "4" and pf["workgroups"] == "256"
    assert int(pf["ws_bytes"]) == 4 * 512 * 32 * (128 * 2 + 4)
    dc = dict(kv.split("=") for kv in lines[1].split()[2:])
    assert lines[1].split()[1] == "decode"
    assert dc["layout"] == "mla" and dc["B"] == "128" and dc["heads_per_wg"] == "64"
    # No workspace: the call runs unsplit.
    assert dc["splits"] == "1" and dc["ws_bytes"] == "0"


@pytest.mark.parametrize("kind", ["asan_ubsan", "tsan"])
def test_oracle_under_sanitizers(kind, tmp_path):
    _need("gcc")
    exe = str(tmp_path / f"oracle_{kind}")
    flags = SAN if kind == "asan_ubsan" else ["-O1", "-g", "-fsanitize=thread"]
    _build(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror"] + flags +
           [os.path.join(ROOT, "oracle", "attention.c"),
            os.path.join(NATIVE, "oracle_host_check.c"), "-lm", "-lpthread", "-o", exe])
    r = _run([exe], 120, ENV)
    if kind == "tsan" and r.returncode != 0 and "FATAL: ThreadSanitizer" in r.stderr:
        pytest.skip("ThreadSanitizer cannot run in this environment: " + r.stderr[:200])
    assert r.returncode == 0, r.stdout + r.stderr[-6000:]
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-6000:]
    assert r.stdout.startswith("oracle ok:")
