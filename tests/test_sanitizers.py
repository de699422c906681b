"""Host code under the sanitizers (CPU only, g++ / gcc; no device code).

- the slot-cache policy (csrc/slot_policy.h) on a seeded random walk of map,
  release, prefetch, evict and resize calls, with AddressSanitizer and
  UndefinedBehaviorSanitizer;
- the host expert FFN and its job queue (csrc/host_ffn.cpp: a spinning thread
  pool with atomics and condition variables), with ASan + UBSan and with
  ThreadSanitizer, jobs submitted from several threads at once;
- the CPU oracle (oracle/oracle.c) on small layers of every weight format,
  with ASan + UBSan.
Each driver exits non-zero on a failed check; a sanitizer report aborts it.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
NATIVE = os.path.join(HERE, "native")
OUT = os.path.join(NATIVE, "_build")
INC = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "expert_ffn_execution_amd", "csrc")
ORACLE = os.path.join(ROOT, "oracle")
ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
TSAN = ["-fsanitize=thread"]


def _build_run(name, cmd):
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, name)
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    assert "Sanitizer" not in r.stderr, r.stderr[-6000:]
    return r.stdout


pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs g++ and gcc")


def test_slot_policy_asan_ubsan():
    out = _build_run("san_policy", ["g++", "-O1", "-g", "-std=c++17", *ASAN, f"-I{INC}",
                                    os.path.join(NATIVE, "san_policy.cpp")])
    assert "policy walk ok" in out


def test_host_ffn_asan_ubsan():
    out = _build_run("san_host_ffn_asan", ["g++", "-O1", "-g", "-std=c++17", "-pthread", *ASAN,
                                           f"-I{INC}", os.path.join(NATIVE, "san_host_ffn.cpp"),
                                           os.path.join(CSRC, "host_ffn.cpp")])
    assert "host ffn ok" in out


def test_host_ffn_tsan():
    out = _build_run("san_host_ffn_tsan", ["g++", "-O1", "-g", "-std=c++17", "-pthread", *TSAN,
                                           f"-I{INC}", os.path.join(NATIVE, "san_host_ffn.cpp"),
                                           os.path.join(CSRC, "host_ffn.cpp")])
    assert "host ffn ok" in out


def test_oracle_asan_ubsan():
    out = _build_run("san_oracle", ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", *ASAN,
                                    f"-I{ORACLE}", os.path.join(NATIVE, "san_oracle.c"),
                                    os.path.join(ORACLE, "oracle.c"), "-lm"])
    assert "oracle ok" in out
