"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: csrc/api.cpp (host code, which holds every check) is compiled with both sanitizers
and linked with the regular kernel objects of the library build into a small C driver
(tests/abi_sanitize/driver.c) that calls every entry point with invalid options, null and
misaligned pointers, short workspaces, empty problems, every workspace-size combination and a
problem beyond the allocation-free prologue's scratch. No call reaches the HIP runtime or a
kernel. The driver must print "ok", exit 0, and the sanitizers must report nothing."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "abi_sanitize")
KERNEL_OBJS = [os.path.join(BUILD, f) for f in ("prologue.hip.o", "forward.hip.o", "backward.hip.o")]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


def test_abi_validation_under_asan_ubsan():
    if not all(os.path.exists(o) for o in KERNEL_OBJS):
        from bit_trainable_attention_amd import build as b
        b.build(verbose=False)
    os.makedirs(OUT, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "bit_trainable_attention_amd", "csrc")]
    api_o, drv_o, exe = (os.path.join(OUT, n) for n in ("api.cpp.o", "driver.o", "driver"))
    _run(["hipcc", "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", *inc, *SAN, "-c",
          os.path.join(ROOT, "bit_trainable_attention_amd", "csrc", "api.cpp"), "-o", api_o])
    _run(["hipcc", "-x", "c", "-O1", "-g", *inc, *SAN, "-c", os.path.join(ROOT, "tests", "abi_sanitize", "driver.c"),
          "-o", drv_o])
    _run(["hipcc", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", drv_o, api_o,
          *KERNEL_OBJS, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
    for marker in ("AddressSanitizer", "LeakSanitizer", "runtime error"):
        assert marker not in r.stderr, r.stderr
