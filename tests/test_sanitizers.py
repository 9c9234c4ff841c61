"""CPU sanitizer runs (no GPU): AddressSanitizer and UndefinedBehaviorSanitizer
over the oracle (gcc) and over the host side of the C-ABI library (hipcc with
the sanitizers on the host pass only; the device code is built as usual and
never launched).  Each runs in a subprocess with the sanitizer runtime
preloaded; any report aborts it."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ENV_COMMON = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0",
              "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(script, preload, *args, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV_COMMON)
    p = subprocess.run([sys.executable, "-c", script, *args], env=env, cwd=ROOT, timeout=timeout,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return p.returncode, p.stdout


PINS = """
import sys
sys.path.insert(0, %r); sys.path.insert(0, %r)
import oracle, oracle_pins
oracle._lib = oracle.load_library(sys.argv[1])
for check in oracle_pins.ALL_CHECKS:
    check()
print("pins ok", len(oracle_pins.ALL_CHECKS))
""" % (ROOT, os.path.join(ROOT, "tests"))


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()
    rc, out = _run(PINS, asan, lib)
    assert rc == 0 and "pins ok" in out, out[-3000:]


ABI = """
import sys
sys.path.insert(0, %r); sys.path.insert(0, %r)
import torch  # noqa: F401
from moe_lora_layer_amd import ops
ops.LIB_PATH = sys.argv[1]
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", %r])
assert ops.library()._name == sys.argv[1]
sys.exit(rc)
""" % (ROOT, os.path.join(ROOT, "tests"), os.path.join(ROOT, "tests", "test_abi.py"))


def _clang_asan_runtime():
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True).stdout.strip()
    if os.path.isabs(out) and os.path.exists(out):
        return out
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_abi_under_asan_ubsan(tmp_path):
    """Every argument check, workspace size, layout and plan of the C ABI
    (tests/test_abi.py) with the host code built under ASan + UBSan."""
    runtime = _clang_asan_runtime()
    if runtime is None:
        pytest.skip("clang ASan runtime not found")
    csrc = os.path.join(ROOT, "moe_lora_layer_amd", "csrc")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                "-fno-omit-frame-pointer"]
    objs = []
    procs = []
    for name in sorted(os.listdir(csrc)):
        if not name.endswith(".hip"):
            continue
        obj = str(tmp_path / (name + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
             "-I" + os.path.join(ROOT, "include"), "-I" + csrc, "-c", os.path.join(csrc, name),
             "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out[-3000:]
    lib = str(tmp_path / "libmoelora_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host",
                    "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan",
                    "-o", lib, *objs], check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    rc, out = _run(ABI, runtime, lib)
    assert rc == 0 and "passed" in out, out[-3000:]
