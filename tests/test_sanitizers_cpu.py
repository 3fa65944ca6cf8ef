"""Sanitizer builds of the host code, run on the CPU only:
  - the oracle (oracle.c) built with AddressSanitizer and
    UndefinedBehaviorSanitizer, every pin run against it;
  - libmsda.so with both sanitizers in its host code (the C ABI's argument
    checks, workspace layouts and status reporting; the device code is built
    as usual), the C-ABI and binding tests run against it without a GPU.
Each runs in a child process with the sanitizer runtime preloaded; any
report fails the test (halt on the first error)."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "scale_deformable_attention_forward_amd")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, preload, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV)
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout, cwd=ROOT)


def _no_reports(r):
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run([gcc, "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off", "-fPIC",
                    "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    r = _run([sys.executable, os.path.join(HERE, "mutant_runner.py"), lib], asan)
    _no_reports(r)
    assert r.stdout.strip().splitlines()[-1] == '{"%s": []}' % lib, r.stdout[-2000:]


_DRIVER = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import scale_deformable_attention_forward_amd as m
m.library_path = lambda: {lib!r}
lib = m.load_library()
assert lib._name == {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {test!r}]))
"""


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    runtime = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not runtime:
        pytest.skip("hipcc or clang's AddressSanitizer runtime not found")
    # sanitizers in the host code only: each -fsanitize= right after -Xarch_host
    host_san = ["-Xarch_host -fsanitize=address", "-Xarch_host -fsanitize=undefined",
                "-Xarch_host -fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    flags += [f for pair in host_san for f in pair.split()]
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    procs = [subprocess.Popen([hipcc, *flags, "-c", s, "-o", str(tmp_path / (os.path.basename(s) + ".o"))],
                              stdout=subprocess.PIPE, stderr=subprocess.STDOUT) for s in srcs]
    for p, s in zip(procs, srcs):
        out = p.communicate(timeout=600)[0]
        assert p.returncode == 0, f"{s}: {out[-2000:]}"
    lib = str(tmp_path / "libmsda_sanitized.so")
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *sorted(map(str, tmp_path.glob("*.hip.o"))), "-o",
            lib, "-shared-libsan"] + [f for pair in host_san[:2] for f in pair.split()]
    subprocess.run(link, check=True, capture_output=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the host code is not instrumented"
    driver = tmp_path / "driver.py"
    driver.write_text(_DRIVER.format(root=ROOT, tests=HERE, lib=lib, test=os.path.join(HERE, "test_abi_cpu.py")))
    _no_reports(_run([sys.executable, str(driver)], runtime[-1]))
