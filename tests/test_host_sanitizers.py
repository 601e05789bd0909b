"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The fp64 oracle (oracle/gdr2_oracle.c) is rebuilt with gcc
  -fsanitize=address,undefined and its pins (tests/test_oracle_pins.py) run
  against that build in a child process.
- The library's host-side argument validation (gdr2_api.hip and
  gdr2_noalloc.hip, every check that runs before a launch) is rebuilt by
  hipcc with the sanitizers on its host pass only, linked with the other
  objects of the normal build, and tests/test_boundary_host.py runs against
  it in a child process.
A sanitizer report makes the child fail (no recovery), and so this test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_86_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only: the child runs the fake-pointer host tests")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(args, env_extra, preload):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    env["LD_PRELOAD"] = preload
    # -s: a sanitizer report goes to the child's stderr, not to a capture
    # that is lost when the sanitizer ends the process
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall",
                    os.path.join(ROOT, "oracle", "gdr2_oracle.c"), "-o", lib, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    out = _child(["tests/test_oracle_pins.py"], {"GDR2_ORACLE_LIB": lib}, asan)
    assert " passed" in out


def test_host_validation_under_asan_ubsan(tmp_path):
    objs = {os.path.basename(p)[: -len(".hip.o")]: p for p in glob.glob(os.path.join(ROOT, "_build", "*.hip.o"))}
    srcs = {os.path.basename(p)[: -len(".hip")]: p for p in glob.glob(os.path.join(CSRC, "*.hip"))}
    if set(objs) != set(srcs):
        pytest.skip("the normal build's objects are missing: run __graft_entry__.build() first")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    link = []
    for name, src in sorted(srcs.items()):
        if name in ("gdr2_api", "gdr2_noalloc"):      # the host validation path
            obj = str(tmp_path / f"{name}.san.o")
            subprocess.run([HIPCC, *flags, *san, "-c", src, "-o", obj], check=True, capture_output=True)
            link.append(obj)
        else:
            link.append(objs[name])
    lib = str(tmp_path / "libgdr2_hostsan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *link, "-o", lib], check=True,
                   capture_output=True)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    out = _child(["tests/test_boundary_host.py"], {"GDR2_HOST_SANITIZED_LIB": lib}, rt[0])
    assert " passed" in out
