"""The C ABI's host validation layer under AddressSanitizer and UndefinedBehaviorSanitizer,
with warnings as errors (CPU only, no GPU work): csrc/api.hip is compiled with the sanitizers on
its host code (-Xarch_host before each -fsanitize=, the device code as the library builds it),
linked with the library's other objects and tests/host_sanitize/validate_main.c (a C caller of
the ABI, free to pass any int where an enum is declared), and run; the driver's calls only size
workspaces or fail validation before any launch."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mamba_selective_scan_02_amd")
CLANG = "/opt/rocm/llvm/bin/clang++"
CLANG_C = "/opt/rocm/llvm/bin/clang"


def _tool(p):
    return os.path.exists(p) or shutil.which(p)


@pytest.mark.skipif(not (_tool(CLANG) and _tool("/opt/rocm/bin/hipcc")),
                    reason="needs the ROCm toolchain")
def test_validation_layer_under_asan_ubsan(tmp_path):
    from mamba_selective_scan_02_amd import build as b
    objs = [o for o in glob.glob(os.path.join(b.BUILD_DIR, "*.hip.o"))
            if not o.endswith("api.hip.o")]
    if len(objs) + 1 != len(glob.glob(os.path.join(b.CSRC, "*.hip"))):
        b.build()
        objs = [o for o in glob.glob(os.path.join(b.BUILD_DIR, "*.hip.o"))
                if not o.endswith("api.hip.o")]
    api_o = str(tmp_path / "api_san.o")
    flags = [f for f in b.HIP_FLAGS if f not in ("-O3",)]
    cmd = [b.hipcc(), "-O1", "-g", *flags, "-Xarch_host", "-Werror",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-c", os.path.join(b.CSRC, "api.hip"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    drv_o = str(tmp_path / "validate_main.o")
    r = subprocess.run([CLANG_C, "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-Werror",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "host_sanitize", "validate_main.c"),
                        "-o", drv_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    exe = str(tmp_path / "validate")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", drv_o, api_o, *objs,
                        "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host validation checks passed" in r.stdout
