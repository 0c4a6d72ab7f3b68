"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the C ABI's validation, workspace layout, tree-spec checks and
the calibrated sparse-tree builder, driven by tests/host_sanitize.cpp with
random and malformed inputs. The sanitizers instrument the host code only;
the device code is built as usual and never launched."""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "medusa_tree_verification_forward_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def test_host_paths_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC) or shutil.which("nproc") is None:
        pytest.skip("hipcc not available")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [
        os.path.join(ROOT, "tests", "host_sanitize.cpp")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_sanitize")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "host paths ok" in r.stdout, report
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
