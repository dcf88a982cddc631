"""The host code of the library under AddressSanitizer (CPU only).

The library is rebuilt with the host side of every source instrumented
(hipcc -Xarch_host -fsanitize=address; device code is untouched) into a
temporary directory, and the host-only tests -- the ABI checks (exports,
workspace sizes, every validation error path) and the capacity planner --
run against it in a child process with the sanitizer runtime preloaded.
Any heap, stack or global out-of-bounds access or use-after-free in the
host code aborts the child with an AddressSanitizer report."""
import glob
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "vision_transformer_encoder_tiled_amd")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(torch.cuda.is_available(), reason="a host-code check: runs on hosts without a GPU")
@pytest.mark.skipif(asan_runtime() is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc and the clang AddressSanitizer runtime")
def test_host_code_is_clean_under_address_sanitizer(tmp_path):
    spec = importlib.util.spec_from_file_location("_vt_build_asan", os.path.join(PKG, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    pkg = tmp_path / "pkg" / "vision_transformer_encoder_tiled_amd"
    pkg.mkdir(parents=True)
    for f in glob.glob(os.path.join(PKG, "*.py")):
        shutil.copy(f, pkg)
    b.build(out=str(pkg / "libvt.so"), obj_dir=str(tmp_path / "obj"), host_flags=HOST_ASAN)
    child = (
        "import ctypes, sys\n"
        "assert hasattr(ctypes.CDLL(None), '__asan_address_is_poisoned')  # the runtime is loaded\n"
        f"sys.path.insert(0, {str(tmp_path / 'pkg')!r})\n"
        "import vision_transformer_encoder_tiled_amd as vt\n"
        f"assert vt.LIB_PATH.startswith({str(tmp_path)!r}), vt.LIB_PATH\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi.py', 'tests/test_planner.py']))\n")
    env = dict(os.environ, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0")
    r = subprocess.run([sys.executable, "-c", child], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
