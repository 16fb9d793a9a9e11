"""The C-ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the library's sources are compiled with the
sanitizers on the host code only (device code unchanged) and linked into
tests/sanitize/abi_driver.cpp, which calls every entry point with arguments
that validation must reject, sizes past the kernels' launch limits and the
size queries at extreme values. Nothing reaches a kernel launch, so this
runs on hosts without a GPU. Any sanitizer finding aborts the driver."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_query_attention_sqa_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

def _library_sources():
    """The library's source list, read from its build script (loaded from
    its file, so that importing the package is not needed)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_sqa_build", os.path.join(ROOT, "sparse_query_attention_sqa_amd",
                                                                          "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return list(mod.SOURCES)


SOURCES = _library_sources()
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
# sanitizers for the host code of each HIP source (each flag after -Xarch_host)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
DRIVER_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _no_gpu_present():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
@pytest.mark.skipif(not _no_gpu_present(), reason="host-only check; runs on GPU-less hosts")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950"] + HOST_SAN + [
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC, "-x", "hip", os.path.join(CSRC, src), "-c", "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv_obj = str(tmp_path / "abi_driver.o")
    r = subprocess.run([CLANG, "-O1", "-g"] + DRIVER_SAN + ["-I", INCLUDE, "-c",
                        os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([CLANG] + DRIVER_SAN + [drv_obj] + objs + ["-L/opt/rocm/lib", "-lamdhip64",
                       "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    print(out[-4000:])
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out
    assert "OK: 0 failure(s)" in r.stdout
