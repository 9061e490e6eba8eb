"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU).  api.hip -- every host-side
argument check, size query and dispatch plan -- is compiled with the
sanitizers on its host pass only (device code unchanged), linked with the
other objects into tests/sanitize/abi_driver.cpp, which drives every entry
point's refusals, size queries and kernel-plan queries with edge values.
Any sanitizer report or failed expectation fails the test."""
import concurrent.futures as cf
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["address", "undefined"]


def _build_lib_module():
    path = os.path.join(ROOT, "bit_gemm_int8_amd", "build_lib.py")
    spec = importlib.util.spec_from_file_location("bl_build_lib_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    bl = _build_lib_module()
    if not (os.path.exists(bl.HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not available")
    out = tmp_path_factory.mktemp("san")
    # the host pass of api.hip with the sanitizers (each flag behind
    # -Xarch_host: the device pass is built as in the library)
    host_san = []
    for flag in [f"-fsanitize={s}" for s in SAN] + ["-fno-sanitize-recover=all",
                                                     "-fno-omit-frame-pointer"]:
        host_san += ["-Xarch_host", flag]

    def compile_one(src):
        obj = str(out / (os.path.splitext(src)[0] + ".o"))
        flags = [f for f in bl.CFLAGS if f != "-O3"] + ["-O1", "-g"] if src == "api.hip" else bl.CFLAGS
        cmd = [bl.HIPCC, *flags, *(host_san if src == "api.hip" else []), "-c",
               os.path.join(bl.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-4000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(bl.SOURCES))) as ex:
        objs = list(ex.map(compile_one, bl.SOURCES))
    drv_obj = str(out / "abi_driver.o")
    san = "-fsanitize=" + ",".join(SAN)
    r = subprocess.run([CLANGXX, "-std=c++17", "-O1", "-g", san, "-fno-sanitize-recover=all",
                        "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                        "-o", drv_obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(out / "abi_driver")
    r = subprocess.run([CLANGXX, san, drv_obj, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    yield exe
    shutil.rmtree(out, ignore_errors=True)


def test_host_code_under_asan_ubsan(driver):
    env = dict(os.environ)
    # the HIP runtime's own allocations at exit are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=98"
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "all host-side checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
