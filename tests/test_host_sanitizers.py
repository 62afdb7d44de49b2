"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Every ``csrc/*.hip`` file is compiled again with the sanitizers on its host code only (each ``-fsanitize`` is
passed through ``-Xarch_host``; the device code is built as usual), linked into a separate library, and driven by
``tests/host_sanitizer/driver.cpp``: every size and workspace query on valid and invalid sides and layers (the
host planning code that lays out workspaces) and the host validation of every entry point with arguments it must
reject before any launch. The test passes when the driver's checks hold and neither sanitizer reports anything
(both are set to abort on the first report). The build is cached under the package's ``_build`` folder, keyed by
the sources and flags.
"""
import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "orthogonal_reparameterized_amd")
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "_build", "sanitize")
DRIVER = os.path.join(ROOT, "tests", "host_sanitizer", "driver.cpp")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-result", "-I", INC] + SAN


def _key(srcs):
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for p in srcs + sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(INC, "poet.h"), DRIVER]:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def _build():
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    key = _key(srcs)
    lib, drv, stamp = os.path.join(OUT, "libpoet_sanitize.so"), os.path.join(OUT, "driver"), os.path.join(OUT, "key")
    if os.path.exists(stamp) and open(stamp).read() == key and os.path.exists(lib) and os.path.exists(drv):
        return drv
    os.makedirs(OUT, exist_ok=True)

    def cc(src):
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(cc, srcs))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-I", INC, DRIVER, "-o", drv,
                        "-L", OUT, "-lpoet_sanitize", f"-Wl,-rpath,{OUT}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    open(stamp, "w").write(key)
    return drv


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_host_code_is_clean_under_asan_and_ubsan():
    drv = _build()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "all checks passed" in r.stdout, report[-6000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report, report[-6000:]
