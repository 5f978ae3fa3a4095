"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the CPU-side code:
the C oracle (oracle/ssd_ref.c, driven by tests/sanitize/oracle_check.c) and
the host side of libssd's C ABI (problem validation, schedule choice,
workspace plans; driven by tests/sanitize/host_check.cpp, no GPU needed).
Each is built in a directory of its own under _build/ (the host objects are
cached by a digest of their sources) and must exit 0 with no sanitizer
report."""
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ssd_scan_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    return report


def test_oracle_under_asan_ubsan():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_check")
    subprocess.run([gcc, *SAN, "-g", "-O1", "-fopenmp", "-std=c11",
                    os.path.join(ROOT, "oracle", "ssd_ref.c"), os.path.join(HERE, "oracle_check.c"),
                    "-lm", "-o", exe], check=True)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "4"})
    assert "oracle checks passed" in out


def _host_objects(hipcc):
    """Every HIP source compiled with its host code under the sanitizers
    (device code as usual), cached by a digest of the sources and headers."""
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    h = hashlib.sha256()
    for d, names in ((CSRC, sorted(os.listdir(CSRC))), (os.path.join(ROOT, "include"),
                                                        sorted(os.listdir(os.path.join(ROOT, "include"))))):
        for n in names:
            if n.endswith((".hip", ".hpp", ".h")):
                with open(os.path.join(d, n), "rb") as f:
                    h.update(n.encode() + f.read())
    objdir = os.path.join(OUT, "host_" + h.hexdigest()[:16])
    os.makedirs(objdir, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # sanitizers on the host code only
             "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        if not os.path.exists(obj):
            r = subprocess.run([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj + ".tmp"],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            os.replace(obj + ".tmp", obj)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        return list(ex.map(one, srcs)), objdir


def test_host_validation_under_asan_ubsan():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    objs, objdir = _host_objects(hipcc)
    drv = os.path.join(objdir, "host_check.o")
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    subprocess.run([hipcc, "-O1", "-g", "-std=c++17", *san, "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(HERE, "host_check.cpp"), "-o", drv], check=True,
                   capture_output=True)
    exe = os.path.join(objdir, "host_check")
    subprocess.run([hipcc, "--offload-arch=gfx950", *san, "-x", "none", drv, *objs, "-o", exe],
                   check=True, capture_output=True)
    # the HIP runtime keeps its allocations until exit: leak checking off
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "host checks passed" in out
