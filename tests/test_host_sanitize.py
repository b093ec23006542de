"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libtq is compiled with both sanitizers on its host side (the gfx950 device
code is built as usual and never launched), linked with tests/host_sanitize_driver.cpp, and
run: the float64 codebooks, the
parameter-block construction of tq_prepare and the argument validation of every entry point
execute under the sanitizers, and any out-of-bounds access, use after free or undefined
behaviour aborts the run.  No kernel is launched.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_embedding_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.timeout(600)
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    # host code at -O1 with the sanitizers; device code (never launched here) unoptimized,
    # except where its register-class constraints need the optimizer (quantize.hip)
    common = ["--offload-arch=gfx950", "-Xarch_host", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
              f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-Wno-unused-command-line-argument", *SAN]
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    procs, objs = [], []
    for f in srcs:
        obj = str(tmp_path / (f + ".o"))
        objs.append(obj)
        dev_opt = ["-Xarch_device", "-O1" if f == "quantize.hip" else "-O0"]
        procs.append(subprocess.Popen([HIPCC, *common, *dev_opt, "-x", "hip", "-c", os.path.join(CSRC, f), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    drv = str(tmp_path / "driver.o")
    procs.append(subprocess.Popen([HIPCC, *common, "-Xarch_device", "-O0", "-x", "hip", "-c",
                                   os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    exe = str(tmp_path / "tq_host_sanitize")
    link = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, drv, "-o", exe],
                          capture_output=True, text=True)
    assert link.returncode == 0, link.stdout + link.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout[-3000:] + run.stderr[-6000:]
