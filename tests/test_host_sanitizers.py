"""The C-ABI entry points' argument validation (api.hip, block.hip host code) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through every entry point by
tests/sanitize/driver.cpp: valid calls (reaching stubbed launchers), each error status, and
extreme sizes whose byte arithmetic would overflow int64 if it were not guarded.  Host code
only: the device parts are compiled without sanitizers and nothing runs on a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_transformer_mmdit_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def test_validators_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    flags = ["-O1", "-g", "-std=c++17", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-I" + os.path.join(ROOT, "include")]
    objs = []

    def cc(args, out):
        r = subprocess.run([hipcc, *flags, *args, "-o", out], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(out)

    for f in ("api", "block"):
        cc(["--offload-arch=gfx950", "-c", os.path.join(CSRC, f + ".hip")], str(tmp_path / (f + ".o")))
    cc(["--cuda-host-only", "-c", os.path.join(SAN, "stubs.hip")], str(tmp_path / "stubs.o"))
    cc(["-x", "c++", "-c", os.path.join(SAN, "driver.cpp")], str(tmp_path / "driver.o"))
    exe = str(tmp_path / "driver")
    r = subprocess.run([hipcc, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "--offload-arch=gfx950", *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "ALL OK" in r.stdout, out[-4000:]
