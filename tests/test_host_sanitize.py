"""The C-ABI layer (validation, partition resolution, workspace sizing, host
partition and cache checks) built for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer and driven by tests/host_abi_check.cpp, whose stubs
stand in for the kernel launchers.  No GPU: api.hip holds no device code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def test_abi_layer_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1", "-std=c++17",
           "-I" + os.path.join(ROOT, "include")]
    objs = []
    for src in (os.path.join(ROOT, "mla_latent_kv_37_amd", "csrc", "api.hip"),
                os.path.join(ROOT, "tests", "host_abi_check.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "-x", "hip", "--offload-host-only"] + san + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        objs.append(obj)
    exe = str(tmp_path / "host_abi_check")
    r = subprocess.run([HIPCC, "--offload-host-only", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", "-o", exe] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host_abi_check: ok" in r.stdout
