"""The C ABI's host-side validation under the address and undefined-behaviour
sanitizers (host code only): tests/c/abi_sweep.cpp sends every entry point a
seeded random mix of extreme sizes, bad pointers and workspaces.  Any
overflow, bad access or undefined status ends the sweep with an error.  The
few calls that pass validation reach a launch on fake pointers, so the test
runs only on a machine without a GPU, where the launch is refused."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_ep_send_amd", "csrc")
SOURCES = ["scan.hip", "fused.hip", "rows.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = [
    pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found"),
    # the sweep's fake pointers are meant for a machine without a GPU
    pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="runs only where there is no GPU"),
]

SAN = ["-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    proc = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert proc.returncode == 0, (cmd[0], proc.returncode, proc.stdout[-2000:], proc.stderr[-4000:])
    return proc


def test_validation_is_clean_under_sanitizers(tmp_path):
    lib = tmp_path / "libepdc_host_san.so"
    exe = tmp_path / "abi_sweep"
    inc = ["-I", os.path.join(ROOT, "include")]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, *inc,
          "-o", str(lib), *[os.path.join(CSRC, s) for s in SOURCES]], timeout=600)
    _run([HIPCC, "--offload-host-only", "-O1", "-std=c++17", *SAN, *inc, "-o", str(exe),
          os.path.join(ROOT, "tests", "c", "abi_sweep.cpp"), "-L", str(tmp_path),
          "-lepdc_host_san", f"-Wl,-rpath,{tmp_path}"], timeout=300)
    # hide every GPU from the sweep as well (it refuses to run if it sees one)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    for seed in ("1", "2"):
        out = _run([str(exe), seed, "1000000"], timeout=300, env=env).stdout
        assert out.startswith("done:"), out
