"""Compile the C-ABI check programs (tests/c/epdc_c_check, tests/c/epdc_c_paths)
against the in-tree libepdc.so with hipcc, host code only.  Called by
__graft_entry__.build()."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "combine_ep_send_amd")
PROGRAMS = ("epdc_c_check", "epdc_c_paths")
BIN = os.path.join(HERE, PROGRAMS[0])


def build(verbose: bool = False) -> str:
    sys.path.insert(0, ROOT)
    from combine_ep_send_amd.build import hipcc

    for name in PROGRAMS:
        out = os.path.join(HERE, name)
        tmp = out + ".tmp"
        cmd = [hipcc(), "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"),
               "-o", tmp, os.path.join(HERE, name + ".cpp"), "-L", PKG, "-lepdc",
               "-Wl,-rpath,$ORIGIN/../../combine_ep_send_amd"]
        if verbose:
            print(" ".join(cmd), flush=True)
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            sys.stderr.write(proc.stdout + proc.stderr)
            raise RuntimeError(f"hipcc failed with status {proc.returncode}")
        os.replace(tmp, out)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
