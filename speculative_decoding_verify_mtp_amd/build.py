"""Builds libmtpverify.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m speculative_decoding_verify_mtp_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmtpverify.so")
# measurement helper (a plain streaming read), built beside the library
PROBE_LIB = os.path.join(PKG, "libmtpprobe.so")
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if found is None:
        raise RuntimeError("hipcc not found (set ROCM_PATH)")
    return found


def command(out: str = LIB, source: str = "mtp_verify.hip") -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
        os.path.join(CSRC, source),
        "-o", out,
    ]


def _compile(out: str, source: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = command(tmp, source)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        noise = "is not a recognized feature for this target"
        text = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        if text.strip():
            sys.stderr.write(text + "\n")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compiles the library and the read probe (always, also when they are
    already there) and returns the library's path.  Each new file replaces
    the old one atomically."""
    _compile(LIB, "mtp_verify.hip", verbose)
    _compile(PROBE_LIB, "read_probe.hip", verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
