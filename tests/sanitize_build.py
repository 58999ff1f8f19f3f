"""Builds of the library with its host code under AddressSanitizer and
UndefinedBehaviorSanitizer, for the CPU sanitizer test (no GPU run loads
this file)."""
import glob
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "speculative_decoding_verification_16_amd")


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The library with its host code (argument checks, workspace layout,
    launch planning) instrumented; the device code is the normal gfx950
    build (every sanitizer flag is host-only)."""
    from speculative_decoding_verification_16_amd.build import hipcc

    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    cmd = [hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-shared-libsan", "-I", os.path.join(ROOT, "include"), "-o", out] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc (sanitised host build) failed:\n" + res.stdout + res.stderr)
    return out
