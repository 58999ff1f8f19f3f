"""Build step of the test oracle: oracle.c -> liboracle.so with the host C compiler."""
from __future__ import annotations

import os
import shutil
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build_oracle(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler (gcc) found to build the oracle")
    src = os.path.join(_HERE, "oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp"
    # -ffp-contract=off: no fused multiply-adds, every step rounds as written
    cmd = [cc, "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def clang() -> str | None:
    """The ROCm LLVM clang (its AddressSanitizer runtime is the one the
    sanitised library build links too), or None."""
    for cand in ("/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            return cand
    return None


def build_oracle_sanitized(out: str, verbose: bool = False) -> str:
    """oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (CPU
    checks of the oracle itself; same arithmetic flags as the normal build)."""
    cc = clang()
    if cc is None:
        raise RuntimeError("clang not found for the sanitised oracle build")
    src = os.path.join(_HERE, "oracle.c")
    cmd = [cc, "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-shared-libsan", "-o", out, src, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))
