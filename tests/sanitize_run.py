"""Run CPU tests against sanitised builds of the oracle and the library.

Usage: python tests/sanitize_run.py ORACLE_SO LIBRARY_SO [pytest args...]
(started by test_sanitizers.py with the AddressSanitizer runtime preloaded).
Both libraries are loaded from the given paths before any test imports them,
then pytest runs in this process.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main() -> int:
    oracle_so, lib_so = sys.argv[1], sys.argv[2]
    import oracle
    import speculative_decoding_verification_16_amd as sv

    oracle._LIB_PATH = oracle_so  # noqa: SLF001 -- the loader reads it on first use
    oracle._load()  # noqa: SLF001
    sv.load_library(lib_so)
    return pytest.main(["-p", "no:cacheprovider", *sys.argv[3:]])


if __name__ == "__main__":
    sys.exit(main())
