"""Run pytest on test files with the attention library and/or the oracle
replaced by sanitizer builds (used by test_sanitizers_cpu.py, in a child
process that has the matching ASan runtime preloaded).

usage: python sanitize_driver.py FA_LIB|- ORACLE_LIB|- pytest-args...
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    fa_lib, oracle_lib, args = sys.argv[1], sys.argv[2], sys.argv[3:]
    if fa_lib != "-":
        from exact_attention_91_amd import fa
        fa._LIB_PATH = fa_lib
    if oracle_lib != "-":
        from oracle import build_oracle
        build_oracle.LIB = oracle_lib
    import pytest
    return pytest.main(args)


if __name__ == "__main__":
    sys.exit(main())
