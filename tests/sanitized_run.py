"""Run pytest in-process against sanitizer builds of the C-ABI library and the oracle.

Usage (the sanitizer runtime must be preloaded into the Python process, see test_sanitizers.py):
    python tests/sanitized_run.py LIBDIFFATTN LIBORACLE -- <pytest arguments>

The binding is pointed at LIBDIFFATTN and the oracle's unmutated library at LIBORACLE before any test loads
either; everything else runs as in an ordinary test session.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def main(argv):
    sep = argv.index("--")
    lib_path, oracle_path = argv[1], argv[2]
    import differential_attention_fwd_amd as da
    import oracle

    da.LIB_PATH = lib_path
    real = oracle.lib_path
    oracle.lib_path = lambda mutant=0: oracle_path if mutant == 0 else real(mutant)
    # Both libraries load from the sanitizer builds (the oracle is not rebuilt over them: they are newer than its
    # source).
    assert da.lib()._name == lib_path and oracle._load()._name == oracle_path
    import pytest

    return pytest.main(["-p", "no:cacheprovider", *argv[sep + 1:]])


if __name__ == "__main__":
    sys.exit(main(sys.argv))
