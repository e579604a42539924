"""Child process of tests/test_sanitize.py: runs one CPU test module against
a sanitizer build of the oracle or of the C-ABI library.

    python tests/sanitize_child.py oracle   LIB   (tests/test_oracle_pins.py)
    python tests/sanitize_child.py boundary LIB   (tests/test_boundary.py)

The sanitizer runtime is preloaded by the parent (LD_PRELOAD)."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)


def main() -> int:
    what, path = sys.argv[1], sys.argv[2]
    if what == "oracle":
        import oracle
        oracle.build = lambda *a, **k: path
        oracle._default_lib = oracle.load_library(path)
        module = "test_oracle_pins.py"
    elif what == "boundary":
        import paged_kv_cache_100_amd as pkv
        pkv.LIB_PATH = path
        module = "test_boundary.py"
    else:
        raise SystemExit(f"unknown target {what}")
    import pytest
    return pytest.main([os.path.join(HERE, module), "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"])


if __name__ == "__main__":
    sys.exit(main())
