"""Child-process driver of test_host_sanitized: the host manager's CPU tests
with the AddressSanitizer + UndefinedBehaviorSanitizer build of the manager
(g++ -fsanitize=address,undefined) standing in for both libraries.

Usage (with the sanitizer runtime preloaded):
    python -m tests.sanitized_run <path to the sanitized libpa_host build>
"""

import ctypes as C
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TESTS = ["tests/test_abi_host.py", "tests/test_prefix_groups.py", "tests/test_validate_step.py",
         "tests/test_oracle_swap.py"]
# need the device entry points, which the host-only build does not have
DESELECT = "not product_library_exports and not ordered_entry_points"


def main() -> int:
    import pytest

    from paged_kv_cache_239_amd import _abi
    lib = C.CDLL(sys.argv[1])
    for name, (res, args) in _abi.HOST_SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    # every pool of the tests, manager-only or not, runs on the sanitized build
    _abi._libs[_abi.HOST_LIB_PATH] = lib
    _abi._libs[_abi.LIB_PATH] = lib
    rc = pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", "-k", DESELECT,
                      *[os.path.join(ROOT, t) for t in TESTS]])
    if rc == 0:
        print("sanitized run ok", flush=True)
    return int(rc)


if __name__ == "__main__":
    sys.exit(main())
