"""Runs tests/test_abi.py (the host-side checks of every entry point, descriptors, limits,
sharing files) against the host-sanitized build of the library.  Started by
tests/test_host_sanitizers.py in a child process with the AddressSanitizer runtime
preloaded: python tests/host_sanitized_runner.py <sanitized library>.  Not collected by
pytest itself."""
import ctypes
import os
import sys

SANITIZED = sys.argv[1]
_cdll = ctypes.CDLL


def _load(name, *args, **kwargs):
    # the package loads libunipin.so from its own directory; hand it the sanitized build
    if isinstance(name, str) and os.path.basename(name) == "libunipin.so":
        name = SANITIZED
    return _cdll(name, *args, **kwargs)


ctypes.CDLL = _load

import pytest  # noqa: E402

here = os.path.dirname(os.path.abspath(__file__))
rc = pytest.main([os.path.join(here, "test_abi.py"), "-q", "-m", "not gpu", "-p", "no:cacheprovider"])
maps = open("/proc/self/maps").read()
print(f"sanitized library mapped: {SANITIZED in maps}; plain library mapped: "
      f"{os.path.join(os.path.dirname(here), 'falcon_attention_kv_amd', 'libunipin.so') in maps}", flush=True)
sys.exit(rc)
