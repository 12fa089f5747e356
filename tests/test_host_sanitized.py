"""The host tests of the C-ABI again, against a build whose host code runs
under AddressSanitizer and UndefinedBehaviorSanitizer (lm_head_vocab_amd.
build_sanitized: api.cpp instrumented, the kernels object unchanged), in a
Python process with the ASan runtime preloaded.  No GPU is used: every call
in test_host_abi.py is a host query or fails validation on the host."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_and_ubsan():
    try:
        from lm_head_vocab_amd import build_sanitized as S
    except ImportError:
        pytest.skip("the sanitized build script is not part of this tree")
    lib = S.build()
    env = S.runtime_env()
    # the sanitized library is the one loaded, with the ASan runtime active
    probe = ("import ctypes, lm_head_vocab_amd as L; L.load_library(); "
             f"assert {lib!r} in open('/proc/self/maps').read(); "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); print('loaded')")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "loaded" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
