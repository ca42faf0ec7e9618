"""The host-only ABI tests again, with the library's host code (plan
validation, argument checks, workspace layouts: vsa_api.cpp) built with
AddressSanitizer.  Runs on the CPU: every call in test_abi_host.py fails
validation before any HIP call, so no device is touched.  The sanitizer build
(_build/asan/libvsa_amd_asan.so) comes from __graft_entry__.build() or
`python -m block_sparse_video_tile_amd.build --asan`.
"""
import os
import subprocess
import sys

import pytest

from block_sparse_video_tile_amd.build import ASAN_LIB_PATH, asan_runtime

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_tests_under_address_sanitizer():
    if not os.path.exists(ASAN_LIB_PATH):
        pytest.skip("sanitizer build absent: python -m block_sparse_video_tile_amd.build --asan")
    env = dict(os.environ)
    env.update(VSA_LIBRARY=ASAN_LIB_PATH, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=23")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert " passed" in res.stdout
