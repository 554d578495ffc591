"""The host code of the C-ABI layer under AddressSanitizer, on the CPU: the
library built with its host code instrumented (-Xarch_host -fsanitize=address)
and driven through every entry point's validation paths by the host program
tests/abi_asan/kda_abi_check.cpp (fake device addresses, no GPU: calls that
pass validation fail at the first HIP call).  A wrong status fails the
program; an invalid host memory access aborts it with a report."""
import os
import subprocess

import pytest

from linear_attention_07_amd import build as kbuild


def test_abi_validation_under_address_sanitizer():
    import torch
    if torch.cuda.is_available():
        pytest.skip("the fake device addresses are for hosts without a GPU")
    inputs = [kbuild.ASAN_CHECK_SRC, os.path.join(kbuild.ROOT, "include", "kda.h")]
    inputs += [os.path.join(kbuild.CSRC, f) for f in os.listdir(kbuild.CSRC)]
    built = [kbuild.ASAN_CHECK, kbuild.ASAN_LIB]
    if not all(os.path.exists(b) for b in built) or \
            min(os.path.getmtime(b) for b in built) < max(os.path.getmtime(f) for f in inputs):
        kbuild.build_asan()
    env = dict(os.environ)
    # the HIP runtime's own allocations at exit are not this library's
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    res = subprocess.run([kbuild.ASAN_CHECK], capture_output=True, text=True, timeout=300,
                         env=env)
    if res.returncode == 77:
        pytest.skip(res.stdout.strip())
    assert res.returncode == 0, res.stdout + res.stderr
    assert "AddressSanitizer" not in res.stderr, res.stderr
    assert "passed under AddressSanitizer" in res.stdout
