"""The plain-C user of the library (tests/c_abi/lsh_c_abi_check.c, built
beside liblsh.so by the build step) runs on the GPU, using only
include/lsh.h and the HIP runtime: a closed form (K = 0) through the
forward (bf16 and float32, two layouts), partials with the LSE merge and
with folding on arrival, the head permute, the allocation-free
block-sparse call, the backward, and a refused argument block."""
import os
import subprocess

import pytest

from long_sequence_head_amd import build as B

pytestmark = pytest.mark.gpu


def test_c_program_through_the_abi():
    if not os.path.exists(B.C_CHECK_BIN):
        pytest.fail("the C ABI check is not built (python -m long_sequence_head_amd.build)")
    print("[case] plain-C ABI check", flush=True)
    r = subprocess.run([B.C_CHECK_BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout
