"""The C ABI without Python: tests/capi/capi_check (built with the library) drives
fp_discover -> fp_threshold_compact -> fp_sparse_attn / fp_dense_attn from C++ on
its own HIP stream and checks list validity, finite outputs, alpha = 0 == dense bit
for bit, and an argument rejection.  Run here as a child process."""
import os
import subprocess

import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capi", "capi_check")


def test_c_abi_consumer():
    assert os.path.exists(BIN), "build the library first (python -m block_sparse_long_pooled_amd.build)"
    print("[case] capi_check", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capi_check passed" in r.stdout
