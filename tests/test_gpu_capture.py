"""Calibration capture on the GPU feeding the covariance kernel: H_X and H_G of every group and
layer of a small random-weight decoder block against the oracle's covariance of the same
captured bfloat16 rows."""
import numpy as np
import pytest

import oracle
from gpu_helpers import DEV, host, rel_fro

pytestmark = pytest.mark.gpu


def test_capture_covariances():
    import torch
    import post_quantization_04_amd as kq  # noqa: F401  (loads the library)
    from post_quantization_04_amd import capture as cap, pipeline
    shape = cap.BlockShape(d=256, heads=4, d_ff=384)
    c = cap.capture(shape, n_seq=4, seq=128, seed=3, device=DEV, micro_batch=2)
    torch.cuda.synchronize()
    for name, t in list(c.x.items()) + list(c.g.items()):
        print(f"capture covariance {name} {tuple(t.shape)}", flush=True)
        h = pipeline.covariance(t.view(torch.int16))
        torch.cuda.synchronize()
        bits = host(t.view(torch.int16)).view(np.uint16)
        want = oracle.covariance([bits])
        assert rel_fro(host(h), want) <= 1e-4, name
