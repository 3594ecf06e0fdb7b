"""Helpers shared by the GPU parity tests: device transfer and the comparisons
of the parity protocol (relative Frobenius errors; code parity through the
oracle's teacher-forced replay)."""
import os

import numpy as np
import pytest

import oracle

DEV = "cuda:0"


def require_gpu():
    import torch
    import post_quantization_04_amd as kq
    if not os.path.exists(kq.lib_path()):
        raise RuntimeError("libkq.so is not built: the GPU tests run the HIP library only")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    kq.lib()


def bits_to_dev(a: np.ndarray):
    """uint16 bf16 bit patterns -> int16 device tensor (the binding reads it as bf16)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def to_dev(a: np.ndarray, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_fro(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def check_codes(codes, zeros, scales, w2, r, bits, group, *, window=1e-5, max_frac=1e-4, scale_rtol=1e-5,
                label=""):
    """Code parity: replay the oracle's sweep on (w2, r), adopting the kernel's
    code or zero only where the rounding argument is within ``window`` of a
    midpoint and the kernel chose the neighbouring value. Every other entry must
    agree exactly; adopted entries must stay under ``max_frac`` of all codes."""
    res = oracle.obs_quantize(w2, r, bits, group, adopt_codes=codes, adopt_zeros=zeros, window=window)
    n = codes.size
    assert res.mismatches == 0, f"{label}: {res.mismatches} codes/zeros differ outside the tie window"
    np.testing.assert_array_equal(res.codes, codes, err_msg=label)
    np.testing.assert_array_equal(res.zeros, zeros, err_msg=label)
    assert res.adopted_codes <= max(1, max_frac * n), f"{label}: {res.adopted_codes} tie-window codes of {n}"
    np.testing.assert_allclose(scales, res.scales.astype(np.float32), rtol=scale_rtol, err_msg=label)
    return res
