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


def scale_tolerance(r_err: float) -> float:
    """Relative tolerance of the group scales given the factor's relative Frobenius error.

    A group's scale comes from the error-fed weights of its columns; the feedback is the
    earlier columns' errors times rows of R, so the scale carries R's relative error (up to a
    factor near one). 1e-5 where R is within 3.3e-6, three times R's error beyond that (in
    the worst-conditioned layers: the float32 factor of a float32 H_X'' at condition ~1e4)."""
    return max(1e-5, 3.0 * r_err)


def check_codes(codes, zeros, scales, w2, r, bits, group, *, window=1e-5, max_frac=1e-4, scale_rtol=1e-5,
                label="", block=None):
    """Code parity: replay the oracle's sweep on (w2, r), adopting the kernel's
    code or zero only where the rounding argument is within ``window`` of a
    midpoint and the kernel chose the neighbouring value. Every other entry must
    agree exactly (``block``: the oracle's lazy-batched sweep, equal to the
    column-by-column one). Adopted codes may be at most ``max_frac`` of all codes and
    adopted zero points at most ``max_frac`` of all zero points (rounded down:
    no adoption at all below 1 / max_frac entries)."""
    if block:  # lazy-batched replay (equal to the column-by-column one; affordable for long rows)
        res = oracle.obs_quantize_blocked(w2, r, bits, group, block, adopt_codes=codes, adopt_zeros=zeros,
                                          window=window)
    else:
        res = oracle.obs_quantize(w2, r, bits, group, adopt_codes=codes, adopt_zeros=zeros, window=window)
    n, nz = codes.size, zeros.size
    print(f"{label}: {res.adopted_codes} tie-window codes of {n}, {res.adopted_zeros} zero points of {nz}",
          flush=True)
    assert res.mismatches == 0, f"{label}: {res.mismatches} codes/zeros differ outside the tie window"
    np.testing.assert_array_equal(res.codes, codes, err_msg=label)
    np.testing.assert_array_equal(res.zeros, zeros, err_msg=label)
    assert res.adopted_codes <= int(max_frac * n), f"{label}: {res.adopted_codes} tie-window codes of {n}"
    assert res.adopted_zeros <= int(max_frac * nz), f"{label}: {res.adopted_zeros} tie-window zeros of {nz}"
    np.testing.assert_allclose(scales, res.scales.astype(np.float32), rtol=scale_rtol, err_msg=label)
    return res


def gptaq_rows(w, d2, r, rows, block=512):
    """Rows of W + W triu(D R^T, 1) R in float64 without forming D R^T: with c_k = sum_{q<k} w[q] D[q, :],
    (w triu(D R^T, 1))[k] = R[k, :] . c_k. Per block of k: R_b . c at the block start, plus the
    pairs inside the block through G = R_b D_b^T (shared by all rows), then c += w_b D_b."""
    din = d2.shape[0]
    ws = w[rows].astype(np.float64)
    c = np.zeros((len(rows), din))
    z = np.zeros((len(rows), din))
    for k0 in range(0, din, block):
        k1 = min(k0 + block, din)
        rb, db = r[k0:k1].astype(np.float64), d2[k0:k1].astype(np.float64)
        g = np.tril(rb @ db.T, -1)                      # g[k, q] = R[k] . D[q] for q < k in the block
        z[:, k0:k1] = c @ rb.T + ws[:, k0:k1] @ g.T
        c += ws[:, k0:k1] @ db
    out = ws.copy()
    for k0 in range(0, din, block):
        k1 = min(k0 + block, din)
        out += z[:, k0:k1] @ r[k0:k1].astype(np.float64)
    return out
