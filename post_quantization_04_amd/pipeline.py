"""The per-layer path as a sequence of libkq calls.

Torch supplies device memory and the stream; every step runs in the
library's kernels. H_G is released as soon as BiIP has used it: the column
sweep never reads it, so the extra dout x dout memory lives only through the
preprocessing.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import (KQ_BIIP_INPUT, KQ_BIIP_INVERSE, KQ_BIIP_OUTPUT, KQ_BIIP_SCALE, KQ_SCORE_KRONQ, KQError,
               KQ_EINVAL, KQ_ENOTPD, Rot, accumulate_cov, accumulate_xcov, biip_rotate, biip_transform,
               cholesky_inv, gptaq_target, make_rot, obs_quantize, sensitivity)

ALL_SIDES = KQ_BIIP_INPUT | KQ_BIIP_OUTPUT | KQ_BIIP_SCALE


@dataclass
class DeviceRot:
    """A rotation spec resident on the device (the tensors back the C struct)."""
    signs: object
    q: object
    rot: Rot


def upload_rot(signs: np.ndarray, q: np.ndarray, device) -> DeviceRot:
    import torch
    s = torch.from_numpy(np.ascontiguousarray(signs, dtype=np.int8)).to(device)
    qq = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).to(device)
    return DeviceRot(s, qq, make_rot(s, qq))


def covariance(a, *, out=None, chunk_rows: Optional[int] = None, stream=None):
    """H = A^T A / N for bf16 A [N, d] on the device (one call, or chunked with beta = 1)."""
    import torch
    n, d = a.shape
    h = torch.empty((d, d), dtype=torch.float32, device=a.device) if out is None else out
    if chunk_rows is None or chunk_rows >= n:
        accumulate_cov(a, h, 1.0 / n, 0.0, stream=stream)
        return h
    for i, r0 in enumerate(range(0, n, chunk_rows)):
        accumulate_cov(a[r0:r0 + chunk_rows], h, 1.0 / n, 0.0 if i == 0 else 1.0, stream=stream)
    return h


def drift_moment(xt, x, h_x, *, out=None, stream=None):
    """D = (Xt - X)^T X / N from the full-precision inputs Xt and the quantized-model inputs X
    (bf16 [N, d], the same tokens) and H_X = X^T X / N: one cross-moment call with beta = -1."""
    import torch
    n, d = x.shape
    dm = torch.empty((d, d), dtype=torch.float32, device=x.device) if out is None else out
    accumulate_xcov(xt, x, dm, 1.0 / n, -1.0, c_in=h_x, stream=stream)
    return dm


@dataclass
class LayerOut:
    w2: object          # rotated weight W'' (float64), overwritten by the dequantised W^''
    hx2: object         # H_X'' (float32), overwritten by R
    s_x: object
    s_g: object
    codes: object
    scales: object
    zeros: object
    info: object
    w_hat: Optional[object] = None


def quantize_layer(w, h_x, h_g, rot_in: DeviceRot, rot_out: DeviceRot, *, bits: int, group: int, block: int,
                   damp: float, flags: int = ALL_SIDES, keep_inputs: bool = True, unrotate: bool = True,
                   check_info: bool = True, preround=None, d_x=None, stream=None) -> LayerOut:
    """BiIP -> damped Cholesky factor of the inverse -> OBS sweep (-> un-rotation).

    ``h_x`` / ``h_g`` are the raw covariances; with ``keep_inputs`` they are
    copied first (the library transforms them in place). ``d_x`` (the drift moment of
    ``drift_moment``) selects the GPTAQ base quantizer: D'' by the input-side map, then the
    drift correction of W'' before the sweep."""
    import torch
    dev = w.device
    dout, din = w.shape
    hx = h_x.clone() if keep_inputs else h_x
    hg = None
    if flags & KQ_BIIP_OUTPUT:
        hg = h_g.clone() if keep_inputs else h_g
    w2 = torch.empty((dout, din), dtype=torch.float64, device=dev)
    s_x = torch.empty(din, dtype=torch.float64, device=dev)
    s_g = torch.empty(dout, dtype=torch.float64, device=dev)
    biip_rotate(w, w2, hx, hg, rot_in.rot if flags & KQ_BIIP_INPUT else None,
                rot_out.rot if flags & KQ_BIIP_OUTPUT else None, flags, s_x, s_g, stream=stream)
    del hg  # H_G'' is not needed by anything after BiIP
    d2 = None
    if d_x is not None:
        d2 = d_x.clone() if keep_inputs else d_x
        if flags & KQ_BIIP_INPUT:
            biip_transform(d2, rot_in.rot, s_x, stream=stream)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    cholesky_inv(hx, damp, info, stream=stream)
    if check_info:
        bad = int(info.item())
        if bad:
            raise KQError(KQ_ENOTPD, f"damped H_X'' is not positive definite at index {bad - 1}")
    if d2 is not None:
        info_t = torch.zeros(1, dtype=torch.int32, device=dev)
        gptaq_target(w2, d2, hx, info=info_t, stream=stream)
        del d2
        if check_info and int(info_t.item()):
            raise KQError(KQ_EINVAL, "the drift correction produced non-finite weights "
                                     "(the drift moment holds a NaN or Inf)")
    ng = din // group if group else 1
    codes = torch.empty((dout, din), dtype=torch.uint8, device=dev)
    scales = torch.empty((dout, ng), dtype=torch.float32, device=dev)
    zeros = torch.empty((dout, ng), dtype=torch.uint8, device=dev)
    obs_quantize(w2, hx, bits, group, block, codes, scales, zeros, preround, stream=stream)
    out = LayerOut(w2, hx, s_x, s_g, codes, scales, zeros, info)
    if unrotate:
        w_hat = torch.empty((dout, din), dtype=torch.float64, device=dev)
        biip_rotate(w2, w_hat, None, None, rot_in.rot if flags & KQ_BIIP_INPUT else None,
                    rot_out.rot if flags & KQ_BIIP_OUTPUT else None, flags | KQ_BIIP_INVERSE, s_x, s_g,
                    stream=stream)
        out.w_hat = w_hat
    return out


def score(h_x, h_g, mode: int = KQ_SCORE_KRONQ, stream=None) -> float:
    import torch
    s = torch.empty(1, dtype=torch.float64, device=h_x.device)
    sensitivity(h_x, h_g, s, mode, stream=stream)
    return float(s.item())
