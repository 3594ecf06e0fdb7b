"""KronQ per-layer quantization written out plainly in float64: the oracle.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module. The test suite, the smoke check of the build entry
point and the CPU-baseline leg of the benchmark are its only users. It shares
no code with the GPU library; its inputs come from ``kq_synth`` alone.

Every step is the plain definition or the plain algorithm, in float64, with
library primitives (matmul, inverse, Cholesky, the Sylvester Hadamard matrix)
as steps and no blocking or fusion beyond what the algorithm states.

Sources (cited by page title and section):
  [KQ-en]   "KronQ: LLM Quantization via Kronecker-Factored Hessian",
            gptget.net English summary: Methodology, Technical Contribution, Abstract.
  [KQ-zh]   gptget.net Chinese summary of the same paper: 方法论 (methodology).
  [KQ-news] "KronQ: Kronecker Hessians break GPTQ's 2-bit wall", aimodeling.com news item.
  [KQ-art]  wmrh.cn popular article on KronQ: sections 二 (the Kronecker split),
            三 (BiIP and the trace score), 四 (H_G cancels from the column update),
            六 (mixed precision), 七 (cost), 八 (ablations, diagonal scaling, the
            GPTAQ base quantizer), Q&A.

Readings where the pages are silent (each also listed in the design notes):
  * s_j = H_jj^(1/4) per side, 1 where H_jj <= 0 (the pages name only "the
    diagonal elements" of H_X and H_G as the basis of the scaling). Parity of
    this exponent against the pages: unpinned.
  * U = (Q_m kron H_p / sqrt(p)) diag(sigma) for d = m * 2^k, m odd.
  * damping: lambda * mean(diag) added to the post-BiIP H_X, no dead-column rule.
  * natural column order; asymmetric min-max grid with the scale stored as
    float32 and the zero point rounded half-to-even and clamped to [0, 2^b-1].
  * group parameters come from the fully error-fed weights when the sweep
    reaches the group's first column; per-row grids come from W'' before the sweep.
  * bit allocation: greedy by score (descending, ties by index) under an
    integer, parameter-weighted budget. Parity against the pages: unpinned.
  * GPTAQ (row f2): every column's input drift (w_q dx_q) compensated by least squares on
    the later columns' inputs, then GPTQ's sweep. Parity against the pages: unpinned (no
    formula there).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Sequence

import numpy as np
import scipy.linalg

import kq_synth

__all__ = [
    "as_f64", "covariance", "syrk_update", "sensitivity", "hadamard", "rotation_matrix",
    "rotation_rows", "rotate_rows", "unrotate_rows", "biip_scales", "biip_forward",
    "biip_inverse", "damped", "chol_inv_upper", "grid", "obs_quantize", "obs_quantize_blocked",
    "obq_reference", "rtn_quantize", "kron_loss", "allocate_bits", "quantize_layer",
    "container_bits", "pack_codes", "unpack_codes", "dequantize", "decode_matvec",
    "ObsResult", "INFEASIBLE", "cross_covariance", "gptaq_target", "gptaq_quantize", "biip_transform",
    "quantize_layer_gptaq", "gptaq_drift_map",
]


def as_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or real arrays -> float64, exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return kq_synth.bf16_bits_to_f64(a)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# step 1: covariances  ([KQ-art] 二; [KQ-news]; [KQ-en] Methodology)
# ---------------------------------------------------------------------------
def covariance(chunks: Iterable[np.ndarray]) -> np.ndarray:
    """H = A^T A / N over all token rows of A.

    With A = X this is the activation covariance H_X that GPTQ already uses as
    the Hessian proxy; with A = G (output gradients from one backward pass) it
    is the gradient covariance H_G. The Kronecker-factored Hessian is
    H_X kron H_G ([KQ-art] 二, [KQ-news]).
    """
    h = None
    n = 0
    for c in chunks:
        a = as_f64(c)
        p = a.T @ a
        h = p if h is None else h + p
        n += a.shape[0]
    if n == 0:
        raise ValueError("covariance of zero tokens is undefined")
    return h / n


def syrk_update(h: Optional[np.ndarray], a: np.ndarray, alpha: float, beta: float) -> np.ndarray:
    """alpha * A^T A + beta * H (the chunked form of ``covariance``)."""
    a = as_f64(a)
    out = alpha * (a.T @ a)
    if beta != 0.0:
        out = out + beta * np.asarray(h, np.float64)
    return out


# ---------------------------------------------------------------------------
# step 5a: sensitivity score  ([KQ-news]; [KQ-art] 三, 六)
# ---------------------------------------------------------------------------
def sensitivity(h_x: np.ndarray, h_g: np.ndarray, mode: str = "kronq") -> float:
    """tr(H_G) * tr(H_X) on the raw covariances; ``hx_only`` gives tr(H_X) alone.

    The trace product is the sub-layer score of [KQ-news] and [KQ-art] 三. The
    H_X-only score is the prior practice that cannot separate q/k/v, which
    share H_X ([KQ-art] 三, 六).
    """
    tx = float(np.trace(np.asarray(h_x, np.float64)))
    if mode == "hx_only":
        return tx
    if mode != "kronq":
        raise ValueError(mode)
    return float(np.trace(np.asarray(h_g, np.float64))) * tx


# ---------------------------------------------------------------------------
# step 2: bidirectional incoherence processing  ([KQ-art] 三, 七, 八, Q&A)
# ---------------------------------------------------------------------------
def hadamard(p: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix of order p (a power of two), entries +-1."""
    return scipy.linalg.hadamard(p).astype(np.float64)


def rotation_matrix(spec: kq_synth.RotSpec) -> np.ndarray:
    """Dense U = (Q_m kron H_p / sqrt(p)) diag(sigma). For small n only."""
    hp = hadamard(spec.p) / np.sqrt(spec.p)
    return np.kron(np.asarray(spec.q, np.float64), hp) * spec.signs.astype(np.float64)[None, :]


def rotation_rows(spec: kq_synth.RotSpec, rows: Sequence[int]) -> np.ndarray:
    """Selected rows of U, built entry by entry from the definition (any n)."""
    rows = np.asarray(rows, np.int64)
    a, b = rows // spec.p, rows % spec.p
    cols = np.arange(spec.n, dtype=np.int64)
    a2, b2 = cols // spec.p, cols % spec.p
    bits = np.bitwise_and(b[:, None], b2[None, :])
    par = np.zeros(bits.shape, np.int64)
    x = bits.copy()
    while np.any(x):
        par ^= (x & 1)
        x >>= 1
    h = np.where(par == 1, -1.0, 1.0) / np.sqrt(spec.p)
    return np.asarray(spec.q, np.float64)[a[:, None], a2[None, :]] * h * spec.signs.astype(np.float64)[None, :]


def rotate_rows(v: np.ndarray, spec: kq_synth.RotSpec) -> np.ndarray:
    """Apply x -> U x to every row of v (returns v U^T), via the Kronecker reshape."""
    v = np.ascontiguousarray(v, np.float64)  # a transposed view makes numpy's batched products crawl
    k, n = v.shape
    if n != spec.n:
        raise ValueError("rotation size mismatch")
    hp = hadamard(spec.p) / np.sqrt(spec.p)
    r = (v * spec.signs.astype(np.float64)[None, :]).reshape(k, spec.m, spec.p)
    r = r @ hp
    r = np.einsum("ab,kbp->kap", np.asarray(spec.q, np.float64), r)
    return r.reshape(k, n)


def unrotate_rows(v: np.ndarray, spec: kq_synth.RotSpec) -> np.ndarray:
    """Apply x -> U^T x to every row of v (returns v U)."""
    v = np.ascontiguousarray(v, np.float64)
    k, n = v.shape
    if n != spec.n:
        raise ValueError("rotation size mismatch")
    hp = hadamard(spec.p) / np.sqrt(spec.p)
    r = v.reshape(k, spec.m, spec.p)
    r = np.einsum("ba,kbp->kap", np.asarray(spec.q, np.float64), r)
    r = r @ hp
    return r.reshape(k, n) * spec.signs.astype(np.float64)[None, :]


def biip_scales(h: np.ndarray) -> np.ndarray:
    """Diagonal scaling of one side: s_j = H_jj^(1/4), 1 where H_jj <= 0.

    [KQ-art] 八: the weights are rescaled from the diagonals of H_X and H_G
    (S_X and S_G) before the rotation. The exponent 1/4 is a reading.
    """
    d = np.diag(np.asarray(h, np.float64)).copy()
    s = np.ones_like(d)
    pos = d > 0
    s[pos] = d[pos] ** 0.25
    return s


def _two_sided(h: np.ndarray, spec: kq_synth.RotSpec) -> np.ndarray:
    """U H U^T."""
    return rotate_rows(rotate_rows(h, spec).T, spec).T


def biip_forward(w: np.ndarray, h_x: np.ndarray, h_g: np.ndarray, rot_in: kq_synth.RotSpec,
                 rot_out: kq_synth.RotSpec, *, inp: bool = True, out: bool = True, scale: bool = True):
    """W'' = U_G S_G W S_X U_X^T, H_X'' = U_X S_X^-1 H_X S_X^-1 U_X^T, H_G'' likewise.

    The input side is processed with H_X and the output side with H_G
    ([KQ-art] 三); scaling precedes the rotation ([KQ-art] 八); the rotation is a
    randomised Hadamard transform ([KQ-art] 七, Q&A; [KQ-zh] 方法论).
    Returns (W'', H_X'', H_G'', s_x, s_g). Disabled sides use s = 1 and U = I.
    """
    w = as_f64(w)
    dout, din = w.shape
    s_x = biip_scales(h_x) if (inp and scale) else np.ones(din)
    s_g = biip_scales(h_g) if (out and scale) else np.ones(dout)
    w1 = s_g[:, None] * w * s_x[None, :]
    hx1 = np.asarray(h_x, np.float64) / s_x[:, None] / s_x[None, :]
    hg1 = None if h_g is None else np.asarray(h_g, np.float64) / s_g[:, None] / s_g[None, :]
    if inp:
        w1 = rotate_rows(w1, rot_in)
        hx1 = _two_sided(hx1, rot_in)
    if out:
        w1 = rotate_rows(w1.T, rot_out).T
        hg1 = _two_sided(hg1, rot_out)
    return w1, hx1, hg1, s_x, s_g


def biip_transform(m: np.ndarray, s: np.ndarray, spec: kq_synth.RotSpec) -> np.ndarray:
    """U S^-1 M S^-1 U^T for any square M (the input-side map of H_X, applied with given scales):
    a second-moment matrix of the layer's inputs in the basis the sweep works in."""
    s = np.asarray(s, np.float64)
    return _two_sided(np.asarray(m, np.float64) / s[:, None] / s[None, :], spec)


def biip_inverse(w2: np.ndarray, rot_in: kq_synth.RotSpec, rot_out: kq_synth.RotSpec,
                 s_x: np.ndarray, s_g: np.ndarray, *, inp: bool = True, out: bool = True) -> np.ndarray:
    """W = S_G^-1 U_G^T W'' U_X S_X^-1 (undo ``biip_forward`` on the weights)."""
    w = np.asarray(w2, np.float64)
    if out:
        w = unrotate_rows(w.T, rot_out).T
    if inp:
        w = unrotate_rows(w, rot_in)
    return w / np.asarray(s_g, np.float64)[:, None] / np.asarray(s_x, np.float64)[None, :]


# ---------------------------------------------------------------------------
# step 3: damping and the Cholesky factor of the inverse
# ---------------------------------------------------------------------------
def damped(h: np.ndarray, lam: float) -> np.ndarray:
    """H + lam * mean(diag H) * I."""
    h = np.array(h, np.float64, copy=True)
    h[np.diag_indices_from(h)] += lam * float(np.mean(np.diag(h)))
    return h


def chol_inv_upper(h: np.ndarray, lam: float) -> np.ndarray:
    """Upper-triangular R with R^T R = (H + lam*mean(diag H)*I)^-1, by the plain route:
    explicit inverse, then the lower Cholesky factor L of it, R = L^T."""
    hinv = np.linalg.inv(damped(h, lam))
    hinv = 0.5 * (hinv + hinv.T)
    return np.linalg.cholesky(hinv).T


# ---------------------------------------------------------------------------
# step 4: GPTQ-style column-wise OBS  ([KQ-en] Methodology; [KQ-zh] 方法论; [KQ-art] 四)
# ---------------------------------------------------------------------------
def grid(wmin: np.ndarray, wmax: np.ndarray, bits: int):
    """Asymmetric b-bit min-max grid per row: returns (scale, zero), float64 arrays.

    The range always contains 0; an all-zero range becomes [-1, 1]. The scale
    is stored as float32, so the grid in use is that float32 value. The zero
    point is the half-to-even rounding of -xmin/s, clamped to [0, 2^b - 1].
    """
    maxq = (1 << bits) - 1
    xmin = np.minimum(np.asarray(wmin, np.float64), 0.0)
    xmax = np.maximum(np.asarray(wmax, np.float64), 0.0)
    flat = (xmin == 0.0) & (xmax == 0.0)
    xmin = np.where(flat, -1.0, xmin)
    xmax = np.where(flat, 1.0, xmax)
    s = ((xmax - xmin) / maxq).astype(np.float32).astype(np.float64)
    z = np.clip(np.rint(-xmin / s), 0, maxq)
    return s, z


def _tie(u: np.ndarray, window: float) -> np.ndarray:
    """True where u lies within ``window`` of a rounding midpoint (k + 1/2)."""
    return np.abs(u - np.floor(u) - 0.5) <= window


@dataclass
class ObsResult:
    codes: np.ndarray        # uint8 [dout, din]
    scales: np.ndarray       # float64 [dout, ngroups] (values representable in float32)
    zeros: np.ndarray        # uint8 [dout, ngroups]
    what: np.ndarray         # dequantised W'' (float64)
    t: np.ndarray            # argument of the rounding, w / s, per entry
    adopted_codes: int = 0   # tie-window entries where the other side's code was taken
    adopted_zeros: int = 0
    mismatches: int = 0      # entries where the other side differs outside the rules


class _Adopt:
    """Teacher-forced replay: inside a tie window take the other side's choice."""

    def __init__(self, codes, zeros, window):
        self.codes = np.asarray(codes)
        self.zeros = np.asarray(zeros)
        self.window = window
        self.codes_n = 0
        self.zeros_n = 0
        self.bad = 0

    def pick(self, own, other, u, offset, maxq):
        other = other.astype(np.float64)
        differ = other != own
        if not np.any(differ):
            return own, 0
        lo = np.clip(np.floor(u) + offset, 0, maxq)
        hi = np.clip(np.floor(u) + 1 + offset, 0, maxq)
        ok = differ & _tie(u, self.window) & ((other == lo) | (other == hi))
        self.bad += int(np.sum(differ & ~ok))
        return np.where(ok, other, own), int(np.sum(ok))


def _params(wg, bits, adopt, gi):
    s, z = grid(wg.min(axis=1), wg.max(axis=1), bits)
    if adopt is not None:
        xmin = np.minimum(wg.min(axis=1), 0.0)
        xmax = np.maximum(wg.max(axis=1), 0.0)
        flat = (xmin == 0.0) & (xmax == 0.0)
        u = np.where(flat, 1.0, -xmin) / s
        z, n = adopt.pick(z, adopt.zeros[:, gi], u, 0, (1 << bits) - 1)
        adopt.zeros_n += n
    return s, z


def obs_quantize(w2: np.ndarray, r: np.ndarray, bits: int, group: int, *, adopt_codes=None,
                 adopt_zeros=None, window: float = 1e-5) -> ObsResult:
    """Column-by-column OBS with the upper Cholesky factor R of the damped H_X''^-1.

    For each column j in natural order: quantise w_j to the row's (or group's)
    grid, take the scaled error e = (w_j - w^_j) / R_jj and remove e * R[j, k]
    from every later column k. H_G does not appear: under the Kronecker
    Hessian the optimal compensation of the remaining columns is independent
    of H_G ([KQ-art] 四), so the update is the GPTQ one.

    ``adopt_codes`` / ``adopt_zeros`` (optional) run the teacher-forced replay
    used for parity: where the rounding argument lies within ``window`` of a
    midpoint and the other side chose the neighbouring value, that value is
    taken so that one legal tie-break does not cascade.
    """
    w = as_f64(w2).copy()
    r = np.asarray(r, np.float64)
    dout, din = w.shape
    maxq = (1 << bits) - 1
    ng = din // group if group else 1
    codes = np.zeros((dout, din), np.uint8)
    scales = np.zeros((dout, ng))
    zeros = np.zeros((dout, ng), np.uint8)
    what = np.zeros((dout, din))
    tt = np.zeros((dout, din))
    adopt = None if adopt_codes is None else _Adopt(adopt_codes, adopt_zeros, window)
    if not group:
        s, z = _params(w, bits, adopt, 0)
        scales[:, 0], zeros[:, 0] = s, z
    for j in range(din):
        if group and j % group == 0:
            s, z = _params(w[:, j:j + group], bits, adopt, j // group)
            scales[:, j // group], zeros[:, j // group] = s, z
        t = w[:, j] / s
        q = np.clip(np.rint(t) + z, 0, maxq)
        if adopt is not None:
            q, n = adopt.pick(q, adopt.codes[:, j], t, z, maxq)
            adopt.codes_n += n
        wq = s * (q - z)
        codes[:, j], what[:, j], tt[:, j] = q, wq, t
        e = (w[:, j] - wq) / r[j, j]
        w[:, j + 1:] -= np.outer(e, r[j, j + 1:])
    out = ObsResult(codes, scales, zeros, what, tt)
    if adopt is not None:
        out.adopted_codes, out.adopted_zeros, out.mismatches = adopt.codes_n, adopt.zeros_n, adopt.bad
    return out


def obs_quantize_blocked(w2: np.ndarray, r: np.ndarray, bits: int, group: int, block: int, *, adopt_codes=None,
                         adopt_zeros=None, window: float = 1e-5) -> ObsResult:
    """The same sweep with lazy batching: in-block feedback column by column, then
    one trailing product W[:, end:] -= E R[blk, end:] per block of ``block`` columns.

    Equal to ``obs_quantize`` in exact arithmetic when every group lies inside one
    block (block % group == 0) or group == 0. ``adopt_codes`` / ``adopt_zeros`` run
    the same teacher-forced replay as in ``obs_quantize``; the blocked form keeps
    the replay affordable for rows thousands of columns long.
    """
    w = as_f64(w2).copy()
    r = np.asarray(r, np.float64)
    dout, din = w.shape
    if din % block or (group and block % group):
        raise ValueError("block must divide din and be a multiple of group")
    maxq = (1 << bits) - 1
    ng = din // group if group else 1
    codes = np.zeros((dout, din), np.uint8)
    scales = np.zeros((dout, ng))
    zeros = np.zeros((dout, ng), np.uint8)
    what = np.zeros((dout, din))
    tt = np.zeros((dout, din))
    adopt = None if adopt_codes is None else _Adopt(adopt_codes, adopt_zeros, window)
    if not group:
        s, z = _params(w, bits, adopt, 0)
        scales[:, 0], zeros[:, 0] = s, z
    for b0 in range(0, din, block):
        b1 = b0 + block
        e_blk = np.zeros((dout, block))
        for j in range(b0, b1):
            if group and j % group == 0:
                s, z = _params(w[:, j:j + group], bits, adopt, j // group)
                scales[:, j // group], zeros[:, j // group] = s, z
            t = w[:, j] / s
            q = np.clip(np.rint(t) + z, 0, maxq)
            if adopt is not None:
                q, n = adopt.pick(q, adopt.codes[:, j], t, z, maxq)
                adopt.codes_n += n
            wq = s * (q - z)
            codes[:, j], what[:, j], tt[:, j] = q, wq, t
            e = (w[:, j] - wq) / r[j, j]
            e_blk[:, j - b0] = e
            w[:, j + 1:b1] -= np.outer(e, r[j, j + 1:b1])
        w[:, b1:] -= e_blk @ r[b0:b1, b1:]
    out = ObsResult(codes, scales, zeros, what, tt)
    if adopt is not None:
        out.adopted_codes, out.adopted_zeros, out.mismatches = adopt.codes_n, adopt.zeros_n, adopt.bad
    return out


def obq_reference(w2: np.ndarray, h_damped: np.ndarray, bits: int, group: int) -> ObsResult:
    """OBS written with the explicit inverse and a Schur downdate after each column.

    After column j is fixed, its row and column are eliminated from H^-1; the
    remaining columns move by -(w_j - w^_j) H^-1[j, k] / H^-1[j, j]. This is the
    textbook optimal-brain-surgeon step, independent of the Cholesky route.
    """
    w = as_f64(w2).copy()
    hinv = np.linalg.inv(np.asarray(h_damped, np.float64))
    dout, din = w.shape
    maxq = (1 << bits) - 1
    ng = din // group if group else 1
    codes = np.zeros((dout, din), np.uint8)
    scales = np.zeros((dout, ng))
    zeros = np.zeros((dout, ng), np.uint8)
    what = np.zeros((dout, din))
    tt = np.zeros((dout, din))
    if not group:
        s, z = grid(w.min(axis=1), w.max(axis=1), bits)
        scales[:, 0], zeros[:, 0] = s, z
    for j in range(din):
        if group and j % group == 0:
            s, z = grid(w[:, j:j + group].min(axis=1), w[:, j:j + group].max(axis=1), bits)
            scales[:, j // group], zeros[:, j // group] = s, z
        t = w[:, j] / s
        q = np.clip(np.rint(t) + z, 0, maxq)
        wq = s * (q - z)
        codes[:, j], what[:, j], tt[:, j] = q, wq, t
        err = w[:, j] - wq
        w[:, j + 1:] -= np.outer(err / hinv[j, j], hinv[j, j + 1:])
        hinv = hinv - np.outer(hinv[:, j], hinv[j, :]) / hinv[j, j]
    return ObsResult(codes, scales, zeros, what, tt)


# ---------------------------------------------------------------------------
# row f2: the GPTAQ base quantizer, asymmetric calibration ([KQ-art] 四, 八)
# ---------------------------------------------------------------------------
# The pages say KronQ's column update is GPTAQ's and that GPTAQ adds an input-drift
# correction to GPTQ ([KQ-art] 四, 八); they do not state its formula. Reading taken here,
# in two stages. X are the inputs the partly quantized model feeds the layer, Xt those of
# the full-precision model, dX = Xt - X, H = X^T X / N, D = dX^T X / N and H~ = H + lam
# mean(diag H) I (GPTQ's damping).
#   1. Drift correction: column q of the layer loses w_q dx_q of output against the
#      full-precision layer; the later columns take its least-squares compensation on their
#      own inputs X_{>q} (damping as ridge rows), delta H~_{>q,>q} = w_q D_{q,>q}. The
#      compensations do not depend on the rounding, so all of them are applied first:
#      W' = W (I + P), row q of P = D_{q,>q} H~_{>q,>q}^-1 (strictly upper triangular).
#   2. GPTQ's column sweep on W' with the same H~.
# Without drift (D = 0) this is GPTQ. Parity against the pages: unpinned (no formula there);
# pinned against the definition of the compensation.
def cross_covariance(a_chunks: Iterable[np.ndarray], b_chunks: Iterable[np.ndarray]) -> np.ndarray:
    """C = A^T B / N in float64 for token-major A, B (bf16 bits or floats) over the same tokens."""
    acc, n = None, 0
    for a, b in zip(a_chunks, b_chunks):
        fa, fb = as_f64(a), as_f64(b)
        part = fa.T @ fb
        acc = part if acc is None else acc + part
        n += fa.shape[0]
    return acc / n


def gptaq_drift_map(h: np.ndarray, d: np.ndarray, lam: float) -> np.ndarray:
    """P, strictly upper triangular: row q = D_{q,>q} H~_{>q,>q}^-1, one solve per row."""
    ht = damped(h, lam)
    dd = np.asarray(d, np.float64)
    n = ht.shape[0]
    p = np.zeros((n, n))
    for q in range(n - 1):
        p[q, q + 1:] = np.linalg.solve(ht[q + 1:, q + 1:], dd[q, q + 1:])
    return p


def gptaq_target(w2: np.ndarray, h: np.ndarray, d: np.ndarray, lam: float) -> np.ndarray:
    """Stage 1: W' = W (I + P), every column's drift compensated on the later columns."""
    w = as_f64(w2)
    return w + w @ gptaq_drift_map(h, d, lam)


def gptaq_quantize(w2: np.ndarray, h: np.ndarray, d: np.ndarray, lam: float, bits: int, group: int,
                   **replay) -> ObsResult:
    """Stages 1 and 2: GPTQ's sweep (``obs_quantize``) of W' with the factor of H~^-1."""
    return obs_quantize(gptaq_target(w2, h, d, lam), chol_inv_upper(h, lam), bits, group, **replay)


def quantize_layer_gptaq(w, h_x, d_x, h_g, rot_in, rot_out, *, bits: int, group: int, damp: float,
                         **replay) -> Dict[str, object]:
    """Row f2 on one layer: BiIP as in ``quantize_layer`` (scales from H_X and H_G), D'' = the
    input-side map of D = dX^T X / N with the same scales and rotation (the second moments of
    the rotated inputs), then the two GPTAQ stages on W'' with H_X'' and D''."""
    w64 = as_f64(w)
    w2, hx2, hg2, s_x, s_g = biip_forward(w64, h_x, h_g, rot_in, rot_out)
    d2 = biip_transform(d_x, s_x, rot_in)
    target = gptaq_target(w2, hx2, d2, damp)
    r = chol_inv_upper(hx2, damp)
    res = obs_quantize(target, r, bits, group, **replay)
    w_hat = biip_inverse(res.what, rot_in, rot_out, s_x, s_g)
    return {"w2": w2, "hx2": hx2, "d2": d2, "s_x": s_x, "s_g": s_g, "target": target, "r": r, "obs": res,
            "w_hat": w_hat}


def rtn_quantize(w2: np.ndarray, bits: int, group: int) -> ObsResult:
    """Round-to-nearest on the same grid, all entries at once, no error feedback."""
    w = as_f64(w2)
    dout, din = w.shape
    maxq = (1 << bits) - 1
    g = group or din
    wg = w.reshape(dout, din // g, g)
    s, z = grid(wg.min(axis=2), wg.max(axis=2), bits)
    t = wg / s[..., None]
    q = np.clip(np.rint(t) + z[..., None], 0, maxq)
    what = s[..., None] * (q - z[..., None])
    return ObsResult(q.reshape(dout, din).astype(np.uint8), s, z.astype(np.uint8),
                     what.reshape(dout, din), t.reshape(dout, din))


# ---------------------------------------------------------------------------
# validation: the Kronecker layer loss  ([KQ-en] Abstract; [KQ-news])
# ---------------------------------------------------------------------------
def kron_loss(dw: np.ndarray, h_x: np.ndarray, h_g: np.ndarray) -> float:
    """tr(dW H_X dW^T H_G), which equals vec(dW)^T (H_X kron H_G) vec(dW) for
    the column-major vec."""
    dw = np.asarray(dw, np.float64)
    return float(np.trace(dw @ np.asarray(h_x, np.float64) @ dw.T @ np.asarray(h_g, np.float64)))


# ---------------------------------------------------------------------------
# step 5b: mixed-precision allocation  ([KQ-art] 六; [KQ-zh] 方法论)
# ---------------------------------------------------------------------------
INFEASIBLE = "infeasible"


def allocate_bits(scores: Sequence[float], n_params: Sequence[int], choices: Sequence[int],
                  target_millibits: int):
    """Greedy upgrade of the most sensitive sub-layers under a fixed average.

    Budget (integer bits) = floor(target_millibits * sum(n) / 1000). Every
    sub-layer starts at min(choices). Visiting sub-layers by score (highest
    first, ties by lower index), each is raised to the largest choice that
    keeps sum(n_l * b_l) within the budget. [KQ-art] 六 upgrades the most
    sensitive class first at a fixed average bit count; the exact greedy rule
    is a reading. A score that is NaN or infinite has no place in the order and
    is an error (ValueError). Returns the list of bits, or INFEASIBLE.
    """
    n = [int(v) for v in n_params]
    ch = sorted(set(int(c) for c in choices))
    if not n or not ch:
        raise ValueError("empty allocation problem")
    if not all(np.isfinite(float(v)) for v in scores):
        raise ValueError("a sensitivity score is not finite (NaN or infinite covariance)")
    total = sum(n)
    budget = (int(target_millibits) * total) // 1000
    bits = [ch[0]] * len(n)
    used = ch[0] * total
    if used > budget:
        return INFEASIBLE
    order = sorted(range(len(n)), key=lambda i: (-float(scores[i]), i))
    for i in order:
        for c in reversed(ch):
            if c <= bits[i]:
                break
            if used + n[i] * (c - bits[i]) <= budget:
                used += n[i] * (c - bits[i])
                bits[i] = c
                break
    return bits


# ---------------------------------------------------------------------------
# after the path: packed codes and the decode matvec  ([KQ-news]: the
# quantized weights ship as packed int4 / int2 with a fused dequantization +
# BiIP matvec for single-token decode; [KQ-art] Q&A: at inference each layer
# applies the two Hadamard transforms, O(d log d) each)
# ---------------------------------------------------------------------------
def container_bits(bits: int) -> int:
    """Bits a code occupies in a packed word: 2 for 2-bit codes, 4 for 3- and 4-bit codes,
    8 above (a reading: the pages name int2 and int4 containers only)."""
    if not 2 <= bits <= 8:
        raise ValueError("bits must be in [2, 8]")
    return 2 if bits == 2 else (4 if bits <= 4 else 8)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """[rows, cols] codes -> [rows, cols * c / 32] uint32 words; word k of a row holds codes
    k * 32 / c + t at bits [c t, c t + c) (c = container_bits(bits))."""
    c = container_bits(bits)
    per = 32 // c
    codes = np.asarray(codes, np.uint64)
    rows, cols = codes.shape
    if cols % per:
        raise ValueError("columns must be a multiple of the codes per word")
    if np.any(codes >= (1 << bits)):
        raise ValueError("code out of range")
    blocks = codes.reshape(rows, cols // per, per)
    words = np.zeros((rows, cols // per), np.uint64)
    for t in range(per):
        words |= blocks[:, :, t] << np.uint64(c * t)
    return words.astype(np.uint32)


def unpack_codes(packed: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """Inverse of ``pack_codes``."""
    c = container_bits(bits)
    per = 32 // c
    words = np.asarray(packed, np.uint64)
    rows = words.shape[0]
    out = np.zeros((rows, cols // per, per), np.uint64)
    for t in range(per):
        out[:, :, t] = (words >> np.uint64(c * t)) & np.uint64((1 << c) - 1)
    return out.reshape(rows, cols).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int) -> np.ndarray:
    """W^''[i][j] = scale[i][g] (code_ij - zero[i][g]), g = j / group (one grid per row for group 0),
    with the scales as stored (float32)."""
    codes = np.asarray(codes, np.float64)
    rows, cols = codes.shape
    gi = (np.arange(cols) // group) if group else np.zeros(cols, np.int64)
    sc = np.asarray(scales, np.float32).astype(np.float64).reshape(rows, -1)
    ze = np.asarray(zeros, np.float64).reshape(rows, -1)
    return sc[:, gi] * (codes - ze[:, gi])


def decode_matvec(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group: int, s_x: np.ndarray,
                  s_g: np.ndarray, rot_in: kq_synth.RotSpec, rot_out: kq_synth.RotSpec, x: np.ndarray, *,
                  inp: bool = True, out: bool = True) -> np.ndarray:
    """y = W^ x for every row x of ``x`` ([tokens, din] -> [tokens, dout]), with the layer's
    quantized weight in original coordinates, W^ = S_G^-1 U_G^T W^'' U_X S_X^-1."""
    w_hat = biip_inverse(dequantize(codes, scales, zeros, group), rot_in, rot_out, s_x, s_g, inp=inp, out=out)
    return np.asarray(x, np.float64) @ w_hat.T


# ---------------------------------------------------------------------------
# the whole per-layer path
# ---------------------------------------------------------------------------
def quantize_layer(w, h_x, h_g, rot_in, rot_out, *, bits: int, group: int, damp: float,
                   inp: bool = True, out: bool = True, scale: bool = True) -> Dict[str, object]:
    """BiIP, damped Cholesky factor of the inverse, OBS sweep, un-rotation, loss."""
    w64 = as_f64(w)
    w2, hx2, hg2, s_x, s_g = biip_forward(w64, h_x, h_g, rot_in, rot_out, inp=inp, out=out, scale=scale)
    r = chol_inv_upper(hx2, damp)
    res = obs_quantize(w2, r, bits, group)
    w_hat = biip_inverse(res.what, rot_in, rot_out, s_x, s_g, inp=inp, out=out)
    return {"w2": w2, "hx2": hx2, "hg2": hg2, "s_x": s_x, "s_g": s_g, "r": r, "obs": res,
            "w_hat": w_hat, "loss": kron_loss(w_hat - w64, h_x, h_g)}
