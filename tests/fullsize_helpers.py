"""Float64 reductions over full-size calibration matrices for the full-size GPU
tests: exact diagonals, sampled covariance entries and projections X V, each
summed over token chunks in a fixed order (threads only split the chunks).
Plus the property checks used where the oracle's own Cholesky factor would
take minutes on the host (widths 13824, 14336 and 28672)."""
import concurrent.futures as cf
import os

import numpy as np

import kq_synth
import oracle

CHUNK = 2048


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def stream(a_bits: np.ndarray, fn):
    """fn(float64 chunk) for every CHUNK-row chunk of a [N, d] bf16 matrix, summed in chunk order."""
    n = a_bits.shape[0]
    starts = list(range(0, n, CHUNK))

    def one(r0):
        return fn(kq_synth.bf16_bits_to_f64(a_bits[r0:r0 + CHUNK]))

    with cf.ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(one, starts))
    out = parts[0]
    for p in parts[1:]:
        out = out + p
    return out


def exact_diag(a_bits: np.ndarray) -> np.ndarray:
    """diag(A^T A / N) in float64."""
    return stream(a_bits, lambda c: np.einsum("ij,ij->j", c, c)) / a_bits.shape[0]


def sampled_cov(a_bits: np.ndarray, chans: np.ndarray) -> np.ndarray:
    """(A^T A / N)[chans][:, chans] from the definition."""
    return stream(a_bits, lambda c: c[:, chans].T @ c[:, chans]) / a_bits.shape[0]


def projected_cov(a_bits: np.ndarray, v: np.ndarray) -> np.ndarray:
    """V^T (A^T A / N) V = (A V)^T (A V) / N for a [d, k] matrix V."""
    def f(c):
        y = c @ v
        return y.T @ y

    return stream(a_bits, f) / a_bits.shape[0]


def full_cov(a_bits: np.ndarray) -> np.ndarray:
    """A^T A / N in float64, 16384-token chunks in order (the oracle's covariance; widths up to ~5120)."""
    return oracle.covariance(a_bits[r0:r0 + 16384] for r0 in range(0, a_bits.shape[0], 16384))


def channels(d: int, n: int, seed: int) -> np.ndarray:
    """A sorted channel sample that spans tiles: the ends of several 256-wide tiles plus random ones."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 255, 256, d // 2, d - 257, d - 256, d - 1]
    pick = rng.choice(d, size=n, replace=False)
    return np.unique(np.clip(np.concatenate([edge, pick]), 0, d - 1))


def entry_error(got: np.ndarray, want: np.ndarray) -> float:
    """Largest |got - want| of a symmetric block, measured against sqrt(H_ii H_jj)."""
    dg = np.sqrt(np.abs(np.diag(want)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - want) / np.outer(dg, dg)))


def transformed_block(a_bits: np.ndarray, s: np.ndarray, spec: kq_synth.RotSpec, idx: np.ndarray) -> np.ndarray:
    """(U S^-1 H S^-1 U^T)[idx][:, idx] for H = A^T A / N, from the definition: the rows idx of
    U S^-1 applied to every token row of A."""
    v = (oracle.rotation_rows(spec, idx) / s[None, :]).T  # [d, k]
    return projected_cov(a_bits, np.ascontiguousarray(v))


def r_residual(r_rows: np.ndarray, rows: np.ndarray, h2: np.ndarray, delta: float) -> float:
    """max |(R H~ R^T)[rows][:, rows] - I| with H~ = H'' + delta I (R upper, R^T R = H~^-1 means
    R H~ R^T = I). h2 is float32 [d, d]; the product runs in float64 over column blocks."""
    d = h2.shape[0]
    rr = np.asarray(r_rows, np.float64)
    prod = np.zeros_like(rr)
    for c0 in range(0, d, 2048):
        prod[:, c0:c0 + 2048] = rr @ h2[:, c0:c0 + 2048].astype(np.float64)
    prod += delta * rr
    m = prod @ rr.T
    return float(np.max(np.abs(m - np.eye(len(rows)))))


def trailing_block_error(r: np.ndarray, h2: np.ndarray, delta: float, k: int) -> float:
    """Rows and columns d-k.. of R depend only on the trailing k x k block of H~ (H~ = V V^T with V
    upper gives H~[t, t] = V[t, t] V[t, t]^T, and R = V^-1): relative Frobenius error of that block
    of R against the oracle's factor of the damped trailing block."""
    d = h2.shape[0]
    t = slice(d - k, d)
    sub = np.asarray(h2[t, t], np.float64).copy()
    sub[np.diag_indices(k)] += delta
    want = oracle.chol_inv_upper(sub, 0.0)
    got = np.asarray(r[t, t], np.float64)
    return float(np.linalg.norm(got - want) / np.linalg.norm(want))


def w2_rows(w64: np.ndarray, s_x: np.ndarray, s_g: np.ndarray, si: kq_synth.RotSpec, so: kq_synth.RotSpec,
            rows: np.ndarray) -> np.ndarray:
    """Rows of W'' = U_G S_G W S_X U_X^T from the definition (U_G's rows built entry by entry)."""
    w_s = s_g[:, None] * w64 * s_x[None, :]
    return oracle.rotate_rows(oracle.rotation_rows(so, rows) @ w_s, si)


def norm_cv(m) -> tuple:
    """(column-norm CV, row-norm CV) of a matrix, in float64 on the device that holds it."""
    import torch
    m = m.double()
    c, r = torch.linalg.vector_norm(m, dim=0), torch.linalg.vector_norm(m, dim=1)
    return float(c.std(unbiased=False) / c.mean()), float(r.std(unbiased=False) / r.mean())
