"""Block-level float64 models of two launch schedules of the HIP library, checked against the
oracle on the CPU: the two-level Cholesky factor of the damped inverse (rank-64 steps inside
256-column super-panels, one rank-256 launch beyond each) and the two-level column sweep
(super-blocks of four blocks). Each model runs every role of every launch from the state the
launch starts from (a role never sees another role's writes of the same launch) and asserts that
no block is written twice in a launch; the result must equal the oracle's plain computation.
These pin the schedules' dependency order, not the kernels' arithmetic (the GPU tests do that)."""
import numpy as np
import pytest

import oracle

B, SP, G, SB = 64, 4, 128, 4


def _spd(rng, n):
    a = rng.standard_normal((n, 2 * n))
    sc = np.exp(rng.uniform(-2, 2, n))
    return sc[:, None] * (a @ a.T / (2 * n)) * sc[None, :]


def chol_model(h, damp):
    d = h.shape[0]
    dp = (d + B - 1) // B * B
    nb = dp // B
    A = np.eye(dp)
    A[:d, :d] = h[::-1, ::-1]
    A[np.arange(d), np.arange(d)] += damp * np.mean(np.diag(h))
    M = np.zeros((dp, dp))

    def blk(X, i, j):
        return X[i * B:(i + 1) * B, j * B:(j + 1) * B]

    for kb in range(nb + 1):
        A0, M0 = A.copy(), M.copy()
        wA, wM = set(), set()

        def put(X, w, i, j, v):
            assert (i, j) not in w, "block written twice in one launch"
            w.add((i, j))
            blk(X, i, j)[:] = v

        s0 = kb // SP * SP
        s1 = min(s0 + SP, nb)
        inner = s0 < kb < nb
        prev = kb % SP != 0
        if kb < nb:  # diagonal role: factor, inverse, panel solve
            akk = blk(A0, kb, kb).copy()
            if prev:
                akk -= blk(A0, kb, kb - 1) @ blk(A0, kb, kb - 1).T
            L = np.linalg.cholesky(np.tril(akk) + np.tril(akk, -1).T)
            Mi = np.linalg.inv(L)
            put(M, wM, kb, kb, Mi)
            for r in range(kb + 1, nb):
                P = blk(A0, r, kb).copy()
                if prev:
                    P -= blk(A0, r, kb - 1) @ blk(A0, kb, kb - 1).T
                put(A, wA, r, kb, P @ Mi.T)
        if kb >= 2:  # row role: row kb - 1 of M
            j = kb - 1
            for c in range(j):
                put(M, wM, j, c, -blk(M0, j, j) @ (blk(M0, j, c) + blk(A0, j, j - 1) @ blk(M0, j - 1, c)))
        if inner and kb + 1 < s1:  # strip of A inside the super-panel
            for i in range(kb + 1, nb):
                for jj in range(kb + 1, s1):
                    put(A, wA, i, jj, blk(A0, i, jj) - blk(A0, i, kb - 1) @ blk(A0, jj, kb - 1).T)
        if inner and kb >= 2:  # substitution sums of the super-panel's rows
            for i in range(kb, s1):
                for c in range(kb - 1):
                    put(M, wM, i, c, blk(M0, i, c) + blk(A0, i, kb - 2) @ blk(M0, kb - 2, c))
        if kb + 1 == s1 and s1 < nb:  # far launch
            A0, M0 = A.copy(), M.copy()
            wA, wM = set(), set()
            for i in range(s1, nb):
                for jj in range(s1, i + 1):
                    acc = sum(blk(A0, i, k) @ blk(A0, jj, k).T for k in range(s0, s1))
                    put(A, wA, i, jj, blk(A0, i, jj) - acc)
            kb0 = max(s0 - 1, 0)
            for i in range(s1, nb):
                for c in range(s1 - 1):
                    acc = sum(blk(A0, i, k) @ blk(M0, k, c) for k in range(kb0, s1 - 1))
                    put(M, wM, i, c, blk(M0, i, c) + acc)
    return np.triu(M[:d, :d][::-1, ::-1])


def obs_model(w2, r, bits, group, blk, nsb):
    w = np.array(w2, np.float64, copy=True)
    dout, din = w.shape
    maxq = (1 << bits) - 1
    codes = np.zeros((dout, din), np.uint8)
    e = np.zeros((2, dout, nsb * blk))
    if not group:
        s_row, z_row = oracle.grid(w.min(axis=1), w.max(axis=1), bits)
    for k in range(din // blk):
        c0 = k * blk
        sb, j = k // nsb, k % nsb
        W0, E0 = w.copy(), e.copy()
        if k > 0 and j == 0:
            near, nq, far, kfar, far_end = E0[(sb + 1) & 1], nsb, E0[(sb + 1) & 1], nsb, din
        elif j > 0:
            near, nq = E0[sb & 1][:, (j - 1) * blk:j * blk], 1
            far, kfar, far_end = near, 1, min((sb + 1) * nsb * blk, din)
        else:
            near, nq, far, kfar, far_end = None, 0, None, 1, c0 + blk
        x = W0[:, c0:c0 + blk].copy()
        if nq:
            x -= near[:, :nq * blk] @ r[c0 - nq * blk:c0, c0:c0 + blk]
        eb = np.zeros((dout, blk))
        for jj in range(blk):
            col = c0 + jj
            if group and col % group == 0:
                s, z = oracle.grid(x[:, jj:jj + group].min(axis=1), x[:, jj:jj + group].max(axis=1), bits)
            elif not group:
                s, z = s_row, z_row
            q = np.clip(np.rint(x[:, jj] / s) + z, 0, maxq)
            wq = s * (q - z)
            codes[:, col] = q
            eb[:, jj] = (x[:, jj] - wq) / r[col, col]
            x[:, jj + 1:] -= np.outer(eb[:, jj], r[col, col + 1:c0 + blk])
            x[:, jj] = wq
        if far_end > c0 + blk:
            w[:, c0 + blk:far_end] = W0[:, c0 + blk:far_end] - far[:, :kfar * blk] @ r[c0 - kfar * blk:c0,
                                                                                      c0 + blk:far_end]
        w[:, c0:c0 + blk] = x
        e[sb & 1][:, j * blk:(j + 1) * blk] = eb
    return codes


@pytest.mark.parametrize("d", [64, 200, 300, 520, 1100])
def test_two_level_cholesky_schedule(d):
    rng = np.random.default_rng(d)
    h = _spd(rng, d)
    want = oracle.chol_inv_upper(h, 0.01)
    got = chol_model(h, 0.01)
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)


@pytest.mark.parametrize("din,blk,group,bits,nsb", [(512, 32, 0, 4, 4), (640, 32, 16, 2, 4), (1024, 64, 64, 3, 4),
                                                    (1152, 128, 128, 2, 4), (384, 128, 128, 4, 4),
                                                    (800, 32, 32, 3, 4), (512, 64, 64, 2, 1)])
def test_two_level_sweep_schedule(din, blk, group, bits, nsb):
    rng = np.random.default_rng(din + blk)
    r = oracle.chol_inv_upper(_spd(rng, din), 0.01)
    w2 = rng.normal(0.0, 0.02, (12, din))
    want = oracle.obs_quantize(w2, r, bits, group)
    near_tie = np.abs(want.t - np.floor(want.t) - 0.5) < 1e-9
    got = obs_model(w2, r, bits, group, blk, nsb)
    assert np.array_equal(got[~near_tie], want.codes[~near_tie])
