"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times, on outputs the float64 oracle can compute one by one.

* LLaMA-2-7B q_proj (4096 x 4096, 262144 tokens), the bench workload, end to
  end: covariance entries on a sampled channel set against their definition
  (sum over all tokens in float64), the exact diagonals and the trace score;
  then BiIP, the Cholesky factor and the OBS sweep against the oracle run on
  the kernel's own covariances (the oracle cannot form a 262144-token
  covariance in seconds): W'', H_X'', H_G'' and R in full, codes on 64 sampled
  rows under the tie-window replay (rows are independent given R) and the
  per-row OBS objective on those rows.
* LLaMA-3-70B down_proj input covariance (28672 channels, 6328 tiles of
  256 x 256): enough token slices that the slices are split over several
  launches; the float32 partials of all slices kept for one reduce, and (with
  the cap on kept partials lowered) summed launch by launch through a float64
  running sum, bit for bit the same.
* LLaMA-3-70B down_proj drift correction of row f2 (8192 x 28672): random D''
  and upper R, sampled rows of the corrected W'' against the formula in
  float64 (each row needs only O(din^2) work).
* LLaMA-2-13B MLP gate_proj BiIP (13824 x 5120): odd factors 27 and 5 of the
  randomised Hadamard transform at their real sizes; sampled rows of W'' and
  sampled entries of H_G'' from the rotation's definition, H_X'' in full.
"""
import numpy as np
import pytest

import kq_synth
import oracle
from gpu_helpers import DEV, bits_to_dev, check_codes, gptaq_rows, host, rel_fro, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _kq():
    import post_quantization_04_amd as kq
    from post_quantization_04_amd import pipeline
    return kq, pipeline


def _channels(d: int, n: int, seed: int) -> np.ndarray:
    """A sorted channel sample that spans tiles: the ends of several 256-wide tiles plus random ones."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 255, 256, d // 2, d - 257, d - 256, d - 1]
    pick = rng.choice(d, size=n, replace=False)
    return np.unique(np.clip(np.concatenate([edge, pick]), 0, d - 1))


def _check_sampled_cov(x_bits: np.ndarray, h_dev, chans: np.ndarray, label: str) -> None:
    """H[U, U] against sum_t x_t[U] x_t[U]^T / N in float64, error measured against sqrt(H_ii H_jj)."""
    import torch
    n = x_bits.shape[0]
    xs = kq_synth.bf16_bits_to_f64(x_bits[:, chans])
    want = xs.T @ xs / n
    idx = torch.from_numpy(chans).to(h_dev.device)
    got = h_dev.index_select(0, idx).index_select(1, idx).double().cpu().numpy()
    scale = np.sqrt(np.outer(np.diag(want), np.diag(want)))
    err = np.abs(got - want) / scale
    print(f"{label}: {chans.size} sampled channels, max error {err.max():.2e} of sqrt(H_ii H_jj)", flush=True)
    assert err.max() <= 2e-6, f"{label}: covariance entry off by {err.max():.2e}"
    np.testing.assert_array_equal(got, got.T)


def _diag(x_bits: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """Exact float64 diagonal of X^T X / N, summed over token chunks."""
    acc = np.zeros(x_bits.shape[1])
    for r0 in range(0, x_bits.shape[0], chunk):
        c = kq_synth.bf16_bits_to_f64(x_bits[r0:r0 + chunk])
        acc += np.einsum("ij,ij->j", c, c)
    return acc / x_bits.shape[0]


def test_fullsize_q_proj_chain():
    """The bench workload end to end (W2, group 128, block 128, BiIP on both sides)."""
    import torch
    kq, pipeline = _kq()
    cfg = kq_synth.config(2)
    sub = cfg.subs[0]
    dout, din, n_tok = sub.dout, sub.din, cfg.n_tokens
    bits = 2
    wl = kq_synth.Workload(cfg)
    print(f"full-size {cfg.name}: generating {n_tok} tokens", flush=True)
    x, g = wl.x("attn_in"), wl.g(sub.name)
    w = wl.weight(sub.name)
    si, so = wl.rot_in("attn_in"), wl.rot_out(sub.name)

    # step 1: covariances, exactly as the bench launches them (one call each)
    hxd = torch.empty((din, din), dtype=torch.float32, device=DEV)
    hgd = torch.empty((dout, dout), dtype=torch.float32, device=DEV)
    xd = bits_to_dev(x)
    kq.accumulate_cov(xd, hxd, 1.0 / n_tok, 0.0)
    del xd
    gd = bits_to_dev(g)
    kq.accumulate_cov(gd, hgd, 1.0 / n_tok, 0.0)
    del gd
    torch.cuda.synchronize()
    _check_sampled_cov(x, hxd, _channels(din, 96, 1), "H_X")
    _check_sampled_cov(g, hgd, _channels(dout, 96, 2), "H_G")
    dx, dg = _diag(x), _diag(g)
    hx64, hg64 = host(hxd).astype(np.float64), host(hgd).astype(np.float64)
    # the diagonal is a sum of positive terms: the same 2e-6 bound, now relative
    np.testing.assert_allclose(np.diag(hx64), dx, rtol=2e-6)
    np.testing.assert_allclose(np.diag(hg64), dg, rtol=2e-6)
    score = pipeline.score(hxd, hgd)
    assert score == pytest.approx(oracle.sensitivity(np.diag(dx), np.diag(dg)), rel=1e-6)
    del x, g

    # steps 2-4 on the kernel's covariances
    w64 = wl.weight_f64(sub.name)
    w2_ref, hx2_ref, hg2_ref, sx_ref, sg_ref = oracle.biip_forward(w64, hx64, hg64, si, so)
    ri, ro = pipeline.upload_rot(si.signs, si.q, DEV), pipeline.upload_rot(so.signs, so.q, DEV)
    w2d = torch.empty((dout, din), dtype=torch.float64, device=DEV)
    s_x = torch.empty(din, dtype=torch.float64, device=DEV)
    s_g = torch.empty(dout, dtype=torch.float64, device=DEV)
    kq.biip_rotate(bits_to_dev(w), w2d, hxd, hgd, ri.rot, ro.rot, pipeline.ALL_SIDES, s_x, s_g)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(s_x), sx_ref, rtol=1e-12)
    np.testing.assert_allclose(host(s_g), sg_ref, rtol=1e-12)
    w2 = host(w2d)
    e_w2, e_hx2, e_hg2 = rel_fro(w2, w2_ref), rel_fro(host(hxd), hx2_ref), rel_fro(host(hgd), hg2_ref)
    print(f"BiIP: W'' {e_w2:.2e}, H_X'' {e_hx2:.2e}, H_G'' {e_hg2:.2e} relative Frobenius", flush=True)
    assert e_w2 <= 1e-6 and e_hx2 <= 1e-6 and e_hg2 <= 1e-6
    del hgd, hg64, hg2_ref

    info = torch.zeros(1, dtype=torch.int32, device=DEV)
    kq.cholesky_inv(hxd, cfg.damp, info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    r_ref = oracle.chol_inv_upper(hx2_ref, cfg.damp)
    r = host(hxd)
    e_r = rel_fro(r, r_ref)
    print(f"Cholesky: R {e_r:.2e} relative Frobenius", flush=True)
    assert e_r <= 1e-4 and e_r <= 1e-5  # measured 3.5e-6

    ng = din // cfg.group
    codes = torch.empty((dout, din), dtype=torch.uint8, device=DEV)
    scales = torch.empty((dout, ng), dtype=torch.float32, device=DEV)
    zeros = torch.empty((dout, ng), dtype=torch.uint8, device=DEV)
    kq.obs_quantize(w2d, hxd, bits, cfg.group, cfg.block, codes, scales, zeros)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, dout - 1], np.random.default_rng(3).choice(dout, 62, replace=False)]))
    res = check_codes(host(codes)[rows], host(zeros)[rows], host(scales)[rows], w2_ref[rows], r_ref, bits,
                      cfg.group, label="q_proj full size")
    # per-row OBS objective dw H dw^T with the damped H_X''
    hd = oracle.damped(hx2_ref, cfg.damp)
    dw_got, dw_want = host(w2d)[rows] - w2_ref[rows], res.what - w2_ref[rows]
    obj_got = np.einsum("ij,jk,ik->i", dw_got, hd, dw_got)
    obj_want = np.einsum("ij,jk,ik->i", dw_want, hd, dw_want)
    print(f"OBS: {rows.size} rows, {res.adopted_codes} tie-window codes, objective {obj_got.sum():.6g} "
          f"(oracle {obj_want.sum():.6g})", flush=True)
    np.testing.assert_allclose(obj_got, obj_want, rtol=1e-3)


def _cov_both_paths(xd, d, n_tok, monkeypatch):
    """H from the kept partials of every slice (one reduce) and from launch-by-launch float64 sums."""
    import torch
    kq, _ = _kq()
    h = torch.empty((d, d), dtype=torch.float32, device=DEV)
    kq.accumulate_cov(xd, h, 1.0 / n_tok, 0.0)
    h_run = torch.empty((d, d), dtype=torch.float32, device=DEV)
    with monkeypatch.context() as m:
        m.setenv("KQ_COV_KEEP_ALL_MAX_BYTES", "0")
        kq.accumulate_cov(xd, h_run, 1.0 / n_tok, 0.0)
    torch.cuda.synchronize()
    # the slices are added one by one in slice order in float64 either way
    assert torch.equal(h, h_run), "kept partials and running sums differ"
    return h


def test_fullsize_down_proj_covariance_slice_groups(monkeypatch):
    """28672 channels (6328 tiles): four token slices over two launches."""
    kq, pipeline = _kq()
    n_tok = 3 * 16384 + 100  # four slices of 16384 tokens, the last one ragged
    cfg = kq_synth.scaled(kq_synth.config(4), n_tokens=n_tok, dims={})
    wl = kq_synth.Workload(cfg)
    x = wl.x("down_in")
    d = x.shape[1]
    assert d == 28672
    print(f"full-size down_proj input covariance: {n_tok} x {d}", flush=True)
    xd = bits_to_dev(x)
    h = _cov_both_paths(xd, d, n_tok, monkeypatch)
    del xd
    _check_sampled_cov(x, h, _channels(d, 96, 4), "H_X down_proj")
    np.testing.assert_allclose(np.diag(host(h)).astype(np.float64), _diag(x), rtol=2e-6)


def test_fullsize_wide_covariance_whole_slice_groups(monkeypatch):
    """11008 channels (946 tiles; LLaMA-2-7B's MLP width), 8 token slices and a ragged ninth: one
    launch of 8 whole slices, one per XCD, then the ragged slice in tile groups."""
    kq, pipeline = _kq()
    n_tok = 8 * 16384 + 5000
    cfg = kq_synth.scaled(kq_synth.config(2), n_tokens=n_tok, dims={"q_proj": (64, 11008)})
    x = kq_synth.Workload(cfg).x("attn_in")
    d = x.shape[1]
    assert d == 11008
    print(f"wide covariance: {n_tok} x {d}", flush=True)
    xd = bits_to_dev(x)
    h = _cov_both_paths(xd, d, n_tok, monkeypatch)
    del xd
    _check_sampled_cov(x, h, _channels(d, 96, 5), "H_X 11008")
    np.testing.assert_allclose(np.diag(host(h)).astype(np.float64), _diag(x), rtol=2e-6)


def test_fullsize_gptaq_target_down_proj():
    """The drift correction at 8192 x 28672 (8 x 8-tile super-blocks, the launch shape the bench
    times): random D'' and upper R (zero below the diagonal, as the factor leaves it), sampled rows
    against the formula in float64."""
    import torch
    kq, _ = _kq()
    dout, din = 8192, 28672
    rng = np.random.default_rng(70)
    print(f"full-size gptaq target {dout} x {din}: generating inputs", flush=True)
    w = rng.random((dout, din)) - 0.5
    d2 = rng.random((din, din), dtype=np.float32)
    d2 -= np.float32(0.5)
    d2 *= np.float32(2e-3)
    r = rng.random((din, din), dtype=np.float32)
    r -= np.float32(0.5)
    r *= np.float32(2.0 / np.sqrt(din))
    for k0 in range(0, din, 1024):  # zero below the diagonal, a block of rows at a time
        r[k0:k0 + 1024, :k0] = 0.0
        r[k0:k0 + 1024, k0:k0 + 1024] = np.triu(r[k0:k0 + 1024, k0:k0 + 1024])
    wd = torch.from_numpy(w).to(DEV)
    kq.gptaq_target(wd, to_dev(d2), to_dev(r))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 4095, 4096, 8190, 8191])
    got = wd[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del wd
    print("reference rows", flush=True)
    want = gptaq_rows(w, d2, r, rows)
    corr = want - w[rows]
    err = np.linalg.norm(got - want, axis=1) / np.linalg.norm(corr, axis=1)
    print(f"gptaq target rows: max error {err.max():.2e} of the correction", flush=True)
    assert err.max() <= 1e-11


def test_fullsize_mlp_biip_odd_factors():
    """gate_proj 13824 x 5120: output side 27 x 512, input side 5 x 1024, both transformed in full."""
    import torch
    kq, pipeline = _kq()
    cfg = kq_synth.scaled(kq_synth.config(3), n_tokens=8192, dims={})
    wl = kq_synth.Workload(cfg)
    sub = cfg.sub("gate_proj")
    dout, din = sub.dout, sub.din
    si, so = wl.rot_in(sub.x_group), wl.rot_out(sub.name)
    assert (so.m, so.p, si.m, si.p) == (27, 512, 5, 1024)
    hxd = pipeline.covariance(bits_to_dev(wl.x(sub.x_group)))
    hgd = pipeline.covariance(bits_to_dev(wl.g(sub.name)))
    torch.cuda.synchronize()
    hx64, hg64 = host(hxd).astype(np.float64), host(hgd).astype(np.float64)
    w = wl.weight(sub.name)
    w64 = wl.weight_f64(sub.name)
    ri, ro = pipeline.upload_rot(si.signs, si.q, DEV), pipeline.upload_rot(so.signs, so.q, DEV)
    w2d = torch.empty((dout, din), dtype=torch.float64, device=DEV)
    s_x = torch.empty(din, dtype=torch.float64, device=DEV)
    s_g = torch.empty(dout, dtype=torch.float64, device=DEV)
    kq.biip_rotate(bits_to_dev(w), w2d, hxd, hgd, ri.rot, ro.rot, pipeline.ALL_SIDES, s_x, s_g)
    torch.cuda.synchronize()
    sx, sg = oracle.biip_scales(hx64), oracle.biip_scales(hg64)
    np.testing.assert_allclose(host(s_x), sx, rtol=1e-12)
    np.testing.assert_allclose(host(s_g), sg, rtol=1e-12)
    # W'' rows from the definition: U_G[rows] (S_G W S_X) U_X^T
    rows = np.unique(np.concatenate([[0, 511, 512, dout - 1], np.random.default_rng(5).choice(dout, 12, False)]))
    w_s = sg[:, None] * w64 * sx[None, :]
    want = oracle.rotate_rows(oracle.rotation_rows(so, rows) @ w_s, si)
    got = host(w2d)[rows]
    e_w = rel_fro(got, want)
    # H_X'' in full
    _, hx2_ref, _, _, _ = oracle.biip_forward(w64[:1], hx64, None, si, so, out=False)
    e_hx = rel_fro(host(hxd), hx2_ref)
    # H_G'' sampled entries: u_i S^-1 H_G S^-1 u_j^T
    u = oracle.rotation_rows(so, rows)
    hs = hg64 / sg[:, None] / sg[None, :]
    want_g = u @ hs @ u.T
    got_g = host(hgd)[np.ix_(rows, rows)].astype(np.float64)
    e_g = np.abs(got_g - want_g).max() / np.sqrt(np.outer(np.diag(want_g), np.diag(want_g))).min()
    print(f"BiIP 13824 x 5120: W'' rows {e_w:.2e}, H_X'' {e_hx:.2e}, H_G'' entries {e_g:.2e}", flush=True)
    assert e_w <= 1e-6 and e_hx <= 1e-6 and e_g <= 1e-6
