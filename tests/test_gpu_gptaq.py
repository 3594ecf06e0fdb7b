"""Row f2 (the GPTAQ base quantizer) on the GPU against the oracle: the cross moment and the
drift moment, the input-side map of a non-symmetric matrix, the drift correction of W'', and
whole layers (codes by the teacher-forced replay, as for GPTQ).

Inputs: kq_synth's x (the inputs the partly quantized model feeds the layer) and xt (the
full-precision model's: a per-channel gain drift and noise on the same draws)."""
import numpy as np
import pytest

import kq_synth
import oracle
from gpu_helpers import DEV, bits_to_dev, check_codes, gptaq_rows, host, rel_fro, require_gpu, scale_tolerance, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _kq():
    import post_quantization_04_amd as kq
    from post_quantization_04_amd import pipeline
    return kq, pipeline


def _workload(n_tokens, dout, din, cfg_id=2, **kw):
    return kq_synth.Workload(kq_synth.scaled(kq_synth.config(cfg_id), n_tokens=n_tokens, dims={"q_proj": (dout, din)},
                                             **kw))


# ---------------------------------------------------------------------------
# cross moment C = Xt^T X / N and drift moment D = C - H_X
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_tokens,d", [(512, 128), (20000, 384), (3001, 100), (40, 64), (1, 8), (73000, 264),
                                        (8170, 136)])
def test_cross_and_drift_moment(n_tokens, d):
    import torch
    kq, pipeline = _kq()
    print(f"xcov n={n_tokens} d={d}", flush=True)
    wl = _workload(n_tokens, 64, d)
    x, xt = wl.x("attn_in"), wl.xt("attn_in")
    xd, xtd = bits_to_dev(x), bits_to_dev(xt)
    c = torch.empty((d, d), dtype=torch.float32, device=DEV)
    kq.accumulate_xcov(xtd, xd, c, 1.0 / n_tokens, 0.0)
    want_c = oracle.cross_covariance([xt], [x])
    assert rel_fro(host(c), want_c) <= 2e-6
    h = pipeline.covariance(xd)
    dm = pipeline.drift_moment(xtd, xd, h)
    torch.cuda.synchronize()
    want_d = want_c - oracle.covariance([x])
    # D = C - H is a difference of two moments each held to 2e-6 relative (their float32
    # accumulation), so its error is bounded by 4e-6 of |C|; |D| is about 0.16 |C| here
    err = np.linalg.norm(host(dm).astype(np.float64) - want_d) / np.linalg.norm(want_c)
    assert err <= 4e-6, f"drift moment error {err:.2e} of |C|"
    if n_tokens >= 512:
        assert rel_fro(host(dm), want_d) <= 3e-5


def test_cross_moment_alpha_beta_strided_and_empty():
    import torch
    kq, pipeline = _kq()
    wl = _workload(9000, 64, 320)
    x, xt = wl.x("attn_in"), wl.xt("attn_in")
    xd, xtd = bits_to_dev(x), bits_to_dev(xt)
    prior = np.random.default_rng(1).standard_normal((256, 256)).astype(np.float32)
    # column slices of wider matrices (pitch 320 != d) and a separate c_in
    c = torch.empty((256, 256), dtype=torch.float32, device=DEV)
    kq.accumulate_xcov(xtd[:, 16:272], xd[:, 40:296], c, 0.5, 0.25, c_in=to_dev(prior))
    want = 0.5 * 9000 * oracle.cross_covariance([xt[:, 16:272]], [x[:, 40:296]]) + 0.25 * prior.astype(np.float64)
    assert rel_fro(host(c), want) <= 2e-6
    # an unaligned column offset takes the register-staged kernel
    c2 = torch.empty((250, 250), dtype=torch.float32, device=DEV)
    kq.accumulate_xcov(xtd[:, 3:253], xd[:, 5:255], c2, 1.0 / 9000, 0.0)
    assert rel_fro(host(c2), oracle.cross_covariance([xt[:, 3:253]], [x[:, 5:255]])) <= 2e-6
    # zero rows: C <- beta C_in; beta = 0 clears without reading
    c3 = to_dev(np.full((256, 256), np.nan, np.float32))
    kq.accumulate_xcov(xtd[:0, :256], xd[:0, :256], c3, 1.0, 0.0)
    torch.cuda.synchronize()
    assert np.all(host(c3) == 0.0)
    kq.accumulate_xcov(xtd[:0, :256], xd[:0, :256], c3, 1.0, 3.0, c_in=to_dev(prior))
    np.testing.assert_array_equal(host(c3), 3.0 * prior)


def test_drift_moment_of_identical_inputs_is_zero():
    """The cross moment is rounded to float32 before H_X is subtracted, so Xt = X gives D = 0
    exactly (and the f2 path then reduces to GPTQ bit for bit, tested below)."""
    import torch
    kq, pipeline = _kq()
    for n_tokens, d in [(20000, 384), (3001, 100)]:
        x = _workload(n_tokens, 64, d).x("attn_in")
        xd = bits_to_dev(x)
        h = pipeline.covariance(xd)
        dm = pipeline.drift_moment(xd, xd, h)
        torch.cuda.synchronize()
        assert np.all(host(dm) == 0.0), f"n={n_tokens} d={d}"


# ---------------------------------------------------------------------------
# input-side map of a non-symmetric matrix with given scales
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [128, 384, 1008, 640])
def test_biip_transform(n):
    kq, pipeline = _kq()
    rng = np.random.default_rng(n)
    m = rng.standard_normal((n, n)).astype(np.float32)
    s = np.exp(rng.normal(0.0, 0.5, n))
    spec = kq_synth.rot_spec(9, "transform", n)
    rot = pipeline.upload_rot(spec.signs, spec.q, DEV)
    md = to_dev(m)
    kq.biip_transform(md, rot.rot, to_dev(s))
    assert rel_fro(host(md), oracle.biip_transform(m, s, spec)) <= 2e-6
    md = to_dev(m)
    kq.biip_transform(md, rot.rot, None)
    assert rel_fro(host(md), oracle.biip_transform(m, np.ones(n), spec)) <= 2e-6


# ---------------------------------------------------------------------------
# the drift correction W' = W + W triu(D R^T, 1) R
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dout,din", [(200, 512), (64, 128), (70, 100), (130, 320)])
def test_gptaq_target(dout, din):
    kq, pipeline = _kq()
    print(f"gptaq target {dout}x{din}", flush=True)
    wl = _workload(6 * din + 512, dout, din)
    x, xt = wl.x("attn_in"), wl.xt("attn_in")
    hx, hg = oracle.covariance([x]), oracle.covariance([wl.g("q_proj")])
    d = oracle.cross_covariance([xt], [x]) - hx
    w2, hx2, _, sx, _ = oracle.biip_forward(wl.weight_f64("q_proj"), hx, hg, wl.rot_in("attn_in"),
                                            wl.rot_out("q_proj"))
    d2 = oracle.biip_transform(d, sx, wl.rot_in("attn_in")).astype(np.float32)
    r32 = oracle.chol_inv_upper(hx2, 0.01).astype(np.float32)
    wd = to_dev(w2)
    kq.gptaq_target(wd, to_dev(d2), to_dev(r32))
    got = host(wd)
    # the arithmetic on the same float32 D'' and R, in float64
    d64, r64 = d2.astype(np.float64), r32.astype(np.float64)
    want = w2 + w2 @ (np.triu(d64 @ r64.T, 1) @ r64)
    corr = want - w2
    assert np.linalg.norm(got - want) <= 1e-11 * np.linalg.norm(corr)
    # against the oracle's drift correction (per-row solves with H~''): R and D'' in float32
    want_o = oracle.gptaq_target(w2, hx2, d2.astype(np.float64), 0.01)
    assert np.linalg.norm(got - want_o) <= 1e-4 * np.linalg.norm(want_o - w2)
    assert rel_fro(got, want_o) <= 2e-6


@pytest.mark.parametrize("dout,din", [(4096, 4096), (4096, 8192)])
def test_gptaq_target_super_tile_edges(dout, din):
    """Widths where the three products run in super-tiles of 2 x 2 (4096) and 4 x 4 tiles (8192):
    random D'' and upper R, sampled rows of the corrected W against the formula in float64."""
    import torch
    kq, _ = _kq()
    print(f"gptaq target {dout}x{din}", flush=True)
    rng = np.random.default_rng(din)
    w = rng.random((dout, din)) - 0.5
    d2 = ((rng.random((din, din), dtype=np.float32) - np.float32(0.5)) * np.float32(2e-3)).astype(np.float32)
    r = np.triu((rng.random((din, din), dtype=np.float32) - np.float32(0.5)) * np.float32(2.0 / np.sqrt(din)))
    wd = torch.from_numpy(w).to(DEV)
    kq.gptaq_target(wd, to_dev(d2), to_dev(r))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, dout // 2, dout - 2, dout - 1])
    got = wd[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    want = gptaq_rows(w, d2, r, rows)
    err = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want - w[rows], axis=1)
    assert err.max() <= 1e-11, f"{err.max():.2e}"


def test_gptaq_target_flags_non_finite_results():
    """A NaN in D'' reaches every later column of the corrected W: info becomes 1; clean inputs leave
    it 0."""
    import torch
    kq, _ = _kq()
    rng = np.random.default_rng(5)
    dout, din = 96, 320
    w = rng.random((dout, din)) - 0.5
    d2 = ((rng.random((din, din)) - 0.5) * 1e-3).astype(np.float32)
    r = np.triu(rng.random((din, din)) - 0.5).astype(np.float32)
    info = torch.zeros(1, dtype=torch.int32, device=DEV)
    kq.gptaq_target(torch.from_numpy(w).to(DEV), to_dev(d2), to_dev(r), info=info)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    d2[7, 200] = np.nan
    wd = torch.from_numpy(w).to(DEV)
    kq.gptaq_target(wd, to_dev(d2), to_dev(r), info=info)
    torch.cuda.synchronize()
    assert int(info.item()) == 1
    assert not bool(torch.isfinite(wd).all())


# ---------------------------------------------------------------------------
# whole layers
# ---------------------------------------------------------------------------
def _run_gptaq_layer(wl, sub, grp, *, bits, drift=True):
    import torch
    kq, pipeline = _kq()
    cfg = wl.cfg
    x = wl.x(grp)
    xd = bits_to_dev(x)
    xtd = bits_to_dev(wl.xt(grp)) if drift else xd
    hx = pipeline.covariance(xd)
    hg = pipeline.covariance(bits_to_dev(wl.g(sub)))
    dm = pipeline.drift_moment(xtd, xd, hx)
    ri = pipeline.upload_rot(wl.rot_in(grp).signs, wl.rot_in(grp).q, DEV)
    ro = pipeline.upload_rot(wl.rot_out(sub).signs, wl.rot_out(sub).q, DEV)
    w = wl.weight(sub)
    wdev = bits_to_dev(w) if w.dtype == np.uint16 else to_dev(w)
    out = pipeline.quantize_layer(wdev, hx, hg, ri, ro, bits=bits, group=cfg.group, block=cfg.block, damp=cfg.damp,
                                  d_x=dm)
    plain = pipeline.quantize_layer(wdev, hx, hg, ri, ro, bits=bits, group=cfg.group, block=cfg.block,
                                    damp=cfg.damp)
    torch.cuda.synchronize()
    return {"codes": host(out.codes), "zeros": host(out.zeros), "scales": host(out.scales), "r": host(out.hx2),
            "w_hat": host(out.w_hat), "hx": host(hx), "hg": host(hg), "d": host(dm),
            "plain_codes": host(plain.codes), "plain_zeros": host(plain.zeros), "plain_scales": host(plain.scales)}


@pytest.mark.parametrize("bits", [2, 4])
def test_layer_gptaq(bits):
    """q_proj recipe at 320 x 512, 24577 tokens, group 128, block 128: the f2 path (drift moment,
    its input-side map, the drift correction, GPTQ's sweep) against the oracle's f2 layer."""
    kq, pipeline = _kq()
    wl = _workload(24577, 320, 512)
    got = _run_gptaq_layer(wl, "q_proj", "attn_in", bits=bits)
    cfg = wl.cfg
    x, xt = wl.x("attn_in"), wl.xt("attn_in")
    hx = oracle.covariance([x])
    d = oracle.cross_covariance([xt], [x]) - hx
    hg = oracle.covariance([wl.g("q_proj")])
    ref = oracle.quantize_layer_gptaq(wl.weight_f64("q_proj"), hx, d, hg, wl.rot_in("attn_in"), wl.rot_out("q_proj"),
                                      bits=bits, group=cfg.group, damp=cfg.damp)
    e_r = rel_fro(got["r"], ref["r"])
    print(f"gptaq layer W{bits}: R {e_r:.2e}", flush=True)
    assert e_r <= 1e-4
    check_codes(got["codes"], got["zeros"], got["scales"], ref["target"], ref["r"], bits, cfg.group,
                label=f"gptaq W{bits}", scale_rtol=scale_tolerance(e_r))
    # the drift correction changes the quantization
    assert np.mean(got["codes"] != got["plain_codes"]) > 0.01


def test_nan_in_full_precision_inputs_is_reported_not_quantized():
    """A NaN only in Xt (the full-precision model's inputs) leaves H_X, the score and the factor
    finite but reaches the drift moment; the drift correction flags it and the layer path raises
    instead of sweeping non-finite weights."""
    kq, pipeline = _kq()
    wl = _workload(6000, 128, 256)
    x, xt = wl.x("attn_in"), wl.xt("attn_in").copy()
    xt[1234, 77] = 0x7FC0  # bf16 quiet NaN
    xd = bits_to_dev(x)
    hx = pipeline.covariance(xd)
    hg = pipeline.covariance(bits_to_dev(wl.g("q_proj")))
    dm = pipeline.drift_moment(bits_to_dev(xt), xd, hx)
    ri = pipeline.upload_rot(wl.rot_in("attn_in").signs, wl.rot_in("attn_in").q, DEV)
    ro = pipeline.upload_rot(wl.rot_out("q_proj").signs, wl.rot_out("q_proj").q, DEV)
    with pytest.raises(kq.KQError) as e:
        pipeline.quantize_layer(bits_to_dev(wl.weight("q_proj")), hx, hg, ri, ro, bits=2, group=128, block=128,
                                damp=0.01, d_x=dm)
    assert e.value.status == kq.KQ_EINVAL


def test_layer_gptaq_without_drift_is_gptq():
    """Xt = X: D = 0 exactly, so the f2 path gives GPTQ's codes, zero points and scales bit for bit."""
    wl = _workload(24577, 320, 512)
    got = _run_gptaq_layer(wl, "q_proj", "attn_in", bits=2, drift=False)
    assert np.all(got["d"] == 0.0)
    np.testing.assert_array_equal(got["codes"], got["plain_codes"])
    np.testing.assert_array_equal(got["zeros"], got["plain_zeros"])
    np.testing.assert_array_equal(got["scales"], got["plain_scales"])
