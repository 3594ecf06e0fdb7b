"""The decode matvec entry point that allocates nothing (kq_decode_matvec_group_noalloc)
against the workspace form (kq_decode_matvec_group) it shares kernels with: two calls in
a row, the second smaller, each equal to the workspace call's result bit for bit, and both
within the decode tolerance of the float64 oracle."""
import numpy as np
import pytest

import kq_synth
import oracle
from gpu_helpers import DEV, host, rel_fro, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _group(rng, douts, din, bits, group, tokens, key):
    """Packed layers sharing one input: (device layer tuples, host pieces for the oracle)."""
    import torch
    import post_quantization_04_amd as kq
    from post_quantization_04_amd import pipeline
    c = oracle.container_bits(bits)
    ri = kq_synth.rot_spec(21, key + "x", din)
    dri = pipeline.upload_rot(ri.signs, ri.q, DEV)
    s_x = rng.uniform(0.3, 3.0, din)
    x = rng.standard_normal((tokens, din)).astype(np.float32)
    dev_layers, host_layers, keep = [], [], [dri]
    for li, dout in enumerate(douts):
        ng = din // group if group else 1
        codes = rng.integers(0, 1 << bits, size=(dout, din), dtype=np.uint8)
        scales = rng.uniform(0.005, 0.05, size=(dout, ng)).astype(np.float32)
        zeros = rng.integers(0, 1 << bits, size=(dout, ng), dtype=np.uint8)
        s_g = rng.uniform(0.3, 3.0, dout)
        ro = kq_synth.rot_spec(21, f"{key}g{li}", dout)
        dro = pipeline.upload_rot(ro.signs, ro.q, DEV)
        keep.append(dro)
        packed = torch.zeros((dout, din * c // 32), dtype=torch.int32, device=DEV)
        kq.pack_codes(to_dev(codes), bits, packed)
        dev_layers.append([packed, to_dev(scales), to_dev(zeros), to_dev(s_g), dro.rot])
        host_layers.append((codes, scales, zeros, s_g, ro))
    return dev_layers, host_layers, (ri, dri, to_dev(s_x), s_x, to_dev(x), x), keep


def _run(douts, din, bits, group, tokens, seed):
    import torch
    import post_quantization_04_amd as kq
    rng = np.random.default_rng(seed)
    dev_layers, host_layers, (ri, dri, s_x_d, s_x, x_d, x), keep = _group(rng, douts, din, bits, group, tokens,
                                                                         f"na{seed}")
    print(f"no-alloc decode: layers {douts} x {din}, {bits} bits, group {group}, {tokens} tokens", flush=True)
    y_ws = [torch.full((tokens, d), float("nan"), device=DEV) for d in douts]
    y_na = [torch.full((tokens, d), float("nan"), device=DEV) for d in douts]
    kq.decode_matvec_group_noalloc([(*L, y) for L, y in zip(dev_layers, y_na)], bits, group, s_x_d, dri.rot, x_d)
    kq.decode_matvec_group([(*L, y) for L, y in zip(dev_layers, y_ws)], bits, group, s_x_d, dri.rot, x_d)
    torch.cuda.synchronize()
    for li, (a, b) in enumerate(zip(y_na, y_ws)):
        ga, gb = host(a), host(b)
        assert np.all(np.isfinite(ga)), f"layer {li}: entries left unwritten"
        np.testing.assert_array_equal(ga, gb, err_msg=f"layer {li}: no-alloc result differs from the workspace call")
        codes, scales, zeros, s_g, ro = host_layers[li]
        want = oracle.decode_matvec(codes, scales, zeros, group, s_x, s_g, ri, ro, x)
        err = rel_fro(ga, want)
        print(f"  layer {li}: equal to the workspace call; {err:.2e} relative Frobenius to the oracle", flush=True)
        assert err <= 2e-5
    del keep


def test_noalloc_matches_workspace_call_twice_then_smaller():
    # first call: three layers with odd-factor output sides (7 x 256, 3 x 512) sharing a 2048-wide
    # input at two tokens; second call: one smaller layer at one token, over the first call's
    # leftover scratch contents
    _run([1792, 1536, 256], 2048, 2, 128, 2, seed=1)
    _run([320], 512, 4, 64, 1, seed=2)


def test_noalloc_rejects_what_the_workspace_call_rejects():
    import torch
    import post_quantization_04_amd as kq
    x = torch.zeros((5, 512), device=DEV)  # five tokens: outside [1, KQ_DECODE_MAX_TOKENS]
    with pytest.raises(kq.KQError) as e:
        kq.lib()  # loaded
        arr = (kq.DecodeLayer * 1)()
        rc = kq.lib().kq_decode_matvec_group_noalloc(arr, 1, 512, 2, 128, None, None, x.data_ptr(), 5, None)
        kq._check(rc, "kq_decode_matvec_group_noalloc")
    assert e.value.status == kq.KQ_EINVAL
