#!/usr/bin/env python3
"""Throughput of the KronQ per-layer quantization path on one MI355X.

One step is one pass of the whole path over every layer of a workload whose
inputs are already resident in HBM:
  1. H_X = X^T X / N of every input group and H_G = G^T G / N of every layer
     (bf16-MFMA symmetric rank-k updates over all N tokens),
  2. the trace scores tr(H_G) tr(H_X) and the bit allocation from them,
  3. BiIP (diagonal rescale + randomised Hadamard rotation on both sides of W,
     with H_X and H_G transformed alongside),
  4. the damped Cholesky factor of H_X''^-1,
  5. the column-wise OBS sweep with its lazy-batch trailing products.
Default workload (--config 4): the LLaMA-3-70B down_proj (W 8192 x 28672 bf16
with input-column outliers, column-norm CV 9.2; X 262144 x 28672 and G
262144 x 8192 bf16), 2-bit, group 128, block 128, damping 0.01: the largest
workload that fits one GPU. --config 1, 2, 3 and 5 run the 64 x 128 linear
layer, the LLaMA-2-7B q_proj (--bits 2 or 4), the LLaMA-2-13B MLP (gate, up,
down at 3 bits) and the LLaMA-3-8B block (seven layers, bits from the
allocation over {2, 3, 4} at 3.0 average bits). Seeded synthetic inputs.

Schedule: for one layer with at most 8192 inputs the Cholesky factor needs
only H_X'' (the input side of BiIP), so it runs on one stream while the H_G
covariance runs on a second stream kept off some CUs; the output side of BiIP
and the sweep follow with every CU. Wider layers, several layers (or --serial)
run on one stream: all covariances, the scores and the allocation (the
sweeps' widths depend on it), then per layer BiIP, the factor and the sweep.

value = weights quantised per second, end to end including the covariance
accumulation. The roofline object covers the kernel with the most time in the
step (bf16-MFMA SYRK, float32-MFMA Cholesky steps or float64-MFMA sweep
steps): its algorithmic flops per launch over its average launch duration,
timed with HIP events that the library records around each launch on its
stream during the timed steps. The CPU baseline is the float64 oracle timed
on a bounded sample of the same workload on this host, scaled to one step.

--peaks measures the machine instead: sustained bf16, float32 and float64
MFMA rates (random and constant operands, with the shader clock they ran at)
and a device-to-device copy, as context for the published peaks the rooflines
are priced against.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--config", type=int, default=4, choices=(1, 2, 3, 4, 5),
                   help="workload: 1 linear 64x128, 2 LLaMA-2-7B q_proj, 3 LLaMA-2-13B MLP, 4 LLaMA-3-70B down_proj "
                        "(default), 5 LLaMA-3-8B block")
    p.add_argument("--bits", type=int, default=2, choices=(2, 4), help="bit width of the LLaMA-2-7B q_proj (--config 2)")
    p.add_argument("--serial", action="store_true",
                   help="run every stage on one stream (per-stage profiles) instead of the two-stream schedule")
    p.add_argument("--gptaq", action="store_true",
                   help="row f2: the GPTAQ base quantizer in the step (drift moment of full-precision inputs of the "
                        "same shape, its input-side map and the drift correction of W'' before the sweep)")
    p.add_argument("--overlap", action="store_true",
                   help="one layer: use the two-stream schedule at any width (by default only up to 8192 inputs)")
    p.add_argument("--reserve-cus", type=int, default=80,
                   help="CUs the second stream leaves to the Cholesky factor (0: no CU mask)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the timed oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after timing, copy 1 GiB device-to-device (a reference kernel for HBM byte counters)")
    p.add_argument("--decode", action="store_true",
                   help="instead of the quantization step: the packed-code decode matvec (one JSON line)")
    p.add_argument("--capture", action="store_true",
                   help="calibration capture of one LLaMA-2-7B block (forward + one backward) and its covariances")
    p.add_argument("--decode-per-layer", action="store_true",
                   help="with --decode: one kq_decode_matvec call per layer instead of one group call per shared input")
    p.add_argument("--peaks", action="store_true",
                   help="instead of the quantization step: sustained MFMA rates and HBM copy bandwidth")
    p.add_argument("--traffic-summary", nargs=4, metavar=("KERNEL", "WORKLOAD", "FETCH_DIR", "WRITE_DIR"),
                   help="no run: turn two rocprofv3 --pmc runs of '--copy-calibration' (FETCH_SIZE, then "
                        "WRITE_SIZE) into the per-launch HBM bytes of KERNEL, written to "
                        "profiles/KERNEL_WORKLOAD_hbm_traffic.json")
    return p.parse_args()


def side_stream(dev, reserve: int):
    """Second stream at default priority; with reserve > 0 its kernels are kept off the last
    `reserve` CUs of the mask (hipExtStreamCreateWithCUMask), which stay free for the
    latency-bound Cholesky steps. Mask bit i is a CU of XCD i mod 8, so the reserved CUs are
    spread evenly over the XCDs; a mask that leaves an XCD no CU is refused."""
    import ctypes
    import torch
    if reserve <= 0:
        return torch.cuda.Stream(device=dev)
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    bits = [1] * n_cu
    for i in range(n_cu - reserve, n_cu):
        bits[i] = 0
    words = [0] * ((n_cu + 31) // 32)
    for i, b in enumerate(bits):
        words[i // 32] |= b << (i % 32)
    # the HIP runtime torch itself loaded (a second copy of the runtime would not know its device state)
    own = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    hip = ctypes.CDLL(own if os.path.exists(own) else "libamdhip64.so")
    handle = ctypes.c_void_p()
    arr = (ctypes.c_uint32 * len(words))(*words)
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(len(words)), arr)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({rc})")
    _OWNED_STREAMS.append((hip, handle))
    return torch.cuda.ExternalStream(handle.value, device=dev)


_OWNED_STREAMS = []


def release_streams() -> None:
    """Destroys the streams side_stream created (after the device is idle)."""
    import torch
    torch.cuda.synchronize()
    while _OWNED_STREAMS:
        hip, handle = _OWNED_STREAMS.pop()
        hip.hipStreamDestroy(handle)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # noqa: BLE001
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(wl, cfg, bits_plan):
    """The float64 oracle, as it stands, on a bounded sample of the workload, scaled to one whole step.

    Per step of the workload the oracle would: form every covariance over all tokens, score and
    allocate, run BiIP, the Cholesky factor of the inverse and the column sweep of every layer. The
    sample times each piece on a slice whose cost scales in a known way: covariances on a token slice
    (cost linear in tokens), BiIP on a layer shrunk by a factor (cost in the bytes of W, H_X and H_G),
    the factor at width <= 4096 (cost d^3), the sweep on a few rows (cost linear in rows). The sample
    takes 10-30 s of host time."""
    import numpy as np

    import kq_synth
    import oracle

    def biip_work(dout, din):
        # the oracle rotates with the dense Hadamard matrix: k rows of n = m p cost k n (p + m)
        (mi, ki), (mo, ko) = kq_synth.split_odd(din), kq_synth.split_odd(dout)
        ci, co = (1 << ki) + mi, (1 << ko) + mo
        return dout * din * (ci + co) + 2 * din * din * ci + 2 * dout * dout * co

    t_total, notes = 0.0, []
    n_tok = cfg.n_tokens
    tok = min(n_tok, 2048)
    # covariances: every X group and every G on `tok` tokens, scaled to n_tok
    t0 = time.perf_counter()
    for grp in cfg.x_groups:
        oracle.covariance([wl.x_chunk(grp, 0)[:tok]])
    for s in cfg.subs:
        oracle.covariance([wl.g_chunk(s.name, 0)[:tok]])
    t = (time.perf_counter() - t0) * (n_tok / tok)
    t_total += t
    notes.append(f"covariances on {tok} of {n_tok} tokens (x{n_tok / tok:g}) {t:.1f} s")
    t_biip = t_chol = t_obs = 0.0
    chol_seen = {}
    for li, s in enumerate(cfg.subs):
        # BiIP on a layer shrunk by f on each side (bytes scale by f^2)
        f = 1
        while s.dout // (2 * f) >= 512 and s.din // (2 * f) >= 512 and (s.dout // (2 * f)) % 2 == 0 \
                and (s.din // (2 * f)) % 2 == 0:
            f *= 2
        do, di = s.dout // f, s.din // f
        rng = np.random.default_rng(li)
        hx = np.eye(di) + 0.01
        hg = np.eye(do) + 0.01
        w = rng.normal(0, 0.02, (do, di))
        si, so = kq_synth.rot_spec(99, f"cpu{di}", di), kq_synth.rot_spec(99, f"cpuo{do}", do)
        t0 = time.perf_counter()
        w2, hx2, _, _, _ = oracle.biip_forward(w, hx, hg, si, so)
        tb = (time.perf_counter() - t0) * (biip_work(s.dout, s.din) / biip_work(do, di))
        t_biip += tb
        # the factor: at min(din, 4096), scaled by d^3; once per input group of equal width
        dc = min(s.din, 4096)
        if dc not in chol_seen:
            h = np.eye(dc) + rng.standard_normal((dc, dc)) * 1e-3
            h = h @ h.T
            t0 = time.perf_counter()
            oracle.chol_inv_upper(h, cfg.damp)
            chol_seen[dc] = time.perf_counter() - t0
        t_chol += chol_seen[dc] * (s.din / dc) ** 3
        # the sweep on 4 rows of the full width (an identity factor costs the same as any other)
        rows = 4
        r = np.eye(s.din)
        t0 = time.perf_counter()
        oracle.obs_quantize_blocked(rng.normal(0, 0.02, (rows, s.din)), r, bits_plan[li], cfg.group, cfg.block)
        t_obs += (time.perf_counter() - t0) * (s.dout / rows)
        del r
    t_total += t_biip + t_chol + t_obs
    notes.append(f"BiIP on layers shrunk to >= 512 per side (x the oracle's rotation work) {t_biip:.1f} s")
    notes.append(f"Cholesky factor of the inverse at width <= 4096 (x d^3) {t_chol:.1f} s")
    notes.append(f"column sweep on 4 rows (x rows) {t_obs:.1f} s")
    weights = sum(s.dout * s.din for s in cfg.subs)
    return {
        "value": round(weights / t_total / 1e6, 5),
        "unit": "Mweights/s",
        "cores": cpu_threads(),
        "kind": "oracle",
        "sample": "float64 oracle, scaled to one step: " + "; ".join(notes) + f"; total {t_total:.1f} s per step",
        "seconds_per_step": round(t_total, 2),
    }


ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
# kernel -> (source file, peak, unit, bound)
KERNELS = {
    "syrk_partial": ("syrk.hip", 2500.0, "TFLOP/s", "mfma"),
    "xcov_partial": ("syrk.hip", 2500.0, "TFLOP/s", "mfma"),
    "gptaq_drift_kernel": ("gptaq.hip", 78.6, "TFLOP/s", "mfma"),
    "gptaq_weight_kernel": ("gptaq.hip", 78.6, "TFLOP/s", "mfma"),
    "gptaq_update_kernel": ("gptaq.hip", 78.6, "TFLOP/s", "mfma"),
    "chol_far_kernel": ("chol.hip", 157.3, "TFLOP/s", "mfma"),
    "chol_step_kernel": ("chol.hip", 157.3, "TFLOP/s", "mfma"),
    "obs_step_kernel": ("obs.hip", 78.6, "TFLOP/s", "mfma"),
}


def chol_far_flops(d: int, b: int = 64, sp: int = 4) -> int:
    """Algorithmic flops of the Cholesky factor's far launches (rank-256 updates after each super-panel
    of sp 64-blocks): the lower triangle of the trailing block of A, and the substitution sums for
    the rows beyond the super-panel over the nonzero part of M (columns up to each k)."""
    nb = -(-d // b)
    total = 0
    for s0 in range(0, nb, sp):
        s1 = min(s0 + sp, nb)
        if s1 >= nb:
            break
        nrem = nb - s1                       # trailing blocks
        total += 2 * b ** 3 * (s1 - s0) * nrem * (nrem + 1) // 2
        for k in range(max(s0 - 1, 0), s1 - 1):  # row blocks beyond s1 x column blocks c <= k
            total += 2 * b ** 3 * nrem * (k + 1)
    return total


def kernel_source(kernel: str) -> str:
    return os.path.join(ROOT, "post_quantization_04_amd", "csrc", KERNELS[kernel][0])


def traffic_file(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.json")


def source_hash(path: str) -> str:
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def pmc_dispatches(run_dir: str, counter: str):
    """[(dispatch id, kernel name, counter value)] from a rocprofv3 --pmc csv run, in dispatch order."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    vals, names = {}, {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                k = int(row["Dispatch_Id"])
                vals[k] = vals.get(k, 0.0) + float(row["Counter_Value"])
                names[k] = row["Kernel_Name"]
    return [(k, names[k], vals[k]) for k in sorted(vals)]


def traffic_summary(kernel: str, workload: str, fetch_dir: str, write_dir: str) -> int:
    """HBM bytes per launch of `kernel`: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what
    the same counter reads for the final 1 GiB device-to-device copy of a '--copy-calibration' run."""
    src = kernel_source(kernel)
    out = {"kernel": kernel, "workload": workload, "source": os.path.relpath(src, ROOT),
           "source_sha256": source_hash(src), "copy_bytes": COPY_BYTES}
    for key, run_dir, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = pmc_dispatches(run_dir, counter)
        copy = rows[-1]  # the calibration copy is the last dispatch of the run
        if kernel in copy[1] or copy[2] <= 0:
            raise RuntimeError(f"{counter}: last dispatch {copy[1]!r} is not the calibration copy")
        mine = [v for _, n, v in rows if f"{kernel}(" in n or f"{kernel}<" in n]
        if not mine:
            raise RuntimeError(f"{counter}: no {kernel} dispatch")
        scale = COPY_BYTES / (copy[2] * 1024.0)
        out[f"{key}_kib_per_launch"] = sum(mine) / len(mine)
        out[f"{key}_launches"] = len(mine)
        out[f"copy_{key}_kib"] = copy[2]
        out[f"{key}_scale"] = scale
        out[f"{key}_bytes_per_launch"] = out[f"{key}_kib_per_launch"] * 1024.0 * scale
    out["traffic_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    path = traffic_file(kernel, workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


def stored_traffic(kernel: str, workload: str):
    """Per-launch HBM bytes of `kernel` from the committed counter summary, or None when the summary is
    missing or was taken on a different version of the kernel's source."""
    try:
        with open(traffic_file(kernel, workload)) as f:
            rec = json.load(f)
        if rec.get("source_sha256") != source_hash(kernel_source(kernel)):
            return None
        return int(round(rec["traffic_bytes_per_launch"]))
    except (OSError, ValueError, KeyError):
        return None


# LLaMA-2-7B linear layers of one decoder block: (name, dout, din)
DECODE_LAYERS = [("q_proj", 4096, 4096), ("k_proj", 4096, 4096), ("v_proj", 4096, 4096), ("o_proj", 4096, 4096),
                 ("gate_proj", 11008, 4096), ("up_proj", 11008, 4096), ("down_proj", 4096, 11008)]
# layers of a block that read the same input (and so share the input side): (din, [layer indices])
DECODE_GROUPS = [(4096, [0, 1, 2]), (4096, [3]), (4096, [4, 5]), (11008, [6])]
DECODE_BLOCKS = 32


def capture_bench(args) -> int:
    """Calibration capture for one LLaMA-2-7B decoder block with seeded random weights: forward
    over 128 sequences of 2048 seeded token states, one backward pass from a seeded linear loss,
    every linear layer's input (per input group) and output gradient kept in bf16; then H_X of
    the four input groups and H_G of the seven layers through the covariance kernel. The block
    is float32 torch (the step before the path); the covariances are the library's."""
    import torch

    import post_quantization_04_amd as kq  # noqa: F401
    from post_quantization_04_amd import capture as cap, pipeline

    dev = torch.device("cuda:0")
    torch.zeros(1, device=dev)
    shape, n_seq, seq = cap.LLAMA2_7B, 128, 2048
    small = cap.BlockShape(d=512, heads=4, d_ff=1024)
    cap.capture(small, n_seq=2, seq=256, seed=1, device=dev)  # warm the torch kernels
    # weights and block inputs are drawn on the host and resident in HBM before timing
    weights = cap.block_weights(shape, 2026, dev, torch.float32)
    inputs = cap.block_inputs(shape, n_seq, seq, 2026, dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    c = cap.capture(shape, n_seq=n_seq, seq=seq, seed=2026, device=dev, micro_batch=4, weights=weights,
                    inputs=inputs)
    torch.cuda.synchronize()
    t_capture = time.perf_counter() - t0
    tensors = list(c.x.items()) + list(c.g.items())
    flops = sum(t.shape[0] * t.shape[1] * (t.shape[1] + 1) for _, t in tensors)
    hs = {name: torch.empty((t.shape[1], t.shape[1]), dtype=torch.float32, device=dev) for name, t in tensors}
    for name, t in tensors:  # warm-up of the covariance path at these widths
        pipeline.covariance(t[:16384].view(torch.int16), out=hs[name])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for name, t in tensors:
        pipeline.covariance(t.view(torch.int16), out=hs[name])
    torch.cuda.synchronize()
    t_cov = time.perf_counter() - t0
    n = c.tokens
    total = t_capture + t_cov
    log(f"capture: {n} tokens in {t_capture:.2f} s; {len(tensors)} covariances in {t_cov * 1e3:.1f} ms "
        f"({flops / t_cov / 1e12:.0f} TFLOP/s)")
    result = {
        "metric": "calibration capture: tokens/s through one LLaMA-2-7B block (forward + one backward, X and G "
                  "kept) and the covariances of all its linear layers",
        "value": round(n / total, 1), "unit": "tokens/s", "n_gpus": 1, "steps": 1, "warmup": 1,
        "ms_per_step": round(total * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 block / bf16 X, G / f32 H", "data": "synthetic",
        "config": {"workload": "LLaMA-2-7B decoder block (d 4096, 32 heads, d_ff 11008), seeded random weights, "
                               "128 x 2048 seeded token states resident in HBM, micro-batches of 4 sequences",
                   "tokens": n},
        "capture_s": round(t_capture, 3), "covariance_ms": round(t_cov * 1e3, 2),
        "covariance_tflops": round(flops / t_cov / 1e12, 1),
        "covariances": {name: list(t.shape) for name, t in tensors},
    }
    print(json.dumps(result))
    return 0


def decode_bench(args) -> int:
    """Single-token decode through packed W2 layers: y = S_G^-1 U_G^T W^'' U_X S_X^-1 x per layer.

    Synthetic packed codes (uniform random 2-bit fields), group-128 scales and zero points, random
    diagonal scales and seeded rotation specs, for the 224 linear layers of LLaMA-2-7B (32 blocks x
    q, k, v, o, gate, up, down). One step = one token through all 224 layers (the linear layers only:
    no attention, norms or activations); layers that read the same input (q/k/v, gate/up) go through
    one group call, which shares the input side. The roofline covers the matvec kernel inside the
    stack: the average weight bytes (packed codes + scales + zero points) per launch over its average
    duration."""
    import numpy as np
    import torch

    import kq_synth
    import post_quantization_04_amd as kq
    from post_quantization_04_amd import pipeline

    dev = torch.device("cuda:0")
    torch.zeros(1, device=dev)
    bits, group = 2, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(2026)
    rots = {n: pipeline.upload_rot(*(lambda sp: (sp.signs, sp.q))(kq_synth.rot_spec(77, f"dec{n}", n)), dev)
            for n in sorted({d for _, o, i in DECODE_LAYERS for d in (o, i)})}
    # per block and input group: one s_x (the input side's scale comes from the shared H_X), and per
    # layer its packed codes, scales, zero points, s_g and output buffer
    groups = []
    for blk in range(DECODE_BLOCKS):
        for din, members in DECODE_GROUPS:
            s_x = torch.rand(din, dtype=torch.float64, device=dev, generator=gen) + 0.5
            mem = []
            for li in members:
                name, dout, _ = DECODE_LAYERS[li]
                packed = torch.randint(-2 ** 31, 2 ** 31 - 1, (dout, din * 2 // 32), dtype=torch.int32,
                                       device=dev, generator=gen)
                scales = torch.rand((dout, din // group), device=dev, generator=gen) * 0.04 + 0.005
                zeros = torch.randint(0, 4, (dout, din // group), dtype=torch.uint8, device=dev, generator=gen)
                s_g = torch.rand(dout, dtype=torch.float64, device=dev, generator=gen) + 0.5
                y = torch.empty((1, dout), device=dev)
                mem.append((packed, scales, zeros, s_g, rots[dout].rot, y))
            groups.append((din, s_x, mem))
    xs = {n: torch.randn((1, n), device=dev, generator=gen) for n in (4096, 11008)}
    wss = {}
    for din, _, mem in groups:
        key = (din, tuple(m[5].shape[1] for m in mem))
        if key not in wss:
            wss[key] = kq.decode_workspace(sum(key[1]), din, 1, dev)
    n_layers = sum(len(m) for _, _, m in groups)
    weight_bytes = sum(p.numel() * 4 + sc.numel() * 4 + z.numel() for _, _, mem in groups
                       for p, sc, z, _, _, _ in mem)

    def group_call(G):
        din, s_x, mem = G
        ws = wss[(din, tuple(m[5].shape[1] for m in mem))]
        if args.decode_per_layer:
            for packed, scales, zeros, s_g, rot_out, y in mem:
                kq.decode_matvec(packed, scales, zeros, bits, group, s_x, s_g, rots[din].rot, rot_out, xs[din], y,
                                 ws=ws)
        else:
            kq.decode_matvec_group(mem, bits, group, s_x, rots[din].rot, xs[din], ws=ws)

    def token():
        for G in groups:
            group_call(G)

    torch.cuda.synchronize()
    for _ in range(args.warmup + 1):
        token()
    torch.cuda.synchronize()
    # the roofline kernel inside the stack (every layer's weights cold, as in a token): HIP
    # events around each matvec launch, averaged over all 224 launches of a few tokens
    kq.timing_enable("decode_kernel")
    for _ in range(3):
        token()
    n_q, ms_q = kq.timing_query("decode_kernel")
    kq.timing_enable(None)
    q_bytes = weight_bytes * 3 / n_q  # average algorithmic bytes per matvec launch
    q_us = ms_q / n_q * 1e3
    # whole token, eager launches
    steps = max(args.steps, 5) * 4
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        token()
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / steps
    # whole token captured once as a HIP graph and replayed
    outs = [m[5] for _, _, mem in groups for m in mem]
    ref = [y.clone() for y in outs]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        token()  # warm the capture stream
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            token()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replay_ok = all(bool(torch.equal(y, r)) for y, r in zip(outs, ref))
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / steps
    ms_tok = min(ms_eager, ms_graph)
    achieved = q_bytes / (q_us * 1e-6) / 1e9
    result = {
        "metric": "W2 decode: tokens per second through the 224 packed linear layers of LLaMA-2-7B",
        "value": round(1e3 / ms_tok, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms_tok, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u2/f32", "data": "synthetic",
        "config": {"workload": "LLaMA-2-7B linear layers (32 x q, k, v, o 4096x4096; gate, up 11008x4096; "
                               "down 4096x11008), W2 group 128, batch 1, BiIP both sides",
                   "weight_bytes_per_token": weight_bytes,
                   "calls": ("one kq_decode_matvec per layer" if args.decode_per_layer else
                             "one kq_decode_matvec_group per shared input: q/k/v, o, gate/up, down")},
        "ms_per_token_eager": round(ms_eager, 4), "ms_per_token_graph": round(ms_graph, 4),
        "graph_replay_matches_eager": replay_ok,
        "stack_gbs": round(weight_bytes / (ms_tok * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": round(q_bytes), "avg_launch_us": round(q_us, 3),
                     "launches": n_q,
                     "note": "matvec launches of whole tokens (weights cold), averaged over the launches: "
                             "algorithmic bytes = packed codes + float32 scales + uint8 zero points"},
    }
    log(f"decode: {ms_eager:.3f} ms/token eager, {ms_graph:.3f} ms/token graph; matvec launch {q_us:.2f} us "
        f"average in the stack ({achieved:.0f} GB/s)")
    print(json.dumps(result))
    return 0


WORKLOAD_TAG = {1: "linear64x128", 2: "llama2-7b_q_proj", 3: "llama2-13b_mlp", 4: "llama3-70b_down_proj",
                5: "llama3-8b_block"}
TIMED_KERNELS = ("syrk_partial", "chol_far_kernel", "chol_step_kernel", "obs_step_kernel", "row_fwht", "col_fwht",
                 "col_mix")
GPTAQ_KERNELS = ("xcov_partial", "gptaq_drift_kernel", "gptaq_weight_kernel", "gptaq_update_kernel")
PROFILED_STEPS = 2  # instrumented steps that give the per-kernel times


def quant_bench(args) -> int:
    """One step = the whole path over every layer of the workload: covariances of every input group
    and every output gradient, scores and the bit allocation, then BiIP, the Cholesky factor of the
    damped inverse and the column sweep of every layer. Inputs are resident in HBM before timing."""
    import numpy as np
    import torch

    import kq_synth
    import post_quantization_04_amd as kq
    from post_quantization_04_amd import pipeline

    dev = torch.device("cuda:0")
    torch.zeros(1, device=dev)
    cfg = kq_synth.config(args.config)
    single = len(cfg.subs) == 1
    # two streams pay where the factor is latency-bound (its 64-wide steps leave CUs idle next to the
    # G covariance); at 28672 inputs the factor's rank-256 launches fill the GPU and one stream is as fast
    overlap = single and not args.serial and not args.gptaq and (cfg.subs[0].din <= 8192 or args.overlap)
    # created before anything else takes a hardware queue: a CU-masked stream needs its own
    side = side_stream(dev, args.reserve_cus) if overlap else None
    wl = kq_synth.Workload(cfg)
    n_tok = cfg.n_tokens
    log(f"libkq {kq.version()}; generating {cfg.name} inputs")
    t0 = time.perf_counter()
    f32, f64 = torch.float32, torch.float64

    def bits_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    xs = {}
    xts = {}
    for grp in cfg.x_groups:
        xs[grp] = bits_dev(wl.x(grp))
        wl.drop("x", grp)
        if args.gptaq:  # full-precision inputs (gain drift and noise on the same draws)
            xts[grp] = bits_dev(wl.xt(grp))
            wl.drop("xt", grp)
    gs, ws_, rots_in, rots_out = {}, {}, {}, {}
    for s in cfg.subs:
        gs[s.name] = bits_dev(wl.g(s.name))
        wl.drop("g", s.name)
        w = wl.weight(s.name)
        ws_[s.name] = bits_dev(w) if w.dtype == np.uint16 else torch.from_numpy(w).to(dev)
        so = wl.rot_out(s.name)
        rots_out[s.name] = pipeline.upload_rot(so.signs, so.q, dev)
    for grp in cfg.x_groups:
        si = wl.rot_in(grp)
        rots_in[grp] = pipeline.upload_rot(si.signs, si.q, dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM after {time.perf_counter() - t0:.1f} s")

    def scratch(n):
        return torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev)

    widths_all = list(cfg.x_groups.values()) + [s.dout for s in cfg.subs]
    # the covariances and (with --gptaq) the cross moments run one after another on one stream and
    # share one workspace
    cov_bytes = max(kq.workspace_size(kq.KQ_OP_ACCUMULATE_COV, n_tok, d) for d in widths_all)
    if args.gptaq:
        cov_bytes = max([cov_bytes] + [kq.workspace_size(kq.KQ_OP_XCOV, n_tok, d) for d in cfg.x_groups.values()])
    ws_cov = scratch(cov_bytes)
    ws_biip = scratch(max(max(kq.workspace_size(kq.KQ_OP_BIIP, s.dout, s.din),
                              kq.workspace_size(kq.KQ_OP_BIIP, s.din, s.din) if args.gptaq else 0)
                          for s in cfg.subs))
    ws_chol = scratch(max(kq.workspace_size(kq.KQ_OP_CHOLESKY, s.din) for s in cfg.subs))
    ws_obs = scratch(max(kq.workspace_size(kq.KQ_OP_OBS, s.dout, s.din, cfg.block) for s in cfg.subs))
    hx_raw = {grp: torch.empty((d, d), dtype=f32, device=dev) for grp, d in cfg.x_groups.items()}
    if args.gptaq:
        ws_xcov = ws_cov
        ws_gptaq = scratch(max(kq.workspace_size(kq.KQ_OP_GPTAQ, s.dout, s.din) for s in cfg.subs))
        dm = {grp: torch.empty((d, d), dtype=f32, device=dev) for grp, d in cfg.x_groups.items()}
    hg = {s.name: torch.empty((s.dout, s.dout), dtype=f32, device=dev) for s in cfg.subs}
    lay = {}
    for s in cfg.subs:
        ng = s.din // cfg.group if cfg.group else 1
        lay[s.name] = dict(
            hx=torch.empty((s.din, s.din), dtype=f32, device=dev),
            w1=torch.empty((s.dout, s.din), dtype=f64, device=dev),
            w2=torch.empty((s.dout, s.din), dtype=f64, device=dev),
            s_x=torch.empty(s.din, dtype=f64, device=dev), s_g=torch.empty(s.dout, dtype=f64, device=dev),
            s_u=torch.empty(max(s.din, s.dout), dtype=f64, device=dev),
            codes=torch.empty((s.dout, s.din), dtype=torch.uint8, device=dev),
            scales=torch.empty((s.dout, ng), dtype=f32, device=dev),
            zeros=torch.empty((s.dout, ng), dtype=torch.uint8, device=dev),
            info=torch.zeros(1, dtype=torch.int32, device=dev),
            d2=torch.empty((s.din, s.din), dtype=f32, device=dev) if args.gptaq else None)
    score_dev = torch.empty(2 * len(cfg.subs), dtype=f64, device=dev)
    score_host = torch.empty(2 * len(cfg.subs), dtype=f64, pin_memory=True)
    n_params = [s.dout * s.din for s in cfg.subs]
    if cfg.alloc_choices:
        choices, target = list(cfg.alloc_choices), cfg.alloc_target_millibits
    else:  # one width for every layer (the 7B q_proj at --bits): the allocation has one choice
        width = args.bits if cfg.id == 2 else cfg.subs[0].bits
        choices, target = [width], width * 1000
    in_flags, out_flags = kq.KQ_BIIP_INPUT | kq.KQ_BIIP_SCALE, kq.KQ_BIIP_OUTPUT | kq.KQ_BIIP_SCALE
    plan_box = {}

    def allocate(scores):
        return kq.allocate_bits(scores, n_params, choices, target)

    def mark(ev, key, st=None):
        if ev is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record(st if st is not None else torch.cuda.current_stream())
            ev.setdefault(key, []).append(e)

    lead = torch.cuda.Stream(device=dev)  # not the null stream: the CU-masked stream is a blocking stream

    def step_overlap(ev):
        # one layer: the Cholesky factor needs only H_X'' (input side of BiIP), so it runs next to
        # the H_G covariance, which goes to a second stream kept off `reserve` CUs once the input side
        # is done; the output side of BiIP and the sweep follow on the lead stream with every CU. Left
        # and right rotations commute.
        s = cfg.subs[0]
        L = lay[s.name]
        grp = s.x_group
        main = torch.cuda.current_stream()
        mark(ev, "cov_x0", main)
        kq.accumulate_cov(xs[grp], L["hx"], 1.0 / n_tok, 0.0, ws=ws_cov)
        mark(ev, "cov_x1", main)
        mark(ev, "score0", main)
        kq.sensitivity(L["hx"], None, score_dev[0:1], kq.KQ_SCORE_HX_ONLY)  # tr(H_X), raw
        mark(ev, "score1", main)
        mark(ev, "biip0", main)
        kq.biip_rotate(ws_[s.name], L["w1"], L["hx"], None, rots_in[grp].rot, None, in_flags, L["s_x"], L["s_u"],
                       ws=ws_biip)
        mark(ev, "biip1", main)
        # the G covariance starts once the input side (which the factor waits for) is done, so it
        # shares the GPU with the factor instead; it reuses the covariance workspace
        e_in = torch.cuda.Event()
        e_in.record(main)
        with torch.cuda.stream(side):
            side.wait_event(e_in)
            mark(ev, "cov_g0", side)
            kq.accumulate_cov(gs[s.name], hg[s.name], 1.0 / n_tok, 0.0, ws=ws_cov)
            mark(ev, "cov_g1", side)
            e_g = torch.cuda.Event()
            e_g.record(side)
        mark(ev, "chol0", main)
        kq.cholesky_inv(L["hx"], cfg.damp, L["info"], ws=ws_chol)
        mark(ev, "chol1", main)
        main.wait_event(e_g)
        mark(ev, "score0", main)
        kq.sensitivity(hg[s.name], None, score_dev[1:2], kq.KQ_SCORE_HX_ONLY)  # tr(H_G), raw
        mark(ev, "score1", main)
        mark(ev, "biip0", main)
        kq.biip_rotate(L["w1"], L["w2"], None, hg[s.name], None, rots_out[s.name].rot, out_flags, L["s_u"], L["s_g"],
                       ws=ws_biip)
        mark(ev, "biip1", main)
        # the traces reach the host by an asynchronous copy; one layer leaves the allocation one
        # choice, so the sweep is enqueued at that width and the allocation (host, on the float64
        # product tr(H_G) tr(H_X)) runs while the sweep does, and is checked
        score_host[0:2].copy_(score_dev[0:2], non_blocking=True)
        e_sc = torch.cuda.Event()
        e_sc.record(main)
        bits = choices[0]
        mark(ev, "obs0", main)
        kq.obs_quantize(L["w2"], L["hx"], bits, cfg.group, cfg.block, L["codes"], L["scales"], L["zeros"], ws=ws_obs)
        mark(ev, "obs1", main)
        e_sc.synchronize()
        plan_box["plan"] = allocate([float(score_host[0]) * float(score_host[1])])

    def step_serial(ev):
        main = torch.cuda.current_stream()
        for grp in cfg.x_groups:
            mark(ev, "cov_x0", main)
            kq.accumulate_cov(xs[grp], hx_raw[grp], 1.0 / n_tok, 0.0, ws=ws_cov)
            mark(ev, "cov_x1", main)
            if args.gptaq:  # drift moment D = Xt^T X / N - H_X
                mark(ev, "drift0", main)
                kq.accumulate_xcov(xts[grp], xs[grp], dm[grp], 1.0 / n_tok, -1.0, c_in=hx_raw[grp], ws=ws_xcov)
                mark(ev, "drift1", main)
        for s in cfg.subs:
            mark(ev, "cov_g0", main)
            kq.accumulate_cov(gs[s.name], hg[s.name], 1.0 / n_tok, 0.0, ws=ws_cov)
            mark(ev, "cov_g1", main)
        mark(ev, "score0", main)
        for i, s in enumerate(cfg.subs):
            kq.sensitivity(hx_raw[s.x_group], hg[s.name], score_dev[i:i + 1], kq.KQ_SCORE_KRONQ)
        score_host[:len(cfg.subs)].copy_(score_dev[:len(cfg.subs)], non_blocking=True)
        main.synchronize()  # the widths of the sweeps depend on the scores
        plan = allocate([float(v) for v in score_host[:len(cfg.subs)]])
        plan_box["plan"] = plan
        mark(ev, "score1", main)
        for i, s in enumerate(cfg.subs):
            L = lay[s.name]
            L["hx"].copy_(hx_raw[s.x_group])  # the factor works in place; the raw H_X serves every layer
            mark(ev, "biip0", main)
            kq.biip_rotate(ws_[s.name], L["w2"], L["hx"], hg[s.name], rots_in[s.x_group].rot, rots_out[s.name].rot,
                           pipeline.ALL_SIDES, L["s_x"], L["s_g"], ws=ws_biip)
            mark(ev, "biip1", main)
            if args.gptaq:
                mark(ev, "gptaq0", main)
                L["d2"].copy_(dm[s.x_group])
                kq.biip_transform(L["d2"], rots_in[s.x_group].rot, L["s_x"], ws=ws_biip)
                mark(ev, "gptaq1", main)
            mark(ev, "chol0", main)
            kq.cholesky_inv(L["hx"], cfg.damp, L["info"], ws=ws_chol)
            mark(ev, "chol1", main)
            if args.gptaq:
                mark(ev, "gptaq0", main)
                kq.gptaq_target(L["w2"], L["d2"], L["hx"], ws=ws_gptaq)
                mark(ev, "gptaq1", main)
            mark(ev, "obs0", main)
            kq.obs_quantize(L["w2"], L["hx"], plan[i], cfg.group, cfg.block, L["codes"], L["scales"], L["zeros"],
                            ws=ws_obs)
            mark(ev, "obs1", main)

    def step(ev=None):
        with torch.cuda.stream(lead):
            (step_overlap if overlap else step_serial)(ev)

    torch.cuda.synchronize()
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    bad = {s.name: int(lay[s.name]["info"].item()) for s in cfg.subs if int(lay[s.name]["info"].item())}
    if bad:
        raise RuntimeError(f"Cholesky factor reported info {bad}")

    # Per-kernel times come from instrumented steps before the timed region, every timed kernel's
    # launches bracketed by HIP events (events around the factor's 560 launches cost about 1 % of a
    # 70B step); the timed steps bracket only the launches of the kernel that dominates the step,
    # which the roofline reports.
    timed = TIMED_KERNELS + (GPTAQ_KERNELS if args.gptaq else ())
    candidates = ("syrk_partial", "chol_far_kernel", "chol_step_kernel", "obs_step_kernel") + (
        GPTAQ_KERNELS if args.gptaq else ())
    log(f"{PROFILED_STEPS} instrumented steps (every timed kernel)")
    kq.timing_enable("|".join(timed))
    for _ in range(PROFILED_STEPS):
        step()
    torch.cuda.synchronize()
    kp = {k: kq.timing_query(k) for k in timed}
    kq.timing_enable(None)
    dominant = max(candidates, key=lambda k: kp[k][1])

    log(f"timing {args.steps} steps ({dominant} launches bracketed)")
    evs = [dict() for _ in range(args.steps)]
    kq.timing_enable(dominant)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_l, ms_l = kq.timing_query(dominant)
    kq.timing_enable(None)
    release_streams()
    plan = plan_box["plan"]

    ms_step = wall * 1e3 / args.steps
    def span(stage):
        tot = 0.0
        for ev in evs:
            for a, b in zip(ev.get(stage + "0", []), ev.get(stage + "1", [])):
                tot += a.elapsed_time(b)
        return tot / args.steps
    stage_ms = {"cov_x": span("cov_x"), "cov_g": span("cov_g"), "score_alloc": span("score"), "biip": span("biip"),
                "cholesky": span("chol"), "obs": span("obs")}
    if args.gptaq:
        stage_ms["drift_moment"] = span("drift")
        stage_ms["gptaq_correction"] = span("gptaq")
    weights = sum(n_params)
    # algorithmic work per step
    cov_flops = sum(n_tok * d * (d + 1) for d in cfg.x_groups.values()) + sum(n_tok * s.dout * (s.dout + 1)
                                                                             for s in cfg.subs)
    chol_flops = sum(2 * s.din ** 3 / 3 for s in cfg.subs)
    obs_flops = sum(s.dout * s.din * (s.din - 1) for s in cfg.subs)
    biip_bytes = sum(s.dout * s.din * ((2 if cfg.w_dtype == "bf16" else 4) + 8) + 8 * s.din ** 2 + 8 * s.dout ** 2
                     for s in cfg.subs)
    far_flops = sum(chol_far_flops(s.din) for s in cfg.subs)
    work = {"syrk_partial": cov_flops, "chol_far_kernel": far_flops, "chol_step_kernel": chol_flops - far_flops,
            "obs_step_kernel": obs_flops}
    if args.gptaq:
        # cross moment: every entry of the square; the correction's three products skip their triangles
        work["xcov_partial"] = sum(2 * n_tok * d * d for d in cfg.x_groups.values())
        work["gptaq_drift_kernel"] = sum(s.din ** 3 / 3 for s in cfg.subs)
        work["gptaq_weight_kernel"] = sum(s.dout * s.din ** 2 for s in cfg.subs)
        work["gptaq_update_kernel"] = sum(s.dout * s.din ** 2 for s in cfg.subs)
    t_accum = (stage_ms["cov_x"] + stage_ms["cov_g"]) / 1e3
    t_quant = sum(stage_ms[k] for k in ("score_alloc", "biip", "cholesky", "obs", "gptaq_correction")
                  if k in stage_ms) / 1e3
    value = weights / (ms_step / 1e3) / 1e6
    log(f"{ms_step:.2f} ms/step; stages {json.dumps({k: round(v, 3) for k, v in stage_ms.items()})}")
    for k, (n, ms) in kp.items():
        if n:
            log(f"  {k}: {n // PROFILED_STEPS} launches, {ms / PROFILED_STEPS:.3f} ms per step (instrumented steps)")
    log(f"  {dominant} in the timed steps: {n_l} launches, {ms_l / args.steps:.3f} ms per step")
    src, peak, unit, bound = KERNELS[dominant]
    achieved = work[dominant] * args.steps / (ms_l / 1e3) / 1e12
    tag = WORKLOAD_TAG[cfg.id]
    result = {
        "metric": "layer quantize throughput (Mweights/s) + H_X/H_G accumulate TFLOP/s",
        "value": round(value, 3),
        "unit": "Mweights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/f32/f64",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: " + ", ".join(f"{s.name} {s.dout}x{s.din}" for s in cfg.subs) +
                         f" ({cfg.w_dtype}); {n_tok} tokens of X and G (bf16); group {cfg.group}, block {cfg.block}, "
                         f"damp {cfg.damp}, BiIP both sides" +
                         (", GPTAQ base quantizer (drift moment of full-precision inputs Xt of the same shape, "
                          "drift correction of W'' before the sweep)" if args.gptaq else "")),
            "bits": dict(zip([s.name for s in cfg.subs], plan)),
            "tokens": n_tok,
            "weights": weights,
        },
        "accumulate_tflops": round(cov_flops / t_accum / 1e12, 2) if t_accum > 0 else None,
        "quantize_mweights_per_s": round(weights / t_quant / 1e6, 2) if t_quant > 0 else None,
        "seconds_per_step": round(ms_step / 1e3, 5),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "kernel_ms_per_step": {k: round(ms / PROFILED_STEPS, 4) for k, (n, ms) in kp.items() if n},
        "kernel_ms_source": (f"{PROFILED_STEPS} instrumented steps before the timed region (HIP events around "
                             f"every launch of these kernels); the timed steps bracket {dominant} only"),
        "roofline": {
            "kernel": dominant,
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": stored_traffic(dominant, tag),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_flops_per_launch": round(work[dominant] * args.steps / max(n_l, 1)),
            "launches": n_l,
            "avg_launch_ms": round(ms_l / max(n_l, 1), 4),
            "note": (f"the kernel with the most time in the step; algorithmic flops "
                     + {"syrk_partial": "N d (d + 1) per covariance",
                        "chol_far_kernel": "of the rank-256 updates after each 256-column super-panel (lower "
                                           "triangle of the trailing matrix and the substitution sums over the "
                                           "nonzero part of L^-1), float32 MFMA",
                        "chol_step_kernel": "2 d^3 / 3 per factor less the far launches' share, float32 MFMA",
                        "obs_step_kernel": "dout din (din - 1) per layer (in-block sweep and lazy-batch updates)",
                        "xcov_partial": "2 N d^2 per cross moment (every entry of the square)",
                        "gptaq_drift_kernel": "din^3 / 3 per layer (the strict upper triangle of D R^T), float64 MFMA",
                        "gptaq_weight_kernel": "dout din^2 per layer (W times the strictly upper Y), float64 MFMA",
                        "gptaq_update_kernel": "dout din^2 per layer (Z times the upper R), float64 MFMA"}[dominant]
                     + "; launch durations from HIP events the library records on each launch's stream"),
        },
        "cpu_baseline": None,
    }

    def roof(bound, amount, ms, peak, unit, scale, note):
        ach = amount / (ms / 1e3) / scale if ms > 0 else 0.0
        return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                "ms": round(ms, 4), "note": note}

    kms = {k: ms / PROFILED_STEPS for k, (n, ms) in kp.items()}
    result["step_rooflines"] = {
        "covariance": roof("mfma", cov_flops, kms["syrk_partial"], 2500.0, "TFLOP/s", 1e12,
                           "syrk_partial launches: N d (d + 1) flop per covariance"),
        "biip": roof("hbm", biip_bytes, stage_ms["biip"], HBM_PEAK_GBS, "GB/s", 1e9,
                     "whole BiIP stage: W read, float64 W'' write, H_X and H_G float32 read and write"),
        "cholesky": roof("mfma", chol_flops, kms["chol_step_kernel"] + kms["chol_far_kernel"], 157.3, "TFLOP/s",
                         1e12, "chol_step_kernel and chol_far_kernel launches: 2 d^3 / 3 flop per factor, against "
                               "the float32 roof"),
        "obs": roof("mfma", obs_flops, kms["obs_step_kernel"], 78.6, "TFLOP/s", 1e12,
                    "obs_step_kernel launches: dout din (din - 1) flop per layer, against the float64 roof"),
    }
    if args.gptaq:
        g_flops = work["gptaq_drift_kernel"] + work["gptaq_weight_kernel"] + work["gptaq_update_kernel"]
        result["step_rooflines"]["drift_moment"] = roof(
            "mfma", work["xcov_partial"], kms["xcov_partial"], 2500.0, "TFLOP/s", 1e12,
            "xcov_partial launches: 2 N d^2 flop per cross moment (every entry of the square)")
        result["step_rooflines"]["gptaq_correction"] = roof(
            "mfma", g_flops, kms["gptaq_drift_kernel"] + kms["gptaq_weight_kernel"] + kms["gptaq_update_kernel"],
            78.6, "TFLOP/s", 1e12, "the three float64 products: din^3 / 3 + 2 dout din^2 flop per layer")
    result["schedule"] = ("two streams: H_X covariance, BiIP input side, Cholesky factor, BiIP output side and "
                          f"sweep on one; H_G covariance on the other from the end of the input side, kept off "
                          f"{args.reserve_cus} CUs" if overlap else
                          "one stream: every covariance, the scores and the allocation, then per layer BiIP, "
                          "Cholesky factor and sweep")
    if args.copy_calibration:
        src_t = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst_t = torch.empty_like(src_t)
        src_t.fill_(1)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t
    if not args.no_cpu_baseline and not args.gptaq:  # the timed oracle sample models the GPTQ path
        log("timing the float64 oracle on a bounded sample")
        del xs, gs
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(wl, cfg, plan)
    print(json.dumps(result), flush=True)
    return 0


PEAK_PROBES = [  # (kind, name, published dense peak TFLOP/s, wave-rounds per launch)
    (0, "bf16 MFMA, random operands", 2500.0, 60000),
    (1, "bf16 MFMA, constant operands", 2500.0, 60000),
    (2, "float32 MFMA, random operands", 157.3, 30000),
    (3, "float32 MFMA, constant operands", 157.3, 30000),
    (4, "float64 MFMA, random operands", 78.6, 30000),
    (5, "float64 MFMA, constant operands", 78.6, 30000),
]


def peaks_bench(args) -> int:
    """Sustained MFMA rates (each probe launched `warmup` + `steps` times, ~50 ms per launch; the
    median of the timed launches) and a 4 GiB device-to-device copy, one JSON line."""
    import ctypes
    import statistics
    import torch
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "post_quantization_04_amd", "libkq_peaks.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m post_quantization_04_amd.build)")
    lib = ctypes.CDLL(path)
    lib.kqp_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.kqp_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.kqp_flops_per_round.restype = ctypes.c_double
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    blocks = lib.kqp_mfma_blocks()
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(4, dtype=torch.int64, device=dev)
    probes = {}
    for kind, name, peak, iters in PEAK_PROBES:
        runs = []
        for rep in range(args.warmup + args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            if lib.kqp_mfma(kind, iters, out.data_ptr(), clk.data_ptr(), ctypes.c_void_p(st.cuda_stream)) != 0:
                raise RuntimeError(f"probe {name} failed to launch")
            e1.record(st)
            e1.synchronize()
            if rep < args.warmup:
                continue
            ms = e0.elapsed_time(e1)
            c = clk.tolist()
            mhz = 100.0 * (c[2] - c[0]) / (c[3] - c[1]) if c[3] > c[1] else None
            flops = lib.kqp_flops_per_round(kind) * iters * blocks * 4
            runs.append((flops / ms / 1e9, mhz, ms))
        tf = statistics.median(r[0] for r in runs)
        mhz = statistics.median(r[1] for r in runs if r[1] is not None)
        probes[name] = {"tflops": round(tf, 1), "frac_of_published": round(tf / peak, 3),
                        "shader_clock_mhz": round(mhz), "ms_per_launch": round(statistics.median(r[2] for r in runs), 2)}
        log(f"{name}: {tf:.1f} TFLOP/s ({tf / peak:.1%} of {peak}), {mhz:.0f} MHz")
    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    copies = []
    for rep in range(args.warmup + args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        if lib.kqp_copy(src.data_ptr(), dst.data_ptr(), nbytes, ctypes.c_void_p(st.cuda_stream)) != 0:
            raise RuntimeError("copy probe failed to launch")
        e1.record(st)
        e1.synchronize()
        if rep >= args.warmup:
            copies.append(2 * nbytes / e0.elapsed_time(e1) / 1e6)
    if not torch.equal(src, dst):
        raise RuntimeError("copy probe: destination differs from source")
    gbs = statistics.median(copies)
    log(f"copy: {gbs:.0f} GB/s read + write ({gbs / HBM_PEAK_GBS:.1%} of {HBM_PEAK_GBS:.0f})")
    runtime = []
    for rep in range(args.warmup + args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        dst.copy_(src)
        e1.record(st)
        e1.synchronize()
        if rep >= args.warmup:
            runtime.append(2 * nbytes / e0.elapsed_time(e1) / 1e6)
    rt = statistics.median(runtime)
    log(f"runtime device copy (torch copy_): {rt:.0f} GB/s read + write")
    print(json.dumps({"metric": "peak_probes", "device": torch.cuda.get_device_name(dev),
                      "launches_timed": args.steps, "mfma": probes,
                      "copy": {"gb_per_s": round(gbs, 1), "bytes_per_launch": 2 * nbytes,
                               "frac_of_published": round(gbs / HBM_PEAK_GBS, 3)},
                      "runtime_copy": {"gb_per_s": round(rt, 1), "bytes_per_launch": 2 * nbytes,
                                       "frac_of_published": round(rt / HBM_PEAK_GBS, 3)}}), flush=True)
    return 0


def main() -> int:
    args = parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; sharding the path over several GPUs is "
                                   "described, not implemented, so --gpus must be 1"}))
        return 2
    if args.decode:
        return decode_bench(args)
    if args.peaks:
        return peaks_bench(args)
    if args.capture:
        return capture_bench(args)
    return quant_bench(args)


if __name__ == "__main__":
    sys.exit(main())
