#!/usr/bin/env python3
"""Throughput of the KronQ per-layer quantization path on one MI355X.

One step is one pass of the whole path over one layer whose inputs are
already resident in HBM:
  1. H_X = X^T X / N and H_G = G^T G / N (bf16-MFMA symmetric rank-k updates
     over all N tokens),
  2. the trace score tr(H_G) tr(H_X) and the bit allocation from it,
  3. BiIP (diagonal rescale + randomised Hadamard rotation on both sides of W,
     with H_X and H_G transformed alongside),
  4. the damped Cholesky factor of H_X''^-1,
  5. the column-wise OBS sweep with its lazy-batch trailing products.
Workload: LLaMA-2-7B q_proj shapes (W 4096 x 4096 bf16; X and G 262144 x 4096
bf16, 128 sequences of 2048 tokens), 2-bit, group 128, block 128, damping
0.01, seeded synthetic inputs.

Schedule: the Cholesky factor needs only H_X'' (the input side of BiIP), so
by default it runs on one stream while the H_G covariance runs on a second
stream that is kept off some CUs, which stay free for the latency-bound factor
steps; the output side of BiIP and the sweep follow on the first stream with
every CU. `--serial` puts every stage on one stream.

value = weights quantised per second, end to end including the covariance
accumulation. The roofline object covers the dominant kernel, the bf16 MFMA
SYRK (syrk_partial): algorithmic flops N d (d + 1) per covariance over the
summed durations of its launches, timed with HIP events that the library
records around each launch on its stream. The CPU baseline is the float64
oracle timed on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3   # MI355X float32 (vector and matrix)
FP64_PEAK_TFLOPS = 78.6    # MI355X float64 MFMA


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--bits", type=int, default=2, choices=(2, 4))
    p.add_argument("--serial", action="store_true",
                   help="run every stage on one stream (per-stage profiles) instead of the two-stream schedule")
    p.add_argument("--reserve-cus", type=int, default=80,
                   help="CUs the second stream leaves to the Cholesky factor (0: no CU mask)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the timed oracle sample")
    p.add_argument("--cpu-tokens", type=int, default=16384, help="tokens in the oracle's covariance sample")
    p.add_argument("--cpu-rows", type=int, default=64, help="weight rows in the oracle's sweep sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after timing, copy 1 GiB device-to-device (a reference kernel for HBM byte counters)")
    p.add_argument("--decode", action="store_true",
                   help="instead of the quantization step: the packed-code decode matvec (one JSON line)")
    p.add_argument("--capture", action="store_true",
                   help="calibration capture of one LLaMA-2-7B block (forward + one backward) and its covariances")
    p.add_argument("--decode-per-layer", action="store_true",
                   help="with --decode: one kq_decode_matvec call per layer instead of one group call per shared input")
    p.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_JSON"),
                   help="no run: turn two rocprofv3 --pmc runs of '--copy-calibration' (FETCH_SIZE, then "
                        "WRITE_SIZE) into the per-launch HBM bytes of the roofline kernel")
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


def cpu_baseline(wl, cfg, sub, bits, tokens, rows):
    """The float64 oracle on a bounded sample, scaled to one full layer."""
    import numpy as np
    import oracle

    n_tok = cfg.n_tokens
    t0 = time.perf_counter()
    hx = oracle.covariance([wl.x("attn_in")[:tokens]])
    hg = oracle.covariance([wl.g(sub.name)[:tokens]])
    t_cov = (time.perf_counter() - t0) * (n_tok / tokens)
    t0 = time.perf_counter()
    s = oracle.sensitivity(hx, hg)
    oracle.allocate_bits([s], [sub.dout * sub.din], [bits], bits * 1000)
    t_score = time.perf_counter() - t0
    t0 = time.perf_counter()
    w2, hx2, _, _, _ = oracle.biip_forward(wl.weight_f64(sub.name), hx, hg, wl.rot_in("attn_in"),
                                           wl.rot_out(sub.name))
    t_biip = time.perf_counter() - t0
    t0 = time.perf_counter()
    r = oracle.chol_inv_upper(hx2, cfg.damp)
    t_chol = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.obs_quantize(w2[:rows], r, bits, cfg.group)
    t_obs = (time.perf_counter() - t0) * (sub.dout / rows)
    total = t_cov + t_score + t_biip + t_chol + t_obs
    return {
        "value": round(sub.dout * sub.din / total / 1e6, 4),
        "unit": "Mweights/s",
        "cores": cpu_threads(),
        "kind": "oracle",
        "sample": (f"float64 oracle: covariances over {tokens} of {n_tok} tokens (x{n_tok / tokens:g}), "
                   f"OBS sweep on {rows} of {sub.dout} rows (x{sub.dout / rows:g}), BiIP, Cholesky and score "
                   f"at full size; seconds per layer {total:.1f}"),
        "seconds_per_layer": round(total, 2),
    }


ROOT = os.path.dirname(os.path.abspath(__file__))
ROOFLINE_KERNEL = "syrk_partial"
ROOFLINE_SOURCE = os.path.join(ROOT, "post_quantization_04_amd", "csrc", "syrk.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "syrk_partial_llama2-7b_q_proj_hbm_traffic.json")
COPY_BYTES = 1 << 30


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


def traffic_summary(fetch_dir: str, write_dir: str, out_json: str) -> int:
    """HBM bytes per launch of the roofline kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for the final 1 GiB device-to-device copy."""
    out = {"kernel": ROOFLINE_KERNEL, "source": os.path.relpath(ROOFLINE_SOURCE, ROOT),
           "source_sha256": source_hash(ROOFLINE_SOURCE), "copy_bytes": COPY_BYTES}
    for key, run_dir, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = pmc_dispatches(run_dir, counter)
        copy = rows[-1]  # the calibration copy is the last dispatch of the run
        if "syrk" in copy[1] or copy[2] <= 0:
            raise RuntimeError(f"{counter}: last dispatch {copy[1]!r} is not the calibration copy")
        mine = [v for _, n, v in rows if f"::{ROOFLINE_KERNEL}(" in n or n.startswith(f"{ROOFLINE_KERNEL}(")]
        if not mine:
            raise RuntimeError(f"{counter}: no {ROOFLINE_KERNEL} dispatch")
        scale = COPY_BYTES / (copy[2] * 1024.0)
        out[f"{key}_kib_per_launch"] = sum(mine) / len(mine)
        out[f"{key}_launches"] = len(mine)
        out[f"copy_{key}_kib"] = copy[2]
        out[f"{key}_scale"] = scale
        out[f"{key}_bytes_per_launch"] = out[f"{key}_kib_per_launch"] * 1024.0 * scale
    out["traffic_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


def stored_traffic():
    """Per-launch HBM bytes of the roofline kernel from the committed counter summary, or None when the
    summary is missing or was taken on a different version of the kernel's source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if rec.get("source_sha256") != source_hash(ROOFLINE_SOURCE):
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
HBM_PEAK_GBS = 8000.0


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


def main() -> int:
    args = parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU; the path's multi-GPU sharding is design only, "
                                   "so --gpus must be 1"}))
        return 2
    if args.decode:
        return decode_bench(args)
    if args.capture:
        return capture_bench(args)

    import numpy as np
    import torch

    import kq_synth
    import post_quantization_04_amd as kq
    from post_quantization_04_amd import pipeline

    dev = torch.device("cuda:0")
    torch.zeros(1, device=dev)
    # created before anything else takes a hardware queue: a CU-masked stream needs its own
    side = None if args.serial else side_stream(dev, args.reserve_cus)
    cfg = kq_synth.config(2)
    sub = cfg.subs[0]
    dout, din, n_tok = sub.dout, sub.din, cfg.n_tokens
    wl = kq_synth.Workload(cfg)

    log(f"libkq {kq.version()}; generating {cfg.name} inputs")
    t0 = time.perf_counter()
    x = wl.x("attn_in")
    g = wl.g(sub.name)
    w = wl.weight(sub.name)
    si, so = wl.rot_in("attn_in"), wl.rot_out(sub.name)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    gd = torch.from_numpy(g.view(np.int16)).to(dev)
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    ri, ro = pipeline.upload_rot(si.signs, si.q, dev), pipeline.upload_rot(so.signs, so.q, dev)

    f32, f64 = torch.float32, torch.float64
    hx = torch.empty((din, din), dtype=f32, device=dev)
    hg = torch.empty((dout, dout), dtype=f32, device=dev)
    score = torch.empty(1, dtype=f64, device=dev)
    w2 = torch.empty((dout, din), dtype=f64, device=dev)
    s_x = torch.empty(din, dtype=f64, device=dev)
    s_g = torch.empty(dout, dtype=f64, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    codes = torch.empty((dout, din), dtype=torch.uint8, device=dev)
    ng = din // cfg.group
    scales = torch.empty((dout, ng), dtype=f32, device=dev)
    zeros = torch.empty((dout, ng), dtype=torch.uint8, device=dev)

    def scratch(n):
        return torch.empty(max(int(n), 1), dtype=torch.uint8, device=dev)

    ws_cov = scratch(max(kq.workspace_size(kq.KQ_OP_ACCUMULATE_COV, n_tok, din),
                         kq.workspace_size(kq.KQ_OP_ACCUMULATE_COV, n_tok, dout)))
    ws_biip = scratch(kq.workspace_size(kq.KQ_OP_BIIP, dout, din))
    ws_chol = scratch(kq.workspace_size(kq.KQ_OP_CHOLESKY, din))
    ws_obs = scratch(kq.workspace_size(kq.KQ_OP_OBS, dout, din, cfg.block))
    flags = pipeline.ALL_SIDES
    stages = ["cov_x", "cov_g", "score_alloc", "biip", "cholesky", "obs"]
    # two-stream schedule: the Cholesky factor needs only H_X'' (input side), so it runs next
    # to the G covariance; the output side of BiIP follows on the second stream
    w1 = torch.empty((dout, din), dtype=f64, device=dev)
    score_x = torch.empty(1, dtype=f64, device=dev)
    score_g = torch.empty(1, dtype=f64, device=dev)
    score_host = torch.empty(2, dtype=f64, pin_memory=True)
    s_unused_x = torch.empty(din, dtype=f64, device=dev)
    s_unused_g = torch.empty(dout, dtype=f64, device=dev)
    in_flags = kq.KQ_BIIP_INPUT | kq.KQ_BIIP_SCALE
    out_flags = kq.KQ_BIIP_OUTPUT | kq.KQ_BIIP_SCALE

    def step_serial(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        kq.accumulate_cov(xd, hx, 1.0 / n_tok, 0.0, ws=ws_cov)
        mark(1)
        kq.accumulate_cov(gd, hg, 1.0 / n_tok, 0.0, ws=ws_cov)
        mark(2)
        kq.sensitivity(hx, hg, score)
        bits = kq.allocate_bits([float(score.item())], [dout * din], [args.bits], args.bits * 1000)[0]
        mark(3)
        kq.biip_rotate(wd, w2, hx, hg, ri.rot, ro.rot, flags, s_x, s_g, ws=ws_biip)
        mark(4)
        kq.cholesky_inv(hx, cfg.damp, info, ws=ws_chol)
        mark(5)
        kq.obs_quantize(w2, hx, bits, cfg.group, cfg.block, codes, scales, zeros, ws=ws_obs)
        mark(6)

    # the lead stream is not the null stream: the CU-masked side stream is a blocking stream,
    # which the null stream would wait for
    lead = torch.cuda.Stream(device=dev)

    def step_overlap(ev=None):
        with torch.cuda.stream(lead):
            overlap_body(ev)

    def overlap_body(ev):
        # ev: events 0..6 and 9..11 on the lead stream, 7..8 on the side stream
        main = torch.cuda.current_stream()
        def mark(i, st):
            if ev is not None:
                ev[i].record(st)
        mark(0, main)
        kq.accumulate_cov(xd, hx, 1.0 / n_tok, 0.0, ws=ws_cov)
        e_cov = torch.cuda.Event()
        e_cov.record(main)  # the G covariance reuses this workspace
        mark(1, main)
        with torch.cuda.stream(side):
            side.wait_event(e_cov)
            mark(7, side)
            kq.accumulate_cov(gd, hg, 1.0 / n_tok, 0.0, ws=ws_cov)
            mark(8, side)
            e_g = torch.cuda.Event()
            e_g.record(side)
        kq.sensitivity(hx, None, score_x, kq.KQ_SCORE_HX_ONLY)  # tr(H_X) of the raw covariance
        mark(2, main)
        kq.biip_rotate(wd, w1, hx, None, ri.rot, None, in_flags, s_x, s_unused_g, ws=ws_biip)
        mark(3, main)
        kq.cholesky_inv(hx, cfg.damp, info, ws=ws_chol)
        mark(4, main)
        # the rest runs on the lead stream, which has every CU
        main.wait_event(e_g)
        mark(9, main)
        kq.sensitivity(hg, None, score_g, kq.KQ_SCORE_HX_ONLY)  # tr(H_G) of the raw covariance
        mark(10, main)
        kq.biip_rotate(w1, w2, None, hg, None, ro.rot, out_flags, s_unused_x, s_g, ws=ws_biip)
        mark(11, main)
        # The traces go to the host without stopping the stream. One layer at one bit width leaves
        # the allocation no choice, so the sweep is enqueued at that width and the allocation (a host
        # routine, on score = tr(H_G) tr(H_X), the float64 product the combined call forms) runs
        # while the sweep does, and is checked.
        score_host[0:1].copy_(score_x, non_blocking=True)
        score_host[1:2].copy_(score_g, non_blocking=True)
        e_sc = torch.cuda.Event()
        e_sc.record(main)
        mark(5, main)
        kq.obs_quantize(w2, hx, args.bits, cfg.group, cfg.block, codes, scales, zeros, ws=ws_obs)
        mark(6, main)
        e_sc.synchronize()
        sc = float(score_host[0]) * float(score_host[1])
        bits = kq.allocate_bits([sc], [dout * din], [args.bits], args.bits * 1000)[0]
        if bits != args.bits:
            raise RuntimeError(f"allocation gave {bits} bits for the one layer, expected {args.bits}")

    step = step_serial if args.serial else step_overlap

    torch.cuda.synchronize()  # inputs were uploaded on the null stream
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(info.item()) != 0:
        raise RuntimeError(f"Cholesky reported info = {int(info.item())}")

    log(f"timing {args.steps} steps")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(12)] for _ in range(args.steps)]
    kq.timing_enable("syrk_partial")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launches, syrk_ms = kq.timing_query("syrk_partial")
    kq.timing_enable(None)
    unshared = None
    if not args.serial:
        # the same kernel with the GPU to itself (the H_X launch of the schedule), three launches
        kq.timing_enable("syrk_partial")
        for _ in range(3):
            kq.accumulate_cov(xd, hx, 1.0 / n_tok, 0.0, ws=ws_cov)
        torch.cuda.synchronize()
        n_u, ms_u = kq.timing_query("syrk_partial")
        kq.timing_enable(None)
        unshared = ms_u / max(n_u, 1)
    release_streams()

    ms_step = wall * 1e3 / args.steps
    def span(a, b):
        return sum(ev[a].elapsed_time(ev[b]) for ev in events) / args.steps
    if args.serial:
        stage_ms = {s: span(i, i + 1) for i, s in enumerate(stages)}
    else:
        # per-stage durations on the stream each ran on; cov_g overlaps the BiIP input side
        # and the Cholesky factor, so the stages add up to more than the step
        stage_ms = {"cov_x": span(0, 1), "cov_g": span(7, 8), "score_alloc": span(1, 2) + span(9, 10),
                    "biip": span(2, 3) + span(10, 11), "cholesky": span(3, 4), "obs": span(5, 6)}
    flops_cov = n_tok * din * (din + 1) + n_tok * dout * (dout + 1)
    t_accum = (stage_ms["cov_x"] + stage_ms["cov_g"]) / 1e3
    t_quant = sum(stage_ms[s] for s in ("score_alloc", "biip", "cholesky", "obs")) / 1e3
    syrk_tflops = flops_cov * args.steps / (syrk_ms / 1e3) / 1e12 if syrk_ms > 0 else 0.0
    value = dout * din / (ms_step / 1e3) / 1e6
    log(f"{ms_step:.2f} ms/step; stages {json.dumps({k: round(v, 3) for k, v in stage_ms.items()})}")
    log(f"syrk_partial: {launches} launches, {syrk_ms / max(launches, 1):.3f} ms avg, {syrk_tflops:.1f} TFLOP/s")

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
            "workload": (f"{cfg.name}: W {dout}x{din} bf16, X and G {n_tok}x{din} bf16, W{args.bits} "
                         f"group {cfg.group} block {cfg.block} damp {cfg.damp}, BiIP both sides"),
            "bits": args.bits,
            "tokens": n_tok,
            "weights": dout * din,
        },
        "accumulate_tflops": round(flops_cov / t_accum / 1e12, 2),
        "quantize_mweights_per_s": round(dout * din / t_quant / 1e6, 2),
        "seconds_per_layer": round(ms_step / 1e3, 5),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": {
            "kernel": "syrk_partial",
            "bound": "mfma",
            "achieved": round(syrk_tflops, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(syrk_tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": stored_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": 2 * n_tok * din + 4 * din * din,
            "launches": launches,
            "avg_launch_ms": round(syrk_ms / max(launches, 1), 4),
            "note": ("average over every launch of the timed region: the H_G launches run on the CU-masked "
                     "second stream next to the Cholesky factor" if not args.serial else "one stream"),
        },
        "cpu_baseline": None,
    }
    # every step's fraction of its own roof (the dominant kernel's is `roofline` above)
    biip_bytes = dout * din * (2 + 8) + 8 * din * din + 8 * dout * dout  # W bf16 in, float64 out; H in place
    obs_flops = dout * din * (din - cfg.block)  # lazy-batch trailing products over all blocks
    chol_flops = 2 * din ** 3 / 3              # factor and triangular inverse
    def step_roof(bound, amount, ms, peak, unit, scale, note):
        ach = amount / (ms / 1e3) / scale if ms > 0 else 0.0
        return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "ms": round(ms, 4), "note": note}
    result["step_rooflines"] = {
        "biip": step_roof("hbm", biip_bytes, stage_ms["biip"], HBM_PEAK_GBS, "GB/s", 1e9,
                          f"{biip_bytes} algorithmic bytes (W bf16 read, float64 W'' write, H_X and H_G float32 "
                          f"read and write); the input side runs next to the H_G covariance"),
        "obs_trailing": step_roof("mfma", obs_flops, stage_ms["obs"], FP64_PEAK_TFLOPS, "TFLOP/s", 1e12,
                                  f"dout din (din - B) = {obs_flops} flop of float64 trailing products over the "
                                  f"whole sweep time (the in-block sweep included)"),
        **({} if args.serial else {"biip_output_side": step_roof(
            "hbm", dout * din * 16 + 8 * dout * dout, span(10, 11), HBM_PEAK_GBS, "GB/s", 1e9,
            "output side alone, with the GPU to itself: float64 W read and write, H_G float32 read and write "
            "(three passes over each matrix, so about three times these bytes move)")}),
        "cholesky": step_roof("mfma", chol_flops, stage_ms["cholesky"], FP32_PEAK_TFLOPS, "TFLOP/s", 1e12,
                              "2 d^3 / 3 flop (factor and inverse) against the float32 roof; runs on the 80 CUs "
                              "left to it next to the H_G covariance" if not args.serial else
                              "2 d^3 / 3 flop (factor and inverse) against the float32 roof"),
    }
    result["schedule"] = ("one stream" if args.serial else
                          f"two streams: H_X covariance, BiIP input side, Cholesky factor, BiIP output side and "
                          f"sweep on one; H_G covariance on the other, kept off {args.reserve_cus} CUs")
    if unshared is not None:
        ach = flops_cov / 2 / (unshared / 1e3) / 1e12 if unshared > 0 else 0.0
        result["roofline"]["unshared"] = {"avg_launch_ms": round(unshared, 4), "achieved": round(ach, 2),
                                          "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                                          "note": "3 launches on the H_X input after the timed region, GPU to itself"}
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl, cfg, sub, args.bits, args.cpu_tokens, args.cpu_rows)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
