"""Seeded synthetic inputs for the KronQ per-layer quantization path.

This module is shared by the CPU oracle and by the GPU path. It holds only
input recipes: shapes, value distributions and random draws. None of the
method's arithmetic lives here.

The recipes stand in for the pages' real workloads (LLaMA-2/3 layers
calibrated on 128 sequences of 2048 tokens). They keep the shapes, the token
count and the value structure the pages describe: outlier input channels, an
output-gradient covariance whose diagonal spans several orders of magnitude,
and an input-column-norm coefficient of variation of 9.2 for the LLaMA-3-70B
down projection.

All random streams derive from ``SeedSequence([1000 + config_id, crc32(name),
*index])``. Activations and gradients are drawn in float32, multiplied by a
per-channel scale and rounded to bfloat16 with round-to-nearest-even. They are
kept as uint16 bit patterns, so both sides read exactly the same values.

The rotation specification of each side (a random sign vector and a random
odd-order orthogonal matrix) is a random draw of the method. It is drawn here
and handed to both sides as an input.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
import zlib
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

CHUNK_TOKENS = 8192
# drift of the full-precision model's inputs against the partly quantized model's: a per-channel
# gain 1 + N(0, DRIFT_GAIN) and independent noise of DRIFT_NOISE x the channel scale
DRIFT_GAIN = 0.1
DRIFT_NOISE = 0.05


# ---------------------------------------------------------------------------
# random streams and bf16 bit patterns
# ---------------------------------------------------------------------------
def stream(config_id: int, name: str, *index: int) -> np.random.Generator:
    """Independent, reproducible random stream for one named input piece."""
    key = [1000 + int(config_id), zlib.crc32(name.encode("utf-8"))] + [int(i) for i in index]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. Inputs here are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class SubLayer:
    name: str
    dout: int
    din: int
    x_group: str            # sub-layers with the same input share one activation matrix
    bits: Optional[int]     # None: chosen by the mixed-precision allocation


@dataclass(frozen=True)
class Config:
    id: int
    name: str
    n_tokens: int
    subs: Tuple[SubLayer, ...]
    group: int              # 0 = one grid per output row
    block: int              # lazy-batch block of the column sweep
    damp: float
    w_dtype: str            # "f32" or "bf16"
    x_scale: str            # "lognormal" or "outlier20"
    g_scale: str            # "lognormal" or "log10uniform"
    w_outlier_cols: int = 0         # input columns of W scaled so the column-norm CV hits w_col_cv
    w_col_cv: float = 0.0
    alloc_choices: Tuple[int, ...] = ()
    alloc_target_millibits: int = 0
    biip: bool = True

    @property
    def x_groups(self) -> Dict[str, int]:
        out: Dict[str, int] = {}
        for s in self.subs:
            out.setdefault(s.x_group, s.din)
        return out

    def sub(self, name: str) -> SubLayer:
        for s in self.subs:
            if s.name == name:
                return s
        raise KeyError(name)

    def n_chunks(self) -> int:
        return (self.n_tokens + CHUNK_TOKENS - 1) // CHUNK_TOKENS

    def chunk_rows(self, c: int) -> int:
        return min(CHUNK_TOKENS, self.n_tokens - c * CHUNK_TOKENS)


def _sl(name, dout, din, grp, bits=None):
    return SubLayer(name, dout, din, grp, bits)


CONFIGS: Dict[int, Config] = {
    # single small linear layer, per-row 4-bit grid
    1: Config(1, "linear64x128", 512, (_sl("linear", 64, 128, "in", 4),), group=0, block=32,
              damp=0.01, w_dtype="f32", x_scale="outlier20", g_scale="lognormal"),
    # LLaMA-2-7B q_proj (run at 2 and at 4 bits)
    2: Config(2, "llama2-7b.q_proj", 262144, (_sl("q_proj", 4096, 4096, "attn_in", 2),), group=128,
              block=128, damp=0.01, w_dtype="bf16", x_scale="lognormal", g_scale="log10uniform"),
    # LLaMA-2-13B MLP
    3: Config(3, "llama2-13b.mlp", 262144,
              (_sl("gate_proj", 13824, 5120, "mlp_in", 3), _sl("up_proj", 13824, 5120, "mlp_in", 3),
               _sl("down_proj", 5120, 13824, "down_in", 3)),
              group=128, block=128, damp=0.01, w_dtype="bf16", x_scale="lognormal", g_scale="lognormal"),
    # LLaMA-3-70B down_proj with extreme input-column outliers
    4: Config(4, "llama3-70b.down_proj", 262144, (_sl("down_proj", 8192, 28672, "down_in", 2),), group=128,
              block=128, damp=0.01, w_dtype="bf16", x_scale="lognormal", g_scale="log10uniform",
              w_outlier_cols=32, w_col_cv=9.2),
    # LLaMA-3-8B decoder block with mixed-precision allocation
    5: Config(5, "llama3-8b.block", 131072,
              (_sl("q_proj", 4096, 4096, "attn_in"), _sl("k_proj", 1024, 4096, "attn_in"),
               _sl("v_proj", 1024, 4096, "attn_in"), _sl("o_proj", 4096, 4096, "o_in"),
               _sl("gate_proj", 14336, 4096, "mlp_in"), _sl("up_proj", 14336, 4096, "mlp_in"),
               _sl("down_proj", 4096, 14336, "down_in")),
              group=128, block=128, damp=0.01, w_dtype="bf16", x_scale="lognormal", g_scale="lognormal",
              alloc_choices=(2, 3, 4), alloc_target_millibits=3000),
}


def config(i: int) -> Config:
    return CONFIGS[i]


def scaled(cfg: Config, *, n_tokens: int, dims: Dict[str, Tuple[int, int]], block: Optional[int] = None,
           group: Optional[int] = None, w_outlier_cols: Optional[int] = None, biip: Optional[bool] = None,
           bits: Optional[Dict[str, int]] = None) -> Config:
    """Same recipe as ``cfg`` at smaller shapes (for tests the oracle finishes in seconds)."""
    subs = []
    for s in cfg.subs:
        dout, din = dims.get(s.name, (s.dout, s.din))
        b = s.bits if bits is None else bits.get(s.name, s.bits)
        subs.append(replace(s, dout=dout, din=din, bits=b))
    return replace(cfg, n_tokens=n_tokens, subs=tuple(subs),
                   block=cfg.block if block is None else block,
                   group=cfg.group if group is None else group,
                   w_outlier_cols=cfg.w_outlier_cols if w_outlier_cols is None else w_outlier_cols,
                   biip=cfg.biip if biip is None else biip)


# ---------------------------------------------------------------------------
# rotation specification (random draw of the method, passed to both sides)
# ---------------------------------------------------------------------------
@dataclass
class RotSpec:
    n: int
    m: int                  # odd factor
    log2p: int              # n = m * 2**log2p
    signs: np.ndarray       # int8 [n], entries +1 / -1
    q: np.ndarray           # float64 [m, m], orthogonal

    @property
    def p(self) -> int:
        return 1 << self.log2p


def split_odd(n: int) -> Tuple[int, int]:
    """n = m * 2**k with m odd."""
    if n <= 0:
        raise ValueError("dimension must be positive")
    k = (n & -n).bit_length() - 1
    return n >> k, k


def random_orthogonal(rng: np.random.Generator, m: int) -> np.ndarray:
    """Haar-random orthogonal m x m matrix (QR of a Gaussian, R's diagonal made positive)."""
    if m == 1:
        return np.ones((1, 1))
    a = rng.standard_normal((m, m))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def rot_spec(config_id: int, key: str, n: int) -> RotSpec:
    m, k = split_odd(n)
    rng = stream(config_id, "rot:" + key, n)
    signs = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    q = random_orthogonal(rng, m)
    return RotSpec(n=n, m=m, log2p=k, signs=signs, q=q)


# ---------------------------------------------------------------------------
# per-layer data
# ---------------------------------------------------------------------------
def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class Workload:
    """Lazily generated, seeded inputs of one configuration."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self._cache: Dict[Tuple, np.ndarray] = {}

    # -- channel scales ---------------------------------------------------
    def x_scales(self, group: str) -> np.ndarray:
        cfg, din = self.cfg, self.cfg.x_groups[group]
        rng = stream(cfg.id, "xscale:" + group, din)
        if cfg.x_scale == "lognormal":
            return np.exp(rng.normal(0.0, 1.5, din)).astype(np.float32)
        if cfg.x_scale == "outlier20":
            s = np.ones(din, np.float32)
            s[rng.choice(din, size=min(4, din), replace=False)] = 20.0
            return s
        raise ValueError(cfg.x_scale)

    def g_scales(self, sub: str) -> np.ndarray:
        cfg, dout = self.cfg, self.cfg.sub(sub).dout
        rng = stream(cfg.id, "gscale:" + sub, dout)
        if cfg.g_scale == "lognormal":
            return np.exp(rng.normal(0.0, 1.5, dout)).astype(np.float32)
        if cfg.g_scale == "log10uniform":
            return (10.0 ** rng.uniform(-2.0, 2.0, dout)).astype(np.float32)
        raise ValueError(cfg.g_scale)

    # -- token-major bf16 matrices ----------------------------------------
    def _chunk_f32(self, kind: str, key: str, c: int, d: int, scales: np.ndarray) -> np.ndarray:
        rows = self.cfg.chunk_rows(c)
        rng = stream(self.cfg.id, kind + ":" + key, c, d)
        a = rng.standard_normal((rows, d), dtype=np.float32)
        a *= scales[None, :]
        return a

    def _chunk(self, kind: str, key: str, c: int, d: int, scales: np.ndarray) -> np.ndarray:
        if kind == "xt":
            # full-precision inputs: the same draws as "x" with a seeded per-channel gain
            # (1 + g_j, g ~ N(0, DRIFT_GAIN)) and independent noise of DRIFT_NOISE x the channel
            # scale, rounded to bf16 on their own
            a = self._chunk_f32("x", key, c, d, scales)
            gain = 1.0 + DRIFT_GAIN * stream(self.cfg.id, "xgain:" + key, d).standard_normal(d)
            rng = stream(self.cfg.id, "xdrift:" + key, c, d)
            a = a * gain.astype(np.float32)[None, :]
            a += DRIFT_NOISE * rng.standard_normal(a.shape, dtype=np.float32) * scales[None, :]
            return f32_to_bf16_bits(a)
        return f32_to_bf16_bits(self._chunk_f32(kind, key, c, d, scales))

    def x_chunk(self, group: str, c: int) -> np.ndarray:
        return self._chunk("x", group, c, self.cfg.x_groups[group], self.x_scales(group))

    def g_chunk(self, sub: str, c: int) -> np.ndarray:
        return self._chunk("g", sub, c, self.cfg.sub(sub).dout, self.g_scales(sub))

    def _full(self, kind: str, key: str, d: int, scales: np.ndarray) -> np.ndarray:
        ck = (kind, key)
        if ck in self._cache:
            return self._cache[ck]
        out = np.empty((self.cfg.n_tokens, d), np.uint16)

        def fill(c):
            r0 = c * CHUNK_TOKENS
            out[r0:r0 + self.cfg.chunk_rows(c)] = self._chunk(kind, key, c, d, scales)

        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(self.cfg.n_chunks())))
        self._cache[ck] = out
        return out

    def x(self, group: str) -> np.ndarray:
        """All calibration activations of one input group, [n_tokens, din] bf16 bits."""
        return self._full("x", group, self.cfg.x_groups[group], self.x_scales(group))

    def g(self, sub: str) -> np.ndarray:
        """All output gradients of one sub-layer, [n_tokens, dout] bf16 bits."""
        return self._full("g", sub, self.cfg.sub(sub).dout, self.g_scales(sub))

    def xt(self, group: str) -> np.ndarray:
        """Full-precision-model inputs of one input group for the asymmetric (GPTAQ) objective,
        [n_tokens, din] bf16 bits: x(group)'s values before rounding with a seeded per-channel
        gain drift (DRIFT_GAIN) and noise (DRIFT_NOISE x the channel scale). x(group) stands
        for the inputs the partly quantised model sees."""
        return self._full("xt", group, self.cfg.x_groups[group], self.x_scales(group))

    def drop(self, kind: str, key: str) -> None:
        self._cache.pop((kind, key), None)

    # -- weights ----------------------------------------------------------
    def weight(self, sub: str) -> np.ndarray:
        """W [dout, din]: float32 values, or bf16 bit patterns (uint16) when w_dtype == 'bf16'."""
        cfg, s = self.cfg, self.cfg.sub(sub)
        rng = stream(cfg.id, "w:" + sub, s.dout, s.din)
        w = rng.normal(0.0, 0.02, (s.dout, s.din))
        if cfg.w_outlier_cols:
            cols = stream(cfg.id, "wcols:" + sub, s.din).choice(s.din, size=cfg.w_outlier_cols, replace=False)
            w[:, cols] *= _solve_outlier_factor(w, cols, cfg.w_col_cv)
        if cfg.w_dtype == "f32":
            return w.astype(np.float32)
        return f32_to_bf16_bits(w.astype(np.float32))

    def weight_f64(self, sub: str) -> np.ndarray:
        w = self.weight(sub)
        return bf16_bits_to_f64(w) if w.dtype == np.uint16 else w.astype(np.float64)

    # -- rotation specs ---------------------------------------------------
    def rot_in(self, group: str) -> RotSpec:
        return rot_spec(self.cfg.id, "in:" + group, self.cfg.x_groups[group])

    def rot_out(self, sub: str) -> RotSpec:
        return rot_spec(self.cfg.id, "out:" + sub, self.cfg.sub(sub).dout)


def column_norm_cv(w: np.ndarray) -> float:
    n = np.linalg.norm(np.asarray(w, np.float64), axis=0)
    return float(n.std() / n.mean())


def _solve_outlier_factor(w: np.ndarray, cols: np.ndarray, target_cv: float) -> float:
    """Factor a for the chosen columns so that the column-norm CV of W equals target_cv."""
    norms = np.linalg.norm(w, axis=0)
    mask = np.zeros(w.shape[1], bool)
    mask[cols] = True

    def cv(a):
        n = np.where(mask, norms * a, norms)
        return n.std() / n.mean()

    lo, hi = 1.0, 2.0
    while cv(hi) < target_cv:
        hi *= 2.0
        if hi > 1e12:
            raise ValueError("column-norm CV target not reachable with this many outlier columns")
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if cv(mid) < target_cv:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)
