"""KronQ per-layer quantization on AMD Instinct MI355X (gfx950).

Python binding of ``libkq.so``: one function per C entry point of
``include/kq.h``, with the same names and argument order. The binding only
marshals arguments (device pointers of torch tensors, the current HIP stream,
scratch buffers); every step of the path runs in the library's HIP kernels.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "KQError", "KQ_OK", "KQ_EINVAL", "KQ_ENOTPD", "KQ_EINFEASIBLE", "KQ_EDEVICE", "KQ_EUNSUPPORTED",
    "KQ_BF16", "KQ_F32", "KQ_F64", "KQ_BIIP_INPUT", "KQ_BIIP_OUTPUT", "KQ_BIIP_SCALE", "KQ_BIIP_INVERSE",
    "KQ_SCORE_KRONQ", "KQ_SCORE_HX_ONLY", "KQ_OP_ACCUMULATE_COV", "KQ_OP_BIIP", "KQ_OP_CHOLESKY", "KQ_OP_OBS",
    "KQ_OP_DECODE", "KQ_OP_LOSS", "KQ_OP_XCOV", "KQ_OP_GPTAQ", "KQ_DECODE_MAX_TOKENS", "KQ_DECODE_MAX_LAYERS",
    "lib", "lib_path", "version", "workspace_size", "accumulate_cov", "sensitivity", "allocate_bits",
    "biip_rotate", "cholesky_inv", "obs_quantize", "pack_codes", "decode_matvec", "decode_matvec_group",
    "decode_matvec_group_noalloc", "decode_workspace", "kron_loss", "Rot", "KQ_DECODE_NOALLOC_SCRATCH",
    "DecodeLayer", "accumulate_xcov", "biip_transform", "gptaq_target",
    "timing_enable", "timing_query",
]

KQ_OK, KQ_EINVAL, KQ_ENOTPD, KQ_EINFEASIBLE, KQ_EDEVICE, KQ_EUNSUPPORTED = range(6)
KQ_BF16, KQ_F32, KQ_F64 = 0, 1, 2
KQ_BIIP_INPUT, KQ_BIIP_OUTPUT, KQ_BIIP_SCALE, KQ_BIIP_INVERSE = 1, 2, 4, 8
KQ_SCORE_KRONQ, KQ_SCORE_HX_ONLY = 0, 1
KQ_OP_ACCUMULATE_COV, KQ_OP_BIIP, KQ_OP_CHOLESKY, KQ_OP_OBS, KQ_OP_DECODE, KQ_OP_LOSS = 0, 1, 2, 3, 4, 5
KQ_OP_XCOV, KQ_OP_GPTAQ = 6, 7
KQ_DECODE_MAX_TOKENS = 4
KQ_DECODE_MAX_LAYERS = 4
KQ_DECODE_NOALLOC_SCRATCH = 2228224

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.environ.get("KQ_LIB", os.path.join(_HERE, "libkq.so"))


class KQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Rot(ctypes.Structure):
    """kq_rot: one side's rotation U = (Q_m kron H_p / sqrt(p)) diag(sigma)."""

    _fields_ = [("n", ctypes.c_int64), ("m", ctypes.c_int32), ("log2p", ctypes.c_int32),
                ("signs", ctypes.c_void_p), ("q", ctypes.c_void_p)]


class DecodeLayer(ctypes.Structure):
    """kq_decode_layer: one layer of a decode group (device pointers; rot_out a host pointer)."""

    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("dout", ctypes.c_int64), ("s_g", ctypes.c_void_p), ("rot_out", ctypes.POINTER(Rot)),
                ("y", ctypes.c_void_p)]


_LIB = None
_VP, _I64, _I32, _U32, _F32, _SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                                    ctypes.c_float, ctypes.c_size_t)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise KQError(KQ_EDEVICE, f"libkq.so not found at {path}; build it with "
                                  f"`python -m post_quantization_04_amd.build`")
    L = ctypes.CDLL(path)
    L.kq_version.restype = ctypes.c_char_p
    L.kq_status_string.restype = ctypes.c_char_p
    L.kq_status_string.argtypes = [ctypes.c_int]
    L.kq_last_error.restype = ctypes.c_char_p
    L.kq_timing_enable.argtypes = [ctypes.c_char_p]
    L.kq_timing_enable.restype = ctypes.c_int
    L.kq_timing_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
    L.kq_timing_query.restype = ctypes.c_int
    L.kq_workspace_size.restype = _SZ
    L.kq_workspace_size.argtypes = [_I32, _I64, _I64, _I64]
    L.kq_accumulate_cov.argtypes = [_VP, _I64, _I64, _I64, _F32, _F32, _VP, _VP, _SZ, _VP]
    L.kq_accumulate_xcov.argtypes = [_VP, _VP, _I64, _I64, _I64, _I64, _F32, _F32, _VP, _VP, _VP, _SZ, _VP]
    L.kq_biip_transform.argtypes = [_VP, _I64, ctypes.POINTER(Rot), _VP, _VP, _SZ, _VP]
    L.kq_gptaq_target.argtypes = [_VP, _VP, _VP, _I64, _I64, _VP, _VP, _SZ, _VP]
    L.kq_sensitivity.argtypes = [_VP, _I64, _VP, _I64, _I32, _VP, _VP]
    L.kq_allocate_bits.argtypes = [_VP, _VP, _I32, _VP, _I32, _I64, _VP]
    L.kq_biip_rotate.argtypes = [_VP, _I32, _I64, _I64, _VP, _VP, _VP, ctypes.POINTER(Rot),
                                 ctypes.POINTER(Rot), _U32, _VP, _VP, _VP, _SZ, _VP]
    L.kq_cholesky_inv.argtypes = [_VP, _I64, _F32, _VP, _VP, _SZ, _VP]
    L.kq_obs_quantize.argtypes = [_VP, _VP, _I64, _I64, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]
    L.kq_pack_codes.argtypes = [_VP, _I64, _I64, _I32, _VP, _VP]
    L.kq_kron_loss.argtypes = [_VP, _VP, _I32, _I64, _I64, _VP, _VP, _VP, _VP, _SZ, _VP]
    L.kq_decode_matvec.argtypes = [_VP, _VP, _VP, _I64, _I64, _I32, _I32, _VP, _VP, ctypes.POINTER(Rot),
                                   ctypes.POINTER(Rot), _VP, _I64, _VP, _VP, _SZ, _VP]
    L.kq_decode_matvec_group.argtypes = [ctypes.POINTER(DecodeLayer), _I32, _I64, _I32, _I32, _VP,
                                         ctypes.POINTER(Rot), _VP, _I64, _VP, _SZ, _VP]
    L.kq_decode_matvec_group_noalloc.argtypes = [ctypes.POINTER(DecodeLayer), _I32, _I64, _I32, _I32, _VP,
                                                 ctypes.POINTER(Rot), _VP, _I64, _VP]
    for name in ("kq_accumulate_cov", "kq_sensitivity", "kq_allocate_bits", "kq_biip_rotate",
                 "kq_cholesky_inv", "kq_obs_quantize", "kq_pack_codes", "kq_decode_matvec",
                 "kq_decode_matvec_group", "kq_decode_matvec_group_noalloc", "kq_kron_loss",
                 "kq_accumulate_xcov", "kq_biip_transform", "kq_gptaq_target"):
        getattr(L, name).restype = ctypes.c_int
    _LIB = L
    return L


def version() -> str:
    return lib().kq_version().decode()


def timing_enable(filter: Optional[str] = "") -> None:
    """Bracket launches of kernels whose name contains ``filter`` with HIP events (None: off)."""
    _check(lib().kq_timing_enable(None if filter is None else filter.encode()), "kq_timing_enable")


def timing_query(name: str):
    """(launches, total milliseconds) of the recorded kernels whose name contains ``name``."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().kq_timing_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)), "kq_timing_query")
    return int(n.value), float(ms.value)


def _check(status: int, what: str) -> None:
    if status != KQ_OK:
        L = lib()
        raise KQError(status, f"{what}: {L.kq_status_string(status).decode()}: {L.kq_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _scratch(nbytes: int, device):
    import torch
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise KQError(KQ_EINVAL, msg)


def workspace_size(op: int, d0: int, d1: int = 0, d2: int = 0) -> int:
    n = lib().kq_workspace_size(op, d0, d1, d2)
    if n == ctypes.c_size_t(-1).value:
        raise KQError(KQ_EINVAL, f"kq_workspace_size: invalid sizes for op {op}")
    return n


def accumulate_cov(a, h, alpha: float, beta: float, *, ws=None, stream=None) -> None:
    """h <- alpha * a^T a + beta * h; a: [rows, d] torch.bfloat16 (or int16/uint16 bits), h: [d, d] float32."""
    import torch
    _need(a.dim() == 2 and h.dim() == 2 and h.shape[0] == h.shape[1] == a.shape[1], "accumulate_cov: shapes")
    _need(a.dtype in (torch.bfloat16, torch.int16, torch.uint16) and h.dtype == torch.float32,
          "accumulate_cov: dtypes")
    _need(a.stride(1) == 1 and h.is_contiguous(), "accumulate_cov: layout")
    rows, d = a.shape
    need = workspace_size(KQ_OP_ACCUMULATE_COV, rows, d)
    if ws is None:
        ws = _scratch(need, h.device)
    _check(lib().kq_accumulate_cov(_ptr(a), rows, d, a.stride(0), alpha, beta, _ptr(h), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)), "kq_accumulate_cov")


def accumulate_xcov(a, b, c, alpha: float, beta: float, c_in=None, *, ws=None, stream=None) -> None:
    """c <- alpha * a^T b + beta * c_in (c_in defaults to c); a, b: [rows, d] bf16 (or int16/uint16 bits)
    over the same tokens, c / c_in: [d, d] float32."""
    import torch
    _need(a.dim() == 2 and b.shape == a.shape and c.dim() == 2 and c.shape[0] == c.shape[1] == a.shape[1],
          "accumulate_xcov: shapes")
    bits = (torch.bfloat16, torch.int16, torch.uint16)
    _need(a.dtype in bits and b.dtype in bits and c.dtype == torch.float32, "accumulate_xcov: dtypes")
    _need(a.stride(1) == 1 and b.stride(1) == 1 and c.is_contiguous(), "accumulate_xcov: layout")
    if c_in is None:
        c_in = c
    _need(c_in.shape == c.shape and c_in.dtype == torch.float32 and c_in.is_contiguous(), "accumulate_xcov: c_in")
    rows, d = a.shape
    need = workspace_size(KQ_OP_XCOV, rows, d)
    if ws is None:
        ws = _scratch(need, c.device)
    _check(lib().kq_accumulate_xcov(_ptr(a), _ptr(b), rows, d, a.stride(0), b.stride(0), alpha, beta, _ptr(c_in),
                                    _ptr(c), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "kq_accumulate_xcov")


def biip_transform(m, rot: Rot, s=None, *, ws=None, stream=None) -> None:
    """m <- U S^-1 m S^-1 U^T in place (the input-side map of BiIP); m: [n, n] float32, s: [n] float64 or None."""
    import torch
    _need(m.dim() == 2 and m.shape[0] == m.shape[1] and m.dtype == torch.float32 and m.is_contiguous(),
          "biip_transform: m must be a contiguous square float32 matrix")
    _need(s is None or (s.dtype == torch.float64 and s.numel() == m.shape[0]), "biip_transform: s")
    n = m.shape[0]
    need = workspace_size(KQ_OP_BIIP, n, n)
    if ws is None:
        ws = _scratch(need, m.device)
    _check(lib().kq_biip_transform(_ptr(m), n, ctypes.byref(rot), _ptr(s), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(stream)), "kq_biip_transform")


def gptaq_target(w, d2, r, *, info=None, ws=None, stream=None) -> None:
    """w <- w + w triu(d2 r^T, 1) r in place; w: [dout, din] float64, d2 and r: [din, din] float32.
    ``info`` (optional int32 device tensor, zeroed by the caller) becomes 1 if a result is not finite."""
    import torch
    _need(w.dim() == 2 and w.dtype == torch.float64 and w.is_contiguous(), "gptaq_target: w")
    din = w.shape[1]
    for m, name in ((d2, "d2"), (r, "r")):
        _need(m.shape == (din, din) and m.dtype == torch.float32 and m.is_contiguous(), f"gptaq_target: {name}")
    dout = w.shape[0]
    need = workspace_size(KQ_OP_GPTAQ, dout, din)
    if ws is None:
        ws = _scratch(need, w.device)
    if info is not None:
        _need(info.dtype == torch.int32 and info.numel() >= 1, "gptaq_target: info must be int32")
    _check(lib().kq_gptaq_target(_ptr(w), _ptr(d2), _ptr(r), dout, din, _ptr(info), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)), "kq_gptaq_target")


def sensitivity(h_x, h_g, score, mode: int = KQ_SCORE_KRONQ, *, stream=None) -> None:
    """score[0] <- tr(h_g) * tr(h_x) (or tr(h_x)); score: float64 device tensor of one element."""
    import torch
    _need(score.dtype == torch.float64 and score.numel() >= 1, "sensitivity: score must be float64")
    dout = 0 if h_g is None else h_g.shape[0]
    _check(lib().kq_sensitivity(_ptr(h_x), h_x.shape[0], _ptr(h_g), dout, mode, _ptr(score), _stream(stream)),
           "kq_sensitivity")


def allocate_bits(score: Sequence[float], n_params: Sequence[int], choices: Sequence[int],
                  target_millibits: int) -> list:
    """Host-side bit allocation; returns the list of bit widths."""
    s = np.ascontiguousarray(score, dtype=np.float64)
    n = np.ascontiguousarray(n_params, dtype=np.int64)
    c = np.ascontiguousarray(choices, dtype=np.int32)
    out = np.zeros(len(s), dtype=np.int32)
    _need(len(s) == len(n), "allocate_bits: score and n_params differ in length")
    _check(lib().kq_allocate_bits(s.ctypes.data, n.ctypes.data, len(s), c.ctypes.data, len(c),
                                  int(target_millibits), out.ctypes.data), "kq_allocate_bits")
    return out.tolist()


def make_rot(signs, q) -> Rot:
    """kq_rot from device tensors: signs int8 [n], q float64 [m, m]."""
    n = signs.numel()
    m = q.shape[0]
    k = (n // m).bit_length() - 1
    return Rot(n=n, m=m, log2p=k, signs=_ptr(signs), q=_ptr(q))


def biip_rotate(w, w_out, h_x, h_g, rot_in: Optional[Rot], rot_out: Optional[Rot], flags: int, s_x, s_g, *,
                ws=None, stream=None) -> None:
    """Forward: w_out = U_G S_G w S_X U_X^T, h_x / h_g transformed in place. Inverse with KQ_BIIP_INVERSE."""
    import torch
    dtypes = {torch.bfloat16: KQ_BF16, torch.int16: KQ_BF16, torch.uint16: KQ_BF16,
              torch.float32: KQ_F32, torch.float64: KQ_F64}
    _need(w.dtype in dtypes and w.is_contiguous() and w_out.dtype == torch.float64 and w_out.is_contiguous(),
          "biip_rotate: w / w_out dtype or layout")
    _need(s_x.dtype == torch.float64 and s_g.dtype == torch.float64, "biip_rotate: scales must be float64")
    dout, din = w.shape
    need = workspace_size(KQ_OP_BIIP, dout, din)
    if ws is None:
        ws = _scratch(need, w.device)
    _check(lib().kq_biip_rotate(_ptr(w), dtypes[w.dtype], dout, din, _ptr(w_out), _ptr(h_x), _ptr(h_g),
                                None if rot_in is None else ctypes.byref(rot_in),
                                None if rot_out is None else ctypes.byref(rot_out), flags, _ptr(s_x), _ptr(s_g),
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "kq_biip_rotate")


def cholesky_inv(h, damp: float, info, *, ws=None, stream=None) -> None:
    """h (float32 [d, d]) <- upper R with R^T R = (h + damp * mean(diag h) * I)^-1; info int32 device [1]."""
    import torch
    _need(h.dtype == torch.float32 and h.is_contiguous() and info.dtype == torch.int32, "cholesky_inv: dtypes")
    d = h.shape[0]
    need = workspace_size(KQ_OP_CHOLESKY, d)
    if ws is None:
        ws = _scratch(need, h.device)
    _check(lib().kq_cholesky_inv(_ptr(h), d, damp, _ptr(info), _ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream(stream)), "kq_cholesky_inv")


def obs_quantize(w, r, bits: int, group: int, block: int, codes, scales, zeros, preround=None, *, ws=None,
                 stream=None) -> None:
    """Column-wise OBS: w (float64 [dout, din]) in W'', out dequantised; codes/scales/zeros written."""
    import torch
    _need(w.dtype == torch.float64 and r.dtype == torch.float32 and codes.dtype == torch.uint8
          and scales.dtype == torch.float32 and zeros.dtype == torch.uint8, "obs_quantize: dtypes")
    dout, din = w.shape
    need = workspace_size(KQ_OP_OBS, dout, din, block)
    if ws is None:
        ws = _scratch(need, w.device)
    _check(lib().kq_obs_quantize(_ptr(w), _ptr(r), dout, din, bits, group, block, _ptr(codes), _ptr(scales),
                                 _ptr(zeros), _ptr(preround), _ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream(stream)), "kq_obs_quantize")


def kron_loss(w_hat, w, h_x, h_g, loss, *, ws=None, stream=None) -> None:
    """loss[0] <- tr((w_hat - w) h_x (w_hat - w)^T h_g); w_hat float64 [dout, din], w bf16 bits / float32 /
    float64, h_x / h_g float32, loss a float64 device tensor of one element."""
    import torch
    dtypes = {torch.bfloat16: KQ_BF16, torch.int16: KQ_BF16, torch.uint16: KQ_BF16,
              torch.float32: KQ_F32, torch.float64: KQ_F64}
    _need(w_hat.dtype == torch.float64 and w_hat.is_contiguous() and w.dtype in dtypes and w.is_contiguous(),
          "kron_loss: w_hat / w dtype or layout")
    _need(tuple(w.shape) == tuple(w_hat.shape), "kron_loss: w and w_hat differ in shape")
    dout, din = w_hat.shape
    _need(h_x.dtype == torch.float32 and h_g.dtype == torch.float32 and h_x.is_contiguous() and h_g.is_contiguous()
          and tuple(h_x.shape) == (din, din) and tuple(h_g.shape) == (dout, dout), "kron_loss: covariances")
    _need(loss.dtype == torch.float64 and loss.numel() >= 1, "kron_loss: loss must be float64")
    need = workspace_size(KQ_OP_LOSS, dout, din)
    if ws is None:
        ws = _scratch(need, w_hat.device)
    _check(lib().kq_kron_loss(_ptr(w_hat), _ptr(w), dtypes[w.dtype], dout, din, _ptr(h_x), _ptr(h_g), _ptr(loss),
                              _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "kq_kron_loss")


def pack_codes(codes, bits: int, packed, *, stream=None) -> None:
    """packed (uint32-sized int32 [rows, cols * c / 32]) <- codes (uint8 [rows, cols]); c = 2, 4 or 8."""
    import torch
    _need(codes.dtype == torch.uint8 and codes.is_contiguous() and packed.dtype == torch.int32
          and packed.is_contiguous(), "pack_codes: dtypes or layout")
    rows, cols = codes.shape
    c = 2 if bits == 2 else (4 if bits <= 4 else 8)
    _need(tuple(packed.shape) == (rows, cols * c // 32), "pack_codes: packed must be [rows, cols * c / 32]")
    _check(lib().kq_pack_codes(_ptr(codes), rows, cols, bits, _ptr(packed), _stream(stream)), "kq_pack_codes")


def decode_workspace(dout: int, din: int, tokens: int, device):
    """A workspace for decode_matvec."""
    import torch
    return torch.empty(workspace_size(KQ_OP_DECODE, dout, din, tokens), dtype=torch.uint8, device=device)


def _check_decode_layer(packed, scales, zeros, bits: int, group: int, din: int, s_g, y, tokens: int) -> int:
    """Shape and dtype checks of one layer's tensors; returns its dout."""
    import torch
    _need(packed.dtype == torch.int32 and scales.dtype == torch.float32 and zeros.dtype == torch.uint8
          and y.dtype == torch.float32 and y.is_contiguous(), "decode_matvec: dtypes or layout")
    _need(s_g is None or s_g.dtype == torch.float64, "decode_matvec: s_g must be float64")
    dout = y.shape[1]
    c = 2 if bits == 2 else (4 if bits <= 4 else 8)
    ngroups = din // group if group else 1
    _need(y.shape[0] == tokens, "decode_matvec: x and y hold different token counts")
    _need(tuple(packed.shape) == (dout, din * c // 32), "decode_matvec: packed must be [dout, din * c / 32]")
    _need(tuple(scales.shape) == (dout, ngroups) and tuple(zeros.shape) == (dout, ngroups),
          "decode_matvec: scales and zeros must be [dout, din / group]")
    _need(scales.is_contiguous() and zeros.is_contiguous() and packed.is_contiguous(),
          "decode_matvec: packed, scales and zeros must be contiguous")
    _need(s_g is None or s_g.numel() == dout, "decode_matvec: s_g must hold dout entries")
    return dout


def decode_matvec(packed, scales, zeros, bits: int, group: int, s_x, s_g, rot_in: Optional[Rot],
                  rot_out: Optional[Rot], x, y, *, ws=None, stream=None) -> None:
    """y (float32 [tokens, dout]) <- S_G^-1 U_G^T W^'' U_X S_X^-1 x for x (float32 [tokens, din])."""
    import torch
    _need(x.dtype == torch.float32 and x.is_contiguous(), "decode_matvec: x must be contiguous float32")
    _need(s_x is None or s_x.dtype == torch.float64, "decode_matvec: s_x must be float64")
    tokens, din = x.shape
    dout = _check_decode_layer(packed, scales, zeros, bits, group, din, s_g, y, tokens)
    _need(s_x is None or s_x.numel() == din, "decode_matvec: s_x must hold din entries")
    if ws is None:
        ws = decode_workspace(dout, din, tokens, x.device)
    _check(lib().kq_decode_matvec(_ptr(packed), _ptr(scales), _ptr(zeros), dout, din, bits, group, _ptr(s_x),
                                  _ptr(s_g), None if rot_in is None else ctypes.byref(rot_in),
                                  None if rot_out is None else ctypes.byref(rot_out), _ptr(x), tokens, _ptr(y),
                                  _ptr(ws), ws.numel(), _stream(stream)), "kq_decode_matvec")


def decode_matvec_group(layers, bits: int, group: int, s_x, rot_in: Optional[Rot], x, *, ws=None,
                        stream=None) -> None:
    """decode_matvec for up to KQ_DECODE_MAX_LAYERS layers reading the same x with the same input
    side. layers: sequence of (packed, scales, zeros, s_g, rot_out, y) per layer."""
    import torch
    _need(x.dtype == torch.float32 and x.is_contiguous(), "decode_matvec: x must be contiguous float32")
    _need(s_x is None or (s_x.dtype == torch.float64 and s_x.numel() == x.shape[1]),
          "decode_matvec: s_x must be float64 with din entries")
    _need(1 <= len(layers) <= KQ_DECODE_MAX_LAYERS, "decode_matvec_group: 1 to KQ_DECODE_MAX_LAYERS layers")
    tokens, din = x.shape
    arr = (DecodeLayer * len(layers))()
    keep = []
    total = 0
    for i, (packed, scales, zeros, s_g, rot_out, y) in enumerate(layers):
        dout = _check_decode_layer(packed, scales, zeros, bits, group, din, s_g, y, tokens)
        total += dout
        arr[i] = DecodeLayer(_ptr(packed), _ptr(scales), _ptr(zeros), dout, _ptr(s_g),
                             None if rot_out is None else ctypes.pointer(rot_out), _ptr(y))
        keep.append(rot_out)
    if ws is None:
        ws = decode_workspace(total, din, tokens, x.device)
    _check(lib().kq_decode_matvec_group(arr, len(layers), din, bits, group, _ptr(s_x),
                                        None if rot_in is None else ctypes.byref(rot_in), _ptr(x), tokens,
                                        _ptr(ws), ws.numel(), _stream(stream)), "kq_decode_matvec_group")


def decode_matvec_group_noalloc(layers, bits: int, group: int, s_x, rot_in: Optional[Rot], x, *,
                                stream=None) -> None:
    """decode_matvec_group without a workspace: the library's fixed device scratch array is used
    (no allocation by the library or by this binding). Calls that overlap on one GPU race on it."""
    import torch
    _need(x.dtype == torch.float32 and x.is_contiguous(), "decode_matvec: x must be contiguous float32")
    _need(s_x is None or (s_x.dtype == torch.float64 and s_x.numel() == x.shape[1]),
          "decode_matvec: s_x must be float64 with din entries")
    _need(1 <= len(layers) <= KQ_DECODE_MAX_LAYERS, "decode_matvec_group: 1 to KQ_DECODE_MAX_LAYERS layers")
    tokens, din = x.shape
    arr = (DecodeLayer * len(layers))()
    keep = []
    for i, (packed, scales, zeros, s_g, rot_out, y) in enumerate(layers):
        dout = _check_decode_layer(packed, scales, zeros, bits, group, din, s_g, y, tokens)
        arr[i] = DecodeLayer(_ptr(packed), _ptr(scales), _ptr(zeros), dout, _ptr(s_g),
                             None if rot_out is None else ctypes.pointer(rot_out), _ptr(y))
        keep.append(rot_out)
    _check(lib().kq_decode_matvec_group_noalloc(arr, len(layers), din, bits, group, _ptr(s_x),
                                                None if rot_in is None else ctypes.byref(rot_in), _ptr(x), tokens,
                                                _stream(stream)), "kq_decode_matvec_group_noalloc")
