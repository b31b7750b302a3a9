"""Python face of the CPU oracle (oracle.c) for the CSA/HCA compressed-attention layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the benchmark's CPU
baseline leg may import this module.  It never imports the HIP package, and the HIP package never
imports it.  All arithmetic happens in oracle.c (fp64, no fusion); this file only marshals numpy
arrays and composes the oracle's own steps (compress -> round to fp32 -> encode, scores -> top-k).

Cache tensors are passed around as dicts: {"fmt": "f32"|"bf16"|"mixed"|"fp4", "dim", "rope", "cap",
"data", "rope_data", "scale"} holding numpy arrays laid out as documented in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT = {"f32": 0, "bf16": 1, "mixed": 2, "fp4": 3}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no FP contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", "-Wall", "-Wno-unused-function", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        _setup(_lib)
    return _lib


class _Cache(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("dim", ctypes.c_int), ("rope", ctypes.c_int), ("cap", ctypes.c_longlong),
                ("data", ctypes.c_void_p), ("rope_data", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("table", ctypes.c_void_p), ("block_rows", ctypes.c_int)]


_P = ctypes.c_void_p


def _setup(L):
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_bf16_encode1.argtypes = [ctypes.c_float]
    L.orc_bf16_encode1.restype = ctypes.c_uint16
    L.orc_bf16_decode1.argtypes = [ctypes.c_uint16]
    L.orc_bf16_decode1.restype = ctypes.c_double
    L.orc_fp8_encode1.argtypes = [ctypes.c_float]
    L.orc_fp8_encode1.restype = ctypes.c_uint8
    L.orc_fp8_decode1.argtypes = [ctypes.c_uint8]
    L.orc_fp8_decode1.restype = ctypes.c_double
    L.orc_fp4_encode1.argtypes = [ctypes.c_double]
    L.orc_fp4_encode1.restype = ctypes.c_uint8
    L.orc_fp4_decode1.argtypes = [ctypes.c_uint8]
    L.orc_fp4_decode1.restype = ctypes.c_double
    L.orc_encode_rows.argtypes = [_P, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P, _P]
    L.orc_decode_rows.argtypes = [ctypes.POINTER(_Cache), ctypes.c_longlong, ctypes.c_longlong, _P]
    L.orc_hadamard_rows.argtypes = [_P, ctypes.c_longlong, ctypes.c_int, _P]
    L.orc_kv_compress.argtypes = [_P] * 8 + [ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_longlong, _P]
    L.orc_indexer_scores.argtypes = [ctypes.POINTER(_Cache), _P, ctypes.POINTER(_Cache)] + [ctypes.c_int] * 6 + [
        ctypes.c_longlong, _P, _P, ctypes.c_int, _P, _P, _P, _P, _P]
    L.orc_rmsnorm_rows.argtypes = [_P, ctypes.c_longlong, ctypes.c_int, _P, ctypes.c_double, _P]
    L.orc_rope_rows.argtypes = [_P, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, _P, ctypes.c_double, _P]
    L.orc_dot_is_fp32_exact.argtypes = [_P, _P, ctypes.c_int]
    L.orc_dot_is_fp32_exact.restype = ctypes.c_int
    L.orc_topk_rows.argtypes = [_P, ctypes.c_longlong, ctypes.c_int, _P, ctypes.c_int, _P, _P, _P]
    L.orc_attn.argtypes = [ctypes.POINTER(_Cache), ctypes.POINTER(_Cache), ctypes.c_int, ctypes.POINTER(_Cache),
                           ctypes.c_longlong, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, _P] + [ctypes.c_int] * 5 + [
                               ctypes.c_double, ctypes.c_longlong, _P, _P, ctypes.c_int, _P, _P]
    L.orc_attn.restype = ctypes.c_int


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ----------------------------------------------------------------------------------------------------
# codec
# ----------------------------------------------------------------------------------------------------
def bf16_encode1(x: float) -> int:
    return int(lib().orc_bf16_encode1(float(x)))


def fp8_encode1(y: float) -> int:
    return int(lib().orc_fp8_encode1(float(y)))


def fp8_decode1(c: int) -> float:
    return float(lib().orc_fp8_decode1(int(c)))


def fp4_encode1(y: float) -> int:
    return int(lib().orc_fp4_encode1(float(y)))


def fp4_decode1(c: int) -> float:
    return float(lib().orc_fp4_decode1(int(c)))


def empty_cache(fmt: str, rows: int, dim: int, rope: int = 0, cap: int | None = None) -> dict:
    """Zero-filled cache arrays for `rows` rows (rows = B * cap)."""
    if fmt == "f32":
        d = dict(data=np.zeros((rows, dim), np.float32), rope_data=None, scale=None)
    elif fmt == "bf16":
        d = dict(data=np.zeros((rows, dim), np.uint16), rope_data=None, scale=None)
    elif fmt == "mixed":
        d = dict(data=np.zeros((rows, dim - rope), np.uint8), rope_data=np.zeros((rows, rope), np.uint16),
                 scale=np.zeros((rows,), np.float32))
    elif fmt == "fp4":
        assert dim % 16 == 0
        d = dict(data=np.zeros((rows, dim // 2), np.uint8), rope_data=None, scale=np.zeros((rows, dim // 32), np.uint8))
    else:
        raise ValueError(fmt)
    d.update(fmt=fmt, dim=dim, rope=rope, cap=cap if cap is not None else rows)
    return d


def encode(x: np.ndarray, fmt: str, rope: int = 0, cap: int | None = None) -> dict:
    """Encode fp32 rows x[..., dim] into a cache dict (rows flattened)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    dim = x.shape[-1]
    if fmt == "fp4" and dim % 32:
        raise ValueError("fp4 rows are whole 32-element scale blocks")
    rows = x.size // dim
    c = empty_cache(fmt, rows, dim, rope, cap)
    lib().orc_encode_rows(_ptr(x), rows, FMT[fmt], dim, rope, _ptr(c["data"]), _ptr(c["rope_data"]), _ptr(c["scale"]))
    return c


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """Rows x[..., n] (n a power of two) times the orthonormal Sylvester-Hadamard matrix, in fp64 (oracle.c)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n > 0 and n & (n - 1) == 0, "the Hadamard rotation needs a power-of-two row length"
    y = np.empty_like(x)
    lib().orc_hadamard_rows(_ptr(x), x.size // n, n, _ptr(y))
    return y


def encode_rotated(x: np.ndarray, fmt: str, cap: int | None = None) -> dict:
    """A writer with the rotation flag: rotate each row (fp64), round to fp32, encode."""
    return encode(hadamard_rotate(x).astype(np.float32), fmt, 0, cap)


def _cstruct(c: dict) -> _Cache:
    table = c.get("table")
    if table is not None:
        assert table.dtype == np.int32 and c["cap"] % c["block_rows"] == 0
    return _Cache(FMT[c["fmt"]], int(c["dim"]), int(c["rope"]), int(c["cap"]), _ptr(c["data"]), _ptr(c["rope_data"]),
                  _ptr(c["scale"]), _ptr(table), int(c.get("block_rows", 0)))


def paged(c: dict, B: int, block_rows: int, perm: np.ndarray) -> dict:
    """The same cache stored as a pool of blocks: dense block j (of sequence b, j = b * nblk + jj) moves to pool block
    perm[j]; the table maps (b, jj) to perm[b * nblk + jj].  Only moves bytes."""
    cap = int(c["cap"])
    assert cap % block_rows == 0
    nblk = cap // block_rows
    assert len(perm) == B * nblk
    out = dict(c, table=np.ascontiguousarray(perm.astype(np.int32)), block_rows=block_rows)
    inv = np.argsort(perm)
    for key in ("data", "rope_data", "scale"):
        a = c[key]
        if a is None:
            continue
        blocks = a.reshape(B * nblk, block_rows, *a.shape[1:])
        out[key] = np.ascontiguousarray(blocks[inv].reshape(a.shape))
    return out


def decode(c: dict, row0: int = 0, rows: int | None = None) -> np.ndarray:
    total = c["data"].shape[0]
    rows = total - row0 if rows is None else rows
    out = np.empty((rows, c["dim"]), np.float64)
    s = _cstruct(c)
    lib().orc_decode_rows(ctypes.byref(s), row0, rows, _ptr(out))
    return out


def plain_cache(x: np.ndarray, fmt: str) -> dict:
    """Wrap already-encoded f32 / bf16-bits arrays [..., dim] as a cache dict (no arithmetic)."""
    x = np.ascontiguousarray(x)
    dim = x.shape[-1]
    rows = x.size // dim
    d = dict(fmt=fmt, dim=dim, rope=0, cap=rows, data=x.reshape(rows, dim), rope_data=None, scale=None)
    return d


# ----------------------------------------------------------------------------------------------------
# stage 1: compression
# ----------------------------------------------------------------------------------------------------
def kv_compress(Ca, Cb, Za, Zb, Ba, Bb, tail_Cb=None, tail_Zb=None, m=4, overlap=True, start_pos=0) -> np.ndarray:
    """Compressed entries in float64, shape [B, ceil(n/m), c]."""
    Ca = np.ascontiguousarray(Ca, np.float32)
    Za = np.ascontiguousarray(Za, np.float32)
    B, n, c = Ca.shape
    if overlap:
        Cb = np.ascontiguousarray(Cb, np.float32)
        Zb = np.ascontiguousarray(Zb, np.float32)
        Bb = np.ascontiguousarray(Bb, np.float32)
        if start_pos > 0:
            tail_Cb = np.ascontiguousarray(tail_Cb, np.float32)
            tail_Zb = np.ascontiguousarray(tail_Zb, np.float32)
    Ba = np.ascontiguousarray(Ba, np.float32)
    assert start_pos % m == 0
    nb = (n + m - 1) // m
    out = np.empty((B, nb, c), np.float64)
    lib().orc_kv_compress(_ptr(Ca), _ptr(Cb) if overlap else None, _ptr(Za), _ptr(Zb) if overlap else None, _ptr(Ba),
                          _ptr(Bb) if overlap else None,
                          _ptr(tail_Cb) if (overlap and start_pos > 0) else None,
                          _ptr(tail_Zb) if (overlap and start_pos > 0) else None, B, n, c, m, int(bool(overlap)),
                          start_pos, _ptr(out))
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Rows x[..., c] RMS-normalised with gains g[c] (oracle.c, double)."""
    x = np.ascontiguousarray(x, np.float64)
    c = x.shape[-1]
    g = np.ascontiguousarray(g, np.float32)
    assert g.shape == (c,)
    y = np.empty_like(x)
    lib().orc_rmsnorm_rows(_ptr(x), x.size // c, c, _ptr(g), float(eps), _ptr(y))
    return y


def rope(x: np.ndarray, pos: np.ndarray, rd: int, base: float) -> np.ndarray:
    """Rotary embedding of the trailing rd channels of rows x[..., c] at positions pos[...] (oracle.c, double)."""
    x = np.ascontiguousarray(x, np.float64)
    c = x.shape[-1]
    p = np.ascontiguousarray(np.broadcast_to(pos, x.shape[:-1]), np.float64)
    y = np.empty_like(x)
    lib().orc_rope_rows(_ptr(x), x.size // c, c, int(rd), _ptr(p), float(base), _ptr(y))
    return y


def compress_epilogue(E: np.ndarray, m: int, start_pos: int, norm_g=None, eps: float = 0.0, rope_dims: int = 0,
                      rope_base: float = 10000.0) -> np.ndarray:
    """The epilogues of the compressed entries E [B, n_entries, c] written from token start_pos on: RMSNorm (gains
    norm_g), then RoPE of the trailing rope_dims channels at each entry's position, the first token of its block
    (m * (start_pos / m + i))."""
    y = np.asarray(E, np.float64)
    if norm_g is not None:
        y = rmsnorm(y, norm_g, eps)
    if rope_dims:
        pos = (m * (start_pos // m + np.arange(y.shape[1], dtype=np.float64)))[None, :]
        y = rope(y, np.broadcast_to(pos, y.shape[:-1]), rope_dims, rope_base)
    return y


def compress_to_cache(entries64: np.ndarray, fmt: str, rope: int = 0) -> dict:
    """Entries are computed in fp32 by the layer: round the double entries to fp32, then encode."""
    return encode(entries64.astype(np.float32), fmt, rope)


# ----------------------------------------------------------------------------------------------------
# stage 2: indexer scores + top-k
# ----------------------------------------------------------------------------------------------------
def indexer_scores(qI: dict, w: np.ndarray, kI: dict, B: int, Sq: int, HI: int, DI: int, N: int, m: int,
                   q_start_pos: int, rows=None, canonical: bool = False, want_abs: bool = False,
                   want_exact: bool = False, seq_pos=None):
    """Returns (s64 [B, nrows, N], s32 or None, abs or None, inexact_count), plus the per-pair exactness
    certificate [B, nrows, N] (uint8, 1 = every head dot is exact in fp32) as a fifth item when want_exact.
    inexact_count is the number of visible (row, entry) pairs without the certificate."""
    rows = np.arange(Sq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    nr = len(rows)
    w = np.ascontiguousarray(w, np.float32)
    s64 = np.empty((B, nr, N), np.float64)
    s32 = np.empty((B, nr, N), np.float32) if canonical else None
    ab = np.empty((B, nr, N), np.float64) if want_abs else None
    ex = np.empty((B, nr, N), np.uint8) if want_exact else None
    bad = ctypes.c_longlong(0)
    q_s, k_s = _cstruct(qI), _cstruct(kI)
    sp = None if seq_pos is None else np.ascontiguousarray(seq_pos, np.int64)
    assert sp is None or sp.shape == (B,)
    lib().orc_indexer_scores(ctypes.byref(q_s), _ptr(w), ctypes.byref(k_s), B, Sq, HI, DI, N, m, q_start_pos, _ptr(sp),
                             _ptr(rows), nr, _ptr(s64), _ptr(s32), _ptr(ab), ctypes.byref(bad), _ptr(ex))
    if want_exact:
        return s64, s32, ab, int(bad.value), ex
    return s64, s32, ab, int(bad.value)


def dot_is_fp32_exact(q: np.ndarray, k: np.ndarray) -> bool:
    """The oracle's certificate that fp32 arithmetic gives sum(q * k) exactly in every summation order."""
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    assert q.shape == k.shape and q.ndim == 1
    return bool(lib().orc_dot_is_fp32_exact(_ptr(q), _ptr(k), len(q)))


def topk(scores: np.ndarray, nvis: np.ndarray, k: int):
    """scores [R, N] (float64 or float32), nvis [R] -> (idx [R, k] ascending + -1 pad, kth [R], next [R])."""
    s = np.ascontiguousarray(scores, np.float64)
    R, N = s.shape
    nv = np.ascontiguousarray(nvis, np.int32)
    idx = np.empty((R, k), np.int32)
    kth = np.empty((R,), np.float64)
    nxt = np.empty((R,), np.float64)
    lib().orc_topk_rows(_ptr(s), R, N, _ptr(nv), k, _ptr(idx), _ptr(kth), _ptr(nxt))
    return idx, kth, nxt


def nvis_rows(B: int, rows, q_start_pos: int, m: int, N: int) -> np.ndarray:
    rows = np.asarray(rows, np.int64)
    nv = np.minimum((q_start_pos + rows) // m, N)
    return np.tile(nv, B).astype(np.int32)


# ----------------------------------------------------------------------------------------------------
# stages 3/4: attention
# ----------------------------------------------------------------------------------------------------
def attn(q: dict, comp: dict, N: int, raw: dict, raw_start: int, S_raw: int, idx, k: int, hca_m: int, sink,
         B: int, Sq: int, H: int, D: int, window: int, scale: float, q_start_pos: int, rows=None, seq_pos=None):
    """Returns (o [B, nrows, H, D] float64, lse [B, nrows, H] float64)."""
    rows = np.arange(Sq, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    nr = len(rows)
    out = np.empty((B, nr, H, D), np.float64)
    lse = np.empty((B, nr, H), np.float64)
    sink = np.ascontiguousarray(sink, np.float32)
    idx_a = None if idx is None else np.ascontiguousarray(idx, np.int32)
    if hca_m == 0 and k > 0 and (idx_a is None or idx_a.size != B * Sq * k):
        raise ValueError("idx must hold [B, Sq, k] entries (row r of the call reads idx[b, r])")
    q_s, c_s, r_s = _cstruct(q), _cstruct(comp), _cstruct(raw)
    sp = None if seq_pos is None else np.ascontiguousarray(seq_pos, np.int64)
    assert sp is None or sp.shape == (B,)
    rc = lib().orc_attn(ctypes.byref(q_s), ctypes.byref(c_s), N, ctypes.byref(r_s), raw_start, S_raw, _ptr(idx_a),
                        k, hca_m, _ptr(sink), B, Sq, H, D, window, float(scale), q_start_pos, _ptr(sp), _ptr(rows), nr,
                        _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("window positions fall outside the raw KV span")
    return out, lse
