"""ctypes binding of liblca.so (include/lca.h).

Argument marshalling only: every step runs in the HIP kernels of liblca.so.  Torch tensors supply device memory
and the current stream.  If the library is not built, importing this module raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblca.so")

LCA_F32, LCA_BF16, LCA_MIXED_FP8, LCA_FP4 = 0, 1, 2, 3
LCA_ROTATE_HADAMARD = 1  # lca_tensor.flags: rows are stored Hadamard-rotated (writers rotate before encoding)
FORMATS = {"f32": LCA_F32, "bf16": LCA_BF16, "mixed": LCA_MIXED_FP8, "fp4": LCA_FP4}
STATUS = {0: "LCA_OK", -1: "LCA_ERR_INVALID_ARG", -2: "LCA_ERR_UNSUPPORTED", -3: "LCA_ERR_WORKSPACE",
          -4: "LCA_ERR_ALIGNMENT", -5: "LCA_ERR_HIP"}


class LcaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = "%s failed: %s" % (fn, STATUS.get(status, status))
        if status == -5:
            msg += " (%s)" % _lib.lca_last_hip_error().decode()
        super().__init__(msg)
        self.status = status


class lca_tensor(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int), ("dim", ctypes.c_int), ("rope_dims", ctypes.c_int),
                ("cap", ctypes.c_longlong), ("data", ctypes.c_void_p), ("rope", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("flags", ctypes.c_int), ("block_table", ctypes.c_void_p),
                ("block_rows", ctypes.c_int), ("pool_rows", ctypes.c_longlong)]


class lca_ragged(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_void_p), ("len", ctypes.c_void_p)]


class lca_epilogue(ctypes.Structure):
    _fields_ = [("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("rope_dims", ctypes.c_int),
                ("rope_base", ctypes.c_float)]


if not os.path.exists(LIB_PATH):
    raise ImportError("liblca.so is not built (run long_context_attention_05_amd/build.py); no fallback exists")
# torch first: liblca.so then binds to the HIP runtime torch has already loaded, so the library's launches run in
# the runtime that owns torch's device memory and streams (loading the library first brings in a second runtime,
# whose calls then find no device)
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_longlong
_F = ctypes.c_float
_S = ctypes.c_size_t

_lib.lca_status_string.argtypes = [_I]
_lib.lca_status_string.restype = ctypes.c_char_p
_lib.lca_last_hip_error.argtypes = []
_lib.lca_last_hip_error.restype = ctypes.c_char_p
_lib.lca_encode.argtypes = [_P, _I, _L, _L, lca_tensor, _P]
_lib.lca_stream_read.argtypes = [_P, _S, _P, _I, _P]
_RG = ctypes.POINTER(lca_ragged)
_lib.kv_compress.argtypes = [_P] * 8 + [_I, _L, _I, _I, _I, _L, ctypes.POINTER(lca_epilogue), _RG, lca_tensor, _P]
_lib.indexer_score_topk_workspace_size.argtypes = [_I, _I, _I, _I]
_lib.indexer_score_topk_workspace_size.restype = _S
_lib.indexer_score_topk.argtypes = [lca_tensor, _P, lca_tensor] + [_I] * 7 + [_L, _P, _P, _P, _S, _RG, _P]
_lib.indexer_score_topk_noalloc.argtypes = [lca_tensor, _P, lca_tensor] + [_I] * 7 + [_L, _P, _P, _RG, _P]
_lib.lca_set_score_events.argtypes = [_P, _P]
_lib.lca_set_score_events.restype = None
_lib.lca_set_attn_events.argtypes = [_P, _P]
_lib.lca_set_attn_events.restype = None
_lib.sparse_mqa_attn_workspace_size.argtypes = [_I] * 5
_lib.sparse_mqa_attn_workspace_size.restype = _S
_lib.sparse_mqa_attn.argtypes = [_P, _I, lca_tensor, _I, lca_tensor, _L, _I, _P, _I, _P] + [_I] * 5 + [
    _F, _L, _P, _I, _P, _P, _S, _RG, _P]
_lib.hca_attn_workspace_size.argtypes = [_I] * 5
_lib.hca_attn_workspace_size.restype = _S
_lib.hca_attn.argtypes = [_P, _I, lca_tensor, _I, _I, lca_tensor, _L, _I, _P] + [_I] * 5 + [
    _F, _L, _P, _I, _P, _P, _S, _RG, _P]


def library():
    return _lib


def status_string(status: int) -> str:
    return _lib.lca_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int):
    if rc != 0:
        raise LcaError(fn, rc)


class CacheTensor:
    """Device storage of one lca_tensor (owns its torch tensors): `cap` rows per sequence for B sequences."""

    def __init__(self, fmt: str, B: int, cap: int, dim: int, rope: int = 0, device="cuda", flags: int = 0):
        import torch
        self.fmt, self.B, self.cap, self.dim, self.rope, self.flags = fmt, B, cap, dim, rope, flags
        rows = B * cap
        self.rope_t = self.scale_t = None
        if fmt == "f32":
            self.data = torch.empty((rows, dim), dtype=torch.float32, device=device)
        elif fmt == "bf16":
            self.data = torch.empty((rows, dim), dtype=torch.int16, device=device)
        elif fmt == "mixed":
            self.data = torch.empty((rows, dim - rope), dtype=torch.uint8, device=device)
            self.rope_t = torch.empty((rows, rope), dtype=torch.int16, device=device)
            self.scale_t = torch.empty((rows,), dtype=torch.float32, device=device)
        elif fmt == "fp4":
            self.data = torch.empty((rows, dim // 2), dtype=torch.uint8, device=device)
            self.scale_t = torch.empty((rows, dim // 32), dtype=torch.uint8, device=device)
        else:
            raise ValueError(fmt)

    def desc(self) -> lca_tensor:
        return lca_tensor(FORMATS[self.fmt], self.dim, self.rope, self.cap, _ptr(self.data), _ptr(self.rope_t),
                          _ptr(self.scale_t), self.flags)


    def host(self) -> dict:
        """Copy to host numpy arrays (for comparisons), as a dict of raw storage arrays."""
        import numpy as np
        d = dict(fmt=self.fmt, dim=self.dim, rope=self.rope, cap=self.cap)
        d["data"] = self.data.cpu().numpy()
        if self.fmt == "bf16":
            d["data"] = d["data"].view(np.uint16)
        d["rope_data"] = None if self.rope_t is None else self.rope_t.cpu().numpy().view(np.uint16)
        d["scale"] = None if self.scale_t is None else self.scale_t.cpu().numpy()
        return d


class PagedCache(CacheTensor):
    """A paged tensor: a pool of `pool_blocks` blocks of `block_rows` rows and a device block table [B][cap /
    block_rows] (int32) mapping each sequence's logical blocks to pool blocks."""

    def __init__(self, fmt: str, B: int, cap: int, dim: int, rope: int, block_rows: int, table, pool_blocks: int,
                 device="cuda", flags: int = 0):
        assert cap % block_rows == 0
        super().__init__(fmt, 1, pool_blocks * block_rows, dim, rope, device, flags)
        self.B, self.cap, self.block_rows, self.pool_rows = B, cap, block_rows, pool_blocks * block_rows
        self.table = table  # device int32 tensor [B, cap / block_rows]
        assert tuple(table.shape) == (B, cap // block_rows)

    def desc(self) -> lca_tensor:
        d = super().desc()
        d.cap = self.cap
        d.block_table = _ptr(self.table)
        d.block_rows = self.block_rows
        d.pool_rows = self.pool_rows
        return d


def plain_desc(t, fmt: str, dim: int, cap: int) -> lca_tensor:
    """Descriptor over an existing dense f32/bf16 tensor (rows = B * cap)."""
    return lca_tensor(FORMATS[fmt], dim, 0, cap, _ptr(t), None, None)


# ----------------------------------------------------------------------------------------------------
# entry points (names as in include/lca.h)
# ----------------------------------------------------------------------------------------------------
def lca_stream_read(src, nbytes: int, out, workgroups: int, stream=None):
    """Measurement helper: one streaming read of `nbytes` at src (see include/lca.h)."""
    _check("lca_stream_read", _lib.lca_stream_read(_ptr(src), nbytes, _ptr(out), workgroups, _stream(stream)))


def lca_encode(src, B: int, rows: int, row0: int, dst: lca_tensor, stream=None):
    _check("lca_encode", _lib.lca_encode(_ptr(src), B, rows, row0, dst, _stream(stream)))


def epilogue(norm_weight=None, norm_eps: float = 0.0, rope_dims: int = 0, rope_base: float = 0.0) -> lca_epilogue:
    """kv_compress's entry epilogues (norm_weight: a device float tensor [c] or None, referenced by the descriptor
    so that it outlives the asynchronous calls)."""
    e = lca_epilogue(_ptr(norm_weight), norm_eps, rope_dims, rope_base)
    e._tensors = (norm_weight,)
    return e


def ragged(pos, lens=None) -> lca_ragged:
    """Per-sequence positions (device int64 tensor [B]) and, for kv_compress, token counts (device int32 [B]).  The
    descriptor holds references to both tensors, so that they outlive the calls that read them asynchronously."""
    r = lca_ragged(_ptr(pos), _ptr(lens))
    r._tensors = (pos, lens)
    return r


def _rg(r):
    return None if r is None else ctypes.byref(r)


def kv_compress(Ca, Cb, Za, Zb, Ba, Bb, tail_Cb, tail_Zb, B: int, n: int, c: int, m: int, overlap: bool,
                start_pos: int, out: lca_tensor, stream=None, epi: lca_epilogue | None = None,
                ragged: lca_ragged | None = None):
    _check("kv_compress", _lib.kv_compress(_ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), _ptr(Ba), _ptr(Bb), _ptr(tail_Cb),
                                           _ptr(tail_Zb), B, n, c, m, int(bool(overlap)), start_pos,
                                           None if epi is None else ctypes.byref(epi), _rg(ragged), out,
                                           _stream(stream)))


def indexer_score_topk_workspace_size(B: int, Sq: int, N: int, k: int) -> int:
    return int(_lib.indexer_score_topk_workspace_size(B, Sq, N, k))


def lca_set_score_events(ev_begin, ev_end):
    """hipEvent_t handles (ints) stamped with the indexer scoring kernel's start and end; None, None to stop."""
    _lib.lca_set_score_events(ev_begin, ev_end)


def lca_set_attn_events(ev_begin, ev_end):
    """hipEvent_t handles (ints) stamped with the attention kernels' start and end (not the split merge); None, None
    to stop."""
    _lib.lca_set_attn_events(ev_begin, ev_end)


def indexer_score_topk(qI: lca_tensor, w, kI: lca_tensor, B: int, Sq: int, HI: int, DI: int, N: int, m: int, k: int,
                       q_start_pos: int, idx_out, score_out, ws, ws_bytes: int, stream=None,
                       ragged: lca_ragged | None = None):
    _check("indexer_score_topk", _lib.indexer_score_topk(qI, _ptr(w), kI, B, Sq, HI, DI, N, m, k, q_start_pos,
                                                         _ptr(idx_out), _ptr(score_out), _ptr(ws), ws_bytes,
                                                         _rg(ragged), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # LCA_NOALLOC_SCRATCH_BYTES


def indexer_score_topk_noalloc(qI: lca_tensor, w, kI: lca_tensor, B: int, Sq: int, HI: int, DI: int, N: int, m: int,
                               k: int, q_start_pos: int, idx_out, score_out, stream=None,
                               ragged: lca_ragged | None = None):
    _check("indexer_score_topk_noalloc",
           _lib.indexer_score_topk_noalloc(qI, _ptr(w), kI, B, Sq, HI, DI, N, m, k, q_start_pos, _ptr(idx_out),
                                           _ptr(score_out), _rg(ragged), _stream(stream)))


def sparse_mqa_attn_workspace_size(B: int, Sq: int, H: int, D: int, max_entries: int) -> int:
    return int(_lib.sparse_mqa_attn_workspace_size(B, Sq, H, D, max_entries))


def sparse_mqa_attn(q, q_format: int, kv_comp: lca_tensor, N: int, kv_raw: lca_tensor, raw_start_pos: int, S_raw: int,
                    idx, k: int, sink, B: int, Sq: int, H: int, D: int, window: int, scale: float, q_start_pos: int,
                    out, out_format: int, lse_out, ws, ws_bytes: int, stream=None,
                    ragged: lca_ragged | None = None):
    _check("sparse_mqa_attn", _lib.sparse_mqa_attn(_ptr(q), q_format, kv_comp, N, kv_raw, raw_start_pos, S_raw,
                                                   _ptr(idx), k, _ptr(sink), B, Sq, H, D, window, scale, q_start_pos,
                                                   _ptr(out), out_format, _ptr(lse_out), _ptr(ws), ws_bytes,
                                                   _rg(ragged), _stream(stream)))


def hca_attn_workspace_size(B: int, Sq: int, H: int, D: int, max_entries: int) -> int:
    return int(_lib.hca_attn_workspace_size(B, Sq, H, D, max_entries))


def hca_attn(q, q_format: int, kv_comp: lca_tensor, N: int, m: int, kv_raw: lca_tensor, raw_start_pos: int, S_raw: int,
             sink, B: int, Sq: int, H: int, D: int, window: int, scale: float, q_start_pos: int, out, out_format: int,
             lse_out, ws, ws_bytes: int, stream=None, ragged: lca_ragged | None = None):
    _check("hca_attn", _lib.hca_attn(_ptr(q), q_format, kv_comp, N, m, kv_raw, raw_start_pos, S_raw, _ptr(sink), B, Sq,
                                     H, D, window, scale, q_start_pos, _ptr(out), out_format, _ptr(lse_out), _ptr(ws),
                                     ws_bytes, _rg(ragged), _stream(stream)))
