"""The C-ABI library loads, exports every symbol include/lca.h declares, and rejects bad arguments on the host
before touching a GPU.  CPU only (no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lca.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|void|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(", src,
                       flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("kv_compress", "indexer_score_topk", "sparse_mqa_attn", "hca_attn", "lca_encode",
              "indexer_score_topk_workspace_size", "sparse_mqa_attn_workspace_size", "hca_attn_workspace_size",
              "lca_status_string", "lca_set_score_events"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    from long_context_attention_05_amd import lca
    lib = lca.library()
    for n in _declared_functions():
        assert hasattr(lib, n), "liblca.so does not export %s" % n


def test_status_strings():
    from long_context_attention_05_amd import lca
    for code, name in lca.STATUS.items():
        assert lca.status_string(code).startswith(name)


def test_workspace_sizes_are_consistent():
    from long_context_attention_05_amd import lca
    assert lca.indexer_score_topk_workspace_size(16, 1, 32768, 512) >= 16 * 32768 * 4
    assert lca.sparse_mqa_attn_workspace_size(4096, 1, 64, 512, 1152) == 0  # enough rows: no split partials
    assert lca.sparse_mqa_attn_workspace_size(16, 1, 64, 512, 640) > 0
    # many rows with a list longer than one 2048-position slice: the MFMA kernels split it and need partials
    assert lca.sparse_mqa_attn_workspace_size(256, 1, 64, 512, 2116) >= 256 * 2 * 64 * 512 * 4
    assert lca.hca_attn_workspace_size(8, 1, 64, 512, 8320) > 0


def _t(fmt=1, dim=512, cap=100, data=16, rope=0, rope_p=None, scale=None, flags=0):
    from long_context_attention_05_amd import lca
    return lca.lca_tensor(fmt, dim, rope, cap, data, rope_p, scale, flags)


def test_host_validation_errors():
    """Argument errors return before any launch (fake aligned/unaligned addresses are never dereferenced)."""
    from long_context_attention_05_amd import lca
    L = lca.library()
    P = 1 << 20  # a fake, 16-byte aligned device address: validation never touches it
    INV, UNS, WS, ALN = -1, -2, -3, -4
    # kv_compress: start_pos not a multiple of m, missing tail, c mismatch, misaligned output
    args = [P] * 8
    assert L.kv_compress(*args, 1, 8, 512, 4, 1, 6, None, None, _t(), None) == INV
    assert L.kv_compress(P, P, P, P, P, P, None, None, 1, 8, 512, 4, 1, 8, None, None, _t(), None) == INV
    assert L.kv_compress(*args, 1, 8, 256, 4, 1, 0, None, None, _t(), None) == INV
    assert L.kv_compress(*args, 1, 8, 512, 4, 1, 0, None, None, _t(data=P + 4), None) == ALN
    assert L.kv_compress(*args, 1, 8, 512, 4, 1, 0, None, None, _t(cap=1), None) == INV  # rows beyond cap
    assert L.kv_compress(*args, 1, 8, 2048, 4, 1, 0, None, None, _t(dim=2048), None) == UNS
    # entry epilogues: odd or oversized rotary span, non-positive base, negative eps, misaligned gains
    E = lca.lca_epilogue
    for epi, want in ((E(None, 0.0, 3, 10000.0), INV), (E(None, 0.0, 514, 10000.0), INV), (E(None, 0.0, 64, 0.0), INV),
                      (E(P, -1.0, 0, 0.0), INV), (E(P + 2, 1e-6, 0, 0.0), ALN)):
        assert L.kv_compress(*args, 1, 8, 512, 4, 1, 0, ctypes.byref(epi), None, _t(), None) == want
    # lca_encode: fp4 dim not a multiple of 16, mixed without rope pointer
    assert L.lca_encode(P, 1, 4, 0, _t(fmt=3, dim=24, scale=P), None) == INV
    assert L.lca_encode(P, 1, 4, 0, _t(fmt=2, rope=64), None) == INV
    # the Hadamard rotation flag: a power-of-two dim, not the mixed format, no unknown bits (readers included)
    assert L.lca_encode(P, 1, 4, 0, _t(dim=96, data=P, flags=1), None) == INV
    assert L.lca_encode(P, 1, 4, 0, _t(fmt=2, rope=64, data=P, rope_p=P, scale=P, flags=1), None) == INV
    assert L.lca_encode(P, 1, 4, 0, _t(data=P, flags=2), None) == INV
    assert L.kv_compress(*([P] * 8), 1, 8, 384, 4, 1, 0, None, None, _t(dim=384, data=P, flags=1), None) == INV
    # indexer: workspace too small, HI too large, fp4 keys with bf16 queries
    q = _t(dim=128, cap=64)
    k = _t(dim=128, cap=1000)
    assert L.indexer_score_topk(q, P, k, 1, 1, 64, 128, 1000, 4, 64, 4000, P, None, P, 16, None, None) == WS
    assert L.indexer_score_topk(_t(dim=128, cap=128), P, k, 1, 1, 128, 128, 1000, 4, 64, 4000, P, None, P, 1 << 30, None,
                                None) == UNS
    assert L.indexer_score_topk(q, P, _t(fmt=3, dim=128, cap=1000, scale=P), 1, 1, 64, 128, 1000, 4, 64, 4000, P, None,
                                P, 1 << 30, None, None) == UNS
    assert L.indexer_score_topk(q, None, k, 1, 1, 64, 128, 1000, 4, 64, 4000, P, None, P, 1 << 30, None, None) == INV
    # the workspace is read and written 16 bytes at a time
    assert L.indexer_score_topk(q, P, k, 1, 1, 64, 128, 1000, 4, 64, 4000, P, None, P + 4, 1 << 30, None, None) == ALN
    # the query tensor must hold exactly Sq * HI rows per sequence (the kernels address rows (b * Sq + r) * HI + h)
    assert L.indexer_score_topk(_t(dim=128, cap=65), P, k, 2, 1, 64, 128, 1000, 4, 64, 4000, P, None, P, 1 << 30, None,
                                None) == INV
    assert L.indexer_score_topk(_t(dim=128, cap=128), P, k, 2, 2, 64, 128, 1000, 4, 64, 4000, P, None, P, 16, None,
                                None) == WS  # cap = Sq * HI passes (the next check, the workspace, fails)
    # DI beyond 128 has no kernel (fp4 rows of 160 dims are otherwise valid)
    assert L.indexer_score_topk(_t(fmt=3, dim=160, cap=64, scale=P), P, _t(fmt=3, dim=160, cap=1000, scale=P), 1, 1,
                                64, 160, 1000, 4, 64, 4000, P, None, P, 1 << 30, None, None) == UNS
    # fp4 rows are whole 32-element scale blocks
    assert L.indexer_score_topk(_t(fmt=3, dim=112, cap=64, scale=P), P, _t(fmt=3, dim=112, cap=1000, scale=P), 1, 1,
                                64, 112, 1000, 4, 64, 4000, P, None, P, 1 << 30, None, None) == INV
    assert L.indexer_score_topk(q, P, _t(dim=128, cap=1000, flags=8), 1, 1, 64, 128, 1000, 4, 64, 4000, P, None, P,
                                1 << 30, None, None) == INV
    # attention: window outside the raw span, workspace missing for a split plan, bad formats
    comp = _t(cap=5000)
    raw = _t(cap=128)
    f = ctypes.c_float(1.0)
    assert L.sparse_mqa_attn(P, 1, comp, 5000, raw, 100, 128, P, 512, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, None,
                             0, None, None) == INV
    assert L.sparse_mqa_attn(P, 1, comp, 5000, raw, 373, 128, P, 512, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, None,
                             0, None, None) == WS
    assert L.sparse_mqa_attn(P, 7, comp, 5000, raw, 373, 128, P, 512, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, P,
                             1 << 30, None, None) == INV
    # a split plan's workspace takes 16-byte partial stores
    assert L.sparse_mqa_attn(P, 1, comp, 5000, raw, 373, 128, P, 512, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, P + 8,
                             1 << 30, None, None) == ALN
    assert L.hca_attn(P, 1, comp, 5000, 0, raw, 373, 128, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, P, 1 << 30, None,
                      None) == INV
    # the float path (fp32 queries or caches) covers H * D <= 8192 only: 64 heads x 512 channels in fp32 has no kernel
    assert L.sparse_mqa_attn(P, 0, comp, 5000, raw, 373, 128, P, 512, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, P,
                             1 << 30, None, None) == UNS
    assert L.sparse_mqa_attn(P, 0, _t(fmt=0, dim=144, cap=5000), 5000, _t(fmt=0, dim=144, cap=128), 373, 128, P, 512,
                             P, 2, 1, 64, 144, 128, f, 500, P, 1, None, P, 1 << 30, None, None) == UNS


def test_paged_and_ragged_validation():
    """Paged tensors: block_rows a power of two dividing cap, a pool of whole blocks under 2^31 rows, an aligned
    table; only compressed caches and keys may be paged; the decode scorers need blocks of 32 rows or more.  Ragged
    position arrays must be 8-byte aligned."""
    from long_context_attention_05_amd import lca
    L = lca.library()
    P = 1 << 20
    INV, UNS, WS, ALN = -1, -2, -3, -4

    def pg(br=32, cap=1024, pool=4096, table=P, fmt=1, dim=128, scale=None):
        t = _t(fmt=fmt, dim=dim, cap=cap, scale=scale)
        t.block_table, t.block_rows, t.pool_rows = table, br, pool
        return t

    q = _t(dim=128, cap=64)
    call = lambda k, ws=16: L.indexer_score_topk(q, P, k, 1, 1, 64, 128, 1000, 4, 64, 4000, P, None, P, ws, None,  # noqa
                                                  None)
    assert call(pg()) == WS  # a valid paged tensor passes validation (then the workspace check fails)
    assert call(pg(br=24)) == INV
    assert call(pg(cap=1000)) == INV
    assert call(pg(pool=4001)) == INV
    assert call(pg(pool=1 << 31)) == INV
    assert call(pg(table=P + 2)) == ALN
    assert call(pg(br=16), ws=1 << 30) == UNS
    assert call(pg(fmt=3, pool=1 << 26, scale=P), ws=1 << 30) == UNS  # fp4 pool of 2 GiB of codes
    # a paged query tensor or raw window is refused
    qp = pg(cap=64, pool=64)
    assert L.indexer_score_topk(qp, P, _t(dim=128, cap=1000), 1, 1, 64, 128, 1000, 4, 64, 4000, P, None, P, 16, None,
                                None) == INV
    f = ctypes.c_float(1.0)
    comp, raw = _t(cap=5000), _t(cap=128)
    rawp = _t(cap=128)
    rawp.block_table, rawp.block_rows, rawp.pool_rows = P, 32, 128
    assert L.sparse_mqa_attn(P, 1, comp, 5000, rawp, 373, 128, P, 512, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, P,
                             16, None, None) == INV
    # ragged positions must be aligned
    rg = lca.lca_ragged(P + 4, None)
    assert L.sparse_mqa_attn(P, 1, comp, 5000, raw, 373, 128, P, 512, P, 2, 1, 64, 512, 128, f, 500, P, 1, None, P,
                             16, ctypes.byref(rg), None) == ALN
    assert L.kv_compress(*([P] * 8), 1, 8, 512, 4, 1, 0, None, ctypes.byref(lca.lca_ragged(P, P + 2)), _t(), None) \
        == ALN


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The Python binding raises when liblca.so is absent: there is no CPU fallback."""
    import importlib.util
    src = os.path.join(ROOT, "long_context_attention_05_amd", "lca.py")
    dst = tmp_path / "lca.py"
    dst.write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("lca_copy", str(dst))
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


def test_descriptor_layout_matches_header(tmp_path):
    """The binding's lca_tensor has the header's size and field offsets (compiled against include/lca.h)."""
    import subprocess
    from long_context_attention_05_amd import lca
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "lca.h"\nint main(void) {\n'
                   '  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(lca_tensor), offsetof(lca_tensor, format),\n'
                   '         offsetof(lca_tensor, dim), offsetof(lca_tensor, rope_dims), offsetof(lca_tensor, cap),\n'
                   '         offsetof(lca_tensor, data), offsetof(lca_tensor, rope), offsetof(lca_tensor, scale),\n'
                   '         offsetof(lca_tensor, flags));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.check_call(["gcc", "-std=c11", "-I", inc, "-x", "c", str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    T = lca.lca_tensor
    want = [ctypes.sizeof(T)] + [getattr(T, f).offset for f in
                                 ("format", "dim", "rope_dims", "cap", "data", "rope", "scale", "flags")]
    assert got == want
    assert lca.LCA_ROTATE_HADAMARD == 1


def test_binding_loads_torch_before_the_library():
    """Importing the package first must not bring in a second HIP runtime: the binding imports torch, and does so
    before it loads liblca.so."""
    import subprocess
    import sys
    code = ("import sys\n"
            "assert 'torch' not in sys.modules\n"
            "import long_context_attention_05_amd\n"
            "assert 'torch' in sys.modules\n")
    subprocess.check_call([sys.executable, "-c", code], cwd=ROOT)
    src = open(os.path.join(ROOT, "long_context_attention_05_amd", "lca.py")).read()
    assert 0 <= src.index("\nimport torch") < src.index("ctypes.CDLL(")


def test_descriptors_keep_their_tensors_alive():
    """The ragged and epilogue descriptors hold the tensors they point at: a temporary passed to them must not be
    freed (and its memory reused) before the asynchronous calls read it."""
    import gc
    import weakref

    import torch
    from long_context_attention_05_amd import lca
    t = torch.zeros(4, dtype=torch.int64)
    g = torch.ones(8, dtype=torch.float32)
    refs = (weakref.ref(t), weakref.ref(g))
    r, e = lca.ragged(t), lca.epilogue(g, 1e-6, 0, 0.0)
    del t, g
    gc.collect()
    assert all(x() is not None for x in refs)
    assert r.pos == refs[0]().data_ptr() and e.norm_weight == refs[1]().data_ptr()
