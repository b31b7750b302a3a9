"""Stage-isolated GPU parity: each C-ABI call against the CPU oracle on the same seeded inputs, at sizes that span
several tiles, a ragged tail and the edge cases (empty, fully visible, padding, ties)."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from tests.gpu_util import (bf16_to_f64, check_bf16_codes, check_fp4_codes, check_mixed_codes, check_topk, gpu_bf16,
                            gpu_encode, gpu_f32, row_rel_err, up, ws)
import lca_inputs as gen

pytestmark = pytest.mark.gpu

lca = pytest.importorskip("long_context_attention_05_amd.lca")


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------------------------------
# codec: quantise-on-write is bit-exact against the oracle's codec
# ------------------------------------------------------------------------------------------------------
def _codec_input(g, B, rows, dim):
    x = g.standard_normal((B, rows, dim)).astype(np.float32)
    x[0, 0] = 0.0
    x[0, 1] *= np.float32(1e-30)
    x[0, 2] *= np.float32(1e30)
    # rows whose fp8 scale is exactly 1 (amax 448) carrying e4m3 midpoints, and fp4 groups with amax 6 + ties
    mids = np.array([0.0009765625 * 1.5, 0.015625 * 1.0625, 1.0625, 1.1875, 3.25, 17.0, 104.0, 416.0], np.float32)
    x[0, 3, :] = 0.0
    x[0, 3, 0] = 448.0
    x[0, 3, 1:1 + len(mids)] = mids
    x[0, 3, 10:10 + len(mids)] = -mids
    ties = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -5.0, 0.1, -0.0, 4.0, 3.0, 1.0, 0.5], np.float32)
    x[0, 4, :16] = ties
    return x


@pytest.mark.parametrize("fmt,dim,rope", [("bf16", 512, 0), ("mixed", 512, 64), ("fp4", 128, 0), ("f32", 64, 0),
                                          ("fp4", 32, 0), ("mixed", 96, 32)])
def test_encode_bit_exact(fmt, dim, rope):
    x = _codec_input(_rng(1), 2, 333, dim)
    got = gpu_encode(x, fmt, rope).host()
    ref = orc.encode(x.reshape(-1, dim), fmt, rope)
    np.testing.assert_array_equal(got["data"].view(np.uint8), ref["data"].view(np.uint8))
    if ref["scale"] is not None:
        np.testing.assert_array_equal(got["scale"].view(np.uint8), ref["scale"].view(np.uint8))
    if ref["rope_data"] is not None:
        np.testing.assert_array_equal(got["rope_data"], ref["rope_data"])


# ------------------------------------------------------------------------------------------------------
# stage 1: compression
# ------------------------------------------------------------------------------------------------------
def _streams(g, B, n, c, m):
    f = lambda *s: g.standard_normal(s).astype(np.float32)
    return dict(Ca=f(B, n, c), Cb=f(B, n, c), Za=f(B, n, c), Zb=f(B, n, c), Ba=(0.1 * f(m, c)).astype(np.float32),
                Bb=(0.1 * f(m, c)).astype(np.float32), tail_Cb=f(B, m, c), tail_Zb=f(B, m, c))


def _gpu_compress(s, B, n, c, m, overlap, start, fmt, rope=0, cap=None):
    nb = (n + m - 1) // m
    cap = start // m + nb if cap is None else cap
    out = lca.CacheTensor(fmt, B, cap, c, rope)
    d = {k: up(v) for k, v in s.items()}
    lca.kv_compress(d["Ca"], d["Cb"] if overlap else None, d["Za"], d["Zb"] if overlap else None, d["Ba"],
                    d["Bb"] if overlap else None, d["tail_Cb"] if (overlap and start) else None,
                    d["tail_Zb"] if (overlap and start) else None, B, n, c, m, overlap, start, out.desc())
    return out


def _oracle_compress(s, m, overlap, start):
    return orc.kv_compress(s["Ca"], s["Cb"], s["Za"], s["Zb"], s["Ba"], s["Bb"], s["tail_Cb"], s["tail_Zb"], m=m,
                           overlap=overlap, start_pos=start)


@pytest.mark.parametrize("B,n,c,m,overlap,start", [(1, 1024, 64, 4, True, 0), (1, 1024, 32, 4, True, 0),
                                                   (2, 1027, 512, 4, True, 64), (3, 5, 128, 4, True, 131072),
                                                   (2, 128 * 5 + 17, 512, 128, False, 0), (2, 1, 512, 128, False, 1 << 20)])
def test_compress_f32_matches_oracle(B, n, c, m, overlap, start):
    s = _streams(_rng(2), B, n, c, m)
    nb = (n + m - 1) // m
    got = _gpu_compress(s, B, n, c, m, overlap, start, "f32").data.view(B, -1, c).cpu().numpy()[:, start // m:]
    ref = _oracle_compress(s, m, overlap, start)
    assert got.shape == ref.shape == (B, nb, c)
    assert row_rel_err(got, ref) <= 1e-4


@pytest.mark.parametrize("fmt,c,rope", [("bf16", 512, 0), ("mixed", 512, 64), ("fp4", 128, 0)])
def test_compress_quantised_outputs(fmt, c, rope):
    B, n, m = 2, 4100, 4
    s = _streams(_rng(3), B, n, c, m)
    got = _gpu_compress(s, B, n, c, m, True, 64, fmt, rope).host()
    E = _oracle_compress(s, m, True, 64)
    nb = E.shape[1]
    sl = lambda a: a.reshape(B, -1, *a.shape[1:])[:, 16:16 + nb].reshape(B * nb, *a.shape[1:])  # noqa: E731
    x = E.reshape(B * nb, c)
    # the codes are decisions taken on fp32 entries that differ from the exact ones by a few ulps: each differing code
    # is one grid step from the oracle's, next to the rounding midpoint (scale and RoPE bytes included)
    if fmt == "bf16":
        n_diff = check_bf16_codes(sl(got["data"]), x)
    elif fmt == "mixed":
        n_diff = check_mixed_codes(dict(data=sl(got["data"]), rope_data=sl(got["rope_data"]), scale=sl(got["scale"])),
                                   x, rope)
    else:
        n_diff = check_fp4_codes(dict(data=sl(got["data"]), scale=sl(got["scale"])), x)
    assert n_diff <= 0.005 * x.size


# ------------------------------------------------------------------------------------------------------
# stage 2: indexer scores + exact top-k
# ------------------------------------------------------------------------------------------------------
def _indexer_case(B, Sq, HI, DI, N, m, k, q_start, fmt, seed, dyadic=False, dup_rows=False, zero_q=False,
                  cluster=0.0, w_off=0):
    g = _rng(seed)
    if zero_q:  # every score is exactly 0: the selection is the first k visible entries
        q = np.zeros((B, Sq, HI, DI), np.float32)
        K = g.standard_normal((B, N, DI)).astype(np.float32)
        w = g.standard_normal((B, Sq, HI)).astype(np.float32)
    elif dyadic:
        q = (g.integers(-3, 4, (B, Sq, HI, DI)) * 0.5).astype(np.float32)
        K = (g.integers(-3, 4, (B, N, DI)) * 0.25).astype(np.float32)
        w = (g.integers(-4, 5, (B, Sq, HI)) * 0.0625).astype(np.float32)
    else:
        q = g.standard_normal((B, Sq, HI, DI)).astype(np.float32)
        K = g.standard_normal((B, N, DI)).astype(np.float32)
        w = (g.standard_normal((B, Sq, HI)) / math.sqrt(HI * DI)).astype(np.float32)
    if dup_rows:
        K[:, 1::3] = K[:, 0:-1:3][:, :K[:, 1::3].shape[1]]
    if cluster:  # the first 4096 keys scaled by a power of two: the high scores crowd into the first slice
        K[:, :4096] *= cluster
    capk = N + 7
    if fmt == "fp4":
        kg = gpu_encode(K, "fp4", cap=capk)
        qg = gpu_encode(q.reshape(B, Sq * HI, DI), "fp4")
        kr = orc.encode(K.reshape(-1, DI), "fp4")
        qr = orc.encode(q.reshape(-1, DI), "fp4")
        hk = kg.host()
        np.testing.assert_array_equal(hk["data"].reshape(B, capk, -1)[:, :N].reshape(-1, DI // 2), kr["data"])
        kr["cap"] = N
    elif fmt == "bf16":
        kb, qb = gen.bf16_bits(K), gen.bf16_bits(q)
        kg, qg = gpu_bf16(kb, cap=capk), gpu_bf16(qb.reshape(B, Sq * HI, DI))
        kr, qr = orc.plain_cache(kb, "bf16"), orc.plain_cache(qb, "bf16")
        kr["cap"] = N
    else:
        kg, qg = gpu_f32(K, cap=capk), gpu_f32(q.reshape(B, Sq * HI, DI))
        kr, qr = orc.plain_cache(K, "f32"), orc.plain_cache(q, "f32")
        kr["cap"] = N
    wd = up(w)
    if w_off:  # the weights w_off floats past a 16-byte boundary (the API asks only for 4-byte alignment)
        buf = torch.zeros(wd.numel() + w_off, dtype=torch.float32, device="cuda")
        buf[w_off:] = wd.reshape(-1)
        wd = buf[w_off:]
        assert wd.data_ptr() % 16 == 4 * w_off
    idx = torch.empty((B, Sq, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Sq, k), dtype=torch.float32, device="cuda")
    nbytes = lca.indexer_score_topk_workspace_size(B, Sq, N, k)
    w_s = ws(nbytes)
    lca.indexer_score_topk(qg.desc(), wd, kg.desc(), B, Sq, HI, DI, N, m, k, q_start, idx, sc, w_s, nbytes)
    torch.cuda.synchronize()
    exact = fmt == "fp4" or dyadic or zero_q
    s64, s32, ab, bad = orc.indexer_scores(qr, w, kr, B, Sq, HI, DI, N, m, q_start, canonical=exact, want_abs=True)
    if exact:
        assert bad == 0, "per-head dots not exact in fp32: the exact comparison does not apply"
    nv = orc.nvis_rows(B, np.arange(Sq), q_start, m, N)
    gamma = 2.0 * (DI + HI) * 2.0 ** -24
    st = check_topk(idx.cpu().numpy().reshape(B * Sq, k), sc.cpu().numpy().reshape(B * Sq, k),
                    s64.reshape(B * Sq, N), ab.reshape(B * Sq, N), nv, k, gamma, exact=exact,
                    s32=None if s32 is None else s32.reshape(B * Sq, N))
    st["s64"], st["nvis"] = s64.reshape(B * Sq, N), nv
    return st


def test_indexer_simt_f32_prefill():
    st = _indexer_case(1, 1024, 4, 32, 256, 4, 32, 0, "f32", 10)
    assert st["exact_rows"] >= st["rows"] * 0.98


@pytest.mark.parametrize("B,N,k", [(3, 2037, 512), (2, 700, 1024), (1, 40000, 1024), (2, 100, 512), (16, 16411, 512)])
def test_indexer_mfma_bf16_decode(B, N, k):
    st = _indexer_case(B, 1, 64, 128, N, 4, k, 4 * N + 3, "bf16", 11)
    assert st["exact_rows"] >= st["rows"] - 1


def test_indexer_mfma_bf16_prefill_causal():
    # rows t = 2240 .. 2279 see 560 .. 569 entries; k = 64; and a chunk at the start where rows see < k entries
    st = _indexer_case(1, 40, 64, 128, 600, 4, 64, 2240, "bf16", 12)
    assert st["exact_rows"] >= st["rows"] - 1
    _indexer_case(2, 37, 64, 128, 600, 4, 8, 0, "bf16", 13)


@pytest.mark.parametrize("B,Sq,N,k,HI,DI", [(2, 1, 3000, 1024, 64, 128), (1, 3, 40000, 1024, 64, 128),
                                             (2, 2, 500, 64, 16, 64), (8, 1, 65613, 1024, 64, 128),
                                             (2, 2, 500, 64, 40, 64), (1, 1, 700, 128, 32, 64)])
def test_indexer_fp4_bit_exact(B, Sq, N, k, HI, DI):
    # (other than 64 x 128 the vector-ALU kernel scores: 40 heads pad to 64, so its fused chains run over four heads
    # with padding; 32 heads give chains of two)
    _indexer_case(B, Sq, HI, DI, N, 4, k, 4 * N, "fp4", 14)


@pytest.mark.parametrize("B,Sq,N,k,q_off,fmt", [(3, 2, 2037, 512, -1, "bf16"), (2, 4, 16411, 512, -2, "bf16"),
                                                (2, 4, 3001, 1024, -3, "fp4"), (1, 2, 70000, 1024, -1, "fp4"),
                                                (4, 3, 8200, 512, 0, "bf16"), (1, 4, 40000, 512, -3, "bf16")])
def test_indexer_decode_multi_row(B, Sq, N, k, q_off, fmt):
    # several query rows per sequence (draft tokens verified together) share the decode kernels, which score an even
    # number of rows two to a workgroup; with q_start just below a multiple of m the rows see N - 1 and N entries
    # (four bf16 rows over 40000 entries: two row pairs, the second one's rows seeing different entry counts)
    st = _indexer_case(B, Sq, 64, 128, N, 4, k, 4 * N + q_off, fmt, 20 + Sq)
    if fmt == "bf16":
        assert st["exact_rows"] >= st["rows"] - 1


@pytest.mark.parametrize("fmt", ["bf16", "fp4"])
def test_indexer_decode_multi_row_short(fmt):
    # rows on either side of k (511 and 512 visible entries, k = 511) and rows that see no entry at all
    _indexer_case(1, 4, 64, 128, 600, 4, 511, 4 * 512 - 2, fmt, 30)
    _indexer_case(2, 4, 64, 128, 600, 4, 64, 2, fmt, 31)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_indexer_all_scores_equal(fmt):
    # many rows (the LDS select) and a decode row (the multi-workgroup select): one key value, so the first k
    # visible entries in index order
    _indexer_case(1, 6, 64 if fmt == "bf16" else 8, 128 if fmt == "bf16" else 32, 700, 4, 40, 4 * 700, fmt, 18,
                  zero_q=True)
    _indexer_case(2, 1, 64 if fmt == "bf16" else 8, 128 if fmt == "bf16" else 32, 3000, 4, 512, 4 * 3000, fmt, 19,
                  zero_q=True)


@pytest.mark.parametrize("fmt,B,N,k,cluster,zero_q", [("fp4", 2, 262144, 1024, 0.0, False),
                                                     ("fp4", 1, 65636, 1024, 4.0, False),
                                                     ("bf16", 1, 40000, 512, 0.0, True)])
def test_indexer_decode_candidate_forms(fmt, B, N, k, cluster, zero_q):
    # the decode select's finishing workgroup holds a row's candidates in registers (up to 6144, six consecutive ones
    # per thread found by one segment search and a walk over the segments), or re-reads them on every pass: rows of
    # 64 slices of plain N(0,1) keys; a row whose top scores crowd into its first slice (the walk crosses one long
    # segment and many short ones); a row of equal scores (every slice is all candidates)
    st = _indexer_case(B, 1, 64, 128, N, 4, k, 4 * N, fmt, 40, zero_q=zero_q, cluster=cluster)
    # the form follows from the scores: the candidates of a 4096-entry slice are its keys in or above the bin (key
    # bits [31:21]) of the k-th largest key
    forms = []
    for row, nv in zip(st["s64"], st["nvis"]):
        bits = (row[:nv].astype(np.float32) + np.float32(0.0)).view(np.uint32)  # -0 counts as +0
        keys = np.where(bits >> 31, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)
        b1 = np.sort(keys >> 21)[::-1][k - 1]
        per_slice = [int((keys[s:s + 4096] >> 21 >= b1).sum()) for s in range(0, nv, 4096)]
        forms.append((max(per_slice), sum(per_slice)))
    if cluster:
        assert all(m > t // 2 and t <= 6144 for m, t in forms), forms  # one slice holds most of them
    elif zero_q:
        assert all(t > 6144 for _, t in forms), forms
    else:
        assert all(t <= 6144 for _, t in forms), forms


@pytest.mark.parametrize("Sq", [1, 2])
def test_indexer_fp4_weights_not_16_byte_aligned(Sq):
    # the fp4 decode scorer reads each lane's head weights in 16-byte loads only when the weights are 16-byte
    # aligned; 4 bytes past a boundary it takes them one by one, with the same results
    _indexer_case(2, Sq, 64, 128, 9000, 4, 512, 4 * 9000, "fp4", 41, w_off=1)


def test_indexer_ties_go_to_lower_index():
    # dyadic bf16 inputs (exact dots) with duplicated key rows: equal scores, ties resolved by entry index
    _indexer_case(2, 3, 64, 128, 900, 4, 100, 4 * 900, "bf16", 15, dyadic=True, dup_rows=True)
    _indexer_case(1, 2, 8, 32, 300, 4, 50, 4 * 300, "f32", 16, dyadic=True, dup_rows=True)


# ------------------------------------------------------------------------------------------------------
# stages 3/4: attention
# ------------------------------------------------------------------------------------------------------
def _attn_case(B, Sq, H, D, N, k, window, q_start, fmt, seed, hca_m=0, sink_mode="normal", idx_mode="random",
               scale=None, rope=64, gain=0.0, out_f32=False, with_lse=True):
    g = _rng(seed)
    q = (g.standard_normal((B, Sq, H, D)) / math.sqrt(D)).astype(np.float32)
    comp = g.standard_normal((B, N, D)).astype(np.float32)
    if gain:  # entry e scaled by 1 + gain * e / N: logits grow along a sorted list, so the running max moves
        comp *= (1.0 + gain * np.arange(N, dtype=np.float32) / N)[None, :, None]
    raw_start = max(0, q_start - window + 1)
    S_raw = q_start + Sq - raw_start
    raw = g.standard_normal((B, max(S_raw, 1), D)).astype(np.float32)
    sink = g.standard_normal(H).astype(np.float32)
    if sink_mode == "none":
        sink[:] = -np.inf
    idx = None
    if hca_m == 0:
        idx = np.full((B, Sq, k), -1, np.int32)
        for b in range(B):
            for r in range(Sq):
                if idx_mode == "random":
                    sel = np.sort(g.choice(N, size=min(k, N), replace=False))
                    idx[b, r, :len(sel)] = sel
                    if k > 8:
                        idx[b, r, k - 3:] = -1  # padding at the end
                elif idx_mode == "empty":
                    pass
    scale = 1.0 if scale is None else scale
    capc, capr = N + 5, max(S_raw, 1) + 3
    qf = "f32" if fmt == "f32" else "bf16"
    if fmt == "f32":
        cg, rg = gpu_f32(comp, capc), gpu_f32(raw, capr)
        cr, rr = orc.plain_cache(comp, "f32"), orc.plain_cache(raw, "f32")
        qd, qr = up(q), orc.plain_cache(q, "f32")
    elif fmt == "bf16":
        cb, rb, qb = gen.bf16_bits(comp), gen.bf16_bits(raw), gen.bf16_bits(q)
        cg, rg = gpu_bf16(cb, capc), gpu_bf16(rb, capr)
        cr, rr = orc.plain_cache(cb, "bf16"), orc.plain_cache(rb, "bf16")
        qd, qr = up(qb), orc.plain_cache(qb, "bf16")
    else:  # mixed
        cg, rg = gpu_encode(comp, "mixed", rope, capc), gpu_encode(raw, "mixed", rope, capr)
        cr, rr = orc.encode(comp.reshape(-1, D), "mixed", rope), orc.encode(raw.reshape(-1, D), "mixed", rope)
        qb = gen.bf16_bits(q)
        qd, qr = up(qb), orc.plain_cache(qb, "bf16")
    cr["cap"], rr["cap"] = N, max(S_raw, 1)
    f32_out = fmt == "f32" or out_f32
    out = torch.empty((B, Sq, H, D), dtype=torch.float32 if f32_out else torch.int16, device="cuda")
    lse = torch.full((B, Sq, H), 12345.0, dtype=torch.float32, device="cuda")
    sd = up(sink)
    of = lca.LCA_F32 if f32_out else lca.LCA_BF16
    qfmt = lca.FORMATS[qf]
    if hca_m:
        nbytes = lca.hca_attn_workspace_size(B, Sq, H, D, window + N)
        w_s = ws(nbytes)
        lca.hca_attn(qd, qfmt, cg.desc(), N, hca_m, rg.desc(), raw_start, S_raw, sd, B, Sq, H, D, window, scale,
                     q_start, out, of, lse if with_lse else None, w_s, nbytes)
    else:
        nbytes = lca.sparse_mqa_attn_workspace_size(B, Sq, H, D, window + k)
        w_s = ws(nbytes)
        lca.sparse_mqa_attn(qd, qfmt, cg.desc(), N, rg.desc(), raw_start, S_raw, up(idx), k, sd, B, Sq, H, D, window,
                            scale, q_start, out, of, lse if with_lse else None, w_s, nbytes)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attn(qr, cr, N, rr, raw_start, S_raw, idx, k, hca_m, sink, B, Sq, H, D, window, scale, q_start)
    o = out.cpu().numpy()
    o = o.astype(np.float64) if f32_out else bf16_to_f64(o.view(np.uint16))
    if not with_lse:  # no lse pointer: nothing may have been written there
        assert torch.all(lse == 12345.0)
    return o, o_ref, lse.cpu().numpy(), l_ref


def test_attn_simt_f32():
    o, ref, l, lr = _attn_case(2, 5, 4, 64, 256, 32, 16, 300, "f32", 20)
    assert row_rel_err(o, ref) <= 1e-4
    np.testing.assert_allclose(l, lr, rtol=1e-5, atol=1e-5)


def test_attn_simt_f32_multisplit_and_mixed():
    o, ref, l, lr = _attn_case(1, 1, 8, 128, 3000, 700, 128, 20000, "f32", 21)
    assert row_rel_err(o, ref) <= 1e-4
    o, ref, _, _ = _attn_case(1, 2, 4, 96, 400, 64, 8, 9000, "mixed", 22, rope=32)
    assert row_rel_err(o, ref) <= 1e-2


@pytest.mark.parametrize("B,Sq,N,k,window,fmt", [(2, 1, 3000, 512, 128, "bf16"), (1, 300, 2000, 64, 128, "bf16"),
                                                  (2, 1, 5000, 1024, 128, "mixed"), (1, 3, 500, 100, 7, "bf16"),
                                                  (3, 1, 900, 300, 40, "mixed"), (1, 1, 5000, 2100, 128, "bf16"),
                                                  (1, 2, 6000, 2100, 128, "mixed"), (4, 4, 20000, 1024, 128, "mixed"),
                                                  (8, 2, 32768, 512, 128, "bf16")])
def test_attn_mfma(B, Sq, N, k, window, fmt):
    o, ref, l, lr = _attn_case(B, Sq, 64, 512, N, k, window, 60000, fmt, 23, scale=1.0)
    assert row_rel_err(o, ref) <= 1e-2
    np.testing.assert_allclose(l, lr, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("fmt", ["bf16", "mixed"])
@pytest.mark.parametrize("k", [384, 385])
def test_attn_decode_forms_at_the_split(k, fmt):
    # few rows: 384 + 128 = 512 list positions take the two passes, 513 the one-pass kernel and the merge (a last tile
    # holding one position, with sink); both against the oracle
    o, ref, l, lr = _attn_case(2, 1, 64, 512, 3000, k, 128, 60000, fmt, 29, scale=1.0)
    assert row_rel_err(o, ref) <= 1e-2
    np.testing.assert_allclose(l, lr, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("B,Sq,N,k,window,q_start,seed", [(1, 300, 500, 64, 128, 0, 41),
                                                          (1, 256, 3000, 2100, 16, 60000, 42),
                                                          (2, 130, 1000, 40, 128, 77, 43)])
def test_attn_many_rows(B, Sq, N, k, window, q_start, seed):
    # the many-row bf16 kernel: windows that grow from one position (q_start 0), a list longer than one slice
    # (two splits and the merge), and rows of two sequences
    o, ref, l, lr = _attn_case(B, Sq, 64, 512, N, k, window, q_start, "bf16", seed, scale=1.0)
    assert row_rel_err(o, ref) <= 1e-2
    np.testing.assert_allclose(l, lr, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("B,Sq,k", [(1, 260, 512), (2, 1, 512), (1, 1, 2100)])
def test_attn_running_max_moves(B, Sq, k):
    # entries later in the (sorted) list have logits up to 40x larger, so the reference max of every head moves many
    # times by more than the rescale slack: the many-row kernel (260 rows), the fused decode kernel (512) and the
    # head-group kernel (2100)
    o, ref, l, lr = _attn_case(B, Sq, 64, 512, 4000, k, 16, 60000, "bf16", 44, scale=1.0, gain=40.0)
    assert row_rel_err(o, ref) <= 1e-2
    np.testing.assert_allclose(l, lr, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("hca_m,k", [(0, 100), (0, 2100), (128, 0)])
def test_attn_bf16_cache_f32_output_no_lse(hca_m, k):
    # fp32 output and no lse pointer on the many-row kernel: one slice, split slices (fp32 partials' bf16 path and
    # the merge) and dense HCA rows
    N = 3000 if hca_m == 0 else 300
    q_start = 60000 if hca_m == 0 else 128 * N + 40
    o, ref, l, lr = _attn_case(1, 260 if hca_m == 0 else 3, 64, 512, N, k, 128, q_start, "bf16", 47, hca_m=hca_m,
                               scale=1.0 / math.sqrt(512), out_f32=True, with_lse=False)
    assert row_rel_err(o, ref) <= 1e-2


def test_attn_many_rows_empty_lists():
    # many rows, no window, every list empty: o = 0, lse = -inf; then only the sink: o = 0, lse = z
    o, ref, l, lr = _attn_case(1, 256, 64, 512, 50, 16, 0, 400, "bf16", 45, sink_mode="none", idx_mode="empty")
    assert np.all(o == 0) and np.all(ref == 0)
    assert np.all(np.isneginf(l)) and np.all(np.isneginf(lr))
    o, ref, l, lr = _attn_case(1, 256, 64, 512, 50, 16, 0, 400, "bf16", 46, idx_mode="empty")
    assert np.all(o == 0)
    np.testing.assert_allclose(l, lr, rtol=1e-6)


@pytest.mark.parametrize("fmt", ["bf16", "mixed"])
def test_hca_short_list_single_split(fmt):
    # window 16 + 40 entries: one slice per row, the output finalized in the attention kernel itself
    o, ref, l, lr = _attn_case(3, 1, 64, 512, 40, 0, 16, 128 * 40 + 7, fmt, 31, hca_m=128)
    assert row_rel_err(o, ref) <= 1e-2
    np.testing.assert_allclose(l, lr, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("fmt,H,D", [("bf16", 64, 512), ("mixed", 64, 512), ("f32", 4, 64)])
def test_hca_dense(fmt, H, D):
    m, N = 128, 300
    o, ref, l, lr = _attn_case(2, 2, H, D, N, 0, 128, m * N + 40, fmt, 24, hca_m=m, scale=1.0 / math.sqrt(D),
                               rope=64 if D == 512 else 16)
    assert row_rel_err(o, ref) <= (1e-4 if fmt == "f32" else 1e-2)
    np.testing.assert_allclose(l, lr, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("fmt,H,D", [("bf16", 64, 512), ("f32", 4, 64)])
def test_attn_degenerate_sets(fmt, H, D):
    # empty index list, no window, no sink: o = 0 and lse = -inf
    o, ref, l, lr = _attn_case(1, 2, H, D, 50, 16, 0, 400, fmt, 25, sink_mode="none", idx_mode="empty")
    assert np.all(o == 0) and np.all(ref == 0)
    assert np.all(np.isneginf(l)) and np.all(np.isneginf(lr))
    # only the sink: o = 0, lse = z
    o, ref, l, lr = _attn_case(1, 1, H, D, 50, 16, 0, 400, fmt, 26, idx_mode="empty")
    assert np.all(o == 0)
    np.testing.assert_allclose(l, lr, rtol=1e-6)
    # first query of a sequence: the window holds only itself
    o, ref, l, lr = _attn_case(1, 1, H, D, 10, 4, 128, 0, fmt, 27, sink_mode="none", idx_mode="empty")
    assert row_rel_err(o, ref) <= (1e-4 if fmt == "f32" else 1e-2)


def test_attn_hca_equals_sparse_with_all_visible():
    """Two GPU entry points over the same list: hca_attn == sparse_mqa_attn with idx = all visible entries.

    They take different kernels (all-heads wide kernel vs. 16-head groups) with different split plans, so the
    probabilities are rounded to bf16 against different running maxima: agreement is to the bf16-path bound."""
    g = _rng(28)
    B, Sq, H, D, N, m, W = 2, 1, 64, 512, 200, 128, 128
    q_start = m * N + 5
    comp = gen.bf16_bits(g.standard_normal((B, N, D)).astype(np.float32))
    raw = gen.bf16_bits(g.standard_normal((B, W, D)).astype(np.float32))
    q = gen.bf16_bits((g.standard_normal((B, Sq, H, D)) / 20).astype(np.float32))
    sink = up(g.standard_normal(H).astype(np.float32))
    cg, rg, qd = gpu_bf16(comp), gpu_bf16(raw), up(q)
    raw_start = q_start - W + 1
    o1 = torch.empty((B, Sq, H, D), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    n1 = lca.hca_attn_workspace_size(B, Sq, H, D, W + N)
    lca.hca_attn(qd, lca.LCA_BF16, cg.desc(), N, m, rg.desc(), raw_start, W, sink, B, Sq, H, D, W, 0.05, q_start, o1,
                 lca.LCA_F32, None, ws(n1), n1)
    idx = up(np.tile(np.arange(N, dtype=np.int32), (B, Sq, 1)))
    n2 = lca.sparse_mqa_attn_workspace_size(B, Sq, H, D, W + N)
    lca.sparse_mqa_attn(qd, lca.LCA_BF16, cg.desc(), N, rg.desc(), raw_start, W, idx, N, sink, B, Sq, H, D, W, 0.05,
                        q_start, o2, lca.LCA_F32, None, ws(n2), n2)
    torch.cuda.synchronize()
    a1, a2 = o1.cpu().numpy().astype(np.float64), o2.cpu().numpy().astype(np.float64)
    assert row_rel_err(a1, a2) <= 1e-2


def test_repeat_calls_bit_identical():
    a = _attn_case(2, 1, 64, 512, 3000, 512, 128, 60000, "bf16", 29)[0]
    b = _attn_case(2, 1, 64, 512, 3000, 512, 128, 60000, "bf16", 29)[0]
    assert np.array_equal(a, b)
