"""Pins of the oracle's layer steps: compression, indexer score and top-k, attention with window and sink.
Every test ties the oracle to something other than itself: closed forms, invariants the pages state,
library routines in special cases, brute force on tiny inputs.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _structural():
    d = {}
    for line in open(os.path.join(GOLD, "structural.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            d[k] = v
    return d


def _streams(g, B, n, c, m):
    f = lambda *s: g.standard_normal(s).astype(np.float32)
    return dict(Ca=f(B, n, c), Cb=f(B, n, c), Za=f(B, n, c), Zb=f(B, n, c), Ba=(0.1 * f(m, c)).astype(np.float32),
                Bb=(0.1 * f(m, c)).astype(np.float32), tail_Cb=f(B, m, c), tail_Zb=f(B, m, c))


# ---------------------------------------------------------------------------------------------------
# compression
# ---------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("m,overlap,start", [(4, True, 0), (4, True, 64), (128, False, 0), (3, True, 6)])
def test_compress_constant_kv_stays_constant(m, overlap, start):
    """Weights are a softmax, so they sum to 1: constant candidates give that constant (also entry 0 and a
    partial tail block)."""
    g = np.random.default_rng(10)
    B, n, c = 2, 5 * m + 1, 8
    s = _streams(g, B, n, c, m)
    val = np.float32(1.7)
    for k in ("Ca", "Cb", "tail_Cb"):
        s[k] = np.full_like(s[k], val)
    E = orc.kv_compress(s["Ca"], s["Cb"], s["Za"], s["Zb"], s["Ba"], s["Bb"], s["tail_Cb"], s["tail_Zb"], m=m,
                        overlap=overlap, start_pos=start)
    assert E.shape == (B, (n + m - 1) // m, c)
    np.testing.assert_allclose(E, 1.7, rtol=1e-6)


def test_compress_one_hot_logits_pick_block_and_stream():
    """A +60 logit on one candidate makes the entry equal to that candidate.  Stream a of block i feeds entry
    i; stream b of block i feeds entry i+1 (adjacent entries overlap by one block)."""
    g = np.random.default_rng(11)
    B, n, c, m = 1, 24, 4, 4
    s = _streams(g, B, n, c, m)
    s["Za"][:] = 0.0
    s["Zb"][:] = 0.0
    s["Ba"][:] = 0.0
    s["Bb"][:] = 0.0
    p_a, p_b = 9, 13  # token 9 in block 2 (stream a); token 13 in block 3 (stream b)
    s["Za"][0, p_a, :] = 60.0
    s["Zb"][0, p_b, :] = 60.0
    E = orc.kv_compress(s["Ca"], s["Cb"], s["Za"], s["Zb"], s["Ba"], s["Bb"], m=m, overlap=True)
    np.testing.assert_allclose(E[0, 2], s["Ca"][0, p_a], rtol=1e-12, atol=1e-20 + 1e-20)
    np.testing.assert_allclose(E[0, 4], s["Cb"][0, p_b], rtol=1e-12)
    # entry 3 sees block 3 via stream a (all logits 0) and block 2 via stream b (all 0): plain mean of 8
    ref3 = (s["Ca"][0, 12:16].astype(np.float64).sum(0) + s["Cb"][0, 8:12].astype(np.float64).sum(0)) / 8
    np.testing.assert_allclose(E[0, 3], ref3, rtol=1e-12)
    # entry 0 has no predecessor: mean of its own 4 stream-a tokens
    np.testing.assert_allclose(E[0, 0], s["Ca"][0, 0:4].astype(np.float64).mean(0), rtol=1e-12)


def test_compress_logit_shift_invariance():
    g = np.random.default_rng(12)
    B, n, c, m = 2, 33, 6, 4
    s = _streams(g, B, n, c, m)
    E0 = orc.kv_compress(**{k: s[k] for k in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")}, m=m, overlap=True)
    shift = g.standard_normal(c).astype(np.float32) * 3
    s2 = dict(s)
    s2["Za"] = (s["Za"] + shift).astype(np.float32)
    s2["Zb"] = (s["Zb"] + shift).astype(np.float32)
    E1 = orc.kv_compress(**{k: s2[k] for k in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")}, m=m, overlap=True)
    np.testing.assert_allclose(E1, E0, rtol=2e-6, atol=1e-6)  # the float32 sums Z + shift round once


def test_compress_chunked_equals_whole():
    """Compressing tokens [0, n) at once equals [0, n1) then [n1, n) with the carried stream-b tail."""
    g = np.random.default_rng(13)
    B, n, c, m, n1 = 2, 40, 5, 4, 16
    s = _streams(g, B, n, c, m)
    keys = ("Ca", "Cb", "Za", "Zb")
    E = orc.kv_compress(*(s[k] for k in keys), s["Ba"], s["Bb"], m=m, overlap=True)
    E1 = orc.kv_compress(*(s[k][:, :n1] for k in keys), s["Ba"], s["Bb"], m=m, overlap=True)
    E2 = orc.kv_compress(*(np.ascontiguousarray(s[k][:, n1:]) for k in keys), s["Ba"], s["Bb"],
                         tail_Cb=np.ascontiguousarray(s["Cb"][:, n1 - m:n1]),
                         tail_Zb=np.ascontiguousarray(s["Zb"][:, n1 - m:n1]), m=m, overlap=True, start_pos=n1)
    np.testing.assert_array_equal(np.concatenate([E1, E2], axis=1), E)


def test_compress_m1_is_identity_and_counts():
    g = np.random.default_rng(14)
    s = _streams(g, 1, 10, 3, 1)
    E = orc.kv_compress(s["Ca"], None, s["Za"], None, s["Ba"], None, m=1, overlap=False)
    np.testing.assert_array_equal(E, s["Ca"].astype(np.float64))
    st = _structural()
    # ceil(n / m) entries: 1e6 tokens at 128:1 -> 7813 < 8000 (67808.cn explainer, section 3); 2^20 -> 8192
    for n, m, want in ((10 ** 6, 128, int(st["hca_entries_1e6"])), (1 << 20, 128, 8192),
                       (int(st["toy_tokens"]), int(st["csa_ratio"]), int(st["toy_entries"]))):
        one = np.zeros((1, n, 1), np.float32)
        E = orc.kv_compress(one, None, one, None, np.zeros((m, 1), np.float32), None, m=m, overlap=False)
        assert E.shape[1] == want
    assert int(st["hca_entries_1e6"]) < int(st["hca_entries_bound_1e6"])


# ---------------------------------------------------------------------------------------------------
# indexer score and top-k
# ---------------------------------------------------------------------------------------------------
def test_indexer_dyadic_scores_exact_and_canonical():
    """Dyadic small-integer inputs: every product and partial sum is exact, so the canonical fp32 score equals
    the double score bit for bit, whatever the summation order."""
    g = np.random.default_rng(20)
    B, Sq, HI, DI, N, m = 2, 3, 8, 16, 37, 4
    q = (g.integers(-4, 5, (B, Sq, HI, DI)) * 0.5).astype(np.float32)
    K = (g.integers(-4, 5, (B, N, DI)) * 0.25).astype(np.float32)
    w = (g.integers(-3, 4, (B, Sq, HI)) * 0.125).astype(np.float32)
    qs, ks = orc.plain_cache(q, "f32"), orc.plain_cache(K, "f32")
    ks["cap"] = N
    s64, s32, ab, bad = orc.indexer_scores(qs, w, ks, B, Sq, HI, DI, N, m, q_start_pos=4 * N + 10, canonical=True,
                                           want_abs=True)
    assert bad == 0
    np.testing.assert_array_equal(s32.astype(np.float64), s64)
    # independent evaluation with numpy's matmul (a library routine) for the head dots
    d = np.einsum("bshd,bnd->bshn", q.astype(np.float64), K.astype(np.float64))
    ref = (np.maximum(d, 0) * w[..., None]).sum(axis=2)
    np.testing.assert_array_equal(s64, ref)


def test_indexer_visibility_and_relu():
    g = np.random.default_rng(21)
    B, Sq, HI, DI, N, m = 1, 8, 4, 16, 10, 4
    q = g.standard_normal((B, Sq, HI, DI)).astype(np.float32)
    K = g.standard_normal((B, N, DI)).astype(np.float32)
    w = np.abs(g.standard_normal((B, Sq, HI))).astype(np.float32)
    qs, ks = orc.plain_cache(q, "f32"), orc.plain_cache(K, "f32")
    ks["cap"] = N
    start = 13  # rows t = 13..20 see floor(t/4) = 3..5 entries: never their own block
    s64, _, _, _ = orc.indexer_scores(qs, w, ks, B, Sq, HI, DI, N, m, start)
    for r in range(Sq):
        nv = (start + r) // m
        assert np.all(np.isfinite(s64[0, r, :nv])) and np.all(np.isneginf(s64[0, r, nv:]))
    # ReLU: flipping K's sign for entries whose dots are all negative gives score 0
    Kneg = -np.abs(K)
    qpos = np.abs(q)
    s64b, _, _, _ = orc.indexer_scores(orc.plain_cache(qpos, "f32"), w, dict(orc.plain_cache(Kneg, "f32"), cap=N),
                                       B, Sq, HI, DI, N, m, 100)
    np.testing.assert_array_equal(s64b, 0.0)


def test_topk_matches_brute_force_with_ties():
    g = np.random.default_rng(22)
    R, N = 50, 64
    s = g.integers(-5, 6, (R, N)).astype(np.float64)  # many ties
    nv = g.integers(0, N + 1, R).astype(np.int32)
    for k in (1, 7, 32, 64, 80):
        idx, kth, nxt = orc.topk(s, nv, k)
        for r in range(R):
            order = sorted(range(nv[r]), key=lambda i: (-s[r, i], i))
            want = sorted(order[:k]) + [-1] * (k - min(k, nv[r]))
            assert list(idx[r]) == want
            if k <= nv[r]:
                assert kth[r] == s[r, order[k - 1]]


def test_topk_toy_example():
    """cosmocat page, section 3: 16 tokens -> 4 entries; the indexer keeps the 2nd and 4th."""
    st = _structural()
    n, m = int(st["toy_tokens"]), int(st["csa_ratio"])
    N = n // m
    s = np.array([[0.1, 0.9, 0.2, 0.7]])
    idx, _, _ = orc.topk(s, np.array([N], np.int32), 2)
    assert list(idx[0]) == [int(x) for x in st["toy_selected"].split(",")]


# ---------------------------------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------------------------------
def _attn_case(g, B, Sq, H, D, N, k, S_raw, raw_start, q_start):
    q = g.standard_normal((B, Sq, H, D)).astype(np.float32) * np.float32(0.3)
    comp = g.standard_normal((B, N, D)).astype(np.float32)
    raw = g.standard_normal((B, S_raw, D)).astype(np.float32)
    idx = np.stack([np.stack([g.permutation(N)[:k] for _ in range(Sq)]) for _ in range(B)]).astype(np.int32)
    return q, comp, raw, idx


def _run_attn(q, comp, raw, idx, sink, window, raw_start, q_start, hca_m=0, N=None, scale=1.0):
    B, Sq, H, D = q.shape
    N = comp.shape[1] if N is None else N
    cs = orc.plain_cache(comp, "f32")
    cs["cap"] = comp.shape[1]
    rs = orc.plain_cache(raw, "f32")
    rs["cap"] = raw.shape[1]
    k = 0 if idx is None else idx.shape[-1]
    return orc.attn(orc.plain_cache(q, "f32"), cs, N, rs, raw_start, raw.shape[1], idx, k, hca_m, sink, B, Sq, H, D,
                    window, scale, q_start)


def test_attn_m1_collapses_to_causal_attention():
    """m = 1, no overlap, k >= n, window 1, no sink, stream a = raw KV: the whole layer (compress -> index ->
    top-k -> attend) equals dense causal MQA over [0, t] -- checked against torch's SDPA in float64."""
    g = np.random.default_rng(30)
    B, n, H, D, HI, DI = 2, 40, 3, 16, 2, 8
    kv = g.standard_normal((B, n, D)).astype(np.float32)
    Z = g.standard_normal((B, n, D)).astype(np.float32)
    E = orc.kv_compress(kv, None, Z, None, np.zeros((1, D), np.float32), None, m=1, overlap=False)
    comp = orc.compress_to_cache(E, "f32")
    comp["cap"] = n
    qI = g.standard_normal((B, n, HI, DI)).astype(np.float32)
    keys = g.standard_normal((B, n, DI)).astype(np.float32)
    w = g.standard_normal((B, n, HI)).astype(np.float32)
    s64, _, _, _ = orc.indexer_scores(orc.plain_cache(qI, "f32"), w, dict(orc.plain_cache(keys, "f32"), cap=n), B, n,
                                      HI, DI, n, 1, 0)
    nv = orc.nvis_rows(B, np.arange(n), 0, 1, n)
    idx, _, _ = orc.topk(s64.reshape(B * n, n), nv, n)
    q = g.standard_normal((B, n, H, D)).astype(np.float32)
    sink = np.full(H, -np.inf, np.float32)
    o, lse = orc.attn(orc.plain_cache(q, "f32"), comp, n, dict(orc.plain_cache(kv, "f32"), cap=n), 0, n,
                      idx.reshape(B, n, n), n, 0, sink, B, n, H, D, 1, 1.0 / math.sqrt(D), 0)
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)       # [B, H, n, D]
    kt = torch.from_numpy(kv.astype(np.float64))[:, None].expand(B, H, n, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, is_causal=True).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_attn_sink_closed_form():
    """The sink adds e^z to the denominator only: o(z) = o(-inf) * S / (S + e^z), S = sum e^l = e^lse(-inf)."""
    g = np.random.default_rng(31)
    B, Sq, H, D, N, k, W = 2, 3, 4, 8, 20, 6, 5
    q, comp, raw, idx = _attn_case(g, B, Sq, H, D, N, k, 40, 0, 30)
    o0, l0 = _run_attn(q, comp, raw, idx, np.full(H, -np.inf, np.float32), W, 0, 30)
    z = np.array([-2.0, 0.0, 1.5, 40.0], np.float32)
    o1, l1 = _run_attn(q, comp, raw, idx, z, W, 0, 30)
    S = np.exp(l0)
    ratio = S / (S + np.exp(z.astype(np.float64)))
    np.testing.assert_allclose(o1, o0 * ratio[..., None], rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(l1, np.logaddexp(l0, z.astype(np.float64)), rtol=1e-12)
    assert np.all(np.abs(o1[:, :, 3]) < 1e-10)  # z -> +inf drives the output to 0


def test_attn_permutation_and_padding():
    g = np.random.default_rng(32)
    B, Sq, H, D, N, k, W = 2, 2, 3, 8, 30, 9, 4
    q, comp, raw, idx = _attn_case(g, B, Sq, H, D, N, k, 50, 0, 40)
    sink = g.standard_normal(H).astype(np.float32)
    o0, l0 = _run_attn(q, comp, raw, idx, sink, W, 0, 40)
    perm = np.ascontiguousarray(idx[..., g.permutation(k)])
    o1, l1 = _run_attn(q, comp, raw, perm, sink, W, 0, 40)
    np.testing.assert_allclose(o1, o0, rtol=1e-12)
    padded = np.concatenate([idx, np.full((B, Sq, 3), -1, np.int32)], axis=-1)
    o2, _ = _run_attn(q, comp, raw, np.ascontiguousarray(padded), sink, W, 0, 40)
    np.testing.assert_allclose(o2, o0, rtol=1e-12)


def test_hca_dense_equals_sparse_with_all_visible():
    g = np.random.default_rng(33)
    B, Sq, H, D, N, m, W = 2, 4, 3, 8, 12, 8, 6
    q, comp, raw, _ = _attn_case(g, B, Sq, H, D, N, 1, 60, 0, 0)
    qstart = 50
    sink = g.standard_normal(H).astype(np.float32)
    od, ld = _run_attn(q, comp, raw, None, sink, W, 0, qstart, hca_m=m, N=N)
    idx = np.full((B, Sq, N), -1, np.int32)
    for r in range(Sq):
        nv = min((qstart + r) // m, N)
        idx[:, r, :nv] = np.arange(nv)
    os_, ls = _run_attn(q, comp, raw, idx, sink, W, 0, qstart, N=N)
    np.testing.assert_allclose(od, os_, rtol=1e-12)
    np.testing.assert_allclose(ld, ls, rtol=1e-12)


def test_attn_empty_set_and_window_bounds():
    g = np.random.default_rng(34)
    q, comp, raw, idx = _attn_case(g, 1, 1, 2, 4, 5, 2, 10, 0, 3)
    o, l = _run_attn(q, comp, raw, np.full_like(idx, -1), np.full(2, -np.inf, np.float32), 0, 0, 3)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    with pytest.raises(ValueError):
        _run_attn(q, comp, raw, idx, np.zeros(2, np.float32), 4, 2, 3)  # window [0, 3] starts before raw_start


def test_own_block_invisible_through_compressed_path():
    """Perturbing the streams of block floor(t/m) and later leaves o(t) unchanged (window KV fixed): a query never
    sees its own block except through the window (itsolotime page, mechanism 1; 67808.cn explainer, section 4)."""
    g = np.random.default_rng(35)
    B, n, c, m, H, HI, DI, k, W = 1, 64, 8, 4, 2, 2, 4, 5, 3
    s = _streams(g, B, n, c, m)
    sI = _streams(g, B, n, DI, m)
    qI = g.standard_normal((B, n, HI, DI)).astype(np.float32)
    w = g.standard_normal((B, n, HI)).astype(np.float32)
    q = g.standard_normal((B, n, H, c)).astype(np.float32)
    raw = g.standard_normal((B, n, c)).astype(np.float32)
    sink = g.standard_normal(H).astype(np.float32)

    def layer(s, sI, t):
        E = orc.kv_compress(*(s[x] for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m=m, overlap=True)
        EI = orc.kv_compress(*(sI[x] for x in ("Ca", "Cb", "Za", "Zb", "Ba", "Bb")), m=m, overlap=True)
        N = E.shape[1]
        comp, keys = orc.compress_to_cache(E, "f32"), orc.compress_to_cache(EI, "f32")
        comp["cap"] = keys["cap"] = N
        s64, _, _, _ = orc.indexer_scores(orc.plain_cache(qI, "f32"), w, keys, B, n, HI, DI, N, m, 0, rows=[t])
        idx, _, _ = orc.topk(s64.reshape(1, N), orc.nvis_rows(B, [t], 0, m, N), k)
        idx_all = np.full((B, n, k), -1, np.int32)  # the oracle reads row t of a [B, Sq, k] list
        idx_all[:, t, :] = idx
        o, _ = orc.attn(orc.plain_cache(q, "f32"), comp, N, dict(orc.plain_cache(raw, "f32"), cap=n), 0, n,
                        idx_all, k, 0, sink, B, n, H, c, W, 0.5, 0, rows=[t])
        return o

    for t in (21, 22, 23, 40):
        o0 = layer(s, sI, t)
        p = (t // m) * m
        s2 = {x: v.copy() for x, v in s.items()}
        sI2 = {x: v.copy() for x, v in sI.items()}
        for d in (s2, sI2):
            for x in ("Ca", "Cb", "Za", "Zb"):
                d[x][:, p:] += g.standard_normal(d[x][:, p:].shape).astype(np.float32) * 5
        np.testing.assert_array_equal(layer(s2, sI2, t), o0)
