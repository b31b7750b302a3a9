"""GPU parity on the five workloads at their full sizes, in the launch configuration bench.py times (the step
classes of long_context_attention_05_amd.steps), against the oracle on every output the oracle can afford or on
sampled rows."""
import math

import numpy as np
import pytest
import torch

import lca_inputs as gen
from oracle import oracle as orc
from tests.gpu_util import (bf16_to_f64, check_bf16_codes, check_fp4_codes, check_mixed_codes, check_topk,
                            row_rel_err)

pytestmark = pytest.mark.gpu

steps = pytest.importorskip("long_context_attention_05_amd.steps")
lca = pytest.importorskip("long_context_attention_05_amd.lca")

GAMMA = lambda DI, HI: 2.0 * (DI + HI) * 2.0 ** -24


def _bf16(x):
    return gen.bf16_bits(x)


def _compress_ref(inp, tag, m, overlap, start, sl=slice(None)):
    g = lambda k: None if k + tag not in inp else inp[k + tag][sl]
    return orc.kv_compress(g("Ca"), g("Cb"), g("Za"), g("Zb"), inp["Ba" + tag], inp.get("Bb" + tag), g("tail_Cb"),
                           g("tail_Zb"), m=m, overlap=overlap, start_pos=start)


def _decoded_entries(cache: lca.CacheTensor, B, rows: slice):
    """Decode device cache rows (bf16 only) to float64 [B, n, dim]."""
    h = cache.host()
    d = h["data"].reshape(B, cache.cap, -1)[:, rows]
    return bf16_to_f64(d)


# ------------------------------------------------------------------------------------------------------
def test_tiny_csa_prefill_f32_full_chain():
    """Workload 1 end to end: compression of both streams -> indexer (fp32) -> top-32 -> attention, all 1024 rows."""
    w = gen.WORKLOADS["tiny_csa_prefill_f32"]
    inp = gen.prefill_inputs(w)
    N = w.Sq // w.m
    main_e = _compress_ref(inp, "", 4, True, 0)
    key_e = _compress_ref(inp, "_I", 4, True, 0)
    # GPU chain through the C-ABI, caches in fp32
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    comp = lca.CacheTensor("f32", 1, N, w.D)
    keys = lca.CacheTensor("f32", 1, N, w.DI)
    for tag, out, c in (("", comp, w.D), ("_I", keys, w.DI)):
        lca.kv_compress(dev(inp["Ca" + tag]), dev(inp["Cb" + tag]), dev(inp["Za" + tag]), dev(inp["Zb" + tag]),
                        dev(inp["Ba" + tag]), dev(inp["Bb" + tag]), None, None, 1, w.Sq, c, 4, True, 0, out.desc())
    qI = dev(inp["qI"])
    idx = torch.empty((1, w.Sq, w.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, w.Sq, w.k), dtype=torch.float32, device="cuda")
    nb = lca.indexer_score_topk_workspace_size(1, w.Sq, N, w.k)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lca.indexer_score_topk(lca.plain_desc(qI, "f32", w.DI, w.Sq * w.HI), dev(inp["w"]), keys.desc(), 1, w.Sq, w.HI,
                           w.DI, N, 4, w.k, 0, idx, sc, ws, nb)
    raw = lca.CacheTensor("f32", 1, w.Sq, w.D)
    raw.data.copy_(dev(inp["raw_kv"]).view(w.Sq, w.D))
    out = torch.empty((1, w.Sq, w.H, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, w.Sq, w.H), dtype=torch.float32, device="cuda")
    na = lca.sparse_mqa_attn_workspace_size(1, w.Sq, w.H, w.D, w.window + w.k)
    wa = torch.empty(max(na, 256), dtype=torch.uint8, device="cuda")
    lca.sparse_mqa_attn(dev(inp["q"]), lca.LCA_F32, comp.desc(), N, raw.desc(), 0, w.Sq, idx, w.k, dev(inp["sink"]), 1,
                        w.Sq, w.H, w.D, w.window, w.scale, 0, out, lca.LCA_F32, lse, wa, na)
    torch.cuda.synchronize()
    # stage 1: both caches within 1e-4
    assert row_rel_err(comp.data.cpu().numpy().reshape(1, N, w.D), main_e) <= 1e-4
    assert row_rel_err(keys.data.cpu().numpy().reshape(1, N, w.DI), key_e) <= 1e-4
    # stage 2, stage-isolated: the oracle scores the key bytes the GPU wrote, with the plain fp32 rounding bound
    kk = dict(orc.plain_cache(keys.data.cpu().numpy().reshape(1, N, w.DI), "f32"), cap=N)
    s64, _, ab, _ = orc.indexer_scores(orc.plain_cache(inp["qI"], "f32"), inp["w"], kk, 1, w.Sq, w.HI, w.DI, N, 4, 0,
                                       want_abs=True)
    nv = orc.nvis_rows(1, np.arange(w.Sq), 0, 4, N)
    gidx = idx.cpu().numpy().reshape(w.Sq, w.k)
    st = check_topk(gidx, sc.cpu().numpy().reshape(w.Sq, w.k), s64.reshape(w.Sq, N), ab.reshape(w.Sq, N), nv, w.k,
                    GAMMA(w.DI, w.HI))
    print("tiny chain: %d of %d rows exact, %d certified near-ties" % (st["exact_rows"], w.Sq, st["near_tie_rows"]))
    assert st["near_tie_rows"] <= 3
    # stage 3, stage-isolated: the oracle attends the GPU's selection over the latent entries the GPU wrote: every row
    kc = dict(orc.plain_cache(comp.data.cpu().numpy().reshape(1, N, w.D), "f32"), cap=N)
    o_ref, l_ref = orc.attn(orc.plain_cache(inp["q"], "f32"), kc, N, dict(orc.plain_cache(inp["raw_kv"], "f32"),
                                                                         cap=w.Sq), 0, w.Sq, gidx.reshape(1, w.Sq, w.k),
                            w.k, 0, inp["sink"], 1, w.Sq, w.H, w.D, w.window, w.scale, 0)
    o = out.cpu().numpy()[0]
    assert row_rel_err(o, o_ref[0]) <= 1e-4
    np.testing.assert_allclose(lse.cpu().numpy()[0], l_ref[0], rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------------------------------------------------
def _check_decode(w, inp, step):
    B, N, Sq = w.B, w.N, w.Sq
    R = B * Sq  # query rows
    torch.cuda.synchronize()
    # appended entries (block N, provisional): latent and indexer key, code by code
    for tag, cache, c, fmt in (("", step.comp[0], w.D, w.main_fmt), ("_I", step.keys[0], w.DI, w.key_fmt)):
        E = _compress_ref(inp, tag, 4, True, w.n_ctx)[:, 0]  # [B, c]
        h = cache.host()
        row = lambda a: a.reshape(B, cache.cap, *a.shape[1:])[:, N]  # noqa: E731
        if fmt == "bf16":
            check_bf16_codes(row(h["data"]), E)
        elif fmt == "mixed":
            check_mixed_codes(dict(data=row(h["data"]), rope_data=row(h["rope_data"]), scale=row(h["scale"])), E,
                              w.rope)
        else:
            check_fp4_codes(dict(data=row(h["data"]), scale=row(h["scale"])), E)
    # indexer: oracle scores over the same key bytes
    exact = w.key_fmt == "fp4"
    if exact:
        kc = orc.encode(inp["keys"].reshape(-1, w.DI), "fp4")
        qc = orc.encode(inp["qI"].reshape(-1, w.DI), "fp4")
        got_k = step.keys[0].host()
        np.testing.assert_array_equal(got_k["data"].reshape(B, N + 1, -1)[:, :N].reshape(-1, w.DI // 2), kc["data"])
        np.testing.assert_array_equal(got_k["scale"].reshape(B, N + 1, -1)[:, :N].reshape(-1, w.DI // 32), kc["scale"])
    else:
        kc = orc.plain_cache(_bf16(inp["keys"]), "bf16")
        qc = orc.plain_cache(_bf16(inp["qI"]), "bf16")
    kc["cap"] = N
    s64, s32, ab, bad = orc.indexer_scores(qc, inp["w"], kc, B, Sq, w.HI, w.DI, N, 4, w.n_ctx, canonical=exact,
                                           want_abs=True)
    if exact:
        assert bad == 0
    nv = orc.nvis_rows(B, list(range(Sq)), w.n_ctx, 4, N)
    gidx = step.idx.cpu().numpy().reshape(R, w.k)
    st = check_topk(gidx, step.scores.cpu().numpy().reshape(R, w.k), s64.reshape(R, N), ab.reshape(R, N), nv, w.k,
                    GAMMA(w.DI, w.HI), exact=exact, s32=None if s32 is None else s32.reshape(R, N))
    # attention, stage-isolated: the oracle attends the GPU's own selection, every row
    if w.main_fmt == "mixed":
        cc = orc.encode(inp["comp"].reshape(-1, w.D), "mixed", w.rope)
        rc = orc.encode(inp["window_kv"].reshape(-1, w.D), "mixed", w.rope)
        got_c = step.comp[0].host()
        np.testing.assert_array_equal(got_c["data"].reshape(B, N + 1, -1)[:, :N].reshape(-1, w.D - w.rope), cc["data"])
        np.testing.assert_array_equal(got_c["scale"].reshape(B, N + 1)[:, :N].reshape(-1), cc["scale"])
    else:
        cc = orc.plain_cache(_bf16(inp["comp"]), "bf16")
        rc = orc.plain_cache(_bf16(inp["window_kv"]), "bf16")
    S_raw = w.window + Sq - 1
    cc["cap"], rc["cap"] = N, S_raw
    qa = orc.plain_cache(_bf16(inp["q"]), "bf16")
    o_ref, l_ref = orc.attn(qa, cc, N, rc, w.n_ctx - w.window + 1, S_raw, gidx.reshape(B, Sq, w.k), w.k, 0,
                            inp["sink"], B, Sq, w.H, w.D, w.window, w.scale, w.n_ctx)
    o = bf16_to_f64(step.out.cpu().numpy().view(np.uint16)).reshape(R, w.H, w.D)
    assert row_rel_err(o, o_ref.reshape(R, w.H, w.D)) <= 1e-2
    np.testing.assert_allclose(step.lse.cpu().numpy().reshape(R, w.H), l_ref.reshape(R, w.H), rtol=1e-4, atol=1e-4)
    print("%s: %d of %d rows exact, %d certified near-ties" % (w.name, st["exact_rows"], R, st["near_tie_rows"]))
    return st


def test_csa_decode_128k_bf16_full():
    w = gen.WORKLOADS["csa_decode_128k_bf16"]
    inp = gen.decode_inputs(w)
    step = steps.CsaDecode(w, inp, copies=1)
    step.run()
    st = _check_decode(w, inp, step)
    assert st["near_tie_rows"] <= 1


def test_csa_decode_1m_mixed_full():
    """fp4 indexer keys and queries: per-head dots are exact, so the selection is bit-identical to the oracle's."""
    w = gen.WORKLOADS["csa_decode_1m_mixed"]
    inp = gen.decode_inputs(w)
    step = steps.CsaDecode(w, inp, copies=1)
    step.run()
    st = _check_decode(w, inp, step)
    assert st["exact_rows"] == w.B


def test_csa_decode_128k_bf16_mtp2_full():
    """Two query rows per sequence (a new token and one draft) through the decode kernels."""
    w = gen.WORKLOADS["csa_decode_128k_bf16_mtp2"]
    inp = gen.decode_inputs(w)
    step = steps.CsaDecode(w, inp, copies=1)
    step.run()
    st = _check_decode(w, inp, step)
    assert st["near_tie_rows"] <= 1


def test_csa_decode_1m_mixed_mtp2_full():
    w = gen.WORKLOADS["csa_decode_1m_mixed_mtp2"]
    inp = gen.decode_inputs(w)
    step = steps.CsaDecode(w, inp, copies=1)
    step.run()
    st = _check_decode(w, inp, step)
    assert st["exact_rows"] == w.B * w.Sq


# ------------------------------------------------------------------------------------------------------
def test_hca_decode_1m_bf16_full():
    w = gen.WORKLOADS["hca_decode_1m_bf16"]
    inp = gen.decode_inputs(w)
    step = steps.HcaDecode(w, inp, copies=1)
    step.run()
    torch.cuda.synchronize()
    B, N = w.B, w.N
    E = orc.kv_compress(inp["Ca"], None, inp["Za"], None, inp["Ba"], None, m=w.m, overlap=False, start_pos=w.n_ctx)
    check_bf16_codes(step.comp[0].host()["data"].reshape(B, N + 1, w.D)[:, N], E[:, 0])
    cc = orc.plain_cache(_bf16(inp["comp"]), "bf16")
    rc = orc.plain_cache(_bf16(inp["window_kv"]), "bf16")
    cc["cap"], rc["cap"] = N, w.window
    o_ref, l_ref = orc.attn(orc.plain_cache(_bf16(inp["q"]), "bf16"), cc, N, rc, w.n_ctx - w.window + 1, w.window, None,
                            0, w.m, inp["sink"], B, 1, w.H, w.D, w.window, w.scale, w.n_ctx)
    o = bf16_to_f64(step.out.cpu().numpy().view(np.uint16)).reshape(B, 1, w.H, w.D)
    assert row_rel_err(o, o_ref) <= 1e-2
    np.testing.assert_allclose(step.lse.cpu().numpy(), l_ref, rtol=1e-3, atol=1e-3)


def test_hca_cache_build_1m_sampled():
    """The one-off 1M-token HCA cache build (8 x 2^20 tokens -> 8 x 8192 entries) checked on sampled entries."""
    w = gen.WORKLOADS["hca_decode_1m_bf16"]
    C, Z, Ba = gen.hca_build_streams_device(w, "cuda")
    out = lca.CacheTensor("bf16", w.B, w.N, w.D)
    Bad = torch.from_numpy(Ba).cuda()
    lca.kv_compress(C, None, Z, None, Bad, None, None, None, w.B, w.n_ctx, w.D, w.m, False, 0, out.desc())
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    picks = [(b, int(i)) for b in range(w.B) for i in rng.choice(w.N, 32, replace=False)] + [(0, 0), (w.B - 1, w.N - 1)]
    got = out.data.view(w.B, w.N, w.D)
    Es, gs = [], []
    for b, i in picks:  # every sampled entry's 128 tokens copied back, compressed by the oracle, codes compared
        cs = C[b:b + 1, i * w.m:(i + 1) * w.m].cpu().numpy()
        zs = Z[b:b + 1, i * w.m:(i + 1) * w.m].cpu().numpy()
        Es.append(orc.kv_compress(cs, None, zs, None, Ba, None, m=w.m, overlap=False)[0, 0])
        gs.append(got[b, i].cpu().numpy().view(np.uint16))
    check_bf16_codes(np.stack(gs), np.stack(Es))
    # entry count: ceil(n / m)
    assert w.N == math.ceil(w.n_ctx / w.m) == 8192
    del C, Z


def test_hca_cache_build_1m_constant_values():
    """Compression weights sum to one, so a context whose values are constant per channel compresses into entries
    equal to those constants, over the whole 1M-token build: every entry of every sequence, the first block
    included, with the drawn logits and position bias.  The constants are powers of two (every product and sum then
    scales exactly) or 3, 6 and 1.5 (rounding leaves them far from a bf16 boundary), so each of the 8 x 8192 x 512
    codes is checked bit for bit -- an invariant that needs no oracle."""
    w = gen.WORKLOADS["hca_decode_1m_bf16"]
    C, Z, Ba = gen.hca_build_streams_device(w, "cuda")
    del C
    vals = torch.tensor([1.0, -2.0, 0.5, 3.0, -0.25, 6.0, 1.5, -1.0], dtype=torch.float32, device="cuda")
    chan = vals.repeat(w.D // vals.numel())
    Cc = chan.expand(w.B, w.n_ctx, w.D).contiguous()
    out = lca.CacheTensor("bf16", w.B, w.N, w.D)
    lca.kv_compress(Cc, None, Z, None, torch.from_numpy(Ba).cuda(), None, None, None, w.B, w.n_ctx, w.D, w.m, False, 0,
                    out.desc())
    torch.cuda.synchronize()
    del Cc, Z
    exp_bits = torch.from_numpy(gen.bf16_bits(chan.cpu().numpy()).astype(np.int16)).cuda()
    got = out.data.view(w.B, w.N, w.D)
    bad = int((got != exp_bits).sum().item())
    assert bad == 0, "%d of %d codes differ from the constants" % (bad, got.numel())


def test_hca_build_then_decode_1m_chained():
    """The HCA path end to end at full size, stage-isolated: the 1M-token cache built on the GPU (kv_compress over
    8 x 2^20 tokens), then hca_attn over it for every sequence, against the oracle attending the GPU-written cache
    (read back) with the same window, queries and sink."""
    w = gen.WORKLOADS["hca_decode_1m_bf16"]
    inp = gen.decode_inputs(w)
    B, N, H, D = w.B, w.N, w.H, w.D
    C, Z, Ba = gen.hca_build_streams_device(w, "cuda")
    comp = lca.CacheTensor("bf16", B, N, D)
    lca.kv_compress(C, None, Z, None, torch.from_numpy(Ba).cuda(), None, None, None, B, w.n_ctx, D, w.m, False, 0,
                    comp.desc())
    torch.cuda.synchronize()
    del C, Z
    raw = steps.make_cache("bf16", B, w.window, D, 0, inp["window_kv"])
    q = torch.from_numpy(_bf16(inp["q"]).view(np.int16)).cuda()
    sink = torch.from_numpy(inp["sink"].astype(np.float32)).cuda()
    out = torch.empty((B, 1, H, D), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
    ws_bytes = lca.hca_attn_workspace_size(B, 1, H, D, w.window + N)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    raw_start = w.n_ctx - w.window + 1
    lca.hca_attn(q, lca.LCA_BF16, comp.desc(), N, w.m, raw.desc(), raw_start, w.window, sink, B, 1, H, D, w.window,
                 w.scale, w.n_ctx, out, lca.LCA_BF16, lse, ws, ws_bytes)
    torch.cuda.synchronize()
    cc = orc.plain_cache(comp.data.view(B, N, D).cpu().numpy().view(np.uint16), "bf16")
    rc = orc.plain_cache(_bf16(inp["window_kv"]), "bf16")
    cc["cap"], rc["cap"] = N, w.window
    o_ref, l_ref = orc.attn(orc.plain_cache(_bf16(inp["q"]), "bf16"), cc, N, rc, raw_start, w.window, None, 0, w.m,
                            inp["sink"], B, 1, H, D, w.window, w.scale, w.n_ctx)
    o = bf16_to_f64(out.cpu().numpy().view(np.uint16)).reshape(B, 1, H, D)
    assert row_rel_err(o, o_ref) <= 1e-2
    np.testing.assert_allclose(lse.cpu().numpy(), l_ref, rtol=1e-3, atol=1e-3)


# ------------------------------------------------------------------------------------------------------
def test_csa_prefill_64k_chunk4k_bf16_sampled():
    """Prefill chunk: 4096 new tokens after 65536 cached ones; the GPU runs the whole chunk, the oracle checks the new
    cache entries and a sample of rows (first, last, spread)."""
    w = gen.WORKLOADS["csa_prefill_64k_chunk4k_bf16"]
    inp = gen.prefill_inputs(w)
    step = steps.CsaPrefill(w, inp)
    step.run()
    torch.cuda.synchronize()
    N0, N = step.N0, step.N
    # new entries of both caches (bf16), code by code against the oracle's compression
    Em = _compress_ref(inp, "", 4, True, w.n_ctx)
    Ek = _compress_ref(inp, "_I", 4, True, w.n_ctx)
    hm, hk = step.comp.host(), step.keys.host()
    check_bf16_codes(hm["data"].reshape(N, w.D)[N0:N], Em[0])
    check_bf16_codes(hk["data"].reshape(N, w.DI)[N0:N], Ek[0])
    # stage-isolated: the oracle scores the GPU-written key cache (given part + the chunk the GPU compressed) with the
    # plain fp32 rounding bound, on 64 rows spread over the chunk plus its first and last rows
    ck = dict(orc.plain_cache(hk["data"].reshape(1, N, w.DI), "bf16"), cap=N)
    cm = dict(orc.plain_cache(hm["data"].reshape(1, N, w.D), "bf16"), cap=N)
    rows = np.unique(np.concatenate([np.linspace(0, w.Sq - 1, 64).astype(np.int32), [1, 3, 2047, 2048]])).astype(
        np.int32)
    s64, _, ab, _ = orc.indexer_scores(orc.plain_cache(_bf16(inp["qI"]), "bf16"), inp["w"], ck, 1, w.Sq, w.HI, w.DI, N,
                                       4, w.n_ctx, rows=rows, want_abs=True)
    nv = orc.nvis_rows(1, rows, w.n_ctx, 4, N)
    gidx = step.idx.cpu().numpy()[0, rows]
    st = check_topk(gidx, step.scores.cpu().numpy()[0, rows], s64.reshape(len(rows), N), ab.reshape(len(rows), N), nv,
                    w.k, GAMMA(w.DI, w.HI))
    print("prefill: %d of %d rows exact, %d certified near-ties" % (st["exact_rows"], len(rows), st["near_tie_rows"]))
    assert st["near_tie_rows"] <= 2
    # attention over the GPU's own selection and latent cache, every sampled row
    raw = orc.plain_cache(_bf16(inp["raw_kv"]), "bf16")
    raw["cap"] = inp["raw_kv"].shape[1]
    full_idx = np.full((1, w.Sq, w.k), -1, np.int32)
    full_idx[0, rows] = gidx
    o_ref, l_ref = orc.attn(orc.plain_cache(_bf16(inp["q"]), "bf16"), cm, N, raw, inp["raw_start"], raw["cap"],
                            full_idx, w.k, 0, inp["sink"], 1, w.Sq, w.H, w.D, w.window, w.scale, w.n_ctx, rows=rows)
    o = bf16_to_f64(step.out.cpu().numpy()[0, rows].view(np.uint16))
    assert row_rel_err(o, o_ref[0]) <= 1e-2
    np.testing.assert_allclose(step.lse.cpu().numpy()[0, rows], l_ref[0], rtol=1e-4, atol=1e-4)
