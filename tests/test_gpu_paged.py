"""Block-managed (paged) caches and ragged batches (itsolotime page, question 5: the compressed cache is managed in
blocks of lcm(4, 128) = 128 tokens -- 32 CSA entries, one HCA entry -- and a serving batch holds sequences of
different lengths), through the C-ABI:
  - decode at the 128K bf16 and 1M mixed shapes (one and two query rows per sequence) with shuffled block tables and
    every sequence at its own position:
    the GPU's paged results equal its dense results bit for bit, the selection matches the oracle's (bit-exact for
    fp4) and every attention row matches the oracle attending the GPU's selection;
  - kv_compress appends into a paged cache with ragged starts and token counts;
  - dense HCA rows over a one-entry-per-block table."""
import numpy as np
import pytest
import torch

import lca_inputs as gen
from oracle import oracle as orc
from tests.gpu_util import bf16_to_f64, check_topk, row_rel_err, up

pytestmark = pytest.mark.gpu

steps = pytest.importorskip("long_context_attention_05_amd.steps")
lca = pytest.importorskip("long_context_attention_05_amd.lca")

GAMMA = lambda DI, HI: 2.0 * (DI + HI) * 2.0 ** -24  # noqa: E731


def _ragged_positions(w, seed):
    """Positions at most the workload's n_ctx, each sequence different (some not a multiple of m)."""
    g = np.random.default_rng(seed)
    pos = w.n_ctx - g.integers(0, min(w.n_ctx // 3, 5000), w.B)
    pos[0] = w.n_ctx
    return pos.astype(np.int64)


def _decode(w, inp, block_rows, pos):
    """One decode call sequence (indexer + attention) over dense or paged caches at per-sequence positions."""
    step = steps.CsaDecode(w, inp, block_rows=block_rows)
    dpos = torch.from_numpy(pos).cuda()
    rg = lca.ragged(dpos)
    q0 = int(pos.max())
    raw_start = q0 - w.window + 1
    lca.indexer_score_topk(step.qI_desc, step.wgt, step.keys[0].desc(), w.B, w.Sq, w.HI, w.DI, w.N, 4, w.k, q0,
                           step.idx, step.scores, step.ws_i, step.ws_i_bytes, ragged=rg)
    lca.sparse_mqa_attn(step.q, lca.LCA_BF16, step.comp[0].desc(), w.N, step.raw[0].desc(), raw_start, step.S_raw,
                        step.idx, w.k, step.sink, w.B, w.Sq, w.H, w.D, w.window, w.scale, q0, step.out, lca.LCA_BF16,
                        step.lse, step.ws_a, step.ws_a_bytes, ragged=rg)
    torch.cuda.synchronize()
    return step


@pytest.mark.parametrize("name", ["csa_decode_128k_bf16", "csa_decode_1m_mixed", "csa_decode_128k_bf16_mtp2",
                                  "csa_decode_1m_mixed_mtp2"])
def test_paged_ragged_decode_full(name):
    # (the two-row workloads score both rows of a sequence in one workgroup from the same paged key stages)
    w = gen.WORKLOADS[name]
    inp = gen.decode_inputs(w)
    pos = _ragged_positions(w, 401)
    print("paged ragged decode %s: positions %s" % (name, pos.tolist()), flush=True)
    dense = _decode(w, inp, 0, pos)
    paged = _decode(w, inp, 32, pos)
    assert isinstance(paged.keys[0], lca.PagedCache) and isinstance(paged.comp[0], lca.PagedCache)
    # the same kernels over the same bytes: bit-identical
    assert torch.equal(paged.idx, dense.idx) and torch.equal(paged.scores.view(torch.int32),
                                                             dense.scores.view(torch.int32))
    assert torch.equal(paged.out, dense.out) and torch.equal(paged.lse.view(torch.int32), dense.lse.view(torch.int32))
    # against the oracle: each sequence at its own position
    B, N, R = w.B, w.N, w.B * w.Sq
    exact = w.key_fmt == "fp4"
    if exact:
        kc = orc.encode(inp["keys"].reshape(-1, w.DI), "fp4")
        qc = orc.encode(inp["qI"].reshape(-1, w.DI), "fp4")
    else:
        kc = orc.plain_cache(gen.bf16_bits(inp["keys"]), "bf16")
        qc = orc.plain_cache(gen.bf16_bits(inp["qI"]), "bf16")
    kc["cap"] = N
    s64, s32, ab, bad = orc.indexer_scores(qc, inp["w"], kc, B, w.Sq, w.HI, w.DI, N, 4, int(pos.max()),
                                           canonical=exact, want_abs=True, seq_pos=pos)
    if exact:
        assert bad == 0
    nv = np.concatenate([orc.nvis_rows(1, np.arange(w.Sq), int(p), 4, N) for p in pos])
    assert len(set(nv.tolist())) > 1
    gidx = paged.idx.cpu().numpy().reshape(R, w.k)
    st = check_topk(gidx, paged.scores.cpu().numpy().reshape(R, w.k), s64.reshape(R, N), ab.reshape(R, N), nv, w.k,
                    GAMMA(w.DI, w.HI), exact=exact, s32=None if s32 is None else s32.reshape(R, N))
    assert st["near_tie_rows"] <= max(1, R // 16)
    if w.main_fmt == "mixed":
        cc = orc.encode(inp["comp"].reshape(-1, w.D), "mixed", w.rope)
        rc = orc.encode(inp["window_kv"].reshape(-1, w.D), "mixed", w.rope)
    else:
        cc = orc.plain_cache(gen.bf16_bits(inp["comp"]), "bf16")
        rc = orc.plain_cache(gen.bf16_bits(inp["window_kv"]), "bf16")
    cc["cap"], rc["cap"] = N, paged.S_raw
    q0 = int(pos.max())
    o_ref, l_ref = orc.attn(orc.plain_cache(gen.bf16_bits(inp["q"]), "bf16"), cc, N, rc, q0 - w.window + 1,
                            paged.S_raw, gidx.reshape(B, w.Sq, w.k), w.k, 0, inp["sink"], B, w.Sq, w.H, w.D, w.window,
                            w.scale, q0, seq_pos=pos)
    o = bf16_to_f64(paged.out.cpu().numpy().view(np.uint16))
    assert row_rel_err(o, o_ref) <= 1e-2
    np.testing.assert_allclose(paged.lse.cpu().numpy(), l_ref, rtol=1e-4, atol=1e-4)


def test_paged_ragged_compress_append():
    """Appends into a paged latent cache (mixed format) and paged fp4 keys: sequence b appends len[b] tokens from
    its own block start pos[b]; the entries land through the table at pos[b] / 4 + i."""
    g = np.random.default_rng(402)
    B, n, m = 6, 8, 4
    pos = np.array([0, 4, 400, 1020, 96, 2048], np.int64)
    lens = np.array([8, 1, 3, 4, 6, 5], np.int32)
    cap = 1024
    for fmt, c, rope in (("mixed", 512, 64), ("fp4", 128, 0)):
        f = lambda *s: g.standard_normal(s).astype(np.float32)  # noqa: E731
        S = dict(Ca=f(B, n, c), Cb=f(B, n, c), Za=f(B, n, c), Zb=f(B, n, c), Ba=0.1 * f(m, c), Bb=0.1 * f(m, c),
                 tail_Cb=f(B, m, c), tail_Zb=f(B, m, c))
        dense = lca.CacheTensor(fmt, B, cap, c, rope)
        for t in (dense.data, dense.rope_t, dense.scale_t):
            if t is not None:
                t.zero_()
        paged = steps.to_paged(dense, 32, 403)
        d = {k: up(v.astype(np.float32)) for k, v in S.items()}
        rg = lca.ragged(torch.from_numpy(pos).cuda(), torch.from_numpy(lens).cuda())
        for out in (dense, paged):
            lca.kv_compress(d["Ca"], d["Cb"], d["Za"], d["Zb"], d["Ba"], d["Bb"], d["tail_Cb"], d["tail_Zb"], B, n, c,
                            m, True, int(pos.max()), out.desc(), ragged=rg)
        torch.cuda.synchronize()
        back = steps.to_paged(dense, 32, 403)  # dense -> the same shuffled layout, to compare the pools bytewise
        torch.cuda.synchronize()
        assert torch.equal(back.data, paged.data) and torch.equal(back.scale_t, paged.scale_t)
        h = dense.host()
        for b in range(B):
            sl = lambda x: np.ascontiguousarray(x[b:b + 1, :lens[b]])  # noqa: E731
            E = orc.kv_compress(sl(S["Ca"]), sl(S["Cb"]), sl(S["Za"]), sl(S["Zb"]), S["Ba"], S["Bb"],
                                np.ascontiguousarray(S["tail_Cb"][b:b + 1]), np.ascontiguousarray(S["tail_Zb"][b:b + 1]),
                                m=m, overlap=True, start_pos=int(pos[b]))
            e0, ne = int(pos[b]) // m, E.shape[1]
            rows = slice(b * cap + e0, b * cap + e0 + ne)
            if fmt == "mixed":
                got = dict(data=h["data"][rows], rope_data=h["rope_data"][rows], scale=h["scale"][rows])
                from tests.gpu_util import check_mixed_codes
                check_mixed_codes(got, E[0], rope)
            else:
                from tests.gpu_util import check_fp4_codes
                check_fp4_codes(dict(data=h["data"][rows], scale=h["scale"][rows]), E[0])
            # nothing else of the sequence was written
            others = np.ones(cap, bool)
            others[e0:e0 + ne] = False
            assert not h["data"][b * cap:(b + 1) * cap][others].any()


def test_paged_hca_one_entry_per_block():
    """Dense HCA rows over a 1M-token cache held as one entry per 128-token block (block_rows = 1), ragged."""
    w = gen.scaled(gen.WORKLOADS["hca_decode_1m_bf16"], B=4, n_ctx=1 << 18)
    inp = gen.decode_inputs(w)
    pos = np.array([w.n_ctx, w.n_ctx - 128 * 37 - 5, w.n_ctx - 3, w.n_ctx - 128 * 500], np.int64)
    base = steps.HcaDecode(w, inp)
    paged_comp = steps.to_paged(base.comp[0], 1, 404)
    torch.cuda.synchronize()
    rg = lca.ragged(torch.from_numpy(pos).cuda())
    q0 = int(pos.max())
    outs = []
    for comp in (base.comp[0], paged_comp):
        out = torch.empty_like(base.out)
        lse = torch.empty_like(base.lse)
        lca.hca_attn(base.q, lca.LCA_BF16, comp.desc(), w.N, w.m, base.raw[0].desc(), q0 - w.window + 1, w.window,
                     base.sink, w.B, 1, w.H, w.D, w.window, w.scale, q0, out, lca.LCA_BF16, lse, base.ws, base.ws_bytes,
                     ragged=rg)
        outs.append((out, lse))
    torch.cuda.synchronize()
    cc = dict(orc.plain_cache(gen.bf16_bits(inp["comp"]), "bf16"), cap=w.N)
    rc = dict(orc.plain_cache(gen.bf16_bits(inp["window_kv"]), "bf16"), cap=w.window)
    o_ref, l_ref = orc.attn(orc.plain_cache(gen.bf16_bits(inp["q"]), "bf16"), cc, w.N, rc, q0 - w.window + 1, w.window,
                            None, 0, w.m, inp["sink"], w.B, 1, w.H, w.D, w.window, w.scale, q0, seq_pos=pos)
    for out, lse in outs:
        o = bf16_to_f64(out.cpu().numpy().view(np.uint16))
        assert row_rel_err(o, o_ref) <= 1e-2
        np.testing.assert_allclose(lse.cpu().numpy(), l_ref, rtol=1e-4, atol=1e-4)
    assert torch.equal(outs[0][0], outs[1][0])
