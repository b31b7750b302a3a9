"""Checkpoint and resume of the decode state through the C-ABI: after a decode step (token n), the compressed
latent cache, the fp4 indexer keys, the raw window and the current block's token streams are written to disk and
read back into fresh device buffers; the next step (token n + 1, which re-compresses the provisional entry of the
block from its two tokens) then gives bit-identical selections, outputs and caches from the original and from the
restored state."""
import numpy as np
import pytest
import torch

import lca_inputs as gen
from long_context_attention_05_amd import lca
from tests.gpu_util import up

pytestmark = pytest.mark.gpu


def _save(path, c: lca.CacheTensor):
    arrs = {k: getattr(c, k).cpu().numpy() for k in ("data", "rope_t", "scale_t") if getattr(c, k) is not None}
    np.savez(path, **arrs)


def _load(path, like: lca.CacheTensor) -> lca.CacheTensor:
    c = lca.CacheTensor(like.fmt, like.B, like.cap, like.dim, like.rope)
    with np.load(path, allow_pickle=False) as z:
        for k in z.files:
            getattr(c, k).copy_(torch.from_numpy(z[k]).cuda())
    return c


def test_decode_resumes_from_saved_state(tmp_path):
    w = gen.scaled(gen.WORKLOADS["csa_decode_1m_mixed"], B=2, n_ctx=4 * 8192, k=256)
    g = gen.rng(120)
    B, N, D, DI, H, HI, W = w.B, w.N, w.D, w.DI, w.H, w.HI, w.window
    n = w.n_ctx  # token n starts block N (provisional entry N)
    comp = lca.CacheTensor("mixed", B, N + 1, D, w.rope)
    keys = lca.CacheTensor("fp4", B, N + 1, DI)
    raw = lca.CacheTensor("mixed", B, W + 1, D, w.rope)  # positions n - W + 1 .. n + 1
    lca.lca_encode(up(gen.normal(g, (B, N, D))), B, N, 0, comp.desc())
    lca.lca_encode(up(gen.normal(g, (B, N, DI))), B, N, 0, keys.desc())
    lca.lca_encode(up(gen.normal(g, (B, W + 1, D))), B, W + 1, 0, raw.desc())
    streams = {tag: {x: gen.normal(g, (B, 2, c)) for x in ("Ca", "Cb", "Za", "Zb")} for tag, c in (("", D), ("_I", DI))}
    tails = {tag: {x: gen.normal(g, (B, 4, c)) for x in ("tail_Cb", "tail_Zb")} for tag, c in (("", D), ("_I", DI))}
    bias = {tag: {x: gen.normal(g, (4, c), 0.1) for x in ("Ba", "Bb")} for tag, c in (("", D), ("_I", DI))}
    qI = lca.CacheTensor("fp4", B, 2 * HI, DI)
    lca.lca_encode(up(gen.normal(g, (B, 2 * HI, DI))), B, 2 * HI, 0, qI.desc())
    wts = up(gen.normal(g, (B, 2, HI), 1.0 / np.sqrt(DI * HI)))
    q = up(gen.bf16_bits(gen.normal(g, (B, 2, H, D))))
    sink = up(gen.normal(g, (H,)))

    def step(t, comp, keys, raw):
        """Decode token t (n or n + 1): append the block's tokens n .. t, score, select, attend."""
        r = t - n
        for tag, cache, c in (("", comp, D), ("_I", keys, DI)):
            s = {x: up(np.ascontiguousarray(v[:, :r + 1])) for x, v in streams[tag].items()}
            tl = {x: up(v) for x, v in tails[tag].items()}
            bs = {x: up(v) for x, v in bias[tag].items()}
            lca.kv_compress(s["Ca"], s["Cb"], s["Za"], s["Zb"], bs["Ba"], bs["Bb"], tl["tail_Cb"], tl["tail_Zb"], B,
                            r + 1, c, 4, True, n, cache.desc())
        idx = torch.empty((B, 1, w.k), dtype=torch.int32, device="cuda")
        sc = torch.empty((B, 1, w.k), dtype=torch.float32, device="cuda")
        # one query row per call: row r's slices of the query tensors, weights and queries
        qrows = lca.CacheTensor("fp4", B, HI, DI)
        qrows.data.view(B, HI, -1).copy_(qI.data.view(B, 2 * HI, -1)[:, r * HI:(r + 1) * HI])
        qrows.scale_t.view(B, HI, -1).copy_(qI.scale_t.view(B, 2 * HI, -1)[:, r * HI:(r + 1) * HI])
        wr = wts[:, r:r + 1].contiguous()
        nb = lca.indexer_score_topk_workspace_size(B, 1, N, w.k)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        lca.indexer_score_topk(qrows.desc(), wr, keys.desc(), B, 1, HI, DI, N, 4, w.k, t, idx, sc, ws, nb)
        out = torch.empty((B, 1, H, D), dtype=torch.int16, device="cuda")
        lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
        na = lca.sparse_mqa_attn_workspace_size(B, 1, H, D, W + w.k)
        wa = torch.empty(max(na, 256), dtype=torch.uint8, device="cuda")
        lca.sparse_mqa_attn(q[:, r:r + 1].contiguous(), lca.LCA_BF16, comp.desc(), N, raw.desc(), n - W + 1, W + 1,
                            idx, w.k, sink, B, 1, H, D, W, w.scale, t, out, lca.LCA_BF16, lse, wa, na)
        torch.cuda.synchronize()
        return idx, sc, out, lse

    step(n, comp, keys, raw)
    for name, c in (("comp", comp), ("keys", keys), ("raw", raw)):
        _save(tmp_path / (name + ".npz"), c)
    comp2, keys2, raw2 = (_load(tmp_path / (nm + ".npz"), c) for nm, c in (("comp", comp), ("keys", keys),
                                                                             ("raw", raw)))
    a = step(n + 1, comp, keys, raw)
    b = step(n + 1, comp2, keys2, raw2)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y)
    for c1, c2 in ((comp, comp2), (keys, keys2), (raw, raw2)):
        assert torch.equal(c1.data, c2.data) and (c1.scale_t is None or torch.equal(c1.scale_t, c2.scale_t))
    # the resumed step re-wrote the provisional entry N from two tokens: it differs from the one-token entry
    assert (a[0] >= 0).all()
