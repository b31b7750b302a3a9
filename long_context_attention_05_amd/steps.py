"""One layer step as a fixed sequence of C-ABI calls over preallocated device buffers.

A CSA decode step is: kv_compress (append the new token to the latent cache and to the indexer-key cache) ->
indexer_score_topk -> sparse_mqa_attn.  An HCA decode step is kv_compress -> hca_attn.  A CSA prefill chunk is
kv_compress of the chunk (both caches) -> indexer_score_topk -> sparse_mqa_attn over every row of the chunk.
This module only allocates buffers, uploads the caller's host arrays and sequences the calls; all arithmetic runs
in liblca.so.  `copies` > 1 keeps independent copies of the large caches so that consecutive steps read distinct
addresses (the 256 MB last-level cache then cannot serve a repeated step); the streamed indexer-key cache can be
copied more often than the gathered latent cache (`key_copies`).

run(c, stream, side): with a side stream, the two compression appends (which write the provisional entry of the
new token's block, read by no query of this step) run on the side stream beside the indexer and the attention;
the side stream joins the main one at the end of the step (a fork and a join, also inside a captured graph).
"""
from __future__ import annotations

import numpy as np
import torch

from . import lca

DEV = "cuda"


def _up(x: np.ndarray) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).to(DEV)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _entry_bytes(fmt: str, dim: int, rope: int) -> int:
    return {"f32": 4 * dim, "bf16": 2 * dim, "mixed": (dim - rope) + 2 * rope + 4, "fp4": dim // 2 + dim // 32}[fmt]


def make_cache(fmt: str, B: int, cap: int, dim: int, rope: int, x: np.ndarray | None) -> lca.CacheTensor:
    """Cache of `cap` rows per sequence; rows [0, x.shape[1]) hold x (bf16 by cast of the given values, mixed/fp4
    encoded on the GPU by lca_encode)."""
    c = lca.CacheTensor(fmt, B, cap, dim, rope)
    if x is None:
        return c
    rows = x.shape[1]
    if fmt == "bf16":
        c.data.view(B, cap, dim)[:, :rows] = _up(_bf16_bits(x))
    elif fmt == "f32":
        c.data.view(B, cap, dim)[:, :rows] = _up(x.astype(np.float32))
    else:
        for b in range(B):  # one sequence at a time keeps the fp32 staging buffer small
            src = _up(x[b:b + 1].astype(np.float32))
            d = c.desc()
            d.data = c.data[b * cap:].data_ptr()
            d.rope = None if c.rope_t is None else c.rope_t[b * cap:].data_ptr()
            d.scale = c.scale_t[b * cap:].data_ptr()
            d.cap = cap
            lca.lca_encode(src, 1, rows, 0, d)
            del src
    return c


def to_paged(c: lca.CacheTensor, block_rows: int, seed: int) -> lca.PagedCache:
    """The same cache as a paged tensor: its blocks of block_rows rows moved to a shuffled pool (block j of the
    dense layout, j = b * cap / block_rows + jj, goes to pool block perm[j]) and a block table pointing at them.  A
    device gather; no arithmetic."""
    cap = (c.cap + block_rows - 1) // block_rows * block_rows
    nblk = cap // block_rows
    B = c.B
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(B * nblk).astype(np.int64)).to(DEV)
    table = perm.to(torch.int32).view(B, nblk).contiguous()
    p = lca.PagedCache(c.fmt, B, cap, c.dim, c.rope, block_rows, table, B * nblk, flags=c.flags)

    def move(dst, src):
        if src is None:
            return
        w = src.shape[1:] if src.dim() > 1 else ()
        s = src.view(B, c.cap, *w)
        padded = torch.zeros((B, cap) + tuple(w), dtype=src.dtype, device=DEV)
        padded[:, :c.cap] = s
        dst.view(B * nblk, block_rows, *w)[perm] = padded.view(B * nblk, block_rows, *w)

    move(p.data, c.data)
    move(p.rope_t, c.rope_t)
    move(p.scale_t, c.scale_t)
    return p


def clone_cache(c: lca.CacheTensor) -> lca.CacheTensor:
    n = c.__class__.__new__(c.__class__)
    n.__dict__.update(c.__dict__)
    n.data = c.data.clone()
    n.rope_t = None if c.rope_t is None else c.rope_t.clone()
    n.scale_t = None if c.scale_t is None else c.scale_t.clone()
    return n


class _Streams:
    """Device copies of one set of compression streams."""

    def __init__(self, inp: dict, tag: str, overlap: bool, with_tail: bool):
        self.Ca, self.Za = _up(inp["Ca" + tag]), _up(inp["Za" + tag])
        self.Ba = _up(inp["Ba" + tag])
        self.Cb = self.Zb = self.Bb = self.tCb = self.tZb = None
        if overlap:
            self.Cb, self.Zb, self.Bb = _up(inp["Cb" + tag]), _up(inp["Zb" + tag]), _up(inp["Bb" + tag])
            if with_tail:
                self.tCb, self.tZb = _up(inp["tail_Cb" + tag]), _up(inp["tail_Zb" + tag])
        self.B, self.n, self.c = inp["Ca" + tag].shape
        self.nbytes = sum(t.numel() * 4 for t in (self.Ca, self.Za, self.Cb, self.Zb, self.tCb, self.tZb)
                          if t is not None)

    def compress(self, m: int, overlap: bool, start_pos: int, out: lca.CacheTensor, stream=None):
        lca.kv_compress(self.Ca, self.Cb, self.Za, self.Zb, self.Ba, self.Bb, self.tCb, self.tZb, self.B, self.n,
                        self.c, m, overlap, start_pos, out.desc(), stream)


def _fork_join(side_work, main_work, stream, side):
    """main_work on `stream`; side_work before it on the same stream, or beside it on `side` (joined at the end)."""
    if side is None:
        side_work(stream)
        main_work(stream)
        return
    main = torch.cuda.current_stream()
    assert stream is None or stream == main.cuda_stream, "a forked step runs on torch's current stream"
    side.wait_stream(main)
    side_work(side.cuda_stream)
    main_work(main.cuda_stream)
    main.wait_stream(side)


def run_many(step, copies, side=None):
    """Steps on the given cache copies in order, on torch's current stream.  With a side stream, every step's
    appends run there (forked once before the first step and joined once after the last), beside the indexer and
    attention chain of all the steps: an append writes the provisional entry of its token's block, which no query
    reads before that block's later tokens have been appended again, and each copy holds its own caches."""
    if side is None or not getattr(step, "forkable", True):
        for c in copies:
            step.run(c, None)
        return
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    for c in copies:
        step.append(c, side.cuda_stream)
    for c in copies:
        step.attend(c, main.cuda_stream)
    main.wait_stream(side)


class CsaDecode:
    """CSA decode step of a batch of B sequences holding n_ctx tokens (N = n_ctx / 4 committed entries); Sq <= 4
    new tokens per sequence (the new token and its drafts) are appended, scored and attended together."""

    def __init__(self, w, inp: dict, copies: int = 1, key_copies: int | None = None, block_rows: int = 0):
        self.w = w
        B, N, D, DI, HI, H, k, Sq = w.B, w.N, w.D, w.DI, w.HI, w.H, w.k, w.Sq
        key_copies = copies if key_copies is None else key_copies
        self.copies = max(copies, key_copies)  # distinct steps before the addresses repeat
        cap = N + 1  # room for the provisional entry of the block the new token starts
        base_comp = make_cache(w.main_fmt, B, cap, D, w.rope, inp["comp"])
        base_keys = make_cache(w.key_fmt, B, cap, DI, 0, inp["keys"])
        self.block_rows = block_rows
        if block_rows:  # block-managed caches: shuffled pools behind block tables
            base_comp = to_paged(base_comp, block_rows, w.seed + 500)
            base_keys = to_paged(base_keys, block_rows, w.seed + 501)
            torch.cuda.synchronize()
        self.S_raw = w.window + Sq - 1
        base_raw = make_cache(w.main_fmt, B, self.S_raw, D, w.rope, inp["window_kv"])
        self.comp = [base_comp] + [clone_cache(base_comp) for _ in range(copies - 1)]
        self.keys = [base_keys] + [clone_cache(base_keys) for _ in range(key_copies - 1)]
        self.raw = [base_raw] + [clone_cache(base_raw) for _ in range(self.copies - 1)]
        self.q = _up(_bf16_bits(inp["q"]))
        if w.qi_fmt == "fp4":
            self.qI = make_cache("fp4", B, Sq * HI, DI, 0, inp["qI"].reshape(B, Sq * HI, DI))
            self.qI_desc = self.qI.desc()
        else:
            self.qI = _up(_bf16_bits(inp["qI"]))
            self.qI_desc = lca.plain_desc(self.qI, "bf16", DI, Sq * HI)
        self.wgt = _up(inp["w"])
        self.sink = _up(inp["sink"])
        self.main = _Streams(inp, "", True, True)
        self.ind = _Streams(inp, "_I", True, True)
        self.idx = torch.empty((B, Sq, k), dtype=torch.int32, device=DEV)
        self.scores = torch.empty((B, Sq, k), dtype=torch.float32, device=DEV)
        self.out = torch.empty((B, Sq, H, D), dtype=torch.int16, device=DEV)
        self.lse = torch.empty((B, Sq, H), dtype=torch.float32, device=DEV)
        self.ws_i_bytes = lca.indexer_score_topk_workspace_size(B, Sq, N, k)
        self.ws_a_bytes = lca.sparse_mqa_attn_workspace_size(B, Sq, H, D, w.window + k)
        self.ws_i = torch.empty(max(self.ws_i_bytes, 256), dtype=torch.uint8, device=DEV)
        self.ws_a = torch.empty(max(self.ws_a_bytes, 256), dtype=torch.uint8, device=DEV)
        self.raw_start = w.n_ctx - w.window + 1

    def append(self, c: int, st):
        """The new tokens' entries: latent cache and indexer keys (the provisional entry N of copy c)."""
        w = self.w
        self.main.compress(4, True, w.n_ctx, self.comp[c % len(self.comp)], st)
        self.ind.compress(4, True, w.n_ctx, self.keys[c % len(self.keys)], st)

    def attend(self, c: int, st):
        """Indexer scores and top-k over copy c's keys, then attention over its latent cache and window."""
        w = self.w
        comp, keys, raw = (self.comp[c % len(self.comp)], self.keys[c % len(self.keys)],
                           self.raw[c % len(self.raw)])
        lca.indexer_score_topk(self.qI_desc, self.wgt, keys.desc(), w.B, w.Sq, w.HI, w.DI, w.N, 4, w.k, w.n_ctx,
                               self.idx, self.scores, self.ws_i, self.ws_i_bytes, st)
        lca.sparse_mqa_attn(self.q, lca.LCA_BF16, comp.desc(), w.N, raw.desc(), self.raw_start, self.S_raw, self.idx,
                            w.k, self.sink, w.B, w.Sq, w.H, w.D, w.window, w.scale, w.n_ctx, self.out, lca.LCA_BF16,
                            self.lse, self.ws_a, self.ws_a_bytes, st)

    def run(self, c: int = 0, stream=None, side=None):
        _fork_join(lambda st: self.append(c, st), lambda st: self.attend(c, st), stream, side)

    # algorithmic traffic and work of one step (what the method must move / compute)
    def score_kernel_bytes(self) -> int:
        w = self.w
        key_b = _entry_bytes(w.key_fmt, w.DI, 0) * w.B * w.N  # every visible key once, whatever Sq
        qi_b = _entry_bytes(w.qi_fmt, w.DI, 0) * w.B * w.Sq * w.HI
        return key_b + qi_b + 4 * w.B * w.Sq * w.HI

    def step_bytes(self) -> int:
        w = self.w
        eb = _entry_bytes(w.main_fmt, w.D, w.rope)
        gather = eb * w.B * w.Sq * (w.k + w.window)
        q_out = 2 * 2 * w.B * w.Sq * w.H * w.D
        idx = 2 * 4 * w.B * w.Sq * w.k
        return self.score_kernel_bytes() + gather + q_out + idx + self.main.nbytes + self.ind.nbytes

    def step_flops(self) -> int:
        w = self.w
        return w.Sq * (2 * w.B * w.HI * w.DI * w.N + 4 * w.B * w.H * w.D * (w.k + w.window))


class CsaDecodeShared(CsaDecode):
    """Cross-layer reuse of the indexer's selection (cosmocat page, section 7: from V4.1 the layers reuse the
    compression and the index instead of each computing its own): one indexer_score_topk per step feeds the
    attention of `layers` consecutive CSA layers.  Each layer keeps its own latent cache, window, queries and sink
    (and appends its own new entry); the indexer keys and their append are shared."""

    def __init__(self, w, inp: dict, layer_inputs: list, copies: int = 1, key_copies: int | None = None):
        super().__init__(w, inp, copies, key_copies)
        B, N, D, H, Sq = w.B, w.N, w.D, w.H, w.Sq
        self.layers = []
        for li in layer_inputs:
            base_comp = make_cache(w.main_fmt, B, N + 1, D, w.rope, li["comp"])
            base_raw = make_cache(w.main_fmt, B, self.S_raw, D, w.rope, li["window_kv"])
            L = dict(comp=[base_comp] + [clone_cache(base_comp) for _ in range(copies - 1)],
                     raw=[base_raw] + [clone_cache(base_raw) for _ in range(copies - 1)],
                     q=_up(_bf16_bits(li["q"])), sink=_up(li["sink"]), main=_Streams(li, "", True, True),
                     out=torch.empty((B, Sq, H, D), dtype=torch.int16, device=DEV),
                     lse=torch.empty((B, Sq, H), dtype=torch.float32, device=DEV),
                     ws=torch.empty(max(self.ws_a_bytes, 256), dtype=torch.uint8, device=DEV))
            self.layers.append(L)

    def _layers(self, c: int):
        comps = [self.comp[c % len(self.comp)]] + [L["comp"][c % len(L["comp"])] for L in self.layers]
        raws = [self.raw[c % len(self.raw)]] + [L["raw"][c % len(L["raw"])] for L in self.layers]
        per_layer = [(self.main, self.q, self.sink, self.out, self.lse, self.ws_a)] + [
            (L["main"], L["q"], L["sink"], L["out"], L["lse"], L["ws"]) for L in self.layers]
        return comps, raws, per_layer

    def append(self, c: int, st):
        w = self.w
        comps, _, per_layer = self._layers(c)
        for (main, *_), comp in zip(per_layer, comps):
            main.compress(4, True, w.n_ctx, comp, st)
        self.ind.compress(4, True, w.n_ctx, self.keys[c % len(self.keys)], st)

    def attend(self, c: int, st):
        w = self.w
        comps, raws, per_layer = self._layers(c)
        lca.indexer_score_topk(self.qI_desc, self.wgt, self.keys[c % len(self.keys)].desc(), w.B, w.Sq, w.HI, w.DI,
                               w.N, 4, w.k, w.n_ctx, self.idx, self.scores, self.ws_i, self.ws_i_bytes, st)
        for (_, q, sink, out, lse, ws), comp, raw in zip(per_layer, comps, raws):
            lca.sparse_mqa_attn(q, lca.LCA_BF16, comp.desc(), w.N, raw.desc(), self.raw_start, self.S_raw, self.idx,
                                w.k, sink, w.B, w.Sq, w.H, w.D, w.window, w.scale, w.n_ctx, out, lca.LCA_BF16, lse, ws,
                                self.ws_a_bytes, st)

    def step_bytes(self) -> int:
        w = self.w
        eb = _entry_bytes(w.main_fmt, w.D, w.rope)
        per_layer = eb * w.B * w.Sq * (w.k + w.window) + 2 * 2 * w.B * w.Sq * w.H * w.D + self.main.nbytes
        return self.score_kernel_bytes() + 2 * 4 * w.B * w.Sq * w.k + self.ind.nbytes + per_layer * (
            1 + len(self.layers))

    def step_flops(self) -> int:
        w = self.w
        return w.Sq * (2 * w.B * w.HI * w.DI * w.N + (1 + len(self.layers)) * 4 * w.B * w.H * w.D * (w.k + w.window))


class SwaDecode:
    """The ratio-0 layer (paper notes, section 2.4: the last entry of the config's compress_ratios is 0, a pure
    sliding-window layer): attention over the last `window` raw tokens and the sink, no compressed entries
    (sparse_mqa_attn with k = 0, no index list, an empty compressed tensor)."""

    def __init__(self, w, inp: dict, copies: int = 1):
        self.w = w
        self.copies = copies
        B, D, H, Sq = w.B, w.D, w.H, w.Sq
        self.S_raw = w.window + Sq - 1
        base_raw = make_cache(w.main_fmt, B, self.S_raw, D, w.rope, inp["window_kv"])
        self.raw = [base_raw] + [clone_cache(base_raw) for _ in range(copies - 1)]
        self.q = _up(_bf16_bits(inp["q"]))
        self.sink = _up(inp["sink"])
        self.out = torch.empty((B, Sq, H, D), dtype=torch.int16, device=DEV)
        self.lse = torch.empty((B, Sq, H), dtype=torch.float32, device=DEV)
        self.ws_bytes = lca.sparse_mqa_attn_workspace_size(B, Sq, H, D, w.window)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=DEV)
        self.raw_start = w.n_ctx - w.window + 1
        fmt = lca.FORMATS[w.main_fmt]
        self.no_comp = lca.lca_tensor(fmt, D, w.rope if w.main_fmt == "mixed" else 0, 1, None, None, None, 0)

    def append(self, c: int, st):
        pass  # the window is the raw state cache; nothing is compressed

    def attend(self, c: int, st):
        w = self.w
        raw = self.raw[c % len(self.raw)]
        lca.sparse_mqa_attn(self.q, lca.LCA_BF16, self.no_comp, 0, raw.desc(), self.raw_start, self.S_raw, None, 0,
                            self.sink, w.B, w.Sq, w.H, w.D, w.window, w.scale, w.n_ctx, self.out, lca.LCA_BF16,
                            self.lse, self.ws, self.ws_bytes, st)

    def run(self, c: int = 0, stream=None, side=None):
        self.attend(c, stream)

    def step_bytes(self) -> int:
        w = self.w
        return _entry_bytes(w.main_fmt, w.D, w.rope) * w.B * w.Sq * w.window + 2 * 2 * w.B * w.Sq * w.H * w.D

    def step_flops(self) -> int:
        w = self.w
        return 4 * w.B * w.Sq * w.H * w.D * w.window


class HcaDecode:
    """HCA decode step: B sequences of n_ctx tokens, N = n_ctx / 128 entries, dense attention."""

    def __init__(self, w, inp: dict, copies: int = 1):
        self.w = w
        self.copies = copies
        B, N, D, H = w.B, w.N, w.D, w.H
        base_comp = make_cache(w.main_fmt, B, N + 1, D, w.rope, inp["comp"])
        base_raw = make_cache(w.main_fmt, B, w.window, D, w.rope, inp["window_kv"])
        self.comp = [base_comp] + [clone_cache(base_comp) for _ in range(copies - 1)]
        self.raw = [base_raw] + [clone_cache(base_raw) for _ in range(copies - 1)]
        self.q = _up(_bf16_bits(inp["q"]))
        self.sink = _up(inp["sink"])
        self.main = _Streams(inp, "", False, False)
        self.out = torch.empty((B, 1, H, D), dtype=torch.int16, device=DEV)
        self.lse = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
        self.ws_bytes = lca.hca_attn_workspace_size(B, 1, H, D, w.window + N)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=DEV)
        self.raw_start = w.n_ctx - w.window + 1

    def append(self, c: int, st):
        self.main.compress(self.w.m, False, self.w.n_ctx, self.comp[c % len(self.comp)], st)

    def attend(self, c: int, st):
        w = self.w
        comp, raw = self.comp[c % len(self.comp)], self.raw[c % len(self.raw)]
        lca.hca_attn(self.q, lca.LCA_BF16, comp.desc(), w.N, w.m, raw.desc(), self.raw_start, w.window, self.sink,
                     w.B, 1, w.H, w.D, w.window, w.scale, w.n_ctx, self.out, lca.LCA_BF16, self.lse, self.ws,
                     self.ws_bytes, st)

    def run(self, c: int = 0, stream=None, side=None):
        _fork_join(lambda st: self.append(c, st), lambda st: self.attend(c, st), stream, side)

    def step_bytes(self) -> int:
        w = self.w
        eb = _entry_bytes(w.main_fmt, w.D, w.rope)
        return eb * w.B * (w.N + w.window) + 2 * 2 * w.B * w.H * w.D + self.main.nbytes

    def attn_kernel_bytes(self) -> int:
        """Algorithmic bytes one attention launch must read: every visible entry and the window once, q once."""
        w = self.w
        eb = _entry_bytes(w.main_fmt, w.D, w.rope)
        return eb * w.B * (w.N + w.window) + 2 * w.B * w.H * w.D

    def step_flops(self) -> int:
        w = self.w
        return 4 * w.B * w.H * w.D * (w.N + w.window)


class CsaPrefill:
    """CSA prefill chunk: Sq new tokens after n_ctx cached ones (N0 = n_ctx / 4 given entries)."""

    def __init__(self, w, inp: dict):
        self.w = w
        B, D, DI, HI, H, k, Sq = w.B, w.D, w.DI, w.HI, w.H, w.k, w.Sq
        self.N0 = w.n_ctx // w.m
        self.N = (w.n_ctx + Sq) // w.m
        self.comp = make_cache(w.main_fmt, B, self.N, D, w.rope, inp.get("comp"))
        self.keys = make_cache(w.key_fmt, B, self.N, DI, 0, inp.get("keys"))
        self.raw_start = inp["raw_start"]
        self.S_raw = inp["raw_kv"].shape[1]
        self.raw = make_cache(w.main_fmt, B, self.S_raw, D, w.rope, inp["raw_kv"])
        self.q = _up(_bf16_bits(inp["q"]))
        self.qI = _up(_bf16_bits(inp["qI"]))
        self.qI_desc = lca.plain_desc(self.qI, "bf16", DI, Sq * HI)
        self.wgt = _up(inp["w"])
        self.sink = _up(inp["sink"])
        self.main = _Streams(inp, "", True, w.n_ctx > 0)
        self.ind = _Streams(inp, "_I", True, w.n_ctx > 0)
        self.idx = torch.empty((B, Sq, k), dtype=torch.int32, device=DEV)
        self.scores = torch.empty((B, Sq, k), dtype=torch.float32, device=DEV)
        self.out = torch.empty((B, Sq, H, D), dtype=torch.int16, device=DEV)
        self.lse = torch.empty((B, Sq, H), dtype=torch.float32, device=DEV)
        self.ws_i_bytes = lca.indexer_score_topk_workspace_size(B, Sq, self.N, k)
        self.ws_a_bytes = lca.sparse_mqa_attn_workspace_size(B, Sq, H, D, w.window + k)
        self.ws_i = torch.empty(max(self.ws_i_bytes, 256), dtype=torch.uint8, device=DEV)
        self.ws_a = torch.empty(max(self.ws_a_bytes, 256), dtype=torch.uint8, device=DEV)

    copies = 1
    forkable = False  # the chunk's own entries are read by its later rows: compression precedes the indexer

    def run(self, c: int = 0, stream=None, side=None):
        w = self.w
        self.main.compress(4, True, w.n_ctx, self.comp, stream)
        self.ind.compress(4, True, w.n_ctx, self.keys, stream)
        lca.indexer_score_topk(self.qI_desc, self.wgt, self.keys.desc(), w.B, w.Sq, w.HI, w.DI, self.N, 4, w.k,
                               w.n_ctx, self.idx, self.scores, self.ws_i, self.ws_i_bytes, stream)
        lca.sparse_mqa_attn(self.q, lca.LCA_BF16, self.comp.desc(), self.N, self.raw.desc(), self.raw_start, self.S_raw,
                            self.idx, w.k, self.sink, w.B, w.Sq, w.H, w.D, w.window, w.scale, w.n_ctx, self.out,
                            lca.LCA_BF16, self.lse, self.ws_a, self.ws_a_bytes, stream)

    def visible_pairs(self) -> int:
        w = self.w
        t = w.n_ctx + np.arange(w.Sq, dtype=np.int64)
        return int(np.minimum(t // w.m, self.N).sum()) * w.B

    def score_kernel_flops(self) -> int:
        return 2 * self.w.HI * self.w.DI * self.visible_pairs()

    def step_flops(self) -> int:
        w = self.w
        return self.score_kernel_flops() + 4 * w.B * w.Sq * w.H * w.D * (w.k + w.window)
