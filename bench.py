#!/usr/bin/env python3
"""Benchmark of one layer step of the CSA/HCA compressed attention on one MI355X.

Default workload: CSA decode at 1M context with the mixed-precision cache (batch 4, 262144 compressed entries per
sequence; 448 fp8 + 64 bf16 channels per entry, fp4 indexer keys and queries; 64 query heads, indexer 64 x 128,
top-1024, window 128 + sink).  A step = kv_compress append (latent + indexer key) -> indexer_score_topk ->
sparse_mqa_attn, on inputs already resident in HBM; the appends write the provisional entry of the new token's
block, which no query of the step reads, so they run on a second stream beside the indexer and the attention.

Timing: the steps are captured in a HIP graph, one step per cache copy, and the graph is replayed; the step time is
the median over 20 windows of replays, each bracketed by HIP events.  The appends of all the graph's steps run on a
second stream, forked once before the first step and joined once after the last.  The streamed cache (indexer keys; the latent
cache for HCA) is kept in enough independent copies that the replays stream at least --stream-gb GB of distinct
addresses, so no step is served from the 256 MB last-level cache; a warm line (one copy, every step on the same
addresses) is reported beside it.  The dominant kernel is timed by HIP events that each of its launches stamps with
its own start and end, in eager steps queued back to back right after the replays.

Prints one JSON line: whole-step throughput (tokens/s = sequences decoded per second), the step's algorithmic HBM
rate, the roofline of the dominant kernel, a measured read-stream rate, and the CPU oracle timed on a bounded sample
of the same workload on this host.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA/HCA layer decode tokens/s at 128K–1M ctx; achieved HBM TB/s vs peak"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3  # 256 CUs x 4 SIMDs x 64 lanes x 2 flops per fused multiply-add x 2.4 GHz


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=280, help="timed steps (at least 20 windows of whole graph replays)")
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="csa_decode_1m_mixed")
    p.add_argument("--copies", type=int, default=4, help="copies of the gathered latent cache")
    p.add_argument("--stream-gb", type=float, default=1.0,
                   help="distinct bytes of the streamed cache (indexer keys; HCA: the latent cache) the steps rotate "
                        "through")
    p.add_argument("--no-warm", action="store_true", help="skip the warm (single copy) measurement")
    p.add_argument("--paged", action="store_true",
                   help="CSA decode: hold the latent cache and the indexer keys as block-managed (paged) tensors, "
                        "32 entries (128 tokens) per block in a shuffled pool behind a block table")
    p.add_argument("--no-cache-build", action="store_true",
                   help="HCA decode: skip timing the one-off build of the whole compressed cache from the context's "
                        "token streams")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="before the steps, run one device copy of this many MiB (a known-size reference for HBM "
                        "byte counters collected around the run)")
    return p.parse_args()


class HipEvents:
    """hipEvent_t pairs through the HIP runtime that torch already loaded, created for timing only
    (hipEventDisableSystemFence: no cache writeback and invalidation when they complete, which would otherwise add
    to the interval they measure)."""

    DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str, workload: str, src_files, per_launch_units: float):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on the current source and
    build flags (the hash covers the kernel's source files and the build script)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash(src_files):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline_csa_decode(w, inp, sample_seqs: int, min_wall_s: float = 1.0):
    """The oracle, as it stands, on `sample_seqs` sequences of the decode step (append, score, top-k, attend),
    repeated until at least `min_wall_s` of wall time (about 10-30 s of CPU time on the machine's cores) has passed."""
    from oracle import oracle as orc
    S = sample_seqs
    sl = slice(0, S)
    reps, t0 = 0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < min_wall_s:
        _oracle_csa_decode_once(w, inp, S, sl)
        reps += 1
    dt = time.perf_counter() - t0
    return dict(value=reps * S * w.Sq / dt, unit="tokens/s", cores=orc.num_threads(), kind="oracle",
                sample="%d repetition(s) of %d of %d sequences of one decode step of %d token(s) (compress append, "
                       "fp64 indexer scores over all %d entries, top-%d, attention); %.2f s wall"
                       % (reps, S, w.B, w.Sq, w.N, w.k, dt))


def _oracle_csa_decode_once(w, inp, S, sl):
    import numpy as np
    import lca_inputs as gen
    from oracle import oracle as orc
    for tag in ("", "_I"):
        orc.kv_compress(inp["Ca" + tag][sl], inp["Cb" + tag][sl], inp["Za" + tag][sl], inp["Zb" + tag][sl],
                        inp["Ba" + tag], inp["Bb" + tag], inp["tail_Cb" + tag][sl], inp["tail_Zb" + tag][sl], m=4,
                        overlap=True, start_pos=w.n_ctx)
    if w.key_fmt == "fp4":
        kc = orc.encode(inp["keys"][sl].reshape(-1, w.DI), "fp4")
        qc = orc.encode(inp["qI"][sl].reshape(-1, w.DI), "fp4")
    else:
        kc = orc.plain_cache(gen.bf16_bits(inp["keys"][sl]), "bf16")
        qc = orc.plain_cache(gen.bf16_bits(inp["qI"][sl]), "bf16")
    kc["cap"] = w.N
    Sq = w.Sq
    s64, s32, _, _ = orc.indexer_scores(qc, inp["w"][sl], kc, S, Sq, w.HI, w.DI, w.N, 4, w.n_ctx,
                                        canonical=(w.key_fmt == "fp4"))
    scores = s32.astype(np.float64) if s32 is not None else s64
    idx, _, _ = orc.topk(scores.reshape(S * Sq, w.N), orc.nvis_rows(S, list(range(Sq)), w.n_ctx, 4, w.N), w.k)
    if w.main_fmt == "mixed":
        cc = orc.encode(inp["comp"][sl].reshape(-1, w.D), "mixed", w.rope)
        rc = orc.encode(inp["window_kv"][sl].reshape(-1, w.D), "mixed", w.rope)
    else:
        cc = orc.plain_cache(gen.bf16_bits(inp["comp"][sl]), "bf16")
        rc = orc.plain_cache(gen.bf16_bits(inp["window_kv"][sl]), "bf16")
    S_raw = w.window + Sq - 1
    cc["cap"], rc["cap"] = w.N, S_raw
    qa = orc.plain_cache(gen.bf16_bits(inp["q"][sl]), "bf16")
    orc.attn(qa, cc, w.N, rc, w.n_ctx - w.window + 1, S_raw, idx.reshape(S, Sq, w.k), w.k, 0, inp["sink"], S, Sq,
             w.H, w.D, w.window, w.scale, w.n_ctx)


def cpu_baseline_csa_prefill(w, inp, sample_rows: int, min_wall_s: float = 1.0):
    """The oracle on `sample_rows` query rows of the prefill chunk (the chunk's compression, fp64 indexer scores of
    those rows over every visible entry, top-k, attention), repeated for at least `min_wall_s` of wall time."""
    from oracle import oracle as orc
    reps, t0 = 0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < min_wall_s:
        _oracle_csa_prefill_once(w, inp, sample_rows)
        reps += 1
    dt = time.perf_counter() - t0
    return dict(value=reps * sample_rows / dt, unit="tokens/s", cores=orc.num_threads(), kind="oracle",
                sample="%d repetition(s) of %d of the %d query rows of the prefill chunk (compression of both streams, "
                       "fp64 indexer scores over every visible entry, top-%d, attention); %.2f s wall"
                       % (reps, sample_rows, w.Sq, w.k, dt))


def _oracle_csa_prefill_once(w, inp, rows_n):
    import numpy as np
    import lca_inputs as gen
    from oracle import oracle as orc
    ents = {}
    for tag in ("", "_I"):
        E = orc.kv_compress(inp["Ca" + tag], inp["Cb" + tag], inp["Za" + tag], inp["Zb" + tag], inp["Ba" + tag],
                            inp["Bb" + tag], inp.get("tail_Cb" + tag), inp.get("tail_Zb" + tag), m=4, overlap=True,
                            start_pos=w.n_ctx)
        ents[tag] = gen.bf16_bits(E.astype(np.float32))
    N0 = w.N
    N = (w.n_ctx + w.Sq) // w.m
    # the given cached part (none without context) followed by the chunk's own entries
    keys = np.concatenate([gen.bf16_bits(inp["keys"]), ents["_I"]], axis=1) if N0 else ents["_I"]
    comp = np.concatenate([gen.bf16_bits(inp["comp"]), ents[""]], axis=1) if N0 else ents[""]
    assert keys.shape[1] == N and comp.shape[1] == N and N0 < N
    rows = np.linspace(0, w.Sq - 1, rows_n).astype(np.int32)
    kc = dict(orc.plain_cache(keys, "bf16"), cap=N)
    qc = orc.plain_cache(gen.bf16_bits(inp["qI"]), "bf16")
    s64, _, _, _ = orc.indexer_scores(qc, inp["w"], kc, w.B, w.Sq, w.HI, w.DI, N, w.m, w.n_ctx, rows=rows)
    idx_r, _, _ = orc.topk(s64.reshape(rows_n, N), orc.nvis_rows(w.B, rows, w.n_ctx, w.m, N), w.k)
    idx = np.full((w.B, w.Sq, w.k), -1, np.int32)
    idx[0, rows] = idx_r
    cc = dict(orc.plain_cache(comp, "bf16"), cap=N)
    rc = dict(orc.plain_cache(gen.bf16_bits(inp["raw_kv"]), "bf16"), cap=inp["raw_kv"].shape[1])
    orc.attn(orc.plain_cache(gen.bf16_bits(inp["q"]), "bf16"), cc, N, rc, inp["raw_start"], inp["raw_kv"].shape[1],
             idx, w.k, 0, inp["sink"], w.B, w.Sq, w.H, w.D, w.window, w.scale, w.n_ctx, rows=rows)


def cpu_baseline_hca_decode(w, inp, sample_seqs: int, min_wall_s: float = 1.0):
    import lca_inputs as gen
    from oracle import oracle as orc
    S = sample_seqs
    sl = slice(0, S)
    reps, t0 = 0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < min_wall_s:
        _oracle_hca_decode_once(w, inp, S, sl)
        reps += 1
    dt = time.perf_counter() - t0
    return dict(value=reps * S / dt, unit="tokens/s", cores=orc.num_threads(), kind="oracle",
                sample="%d repetition(s) of %d of %d sequences of one HCA decode step (append + dense attention over "
                       "%d entries); %.2f s wall" % (reps, S, w.B, w.N, dt))


def _oracle_hca_decode_once(w, inp, S, sl):
    import lca_inputs as gen
    from oracle import oracle as orc
    orc.kv_compress(inp["Ca"][sl], None, inp["Za"][sl], None, inp["Ba"], None, m=w.m, overlap=False,
                    start_pos=w.n_ctx)
    cc = orc.plain_cache(gen.bf16_bits(inp["comp"][sl]), "bf16")
    rc = orc.plain_cache(gen.bf16_bits(inp["window_kv"][sl]), "bf16")
    cc["cap"], rc["cap"] = w.N, w.window
    qa = orc.plain_cache(gen.bf16_bits(inp["q"][sl]), "bf16")
    orc.attn(qa, cc, w.N, rc, w.n_ctx - w.window + 1, w.window, None, 0, w.m, inp["sink"], S, 1, w.H, w.D, w.window,
             w.scale, w.n_ctx)


def measured_read_peak(lca, torch, nbytes: int = 2 << 30):
    """Best rate of the library's plain streaming read (lca_stream_read) over a few grid sizes: the read stream HBM
    sustains on this device, reported next to the published peak."""
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = None
    for wg in (1024, 2048, 4096, 8192):
        for _ in range(2):
            lca.lca_stream_read(src, nbytes, out, wg)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in evs:
            a.record()
            lca.lca_stream_read(src, nbytes, out, wg)
            b.record()
        torch.cuda.synchronize()
        ms = min(a.elapsed_time(b) for a, b in evs)
        gbps = nbytes / (ms / 1e3) / 1e9
        if best is None or gbps > best[0]:
            best = (gbps, wg)
    del src, out
    return {"GBps": best[0], "bytes": nbytes, "workgroups": best[1], "kernel": "stream_read_kernel"}


def time_cache_build(w, torch, lca, gen, runs: int = 5):
    """The one-off HCA cache build: kv_compress over every token of the context (B x n_ctx rows of the C and Z
    streams, fp32) into the bf16 compressed cache, timed with HIP events around each of `runs` builds (median).
    Algorithmic bytes: both streams read once plus the cache written once."""
    from long_context_attention_05_amd import steps as steps_mod
    rope = w.rope if w.main_fmt == "mixed" else 0
    C, Z, Ba = gen.hca_build_streams_device(w, "cuda")
    out = lca.CacheTensor(w.main_fmt, w.B, w.N, w.D, rope)
    Bad = torch.from_numpy(Ba).cuda()

    def build():
        lca.kv_compress(C, None, Z, None, Bad, None, None, None, w.B, w.n_ctx, w.D, w.m, False, 0, out.desc())

    build()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for a, b in evs:
        a.record()
        build()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[runs // 2]
    nbytes = 2 * w.B * w.n_ctx * w.D * 4 + w.B * w.N * steps_mod._entry_bytes(w.main_fmt, w.D, rope)
    del C, Z, out
    torch.cuda.empty_cache()
    return {"kernel": "compress_kernel", "tokens": w.B * w.n_ctx, "entries": w.B * w.N, "ms": ms,
            "algorithmic_bytes": nbytes, "achieved_GBps": nbytes / (ms / 1e3) / 1e9,
            "frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "timed_with": "HIP events around each of %d whole builds (median)" % runs}


def time_steps(step, torch, steps_mod, n_distinct: int, steps: int, warmup: int, ev, set_events, windows: int = 20,
               same_copy: bool = False, head_start=None):
    """Capture n_distinct consecutive steps (one per cache copy; all on copy 0 when same_copy) in a HIP graph and
    replay it.  Every step's appends run on a second stream, forked before the first step and joined after the last
    (steps_mod.run_many).

    Returns (median ms per step over the windows, steps timed, per-launch ms of the dominant kernel, how it was
    timed).  The dominant kernel is timed by HIP events that each of its launches stamps with its own start and end
    (the library's hook) in eager steps right after the replays, one per cache copy.  head_start(), when given,
    enqueues a few milliseconds of unrelated GPU work first, so that the host queues the eager steps faster than the
    GPU runs them and each one starts right behind the previous one, as in the graph."""
    side = torch.cuda.Stream()  # default priority, like every stream here
    order = [0 if same_copy else c for c in range(n_distinct)]
    # eager warm-up outside the graph (first-use setup such as kernel attributes happens here)
    for _ in range(max(1, warmup // max(1, n_distinct))):
        steps_mod.run_many(step, order, side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps_mod.run_many(step, order, side)
    reps = max(1, -(-steps // (windows * n_distinct)))
    for _ in range(max(1, warmup // n_distinct)):
        g.replay()
    torch.cuda.synchronize()
    wins = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(windows)]
    for a, b in wins:
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) / (reps * n_distinct) for a, b in wins)
    med = 0.5 * (per_step[(windows - 1) // 2] + per_step[windows // 2])
    del g
    # eager steps back to back on one stream (no fork), so that each timed launch queues behind the previous work
    n_k = max(2 * n_distinct, 20)
    pairs = [(ev.create(), ev.create()) for _ in range(n_k)]
    if head_start is not None:
        head_start()
    for i in range(n_k):
        set_events(pairs[i][0], pairs[i][1])
        step.run(0 if same_copy else i % n_distinct, None, None)
    set_events(None, None)
    torch.cuda.synchronize()
    kms = [ev.elapsed_ms(a, b) for a, b in pairs]
    how = ("dispatch-stamped HIP events (hipExtLaunchKernel, no system fence) on each of %d launches in eager steps "
           "queued back to back%s" % (n_k, " behind a head start of GPU work" if head_start is not None else ""))
    return med, windows * reps * n_distinct, sum(kms) / len(kms), how


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer path runs on a single MI355X and has no multi-GPU mode "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np  # noqa: F401
    import torch
    import lca_inputs as gen
    from long_context_attention_05_amd import lca, steps

    w = gen.WORKLOADS[args.workload]
    torch.cuda.init()
    t_gen = time.perf_counter()
    stream_bytes = int(args.stream_gb * 1e9)
    if w.is_decode:
        inp = gen.decode_inputs(w)
        if w.layer == "swa":
            per_copy = steps._entry_bytes(w.main_fmt, w.D, w.rope) * w.B * (w.window + w.Sq - 1)
            n_distinct = max(args.copies, -(-stream_bytes // per_copy))
            step = steps.SwaDecode(w, inp, copies=n_distinct)
            streamed = n_distinct * per_copy
        elif w.HI == 0:
            per_copy = steps._entry_bytes(w.main_fmt, w.D, w.rope) * w.B * w.N
            n_distinct = max(args.copies, -(-stream_bytes // per_copy))
            step = steps.HcaDecode(w, inp, copies=n_distinct)
            streamed = n_distinct * per_copy
        elif w.layer == "shared2":
            per_copy = steps._entry_bytes(w.key_fmt, w.DI, 0) * w.B * w.N
            key_copies = max(args.copies, -(-stream_bytes // per_copy))
            step = steps.CsaDecodeShared(w, inp, [gen.layer_inputs(w, 1)], copies=args.copies, key_copies=key_copies)
            n_distinct = step.copies
            streamed = key_copies * per_copy
        else:
            per_copy = steps._entry_bytes(w.key_fmt, w.DI, 0) * w.B * w.N
            key_copies = max(args.copies, -(-stream_bytes // per_copy))
            step = steps.CsaDecode(w, inp, copies=args.copies, key_copies=key_copies,
                                   block_rows=32 if args.paged else 0)
            n_distinct = step.copies
            streamed = key_copies * per_copy
    else:
        inp = gen.prefill_inputs(w)
        step = steps.CsaPrefill(w, inp)
        n_distinct, streamed = 1, 0
    torch.cuda.synchronize()
    print("inputs ready in %.1f s (%d distinct steps, %.2f GB of streamed cache)" %
          (time.perf_counter() - t_gen, n_distinct, streamed / 1e9), file=sys.stderr, flush=True)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src_t = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst_t = torch.empty_like(src_t)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t

    ev = HipEvents()
    has_scores = w.HI > 0 and w.layer != "swa"  # CSA: the indexer scoring kernel dominates; else the attention
    set_events = lca.lca_set_score_events if has_scores else lca.lca_set_attn_events
    # a head start for the eager launches: reads of a 1 GiB buffer, enough to queue the eager steps behind them
    hs_buf = torch.empty(1 << 28, dtype=torch.int32, device="cuda").fill_(1)
    hs_out = torch.zeros(1, dtype=torch.int32, device="cuda")

    def head_start(reads: int = 16):
        for _ in range(reads):
            lca.lca_stream_read(hs_buf, hs_buf.numel() * 4, hs_out, 4096)

    ms_per_step, K, avg_ms, how = time_steps(step, torch, steps, n_distinct, args.steps, args.warmup, ev, set_events,
                                             head_start=head_start)
    print("timed %d steps (graph replays): %.4f ms/step; dominant kernel %.2f us" % (K, ms_per_step, avg_ms * 1e3),
          file=sys.stderr, flush=True)
    warm = None
    if w.is_decode and not args.no_warm and n_distinct > 1:
        wms, wk, wavg, _ = time_steps(step, torch, steps, n_distinct, args.steps, args.warmup, ev,
                                      set_events, same_copy=True, head_start=head_start)
        warm = {"label": "warm: one cache copy, every step on the same addresses (last-level cache hits)",
                "ms_per_step": wms, "value": w.B * w.Sq / (wms / 1e3), "steps": wk, "dominant_kernel_us": wavg * 1e3}

    tokens = w.B * w.Sq  # tokens through the step (a shared-selection step carries them through two layers)
    value = tokens / (ms_per_step / 1e3)
    res = {"metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": {"bf16": "bf16", "mixed": "bf16/fp8/fp4"}[w.main_fmt] if w.main_fmt != "f32" else "f32",
           "data": "synthetic",
           "config": {"workload": w.name, "batch": w.B, "context_tokens": w.n_ctx, "query_rows": w.Sq,
                      "compress_ratio": w.m, "latent_dim": w.D, "heads": w.H, "indexer": [w.HI, w.DI], "topk": w.k,
                      "window": w.window, "cache_format": w.main_fmt, "key_format": w.key_fmt,
                      "distinct_steps": n_distinct, "streamed_cache_bytes": streamed,
                      "cache_layout": ("paged: 32-entry (128-token) blocks in a shuffled pool" if
                                       getattr(step, "block_rows", 0) else "dense"),
                      "timing": "HIP graph of %d steps replayed, median of 20 event windows" % n_distinct}}
    if hasattr(step, "step_bytes"):
        sb = step.step_bytes()
        res["step_algorithmic_bytes"] = sb
        res["achieved_hbm_GBps"] = sb / (ms_per_step / 1e3) / 1e9
        res["hbm_frac_of_peak"] = res["achieved_hbm_GBps"] / HBM_PEAK_GBPS
    res["step_algorithmic_flops"] = step.step_flops()
    res["achieved_TFLOPs"] = step.step_flops() / (ms_per_step / 1e3) / 1e12
    if warm:
        res["warm"] = warm

    if not has_scores:
        src = ["long_context_attention_05_amd/csrc/attn.hip", "long_context_attention_05_amd/csrc/lca_device.h",
               "long_context_attention_05_amd/build.py"]
        if w.layer == "swa":  # few rows, a 128-entry window list: the two-pass decode attention (both passes timed)
            kname = "attn_dec_score_kernel+attn_dec_value_kernel"
            per_launch = step.step_bytes()
        else:  # dense HCA rows: the many-row kernel over a bf16 cache, the wide kernel over the mixed cache
            kname = "attn_pfs_kernel" if w.main_fmt == "bf16" else "attn_wide_kernel"
            per_launch = step.attn_kernel_bytes()
        achieved = per_launch / (avg_ms / 1e3) / 1e9
        res["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBPS,
                           "traffic": traffic_record(kname, w.name, src, per_launch),
                           "avg_launch_us": avg_ms * 1e3, "algorithmic_bytes_per_launch": per_launch,
                           "timed_with": how}
    src = ["long_context_attention_05_amd/csrc/indexer.hip", "long_context_attention_05_amd/csrc/lca_device.h",
           "long_context_attention_05_amd/build.py"]
    if has_scores:
        if w.is_decode:
            kname = "idx_score_decode_fp4_ring" if w.key_fmt == "fp4" else "idx_score_decode_bf16"
            per_launch = step.score_kernel_bytes()
            achieved = per_launch / (avg_ms / 1e3) / 1e9
            res["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": achieved,
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                               # counters taken on the dense layout say nothing of a paged one
                               "traffic": traffic_record(kname, w.name + ("_paged" if args.paged else ""), src,
                                                         per_launch),
                               "avg_launch_us": avg_ms * 1e3, "algorithmic_bytes_per_launch": per_launch,
                               "timed_with": how}
        else:
            per_launch = step.score_kernel_flops()
            achieved = per_launch / (avg_ms / 1e3) / 1e12
            # 64 heads x 128 dims of bf16 take the MFMA kernel; other shapes and fp32 the vector-ALU one
            mfma = w.HI == 64 and w.DI == 128 and w.key_fmt == "bf16"
            kname, bound, peak = (("idx_score_mfma", "mfma", BF16_PEAK_TFLOPS) if mfma else
                                  ("idx_score_simt", "alu", FP32_VECTOR_PEAK_TFLOPS))
            res["roofline"] = {"kernel": kname, "bound": bound, "achieved": achieved,
                               "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                               "traffic": traffic_record(kname, w.name, src, per_launch),
                               "avg_launch_us": avg_ms * 1e3, "algorithmic_flops_per_launch": per_launch,
                               "timed_with": how}
    del step, hs_buf
    torch.cuda.empty_cache()
    if w.is_decode and w.HI == 0 and w.layer != "swa" and not args.no_cache_build:
        res["cache_build"] = time_cache_build(w, torch, lca, gen)
        print("cache build: %.3f ms (%.0f GB/s)" % (res["cache_build"]["ms"], res["cache_build"]["achieved_GBps"]),
              file=sys.stderr, flush=True)
    if res["roofline"]["bound"] == "hbm":
        rp = measured_read_peak(lca, torch)
        res["roofline"]["measured_read_peak"] = rp
        res["roofline"]["frac_of_measured_read_peak"] = res["roofline"]["achieved"] / rp["GBps"]
        if "achieved_hbm_GBps" in res:
            res["step_frac_of_measured_read_peak"] = res["achieved_hbm_GBps"] / rp["GBps"]
        if "cache_build" in res:
            res["cache_build"]["frac_of_measured_read_peak"] = res["cache_build"]["achieved_GBps"] / rp["GBps"]
    if not args.no_cpu_baseline:
        if w.layer in ("swa", "shared2"):
            pass  # extra lines beside the five workloads: no CPU baseline
        elif w.is_decode and w.HI > 0:
            res["cpu_baseline"] = cpu_baseline_csa_decode(w, inp, sample_seqs=w.B)
        elif w.is_decode:
            res["cpu_baseline"] = cpu_baseline_hca_decode(w, inp, sample_seqs=w.B)
        else:
            res["cpu_baseline"] = cpu_baseline_csa_prefill(w, inp, sample_rows=16)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
