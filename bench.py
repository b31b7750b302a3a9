#!/usr/bin/env python3
"""Benchmark of one layer step of the CSA/HCA compressed attention on one MI355X.

Default workload: CSA decode at 128K context, bf16 (batch 16, 32768 compressed entries per sequence, 64 query heads,
indexer 64 x 128, top-512, window 128 + sink).  A step = kv_compress append (latent + indexer key) ->
indexer_score_topk -> sparse_mqa_attn, on inputs already resident in HBM.  Large caches are kept in `--copies`
independent copies used round-robin so that a step cannot be served from the 256 MB last-level cache.

Prints one JSON line: whole-step throughput (tokens/s = sequences decoded per second), the step's algorithmic HBM
rate, the roofline of the dominant kernel (indexer scoring, timed with HIP events around each of its launches) and
the CPU oracle timed on a bounded sample of the same workload on this host.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="csa_decode_128k_bf16")
    p.add_argument("--copies", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="before the steps, run one device copy of this many MiB (a known-size reference for HBM "
                        "byte counters collected around the run)")
    return p.parse_args()


class HipEvents:
    """hipEvent_t pairs through the HIP runtime that torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
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


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer path runs on a single MI355X and has no multi-GPU mode "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import lca_inputs as gen
    from long_context_attention_05_amd import lca, steps

    w = gen.WORKLOADS[args.workload]
    torch.cuda.init()
    t_gen = time.perf_counter()
    if w.is_decode:
        inp = gen.decode_inputs(w)
        step = (steps.HcaDecode if w.HI == 0 else steps.CsaDecode)(w, inp, copies=args.copies)
        copies = args.copies
    else:
        inp = gen.prefill_inputs(w)
        step = steps.CsaPrefill(w, inp)
        copies = 1
    torch.cuda.synchronize()
    print("inputs ready in %.1f s" % (time.perf_counter() - t_gen), file=sys.stderr, flush=True)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src_t = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        dst_t = torch.empty_like(src_t)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t

    ev = HipEvents()
    has_scores = w.HI > 0   # CSA: the indexer scoring kernel dominates; HCA: the attention kernel
    K = args.steps
    pairs = [(ev.create(), ev.create()) for _ in range(K)]
    set_events = lca.lca_set_score_events if has_scores else lca.lca_set_attn_events
    stream = torch.cuda.current_stream().cuda_stream

    for i in range(args.warmup):
        step.run(i % copies, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        set_events(pairs[i][0], pairs[i][1])
        step.run(i % copies, stream)
    set_events(None, None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / K
    print("timed %d steps: %.4f ms/step" % (K, ms_per_step), file=sys.stderr, flush=True)

    tokens = w.B * w.Sq
    value = tokens / (ms_per_step / 1e3)
    res = {"metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": {"bf16": "bf16", "mixed": "bf16/fp8/fp4"}[w.main_fmt] if w.main_fmt != "f32" else "f32",
           "data": "synthetic",
           "config": {"workload": w.name, "batch": w.B, "context_tokens": w.n_ctx, "query_rows": w.Sq,
                      "compress_ratio": w.m, "latent_dim": w.D, "heads": w.H, "indexer": [w.HI, w.DI], "topk": w.k,
                      "window": w.window, "cache_format": w.main_fmt, "key_format": w.key_fmt,
                      "rotated_copies": copies}}
    if hasattr(step, "step_bytes"):
        sb = step.step_bytes()
        res["step_algorithmic_bytes"] = sb
        res["achieved_hbm_GBps"] = sb / (ms_per_step / 1e3) / 1e9
        res["hbm_frac_of_peak"] = res["achieved_hbm_GBps"] / HBM_PEAK_GBPS
    res["step_algorithmic_flops"] = step.step_flops()
    res["achieved_TFLOPs"] = step.step_flops() / (ms_per_step / 1e3) / 1e12

    durs = [ev.elapsed_ms(a, b) for a, b in pairs]
    avg_ms = sum(durs) / len(durs)
    if not has_scores:
        src = ["long_context_attention_05_amd/csrc/attn.hip", "long_context_attention_05_amd/csrc/lca_device.h",
               "long_context_attention_05_amd/build.py"]
        # dense HCA rows: the many-row kernel over a bf16 cache, the wide kernel over the mixed cache
        kname = "attn_pfs_kernel" if w.main_fmt == "bf16" else "attn_wide_kernel"
        per_launch = step.attn_kernel_bytes()
        achieved = per_launch / (avg_ms / 1e3) / 1e9
        res["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBPS,
                           "traffic": traffic_record(kname, w.name, src, per_launch),
                           "avg_launch_us": avg_ms * 1e3, "algorithmic_bytes_per_launch": per_launch}
    src = ["long_context_attention_05_amd/csrc/indexer.hip", "long_context_attention_05_amd/csrc/lca_device.h",
           "long_context_attention_05_amd/build.py"]
    if has_scores:
        if w.is_decode:
            kname = "idx_score_decode_fp4_ring" if w.key_fmt == "fp4" else "idx_score_decode_bf16"
            per_launch = step.score_kernel_bytes()
            achieved = per_launch / (avg_ms / 1e3) / 1e9
            res["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": achieved,
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                               "traffic": traffic_record(kname, w.name, src, per_launch),
                               "avg_launch_us": avg_ms * 1e3, "algorithmic_bytes_per_launch": per_launch}
        else:
            per_launch = step.score_kernel_flops()
            achieved = per_launch / (avg_ms / 1e3) / 1e12
            res["roofline"] = {"kernel": "idx_score_mfma", "bound": "mfma", "achieved": achieved,
                               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                               "traffic": traffic_record("idx_score_mfma", w.name, src, per_launch),
                               "avg_launch_us": avg_ms * 1e3, "algorithmic_flops_per_launch": per_launch}
    if not args.no_cpu_baseline:
        if w.is_decode and w.HI > 0:
            res["cpu_baseline"] = cpu_baseline_csa_decode(w, inp, sample_seqs=w.B)
        elif w.is_decode:
            res["cpu_baseline"] = cpu_baseline_hca_decode(w, inp, sample_seqs=w.B)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
