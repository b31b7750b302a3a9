"""Seeded synthetic inputs for the CSA/HCA compressed-attention layer.

This module only draws random numbers and arranges them into the shapes of the workloads; it holds none of
the layer's arithmetic.  Both the HIP path (tests, benchmark) and the CPU oracle take their inputs from
here.  Values that a workload declares as bfloat16 are produced by torch's float32 -> bfloat16 cast (a
library cast of the draws); values that a workload stores in fp8/fp4 are returned as float32 and each
side quantises them with its own codec.

Draw order: one numpy Generator(PCG64(seed)) per workload; tensors are drawn in the order they are listed in
each function, each as standard normals in float32 (numpy's float32 ziggurat), then scaled.
"N(0, 0.1)" is read as standard deviation 0.1.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, via torch's cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 values (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """Shape of one layer invocation."""
    name: str
    seed: int
    B: int
    n_ctx: int          # tokens already in the context (compressed part)
    Sq: int             # query rows per sequence in the call
    m: int              # compression ratio
    D: int              # latent (key = value) dim
    rope: int           # trailing RoPE dims
    H: int              # query heads (MQA)
    HI: int             # indexer heads (0 for HCA)
    DI: int             # indexer head dim
    k: int              # top-k (0 for HCA)
    window: int
    main_fmt: str       # compressed / window KV cache format
    key_fmt: str        # indexer key format
    q_fmt: str          # attention query dtype ("f32" | "bf16")
    qi_fmt: str         # indexer query format
    q_std: float        # std of the attention queries
    scale: float        # softmax scale sigma
    layer: str = ""     # "" (CSA if HI else HCA), "swa" (ratio-0 window-only layer) or "shared2" (two CSA layers
                        # whose attention shares one indexer selection)

    @property
    def N(self) -> int:
        return self.n_ctx // self.m

    @property
    def is_decode(self) -> bool:
        """A decode step: one token, or a few draft tokens verified together, against a given cache."""
        return self.n_ctx > 0 and self.Sq <= 4


# The five workloads of the layer (sizes from the pages' 128K-1M contexts, Pro/Flash k = 1024/512).
WORKLOADS = {
    "tiny_csa_prefill_f32": Workload("tiny_csa_prefill_f32", 101, 1, 0, 1024, 4, 64, 0, 4, 4, 32, 32, 128,
                                     "f32", "f32", "f32", "f32", 1.0 / 8.0, 1.0),
    "csa_decode_128k_bf16": Workload("csa_decode_128k_bf16", 102, 16, 131072, 1, 4, 512, 64, 64, 64, 128, 512, 128,
                                     "bf16", "bf16", "bf16", "bf16", 1.0 / math.sqrt(512), 1.0),
    "csa_prefill_64k_chunk4k_bf16": Workload("csa_prefill_64k_chunk4k_bf16", 103, 1, 65536, 4096, 4, 512, 64, 64, 64,
                                             128, 1024, 128, "bf16", "bf16", "bf16", "bf16", 1.0,
                                             1.0 / math.sqrt(512)),
    "hca_decode_1m_bf16": Workload("hca_decode_1m_bf16", 104, 8, 1 << 20, 1, 128, 512, 64, 64, 0, 0, 0, 128,
                                   "bf16", "bf16", "bf16", "bf16", 1.0, 1.0 / math.sqrt(512)),
    "csa_decode_1m_mixed": Workload("csa_decode_1m_mixed", 105, 4, 1 << 20, 1, 4, 512, 64, 64, 64, 128, 1024, 128,
                                    "mixed", "fp4", "bf16", "fp4", 1.0, 1.0 / math.sqrt(512)),
    # multi-token prediction: each step verifies two tokens per sequence (the new one and one draft)
    "csa_decode_128k_bf16_mtp2": Workload("csa_decode_128k_bf16_mtp2", 106, 16, 131072, 2, 4, 512, 64, 64, 64, 128,
                                          512, 128, "bf16", "bf16", "bf16", "bf16", 1.0 / math.sqrt(512), 1.0),
    "csa_decode_1m_mixed_mtp2": Workload("csa_decode_1m_mixed_mtp2", 107, 4, 1 << 20, 2, 4, 512, 64, 64, 64, 128,
                                         1024, 128, "mixed", "fp4", "bf16", "fp4", 1.0, 1.0 / math.sqrt(512)),
    # the ratio-0 layer: window + sink only, at the decode shape of the 128K workload (the cache and indexer draws are
    # made but unused)
    "swa_decode_128k_bf16": Workload("swa_decode_128k_bf16", 108, 16, 131072, 1, 4, 512, 64, 64, 64, 128, 512, 128,
                                     "bf16", "bf16", "bf16", "bf16", 1.0 / math.sqrt(512), 1.0, "swa"),
    # two CSA layers, one indexer selection feeding both layers' attention (the second layer's own cache, window,
    # queries and sink come from layer_inputs)
    "csa_decode_128k_bf16_shared2": Workload("csa_decode_128k_bf16_shared2", 109, 16, 131072, 1, 4, 512, 64, 64, 64,
                                             128, 512, 128, "bf16", "bf16", "bf16", "bf16", 1.0 / math.sqrt(512), 1.0,
                                             "shared2"),
}


def layer_inputs(w: Workload, layer: int) -> dict:
    """A further attention layer's own inputs for a step that shares one indexer selection across layers: the
    decode draws of the same shape under seed + 1000 * layer (only the latent cache, window, queries, sink and the
    latent compression streams are used)."""
    return decode_inputs(dataclasses.replace(w, seed=w.seed + 1000 * layer))


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some sizes overridden (smaller parity cases)."""
    return dataclasses.replace(w, **kw)


def decode_inputs(w: Workload) -> dict:
    """One decode step (Sq <= 4 new tokens at positions n_ctx .. n_ctx + Sq - 1; n_ctx is a multiple of m) over a
    cache that is given directly.

    Draw order: comp cache [B, N, D]; indexer keys [B, N, DI]; window KV [B, window + Sq - 1, D] (raw positions
    n_ctx - window + 1 .. n_ctx + Sq - 1); q [B, Sq, H, D] * q_std; qI [B, Sq, HI, DI]; w [B, Sq, HI] / sqrt(DI * HI);
    sink [H]; then the new tokens' compression streams (Ca, Cb, Za, Zb [B, Sq, D] and [B, Sq, DI]) and the
    carried previous block's stream-b tail (tail_Cb, tail_Zb [B, m, D] / [B, m, DI]) and the position
    biases Ba, Bb [m, D] / [m, DI] (std 0.1).  For HCA (no indexer) the indexer tensors are skipped and
    the streams have a single C/Z pair of width D.
    """
    g = rng(w.seed)
    N = w.N
    out = dict(workload=w)
    out["comp"] = normal(g, (w.B, N, w.D))
    if w.HI:
        out["keys"] = normal(g, (w.B, N, w.DI))
    out["window_kv"] = normal(g, (w.B, w.window + w.Sq - 1, w.D))
    out["q"] = normal(g, (w.B, w.Sq, w.H, w.D), w.q_std)
    if w.HI:
        out["qI"] = normal(g, (w.B, w.Sq, w.HI, w.DI))
        out["w"] = normal(g, (w.B, w.Sq, w.HI), 1.0 / math.sqrt(w.DI * w.HI))
    out["sink"] = normal(g, (w.H,))
    overlap = (w.m == 4)
    for tag, c in (("", w.D),) + ((("_I", w.DI),) if w.HI else ()):
        out["Ca" + tag] = normal(g, (w.B, w.Sq, c))
        out["Za" + tag] = normal(g, (w.B, w.Sq, c))
        if overlap:
            out["Cb" + tag] = normal(g, (w.B, w.Sq, c))
            out["Zb" + tag] = normal(g, (w.B, w.Sq, c))
            out["tail_Cb" + tag] = normal(g, (w.B, w.m, c))
            out["tail_Zb" + tag] = normal(g, (w.B, w.m, c))
        out["Ba" + tag] = normal(g, (w.m, c), 0.1)
        if overlap:
            out["Bb" + tag] = normal(g, (w.m, c), 0.1)
    return out


def prefill_inputs(w: Workload) -> dict:
    """A prefill chunk of Sq new tokens at positions n_ctx .. n_ctx + Sq - 1.

    Draw order: given comp cache part [B, N0, D] and keys [B, N0, DI] (N0 = n_ctx / m, skipped when 0);
    main streams Ca, Cb, Za, Zb [B, Sq, D]; stream-b tail tail_Cb, tail_Zb [B, m, D] (only when n_ctx > 0);
    Ba, Bb [m, D] std 0.1; the same for the indexer streams with width DI; raw KV [B, S_raw, D] covering
    positions max(0, n_ctx - window + 1) .. n_ctx + Sq - 1; q [B, Sq, H, D] * q_std; qI [B, Sq, HI, DI];
    w [B, Sq, HI] / sqrt(DI * HI); sink [H].
    """
    g = rng(w.seed)
    N0 = w.N
    out = dict(workload=w)
    if N0:
        out["comp"] = normal(g, (w.B, N0, w.D))
        out["keys"] = normal(g, (w.B, N0, w.DI))
    for tag, c in (("", w.D), ("_I", w.DI)):
        for nm in ("Ca", "Cb", "Za", "Zb"):
            out[nm + tag] = normal(g, (w.B, w.Sq, c))
        if w.n_ctx > 0:
            out["tail_Cb" + tag] = normal(g, (w.B, w.m, c))
            out["tail_Zb" + tag] = normal(g, (w.B, w.m, c))
        out["Ba" + tag] = normal(g, (w.m, c), 0.1)
        out["Bb" + tag] = normal(g, (w.m, c), 0.1)
    raw_start = max(0, w.n_ctx - w.window + 1)
    out["raw_start"] = raw_start
    out["raw_kv"] = normal(g, (w.B, w.n_ctx + w.Sq - raw_start, w.D))
    out["q"] = normal(g, (w.B, w.Sq, w.H, w.D), w.q_std)
    out["qI"] = normal(g, (w.B, w.Sq, w.HI, w.DI))
    out["w"] = normal(g, (w.B, w.Sq, w.HI), 1.0 / math.sqrt(w.DI * w.HI))
    out["sink"] = normal(g, (w.H,))
    return out


def hca_build_streams_device(w: Workload, device, n_tokens: int | None = None):
    """HCA cache-build streams for a long context, drawn on the GPU with torch's seeded generator.

    Draw order (torch.Generator(device).manual_seed(seed)): C [B, n, D] N(0,1), Z [B, n, D] N(0,1); then on
    the host with numpy Generator(PCG64(seed + 1000)): Ba [m, D] std 0.1.  The device tensors are inputs
    only; a sampled block can be copied back to the host so the oracle sees the same draws.
    """
    import torch
    n = w.n_ctx if n_tokens is None else n_tokens
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    C = torch.randn((w.B, n, w.D), generator=gen, device=device, dtype=torch.float32)
    Z = torch.randn((w.B, n, w.D), generator=gen, device=device, dtype=torch.float32)
    Ba = normal(rng(w.seed + 1000), (w.m, w.D), 0.1)
    return C, Z, Ba
