"""indexer_score_topk_noalloc (scratch in a fixed device array of the library, no allocation) against
indexer_score_topk with a caller-allocated workspace, through the C-ABI: the same kernels, so indices and scores
must be bit-identical.  Two calls in a row, the second smaller, then the first again (the array keeps the last
call's contents); a call whose workspace would exceed the array is refused on the host."""
import numpy as np
import pytest
import torch

import lca_inputs as gen
from long_context_attention_05_amd import lca
from tests.gpu_util import gpu_bf16, gpu_encode, up, ws

pytestmark = pytest.mark.gpu


def _case(seed, fmt, B, Sq, HI, DI, N, k):
    g = np.random.default_rng(seed)
    K = g.standard_normal((B, N, DI)).astype(np.float32)
    q = g.standard_normal((B, Sq * HI, DI)).astype(np.float32)
    w = (g.standard_normal((B, Sq, HI)) / np.sqrt(HI * DI)).astype(np.float32)
    if fmt == "fp4":
        kg, qg = gpu_encode(K, "fp4", cap=N + 3), gpu_encode(q, "fp4")
    else:
        kg, qg = gpu_bf16(gen.bf16_bits(K), cap=N + 3), gpu_bf16(gen.bf16_bits(q))
    return qg, up(w), kg


def _both(qg, wd, kg, B, Sq, HI, DI, N, m, k, q_start):
    outs = []
    for noalloc in (False, True):
        idx = torch.full((B, Sq, k), 7, dtype=torch.int32, device="cuda")
        sc = torch.full((B, Sq, k), 3.0, dtype=torch.float32, device="cuda")
        if noalloc:
            lca.indexer_score_topk_noalloc(qg.desc(), wd, kg.desc(), B, Sq, HI, DI, N, m, k, q_start, idx, sc)
        else:
            nb = lca.indexer_score_topk_workspace_size(B, Sq, N, k)
            lca.indexer_score_topk(qg.desc(), wd, kg.desc(), B, Sq, HI, DI, N, m, k, q_start, idx, sc, ws(nb), nb)
        torch.cuda.synchronize()
        outs.append((idx.cpu(), sc.cpu()))
    (i0, s0), (i1, s1) = outs
    assert torch.equal(i0, i1), "indices differ between the workspace and the no-allocation entry points"
    assert torch.equal(s0.view(torch.int32), s1.view(torch.int32)), "scores differ"
    assert (i0[..., : min(k, N)] >= 0).all()
    return i0


def test_noalloc_matches_workspace_entry_point():
    print("no-alloc case 1: fp4 decode, B=2 N=40000 k=512", flush=True)
    a = _case(201, "fp4", 2, 1, 64, 128, 40000, 512)
    first = _both(*a, 2, 1, 64, 128, 40000, 4, 512, 4 * 40000)
    print("no-alloc case 2: bf16, two rows, B=1 N=9000 k=256 (smaller)", flush=True)
    b = _case(202, "bf16", 1, 2, 64, 128, 9000, 256)
    _both(*b, 1, 2, 64, 128, 9000, 4, 256, 4 * 9000)
    print("no-alloc case 3: many rows, B=1 Sq=64 N=3000 k=128", flush=True)
    c = _case(203, "bf16", 1, 64, 16, 64, 3000, 128)
    _both(*c, 1, 64, 16, 64, 3000, 4, 128, 4 * 3000 - 40)
    print("no-alloc case 1 again", flush=True)
    again = _both(*a, 2, 1, 64, 128, 40000, 4, 512, 4 * 40000)
    assert torch.equal(first, again)


def test_noalloc_refuses_more_than_its_scratch():
    B, Sq, N, k = 16, 4, 262144, 1024
    assert lca.indexer_score_topk_workspace_size(B, Sq, N, k) > lca.NOALLOC_SCRATCH_BYTES
    qg, wd, kg = _case(204, "bf16", 1, 1, 4, 32, 64, 8)  # small real tensors: the call is refused before any launch
    q = lca.lca_tensor(lca.LCA_BF16, 32, 0, Sq * 4, qg.data.data_ptr(), None, None, 0)
    kd = lca.lca_tensor(lca.LCA_BF16, 32, 0, N, kg.data.data_ptr(), None, None, 0)
    idx = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(lca.LcaError) as e:
        lca.indexer_score_topk_noalloc(q, wd, kd, B, Sq, 4, 32, N, 4, k, 4 * N, idx, None)
    assert e.value.status == -3
