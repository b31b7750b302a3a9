"""Pins of the oracle's compression weights (position bias, softmax temperature, stream/block assignment), the
sink's independence from the softmax scale, the fp32 exactness certificate of the indexer dots, the canonical fp32
order of the indexer's head sum, and two metamorphic properties (power-of-two scaling, batch isolation).  Every expected value is a hand-derived closed
form, brute force, or a property the definition fixes.  CPU only."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc

LN = lambda v: np.float32(math.log(v))  # noqa: E731


def _zeros(B, n, c):
    return np.zeros((B, n, c), np.float32)


# ---------------------------------------------------------------------------------------------------
# compression: position bias B[r][j], temperature 1, stream a -> block i, stream b -> block i-1
# (paper notes, section 2.3, the Compressor excerpt: the bias `ape` of shape [ratio, channels] is added to
#  the gate scores over the position-in-block axis before the softmax; text under Eq. 11-12: the first m
#  candidates come from the current block, the last m from the previous one)
# ---------------------------------------------------------------------------------------------------
def test_compress_bias_weights_closed_form_csa():
    """m = 2, one channel, Z = 0, integer values.  Biases ln 1, ln 2 (stream a) and ln 3, ln 4 (stream b) give
    softmax weights 1:2:3:4, so entry i >= 1 is (Ca[2i] + 2 Ca[2i+1] + 3 Cb[2i-2] + 4 Cb[2i-1]) / 10 and entry 0,
    which has no predecessor, is (Ca[0] + 2 Ca[1]) / 3."""
    n, m = 8, 2
    Ca = np.arange(1, n + 1, dtype=np.float32).reshape(1, n, 1)        # 1..8
    Cb = (10 * np.arange(1, n + 1, dtype=np.float32)).reshape(1, n, 1)  # 10..80
    Ba = np.array([[LN(1)], [LN(2)]], np.float32)
    Bb = np.array([[LN(3)], [LN(4)]], np.float32)
    E = orc.kv_compress(Ca, Cb, _zeros(1, n, 1), _zeros(1, n, 1), Ba, Bb, m=m, overlap=True)[0, :, 0]
    a, b = Ca[0, :, 0].astype(np.float64), Cb[0, :, 0].astype(np.float64)
    want = [(a[0] + 2 * a[1]) / 3] + [(a[2 * i] + 2 * a[2 * i + 1] + 3 * b[2 * i - 2] + 4 * b[2 * i - 1]) / 10
                                      for i in range(1, n // m)]
    np.testing.assert_allclose(E, want, rtol=1e-6)  # ln v rounded to fp32: e^fl32(ln v) = v (1 + O(1e-7))


def test_compress_bias_weights_closed_form_hca():
    """m = 4, no overlap (HCA): biases ln 1..ln 4 weight the block's tokens 1:2:3:4."""
    n, m = 12, 4
    C = np.arange(1, n + 1, dtype=np.float32).reshape(1, n, 1) ** 2
    Ba = np.array([[LN(r + 1)] for r in range(m)], np.float32)
    E = orc.kv_compress(C, None, _zeros(1, n, 1), None, Ba, None, m=m, overlap=False)[0, :, 0]
    c = C[0, :, 0].astype(np.float64)
    want = [sum((r + 1) * c[m * i + r] for r in range(m)) / 10 for i in range(n // m)]
    np.testing.assert_allclose(E, want, rtol=1e-6)


def test_compress_temperature_two_candidates():
    """Two candidates whose logits differ by ln 3 get weights 1/4 and 3/4 (softmax at temperature 1), whether the
    difference sits in the token logit Z or in the position bias B; both together multiply (ln 3 + ln 2: 1/7, 6/7)."""
    C = np.array([[[4.0], [8.0]]], np.float32)
    for Z, Ba, want in (([0.0, LN(3)], [0.0, 0.0], (4 + 3 * 8) / 4),
                        ([0.0, 0.0], [0.0, LN(3)], (4 + 3 * 8) / 4),
                        ([0.0, LN(3)], [0.0, LN(2)], (4 + 6 * 8) / 7),
                        ([LN(3), 0.0], [0.0, 0.0], (3 * 4 + 8) / 4)):
        Zt = np.array(Z, np.float32).reshape(1, 2, 1)
        Bt = np.array(Ba, np.float32).reshape(2, 1)
        E = orc.kv_compress(C, None, Zt, None, Bt, None, m=2, overlap=False)
        np.testing.assert_allclose(E[0, 0, 0], want, rtol=1e-6)


def test_compress_bias_one_hot_per_channel():
    """A +60 bias on position r_j = j mod m in channel j makes channel j of every entry the stream's token at that
    position (weights e^60 : 1 leave the rest below 1e-25).  Stream a: entry i takes Ca[m i + r_j]; stream b: entry
    i >= 1 takes Cb[m (i - 1) + r_j] and entry 0 (no predecessor) is the mean of its own block."""
    g = np.random.default_rng(40)
    B, n, c, m = 2, 24, 7, 4
    f = lambda *s: g.standard_normal(s).astype(np.float32)  # noqa: E731
    Ca, Cb = f(B, n, c), f(B, n, c)
    Z = _zeros(B, n, c)
    rj = np.arange(c) % m
    hot = np.zeros((m, c), np.float32)
    hot[rj, np.arange(c)] = 60.0
    zero = np.zeros((m, c), np.float32)
    nb = n // m
    E = orc.kv_compress(Ca, Cb, Z, Z, hot, zero, m=m, overlap=True)
    for i in range(nb):
        np.testing.assert_allclose(E[:, i], Ca[:, m * i + rj, np.arange(c)], rtol=1e-12, atol=1e-12)
    E = orc.kv_compress(Ca, Cb, Z, Z, zero, hot, m=m, overlap=True)
    np.testing.assert_allclose(E[:, 0], Ca[:, 0:m].astype(np.float64).mean(1), rtol=1e-12)
    for i in range(1, nb):
        np.testing.assert_allclose(E[:, i], Cb[:, m * (i - 1) + rj, np.arange(c)], rtol=1e-12, atol=1e-12)
    # HCA (one stream, m = 8)
    m8 = 8
    r8 = np.arange(c) % m8
    hot8 = np.zeros((m8, c), np.float32)
    hot8[r8, np.arange(c)] = 60.0
    E = orc.kv_compress(Ca, None, Z, None, hot8, None, m=m8, overlap=False)
    for i in range(n // m8):
        np.testing.assert_allclose(E[:, i], Ca[:, m8 * i + r8, np.arange(c)], rtol=1e-12, atol=1e-12)


def test_compress_bias_constant_over_positions_is_invariant():
    """A per-channel constant added to every position's bias (both streams alike) shifts every logit of an entry
    equally: the softmax, hence the entry, is unchanged (up to the fp32 rounding of B + constant)."""
    g = np.random.default_rng(41)
    B, n, c, m = 2, 21, 5, 4
    f = lambda *s: g.standard_normal(s).astype(np.float32)  # noqa: E731
    Ca, Cb, Za, Zb = f(B, n, c), f(B, n, c), f(B, n, c), f(B, n, c)
    Ba, Bb = 0.1 * f(m, c), 0.1 * f(m, c)
    shift = 2.0 * f(c)
    E0 = orc.kv_compress(Ca, Cb, Za, Zb, Ba, Bb, m=m, overlap=True)
    E1 = orc.kv_compress(Ca, Cb, Za, Zb, (Ba + shift).astype(np.float32), (Bb + shift).astype(np.float32), m=m,
                         overlap=True)
    np.testing.assert_allclose(E1, E0, rtol=1e-5, atol=1e-6)
    # shifting only one stream's bias does change entries >= 1 (the two streams' weights are relative)
    E2 = orc.kv_compress(Ca, Cb, Za, Zb, (Ba + shift).astype(np.float32), Bb, m=m, overlap=True)
    np.testing.assert_allclose(E2[:, 0], E0[:, 0], rtol=1e-5, atol=1e-6)  # entry 0 has stream a only
    assert np.abs(E2[:, 1:] - E0[:, 1:]).max() > 1e-2


def test_compress_power_of_two_scaling_is_exact():
    """Scaling every value C by 2^k scales every entry by exactly 2^k (the weights do not depend on C)."""
    g = np.random.default_rng(42)
    B, n, c, m = 2, 19, 6, 4
    f = lambda *s: g.standard_normal(s).astype(np.float32)  # noqa: E731
    Ca, Cb, Za, Zb = f(B, n, c), f(B, n, c), f(B, n, c), f(B, n, c)
    Ba, Bb = 0.1 * f(m, c), 0.1 * f(m, c)
    E = orc.kv_compress(Ca, Cb, Za, Zb, Ba, Bb, m=m, overlap=True)
    for k in (-7, 3, 20):
        s = np.float32(2.0 ** k)
        Ek = orc.kv_compress(Ca * s, Cb * s, Za, Zb, Ba, Bb, m=m, overlap=True)
        np.testing.assert_array_equal(Ek, E * 2.0 ** k)


# ---------------------------------------------------------------------------------------------------
# batch isolation: sequence b's outputs depend on sequence b's inputs only
# ---------------------------------------------------------------------------------------------------
def test_batch_isolation_every_stage():
    g = np.random.default_rng(43)
    B, n, c, m, H, HI, DI, k, W = 3, 32, 8, 4, 2, 3, 16, 4, 5
    f = lambda *s: g.standard_normal(s).astype(np.float32)  # noqa: E731
    st = dict(Ca=f(B, n, c), Cb=f(B, n, c), Za=f(B, n, c), Zb=f(B, n, c))
    Ba, Bb = 0.1 * f(m, c), 0.1 * f(m, c)
    N = n // m
    keys = f(B, N, DI)
    qI, w = f(B, 2, HI, DI), f(B, 2, HI)
    q, raw = f(B, 2, H, c), f(B, n + 2, c)
    sink = f(H)

    def run(st, keys, qI, w, q, raw):
        E = orc.kv_compress(st["Ca"], st["Cb"], st["Za"], st["Zb"], Ba, Bb, m=m, overlap=True)
        comp = orc.compress_to_cache(E, "f32")
        comp["cap"] = N
        kc = dict(orc.plain_cache(keys, "f32"), cap=N)
        s64, _, _, _ = orc.indexer_scores(orc.plain_cache(qI, "f32"), w, kc, B, 2, HI, DI, N, m, n)
        idx, _, _ = orc.topk(s64.reshape(B * 2, N), orc.nvis_rows(B, [0, 1], n, m, N), k)
        o, lse = orc.attn(orc.plain_cache(q, "f32"), comp, N, dict(orc.plain_cache(raw, "f32"), cap=n + 2), 0, n + 2,
                          idx.reshape(B, 2, k), k, 0, sink, B, 2, H, c, W, 0.5, n)
        return E, s64, idx.reshape(B, 2, k), o, lse

    ref = run(st, keys, qI, w, q, raw)
    st2 = {x: v.copy() for x, v in st.items()}
    keys2, qI2, w2, q2, raw2 = keys.copy(), qI.copy(), w.copy(), q.copy(), raw.copy()
    for a in list(st2.values()) + [keys2, qI2, w2, q2, raw2]:
        a[1] = g.standard_normal(a[1].shape).astype(np.float32) * 3  # replace sequence 1 entirely
    got = run(st2, keys2, qI2, w2, q2, raw2)
    for r, x in zip(ref, got):
        np.testing.assert_array_equal(x[0], r[0])
        np.testing.assert_array_equal(x[2], r[2])
        assert not np.array_equal(x[1], r[1])


# ---------------------------------------------------------------------------------------------------
# sink: e^z joins the denominator only, whatever the softmax scale (itsolotime page, mechanism 3)
# ---------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("scale", [1.0 / math.sqrt(8), 0.3, 2.0])
def test_sink_closed_form_at_any_scale(scale):
    """o(z) = o(-inf) * S / (S + e^z) with S = e^lse(-inf): the sink logit is not multiplied by the scale."""
    g = np.random.default_rng(44)
    B, Sq, H, D, N, k, W = 2, 2, 4, 8, 20, 6, 5
    q = g.standard_normal((B, Sq, H, D)).astype(np.float32)
    comp = g.standard_normal((B, N, D)).astype(np.float32)
    raw = g.standard_normal((B, 40, D)).astype(np.float32)
    idx = np.stack([np.stack([g.permutation(N)[:k] for _ in range(Sq)]) for _ in range(B)]).astype(np.int32)
    cs, rs = dict(orc.plain_cache(comp, "f32"), cap=N), dict(orc.plain_cache(raw, "f32"), cap=40)

    def run(sink):
        return orc.attn(orc.plain_cache(q, "f32"), cs, N, rs, 0, 40, idx, k, 0, sink, B, Sq, H, D, W, scale, 30)

    o0, l0 = run(np.full(H, -np.inf, np.float32))
    z = np.array([-2.0, 0.5, 1.5, 3.0], np.float32)
    o1, l1 = run(z)
    S = np.exp(l0)
    ratio = S / (S + np.exp(z.astype(np.float64)))
    np.testing.assert_allclose(o1, o0 * ratio[..., None], rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(l1, np.logaddexp(l0, z.astype(np.float64)), rtol=1e-12)
    # and the logits are scaled: doubling q is the same as doubling the scale
    o2, _ = orc.attn(orc.plain_cache((2 * q).astype(np.float32), "f32"), cs, N, rs, 0, 40, idx, k, 0, z, B, Sq, H,
                     D, W, scale, 30)
    o3, _ = orc.attn(orc.plain_cache(q, "f32"), cs, N, rs, 0, 40, idx, k, 0, z, B, Sq, H, D, W, 2 * scale, 30)
    np.testing.assert_allclose(o2, o3, rtol=1e-12)


# ---------------------------------------------------------------------------------------------------
# the fp32 exactness certificate of the indexer's head dots
# ---------------------------------------------------------------------------------------------------
def _fp32_sums(p, g, n_orders=24):
    """fp32 sums of the products p in several orders: sequential, reversed, pairwise, random permutations."""
    p32 = p.astype(np.float32)
    assert np.array_equal(p32.astype(np.float64), p), "products must be fp32 values"

    def seq(v):
        acc = np.float32(0)
        for x in v:
            acc = np.float32(acc + x)
        return acc

    def pairwise(v):
        v = list(v)
        while len(v) > 1:
            v = [np.float32(v[i] + v[i + 1]) if i + 1 < len(v) else v[i] for i in range(0, len(v), 2)]
        return v[0]

    out = [seq(p32), seq(p32[::-1]), pairwise(p32)]
    for _ in range(n_orders):
        out.append(seq(p32[g.permutation(len(p32))]))
    return out


def test_certificate_against_brute_force_orders():
    """Certified dots give the exact value in every summation order tried; constructed wide-spread dots whose
    orders disagree are rejected."""
    g = np.random.default_rng(45)
    n_cert = n_needed = 0
    for trial in range(400):
        n = 32
        spread = int(g.integers(0, 40))
        q = (g.integers(-6, 7, n) * 0.5 * 2.0 ** g.integers(-spread, 1, n)).astype(np.float64)
        k = (g.integers(-6, 7, n) * 0.5).astype(np.float64)
        exact = float(np.sum(q * k))  # small dyadic values: the double sum is exact
        cert = orc.dot_is_fp32_exact(q, k)
        sums = _fp32_sums(q * k, g)
        if cert:
            n_cert += 1
            assert all(float(s) == exact for s in sums), trial
        elif len({float(s) for s in sums}) > 1:
            n_needed += 1  # orders disagree: rejecting was necessary
    assert 50 < n_cert < 400 and n_needed > 50
    # cancelling groups: +X, a tiny group, -X.  The final value is an fp32 number, but (X + t) - X rounds to 0.
    big = np.full(16, 6.0 * 2 ** 10)
    tiny = np.full(16, 0.5 * 2.0 ** -20)
    q = np.concatenate([big, tiny, -big])
    k = np.ones_like(q)
    assert not orc.dot_is_fp32_exact(q, k)
    assert float(_fp32_sums(q * k, g)[0]) == 0.0 and np.sum(q * k) == 2.0 ** -17
    # a fp4 x fp4 head with small scale spread is certified
    assert orc.dot_is_fp32_exact(np.concatenate([big, -big]), np.ones(32))
    assert orc.dot_is_fp32_exact(np.zeros(8), np.ones(8))


def test_certificate_on_fp4_rows():
    """N(0,1) rows encoded to fp4 (one scale per 32-element block): every pair is certified.  A row built with one
    block 2^30 below cancelling blocks is not, and the inexact count names exactly those pairs."""
    g = np.random.default_rng(46)
    B, Sq, HI, DI, N, m = 1, 1, 4, 128, 12, 4
    qx = g.standard_normal((B * Sq * HI, DI)).astype(np.float32)
    kx = g.standard_normal((B * N, DI)).astype(np.float32)
    w = np.abs(g.standard_normal((B, Sq, HI))).astype(np.float32)
    qc, kc = orc.encode(qx, "fp4"), orc.encode(kx, "fp4")
    kc["cap"] = N
    _, s32, _, bad, ex = orc.indexer_scores(qc, w, kc, B, Sq, HI, DI, N, m, 4 * N, canonical=True, want_exact=True)
    assert bad == 0 and ex.all()
    # entry 5: blocks +X, tiny, -X, 0 against a query head of all ones
    kx2 = kx.copy()
    kx2[5] = np.concatenate([np.full(32, 6.0 * 2 ** 10), np.full(32, 0.5 * 2.0 ** -20), np.full(32, -6.0 * 2 ** 10),
                             np.zeros(32)]).astype(np.float32)
    qx2 = qx.copy()
    qx2[0] = 1.0
    qc2, kc2 = orc.encode(qx2, "fp4"), orc.encode(kx2, "fp4")
    kc2["cap"] = N
    s64, _, _, bad, ex = orc.indexer_scores(qc2, w, kc2, B, Sq, HI, DI, N, m, 4 * N, canonical=True, want_exact=True)
    assert bad == 1 and not ex[0, 0, 5] and ex[0, 0, np.arange(N) != 5].all()


# ---------------------------------------------------------------------------------------------------
# ratio-0 layer: pure sliding-window attention with the sink (paper notes, section 2.4, the compress_ratios list
# of the config excerpt ends in a ratio-0 layer)
# ---------------------------------------------------------------------------------------------------
def test_window_only_layer_is_banded_causal_attention():
    """k = 0 and no compressed entries: the layer is causal attention over the last `window` raw tokens, checked
    against torch's scaled_dot_product_attention with a banded causal mask in fp64; a sink adds e^z to the
    denominator (closed form)."""
    import torch
    g = np.random.default_rng(47)
    B, n, H, D, W = 2, 50, 3, 16, 7
    kv = g.standard_normal((B, n, D)).astype(np.float32)
    q = g.standard_normal((B, n, H, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    empty = dict(orc.plain_cache(kv[:, :1], "f32"), cap=1)
    rs = dict(orc.plain_cache(kv, "f32"), cap=n)

    def run(sink):
        return orc.attn(orc.plain_cache(q, "f32"), empty, 0, rs, 0, n, None, 0, 0, sink, B, n, H, D, W, scale, 0)

    o, lse = run(np.full(H, -np.inf, np.float32))
    t = np.arange(n)
    band = (t[None, :] <= t[:, None]) & (t[None, :] > t[:, None] - W)
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(kv.astype(np.float64))[:, None].expand(B, H, n, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=torch.from_numpy(band),
                                                           scale=scale).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)
    z = g.standard_normal(H).astype(np.float32)
    o1, _ = run(z)
    S = np.exp(lse)
    np.testing.assert_allclose(o1, o * (S / (S + np.exp(z.astype(np.float64))))[..., None], rtol=1e-12)


# ---------------------------------------------------------------------------------------------------
# epilogues on compressed entries: RMSNorm and rotary position embedding (paper notes, section 2.3: the
# Compressor's RMSNorm over the entry's head_dim; the Indexer excerpt's rotary embedding of the trailing rd dims)
# ---------------------------------------------------------------------------------------------------
def test_rmsnorm_closed_forms():
    # hand case: x = (3, 4), mean square 12.5, gains (1, 2): y = (3, 8) / sqrt(12.5)
    y = orc.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0], np.float32), 0.0)
    np.testing.assert_allclose(y, [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=1e-15)
    # with eps: x = (1, 1, 1, 1), eps = 3: y = 1 / sqrt(1 + 3) = 0.5
    np.testing.assert_allclose(orc.rmsnorm(np.ones((1, 4)), np.ones(4, np.float32), 3.0), 0.5, rtol=1e-15)
    g = np.random.default_rng(48)
    x = g.standard_normal((5, 64))
    ones = np.ones(64, np.float32)
    y = orc.rmsnorm(x, ones, 0.0)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orc.rmsnorm(7.5 * x, ones, 0.0), y, rtol=1e-13)
    gains = g.standard_normal(64).astype(np.float32)
    np.testing.assert_allclose(orc.rmsnorm(x, gains, 0.0), y * gains, rtol=1e-13)


def test_rope_closed_forms():
    g = np.random.default_rng(49)
    c, rd = 12, 8
    x = g.standard_normal((6, c))
    # position 0 is the identity; the leading c - rd channels are never touched
    np.testing.assert_array_equal(orc.rope(x, np.zeros(6), rd, 10000.0), x)
    y = orc.rope(x, np.arange(6) * 37.0, rd, 10000.0)
    np.testing.assert_array_equal(y[:, :c - rd], x[:, :c - rd])
    # pair norms preserved
    pn = lambda v: np.hypot(v[:, c - rd::2], v[:, c - rd + 1::2])  # noqa: E731
    np.testing.assert_allclose(pn(y), pn(x), rtol=1e-13)
    # hand angles: pair 0 turns by p radians; with rd = 4, base 10000, pair 1 turns by p / 100
    e = np.array([[1.0, 0.0, 1.0, 0.0]])
    for p in (1.0, 2.5, 100.0):
        r = orc.rope(e, np.array([p]), 4, 10000.0)
        np.testing.assert_allclose(r, [[math.cos(p), math.sin(p), math.cos(p / 100), math.sin(p / 100)]], rtol=1e-13,
                                   atol=1e-15)
    # composition: rotating by p then by q equals rotating by p + q
    p, q = 123.0, 4567.0
    np.testing.assert_allclose(orc.rope(orc.rope(x, p, rd, 500.0), q, rd, 500.0), orc.rope(x, p + q, rd, 500.0),
                               rtol=1e-9, atol=1e-12)
    # relative positions: <R(p) a, R(q) b> depends only on p - q (over the rotated channels)
    a, b = x[0], x[1]
    d1 = orc.rope(a[None], 1000.0, rd, 10000.0)[0, c - rd:] @ orc.rope(b[None], 900.0, rd, 10000.0)[0, c - rd:]
    d2 = orc.rope(a[None], 5100.0, rd, 10000.0)[0, c - rd:] @ orc.rope(b[None], 5000.0, rd, 10000.0)[0, c - rd:]
    assert abs(d1 - d2) < 1e-9


def test_compress_epilogue_positions():
    """The epilogue composition: entry i written from start_pos takes the rotary position m * (start_pos / m + i),
    the first token of its block; a constant entry normalises to the gains."""
    g = np.random.default_rng(50)
    B, n, c, m, rd = 2, 16, 8, 4, 4
    E = g.standard_normal((B, n // m, c))
    y = orc.compress_epilogue(E, m, 64, rope_dims=rd, rope_base=10.0)
    for i in range(n // m):
        np.testing.assert_allclose(y[:, i], orc.rope(E[:, i], float(m * (16 + i)), rd, 10.0), rtol=1e-15)
    gains = g.standard_normal(c).astype(np.float32)
    y = orc.compress_epilogue(np.full((1, 3, c), -2.5), m, 0, norm_g=gains, eps=0.0)
    np.testing.assert_allclose(y, np.broadcast_to(-gains.astype(np.float64), (1, 3, c)), rtol=1e-15)


# ---------------------------------------------------------------------------------------------------
# block-managed (paged) caches and ragged batches (itsolotime page, question 5: the compressed cache is
# managed in blocks of lcm(4, 128) = 128 tokens, i.e. 32 CSA entries or one HCA entry per block)
# ---------------------------------------------------------------------------------------------------
def test_paged_cache_equals_dense():
    """Moving every block of a cache to a shuffled pool slot, with the table pointing at it, changes nothing: scores,
    selections and attention outputs are bit-identical to the dense cache's (indexer keys and latent cache alike;
    block sizes 32 and 1)."""
    g = np.random.default_rng(51)
    B, Sq, HI, DI, H, D, N, k, W, m = 3, 2, 4, 32, 3, 32, 128, 9, 6, 4
    cap = 160
    keys = g.standard_normal((B, cap, DI)).astype(np.float32)
    comp = g.standard_normal((B, cap, D)).astype(np.float32)
    raw = g.standard_normal((B, W + Sq, D)).astype(np.float32)
    qI = g.standard_normal((B, Sq, HI, DI)).astype(np.float32)
    w = g.standard_normal((B, Sq, HI)).astype(np.float32)
    q = g.standard_normal((B, Sq, H, D)).astype(np.float32)
    sink = g.standard_normal(H).astype(np.float32)
    q0 = 4 * N
    kd, cd = orc.encode(keys, "fp4", cap=cap), orc.encode(comp, "mixed", 8, cap=cap)
    rc = dict(orc.encode(raw, "mixed", 8), cap=W + Sq)
    qc = orc.encode(qI, "fp4")
    for br in (32, 1):
        perm_k = g.permutation(B * cap // br)
        perm_c = g.permutation(B * cap // br)
        kp, cp = orc.paged(kd, B, br, perm_k), orc.paged(cd, B, br, perm_c)
        assert not np.array_equal(kp["data"], kd["data"])
        s_d, s32_d, _, _ = orc.indexer_scores(qc, w, kd, B, Sq, HI, DI, N, m, q0, canonical=True)
        s_p, s32_p, _, _ = orc.indexer_scores(qc, w, kp, B, Sq, HI, DI, N, m, q0, canonical=True)
        np.testing.assert_array_equal(s_p, s_d)
        np.testing.assert_array_equal(s32_p, s32_d)
        idx, _, _ = orc.topk(s32_d.reshape(B * Sq, N).astype(np.float64),
                             orc.nvis_rows(B, np.arange(Sq), q0, m, N), k)
        args = (rc, q0 - W + 1, W + Sq, idx.reshape(B, Sq, k), k, 0, sink, B, Sq, H, D, W, 0.2, q0)
        o_d, l_d = orc.attn(orc.plain_cache(q, "f32"), cd, N, *args)
        o_p, l_p = orc.attn(orc.plain_cache(q, "f32"), cp, N, *args)
        np.testing.assert_array_equal(o_p, o_d)
        np.testing.assert_array_equal(l_p, l_d)
        # dense HCA rows through a one-entry-per-block table
        h_d, _ = orc.attn(orc.plain_cache(q, "f32"), cd, N, rc, q0 - W + 1, W + Sq, None, 0, m, sink, B, Sq, H, D, W,
                          0.2, q0)
        h_p, _ = orc.attn(orc.plain_cache(q, "f32"), cp, N, rc, q0 - W + 1, W + Sq, None, 0, m, sink, B, Sq, H, D, W,
                          0.2, q0)
        np.testing.assert_array_equal(h_p, h_d)


def test_ragged_batch_equals_separate_calls():
    """Sequences at their own positions (seq_pos) give, for each sequence, exactly the result of a call on that
    sequence alone at its position; its raw rows keep the call's offset from the query position."""
    g = np.random.default_rng(52)
    B, Sq, HI, DI, H, D, N, k, W, m = 3, 2, 4, 16, 3, 32, 100, 7, 5, 4
    pos = np.array([4 * 100, 4 * 37 + 2, 4 * 63 + 1], np.int64)
    q0 = int(pos.max())
    keys = g.standard_normal((B, N, DI)).astype(np.float32)
    comp = g.standard_normal((B, N, D)).astype(np.float32)
    S_raw = W + Sq - 1
    raw = g.standard_normal((B, S_raw, D)).astype(np.float32)
    qI = g.standard_normal((B, Sq, HI, DI)).astype(np.float32)
    w = g.standard_normal((B, Sq, HI)).astype(np.float32)
    q = g.standard_normal((B, Sq, H, D)).astype(np.float32)
    sink = g.standard_normal(H).astype(np.float32)
    kc, cc, rc = (dict(orc.plain_cache(x, "f32"), cap=x.shape[1]) for x in (keys, comp, raw))
    s_r, _, _, _ = orc.indexer_scores(orc.plain_cache(qI, "f32"), w, kc, B, Sq, HI, DI, N, m, q0, seq_pos=pos)
    nv = np.concatenate([orc.nvis_rows(1, np.arange(Sq), int(p), m, N) for p in pos])
    idx, _, _ = orc.topk(s_r.reshape(B * Sq, N), nv, k)
    idx = idx.reshape(B, Sq, k)
    o_r, l_r = orc.attn(orc.plain_cache(q, "f32"), cc, N, rc, q0 - W + 1, S_raw, idx, k, 0, sink, B, Sq, H, D, W, 0.3,
                        q0, seq_pos=pos)
    for b in range(B):
        one = lambda x: dict(orc.plain_cache(np.ascontiguousarray(x[b:b + 1]), "f32"), cap=x.shape[1])  # noqa: E731
        s1, _, _, _ = orc.indexer_scores(orc.plain_cache(np.ascontiguousarray(qI[b:b + 1]), "f32"), w[b:b + 1],
                                         one(keys), 1, Sq, HI, DI, N, m, int(pos[b]))
        np.testing.assert_array_equal(s1[0], s_r[b])
        o1, l1 = orc.attn(orc.plain_cache(np.ascontiguousarray(q[b:b + 1]), "f32"), one(comp), N, one(raw),
                          int(pos[b]) - W + 1, S_raw, np.ascontiguousarray(idx[b:b + 1]), k, 0, sink, 1, Sq, H, D, W,
                          0.3, int(pos[b]))
        np.testing.assert_array_equal(o1[0], o_r[b])
        np.testing.assert_array_equal(l1[0], l_r[b])
    # the visible counts differ per sequence: floor((pos + r) / m)
    assert len(set(nv.tolist())) == B * Sq - 1 or len(set(nv.tolist())) >= B


# ---------------------------------------------------------------------------------------------------
# the canonical fp32 indexer score: the paper notes fix no summation order for Eq. 16's head sum; the library's
# order is sixteen fused multiply-add chains over the heads j, j + 16, j + 32, ... then a halving tree over the
# chains (a plain halving tree below 16 heads).  Emulated here with exact rationals and one fp32 rounding per step.
# ---------------------------------------------------------------------------------------------------
def _round_f32(x: Fraction) -> Fraction:
    """x rounded to the nearest fp32 value, ties to even (subnormals included; no overflow in these tests)."""
    if x == 0:
        return Fraction(0)
    sign, a = (-1 if x < 0 else 1), abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def _chained_sum(w, r):
    P = len(r)
    if P >= 16:
        c = []
        for j in range(16):
            v = _round_f32(w[j] * r[j])
            for h in range(j + 16, P, 16):
                v = _round_f32(w[h] * r[h] + v)  # fused multiply-add: one rounding
            c.append(v)
    else:
        c = [_round_f32(w[h] * r[h]) for h in range(P)]
    while len(c) > 1:
        half = len(c) // 2
        c = [_round_f32(c[j] + c[j + half]) for j in range(half)]
    return c[0]


def _plain_halving_sum(w, r):
    c = [_round_f32(w[h] * r[h]) for h in range(len(r))]
    while len(c) > 1:
        half = len(c) // 2
        c = [_round_f32(c[j] + c[j + half]) for j in range(half)]
    return c[0]


@pytest.mark.parametrize("HI", [64, 20, 4])
def test_canonical_score_order(HI):
    """fp4 queries and keys (every dot certified exact) with arbitrary fp32 weights, so that the head sum rounds:
    the oracle's canonical fp32 score equals the exact-rational emulation of the chained order bit for bit, and (for
    16 heads or more) differs from a plain halving tree of rounded products on some entries."""
    g = np.random.default_rng(60 + HI)
    B, Sq, DI, N, m = 1, 1, 32, 24, 4
    qx = g.standard_normal((HI, DI)).astype(np.float32)
    kx = g.standard_normal((N, DI)).astype(np.float32)
    w = (g.standard_normal((B, Sq, HI)) * 0.37).astype(np.float32)
    qc, kc = orc.encode(qx, "fp4"), orc.encode(kx, "fp4")
    kc["cap"] = N
    _, s32, _, bad, _ = orc.indexer_scores(qc, w, kc, B, Sq, HI, DI, N, m, 4 * N, canonical=True, want_exact=True)
    assert bad == 0
    qd, kd = orc.decode(qc), orc.decode(kc)
    P = 1
    while P < HI:
        P *= 2
    wf = [Fraction(float(x)) for x in w[0, 0]] + [Fraction(0)] * (P - HI)
    differ = 0
    for i in range(N):
        r = [max(sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qd[h], kd[i])), Fraction(0)),
                 Fraction(0)) for h in range(HI)] + [Fraction(0)] * (P - HI)
        want = _chained_sum(wf, r)
        assert np.float32(s32[0, 0, i]) == np.float32(float(want)), (HI, i)
        differ += _plain_halving_sum(wf, r) != want
    if HI >= 16:
        assert differ > 0
