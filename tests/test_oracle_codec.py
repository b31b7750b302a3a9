"""Pins of the oracle's number formats (bf16, fp8 e4m3, fp4 e2m1) against library casts and the format
tables.  CPU only."""
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _edge_f32(n, seed):
    g = np.random.default_rng(seed)
    x = np.concatenate([
        g.standard_normal(n).astype(np.float32),
        (g.standard_normal(n) * 1e-3).astype(np.float32),
        (g.standard_normal(n) * 1e4).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1e-40, -1e-40, 3.0e38, 1.00390625, 1.01171875, 65504.0], np.float32),
    ])
    return x


def test_bf16_matches_torch_cast():
    x = _edge_f32(20000, 1)
    # add exact bf16 midpoints (ties) to exercise round-half-even
    mids = (np.arange(0x3F800000, 0x3F800000 + 0x10000 * 64, 0x10000, dtype=np.uint32) + 0x8000).view(np.float32)
    x = np.concatenate([x, mids, -mids])
    c = orc.encode(x.reshape(-1, 1), "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(c["data"].reshape(-1), ref)
    dec = orc.decode(c).reshape(-1)
    np.testing.assert_array_equal(dec, torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_fp8_all_codes_round_trip():
    for code in range(256):
        v = orc.fp8_decode1(code)
        if code in (0x7F, 0xFF):
            assert np.isnan(v)
            continue
        assert orc.fp8_encode1(np.float32(v)) == code, code
    # decode table equals torch's e4m3fn interpretation of the same bytes
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([orc.fp8_decode1(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_fp8_rounding_matches_torch_cast():
    g = np.random.default_rng(2)
    y = np.concatenate([
        (g.uniform(-448, 448, 4000)).astype(np.float32),
        (g.standard_normal(4000) * 0.05).astype(np.float32),
        (g.standard_normal(2000) * 1e-3).astype(np.float32),
    ])
    # midpoints between adjacent e4m3 values (ties)
    vals = np.unique(np.abs(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()))
    vals = vals[~np.isnan(vals)]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    y = np.concatenate([y, mids, -mids, np.array([0.0, -0.0, 448.0, -448.0], np.float32)])
    ours = np.array([orc.fp8_encode1(v) for v in y], np.uint8)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_mixed_row_encoding_scale_rule():
    """fp8 part: s = fl32(amax / 448) over the non-RoPE dims, codes = e4m3(clamp(fl32(x / s))); RoPE dims bf16."""
    g = np.random.default_rng(3)
    x = g.standard_normal((64, 512)).astype(np.float32)
    x[5, :448] = 0.0  # all-zero fp8 part -> scale 1
    c = orc.encode(x, "mixed", rope=64)
    amax = np.abs(x[:, :448]).max(axis=1)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    np.testing.assert_array_equal(c["scale"], s)
    y = np.clip(x[:, :448] / s[:, None], -448, 448).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(c["data"], ref)
    np.testing.assert_array_equal(c["rope_data"],
                                  torch.from_numpy(x[:, 448:].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    dec = orc.decode(c)
    # decoded fp8 part within half an e4m3 step of the input, scaled
    err = np.abs(dec[:, :448] - x[:, :448].astype(np.float64))
    assert np.all(err <= (np.abs(x[:, :448]) * 2.0 ** -4 + s[:, None] * 2.0 ** -10) * (1 + 1e-12))


def _golden_e2m1():
    table, ties = {}, []
    for line in open(os.path.join(GOLD, "e2m1_format.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == "tie":
            ties.append((float(parts[1]), int(parts[2])))
        else:
            table[int(parts[0])] = float(parts[1])
    return table, ties


def test_fp4_table_and_ties_from_format_spec():
    table, ties = _golden_e2m1()
    for code, v in table.items():
        d = orc.fp4_decode1(code)
        assert d == v and np.signbit(d) == np.signbit(v), code
        assert orc.fp4_encode1(v) == code
    for y, code in ties:
        assert orc.fp4_encode1(y) == code, y


def test_fp4_encode_is_nearest_value():
    table, _ = _golden_e2m1()
    mags = np.array([table[c] for c in range(8)])
    for y in np.linspace(-7, 7, 2801):
        c = orc.fp4_encode1(y)
        dist = np.abs(np.abs(y) - mags)
        best = np.flatnonzero(dist == dist.min())
        assert (c & 7) in best  # nearest magnitude (ties resolved separately above)
        if (c & 7) != 0 or y < 0:
            assert bool(c & 8) == bool(np.signbit(y))


def test_fp4_group_scale_rule():
    """One scale per block of 32 consecutive elements (the 1x32 FP4 sub-blocks with their own scale factors of the
    page "百万token成本暴降90%！DeepSeek-V4揭秘", question 4): the smallest e with amax <= 6 * 2^e over the block;
    stored as E8M0 byte e + 127."""
    g = np.random.default_rng(4)
    x = g.standard_normal((200, 128)).astype(np.float32) * np.float32(2.0) ** g.integers(-20, 20, (200, 1)).astype(np.float32)
    x[0, :32] = 0.0
    x[1, :32] = 6.0
    x[2, :32] = 6.0001
    # a large first half and a tiny second half of one block share the large half's scale (a 16-element block
    # would give the tiny half its own)
    x[4, :16] = 96.0
    x[4, 16:32] = 0.01
    c = orc.encode(x, "fp4")
    assert c["scale"].shape == (200, 4)
    e = c["scale"].astype(np.int64) - 127
    amax = np.abs(x.reshape(200, 4, 32)).max(axis=2).astype(np.float64)
    nz = amax > 0
    assert np.all(amax[nz] <= 6.0 * 2.0 ** e[nz])
    assert np.all(amax[nz] > 6.0 * 2.0 ** (e[nz] - 1))
    assert e[0, 0] == -127 and e[1, 0] == 0 and e[2, 0] == 1 and e[4, 0] == 4
    dec = orc.decode(c).reshape(200, 4, 32)
    assert np.all(dec[4, 0, :16] == 96.0) and np.all(dec[4, 0, 16:] == 0.0)
    # error of round-to-nearest on the e2m1 grid: at most half the grid step at that magnitude (step <= 2 * 2^e)
    err = np.abs(dec - x.reshape(200, 4, 32))
    assert np.all(err <= 2.0 ** e[:, :, None] * 1.0 + 1e-30)
    # packing: element 2j in the low nibble
    b = c["data"][3, 0]
    assert orc.fp4_decode1(b & 0xF) * 2.0 ** e[3, 0] == dec[3, 0, 0]
    assert orc.fp4_decode1(b >> 4) * 2.0 ** e[3, 0] == dec[3, 0, 1]
