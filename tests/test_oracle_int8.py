"""Pins for the oracle's group-wise int8 codec, its int8 cache write and int8
attention.

The codec is checked against a brute-force nearest-integer search, its error
bound, symmetry, power-of-two scaling, the all-zero group and torch's own
per-channel int8 quantiser (away from rounding ties, where a reciprocal-based
quantiser may legitimately differ); the cache write by definition; attention
over an int8 cache against the textbook attention of the dequantised values.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import int8_group_encode
from workloads import make_decode_case


def brute_codes(x, scale):
    """Nearest integer in [-127, 127] to float32(x / scale), ties to the even one."""
    out = np.zeros(x.shape, dtype=np.int64)
    for idx in np.ndindex(x.shape):
        s = scale[idx[:-1]]
        if s == 0:
            continue
        q = float(np.float32(np.float32(x[idx]) / s))
        best = None
        for c in range(-127, 128):
            d = abs(q - c)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        out[idx] = best[1]
    return out


@pytest.mark.parametrize("seed", range(4))
def test_codes_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 64)) * rng.uniform(0.01, 50)).astype(np.float32)
    x[0, :8] = np.float32(0.5) * np.arange(8) / 127 * np.abs(x[0]).max()   # near-ties
    codes, scale = int8_group_encode(x)
    assert np.array_equal(codes.astype(np.int64), brute_codes(x, scale))
    assert np.array_equal(scale, (np.abs(x).max(-1) / np.float32(127)).astype(np.float32))


def test_error_bound_symmetry_and_extremes():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((200, 128)) * np.exp(rng.uniform(-8, 8, (200, 1)))).astype(np.float32)
    codes, scale = int8_group_encode(x)
    err = np.abs(x.astype(np.float64) - codes * scale[:, None].astype(np.float64))
    assert np.all(err <= scale[:, None] * (0.5 + 1e-6))
    assert np.all(np.abs(codes).max(-1) == 127)          # the largest magnitude maps to 127
    c2, s2 = int8_group_encode(-x)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scale)
    c3, s3 = int8_group_encode(x * np.float32(8))         # power-of-two scaling is exact
    assert np.array_equal(c3, codes) and np.array_equal(s3, scale * np.float32(8))
    c0, s0 = int8_group_encode(np.zeros((2, 64), np.float32))
    assert np.all(c0 == 0) and np.all(s0 == 0)


def test_agrees_with_torch_per_channel_quantiser_away_from_ties():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    codes, scale = int8_group_encode(x)
    tq = torch.quantize_per_channel(torch.from_numpy(x), torch.from_numpy(scale.astype(np.float64)),
                                    torch.zeros(64, dtype=torch.int64), 0, torch.qint8)
    t_codes = tq.int_repr().numpy()
    q = x / scale[:, None]
    frac = np.abs(q - np.trunc(q))
    away = np.abs(frac - 0.5) > 1e-4
    assert np.array_equal(codes[away], t_codes[away])
    assert np.abs(codes.astype(int) - t_codes.astype(int)).max() <= 1


def test_int8_cache_write_by_definition():
    rng = np.random.default_rng(1)
    NB, Hkv, bs, D = 6, 2, 4, 64
    kp = rng.integers(-128, 128, size=(NB, Hkv, bs, D)).astype(np.int8)
    vp = kp.copy()
    ks = rng.uniform(0, 1, (NB, Hkv, bs)).astype(np.float32)
    vs = ks.copy()
    k0, v0, ks0, vs0 = kp.copy(), vp.copy(), ks.copy(), vs.copy()
    kn = rng.standard_normal((3, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((3, Hkv, D)).astype(np.float16)
    slots = [5, -1, 22]
    oracle.kv_write_int8(kp, vp, ks, vs, kn, vn, "f16", slots, bs)
    touched = np.zeros((NB, bs), bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, o = divmod(slot, bs)
        touched[b, o] = True
        c, s = int8_group_encode(kn[i].astype(np.float32))
        assert np.array_equal(kp[b, :, o], c) and np.array_equal(ks[b, :, o], s)
        c, s = int8_group_encode(vn[i].astype(np.float32))
        assert np.array_equal(vp[b, :, o], c) and np.array_equal(vs[b, :, o], s)
    for b in range(NB):
        for o in range(bs):
            if not touched[b, o]:
                assert np.array_equal(kp[b, :, o], k0[b, :, o]) and ks[b, :, o].tolist() == ks0[b, :, o].tolist()
                assert np.array_equal(vp[b, :, o], v0[b, :, o]) and vs[b, :, o].tolist() == vs0[b, :, o].tolist()


def test_int8_attention_equals_attention_of_dequantised_values():
    """Attention over the int8 cache = textbook attention over code * scale, with
    the values decoded independently (torch int8 -> float64, times the scale)."""
    rng = np.random.default_rng(4)
    S, H, Hkv, D, bs, NB = 3, 4, 2, 16, 4, 12
    ctx = [5, 9, 1]
    kp = rng.integers(-127, 128, size=(NB, Hkv, bs, D)).astype(np.int8)
    vp = rng.integers(-127, 128, size=(NB, Hkv, bs, D)).astype(np.int8)
    ks = rng.uniform(0.001, 0.05, (NB, Hkv, bs)).astype(np.float32)
    vs = rng.uniform(0.001, 0.05, (NB, Hkv, bs)).astype(np.float32)
    tables = np.array([[0, 3, -1], [7, 1, 4], [10, -1, -1]], dtype=np.int32)
    q = rng.standard_normal((S, H, D)).astype(np.float32)
    got = oracle.paged_attention(q, "f32", kp, vp, "int8", tables, ctx, bs, 0.3, ks, vs)
    G = H // Hkv
    for s in range(S):
        n = ctx[s]
        t = np.arange(n)
        blk, off = tables[s][t // bs], t % bs
        K = torch.from_numpy(kp[blk, :, off, :]).double() * torch.from_numpy(ks[blk, :, off]).double()[..., None]
        V = torch.from_numpy(vp[blk, :, off, :]).double() * torch.from_numpy(vs[blk, :, off]).double()[..., None]
        for h in range(H):
            z = 0.3 * (K[:, h // G, :] @ torch.from_numpy(q[s, h]).double())
            w = torch.softmax(z, 0)
            ref = (w[:, None] * V[:, h // G, :]).sum(0).numpy()
            assert np.abs(got[s, h] - ref).max() < 1e-12
