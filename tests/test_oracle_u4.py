"""Pins of the oracle's 4-bit KV cache, CPU only.

The pages name INT4 KV-cache quantization (caojiahao2.github.io section 2.3,
"INT8/INT4") and give the linear b-bit quantizer (docs.lazyllm.ai lesson 4,
section 3.2): x_q = round((x - x_min) / (x_max - x_min)
* (2^b - 1)), dequantized as x_min + x_q / (2^b - 1) * (x_max - x_min); here
b = 4 over each (slot, kv head) row.  Pinned by exact rational arithmetic of
that formula (single-precision rounding of each step written out with
Fractions), closed forms (row min -> 0, row max -> 15, constant rows), the
half-step error bound, and attention against SDPA on the dequantized rows.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle

BS = 16


def _rn32(v: Fraction) -> Fraction:
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = a / Fraction(2) ** (e - 23)
    n, r = divmod(q.numerator, q.denominator)
    rem = Fraction(r, q.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * Fraction(n) * Fraction(2) ** (e - 23)


def _rne(v: Fraction) -> int:
    n = math.floor(v)
    rem = v - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _unpack(codes, D):
    lo = codes & 15
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (D,), np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def test_quantizer_matches_exact_rational_arithmetic():
    g = np.random.default_rng(21)
    rows = (g.standard_normal((200, 64)) * g.uniform(0.01, 20, (200, 1))
            + g.uniform(-3, 3, (200, 1))).astype(np.float16)
    codes, meta = oracle.quantize_rows_u4(rows.view(np.uint16), "f16")
    got = _unpack(codes, 64)
    for i in range(rows.shape[0]):
        xs = [Fraction(float(x)) for x in rows[i].astype(np.float64)]
        lo, hi = min(xs), max(xs)
        rng_ = _rn32(hi - lo)
        assert Fraction(float(meta[i, 0])) == lo and Fraction(float(meta[i, 1])) == rng_
        want = [min(15, max(0, _rne(_rn32(_rn32(_rn32(x - lo) / rng_) * 15)))) for x in xs]
        assert got[i].tolist() == want, i


def test_min_max_and_constant_rows():
    g = np.random.default_rng(22)
    x = g.standard_normal((50, 128)).astype(np.float32)
    codes, meta = oracle.quantize_rows_u4(x, "f32")
    c = _unpack(codes, 128)
    r = np.arange(50)
    assert (c[r, x.argmin(1)] == 0).all() and (c[r, x.argmax(1)] == 15).all()
    assert c.min() >= 0 and c.max() <= 15
    const = np.full((3, 32), 2.5, np.float32)
    cc, mm = oracle.quantize_rows_u4(const, "f32")
    assert (cc == 0).all() and (mm[:, 0] == 2.5).all() and (mm[:, 1] == 0).all()


def test_dequantized_error_is_within_half_a_step():
    g = np.random.default_rng(23)
    x = g.standard_normal((300, 128)).astype(np.float32)
    codes, meta = oracle.quantize_rows_u4(x, "f32")
    deq = meta[:, :1].astype(np.float64) + _unpack(codes, 128) / 15.0 * meta[:, 1:].astype(np.float64)
    step = meta[:, 1:].astype(np.float64) / 15.0
    assert (np.abs(deq - x) <= step / 2 * (1 + 1e-5) + 1e-7).all()


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2)])
def test_attention_over_u4_cache_matches_sdpa(Hq, Hkv):
    g = np.random.default_rng(24)
    B, D, NB = 3, 64, 30
    lens = np.array([17, 1, 90], np.int32)
    kc = g.integers(0, 256, (NB, Hkv, BS, D // 2)).astype(np.uint8)
    vc = g.integers(0, 256, (NB, Hkv, BS, D // 2)).astype(np.uint8)
    km = np.stack([g.uniform(-2, 0, (NB, Hkv, BS)), g.uniform(0.5, 4, (NB, Hkv, BS))], -1).astype(np.float32)
    vm = np.stack([g.uniform(-2, 0, (NB, Hkv, BS)), g.uniform(0.5, 4, (NB, Hkv, BS))], -1).astype(np.float32)
    perm = g.permutation(NB)
    bt = np.full((B, 8), -1, np.int32)
    k = 0
    for b in range(B):
        nb = -(-int(lens[b]) // BS)
        bt[b, :nb] = perm[k:k + nb]
        k += nb
    q = g.standard_normal((B, Hq, D)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(D)))
    out = oracle.paged_decode(q, "f32", kc, vc, "u4", bt, lens, scale, k_scale=km, v_scale=vm)
    kd = km[..., :1].astype(np.float64) + _unpack(kc, D) / 15.0 * km[..., 1:].astype(np.float64)
    vd = vm[..., :1].astype(np.float64) + _unpack(vc, D) / 15.0 * vm[..., 1:].astype(np.float64)
    for b in range(B):
        n = int(lens[b])
        t = np.arange(n)
        K = torch.from_numpy(kd[bt[b, t // BS], :, t % BS]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        V = torch.from_numpy(vd[bt[b, t // BS], :, t % BS]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b].astype(np.float64))[:, None], K, V, scale=scale)[:, 0]
        assert np.abs(out[b] - ref.numpy()).max() < 1e-12


def test_cache_write_u4_uses_the_quantizer():
    g = np.random.default_rng(25)
    T, Hkv, D, NB = 5, 2, 64, 4
    k = g.standard_normal((T, Hkv, D)).astype(np.float16).view(np.uint16)
    v = g.standard_normal((T, Hkv, D)).astype(np.float16).view(np.uint16)
    kc = np.full((NB, Hkv, 16, D // 2), 0xAB, np.uint8)
    vc = kc.copy()
    km = np.zeros((NB, Hkv, 16, 2), np.float32)
    vm = np.zeros_like(km)
    slots = np.array([3, 17, -1, 63, 40], np.int64)
    oracle.kv_cache_write(k, v, kc, vc, slots, "f16", "u4", km, vm)
    ck, mk = oracle.quantize_rows_u4(k, "f16")
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        assert np.array_equal(kc[sl // 16, :, sl % 16], ck[i])
        assert np.array_equal(km[sl // 16, :, sl % 16], mk[i])
    assert (kc[0, :, 0] == 0xAB).all()
