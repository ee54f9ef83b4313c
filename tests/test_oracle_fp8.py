"""Pins of the oracle's FP8 (e4m3) KV-cache support, CPU only.

- decode of all 256 codes and nearest-even encode against torch's
  float8_e4m3fn conversions (a library routine);
- the per-row quantizer (s = amax / 448 in single precision, r = x / s in
  single precision, clamped to +-448, nearest e4m3 value with ties to even)
  against exact rational arithmetic, with the e4m3 values enumerated here from
  the format's definition;
- attention over an FP8 cache against torch's scaled_dot_product_attention in
  float64 on the dequantized rows (code value x row scale).

The FP8 KV cache is named by the pages (docs.lazyllm.ai lesson 4, section 5.3:
FP8 as the wider-range alternative to INT8; juejin "LLM Engineer's Handbook",
latest developments: FP8 KV caches in serving engines); its scale rule is the
INT8 rule of section 5.3 with the format's largest value, 448, in place of 127.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

E4M3 = torch.float8_e4m3fn


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(E4M3).to(torch.float64).numpy()


def _torch_encode(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(E4M3).view(torch.uint8).numpy()


def test_decode_every_code_matches_torch():
    ref = _torch_decode(np.arange(256))
    got = np.array([oracle.f8_to_f64(c) for c in range(256)])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _test_values():
    g = np.random.default_rng(11)
    fin = np.sort(np.unique(_torch_decode(np.arange(127))))
    mids = (fin[1:] + fin[:-1]) / 2                      # every tie between neighbours
    return np.concatenate([g.uniform(-448, 448, 20000), g.standard_normal(20000),
                           g.standard_normal(5000) * 2.0 ** -7, mids, -mids,
                           [0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10]]
                          ).astype(np.float32)


def test_encode_matches_torch_round_to_nearest_even():
    x = _test_values()
    few = x[::50]
    assert [oracle.f8_from_f32(float(v)) for v in few] == _torch_encode(few).tolist()
    # the quantizer with amax = 448 has s = 1 exactly, so its codes are the plain encode
    row = np.concatenate([[448.0], x]).astype(np.float32)
    codes, s = oracle.quantize_rows(row[None], "f32", "f8")
    assert s[0] == 1.0
    assert np.array_equal(codes[0], _torch_encode(row))


def _e4m3_values():
    """(code, value) of every non-negative finite e4m3 code, from the format:
    exponent field e (bias 7), mantissa m (3 bits), e = 0 subnormal."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((c, v))
    return out


_VALS = _e4m3_values()


def _nearest_code(r: Fraction) -> int:
    a = abs(r)
    best = min(_VALS, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return best[0] | (0x80 if r < 0 else 0)


def _rn32(v: Fraction) -> Fraction:
    """Nearest IEEE binary32 (ties to even), normal or subnormal range."""
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


def test_quantizer_matches_exact_rational_arithmetic():
    g = np.random.default_rng(5)
    rows = (g.standard_normal((150, 64)) * g.uniform(0.01, 30, (150, 1))).astype(np.float16)
    codes, scales = oracle.quantize_rows(rows.view(np.uint16), "f16", "f8")
    for i in range(rows.shape[0]):
        xs = [Fraction(float(x)) for x in rows[i].astype(np.float64)]
        s = _rn32(max(abs(x) for x in xs) / 448)
        assert Fraction(float(scales[i])) == s
        want = [_nearest_code(max(Fraction(-448), min(Fraction(448), _rn32(x / s)))) for x in xs]
        assert codes[i].tolist() == want, i


def test_row_maximum_and_zero_row():
    g = np.random.default_rng(6)
    x = g.standard_normal((64, 128)).astype(np.float32)
    codes, scales = oracle.quantize_rows(x, "f32", "f8")
    am = np.abs(x).argmax(1)
    top = codes[np.arange(64), am]
    assert np.array_equal(top, np.where(x[np.arange(64), am] > 0, 0x7E, 0xFE))
    assert not np.isnan(_torch_decode(codes)).any()
    zc, zs = oracle.quantize_rows(np.zeros((2, 32), np.float32), "f32", "f8")
    assert (zc == 0).all() and (zs == 0).all()


def test_dequantized_error_is_within_half_an_e4m3_step():
    # |x - code * s| <= s * (half the gap at |x / s|) <= amax * 2^-4 for normal values
    g = np.random.default_rng(7)
    x = g.standard_normal((200, 128)).astype(np.float32)
    codes, s = oracle.quantize_rows(x, "f32", "f8")
    deq = _torch_decode(codes) * s[:, None].astype(np.float64)
    amax = np.abs(x).max(1, keepdims=True)
    assert (np.abs(deq - x) <= amax * 2.0 ** -4 + 1e-12).all()


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2)])
def test_attention_over_fp8_cache_matches_sdpa(Hq, Hkv):
    g = np.random.default_rng(8)
    B, D, NB, bs = 3, 64, 40, 16
    lens = np.array([17, 1, 90], np.int32)
    codes_k = g.integers(0, 256, (NB, Hkv, bs, D)).astype(np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x10         # no NaN codes
    codes_v = g.integers(0, 256, (NB, Hkv, bs, D)).astype(np.uint8)
    codes_v[(codes_v & 0x7F) == 0x7F] = 0x21
    ks = g.uniform(0.001, 0.01, (NB, Hkv, bs)).astype(np.float32)
    vs = g.uniform(0.001, 0.01, (NB, Hkv, bs)).astype(np.float32)
    perm = g.permutation(NB)
    mbs = 8
    bt = np.full((B, mbs), -1, np.int32)
    k = 0
    for b in range(B):
        nb = -(-int(lens[b]) // bs)
        bt[b, :nb] = perm[k:k + nb]
        k += nb
    q = g.standard_normal((B, Hq, D)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(D)))
    out = oracle.paged_decode(q, "f32", codes_k, codes_v, "f8", bt, lens, scale, k_scale=ks,
                              v_scale=vs)
    kd = _torch_decode(codes_k) * ks[..., None]
    vd = _torch_decode(codes_v) * vs[..., None]
    for b in range(B):
        n = int(lens[b])
        t = np.arange(n)
        K = kd[bt[b, t // bs], :, t % bs]            # [n][Hkv][D]
        V = vd[bt[b, t // bs], :, t % bs]
        Kh = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        Vh = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b].astype(np.float64))[:, None], Kh, Vh, scale=scale)[:, 0]
        assert np.abs(out[b] - ref.numpy()).max() < 1e-12


def test_cache_write_fp8_uses_the_quantizer():
    g = np.random.default_rng(9)
    T, Hkv, D, NB = 5, 2, 64, 4
    k = g.standard_normal((T, Hkv, D)).astype(np.float16).view(np.uint16)
    v = g.standard_normal((T, Hkv, D)).astype(np.float16).view(np.uint16)
    kc = np.zeros((NB, Hkv, 16, D), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((NB, Hkv, 16), np.float32)
    vs = np.zeros_like(ks)
    slots = np.array([3, 17, -1, 63, 40], np.int64)
    oracle.kv_cache_write(k, v, kc, vc, slots, "f16", "f8", ks, vs)
    ck, sk = oracle.quantize_rows(k, "f16", "f8")
    for i, sl in enumerate(slots):
        if sl < 0:
            continue
        assert np.array_equal(kc[sl // 16, :, sl % 16], ck[i])
        assert np.array_equal(ks[sl // 16, :, sl % 16], sk[i])
    assert (kc[0, :, 0] == 0).all()
