"""Pins of the multi-query oracle (several query tokens per sequence, causal),
CPU only.

The verification pass of speculative decoding scores k draft tokens in one
target-model pass (caojiahao2.github.io section 6; lazyllm lesson 4, the
speculative-decoding algorithm): each of the last q_len positions of a
sequence attends to every position up to and including its own.  Pinned
against torch's scaled_dot_product_attention in float64 with an explicit
causal-offset mask, and closed forms.
"""
import math

import numpy as np
import pytest
import torch

import oracle

BS = 16


def _bits(t):
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


DT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def _pool(K_list, V_list, num_blocks, seed, dtype):
    g = np.random.default_rng(seed)
    Hkv, D = K_list[0].shape[1], K_list[0].shape[2]
    need = [-(-k.shape[0] // BS) for k in K_list]
    perm = g.permutation(num_blocks)
    tables = np.full((len(K_list), max(need)), -1, np.int32)
    kp = torch.full((num_blocks, Hkv, BS, D), float("nan"), dtype=dtype)
    vp = torch.full_like(kp, float("nan"))
    pos = 0
    for b in range(len(K_list)):
        for j in range(need[b]):
            phys = int(perm[pos]); pos += 1
            tables[b, j] = phys
            ck, cv = K_list[b][j * BS:(j + 1) * BS], V_list[b][j * BS:(j + 1) * BS]
            kp[phys, :, :ck.shape[0]] = ck.transpose(0, 1)
            vp[phys, :, :cv.shape[0]] = cv.transpose(0, 1)
    return kp, vp, tables


def _case(dtype, Hq, Hkv, D, lens, qlens, seed):
    g = np.random.default_rng(seed)
    K = [torch.from_numpy(g.standard_normal((n, Hkv, D), dtype=np.float32)).to(dtype)
         for n in lens]
    V = [torch.from_numpy(g.standard_normal((n, Hkv, D), dtype=np.float32)).to(dtype)
         for n in lens]
    T = sum(qlens)
    q = torch.from_numpy(g.standard_normal((T, Hq, D), dtype=np.float32)).to(dtype)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    kp, vp, bt = _pool(K, V, 64, seed, dtype)
    return K, V, q, qsl, kp, vp, bt


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 64), (8, 2, 32), (6, 1, 64)])
def test_multi_matches_sdpa_with_causal_offset(dtype, Hq, Hkv, D):
    lens = [1, 16, 40, 100, 9]
    qlens = [1, 16, 5, 33, 9]              # the last sequence is a prefill from empty
    K, V, q, qsl, kp, vp, bt = _case(dtype, Hq, Hkv, D, lens, qlens, seed=D + Hq)
    scale = float(np.float32(1 / math.sqrt(D)))
    out = oracle.paged_multi(_bits(q), DT[dtype], _bits(kp), _bits(vp), DT[dtype], bt,
                             np.array(lens, np.int32), qsl, scale)
    g = Hq // Hkv
    for b, (n, ql) in enumerate(zip(lens, qlens)):
        qq = q[qsl[b]:qsl[b + 1]].to(torch.float64).transpose(0, 1)[None]    # [1][Hq][ql][D]
        kk = K[b].to(torch.float64).transpose(0, 1).repeat_interleave(g, 0)[None]
        vv = V[b].to(torch.float64).transpose(0, 1).repeat_interleave(g, 0)[None]
        pos = n - ql + torch.arange(ql)
        mask = torch.arange(n)[None, :] <= pos[:, None]                      # [ql][n]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                               scale=scale)[0]
        got = out[qsl[b]:qsl[b + 1]].transpose(1, 0, 2)
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_prefill_first_query_returns_v0_and_equal_keys_give_prefix_means():
    Hq = Hkv = 2
    D, n = 32, 37
    g = np.random.default_rng(4)
    Kr = torch.from_numpy(np.repeat(g.standard_normal((1, Hkv, D), dtype=np.float32), n, 0))
    V = torch.from_numpy(g.standard_normal((n, Hkv, D), dtype=np.float32))
    q = torch.from_numpy(g.standard_normal((n, Hq, D), dtype=np.float32))
    kp, vp, bt = _pool([Kr], [V], 8, 1, torch.float32)
    out = oracle.paged_multi(q.numpy(), "f32", kp.numpy(), vp.numpy(), "f32", bt,
                             np.array([n], np.int32), np.array([0, n], np.int32), 0.3)
    assert np.array_equal(out[0], V[0].double().numpy())
    for j in range(n):                       # equal keys: mean of V over positions 0..j
        np.testing.assert_allclose(out[j], V[:j + 1].double().mean(0).numpy(), rtol=0,
                                   atol=1e-12)


def test_single_query_is_the_decode():
    lens = [17, 300, 1]
    K, V, q, qsl, kp, vp, bt = _case(torch.float16, 8, 2, 64, lens, [1, 1, 1], seed=9)
    cl = np.array(lens, np.int32)
    multi = oracle.paged_multi(_bits(q), "f16", _bits(kp), _bits(vp), "f16", bt, cl, qsl, 0.125)
    dec = oracle.paged_decode(_bits(q), "f16", _bits(kp), _bits(vp), "f16", bt, cl, 0.125)
    assert np.array_equal(multi, dec)


def test_more_queries_than_tokens_gives_zero_rows():
    K, V, q, qsl, kp, vp, bt = _case(torch.float32, 2, 2, 32, [3], [5], seed=2)
    out = oracle.paged_multi(q.numpy(), "f32", kp.numpy(), vp.numpy(), "f32", bt,
                             np.array([3], np.int32), qsl, 0.2)
    assert (out[:2] == 0).all() and np.isfinite(out[2:]).all()
