"""GPU parity of sliding-window decode (pkv_paged_attn_decode_sliding)
against the oracle's window decode.

The window keeps only a sequence's most recent positions (caojiahao2.github.io
section 2.3).  To prove that nothing before the window is read, every test
sets the block-table entries of whole blocks before the window to -1 (as after
pkv_bm_release_before) and poisons the positions before the window inside its
first block with NaN (scales, for INT8 / FP8 caches).  Bound: the dtype
tolerances of the full decode.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (BS, DT, OracleView, as_f64, gpu_populate, hide_before_window, host,
                     max_abs_err, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_264_amd as m
    m._load()
    return m


def _cfg(dtype, cache, D, Hq, Hkv, lens, seed):
    return dict(B=len(lens), ctx=list(lens), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, cache=cache,
                pool=None, seed=seed, max_ctx=max(max(lens), 16))


PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "i8"), ("bf16", "f8")]
LENS = [1, 15, 16, 17, 250, 700, 33, 2000]


@pytest.mark.parametrize("dtype,cache", PAIRS)
@pytest.mark.parametrize("window", [1, 16, 17, 100, 513, 5000])
@pytest.mark.parametrize("P", [0, 64])
def test_window_decode_matches_oracle(pkv, dtype, cache, window, P):
    batch = W.make_batch(cfg=_cfg(dtype, cache, 128, 8, 2, LENS, seed=window + P), device="cuda")
    gpu_populate(pkv, batch)
    view = OracleView(batch, np.arange(batch.B), window=window)   # host copies first
    # position N-1 (the step's new token) is written by the cache write on both sides
    pkv.kv_cache_write(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_new,
                       batch.k_scale, batch.v_scale)
    view.write_new_tokens(batch)
    bt = hide_before_window(batch, window, batch.layout.context_lens)
    out = pkv.paged_attn_decode_sliding(batch.q, batch.k_cache, batch.v_cache, bt,
                                        batch.context_lens, batch.scale, window,
                                        k_scale=batch.k_scale, v_scale=batch.v_scale,
                                        partition_size=P)
    torch.cuda.synchronize()
    ref = view.decode()
    err = max_abs_err(out, ref)
    print(f"[window] {dtype}/{cache} W={window} P={P} max_abs_err={err:.3e}", flush=True)
    assert torch.isfinite(out.float()).all()
    assert err <= tol_for(dtype, cache)


@pytest.mark.parametrize("dtype,cache", [("f16", "f16"), ("f16", "i8"), ("bf16", "f8")])
@pytest.mark.parametrize("window", [1, 17, 256])
def test_window_decode_with_append(pkv, dtype, cache, window):
    """The fused append inside a window: the new token (position N-1) is
    stored into its slot and attended to; cache bytes of the new slot equal
    the oracle's write."""
    lens = [1, 16, 17, 300, 33, 129, 1000]
    batch = W.make_batch(cfg=_cfg(dtype, cache, 128, 16, 2, lens, seed=window), device="cuda")
    gpu_populate(pkv, batch)
    view = OracleView(batch, np.arange(batch.B), window=window)
    bt = hide_before_window(batch, window, batch.layout.context_lens)
    out = pkv.paged_attn_decode_sliding(batch.q, batch.k_cache, batch.v_cache, bt,
                                        batch.context_lens, batch.scale, window,
                                        k_new=batch.k_new, v_new=batch.v_new,
                                        k_scale=batch.k_scale, v_scale=batch.v_scale)
    torch.cuda.synchronize()
    view.write_new_tokens(batch)
    ref = view.decode()
    err = max_abs_err(out, ref)
    print(f"[window+append] {dtype}/{cache} W={window} max_abs_err={err:.3e}", flush=True)
    assert torch.isfinite(out.float()).all()
    assert err <= tol_for(dtype, cache)
    for i, n in enumerate(view.context_lens):
        t = int(n) - 1
        blk_g = int(batch.layout.block_tables[i, t // BS])
        blk_o = view.block_tables[i, t // BS]
        assert np.array_equal(host(batch.k_cache[blk_g, :, t % BS]).view(np.uint8),
                              view.k_cache[blk_o, :, t % BS].view(np.uint8))


def test_window_zero_is_the_full_decode(pkv):
    batch = W.make_batch(cfg=_cfg("f16", "f16", 64, 4, 4, LENS, seed=3), device="cuda")
    full = pkv.paged_attn_decode(batch.q, batch.k_cache, batch.v_cache, batch.block_tables,
                                 batch.context_lens, batch.scale, partition_size=64)
    win = pkv.paged_attn_decode_sliding(batch.q, batch.k_cache, batch.v_cache,
                                        batch.block_tables, batch.context_lens, batch.scale, 0,
                                        partition_size=64)
    torch.cuda.synchronize()
    assert torch.equal(full, win)


def test_window_decode_through_the_block_manager(pkv):
    """Decode step by step with a window of W, releasing the blocks that fall
    out of it: the pool never holds more than ceil(W / 16) + 1 blocks per
    sequence, and every step matches the oracle on the window's tokens."""
    Hq, Hkv, D, W_ = 8, 2, 64, 40
    B, steps = 3, 90
    prompt = [5, 33, 70]
    total = sum(prompt) + B * steps
    k_rows = W.token_rows(total, Hkv, D, "f16", 41, W.S_TOKEN_K)
    v_rows = W.token_rows(total, Hkv, D, "f16", 41, W.S_TOKEN_V)
    qs = W.token_rows(steps * B, Hq, D, "f16", 41, W.S_STEP_Q)
    NB = 64
    bm = pkv.BlockManager(NB)
    kc = torch.full((NB, Hkv, BS, D), float("nan"), dtype=torch.float16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    toks = {b: [] for b in range(B)}
    nxt = 0
    for b in range(B):
        bm.add_sequence(b)
        slots, _ = bm.append([b], [prompt[b]])
        ids = list(range(nxt, nxt + prompt[b]))
        nxt += prompt[b]
        toks[b] += ids
        pkv.kv_cache_write(k_rows[ids].cuda(), v_rows[ids].cuda(), kc, vc,
                           torch.from_numpy(slots).cuda())
    scale = float(np.float32(1 / np.sqrt(D)))
    mbs = -(-(max(prompt) + steps) // BS)
    peak = 0
    for st in range(steps):
        bm.append(list(range(B)), [1] * B)
        ids = list(range(nxt, nxt + B))
        nxt += B
        for b in range(B):
            toks[b].append(ids[b])
        tables, lens = bm.block_tables(list(range(B)), mbs)
        q = qs[st * B:(st + 1) * B]
        out = pkv.paged_attn_decode_sliding(q.cuda(), kc, vc, torch.from_numpy(tables).cuda(),
                                            torch.from_numpy(lens).cuda(), scale, W_,
                                            k_new=k_rows[ids].cuda(), v_new=v_rows[ids].cuda())
        torch.cuda.synchronize()
        # oracle: each sequence's last W tokens, contiguous
        kh, vh = host(k_rows), host(v_rows)
        for b in range(B):
            last = toks[b][-W_:]
            n = len(last)
            nblk = -(-n // BS)
            kk = np.zeros((nblk, Hkv, BS, D), np.uint16)
            vv = np.zeros_like(kk)
            pos = np.arange(n)
            kk[pos // BS, :, pos % BS] = kh[last]
            vv[pos // BS, :, pos % BS] = vh[last]
            ref = oracle.paged_decode(host(q[b:b + 1]), "f16", kk, vv, "f16",
                                      np.arange(nblk, dtype=np.int32)[None],
                                      np.array([n], np.int32), scale)
            assert np.abs(as_f64(out[b:b + 1]) - ref).max() <= 2e-3, (st, b)
        for b in range(B):
            bm.release_before(b, int(lens[b]) + 1 - W_)   # what the next step's window needs
        used = NB - bm.num_free_blocks
        peak = max(peak, used)
    assert peak <= B * (-(-W_ // BS) + 1)
