"""Seeded random-shape parity sweep, output guard bands, two streams at once,
and the binding's refusal of wrongly shaped outputs.

Sweep: 200 cases drawn from numpy.random.default_rng([2026, i]): up to 8
sequences of 0..300 tokens (NaN-poisoned pools), head_dim 64 / 128 / 256,
1..4 kv heads with query groups of 1, 2, 4 or 8, every supported (q, cache)
dtype pair, partition sizes from 16 tokens to the library default, and the
three decode entry points (plain, fused append, sliding window with a random
window).  Every case compares every output element with the oracle at the
dtype bound, and checks that nothing is written around the output buffer or
the caller's workspace (sentinel guard bands).  A second sweep of 64 cases
(default_rng([2027, i])) takes 4 to 63 q heads per kv head with 16-bit q,
the decodes that run on the matrix cores, over every cache format.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from helpers import (BS, DT, OracleView, gpu_populate, guarded, hide_before_window, host,
                     max_abs_err, tol_for)

PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "i8"), ("bf16", "i8"),
         ("f16", "f8"), ("bf16", "f8"), ("f16", "u4"), ("bf16", "u4")]
N_CASES, N_CHUNKS = 200, 8


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_264_amd as m
    m._load()
    return m


def draw_case(i: int) -> dict:
    g = np.random.default_rng([2026, i])
    dtype, cache = PAIRS[int(g.integers(len(PAIRS)))]
    D = int(g.choice([128, 256])) if cache == "u4" else int(g.choice([64, 128, 256]))
    group = int(g.choice([1, 2, 4, 8]))
    Hkv = int(g.integers(1, 5))
    B = int(g.integers(1, 9))
    lens = g.integers(0, 301, size=B)
    lens[g.random(B) < 0.1] = 0                       # some empty sequences
    mode = str(g.choice(["decode", "append", "sliding"]))
    window = int(g.choice([1, 16, 17, 50, 100, 200, 1000])) if mode == "sliding" else 0
    P = int(g.choice([0, 16, 32, 48, 64, 128, 256]))
    return dict(dtype=dtype, cache=cache, D=D, Hq=Hkv * group, Hkv=Hkv, lens=[int(x) for x in lens],
                mode=mode, window=window, P=P, seed=1000 + i)


def run_case(pkv, c: dict):
    lens = c["lens"]
    cfg = dict(B=len(lens), ctx=list(lens), Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"],
               cache=c["cache"], pool=max(W.default_pool_blocks(lens), 4), seed=c["seed"],
               max_ctx=max(max(lens), 16))
    batch = W.make_batch(cfg=cfg, device="cuda", poison=True)
    gpu_populate(pkv, batch)
    window = c["window"]
    view = OracleView(batch, np.arange(batch.B), window=window)   # host copies first
    bt = hide_before_window(batch, window, batch.layout.context_lens) if window else \
        batch.block_tables
    out, out_guard = guarded(tuple(batch.q.shape), batch.q.dtype)
    mbs = batch.block_tables.shape[1]
    mbs_eff = min(mbs, window // BS + 2) if window else mbs
    need = pkv.decode_workspace_size(batch.B, batch.Hq, batch.Hkv, batch.D, mbs_eff, c["P"],
                                     batch.k_cache.dtype)
    ws, ws_guard = guarded((max(need, 256),), torch.uint8)
    kw = dict(k_scale=batch.k_scale, v_scale=batch.v_scale, partition_size=c["P"], workspace=ws,
              out=out)
    if c["mode"] == "decode":
        pkv.kv_cache_write(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache,
                           batch.slot_new, batch.k_scale, batch.v_scale)
        pkv.paged_attn_decode(batch.q, batch.k_cache, batch.v_cache, bt, batch.context_lens,
                              batch.scale, **kw)
    elif c["mode"] == "append":
        pkv.paged_attn_decode_append(batch.q, batch.k_new, batch.v_new, batch.k_cache,
                                     batch.v_cache, bt, batch.context_lens, batch.scale, **kw)
    else:
        pkv.paged_attn_decode_sliding(batch.q, batch.k_cache, batch.v_cache, bt,
                                      batch.context_lens, batch.scale, window,
                                      k_new=batch.k_new, v_new=batch.v_new, **kw)
    torch.cuda.synchronize()
    out_guard()
    ws_guard()
    view.write_new_tokens(batch)
    ref = view.decode()
    err = max_abs_err(out, ref)
    tol = tol_for(c["dtype"], c["cache"])
    return err, tol


@pytest.mark.gpu
@pytest.mark.parametrize("chunk", range(N_CHUNKS))
def test_random_shape_sweep(pkv, chunk):
    per = N_CASES // N_CHUNKS
    worst = 0.0
    for i in range(chunk * per, (chunk + 1) * per):
        c = draw_case(i)
        err, tol = run_case(pkv, c)
        print(f"[sweep {i}] {c['dtype']}/{c['cache']} D={c['D']} Hq={c['Hq']} Hkv={c['Hkv']} "
              f"lens={c['lens']} {c['mode']} W={c['window']} P={c['P']} err={err:.2e} "
              f"tol={tol:.1e}", flush=True)
        assert err <= tol, (i, c, err)
        worst = max(worst, err / tol)
    print(f"[sweep chunk {chunk}] worst err/tol {worst:.3f}", flush=True)


# The matrix-core decode (16-bit q; 8 to 63 q heads per kv head, 4 to 63
# over a quantized cache): groups that fill one to four 16-row tiles, every
# cache format it takes, the plain and fused calls, and (off the route)
# sliding windows.
ROUTE_PAIRS = [("f16", "f16"), ("bf16", "bf16"), ("f16", "i8"), ("bf16", "i8"), ("f16", "f8"),
               ("bf16", "f8"), ("f16", "u4"), ("bf16", "u4")]
N_ROUTE, N_ROUTE_CHUNKS = 64, 4


def draw_route_case(i: int) -> dict:
    g = np.random.default_rng([2027, i])
    dtype, cache = ROUTE_PAIRS[int(g.integers(len(ROUTE_PAIRS)))]
    D = int(g.choice([128, 256])) if cache == "u4" else int(g.choice([64, 128, 256]))
    group = int(g.choice([4, 8, 12, 16, 24, 32, 48, 63]))
    Hkv = int(g.integers(1, 3))
    B = int(g.integers(1, 7))
    lens = g.integers(0, 601, size=B)
    lens[g.random(B) < 0.1] = 0
    mode = str(g.choice(["decode", "append", "append", "sliding"]))
    window = int(g.choice([1, 17, 100, 1000])) if mode == "sliding" else 0
    P = int(g.choice([0, 0, 16, 64, 256]))
    return dict(dtype=dtype, cache=cache, D=D, Hq=Hkv * group, Hkv=Hkv, lens=[int(x) for x in lens],
                mode=mode, window=window, P=P, seed=5000 + i)


@pytest.mark.gpu
@pytest.mark.parametrize("chunk", range(N_ROUTE_CHUNKS))
def test_matrix_core_decode_sweep(pkv, chunk):
    per = N_ROUTE // N_ROUTE_CHUNKS
    worst = 0.0
    for i in range(chunk * per, (chunk + 1) * per):
        c = draw_route_case(i)
        err, tol = run_case(pkv, c)
        print(f"[route {i}] {c['dtype']}/{c['cache']} D={c['D']} Hq={c['Hq']} Hkv={c['Hkv']} "
              f"lens={c['lens']} {c['mode']} W={c['window']} P={c['P']} err={err:.2e} "
              f"tol={tol:.1e}", flush=True)
        assert err <= tol, (i, c, err)
        worst = max(worst, err / tol)
    print(f"[route chunk {chunk}] worst err/tol {worst:.3f}", flush=True)


def test_route_sweep_covers_the_space():
    cases = [draw_route_case(i) for i in range(N_ROUTE)]
    assert {(c["dtype"], c["cache"]) for c in cases} == set(ROUTE_PAIRS)
    assert {(c["Hq"] // c["Hkv"] + 15) // 16 for c in cases} == {1, 2, 3, 4}
    assert {c["mode"] for c in cases} == {"decode", "append", "sliding"}


def test_sweep_covers_the_space():
    """The drawn cases reach every dtype pair, head dim, group, entry point
    and partition size (a check of the generator, no GPU work)."""
    cases = [draw_case(i) for i in range(N_CASES)]
    assert {(c["dtype"], c["cache"]) for c in cases} == set(PAIRS)
    assert {c["D"] for c in cases} == {64, 128, 256}
    assert {c["Hq"] // c["Hkv"] for c in cases} == {1, 2, 4, 8}
    assert {c["mode"] for c in cases} == {"decode", "append", "sliding"}
    assert {c["P"] for c in cases} == {0, 16, 32, 48, 64, 128, 256}
    assert any(0 in c["lens"] for c in cases)


@pytest.mark.gpu
def test_two_streams_at_once(pkv):
    """Two decodes on two streams, each with the binding's own per-call
    workspace and partitions small enough that both write partials, issued
    back to back ten times without synchronizing; both results match the
    oracle every time (shared partials would mix the two)."""
    cfgs = [dict(B=3, ctx=[3000, 5000, 700], Hq=8, Hkv=2, D=128, dtype="f16", cache="f16",
                 pool=None, seed=41, max_ctx=5000),
            dict(B=4, ctx=[4000, 100, 2500, 6000], Hq=4, Hkv=4, D=64, dtype="bf16",
                 cache="bf16", pool=None, seed=42, max_ctx=6000)]
    batches = [W.make_batch(cfg=c, device="cuda", poison=True) for c in cfgs]
    refs = [OracleView(b, np.arange(b.B)).decode() for b in batches]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(10):
        for b, s in zip(batches, streams):
            with torch.cuda.stream(s):
                outs.append(pkv.paged_attn_decode(b.q, b.k_cache, b.v_cache, b.block_tables,
                                                  b.context_lens, b.scale, partition_size=64))
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        b = batches[i % 2]
        err = max_abs_err(o, refs[i % 2])
        assert err <= tol_for(DT[b.q.dtype], DT[b.k_cache.dtype]), (i, err)


@pytest.mark.gpu
def test_binding_refuses_misshaped_outputs(pkv):
    """An output buffer of the wrong shape would be a device write out of
    bounds: the binding refuses it before calling the library."""
    b = W.make_batch(cfg=dict(B=3, ctx=[40, 17, 5], Hq=8, Hkv=2, D=64, dtype="f16", cache="f16",
                              pool=None, seed=5, max_ctx=40), device="cuda")
    bad = torch.empty((b.B, b.Hkv, b.D), dtype=b.q.dtype, device="cuda")   # [B][Hkv][D]
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                              b.scale, out=bad)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode_append(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache,
                                     b.block_tables, b.context_lens, b.scale, out=bad)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode_sliding(b.q, b.k_cache, b.v_cache, b.block_tables,
                                      b.context_lens, b.scale, 16, out=bad)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode_partials(b.q, b.k_cache, b.v_cache, b.block_tables,
                                       b.context_lens, b.scale, 16, out=bad)
    qsl = torch.arange(b.B + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        pkv.paged_attn_multi(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, qsl,
                             b.scale, 1, out=bad)
    m, l, o = pkv.paged_attn_decode_partials(b.q, b.k_cache, b.v_cache, b.block_tables,
                                             b.context_lens, b.scale, 16)
    with pytest.raises(ValueError):        # m / l not [B][Hq][NP]
        pkv.paged_attn_reduce(m[:, :4].contiguous(), l, o, b.context_lens, 16)
    with pytest.raises(ValueError):        # one context length short
        pkv.paged_attn_reduce(m, l, o, b.context_lens[:2].contiguous(), 16)
    with pytest.raises(ValueError):
        pkv.paged_attn_reduce(m, l, o, b.context_lens, 16, out=bad.float())
    # the right shapes still work
    good = pkv.paged_attn_reduce(m, l, o, b.context_lens, 16, out_dtype=torch.float16)
    ref = OracleView(b, np.arange(b.B)).decode()
    assert max_abs_err(good, ref) <= 2e-3
    assert host(b.q).shape == tuple(b.q.shape)


@pytest.mark.gpu
def test_read_helpers_run(pkv):
    """The measurement helpers run without error: the read-only ones over a
    NaN-poisoned batch and a list of items that includes out-of-range entries
    (skipped), the matrix-core and LDS rate kernels on a few work-groups."""
    b = W.make_batch(cfg=dict(B=3, ctx=[40, 0, 300], Hq=4, Hkv=4, D=128, dtype="f16", cache="f16",
                              pool=None, seed=9, max_ctx=300), device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    items = torch.tensor([[s, h] for s in range(3) for h in range(4)] + [[3, 0], [0, 4], [-1, 0]],
                         dtype=torch.int32, device="cuda")
    pkv.tile_read(b.k_cache, b.v_cache, b.block_tables, b.context_lens, items, sink)
    pkv.stream_read(b.k_cache.view(-1)[:1000], sink)
    pkv.mfma_rate(8, 3, sink)
    for pattern in range(4):
        pkv.lds_read_rate(pattern, 4, 3, sink)
    torch.cuda.synchronize()
