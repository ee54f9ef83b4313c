"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars: bit-exact for cache-write placement and INT8 codes / scales; max-abs
error <= 2e-3 (fp16 KV), 1.6e-2 (bf16 KV), 2e-3 (INT8 KV, oracle on the same
dequantized values) and 1e-5 (fp32 KV) for attention outputs.  Unused pool
slots are NaN-poisoned in every attention case, so a kernel that reads outside
a context cannot pass.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (BS, DT, TOL, OracleView, as_f64, gpu_populate, gpu_step, guarded,
                     hide_before_window, host, max_abs_err, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_264_amd as m
    m._load()
    return m


def _cfg(dtype, cache, D, Hq, Hkv, lens, pool=None, seed=0):
    return dict(B=len(lens), ctx=list(lens), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, cache=cache,
                pool=pool, seed=seed, max_ctx=max(max(lens), 16))


def _check_step(pkv, batch, seqs=None, partition_size=0, tol=None):
    seqs = np.arange(batch.B) if seqs is None else np.asarray(seqs)
    view = OracleView(batch, seqs)           # host copies taken before the GPU step
    out = gpu_step(pkv, batch, partition_size=partition_size)
    torch.cuda.synchronize()
    view.write_new_tokens(batch)
    ref = view.decode()
    got = out[torch.from_numpy(seqs).to(out.device)]
    err = max_abs_err(got, ref)
    tol = tol_for(DT[batch.q.dtype], DT[batch.k_cache.dtype]) if tol is None else tol
    print(f"[parity] {batch.name} B={batch.B} Hq={batch.Hq} Hkv={batch.Hkv} D={batch.D} "
          f"{DT[batch.q.dtype]}/{DT[batch.k_cache.dtype]} P={partition_size} "
          f"max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert torch.isfinite(out.float()).all(), "non-finite output (poisoned slot read?)"
    assert err <= tol
    return out, view


PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "i8"), ("bf16", "i8"),
         ("f16", "f8"), ("bf16", "f8"), ("f16", "u4"), ("bf16", "u4")]
LENS = [1, 15, 16, 17, 250, 700, 33]


def _supported(cases):
    """Parameter tuples without 4-bit caches at head_dim 64 (a 32-byte 4-bit
    row would put two blocks in one wave load; the ABI refuses it, which
    tests/test_abi_host.py checks)."""
    return [c for c in cases if not (c[1] == "u4" and c[2] == 64)]   # (., cache, D, ...)


@pytest.mark.parametrize("dtype,cache,D", _supported([(d, c, D) for d, c in PAIRS
                                                      for D in (64, 128, 256)]))
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (16, 2), (6, 3)])
def test_decode_matrix(pkv, dtype, cache, D, Hq, Hkv):
    batch = W.make_batch(cfg=_cfg(dtype, cache, D, Hq, Hkv, LENS, seed=D + Hq), device="cuda")
    gpu_populate(pkv, batch)
    _check_step(pkv, batch)


@pytest.mark.parametrize("P", [16, 48, 64, 256, 1024])
@pytest.mark.parametrize("dtype,cache", [("f16", "f16"), ("bf16", "i8"), ("f16", "f8")])
def test_partition_sizes(pkv, P, dtype, cache):
    batch = W.make_batch(cfg=_cfg(dtype, cache, 128, 8, 2, [5, 64, 129, 1000, 1500], seed=P),
                         device="cuda")
    gpu_populate(pkv, batch)
    _check_step(pkv, batch, partition_size=P)


@pytest.mark.parametrize("P", [16, 64, 0])
@pytest.mark.parametrize("dtype,cache,Hq,Hkv", [("f16", "f16", 4, 4), ("bf16", "bf16", 8, 2),
                                                ("f16", "f16", 8, 4), ("bf16", "i8", 4, 4)])
def test_schedule_ties_and_ragged_batch(pkv, P, dtype, cache, Hq, Hkv):
    """Longest-first ranking with many equal partition lengths, empty
    sequences and a batch size (21) that is not a multiple of the eight keys
    a rank step reads: every work item must be taken exactly once (a
    duplicated or skipped item leaves a wrong or unwritten output row)."""
    lens = [100, 100, 0, 100, 37, 100, 1, 100, 100, 250, 100, 37, 37, 16, 17, 100, 250, 0, 100,
            64, 100]
    batch = W.make_batch(cfg=_cfg(dtype, cache, 128, Hq, Hkv, lens, seed=77 + P), device="cuda")
    gpu_populate(pkv, batch)
    _check_step(pkv, batch, partition_size=P)


@pytest.mark.parametrize("dtype,cache,D,Hq,Hkv", [("f16", "f16", 64, 16, 16),
                                                   ("bf16", "bf16", 64, 48, 48),
                                                   ("f16", "i8", 128, 32, 32),
                                                   ("f16", "u4", 128, 32, 8)])
def test_xcd_head_order(pkv, dtype, cache, D, Hq, Hkv):
    """With a multiple of 16 q-head tiles per sequence (16, 48 and 32 one-head
    tiles; 16 two-head tiles of a 4-bit GQA batch, two per kv head) the decode
    takes the tiles in its XCD order: every head of every sequence must still
    be computed once, from its own kv head."""
    lens = [1, 37, 300, 16, 129, 0, 70]
    batch = W.make_batch(cfg=_cfg(dtype, cache, D, Hq, Hkv, lens, seed=Hq + D), device="cuda")
    gpu_populate(pkv, batch)
    _check_step(pkv, batch)
    _check_step(pkv, batch, partition_size=64)


@pytest.mark.parametrize("dtype,cache,D", [("f16", "f16", 128), ("bf16", "i8", 128),
                                           ("f16", "f8", 64), ("bf16", "u4", 256)])
def test_multi_query_attention_heads(pkv, dtype, cache, D):
    """MQA: 32 q heads over one kv head (four 8-head tiles, or 4-head and
    2-head tiles for 8-bit and 4-bit caches, all reading the same K/V)."""
    lens = [1, 300, 16, 77, 1000]
    batch = W.make_batch(cfg=_cfg(dtype, cache, D, 32, 1, lens, seed=D + 1), device="cuda")
    gpu_populate(pkv, batch)
    _check_step(pkv, batch)
    _check_step(pkv, batch, partition_size=128)


def test_tiny_config(pkv):
    batch = W.make_batch("tiny", device="cuda")
    _check_step(pkv, batch)


def test_zero_context_and_empty_batch(pkv):
    batch = W.make_batch(cfg=_cfg("f16", "f16", 128, 4, 4, [0, 20, 0, 3]), device="cuda")
    out = gpu_step(pkv, batch)
    torch.cuda.synchronize()
    assert (out[0] == 0).all() and (out[2] == 0).all()
    _check_step(pkv, W.make_batch(cfg=_cfg("f16", "f16", 128, 4, 4, [0, 20, 0, 3]),
                                  device="cuda"))
    # B = 0 and T = 0 enqueue nothing and succeed
    q = torch.empty((0, 4, 128), dtype=torch.float16, device="cuda")
    res = pkv.paged_attn_decode(q, batch.k_cache, batch.v_cache,
                                torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                                torch.empty((0,), dtype=torch.int32, device="cuda"), 0.1)
    assert res.shape == (0, 4, 128)
    e = torch.empty((0, 4, 128), dtype=torch.float16, device="cuda")
    pkv.kv_cache_write(e, e, batch.k_cache, batch.v_cache,
                       torch.empty((0,), dtype=torch.int64, device="cuda"))


def test_single_token_returns_v0_exactly(pkv):
    for dtype in ("f32", "f16", "bf16"):
        batch = W.make_batch(cfg=_cfg(dtype, dtype, 128, 8, 2, [1, 1, 1]), device="cuda")
        out = gpu_step(pkv, batch)
        torch.cuda.synchronize()
        for s in range(3):
            v0 = batch.v_new[s]                    # position 0 is the new token
            assert torch.equal(out[s], v0.repeat_interleave(4, dim=0)), dtype


def test_identical_keys_give_mean_of_v(pkv):
    batch = W.make_batch(cfg=_cfg("f32", "f32", 64, 2, 2, [40, 300]), device="cuda")
    batch.k_new.copy_(batch.k_new[0:1].expand_as(batch.k_new))
    for s, n in enumerate([40, 300]):
        for t in range(n):
            blk = int(batch.layout.block_tables[s, t // BS])
            batch.k_cache[blk, :, t % BS] = batch.k_new[0]
    out = gpu_step(pkv, batch)
    torch.cuda.synchronize()
    for s, n in enumerate([40, 300]):
        rows = [batch.v_cache[int(batch.layout.block_tables[s, t // BS]), :, t % BS]
                .double() for t in range(n)]
        mean = torch.stack(rows).mean(0).cpu().numpy()
        assert np.abs(as_f64(out[s]) - mean).max() < 1e-5


def test_placement_permutation_invariance_bit_exact(pkv):
    batch = W.make_batch(cfg=_cfg("bf16", "bf16", 128, 8, 2, [900, 31, 400]), device="cuda")
    out1 = gpu_step(pkv, batch).clone()
    NB = batch.num_blocks
    perm = torch.from_numpy(np.random.default_rng(9).permutation(NB)).cuda()
    inv = torch.argsort(perm)
    k2, v2 = batch.k_cache[inv].contiguous(), batch.v_cache[inv].contiguous()
    bt = batch.block_tables.clone().long()
    bt = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).int().contiguous()
    out2 = pkv.paged_attn_decode(batch.q, k2, v2, bt, batch.context_lens, batch.scale)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_deterministic_reruns(pkv):
    batch = W.make_batch(cfg=_cfg("f16", "i8", 128, 8, 8, [2000, 77, 1500, 16]), device="cuda")
    gpu_populate(pkv, batch)
    a = gpu_step(pkv, batch, partition_size=64).clone()
    b = gpu_step(pkv, batch, partition_size=64).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# partials + standalone reduce
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,cache,P", [("f32", "f32", 16), ("f16", "f16", 64),
                                           ("bf16", "bf16", 128), ("f16", "i8", 32)])
def test_partials_and_reduce(pkv, dtype, cache, P):
    lens = [3, 16, 100, 513, 0]
    batch = W.make_batch(cfg=_cfg(dtype, cache, 64, 4, 2, lens, seed=P), device="cuda")
    gpu_populate(pkv, batch)
    view = OracleView(batch, np.arange(batch.B))
    pkv.kv_cache_write(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_new,
                       batch.k_scale, batch.v_scale)
    view.write_new_tokens(batch)
    NP = pkv.num_partitions(batch.block_tables.shape[1], P)
    m, l, o = pkv.paged_attn_decode_partials(batch.q, batch.k_cache, batch.v_cache,
                                             batch.block_tables, batch.context_lens, batch.scale,
                                             P, k_scale=batch.k_scale, v_scale=batch.v_scale)
    out = pkv.paged_attn_reduce(m, l, o, batch.context_lens, P, out_dtype=batch.q.dtype)
    # phase 1 with an output pointer finishes single-partition sequences; the
    # merge then skips them
    out2 = torch.full_like(batch.q, float("nan"))
    m2, l2, o2 = pkv.paged_attn_decode_partials(batch.q, batch.k_cache, batch.v_cache,
                                                batch.block_tables, batch.context_lens,
                                                batch.scale, P, k_scale=batch.k_scale,
                                                v_scale=batch.v_scale, out=out2)
    pkv.paged_attn_reduce(m2, l2, o2, batch.context_lens, P, out=out2, skip_single_partition=True)
    torch.cuda.synchronize()
    for s_, n in enumerate(lens):
        if n <= P:   # finished in phase 1: no partial written
            assert torch.isnan(m2[s_]).all()
    rm, rl, ro = oracle.paged_partials(view.q, view.q_dtype, view.k_cache, view.v_cache,
                                       view.cache_dtype, view.block_tables, view.context_lens,
                                       view.scale, P, NP, k_scale=view.k_scale,
                                       v_scale=view.v_scale)
    tol = tol_for(dtype, cache)
    for s, n in enumerate(lens):
        npart = -(-n // P)
        if npart == 0:
            continue
        assert np.abs(as_f64(m[s, :, :npart]) - rm[s, :, :npart]).max() < 1e-3 * max(
            1.0, np.abs(rm[s, :, :npart]).max())
        np.testing.assert_allclose(as_f64(l[s, :, :npart]), rl[s, :, :npart], rtol=1e-4)
        assert np.abs(as_f64(o[s, :, :npart]) - ro[s, :, :npart]).max() <= tol
    ref = view.decode()
    assert max_abs_err(out, ref) <= tol
    assert max_abs_err(out2, ref) <= tol
    fused = pkv.paged_attn_decode(batch.q, batch.k_cache, batch.v_cache, batch.block_tables,
                                  batch.context_lens, batch.scale, k_scale=batch.k_scale,
                                  v_scale=batch.v_scale, partition_size=P)
    torch.cuda.synchronize()
    assert max_abs_err(fused, ref) <= tol


def test_reduce_on_synthetic_partials(pkv):
    g = np.random.default_rng(17)
    B, Hq, NP, D, P = 3, 4, 9, 128, 32
    m = g.standard_normal((B, Hq, NP)) * 3
    l = g.uniform(1, 20, (B, Hq, NP))
    o = g.standard_normal((B, Hq, NP, D))
    lens = np.array([NP * P, 5 * P - 3, 0], np.int32)
    out = pkv.paged_attn_reduce(torch.from_numpy(m).float().cuda(),
                                torch.from_numpy(l).float().cuda(),
                                torch.from_numpy(o).float().cuda(),
                                torch.from_numpy(lens).cuda(), P)
    torch.cuda.synchronize()
    mf, lf, of = (x.astype(np.float32).astype(np.float64) for x in (m, l, o))
    for s in range(B):
        npart = -(-int(lens[s]) // P)
        if npart == 0:
            assert (out[s] == 0).all()
            continue
        ref = oracle.merge_partials(mf[s:s + 1, :, :npart], lf[s:s + 1, :, :npart],
                                    of[s:s + 1, :, :npart])
        assert np.abs(as_f64(out[s]) - ref[0]).max() < 1e-5


# ---------------------------------------------------------------------------
# cache write: bit-exact placement and INT8 codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("src,cache,D", _supported(
    [(s, c, D) for s, c in [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f32", "i8"),
                            ("f16", "i8"), ("bf16", "i8"), ("f32", "f8"), ("f16", "f8"),
                            ("bf16", "f8"), ("f32", "u4"), ("f16", "u4"), ("bf16", "u4")]
     for D in (64, 128, 256)]))
def test_cache_write_bit_exact(pkv, src, cache, D):
    NB, Hkv, T = 40, 4, 64
    g = np.random.default_rng(D)
    slots = W.random_slots(NB, T, seed=D)
    slots[::7] = -1                                          # skipped tokens
    tdt = W.TORCH_DTYPE
    k = torch.from_numpy(g.standard_normal((T, Hkv, D), dtype=np.float32) * 3).to(tdt[src])
    v = torch.from_numpy(g.standard_normal((T, Hkv, D), dtype=np.float32)).to(tdt[src])
    if cache == "i8":
        k[0] = 0.0                                           # zero row -> s = 0
        k[1, :, :] = 0.5; k[1, :, 0] = 127.0                  # ties with s = 1
    if cache == "f8":
        k[0] = 0.0
        # s = 1: the row holds 448 and e4m3 ties (midpoints between neighbours)
        mids = torch.tensor([1.0625, 1.1875, 17.0, 0.0029296875, -2.25, 3.25, 0.013671875])
        k[1, :, :] = 0.5; k[1, :, 0] = 448.0
        k[1, :, 1:1 + len(mids)] = mids.to(k.dtype)
    # sentinel bytes everywhere in the pool
    row = {"f32": 4 * D, "f16": 2 * D, "bf16": 2 * D, "u4": D // 2}.get(cache, D)
    kc = torch.from_numpy(g.integers(0, 256, (NB, Hkv, BS, row), dtype=np.uint8))
    if cache == "f8":                                        # sentinel codes, no NaN
        kc[(kc & 0x7F) == 0x7F] = 0x3C
    vc = torch.from_numpy(g.integers(0, 256, kc.shape, dtype=np.uint8))
    kc = kc.view(tdt[cache]).contiguous(); vc = vc.view(tdt[cache]).contiguous()
    ks = vs = None
    if cache == "u4":
        k[0] = 0.7                                           # constant row -> range 0
        # a row with ties: min 0, max 15 -> range 15, (x - 0) / 15 * 15 = x
        k[1, :, :] = 7.5; k[1, :, 0] = 0.0; k[1, :, 1] = 15.0; k[1, :, 2] = 2.5
    if cache in W.SCALED:
        shape = (NB, Hkv, BS, 2) if cache == "u4" else (NB, Hkv, BS)
        ks = torch.from_numpy(g.standard_normal(shape, dtype=np.float32))
        vs = torch.from_numpy(g.standard_normal(shape, dtype=np.float32))
    hk, hv = host(kc), host(vc)
    hks = None if ks is None else ks.numpy().copy()
    hvs = None if vs is None else vs.numpy().copy()
    oracle.kv_cache_write(host(k), host(v), hk, hv, slots, src, cache, hks, hvs)
    gk, gv = kc.cuda(), vc.cuda()
    gks = None if ks is None else ks.cuda()
    gvs = None if vs is None else vs.cuda()
    pkv.kv_cache_write(k.cuda(), v.cuda(), gk, gv, torch.from_numpy(slots).cuda(), gks, gvs)
    torch.cuda.synchronize()
    assert np.array_equal(host(gk).view(np.uint8), hk.view(np.uint8))
    assert np.array_equal(host(gv).view(np.uint8), hv.view(np.uint8))
    if cache in W.SCALED:
        assert np.array_equal(host(gks).view(np.uint32), hks.view(np.uint32))
        assert np.array_equal(host(gvs).view(np.uint32), hvs.view(np.uint32))


def test_int8_codes_bit_exact_many_rows(pkv):
    """400k fp16 rows of D=128 quantized by both sides, compared bit for bit."""
    T, Hkv, D = 4096, 32, 128
    g = torch.Generator(device="cuda"); g.manual_seed(2024)
    k = torch.randn((T, Hkv, D), generator=g, device="cuda").half()
    v = (torch.randn((T, Hkv, D), generator=g, device="cuda") * 7).half()
    NB = T // BS
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    kc = torch.empty((NB, Hkv, BS, D), dtype=torch.int8, device="cuda")
    vc = torch.empty_like(kc)
    ks = torch.empty((NB, Hkv, BS), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    pkv.kv_cache_write(k, v, kc, vc, slots, ks, vs)
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_rows(host(k), "f16")
    # slot t = token t: block t // 16, offset t % 16 -> [NB][16][Hkv][D] order
    got = host(kc).reshape(NB, Hkv, BS, D).transpose(0, 2, 1, 3).reshape(T, Hkv, D)
    gsc = host(ks).reshape(NB, Hkv, BS).transpose(0, 2, 1).reshape(T, Hkv)
    assert np.array_equal(got, codes)
    assert np.array_equal(gsc.view(np.uint32), scales.view(np.uint32))
    codes_v, scales_v = oracle.quantize_rows(host(v), "f16")
    gotv = host(vc).reshape(NB, Hkv, BS, D).transpose(0, 2, 1, 3).reshape(T, Hkv, D)
    assert np.array_equal(gotv, codes_v)
    gsv = host(vs).reshape(NB, Hkv, BS).transpose(0, 2, 1).reshape(T, Hkv)
    assert np.array_equal(gsv.view(np.uint32), scales_v.view(np.uint32))


# ---------------------------------------------------------------------------
# the workloads at full size, through the call and the launch configuration
# the bench times, every sequence and every head compared
# ---------------------------------------------------------------------------

FULL = ["tiny", "llama7b", "gqa", "gqa8", "gqa8-int8", "long", "int8", "fp8", "int4", "window", "tp8", "dp8",
        "cp8"]


def bench_partition(pkv, batch):
    """(partition size, effective max blocks per sequence) as bench.py picks
    them: the workload's own partition size, else the library default over
    the blocks a sequence can touch (a window's blocks only)."""
    mbs = batch.block_tables.shape[1]
    window = int(batch.cfg.get("window", 0))
    mbs_eff = min(mbs, window // BS + 2) if window else mbs
    P = batch.cfg.get("partition_size", 0)
    return (P or pkv.default_partition_size(batch.B, batch.Hq, batch.Hkv, mbs_eff,
                                            batch.k_cache.dtype)), mbs_eff


def _slot_rows(t, blk, off):
    """Rows [B][Hkv][...] of a pool tensor at (block blk[i], offset off[i])."""
    if isinstance(t, torch.Tensor):
        return host(t[torch.from_numpy(blk).to(t.device), :, torch.from_numpy(off).to(t.device)])
    return t[blk, :, off]


@pytest.mark.parametrize("name", FULL)
def test_full_config(pkv, name):
    """The fused step (pkv_paged_attn_decode_append; the sliding-window entry
    with its append for the window workload) with the bench's partition size,
    against the oracle's cache write of the new tokens followed by its decode,
    on every sequence and head; the appended slots' bytes (and scales) bit for
    bit; output and workspace inside sentinel guard bands.  Then the separate
    path (cache write, decode) on the same batch, against the same result."""
    batch = W.make_batch(name, device="cuda", poison=True)
    gpu_populate(pkv, batch)
    window = int(batch.cfg.get("window", 0))
    view = OracleView(batch, np.arange(batch.B), window=window)  # host copies before the step
    lens = batch.layout.context_lens
    bt = hide_before_window(batch, window, lens) if window else batch.block_tables
    P, mbs_eff = bench_partition(pkv, batch)
    NP = pkv.num_partitions(mbs_eff, P)
    out, out_guard = guarded(tuple(batch.q.shape), batch.q.dtype)
    need = pkv.decode_workspace_size(batch.B, batch.Hq, batch.Hkv, batch.D, mbs_eff, P,
                                     batch.k_cache.dtype)
    ws, ws_guard = guarded((need,), torch.uint8)
    kw = dict(k_scale=batch.k_scale, v_scale=batch.v_scale, partition_size=P, workspace=ws)
    if window:
        pkv.paged_attn_decode_sliding(batch.q, batch.k_cache, batch.v_cache, bt,
                                      batch.context_lens, batch.scale, window, k_new=batch.k_new,
                                      v_new=batch.v_new, out=out, **kw)
    else:
        pkv.paged_attn_decode_append(batch.q, batch.k_new, batch.v_new, batch.k_cache,
                                     batch.v_cache, bt, batch.context_lens, batch.scale,
                                     out=out, **kw)
    torch.cuda.synchronize()
    out_guard()
    ws_guard()
    view.write_new_tokens(batch)
    ref = view.decode()
    err = max_abs_err(out, ref)
    tol = tol_for(DT[batch.q.dtype], DT[batch.k_cache.dtype])
    print(f"[full fused] {name} B={batch.B} P={P} NP={NP} sequences={batch.B} "
          f"max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert torch.isfinite(out.float()).all(), "non-finite output (poisoned slot read?)"
    assert err <= tol

    # the appended slot (position N-1) of every sequence, every kv head
    has = lens > 0
    t = (lens[has] - 1).astype(np.int64)
    rows = np.arange(batch.B)[has]
    blk_g = batch.layout.block_tables[rows, t // BS].astype(np.int64)
    blk_o = view.block_tables[rows, t // BS].astype(np.int64)
    off = t % BS
    for g_t, o_t in ((batch.k_cache, view.k_cache), (batch.v_cache, view.v_cache)):
        assert np.array_equal(_slot_rows(g_t, blk_g, off).view(np.uint8),
                              _slot_rows(o_t, blk_o, off).view(np.uint8))
    if batch.k_scale is not None:
        for g_t, o_t in ((batch.k_scale, view.k_scale), (batch.v_scale, view.v_scale)):
            assert np.array_equal(_slot_rows(g_t, blk_g, off).view(np.uint32),
                                  _slot_rows(o_t, blk_o, off).view(np.uint32))
        # the whole quantized pool of the batch equals the oracle's, codes byte
        # for byte and the scales of every attended slot bit for bit
        idx = torch.from_numpy(view.block_ids).cuda()
        assert np.array_equal(host(batch.k_cache[idx]).view(np.uint8), view.k_cache.view(np.uint8))
        assert np.array_equal(host(batch.v_cache[idx]).view(np.uint8), view.v_cache.view(np.uint8))
        used = np.zeros((len(view.block_ids), BS), bool)
        for i, n in enumerate(view.context_lens):
            n = int(n)
            j0 = view.first_block(n)
            pos = np.arange(j0 * BS, n)
            used[view.block_tables[i, pos // BS], pos % BS] = True
        for g_t, o_t in ((batch.k_scale, view.k_scale), (batch.v_scale, view.v_scale)):
            g_h = host(g_t[idx]).transpose(0, 2, 1, *range(3, g_t.dim()))
            o_h = o_t.transpose(0, 2, 1, *range(3, o_t.ndim))
            assert np.array_equal(g_h[used].view(np.uint32), o_h[used].view(np.uint32))

    # the separate path: the cache write stores the same bytes again
    pkv.kv_cache_write(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_new,
                       batch.k_scale, batch.v_scale)
    out2 = torch.empty_like(batch.q)
    if window:
        pkv.paged_attn_decode_sliding(batch.q, batch.k_cache, batch.v_cache, bt,
                                      batch.context_lens, batch.scale, window, out=out2, **kw)
    else:
        pkv.paged_attn_decode(batch.q, batch.k_cache, batch.v_cache, bt, batch.context_lens,
                              batch.scale, out=out2, **kw)
    torch.cuda.synchronize()
    ws_guard()
    err2 = max_abs_err(out2, ref)
    print(f"[full separate] {name} max_abs_err={err2:.3e}", flush=True)
    assert err2 <= tol


def test_workspace_reuse_across_shapes(pkv):
    """One cached workspace serves calls of different shapes back to back: a
    call's partials never land on another call's merge counters."""
    shapes = [([3000, 900, 5000], 8, 8, 128, 64), ([40, 300], 2, 2, 64, 16),
              ([100] * 9, 16, 4, 64, 32), ([700, 1], 4, 4, 256, 48)]
    for i, (lens, Hq, Hkv, D, P) in enumerate(shapes * 2):
        batch = W.make_batch(cfg=_cfg("f16", "f16", D, Hq, Hkv, lens, seed=i), device="cuda")
        _check_step(pkv, batch, partition_size=P)


def test_large_batch_natural_order(pkv):
    """More sequences than the longest-first scheduler ranks: natural order."""
    g = np.random.default_rng(31)
    lens = [int(x) for x in g.integers(0, 300, size=300)]
    batch = W.make_batch(cfg=_cfg("f16", "f16", 64, 4, 2, lens, seed=31), device="cuda")
    _check_step(pkv, batch, partition_size=64)
    batch = W.make_batch(cfg=_cfg("bf16", "i8", 128, 8, 8, lens[:257], seed=32), device="cuda")
    gpu_populate(pkv, batch)
    _check_step(pkv, batch)


@pytest.mark.parametrize("dtype,cache,D,Hq,Hkv,P", _supported(
    [(d, c) + shape for d, c in PAIRS
     for shape in [(128, 8, 8, 0), (64, 16, 2, 32), (256, 4, 1, 64), (128, 8, 2, 0),
                   (128, 16, 2, 64), (256, 16, 2, 0), (128, 48, 1, 64), (128, 64, 16, 0),
                   (128, 128, 16, 0)]]))
def test_decode_append_matches_write_then_decode(pkv, dtype, cache, D, Hq, Hkv, P):
    """The fused step equals the cache write of the new tokens followed by the
    decode: cache bytes bit-exact against the oracle's write, outputs within
    the dtype bound.  (With 16-bit q, 8 to 63 q heads per kv head, or 4 to 63
    over a quantized cache, take the matrix cores, where one of a kv head's
    1-3 row tiles stores the row, quantized there for a quantized cache, and
    every one computes with it; 16 kv heads take the XCD head order.)"""
    lens = [1, 16, 17, 300, 33, 0, 129]
    batch = W.make_batch(cfg=_cfg(dtype, cache, D, Hq, Hkv, lens, seed=D + P), device="cuda")
    gpu_populate(pkv, batch)
    view = OracleView(batch, np.arange(batch.B))
    out = pkv.paged_attn_decode_append(batch.q, batch.k_new, batch.v_new, batch.k_cache,
                                       batch.v_cache, batch.block_tables, batch.context_lens,
                                       batch.scale, k_scale=batch.k_scale, v_scale=batch.v_scale,
                                       partition_size=P)
    torch.cuda.synchronize()
    view.write_new_tokens(batch)
    ref = view.decode()
    err = max_abs_err(out, ref)
    print(f"[append] {dtype}/{cache} D={D} Hq={Hq} Hkv={Hkv} P={P} max_abs_err={err:.3e}")
    assert torch.isfinite(out.float()).all()
    assert err <= tol_for(dtype, cache)
    idx = torch.from_numpy(view.block_ids).cuda()
    assert np.array_equal(host(batch.k_cache[idx]).view(np.uint8), view.k_cache.view(np.uint8)) \
        if cache not in W.SCALED else True
    # every slot the oracle wrote holds the same bytes on the GPU
    for i, (s_, n) in enumerate(zip(view.seqs, view.context_lens)):
        if n == 0:
            continue
        t = n - 1
        blk_o = view.block_tables[i, t // BS]
        blk_g = int(batch.layout.block_tables[s_, t // BS])
        assert np.array_equal(host(batch.k_cache[blk_g, :, t % BS]).view(np.uint8),
                              view.k_cache[blk_o, :, t % BS].view(np.uint8))
        assert np.array_equal(host(batch.v_cache[blk_g, :, t % BS]).view(np.uint8),
                              view.v_cache[blk_o, :, t % BS].view(np.uint8))
        if cache in W.SCALED:
            assert np.array_equal(host(batch.k_scale[blk_g, :, t % BS]).view(np.uint32),
                                  view.k_scale[blk_o, :, t % BS].view(np.uint32))
            assert np.array_equal(host(batch.v_scale[blk_g, :, t % BS]).view(np.uint32),
                                  view.v_scale[blk_o, :, t % BS].view(np.uint32))
