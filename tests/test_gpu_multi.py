"""GPU parity of multi-query causal attention (pkv_paged_attn_multi, MFMA)
against the oracle.

Every sequence of a NaN-poisoned pool gets q_len queries at its last
positions (1 = plain decode, up to the whole context = prefill from empty);
outputs are compared element by element with the fp64 oracle.  Bound: the
decode bound of the dtype plus the rounding of the softmax weights to the q
dtype before they multiply V on the matrix cores, u * max|V| (u = 2^-11 for
fp16, 2^-8 for bf16): |sum_t (p_t + d_t) v_t - sum_t p_t v_t| / l <= u max|v|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import BS, DT, TOL, OracleView, as_f64, guarded, host

pytestmark = pytest.mark.gpu
U_P = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_264_amd as m
    m._load()
    return m


def _run(pkv, dtype, D, Hq, Hkv, lens, qlens, P=0, seed=0, scale=None):
    cfg = dict(B=len(lens), ctx=list(lens), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, cache=dtype,
               pool=None, seed=seed, max_ctx=max(max(lens), 16))
    batch = W.make_batch(cfg=cfg, device="cuda")
    T = int(sum(qlens))
    q = W.token_rows(T, Hq, D, dtype, seed, W.S_STEP_Q).cuda()
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    view = OracleView(batch, np.arange(batch.B))
    scale = batch.scale if scale is None else scale
    out = pkv.paged_attn_multi(q, batch.k_cache, batch.v_cache, batch.block_tables,
                               batch.context_lens, torch.from_numpy(qsl).cuda(), scale,
                               max(qlens), partition_size=P)
    torch.cuda.synchronize()
    ref = oracle.paged_multi(host(q), dtype, view.k_cache, view.v_cache, dtype,
                             view.block_tables, view.context_lens, qsl, scale)
    vmax = float(np.nanmax(np.abs(as_f64(batch.v_cache).reshape(-1)[
        np.isfinite(as_f64(batch.v_cache).reshape(-1))])))
    tol = TOL[dtype] + U_P[dtype] * vmax
    got = as_f64(out)
    err = float(np.abs(got - ref).max()) if np.isfinite(got).all() else float("inf")
    print(f"[multi] {dtype} D={D} Hq={Hq} Hkv={Hkv} qlens={qlens} P={P} "
          f"max_abs_err={err:.3e} tol={tol:.2e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= tol
    return err


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (32, 8), (4, 1)])
def test_multi_matrix(pkv, dtype, D, Hq, Hkv):
    lens = [1, 16, 17, 250, 700, 33, 100]
    qlens = [1, 4, 8, 16, 5, 33, 100]          # the last one is a prefill from empty
    _run(pkv, dtype, D, Hq, Hkv, lens, qlens, seed=D + Hq)


@pytest.mark.parametrize("Hkv", [16, 32, 48])
def test_multi_xcd_head_order(pkv, Hkv):
    """Short query runs with one work-group per (sequence, kv head) and a
    multiple of 16 kv heads: the kernel takes the kv heads in its XCD order;
    every head of every query row must still come from its own kv head."""
    lens = [1, 16, 17, 250, 33]
    qlens = [1, 4, 8, 16, 5]
    _run(pkv, "f16", 64, Hkv, Hkv, lens, qlens, seed=Hkv)


@pytest.mark.parametrize("P", [16, 48, 64, 512])
def test_multi_partitions(pkv, P):
    lens = [5, 64, 129, 1000, 1500]
    qlens = [5, 7, 16, 17, 64]
    _run(pkv, "f16", 128, 8, 2, lens, qlens, P=P, seed=P)


def test_multi_single_query_matches_decode(pkv):
    lens = [1, 16, 17, 300, 33]
    cfg = dict(B=5, ctx=lens, Hq=8, Hkv=2, D=128, dtype="f16", cache="f16", pool=None, seed=4,
               max_ctx=300)
    batch = W.make_batch(cfg=cfg, device="cuda")
    qsl = torch.arange(6, dtype=torch.int32, device="cuda")
    multi = pkv.paged_attn_multi(batch.q, batch.k_cache, batch.v_cache, batch.block_tables,
                                 batch.context_lens, qsl, batch.scale, 1)
    dec = pkv.paged_attn_decode(batch.q, batch.k_cache, batch.v_cache, batch.block_tables,
                                batch.context_lens, batch.scale)
    torch.cuda.synchronize()
    # different rounding (P in fp16 on the matrix cores) but the same attention
    assert float((multi.float() - dec.float()).abs().max()) <= 2e-3 + 2.0 ** -11 * 5


_FULL_RUNS: dict = {}


def _full_multi_run(pkv, name):
    """A multi-query workload at full size as bench.py launches it (the cache
    write of the query tokens' K/V, then pkv_paged_attn_multi with the default
    partition size), output inside sentinel guard bands; run once per module
    and kept for the checks that follow."""
    if name in _FULL_RUNS:
        return _FULL_RUNS[name]
    batch = W.make_batch(name, device="cuda", poison=True)
    ql = batch.cfg["q_len"]
    lens = batch.layout.context_lens.astype(np.int64)
    qlens = np.minimum(lens, ql)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    q = W.token_rows(T, batch.Hq, batch.D, "f16", batch.seed, W.S_STEP_Q, "cuda")
    k_new = W.token_rows(T, batch.Hkv, batch.D, "f16", batch.seed, W.S_NEWK, "cuda")
    v_new = W.token_rows(T, batch.Hkv, batch.D, "f16", batch.seed, W.S_NEWV, "cuda")
    slots = np.concatenate([W.slots_for(batch.layout, b, np.arange(int(n) - int(k), int(n)))
                            for b, (n, k) in enumerate(zip(lens, qlens))])
    pkv.kv_cache_write(k_new, v_new, batch.k_cache, batch.v_cache, torch.from_numpy(slots).cuda())
    out, out_guard = guarded((T, batch.Hq, batch.D), torch.float16)
    pkv.paged_attn_multi(q, batch.k_cache, batch.v_cache, batch.block_tables,
                         batch.context_lens, torch.from_numpy(qsl).cuda(), batch.scale, ql,
                         out=out)
    torch.cuda.synchronize()
    out_guard()
    got = as_f64(out)
    assert np.isfinite(got).all()
    _FULL_RUNS[name] = (batch, q, qsl, qlens, got)
    return _FULL_RUNS[name]


def _full_multi_check(pkv, name, seqs):
    """Every query row and head of the given sequences against the oracle."""
    batch, q, qsl, qlens, got = _full_multi_run(pkv, name)
    seqs = np.asarray(seqs, np.int64)
    view = OracleView(batch, seqs)        # the pool with the queries' K/V
    rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs])
    sub_qsl = np.concatenate([[0], np.cumsum(qlens[seqs])]).astype(np.int32)
    ref = oracle.paged_multi(host(q[torch.from_numpy(rows).cuda()]), "f16", view.k_cache,
                             view.v_cache, "f16", view.block_tables, view.context_lens, sub_qsl,
                             batch.scale)
    vals = view.v_cache.view(np.float16).astype(np.float64).reshape(-1)
    vmax = float(np.abs(vals[np.isfinite(vals)]).max())
    err = float(np.abs(got[rows] - ref).max())
    tol = TOL["f16"] + U_P["f16"] * vmax
    print(f"[multi {name}] sequences {seqs.tolist()} query rows={len(rows)} "
          f"max_abs_err={err:.3e} tol={tol:.2e}", flush=True)
    assert err <= tol


def test_multi_verify_workload_full(pkv):
    """The speculative-verification shape: 64 LLaMA-7B sequences, 8 queries
    each, U[512, 4096] contexts (the short-run kernel); every sequence."""
    _full_multi_check(pkv, "verify", np.arange(W.CONFIGS["verify"]["B"]))


@pytest.mark.parametrize("part", range(4))
def test_multi_prefill_workload_full(pkv, part):
    """The chunked-prefill shape: 16 LLaMA-7B sequences, the last 512 of
    U[1024, 4096] positions being queries (the tiled kernel).  One launch;
    the oracle checks a quarter of the sequences per case (every query row
    and head of each), all 16 over the four cases."""
    _full_multi_check(pkv, "prefill", np.arange(part, W.CONFIGS["prefill"]["B"], 4))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (32, 8)])
@pytest.mark.parametrize("P", [0, 32])
def test_multi_short_query_runs(pkv, dtype, Hq, Hkv, P):
    """Fewer than 64 rows per (sequence, kv head): the 16-row-tile kernel,
    with several row tiles when the group is wide."""
    lens = [3, 16, 17, 250, 700, 33]
    qlens = [1, 2, 3, 4, 8, 7]
    _run(pkv, dtype, 128, Hq, Hkv, lens, qlens, P=P, seed=Hq + P)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_multi_prefill_chunks(pkv, D):
    """Long query runs (the tiled kernel): 300-token chunks at the end of
    longer contexts and a whole prompt, several work-groups per sequence."""
    lens = [1000, 300, 777]
    qlens = [300, 300, 129]
    _run(pkv, "f16", D, 8, 4, lens, qlens, seed=D)


@pytest.mark.parametrize("scale", [-0.088388346, 0.0])
@pytest.mark.parametrize("qlens", [[300, 129, 64], [3, 8, 1]])
@pytest.mark.parametrize("P", [0, 256])
def test_multi_negative_and_zero_scale(pkv, scale, qlens, P):
    """The scale is any fp32 value: a negative one reverses the order of the
    scores (the softmax then favours the smallest q . k), zero gives the
    plain mean of V over each query's positions.  Long query runs (the tiled
    kernel) and short ones, whole and split contexts."""
    _run(pkv, "f16", 128, 8, 4, [1000, 300, 777], qlens, P=P, seed=7, scale=scale)
