"""Test plumbing shared by the parity tests: host copies of seeded inputs for
the oracle, and the decode step (cache write of the new tokens, then
attention) run by each side independently."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

BS = W.BLOCK_SIZE
DT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.int8: "i8",
      torch.float8_e4m3fn: "f8", torch.uint8: "u4"}
# max-abs-error bounds by element type (fp32 is the proposed bound for the fp32
# case).  A case is held to the looser bound of its cache type and its q/out
# type: a bf16 output alone carries up to 2^-9 relative rounding error, which
# exceeds 2e-3 for |out| > 1, so bf16 q with an INT8 cache takes the bf16 bound.
# INT8, FP8 and 4-bit caches are compared with the oracle on the same
# dequantized values, so only accumulation order and output rounding differ:
# 2e-3.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1.6e-2, "i8": 2e-3, "f8": 2e-3, "u4": 2e-3}


def tol_for(q_dtype: str, cache_dtype: str) -> float:
    return max(TOL[q_dtype], TOL[cache_dtype])


def host(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; 16-bit floats as their raw uint16 bits, e4m3 as uint8."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    return t.numpy().copy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


class OracleView:
    """Host-side inputs of the oracle for a subset of sequences: the pool is
    compacted to the blocks those sequences use and their tables renumbered
    (paging makes the result independent of where blocks sit)."""

    def __init__(self, batch: W.Batch, seqs, window: int = 0):
        self.seqs = np.asarray(seqs, np.int64)
        self.window = window
        lay = batch.layout
        lens = lay.context_lens[self.seqs]
        blocks = []
        for s, n in zip(self.seqs, lens):
            j0 = self.first_block(n)
            blocks.extend(int(x) for x in lay.block_tables[s, j0:W.blocks_needed(n)])
        self.block_ids = np.asarray(blocks, np.int64)
        # pool id -> compacted id (-1: not used by these sequences)
        self.remap = np.full(batch.num_blocks, -1, np.int64)
        self.remap[self.block_ids] = np.arange(len(self.block_ids))
        mbs = lay.block_tables.shape[1]
        bt = np.full((len(self.seqs), mbs), -1, np.int32)
        for i, (s, n) in enumerate(zip(self.seqs, lens)):
            j0, j1 = self.first_block(n), W.blocks_needed(n)
            bt[i, j0:j1] = self.remap[lay.block_tables[s, j0:j1]]
        self.block_tables = bt
        self.context_lens = lens.astype(np.int32)
        self.q = host(batch.q[torch.from_numpy(self.seqs).to(batch.q.device)])
        self.q_dtype = DT[batch.q.dtype]
        self.cache_dtype = DT[batch.k_cache.dtype]
        self.src_dtype = DT[batch.k_new.dtype]
        self.scale = batch.scale
        nb = max(len(self.block_ids), 1)
        idx = torch.from_numpy(self.block_ids).to(batch.k_cache.device)
        if self.cache_dtype in W.SCALED:
            # the oracle builds its own INT8 / FP8 pool from the fp source rows
            Hkv, D = batch.Hkv, batch.D
            u4 = self.cache_dtype == "u4"
            self.k_cache = np.zeros((nb, Hkv, BS, D // 2 if u4 else D),
                                    np.int8 if self.cache_dtype == "i8" else np.uint8)
            self.v_cache = np.zeros_like(self.k_cache)
            self.k_scale = np.full((nb, Hkv, BS, 2) if u4 else (nb, Hkv, BS), np.nan, np.float32)
            self.v_scale = np.full_like(self.k_scale, np.nan)
            offs = batch.extra["src_offsets"]
            rows = np.concatenate([np.arange(offs[s], offs[s + 1]) for s in self.seqs]) \
                if len(self.seqs) else np.zeros(0, np.int64)
            ridx = torch.from_numpy(rows).to(batch.k_src.device)
            slots = batch.slot_src.cpu().numpy()[rows]
            oracle.kv_cache_write(host(batch.k_src[ridx]), host(batch.v_src[ridx]), self.k_cache,
                                  self.v_cache, self.compact_slots(slots), self.src_dtype,
                                  self.cache_dtype,
                                  self.k_scale, self.v_scale)
        else:
            # (no block used at all: one pool block that no table entry names)
            idx = idx if len(idx) else torch.zeros(1, dtype=torch.int64, device=idx.device)
            self.k_cache = host(batch.k_cache[idx])
            self.v_cache = host(batch.v_cache[idx])
            self.k_scale = self.v_scale = None

    def first_block(self, n: int) -> int:
        """First block a sliding window of self.window positions reads (0: all)."""
        n = int(n)
        if self.window <= 0 or n <= self.window:
            return 0
        return (n - self.window) // BS

    def compact_slots(self, slots):
        slots = np.asarray(slots, np.int64)
        ok = (slots >= 0) & (slots < len(self.remap) * BS)
        blk = np.where(ok, self.remap[np.where(ok, slots // BS, 0)], -1)
        return np.where(blk >= 0, blk * BS + slots % BS, -1).astype(np.int64)

    def write_new_tokens(self, batch: W.Batch):
        """The decode step's cache write of the new tokens, on the host image."""
        sidx = torch.from_numpy(self.seqs).to(batch.k_new.device)
        slots = self.compact_slots(batch.slot_new.cpu().numpy()[self.seqs])
        oracle.kv_cache_write(host(batch.k_new[sidx]), host(batch.v_new[sidx]), self.k_cache,
                              self.v_cache, slots, self.src_dtype, self.cache_dtype, self.k_scale,
                              self.v_scale)

    def decode(self, rows=None, nthreads=0):
        return oracle.paged_decode(self.q, self.q_dtype, self.k_cache, self.v_cache,
                                   self.cache_dtype, self.block_tables, self.context_lens,
                                   self.scale, k_scale=self.k_scale, v_scale=self.v_scale,
                                   rows=rows, nthreads=nthreads, window=self.window)


def gpu_populate(pkv, batch: W.Batch):
    """INT8 / FP8 batches: quantize the source rows into the pool with the library."""
    if batch.k_src is not None and batch.k_src.shape[0] > 0:
        pkv.kv_cache_write(batch.k_src, batch.v_src, batch.k_cache, batch.v_cache,
                           batch.slot_src, batch.k_scale, batch.v_scale)


def gpu_step(pkv, batch: W.Batch, partition_size=0, out=None):
    """One decode step on the GPU: append the new tokens, then attend."""
    pkv.kv_cache_write(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_new,
                       batch.k_scale, batch.v_scale)
    return pkv.paged_attn_decode(batch.q, batch.k_cache, batch.v_cache, batch.block_tables,
                                 batch.context_lens, batch.scale, out=out,
                                 k_scale=batch.k_scale, v_scale=batch.v_scale,
                                 partition_size=partition_size)


def max_abs_err(gpu_out: torch.Tensor, ref: np.ndarray) -> float:
    g = as_f64(gpu_out)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if not np.isfinite(g).all():
        return float("inf")
    return float(np.abs(g - ref).max()) if g.size else 0.0


def hide_before_window(batch: W.Batch, window: int, n_of) -> torch.Tensor:
    """Block tables with the entries of whole blocks before the window set to
    -1 (as after pkv_bm_release_before), and the positions before the window
    inside its first block poisoned on the GPU: NaN K/V for float caches, NaN
    scales for quantized ones, and for FP8 also the NaN code 0x7F in K and V,
    so that a zero weight times such a value cannot pass.  n_of[b] is the
    context length the decode will see."""
    bt = batch.block_tables.clone()
    for b in range(batch.B):
        n = int(n_of[b])
        if window <= 0 or n <= window:
            continue
        lo = n - window
        j0 = lo // BS
        bt[b, :j0] = -1
        if lo % BS:
            blk = int(batch.layout.block_tables[b, j0])
            if batch.k_scale is not None:
                batch.k_scale[blk, :, :lo % BS] = float("nan")
                batch.v_scale[blk, :, :lo % BS] = float("nan")
                if batch.k_cache.dtype == torch.float8_e4m3fn:
                    batch.k_cache.view(torch.uint8)[blk, :, :lo % BS] = 0x7F
                    batch.v_cache.view(torch.uint8)[blk, :, :lo % BS] = 0x7F
            else:
                batch.k_cache[blk, :, :lo % BS] = float("nan")
                batch.v_cache[blk, :, :lo % BS] = float("nan")
    return bt


def guarded(shape, dtype: torch.dtype, device="cuda", guard_bytes: int = 512):
    """A contiguous tensor of `shape` inside a larger buffer whose first and
    last guard_bytes hold a sentinel bit pattern (0xA5 bytes).  Returns
    (tensor, check) where check() asserts the guard bands are untouched."""
    el = torch.empty((), dtype=dtype).element_size()
    g = guard_bytes // el
    n = int(np.prod(shape)) if len(shape) else 1
    raw = torch.full((guard_bytes * 2 + n * el,), 0xA5, dtype=torch.uint8, device=device)
    t = raw[guard_bytes:guard_bytes + n * el].view(dtype).view(*shape)
    assert t.data_ptr() % 256 == 0 or guard_bytes % 256 != 0

    def check():
        head = raw[:guard_bytes].cpu().numpy()
        tail = raw[guard_bytes + n * el:].cpu().numpy()
        assert (head == 0xA5).all(), "write before the buffer"
        assert (tail == 0xA5).all(), "write past the buffer"
        assert g >= 0

    return t, check
