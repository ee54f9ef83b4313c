"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays out the inputs a serving
system's block manager would hand to the kernels: context lengths, a block
pool, block tables, slot mappings for new tokens, and random q/K/V values.
It holds none of the attention, softmax or quantization arithmetic, and both
the CPU oracle and the HIP path receive exactly the arrays it produces.

Workload shapes follow the pages' LLaMA-7B / LLaMA-2-7B serving example
(docs.lazyllm.ai lesson 4, section 4.1: 32 heads x 128 dims, FP16, 32k context,
16 concurrent requests; caojiahao2.github.io section 2.2: LLaMA-7B shapes) and
the 16-token blocks of section 4.2 of the lazyllm page.  No dataset is used.

Random streams: ``numpy.random.default_rng([seed, stream])`` on the host for
structure (context lengths, block placement, outlier channels, random slots);
bulk values are N(0,1) float32, drawn with numpy on the CPU and with torch's
device generator (seeded from the same (seed, stream)) on a GPU, then rounded
to the storage dtype (round-to-nearest-even).  CPU and GPU batches of the same
seed therefore share structure but not values; each is deterministic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16

# stream ids of default_rng([seed, stream])
S_CTX, S_PERM, S_Q, S_K, S_V, S_OUTLIER, S_SLOTS, S_NEWK, S_NEWV = range(9)

CONFIGS = {
    # B=4, context {17,33,64,100}, 8 MHA heads, D=64, fp32, 64-block pool.
    "tiny": dict(B=4, ctx=[17, 33, 64, 100], Hq=8, Hkv=8, D=64, dtype="f32", cache="f32",
                 pool=64, seed=1, max_ctx=100),
    # LLaMA-7B-shaped MHA decode: 32/32 heads, D=128, fp16, B=64, ctx U[512,4096].
    "llama7b": dict(B=64, ctx=(512, 4096), Hq=32, Hkv=32, D=128, dtype="f16", cache="f16",
                    pool=None, seed=2, max_ctx=4096),
    # GQA decode: 32 q heads / 8 kv heads, D=128, bf16, B=128, ctx U[1024,8192].
    "gqa": dict(B=128, ctx=(1024, 8192), Hq=32, Hkv=8, D=128, dtype="bf16", cache="bf16",
                pool=None, seed=3, max_ctx=8192),
    # Long context: 16 x 32768, 32/32 heads, D=128, fp16, 1% of key channels x20,
    # split into 512-token partitions.
    "long": dict(B=16, ctx=[32768] * 16, Hq=32, Hkv=32, D=128, dtype="f16", cache="f16",
                 pool=None, seed=4, max_ctx=32768, outlier_frac=0.01, outlier_mult=20.0,
                 partition_size=512),
    # INT8 KV cache at the LLaMA-7B shape; q fp16; cache populated by the
    # quantizing cache write.
    "int8": dict(B=64, ctx=(512, 4096), Hq=32, Hkv=32, D=128, dtype="f16", cache="i8",
                 pool=None, seed=5, max_ctx=4096),
    # Sliding-window decode at the LLaMA-7B shape: contexts U[4096, 12288], each
    # sequence attends to its last 4096 positions (blocks before the window are
    # released: their table entries are -1).
    "window": dict(B=64, ctx=(4096, 12288), Hq=32, Hkv=32, D=128, dtype="f16", cache="f16",
                   pool=None, seed=9, max_ctx=12288, window=4096),
    # Speculative-decoding verification at the LLaMA-7B shape: every sequence
    # scores q_len = 8 tokens (7 drafts + 1) over U[512, 4096] cached tokens
    # (the 8 included), in one multi-query pass.
    "verify": dict(B=64, ctx=(512, 4096), Hq=32, Hkv=32, D=128, dtype="f16", cache="f16",
                   pool=None, seed=10, max_ctx=4096, q_len=8),
    # Chunked prefill at the LLaMA-7B shape: every sequence adds a 512-token
    # chunk of its prompt over U[1024, 4096] cached tokens (the chunk included).
    "prefill": dict(B=16, ctx=(1024, 4096), Hq=32, Hkv=32, D=128, dtype="f16", cache="f16",
                    pool=None, seed=11, max_ctx=4096, q_len=512),
    # 4-bit KV cache at the LLaMA-7B shape (per-row min/max, two codes a byte).
    "int4": dict(B=64, ctx=(512, 4096), Hq=32, Hkv=32, D=128, dtype="f16", cache="u4",
                 pool=None, seed=12, max_ctx=4096),
    # FP8 (e4m3) KV cache at the LLaMA-7B shape, populated the same way.
    "fp8": dict(B=64, ctx=(512, 4096), Hq=32, Hkv=32, D=128, dtype="f16", cache="f8",
                pool=None, seed=8, max_ctx=4096),
    # GQA with 8 q heads per kv head (64 q / 8 kv heads, D=128, bf16: the
    # attention of a LLaMA-70B-shaped layer), B=64, ctx U[512,4096].
    "gqa8": dict(B=64, ctx=(512, 4096), Hq=64, Hkv=8, D=128, dtype="bf16", cache="bf16",
                 pool=None, seed=14, max_ctx=4096),
    # The same layer shape over an INT8 cache (codes + fp32 scale per row,
    # quantized on write; bf16 q).
    "gqa8-int8": dict(B=64, ctx=(512, 4096), Hq=64, Hkv=8, D=128, dtype="bf16", cache="i8",
                      pool=None, seed=15, max_ctx=4096),
    # One GPU's share of the LLaMA-7B batch when 8 GPUs split it: by kv head
    # (4 of the 32 heads, every sequence; the same context lengths), by
    # sequence (8 sequences of the same length distribution, all heads), and
    # one GPU's share of the Long batch split by context (4,096 of each
    # sequence's 32,768 positions, 512-token partitions whose merge stands in
    # for the one after the all-gather of the partials).
    "tp8": dict(B=64, ctx=(512, 4096), Hq=4, Hkv=4, D=128, dtype="f16", cache="f16",
                pool=None, seed=2, max_ctx=4096),
    "dp8": dict(B=8, ctx=(512, 4096), Hq=32, Hkv=32, D=128, dtype="f16", cache="f16",
                pool=None, seed=13, max_ctx=4096),
    "cp8": dict(B=16, ctx=[4096] * 16, Hq=32, Hkv=32, D=128, dtype="f16", cache="f16",
                pool=None, seed=4, max_ctx=4096, outlier_frac=0.01, outlier_mult=20.0,
                partition_size=512),
}

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "i8": torch.int8, "f8": torch.float8_e4m3fn, "u4": torch.uint8}
# quantized caches, populated by the quantizing cache write: 1-byte codes with
# one fp32 scale per (slot, kv head) ("i8", "f8"), or 4-bit codes two per byte
# with an fp32 (x_min, range) pair per (slot, kv head) ("u4")
SCALED = ("i8", "f8", "u4")


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def draw_context_lens(cfg: dict, seed: int) -> np.ndarray:
    ctx = cfg["ctx"]
    if isinstance(ctx, tuple):
        lo, hi = ctx
        return rng(seed, S_CTX).integers(lo, hi, size=cfg["B"], endpoint=True).astype(np.int32)
    return np.asarray(ctx, dtype=np.int32)


def blocks_needed(n: int) -> int:
    return -(-int(n) // BLOCK_SIZE)


@dataclass
class Layout:
    """Block-manager output: where each sequence's logical blocks live."""
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B][MBS]; entries past a sequence's last block = -1
    num_blocks: int
    used_blocks: np.ndarray   # int64 ids of physical blocks holding data


def plan_layout(context_lens, num_blocks, max_blocks_per_seq, seed) -> Layout:
    """Assign logical blocks consecutively from a seeded permutation of the pool."""
    context_lens = np.asarray(context_lens, np.int32)
    B = len(context_lens)
    need = [blocks_needed(n) for n in context_lens]
    total = sum(need)
    if total > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {total}")
    if max(need, default=0) > max_blocks_per_seq:
        raise ValueError("a context is longer than max_blocks_per_seq * 16")
    perm = rng(seed, S_PERM).permutation(num_blocks).astype(np.int32)
    tables = np.full((B, max_blocks_per_seq), -1, np.int32)
    pos = 0
    for b in range(B):
        tables[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    return Layout(context_lens, tables, int(num_blocks), perm[:total].astype(np.int64))


def slots_for(layout: Layout, b: int, positions) -> np.ndarray:
    """Slot ids (block * 16 + offset) the block manager assigns to the given
    token positions of sequence b."""
    positions = np.asarray(positions, np.int64)
    blk = layout.block_tables[b, positions // BLOCK_SIZE].astype(np.int64)
    return blk * BLOCK_SIZE + positions % BLOCK_SIZE


def _normal(shape, seed, stream, device, dtype="f32", chunk_rows=None):
    """N(0,1) float32 rounded to `dtype`, on `device`."""
    tdt = TORCH_DTYPE[dtype]
    device = torch.device(device)
    if device.type == "cpu":
        a = rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
        return torch.from_numpy(a).to(tdt)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(stream))
    out = torch.empty(shape, dtype=tdt, device=device)
    rows = shape[0]
    step = chunk_rows or max(1, rows)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                                 dtype=torch.float32).to(tdt)
    return out


def _fill_normal_(t, seed, stream, chunk_rows=None, post=None):
    """In-place N(0,1) fill of a device/CPU tensor, in chunks along dim 0."""
    device = t.device
    rows = t.shape[0]
    if device.type == "cpu":
        a = rng(seed, stream).standard_normal(size=tuple(t.shape), dtype=np.float32)
        x = torch.from_numpy(a)
        if post is not None:
            x = post(x)
        t.copy_(x.to(t.dtype))
        return t
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(stream))
    step = chunk_rows or rows
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0,) + tuple(t.shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if post is not None:
            x = post(x)
        t[r0:r1] = x.to(t.dtype)
    return t


@dataclass
class Batch:
    name: str
    cfg: dict
    seed: int
    layout: Layout
    q: torch.Tensor                 # [B][Hq][D]
    k_cache: torch.Tensor           # [NB][Hkv][16][D]
    v_cache: torch.Tensor
    k_scale: torch.Tensor | None    # [NB][Hkv][16] float32 (INT8 only)
    v_scale: torch.Tensor | None
    block_tables: torch.Tensor      # int32 [B][MBS]
    context_lens: torch.Tensor      # int32 [B]
    k_new: torch.Tensor             # [B][Hkv][D] the decode step's new token
    v_new: torch.Tensor
    slot_new: torch.Tensor          # int64 [B], slot of position context_len-1
    scale: float
    # INT8 only: source rows of positions 0..N_b-2 and their slots
    k_src: torch.Tensor | None = None
    v_src: torch.Tensor | None = None
    slot_src: torch.Tensor | None = None
    outlier_channels: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.k_cache.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]


def default_pool_blocks(context_lens) -> int:
    return int(math.ceil(1.1 * sum(blocks_needed(n) for n in context_lens)))


def make_batch(name: str | None = None, device="cpu", seed: int | None = None, poison=True,
               cfg: dict | None = None) -> Batch:
    """Build the named workload (or a custom `cfg` with the same keys).

    poison=True fills every pool slot that holds no token with NaN (K and V for
    float caches; the per-token scales for INT8 caches) so that a kernel which
    reads outside the context cannot go unnoticed (the per-token scales for
    INT8 / FP8 caches); poison=False fills them with zeros (timing runs).
    """
    if cfg is None:
        cfg = CONFIGS[name]
    cfg = dict(cfg)
    seed = cfg.get("seed", 0) if seed is None else seed
    device = torch.device(device)
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    dtype, cache = cfg["dtype"], cfg["cache"]
    lens = draw_context_lens(cfg, seed)
    mbs = cfg.get("max_blocks_per_seq") or blocks_needed(cfg.get("max_ctx") or int(lens.max()))
    nb = cfg.get("pool") or default_pool_blocks(lens)
    layout = plan_layout(lens, nb, mbs, seed)
    scale = float(np.float32(1.0 / math.sqrt(D)))

    # outlier key channels: (kv_head, d) pairs sampled without replacement
    outl = None
    if cfg.get("outlier_frac"):
        n_ch = int(math.ceil(cfg["outlier_frac"] * Hkv * D))
        flat = rng(seed, S_OUTLIER).choice(Hkv * D, size=n_ch, replace=False)
        outl = np.stack([flat // D, flat % D], axis=1).astype(np.int64)
    mult = float(cfg.get("outlier_mult", 1.0))

    def k_post(x):  # scale outlier channels in fp32 before the storage cast
        if outl is None:
            return x
        m = torch.ones(Hkv, D, dtype=torch.float32)
        m[outl[:, 0], outl[:, 1]] = mult
        return x * m.to(x.device).view(*([1] * (x.dim() - 2)), Hkv, D)

    chunk = 256
    q = _normal((B, Hq, D), seed, S_Q, device, dtype)
    k_new = torch.empty((B, Hkv, D), dtype=TORCH_DTYPE[dtype], device=device)
    v_new = torch.empty_like(k_new)
    _fill_normal_(k_new, seed, S_NEWK, post=k_post)
    _fill_normal_(v_new, seed, S_NEWV)
    slot_new = np.array([slots_for(layout, b, [max(int(n) - 1, 0)])[0] if n > 0 else -1
                         for b, n in enumerate(lens)], np.int64)

    k_scale = v_scale = k_src = v_src = slot_src = src_offsets = None
    if cache in SCALED:
        row = D // 2 if cache == "u4" else D
        k_cache = torch.zeros((nb, Hkv, BLOCK_SIZE, row), dtype=torch.uint8,
                              device=device).view(TORCH_DTYPE[cache])
        v_cache = torch.zeros((nb, Hkv, BLOCK_SIZE, row), dtype=torch.uint8,
                              device=device).view(TORCH_DTYPE[cache])
        fill = float("nan") if poison else 0.0
        meta = (nb, Hkv, BLOCK_SIZE, 2) if cache == "u4" else (nb, Hkv, BLOCK_SIZE)
        k_scale = torch.full(meta, fill, dtype=torch.float32, device=device)
        v_scale = torch.full_like(k_scale, fill)
        # prefill rows: positions 0..N_b-2 of every sequence, in sequence order
        slots = [slots_for(layout, b, np.arange(max(int(n) - 1, 0))) for b, n in enumerate(lens)]
        slot_src_np = np.concatenate(slots) if slots else np.zeros(0, np.int64)
        T = len(slot_src_np)
        k_src = torch.empty((T, Hkv, D), dtype=TORCH_DTYPE[dtype], device=device)
        v_src = torch.empty_like(k_src)
        _fill_normal_(k_src, seed, S_K, chunk_rows=1 << 14, post=k_post)
        _fill_normal_(v_src, seed, S_V, chunk_rows=1 << 14)
        slot_src = torch.from_numpy(slot_src_np).to(device)
        src_offsets = np.concatenate([[0], np.cumsum([len(x) for x in slots])]).astype(np.int64)
    else:
        tdt = TORCH_DTYPE[cache]
        k_cache = torch.empty((nb, Hkv, BLOCK_SIZE, D), dtype=tdt, device=device)
        v_cache = torch.empty_like(k_cache)
        _fill_normal_(k_cache, seed, S_K, chunk_rows=chunk,
                      post=(None if outl is None else
                            (lambda x: k_post(x.transpose(1, 2)).transpose(1, 2))))
        _fill_normal_(v_cache, seed, S_V, chunk_rows=chunk)
        fill = float("nan") if poison else 0.0
        unused = np.setdiff1d(np.arange(nb), layout.used_blocks)
        if len(unused):
            idx = torch.from_numpy(unused).to(device)
            k_cache.index_fill_(0, idx, fill)
            v_cache.index_fill_(0, idx, fill)
        for b, n in enumerate(lens):
            n = int(n)
            if n % BLOCK_SIZE:
                last = int(layout.block_tables[b, (n - 1) // BLOCK_SIZE])
                k_cache[last, :, n % BLOCK_SIZE:, :] = fill
                v_cache[last, :, n % BLOCK_SIZE:, :] = fill

    return Batch(name=name or "custom", cfg=cfg, seed=seed, layout=layout, q=q,
                 k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
                 block_tables=torch.from_numpy(layout.block_tables).to(device),
                 context_lens=torch.from_numpy(lens).to(device), k_new=k_new, v_new=v_new,
                 slot_new=torch.from_numpy(slot_new).to(device), scale=scale, k_src=k_src,
                 v_src=v_src, slot_src=slot_src, outlier_channels=outl,
                 extra={"src_offsets": src_offsets})


def random_slots(num_blocks: int, T: int, seed: int) -> np.ndarray:
    """T distinct random slots of a pool (for cache-write tests)."""
    return rng(seed, S_SLOTS).choice(num_blocks * BLOCK_SIZE, size=T, replace=False).astype(
        np.int64)


def algorithmic_bytes(context_lens, Hq, Hkv, D, e_kv, e_q, int8_scales=False,
                      meta_bytes=None) -> int:
    """Bytes a decode step over this batch must move at least: every context
    token's K and V rows (e_kv bytes per element, 0.5 for 4-bit codes; plus a
    4-byte scale each for INT8 / FP8, or meta_bytes per row), q and out, the
    block-table entries actually used and the context lengths."""
    lens = np.asarray(context_lens, np.int64)
    tok = int(lens.sum())
    meta = meta_bytes if meta_bytes is not None else (4 if int8_scales else 0)
    per_tok = int(Hkv * 2 * (D * e_kv + meta))
    B = len(lens)
    return (tok * per_tok + B * Hq * D * 2 * e_q
            + int(sum(blocks_needed(n) for n in lens)) * 4 + 4 * B)


# Parallel sampling over shared prompts (the prefix-sharing workload of the
# block manager): `prompts` prompts with lengths U[lo, hi] are each continued
# by `samples` sequences (parallel sampling / beams, lecture 13 notes,
# "PagedAttention" advantages), which then decode `gen` tokens each.
# LLaMA-7B shapes as above.
SAMPLING = {
    "sampling-small": dict(prompts=3, samples=3, prompt_len=[37, 16, 100], Hq=8, Hkv=2, D=128,
                           dtype="f16", cache="f16", gen=20, seed=6),
    "sampling": dict(prompts=16, samples=4, prompt_len=(512, 2048), Hq=32, Hkv=32, D=128,
                     dtype="f16", cache="f16", gen=64, seed=7),
}
S_PROMPT, S_TOKEN_K, S_TOKEN_V, S_STEP_Q = 20, 21, 22, 23


def sampling_prompt_lens(cfg: dict) -> np.ndarray:
    pl = cfg["prompt_len"]
    if isinstance(pl, (list, tuple)) and len(pl) == cfg["prompts"] and not (
            isinstance(pl, tuple) and len(pl) == 2):
        return np.asarray(pl, np.int64)
    lo, hi = pl
    return rng(cfg["seed"], S_PROMPT).integers(lo, hi, size=cfg["prompts"],
                                               endpoint=True).astype(np.int64)


def token_rows(n: int, Hkv: int, D: int, dtype: str, seed: int, stream: int,
               device="cpu") -> torch.Tensor:
    """[n][Hkv][D] N(0,1) rows rounded to dtype: the K (or V) row of token id
    0..n-1.  Row values depend only on (seed, stream, n, device)."""
    return _normal((n, Hkv, D), seed, stream, device, dtype)


def multi_query_flops(context_lens, q_len: int, Hq: int, D: int) -> int:
    """Flops of causal multi-query attention: every query at position p scores
    p + 1 keys and sums p + 1 values, 2 D flops each, per q head."""
    total = 0
    for n in np.asarray(context_lens, np.int64):
        ql = min(int(q_len), int(n))
        p = np.arange(int(n) - ql, int(n), dtype=np.int64)
        total += int((p + 1).sum()) * 4 * D * Hq
    return total
