"""Python binding of libpkv (paged KV-cache decode attention for MI355X).

Thin ctypes layer over the C ABI declared in ``include/pkv.h``: it checks
torch metadata (device, dtype, shape, contiguity), passes raw device pointers
and the current HIP stream, and raises ``RuntimeError`` on a non-OK status.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  Function names are the C entry points without their ``pkv_``
prefix.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "kv_cache_write", "paged_attn_decode", "paged_attn_decode_append",
    "paged_attn_decode_append_static", "STATIC_SCRATCH_BYTES",
    "paged_attn_decode_sliding", "paged_attn_multi",
    "paged_attn_decode_partials", "paged_attn_reduce",
    "decode_workspace_size", "default_partition_size", "num_partitions",
    "BlockManager", "copy_blocks", "stream_read", "tile_read", "mfma_rate", "lds_read_rate",
    "library_path", "PkvError", "BLOCK_SIZE",
]

BLOCK_SIZE = 16
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv.so")

F32, F16, BF16, I8, F8_E4M3, U4 = 0, 1, 2, 3, 4, 5
# a 4-bit cache is a torch.uint8 tensor [NB][Hkv][16][D/2] (two codes per
# byte) with scale arrays [NB][Hkv][16][2] float32 holding (x_min, range)
_DTYPE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.int8: I8,
          torch.float8_e4m3fn: F8_E4M3, torch.uint8: U4}
# caches of 1-byte codes with one float32 scale per (slot, kv head)
SCALED_DTYPES = (torch.int8, torch.float8_e4m3fn)


def _head_dim(cache: torch.Tensor) -> int:
    return cache.shape[3] * 2 if cache.dtype == torch.uint8 else cache.shape[3]


def _check_scales(k_cache, k_scale, v_scale, NB, Hkv, bs):
    if k_cache.dtype in SCALED_DTYPES:
        _dev(k_scale, "k_scale", dtype=torch.float32, ndim=3)
        _dev(v_scale, "v_scale", dtype=torch.float32, ndim=3)
        if tuple(k_scale.shape) != (NB, Hkv, bs) or v_scale.shape != k_scale.shape:
            raise ValueError("scale arrays must be [num_blocks][num_kv_heads][16]")
    elif k_cache.dtype == torch.uint8:
        _dev(k_scale, "k_scale", dtype=torch.float32, ndim=4)
        _dev(v_scale, "v_scale", dtype=torch.float32, ndim=4)
        if tuple(k_scale.shape) != (NB, Hkv, bs, 2) or v_scale.shape != k_scale.shape:
            raise ValueError("4-bit scale arrays must be [num_blocks][num_kv_heads][16][2]")


class PkvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"pkv status {status}: {detail}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libpkv.so not found at {_LIB_PATH}: the HIP library must be built first "
            "(python -m paged_kv_cache_264_amd.build, or __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    P, I, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                        ctypes.c_size_t)
    L.pkv_kv_cache_write.argtypes = [P, P, P, P, P, P, P, I64, I, I, I, I64, I, I, P]
    L.pkv_kv_cache_write.restype = I
    L.pkv_default_partition_size.argtypes = [I, I, I, I, I]
    L.pkv_default_partition_size.restype = I
    L.pkv_decode_workspace_size.argtypes = [I, I, I, I, I, I, I]
    L.pkv_decode_workspace_size.restype = SZ
    L.pkv_paged_attn_decode.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I64, F, I, P,
                                        SZ, I, I, P]
    L.pkv_paged_attn_decode.restype = I
    L.pkv_paged_attn_decode_append.argtypes = [P, P, P, P, P, P, P, P, P, I, P, I, I, I, I, I,
                                               I64, F, I, P, SZ, I, I, P]
    L.pkv_paged_attn_decode_append.restype = I
    L.pkv_paged_attn_decode_append_static.argtypes = [P, P, P, P, P, P, P, P, P, I, P, I, I, I,
                                                      I, I, I64, F, I, I, I, P]
    L.pkv_paged_attn_decode_append_static.restype = I
    L.pkv_paged_attn_decode_sliding.argtypes = [P, P, P, P, P, P, P, P, P, I, P, I, I, I, I, I,
                                                I64, F, I, I, P, SZ, I, I, P]
    L.pkv_paged_attn_decode_sliding.restype = I
    L.pkv_bm_release_before.argtypes = [P, I64, I64]
    L.pkv_bm_release_before.restype = I
    L.pkv_paged_attn_multi.argtypes = [P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, I64, F, I,
                                       P, SZ, I, I, P]
    L.pkv_paged_attn_multi.restype = I
    L.pkv_paged_attn_decode_shared_prefix.argtypes = [P, P, P, P, P, P, P, I, P, P, P, I, I, I, I,
                                                      I, I, I, I64, F, P, SZ, I, I, P]
    L.pkv_paged_attn_decode_shared_prefix.restype = I
    L.pkv_shared_prefix_workspace_size.argtypes = [I, I, I, I, I, I, I]
    L.pkv_shared_prefix_workspace_size.restype = SZ
    L.pkv_multi_workspace_size.argtypes = [I, I, I, I, I]
    L.pkv_multi_workspace_size.restype = SZ
    L.pkv_multi_default_partition_size.argtypes = [I, I, I, I, I]
    L.pkv_multi_default_partition_size.restype = I
    L.pkv_paged_attn_decode_partials.argtypes = [P, P, P, P, P, P, P, P, P, P, I, P, I, I, I, I,
                                                 I, I64, F, I, I, I, I, P]
    L.pkv_paged_attn_decode_partials.restype = I
    L.pkv_paged_attn_reduce.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P]
    L.pkv_paged_attn_reduce.restype = I
    L.pkv_copy_blocks.argtypes = [P, P, P, P, P, I64, I, I, I, I64, I, P]
    L.pkv_copy_blocks.restype = I
    L.pkv_bm_create.argtypes = [I64, I, ctypes.POINTER(P)]
    L.pkv_bm_create.restype = I
    L.pkv_bm_destroy.argtypes = [P]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_add_sequence.argtypes = [P, I64]
    L.pkv_bm_add_sequence.restype = I
    L.pkv_bm_fork.argtypes = [P, I64, I64]
    L.pkv_bm_fork.restype = I
    L.pkv_bm_free_sequence.argtypes = [P, I64]
    L.pkv_bm_free_sequence.restype = I
    L.pkv_bm_append.argtypes = [P, P, P, I, P, P, I64, ctypes.POINTER(I64)]
    L.pkv_bm_append.restype = I
    L.pkv_bm_block_tables.argtypes = [P, P, I, I, P, P]
    L.pkv_bm_block_tables.restype = I
    L.pkv_bm_num_free_blocks.argtypes = [P]
    L.pkv_bm_num_free_blocks.restype = I64
    L.pkv_bm_sequence_length.argtypes = [P, I64]
    L.pkv_bm_sequence_length.restype = I64
    L.pkv_stream_read.argtypes = [P, I64, P, P]
    L.pkv_stream_read.restype = I
    L.pkv_tile_read.argtypes = [P, P, P, I, P, I, P, I, I, I, I64, I, P, P]
    L.pkv_tile_read.restype = I
    L.pkv_mfma_rate.argtypes = [I, I, P, P]
    L.pkv_mfma_rate.restype = I
    L.pkv_lds_read_rate.argtypes = [I, I, I, P, P]
    L.pkv_lds_read_rate.restype = I
    L.pkv_status_string.argtypes = [I]
    L.pkv_status_string.restype = ctypes.c_char_p
    L.pkv_last_error.argtypes = []
    L.pkv_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check_status(rc: int):
    if rc != 0:
        L = _load()
        raise PkvError(rc, f"{L.pkv_status_string(rc).decode()}: {L.pkv_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {tuple(t.shape)})")
    return t


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _code(dtype: torch.dtype, name: str) -> int:
    if dtype not in _DTYPE:
        raise TypeError(f"{name}: unsupported dtype {dtype}")
    return _DTYPE[dtype]


def default_partition_size(num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq,
                           cache_dtype: torch.dtype) -> int:
    """The partition size the decode entry points use when passed 0, for a
    cache of cache_dtype (the torch dtype of k_cache)."""
    return _load().pkv_default_partition_size(num_seqs, num_q_heads, num_kv_heads,
                                              max_blocks_per_seq, _code(cache_dtype, "cache_dtype"))


def num_partitions(max_blocks_per_seq: int, partition_size: int) -> int:
    return -(-max_blocks_per_seq * BLOCK_SIZE // partition_size)


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          partition_size, cache_dtype: torch.dtype) -> int:
    """Workspace bytes of a decode over a cache of cache_dtype (partition_size
    0: the default size)."""
    return _load().pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_blocks_per_seq, partition_size,
                                             _code(cache_dtype, "cache_dtype"))


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A workspace of at least nbytes for one call, from torch's caching
    allocator on the current stream.  The allocator hands a freed block to
    another allocation only on the stream it was allocated on (in stream
    order), so calls on different streams never share partials, and the
    buffer stays valid until the call's kernels have run."""
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _out(out, q, name="out"):
    """The caller's output buffer (same dtype and shape as q), or a new one."""
    if out is None:
        return torch.empty_like(q)
    _dev(out, name, dtype=q.dtype, ndim=3)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"{name} must have q's shape {tuple(q.shape)} (got {tuple(out.shape)})")
    if out.device != q.device:
        raise ValueError(f"{name} must be on q's device")
    return out


def kv_cache_write(k, v, k_cache, v_cache, slot_mapping, k_scale=None, v_scale=None):
    """Write new tokens' K/V rows ([T][Hkv][D]) into the pool at their slots;
    INT8 caches quantize on write (scales [NB][Hkv][16] float32)."""
    _dev(k, "k", ndim=3)
    _dev(v, "v", dtype=k.dtype, ndim=3)
    _dev(k_cache, "k_cache", ndim=4)
    _dev(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _dev(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1)
    T, Hkv, D = k.shape
    NB, Hkv2, bs, _ = k_cache.shape
    D2 = _head_dim(k_cache)
    if v.shape != k.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D):
        raise ValueError("k/v and cache shapes disagree")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one entry per token")
    _check_scales(k_cache, k_scale, v_scale, NB, Hkv, bs)
    rc = _load().pkv_kv_cache_write(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                    _ptr(v_scale), _ptr(slot_mapping), T, Hkv, D, bs, NB,
                                    _code(k.dtype, "k"), _code(k_cache.dtype, "k_cache"),
                                    _stream(k))
    _check_status(rc)


def _decode_common(q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale):
    _dev(q, "q", ndim=3)
    _dev(k_cache, "k_cache", ndim=4)
    _dev(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    B, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    if _head_dim(k_cache) != D or v_cache.shape != k_cache.shape:
        raise ValueError("q / cache shapes disagree")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables and context_lens need one row per sequence")
    _check_scales(k_cache, k_scale, v_scale, NB, Hkv, bs)
    return B, Hq, D, NB, Hkv, bs


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None,
                      k_scale=None, v_scale=None, partition_size=0, workspace=None):
    """softmax(scale * q K^T) V per sequence and q head over the paged cache."""
    B, Hq, D, NB, Hkv, bs = _decode_common(q, k_cache, v_cache, block_tables, context_lens,
                                           k_scale, v_scale)
    out = _out(out, q)
    mbs = block_tables.shape[1]
    need = decode_workspace_size(B, Hq, Hkv, D, mbs, partition_size, k_cache.dtype)
    if workspace is None:
        workspace = _workspace(q.device, need)
    else:
        _dev(workspace, "workspace")
        if workspace.device != q.device:
            raise ValueError("workspace must be on q's device")
    rc = _load().pkv_paged_attn_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), mbs, _ptr(context_lens), B, Hq, Hkv, D, bs, NB, float(scale),
        int(partition_size), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _code(q.dtype, "q"), _code(k_cache.dtype, "k_cache"), _stream(q))
    _check_status(rc)
    return out


def paged_attn_decode_append(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                             out=None, k_scale=None, v_scale=None, partition_size=0,
                             workspace=None):
    """One decode step: write each sequence's new token (k_new, v_new
    [B][Hkv][D], q dtype) at position context_len-1, then attend."""
    B, Hq, D, NB, Hkv, bs = _decode_common(q, k_cache, v_cache, block_tables, context_lens,
                                           k_scale, v_scale)
    _dev(k_new, "k_new", dtype=q.dtype, ndim=3)
    _dev(v_new, "v_new", dtype=q.dtype, ndim=3)
    if tuple(k_new.shape) != (B, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim]")
    out = _out(out, q)
    mbs = block_tables.shape[1]
    need = decode_workspace_size(B, Hq, Hkv, D, mbs, partition_size, k_cache.dtype)
    if workspace is None:
        workspace = _workspace(q.device, need)
    else:
        _dev(workspace, "workspace")
        if workspace.device != q.device:
            raise ValueError("workspace must be on q's device")
    rc = _load().pkv_paged_attn_decode_append(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), mbs, _ptr(context_lens), B, Hq, Hkv,
        D, bs, NB, float(scale), int(partition_size), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _code(q.dtype, "q"),
        _code(k_cache.dtype, "k_cache"), _stream(q))
    _check_status(rc)
    return out


STATIC_SCRATCH_BYTES = 32 << 20   # PKV_STATIC_SCRATCH_BYTES of include/pkv.h


def paged_attn_decode_append_static(q, k_new, v_new, k_cache, v_cache, block_tables,
                                    context_lens, scale, out, k_scale=None, v_scale=None,
                                    partition_size=0):
    """paged_attn_decode_append with the partials in the library's static
    per-GPU scratch array (STATIC_SCRATCH_BYTES) instead of a workspace: the
    C entry point allocates nothing.  `out` is required (this wrapper does not
    allocate either).  Calls that overlap on one GPU race."""
    B, Hq, D, NB, Hkv, bs = _decode_common(q, k_cache, v_cache, block_tables, context_lens,
                                           k_scale, v_scale)
    _dev(k_new, "k_new", dtype=q.dtype, ndim=3)
    _dev(v_new, "v_new", dtype=q.dtype, ndim=3)
    if tuple(k_new.shape) != (B, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim]")
    if out is None:
        raise ValueError("out is required")
    out = _out(out, q)
    rc = _load().pkv_paged_attn_decode_append_static(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Hq, Hkv, D, bs, NB, float(scale), int(partition_size),
        _code(q.dtype, "q"), _code(k_cache.dtype, "k_cache"), _stream(q))
    _check_status(rc)
    return out


def shared_prefix_workspace_size(num_seqs, num_groups, max_group_size, num_q_heads, num_kv_heads,
                                 head_dim, max_blocks_per_seq):
    return int(_load().pkv_shared_prefix_workspace_size(num_seqs, num_groups, max_group_size,
                                                        num_q_heads, num_kv_heads, head_dim,
                                                        max_blocks_per_seq))


def paged_attn_decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, prefix_lens,
                                    group_start, scale, max_group_size, k_new=None, v_new=None,
                                    out=None, workspace=None):
    """Decode of groups of sequences that continue one prompt: sequences
    group_start[g] .. group_start[g+1]-1 (int32 [G+1] on the GPU) share their
    first prefix_lens[b] positions (int32 [B], equal within a group, the same
    physical blocks), which are read once per group.  Same result as
    paged_attn_decode (or paged_attn_decode_append with k_new / v_new)."""
    B, Hq, D, NB, Hkv, bs = _decode_common(q, k_cache, v_cache, block_tables, context_lens,
                                           None, None)
    _dev(prefix_lens, "prefix_lens", dtype=torch.int32, ndim=1)
    _dev(group_start, "group_start", dtype=torch.int32, ndim=1)
    if prefix_lens.shape[0] != B:
        raise ValueError("prefix_lens needs one entry per sequence")
    G = group_start.shape[0] - 1
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _dev(k_new, "k_new", dtype=q.dtype, ndim=3)
        _dev(v_new, "v_new", dtype=q.dtype, ndim=3)
        if tuple(k_new.shape) != (B, Hkv, D) or v_new.shape != k_new.shape:
            raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim]")
    out = _out(out, q)
    mbs = block_tables.shape[1]
    need = shared_prefix_workspace_size(B, G, int(max_group_size), Hq, Hkv, D, mbs)
    if workspace is None:
        workspace = _workspace(q.device, need)
    else:
        _dev(workspace, "workspace")
        if workspace.device != q.device:
            raise ValueError("workspace must be on q's device")
    rc = _load().pkv_paged_attn_decode_shared_prefix(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), mbs, _ptr(context_lens), _ptr(prefix_lens), _ptr(group_start), G,
        int(max_group_size), B, Hq, Hkv, D, bs, NB, float(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _code(q.dtype, "q"),
        _code(k_cache.dtype, "k_cache"), _stream(q))
    _check_status(rc)
    return out


def paged_attn_decode_sliding(q, k_cache, v_cache, block_tables, context_lens, scale,
                              sliding_window, k_new=None, v_new=None, out=None, k_scale=None,
                              v_scale=None, partition_size=0, workspace=None):
    """Decode over each sequence's last `sliding_window` positions only; with
    k_new / v_new given, the new token is appended first (as in
    paged_attn_decode_append)."""
    B, Hq, D, NB, Hkv, bs = _decode_common(q, k_cache, v_cache, block_tables, context_lens,
                                           k_scale, v_scale)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _dev(k_new, "k_new", dtype=q.dtype, ndim=3)
        _dev(v_new, "v_new", dtype=q.dtype, ndim=3)
        if tuple(k_new.shape) != (B, Hkv, D) or v_new.shape != k_new.shape:
            raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim]")
    out = _out(out, q)
    mbs = block_tables.shape[1]
    mbs_eff = min(mbs, int(sliding_window) // BLOCK_SIZE + 2) if sliding_window > 0 else mbs
    need = decode_workspace_size(B, Hq, Hkv, D, mbs_eff, partition_size, k_cache.dtype)
    if workspace is None:
        workspace = _workspace(q.device, need)
    else:
        _dev(workspace, "workspace")
        if workspace.device != q.device:
            raise ValueError("workspace must be on q's device")
    rc = _load().pkv_paged_attn_decode_sliding(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), mbs, _ptr(context_lens), B, Hq, Hkv,
        D, bs, NB, float(scale), int(sliding_window), int(partition_size), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _code(q.dtype, "q"),
        _code(k_cache.dtype, "k_cache"), _stream(q))
    _check_status(rc)
    return out


def paged_attn_multi(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale,
                     max_query_len, out=None, partition_size=0, workspace=None):
    """Causal attention of several query tokens per sequence (speculative
    verification, prefill chunks): q [T][Hq][D]; the queries of sequence b are
    rows query_start_loc[b] .. query_start_loc[b+1]-1 (int32 [B+1] on the GPU)
    and sit at its last positions (their K/V already in the cache)."""
    _dev(q, "q", ndim=3)
    _dev(k_cache, "k_cache", dtype=q.dtype, ndim=4)
    _dev(v_cache, "v_cache", dtype=q.dtype, ndim=4)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _dev(query_start_loc, "query_start_loc", dtype=torch.int32, ndim=1)
    T, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    B = context_lens.shape[0]
    if D2 != D or v_cache.shape != k_cache.shape or query_start_loc.shape[0] != B + 1 or \
            block_tables.shape[0] != B:
        raise ValueError("q / cache / table / query_start_loc shapes disagree")
    out = _out(out, q)
    mbs = block_tables.shape[1]
    L = _load()
    P = partition_size or L.pkv_multi_default_partition_size(B, int(max_query_len), Hq, Hkv, mbs)
    need = L.pkv_multi_workspace_size(T, Hq, D, mbs, P) if P else 0
    if workspace is None:
        workspace = _workspace(q.device, need)
    else:
        _dev(workspace, "workspace")
        if workspace.device != q.device:
            raise ValueError("workspace must be on q's device")
    rc = L.pkv_paged_attn_multi(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), mbs,
        _ptr(context_lens), _ptr(query_start_loc), B, T, int(max_query_len), Hq, Hkv, D, bs, NB,
        float(scale), int(partition_size), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _code(q.dtype, "q"),
        _code(k_cache.dtype, "k_cache"), _stream(q))
    _check_status(rc)
    return out


def paged_attn_decode_partials(q, k_cache, v_cache, block_tables, context_lens, scale,
                               partition_size, num_partitions_=None, k_scale=None, v_scale=None,
                               out=None, partials=None):
    """Phase 1 of the split decode: per-partition (m, l, o) fp32 partials
    m, l [B][Hq][NP] and o [B][Hq][NP][D].  With `out` given, sequences that fit
    in one partition are finished into `out` and write no partial.  Entries
    that are not written keep their previous contents (NaN when allocated
    here).  Returns (m, l, o)."""
    B, Hq, D, NB, Hkv, bs = _decode_common(q, k_cache, v_cache, block_tables, context_lens,
                                           k_scale, v_scale)
    mbs = block_tables.shape[1]
    NP = num_partitions_ or num_partitions(mbs, partition_size)
    if partials is None:
        m = torch.full((B, Hq, NP), float("nan"), dtype=torch.float32, device=q.device)
        l = torch.full_like(m, float("nan"))
        o = torch.full((B, Hq, NP, D), float("nan"), dtype=torch.float32, device=q.device)
    else:
        m, l, o = partials
        _dev(m, "m_part", dtype=torch.float32, ndim=3)
        _dev(l, "l_part", dtype=torch.float32, ndim=3)
        _dev(o, "o_part", dtype=torch.float32, ndim=4)
        if tuple(m.shape) != (B, Hq, NP) or l.shape != m.shape or tuple(o.shape) != (B, Hq, NP, D):
            raise ValueError("partials must be [B][Hq][NP] and [B][Hq][NP][D]")
    if out is not None:
        out = _out(out, q)
    rc = _load().pkv_paged_attn_decode_partials(
        _ptr(out), _ptr(m), _ptr(l), _ptr(o), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), mbs, _ptr(context_lens), B, Hq, Hkv, D,
        bs, NB, float(scale), int(partition_size), NP, _code(q.dtype, "q"),
        _code(k_cache.dtype, "k_cache"), _stream(q))
    _check_status(rc)
    return m, l, o


def paged_attn_reduce(m_part, l_part, o_part, context_lens, partition_size, out=None,
                      out_dtype=torch.float32, skip_single_partition=False):
    """Phase 2: merge partials into out [B][Hq][D].  skip_single_partition
    leaves sequences with at most one partition untouched."""
    _dev(m_part, "m_part", dtype=torch.float32, ndim=3)
    _dev(l_part, "l_part", dtype=torch.float32, ndim=3)
    _dev(o_part, "o_part", dtype=torch.float32, ndim=4)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    B, Hq, NP, D = o_part.shape
    if tuple(m_part.shape) != (B, Hq, NP) or l_part.shape != m_part.shape:
        raise ValueError(f"m_part and l_part must be [B][Hq][NP] = {(B, Hq, NP)} (got "
                         f"{tuple(m_part.shape)}, {tuple(l_part.shape)})")
    if context_lens.shape[0] != B:
        raise ValueError(f"context_lens needs one entry per sequence ({B})")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=o_part.device)
    _dev(out, "out", ndim=3)
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError(f"out must be [B][Hq][D] = {(B, Hq, D)} (got {tuple(out.shape)})")
    rc = _load().pkv_paged_attn_reduce(_ptr(out), _ptr(m_part), _ptr(l_part), _ptr(o_part),
                                       _ptr(context_lens), B, Hq, D, int(partition_size), NP,
                                       1 if skip_single_partition else 0,
                                       _code(out.dtype, "out"), _stream(o_part))
    _check_status(rc)
    return out


def copy_blocks(k_cache, v_cache, copy_pairs, k_scale=None, v_scale=None):
    """Copy whole pool blocks (all kv heads of K and V, and the scale rows of
    an INT8 cache) for each (src, dst) row of copy_pairs ([n][2] int32 on the
    GPU): the copy-on-write step of BlockManager.append."""
    _dev(k_cache, "k_cache", ndim=4)
    _dev(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _dev(copy_pairs, "copy_pairs", dtype=torch.int32, ndim=2)
    if copy_pairs.shape[1] != 2:
        raise ValueError("copy_pairs must be [n][2]")
    NB, Hkv, bs, _ = k_cache.shape
    D = _head_dim(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes disagree")
    _check_scales(k_cache, k_scale, v_scale, NB, Hkv, bs)
    rc = _load().pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                 _ptr(copy_pairs), copy_pairs.shape[0], Hkv, D, bs, NB,
                                 _code(k_cache.dtype, "k_cache"), _stream(k_cache))
    _check_status(rc)


def stream_read(src: torch.Tensor, sink: torch.Tensor):
    """Measurement helper: read every byte of `src` once (plain streaming
    read, no arithmetic).  `sink` is a 1-element int32 device tensor."""
    _dev(src, "src")
    _dev(sink, "sink", dtype=torch.int32)
    rc = _load().pkv_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                 _stream(src))
    _check_status(rc)


def tile_read(k_cache, v_cache, block_tables, context_lens, items, sink):
    """Measurement helper: the decode's K/V tile reads without arithmetic, one
    work-group per (sequence, kv head) row of `items` (int32 [n][2] on the
    GPU), in that order.  4 KiB tiles only."""
    _dev(k_cache, "k_cache", ndim=4)
    _dev(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4)
    _dev(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _dev(items, "items", dtype=torch.int32, ndim=2)
    _dev(sink, "sink", dtype=torch.int32)
    if items.shape[1] != 2 or block_tables.shape[0] != context_lens.shape[0]:
        raise ValueError("items must be [n][2] and the tables one row per sequence")
    NB, Hkv, bs, _ = k_cache.shape
    rc = _load().pkv_tile_read(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                               block_tables.shape[1], _ptr(context_lens), context_lens.shape[0],
                               _ptr(items), items.shape[0], Hkv, _head_dim(k_cache), NB,
                               _code(k_cache.dtype, "k_cache"), _ptr(sink), _stream(k_cache))
    _check_status(rc)


def mfma_rate(groups: int, rounds: int, sink: torch.Tensor):
    """Measurement helper: `groups` work-groups of 4 waves, each wave `rounds`
    rounds of 8 independent 16x16x32 fp16 MFMAs (16,384 flops each), no
    memory traffic.  `sink` is a 1-element int32 device tensor."""
    _dev(sink, "sink", dtype=torch.int32)
    _check_status(_load().pkv_mfma_rate(int(groups), int(rounds), _ptr(sink), _stream(sink)))


def lds_read_rate(pattern: int, groups: int, rounds: int, sink: torch.Tensor):
    """Measurement helper: the prefill kernel's LDS operand reads, 8 KiB per
    wave and round over `groups` work-groups of 8 waves (pattern 0: K reads on
    the K layout, 1: K reads on the V layout, 2: V^T transpose reads on the V
    layout, 3: transpose reads on the K layout)."""
    _dev(sink, "sink", dtype=torch.int32)
    _check_status(_load().pkv_lds_read_rate(int(pattern), int(groups), int(rounds), _ptr(sink),
                                            _stream(sink)))


def _host(x, name, dtype):
    """Pointer of a host buffer: a C-contiguous numpy array or CPU torch tensor
    (pinned or not) of the given numpy dtype."""
    import numpy as np
    if isinstance(x, torch.Tensor):
        if x.device.type != "cpu" or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous host tensor")
        if x.numpy().dtype != np.dtype(dtype):
            raise TypeError(f"{name} must be {np.dtype(dtype)}")
        return ctypes.c_void_p(x.data_ptr()), x.numel()
    if not isinstance(x, np.ndarray) or not x.flags.c_contiguous or x.dtype != np.dtype(dtype):
        raise TypeError(f"{name} must be a C-contiguous numpy {np.dtype(dtype)} array")
    return ctypes.c_void_p(x.ctypes.data), x.size


class BlockManager:
    """The pool's block allocator and per-sequence block tables, with prefix
    sharing (reference counts, copy-on-write of a shared partly filled last
    block).  Host-side; wraps the pkv_bm_* functions of libpkv."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        L = _load()
        h = ctypes.c_void_p()
        _check_status(L.pkv_bm_create(num_blocks, block_size, ctypes.byref(h)))
        self._L = L
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if getattr(self, "_h", None):
            self._L.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_sequence(self, seq_id: int):
        _check_status(self._L.pkv_bm_add_sequence(self._h, seq_id))

    def fork(self, parent_id: int, child_id: int):
        _check_status(self._L.pkv_bm_fork(self._h, parent_id, child_id))

    def free_sequence(self, seq_id: int):
        _check_status(self._L.pkv_bm_free_sequence(self._h, seq_id))

    def release_before(self, seq_id: int, position: int):
        """Release the whole blocks of seq_id that end at or before `position`
        (sliding-window decode); their table entries become -1."""
        _check_status(self._L.pkv_bm_release_before(self._h, seq_id, position))

    @property
    def num_free_blocks(self) -> int:
        return self._L.pkv_bm_num_free_blocks(self._h)

    def sequence_length(self, seq_id: int) -> int:
        return self._L.pkv_bm_sequence_length(self._h, seq_id)

    def append(self, seq_ids, num_tokens):
        """Room for num_tokens[i] new tokens at the end of seq_ids[i].  Returns
        (slot_mapping int64 [sum], copy_pairs int32 [n][2]) as numpy arrays;
        the copies must be made (copy_blocks) before the new tokens are
        written."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        cnt = np.ascontiguousarray(num_tokens, dtype=np.int32)
        if ids.ndim != 1 or cnt.shape != ids.shape:
            raise ValueError("seq_ids and num_tokens must be 1-D of one length")
        slots = np.empty(int(np.maximum(cnt, 0).sum()), dtype=np.int64)
        pairs = np.empty((len(ids), 2), dtype=np.int32)
        n = ctypes.c_int64(0)
        _check_status(self._L.pkv_bm_append(
            self._h, ctypes.c_void_p(ids.ctypes.data), ctypes.c_void_p(cnt.ctypes.data), len(ids),
            ctypes.c_void_p(slots.ctypes.data), ctypes.c_void_p(pairs.ctypes.data), len(ids),
            ctypes.byref(n)))
        return slots, pairs[:n.value]

    def block_tables(self, seq_ids, max_blocks_per_seq: int, out=None):
        """(block_tables int32 [B][max_blocks_per_seq], context_lens int32 [B]);
        `out` may give two host buffers (numpy or CPU torch, e.g. pinned) to
        fill instead of new numpy arrays."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        B = len(ids)
        if out is None:
            out = (np.empty((B, max_blocks_per_seq), dtype=np.int32), np.empty(B, dtype=np.int32))
        pt, nt = _host(out[0], "block_tables", np.int32)
        pl, nl = _host(out[1], "context_lens", np.int32)
        if nt < B * max_blocks_per_seq or nl < B:
            raise ValueError("output buffers too small")
        _check_status(self._L.pkv_bm_block_tables(self._h, ctypes.c_void_p(ids.ctypes.data), B,
                                                  max_blocks_per_seq, pt, pl))
        return out
