"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

- libpkv.so loads and exports every function include/pkv.h declares;
- argument errors that the host can see return the documented status before
  anything is enqueued (these calls reach no HIP API);
- the Python binding refuses tensors that are not on a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")
LIB = os.path.join(ROOT, "paged_kv_cache_264_amd", "libpkv.so")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EHIP, ECAP, ESEQ = range(9)
F32, F16, BF16, I8, F8, U4 = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libpkv.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_status_string.restype = ctypes.c_char_p
    L.pkv_decode_workspace_size.restype = ctypes.c_size_t
    return L


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(\S+)", out))
    for n in names:
        assert n in exported, n
        getattr(lib, n)


def test_status_strings(lib):
    for s in range(9):
        assert lib.pkv_status_string(s) != b"unknown status"
    assert lib.pkv_status_string(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, ks=None, vs=None, bt=FAKE, mbs=8, cl=FAKE, B=2,
             Hq=8, Hkv=2, D=128, bs=16, NB=10, scale=0.1, P=0, ws=FAKE, wsb=1 << 30,
             qd=F16, cd=F16)
    a.update(kw)
    f = lib.pkv_paged_attn_decode
    f.argtypes = [P, P, P, P, P, P, P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_int, P,
                  ctypes.c_size_t, ctypes.c_int, ctypes.c_int, P]
    return f(a["out"], a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["mbs"], a["cl"],
             a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["scale"], a["P"], a["ws"],
             a["wsb"], a["qd"], a["cd"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), ESHAPE),
    (dict(Hkv=0), ESHAPE),
    (dict(B=-1), ESHAPE),
    (dict(D=96), EUNSUP),
    (dict(bs=32), EUNSUP),
    (dict(qd=F32, cd=F16), EDTYPE),
    (dict(qd=F32, cd=I8), EDTYPE),
    (dict(qd=I8, cd=I8), EDTYPE),
    (dict(q=None), ENULL),
    (dict(bt=None), ENULL),
    (dict(cd=I8), ENULL),                 # INT8 cache without scales
    (dict(cd=F8), ENULL),                 # FP8 cache without scales
    (dict(qd=F32, cd=F8), EDTYPE),
    (dict(qd=F8, cd=F8), EDTYPE),
    (dict(cd=6), EDTYPE),
    (dict(cd=U4), ENULL),                 # 4-bit cache without (min, range) arrays
    (dict(cd=U4, D=64, ks=FAKE, vs=FAKE), EUNSUP),
    (dict(qd=F32, cd=U4), EDTYPE),
    (dict(out=None), ENULL),
    (dict(P=24), ESHAPE),
    (dict(P=-16), ESHAPE),
    (dict(ws=None), EWS),
    (dict(wsb=100), EWS),
    (dict(q=ctypes.c_void_p(0x1004)), ESHAPE),   # misaligned
    # a 4-bit row's (x_min, range) pair is one 8-byte load
    (dict(cd=U4, ks=ctypes.c_void_p(0x1004), vs=FAKE), ESHAPE),
    (dict(cd=U4, ks=FAKE, vs=ctypes.c_void_p(0x100c)), ESHAPE),
])
def test_decode_argument_errors(lib, kw, status):
    assert decode(lib, **kw) == status
    assert lib.pkv_last_error()


def test_empty_batch_is_ok_without_launch(lib):
    assert decode(lib, B=0, out=None, q=None, bt=None, cl=None, ws=None) == OK


def test_workspace_size(lib):
    f = lib.pkv_decode_workspace_size
    f.argtypes = [ctypes.c_int] * 7
    assert f(64, 32, 32, 128, 256, 512, F16) > 64 * 32 * 8 * 128 * 4
    assert f(64, 32, 32, 96, 256, 512, F16) == 0
    assert f(64, 32, 32, 128, 256, 24, F16) == 0
    assert f(4, 8, 3, 64, 8, 0, F16) == 0
    assert f(64, 32, 32, 128, 256, 512, 9) == 0      # no such cache dtype
    # the default size's partials: a split batch needs room, one that is not
    # split needs none beyond the alignment
    assert f(1, 32, 8, 128, 2048, 0, BF16) > 8 * 32 * 128 * 4
    lib.pkv_default_partition_size.argtypes = [ctypes.c_int] * 5
    d = lib.pkv_default_partition_size
    for args in [(64, 32, 32, 256), (1, 32, 8, 2048), (16, 32, 32, 2048), (128, 32, 8, 512)]:
        for dt in (F32, F16, BF16, I8, F8, U4):
            p = d(*args, dt)
            assert p >= 256 and p % 16 == 0 and p & (p - 1) == 0
    assert d(64, 32, 32, 256, 9) == 0
    # about 1024 work-groups at the longest context for one-head tiles, 256
    # for tiles of several q heads (counted as launched: num_seqs x num_q_heads
    # / heads per tile); fewer than 1024 (sequence, kv head) items: at most
    # 4096 tokens
    assert d(16, 32, 32, 2048, F16) == 4096      # 512 items, 32k tokens
    assert d(2, 32, 32, 1024, F16) == 1024       # 64 items, 16k tokens
    assert d(64, 4, 4, 256, F16) == 1024         # 256 items, 4k tokens
    assert d(4, 32, 8, 2048, BF16) == 4096       # GQA: 32 items, 32k tokens
    assert d(1, 32, 8, 2048, BF16) == 1024       # GQA: 8 items, 32k tokens
    assert d(64, 32, 8, 256, BF16) == 4096       # GQA: 512 items, 4k tokens (cap)
    assert d(16, 32, 8, 256, F16) == 2048        # 4 heads per kv head, one 16-bit tile: 128 tiles
    assert d(16, 16, 8, 256, U4) == 2048         # 2 heads per kv head, one 4-bit tile: 128 tiles
    # >= 1024 items already fill the chip: up to 8192 tokens
    assert d(128, 32, 8, 512, BF16) == 8192      # the GQA batch: no sequence split
    assert d(64, 32, 32, 256, F16) == 8192       # 4096-token contexts stay whole
    assert d(256, 32, 8, 64, BF16) == 8192       # 2048 GQA items of at most 1024 tokens
    assert d(256, 32, 32, 4, F16) == 512         # 8192 items of at most 64 tokens
    assert d(1, 32, 32, 64, F16) == 1024         # one-head tiles of at most 1024 tokens: no split
    assert d(16, 32, 32, 64, I8) == 1024
    assert d(1, 32, 32, 256, F16) == 256         # 4096 tokens: split
    assert d(1, 32, 8, 64, BF16) == 256          # GQA tiles keep the rule
    # 8 to 63 q heads per kv head, 4 to 63 over a quantized cache (the matrix
    # cores; 16-bit q assumed for a quantized cache): the own rule over
    # (sequence, kv head, 16-row tile) items
    assert d(16, 32, 8, 256, I8) == 2048         # 4 per kv head: 128 row tiles, 4k tokens
    assert d(4, 32, 8, 1024, F8) == 2048         # 32 row tiles, 16k tokens
    assert d(64, 32, 4, 256, I8) == 4096         # 256 row tiles, 4k tokens
    assert d(32, 32, 2, 256, U4) == 1024         # 64 row tiles, 4k tokens
    assert d(64, 64, 8, 256, F8) == 4096         # 512 row tiles (cap)
    assert d(64, 32, 4, 256, F16) == 4096        # 256 row tiles, 4k tokens
    assert d(64, 64, 8, 256, BF16) == 4096       # 512 row tiles (cap)
    assert d(64, 32, 1, 256, BF16) == 2048       # 32 per kv head: 2 row tiles, 128 in all
    assert d(8, 64, 8, 1024, F16) == 4096        # 64 row tiles, 16k tokens
    assert d(16, 32, 2, 256, F16) == 512         # 32 row tiles, 4k tokens
    assert d(256, 64, 8, 256, BF16) == 8192      # 2048 row tiles (cap)
    m = lib.pkv_multi_default_partition_size
    m.argtypes = [ctypes.c_int] * 5
    # multi-query: about 512 work-groups at the longest context, 1024 once
    # the (sequence, row tile, kv head) items reach 1024
    assert m(8, 8, 32, 32, 256) == 2048     # 256 items, 4k tokens
    assert m(4, 4, 32, 8, 2048) == 2048     # GQA, 16 rows: 32 items, 32k tokens
    assert m(16, 8, 32, 8, 512) == 4096     # GQA, 32 rows: 256 items, 8k tokens
    assert m(64, 8, 32, 32, 256) == 8192    # the verify batch: 2048 items
    assert m(16, 512, 32, 32, 256) == 8192  # the prefill batch
    assert m(4, 0, 32, 8, 16) == 0 and m(4, 8, 32, 6, 16) == 0


def test_cache_write_argument_errors(lib):
    f = lib.pkv_kv_cache_write
    f.argtypes = [P, P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_int, ctypes.c_int, P]
    base = [FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 4, 2, 128, 16, 10, F16, F16, None]

    def call(i, val):
        a = list(base)
        a[i] = val
        return f(*a)

    assert call(7, -1) == ESHAPE            # num_tokens
    assert call(9, 80) == EUNSUP            # head_dim
    assert call(10, 8) == EUNSUP            # block_size
    assert call(13, BF16) == EDTYPE         # cache dtype != src and != I8
    assert call(12, I8) == EDTYPE           # src must be float
    assert call(12, F8) == EDTYPE
    assert call(13, F8) == ENULL            # FP8 without scales
    assert call(0, None) == ENULL
    assert call(13, I8) == ENULL            # INT8 without scales
    # 4-bit rows store (x_min, range) as one 8-byte word: scales must be
    # 8-byte aligned (the decode entry points ask the same)
    u4 = list(base)
    u4[13] = U4
    u4[4], u4[5] = ctypes.c_void_p(0x1004), FAKE
    assert f(*u4) == ESHAPE
    u4[4], u4[5] = FAKE, ctypes.c_void_p(0x100c)
    assert f(*u4) == ESHAPE
    u4[9] = 64                              # 4-bit rows need head_dim 128 or 256
    assert f(*u4) == EUNSUP
    assert call(7, 0) == OK                 # nothing to write: no launch


def test_reduce_argument_errors(lib):
    f = lib.pkv_paged_attn_reduce
    f.argtypes = [P, P, P, P, P] + [ctypes.c_int] * 7 + [P]
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 20, 4, 0, F16, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 100, 16, 4, 0, F16, None) == EUNSUP
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 16, 4, 0, I8, None) == EDTYPE
    assert f(None, FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 16, 4, 1, F16, None) == ENULL
    assert f(None, None, None, None, None, 0, 4, 128, 16, 4, 0, F16, None) == OK
    # o_part rows are read as 16-byte pieces: a misaligned pointer is refused
    # before anything is enqueued
    odd = ctypes.c_void_p(0x1004)
    assert f(FAKE, FAKE, FAKE, odd, FAKE, 2, 4, 128, 16, 4, 0, F16, None) == ESHAPE


def test_partials_argument_errors(lib):
    f = lib.pkv_paged_attn_decode_partials
    I = ctypes.c_int
    f.argtypes = [P, P, P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, ctypes.c_int64,
                  ctypes.c_float, I, I, I, I, P]
    base = [None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 8, FAKE, 2, 8, 2, 128,
            16, 10, 0.1, 64, 2, F16, F16, None]

    def call(i, val):
        a = list(base)
        a[i] = val
        return f(*a)

    assert call(19, 0) == ESHAPE            # partition size must be given
    assert call(19, 40) == ESHAPE           # not a multiple of 16
    assert call(20, 1) == ESHAPE            # num_partitions < ceil(8*16/64)
    assert call(1, None) == ENULL           # m_part
    assert call(0, ctypes.c_void_p(0x1008)) == ESHAPE   # misaligned out


def test_binding_rejects_host_tensors():
    import paged_kv_cache_264_amd as pkv
    q = torch.zeros((1, 4, 64))
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(q, torch.zeros((4, 4, 16, 64)), torch.zeros((4, 4, 16, 64)),
                              torch.zeros((1, 4), dtype=torch.int32),
                              torch.zeros((1,), dtype=torch.int32), 0.125)


def test_append_argument_errors(lib):
    f = lib.pkv_paged_attn_decode_append
    I = ctypes.c_int
    f.argtypes = [P, P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, ctypes.c_int64, ctypes.c_float,
                  I, P, ctypes.c_size_t, I, I, P]
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 8, FAKE, 2, 8, 2, 128, 16, 10,
            0.1, 0, FAKE, 1 << 30, F16, F16, None]

    def call(i, val):
        a = list(base)
        a[i] = val
        return f(*a)

    assert call(2, None) == ENULL           # k_new
    assert call(3, None) == ENULL           # v_new
    assert call(2, ctypes.c_void_p(0x1002)) == ESHAPE
    assert call(14, 96) == EUNSUP
    assert call(22, I8) == ENULL            # INT8 without scales
    assert call(11, 0) == OK                # empty batch


def test_copy_blocks_argument_errors(lib):
    f = lib.pkv_copy_blocks
    f.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_int, P]
    base = [FAKE, FAKE, None, None, FAKE, 3, 2, 128, 16, 10, F16, None]

    def call(i, val):
        a = list(base)
        a[i] = val
        return f(*a)

    assert call(5, -1) == ESHAPE            # num_pairs
    assert call(6, 0) == ESHAPE             # num_kv_heads
    assert call(7, 96) == EUNSUP            # head_dim
    assert call(8, 32) == EUNSUP            # block_size
    assert call(10, 9) == EDTYPE
    assert call(4, None) == ENULL           # copy_pairs
    assert call(10, I8) == ENULL            # INT8 without scales
    assert call(0, ctypes.c_void_p(0x1004)) == ESHAPE
    assert call(5, 0) == OK                 # nothing to copy: no launch


def test_block_manager_null_handle(lib):
    lib.pkv_bm_add_sequence.argtypes = [P, ctypes.c_int64]
    lib.pkv_bm_num_free_blocks.argtypes = [P]
    lib.pkv_bm_num_free_blocks.restype = ctypes.c_int64
    lib.pkv_bm_sequence_length.argtypes = [P, ctypes.c_int64]
    lib.pkv_bm_sequence_length.restype = ctypes.c_int64
    lib.pkv_bm_create.argtypes = [ctypes.c_int64, ctypes.c_int, P]
    assert lib.pkv_bm_add_sequence(None, 1) == ENULL
    assert lib.pkv_bm_num_free_blocks(None) == -1
    assert lib.pkv_bm_sequence_length(None, 1) == -1
    assert lib.pkv_bm_create(10, 16, None) == ENULL


def test_shared_prefix_argument_errors(lib):
    f = lib.pkv_paged_attn_decode_shared_prefix
    I = ctypes.c_int
    f.argtypes = [P, P, P, P, P, P, P, I, P, P, P, I, I, I, I, I, I, I, ctypes.c_int64,
                  ctypes.c_float, P, ctypes.c_size_t, I, I, P]
    # out q k_new v_new k v bt mbs cl prefix group_start G maxg B Hq Hkv D bs NB scale ws wsb qd cd
    base = [FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, 2, 4, 8, 8, 2, 128, 16,
            10, 0.1, FAKE, 1 << 30, F16, F16, None]

    def call(**kw):
        a = list(base)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return f(*a)

    assert call(a22=F32, a23=F32) == EDTYPE      # fp32: the prefix piece runs on MFMA (16-bit)
    assert call(a23=I8) == ENULL                 # INT8 cache (no scales taken): rejected
    assert call(a22=BF16, a23=F16) == EDTYPE
    assert call(a2=FAKE) == ENULL                # k_new without v_new
    assert call(a11=0) == ESHAPE                 # no groups for 8 sequences
    assert call(a11=9) == ESHAPE                 # more groups than sequences
    assert call(a12=0) == ESHAPE                 # max_group_size
    assert call(a9=None) == ENULL                # prefix_lens
    assert call(a10=None) == ENULL               # group_start
    assert call(a0=None) == ENULL                # out
    assert call(a21=100) == EWS
    assert call(a20=None) == EWS
    assert call(a20=ctypes.c_void_p(0x1010)) == EWS   # not 256-byte aligned
    assert call(a16=96) == EUNSUP
    assert call(a13=0, a0=None, a9=None, a10=None) == OK   # empty batch, no launch
    g = lib.pkv_shared_prefix_workspace_size
    g.argtypes = [I] * 7
    assert g(64, 16, 4, 32, 32, 128, 256) >= 2 * 64 * 32 * (128 + 2) * 4
    assert g(64, 16, 0, 32, 32, 128, 256) == 0
    assert g(64, 16, 4, 32, 32, 96, 256) == 0


def test_static_scratch_entry_refuses_oversized_partials(lib):
    """The no-allocation decode refuses, before any HIP call, a batch whose
    partials would not fit its static scratch (256 sequences x 32 heads x
    2048 partitions of 16 tokens: ~8.7 GB of partials)."""
    f = lib.pkv_paged_attn_decode_append_static
    I = ctypes.c_int
    f.argtypes = [P] * 9 + [I, P, I, I, I, I, I, ctypes.c_int64, ctypes.c_float, I, I, I, P]
    args = [FAKE] * 9 + [2048, FAKE, 256, 32, 32, 128, 16, 40000, 0.1, 16, F16, F16, None]
    assert f(*args) == EWS
    assert b"static scratch" in lib.pkv_last_error()
    args[14] = 96                              # head_dim checked first
    assert f(*args) == EUNSUP
    args[14] = 128
    args[2] = None                             # k_new required
    args[11] = 2
    assert f(*args) == ENULL
    args[11] = 0                               # no sequence: nothing to do
    assert f(*args) == OK


def test_read_helpers_argument_errors(lib):
    """The measurement helpers refuse what the host can see to be wrong,
    before any launch."""
    I, I64 = ctypes.c_int, ctypes.c_int64
    f = lib.pkv_stream_read
    f.argtypes = [P, I64, P, P]
    assert f(FAKE, -1, FAKE, None) == ESHAPE
    assert f(None, 64, FAKE, None) == ENULL
    assert f(ctypes.c_void_p(0x1004), 64, FAKE, None) == ESHAPE
    assert f(None, 0, None, None) == OK
    g = lib.pkv_tile_read
    g.argtypes = [P, P, P, I, P, I, P, I, I, I, I64, I, P, P]
    base = [FAKE, FAKE, FAKE, 8, FAKE, 2, FAKE, 4, 2, 128, 10, F16, FAKE, None]

    def call(i, val):
        a = list(base)
        a[i] = val
        return g(*a)

    assert call(9, 64) == EUNSUP            # 2 KiB tiles
    assert call(11, I8) == EUNSUP           # 1-byte codes at head_dim 128: 2 KiB tiles
    assert call(8, 0) == ESHAPE             # num_kv_heads
    assert call(6, None) == ENULL           # items
    assert call(6, ctypes.c_void_p(0x1004)) == ESHAPE
    assert call(7, 0) == OK                 # no item: no launch
    m = lib.pkv_mfma_rate
    m.argtypes = [I, I, P, P]
    assert m(0, 10, FAKE, None) == ESHAPE
    assert m(4, 0, FAKE, None) == ESHAPE
    assert m((1 << 20) + 1, 10, FAKE, None) == ESHAPE
    assert m(4, 10, None, None) == ENULL
    r = lib.pkv_lds_read_rate
    r.argtypes = [I, I, I, P, P]
    assert r(4, 4, 10, FAKE, None) == ESHAPE   # patterns are 0..3
    assert r(-1, 4, 10, FAKE, None) == ESHAPE
    assert r(0, 0, 10, FAKE, None) == ESHAPE
    assert r(2, 4, -3, FAKE, None) == ESHAPE
    assert r(1, 4, 10, None, None) == ENULL
