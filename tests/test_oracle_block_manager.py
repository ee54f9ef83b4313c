"""Pins of the block-manager oracle (CPU only).

The oracle's ``blocks_in_use`` is the number of distinct (logical block,
token ids) pairs; these tests hold it to closed forms that follow from the
paging scheme alone (lecture 13 notes, section "PagedAttention"; lazyllm
lesson 4, section 4.2): independent sequences never share, n samples of one
prompt share the prompt's full blocks and nothing else, forks without writes
cost nothing, freeing returns everything.
"""
import math

import numpy as np
import pytest

from oracle.block_manager import SequenceSet

BS = 16


def test_independent_sequences_use_ceil_blocks():
    rng = np.random.default_rng(7)
    s = SequenceSet(BS)
    lens = rng.integers(0, 200, size=40)
    for i, n in enumerate(lens):
        s.add(i)
        s.append(i, int(n))
    assert s.blocks_in_use() == sum(math.ceil(int(n) / BS) for n in lens)
    assert s.blocks_in_use() == s.blocks_without_sharing()


@pytest.mark.parametrize("L", [1, 15, 16, 17, 100, 512, 1000])
@pytest.mark.parametrize("n", [1, 2, 4, 7])
@pytest.mark.parametrize("t", [0, 1, 5, 16, 33])
def test_parallel_sampling_closed_form(L, n, t):
    s = SequenceSet(BS)
    s.add(0)
    s.append(0, L)
    for c in range(1, n):
        s.fork(0, c)
    for c in range(n):
        s.append(c, t)
    r = L % BS
    if t == 0 or n == 1:
        expect = math.ceil((L + t) / BS) if n == 1 else math.ceil(L / BS)
    elif r == 0:
        expect = L // BS + n * math.ceil(t / BS)
    else:
        expect = L // BS + n * math.ceil((r + t) / BS)
    assert s.blocks_in_use() == expect
    assert s.blocks_without_sharing() == n * math.ceil((L + t) / BS)


def test_fork_without_writes_costs_nothing_and_free_returns_all():
    s = SequenceSet(BS)
    s.add(0)
    s.append(0, 37)
    before = s.blocks_in_use()
    for c in range(1, 6):
        s.fork(0, c)
    assert s.blocks_in_use() == before
    s.append(3, 1)                 # one writer into the shared partial block: one more block
    assert s.blocks_in_use() == before + 1
    s.free(0)
    assert s.blocks_in_use() == before + 1      # the other children still hold the original
    for c in range(1, 6):
        s.free(c)
    assert s.blocks_in_use() == 0


def test_every_writer_gets_its_own_tail_block():
    # A 20-token prompt (one full block + 4 tokens) forked into 3; all three write once:
    # 1 shared full block + 3 private second blocks (the last writer may keep the original).
    s = SequenceSet(BS)
    s.add(0)
    s.append(0, 20)
    s.fork(0, 1)
    s.fork(0, 2)
    for c in (1, 0, 2):
        s.append(c, 1)
    assert s.blocks_in_use() == 4
    # token ids of the shared prefix are the same objects in every sequence
    assert s.tokens(0)[:20] == s.tokens(1)[:20] == s.tokens(2)[:20]
    assert len({s.tokens(c)[20] for c in range(3)}) == 3


def test_nested_forks_beam_like():
    # A prompt of 32 tokens (2 full blocks); fork into 2; each writes 16 (a full block);
    # each forks again and the grandchildren write 3 tokens each.
    s = SequenceSet(BS)
    s.add(0)
    s.append(0, 32)
    s.fork(0, 1)
    s.append(0, 16)
    s.append(1, 16)
    s.fork(0, 2)
    s.fork(1, 3)
    for c in range(4):
        s.append(c, 3)
    # 2 prompt blocks + 2 generation blocks + 4 private partial blocks
    assert s.blocks_in_use() == 2 + 2 + 4
    assert s.blocks_without_sharing() == 4 * 4


@pytest.mark.parametrize("N,W", [(100, 16), (100, 37), (4096, 1024), (5000, 4096), (30, 64),
                                 (32, 16), (33, 1)])
def test_sliding_window_memory_is_fixed(N, W):
    s = SequenceSet(BS)
    s.add(0)
    peak = 0
    for t in range(1, N + 1):            # one token per step, releasing as it goes
        s.append(0, 1)
        s.release_before(0, t - W)
        peak = max(peak, s.blocks_in_use())
    assert s.blocks_in_use() == math.ceil(N / BS) - max(N - W, 0) // BS
    # a window of W tokens never needs more than ceil(W / 16) + 1 blocks
    assert peak <= math.ceil(W / BS) + 1


def test_release_keeps_shared_prefix_of_other_sequences():
    s = SequenceSet(BS)
    s.add(0)
    s.append(0, 64)                      # 4 full blocks
    s.fork(0, 1)
    s.release_before(0, 40)              # sequence 0 drops blocks 0, 1; sequence 1 keeps them
    assert s.blocks_in_use() == 4
    s.release_before(1, 48)              # sequence 1 drops 0..2; sequence 0 still holds 2
    assert s.blocks_in_use() == 2
    s.release_before(0, 63)              # block 3 (the last full one) is still needed
    assert s.blocks_in_use() == 1
    s.append(0, 1)
    s.append(1, 1)
    assert s.blocks_in_use() == 3
