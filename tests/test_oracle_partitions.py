"""Pins of the oracle's partition boundaries (oracle.paged_partials).

A context of N tokens with partition size P is cut into ceil(N / P)
partitions of equal, block-aligned length span = 16 * ceil(ceil(N / count) /
16); partition p covers [p * span, min((p + 1) * span, N)).  The final output
does not depend on the split (the merge of running maxima and sums is exact:
caojiahao2.github.io section 3.2); only the exported phase-1 partials show
it.  The expected spans below are written out by hand, not computed by the
rule, and include the cases where the equal-length split differs from cutting
at multiples of P (N = 1040, P = 512: three partitions of 352 tokens, not
512 + 512 + 16).

How the spans are read back from the oracle: with q = 0 every score is 0, so
a partition's l is its token count and its o is the mean of its V rows; with
V row t filled with the value t, o = (t0 + t1 - 1) / 2.  Both boundaries
follow from (l, o).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

BS = 16

# (N, P) -> list of [t0, t1) spans, by hand
CASES = [
    ((1000, 512), [(0, 512), (512, 1000)]),
    ((1024, 512), [(0, 512), (512, 1024)]),                 # N = kP
    ((1025, 512), [(0, 352), (352, 704), (704, 1025)]),     # N = kP + 1
    ((1040, 512), [(0, 352), (352, 704), (704, 1040)]),     # not 512 + 512 + 16
    ((4100, 4096), [(0, 2064), (2064, 4100)]),
    ((5, 512), [(0, 5)]),                                   # N < 16
    ((15, 16), [(0, 15)]),
    ((16, 16), [(0, 16)]),
    ((17, 16), [(0, 16), (16, 17)]),
    ((33, 16), [(0, 16), (16, 32), (32, 33)]),
    ((100, 48), [(0, 48), (48, 96), (96, 100)]),
    ((130, 64), [(0, 48), (48, 96), (96, 130)]),
    ((1, 16), [(0, 1)]),
    ((0, 64), []),
]


def _spans_from_oracle(N: int, P: int, NP: int):
    D, Hq, Hkv = 64, 1, 1
    nblk = max(-(-N // BS), 1)
    # blocks placed in reverse order in the pool, so a wrong block index would
    # show up as a wrong position mean
    k = np.random.default_rng(N + P).standard_normal((nblk, Hkv, BS, D)).astype(np.float32)
    v = np.empty((nblk, Hkv, BS, D), np.float32)
    for j in range(nblk):
        phys = nblk - 1 - j
        for off in range(BS):
            v[phys, 0, off, :] = j * BS + off
    bt = np.array([[nblk - 1 - j for j in range(nblk)]], np.int32)
    q = np.zeros((1, Hq, D), np.float32)
    m, l, o = oracle.paged_partials(q, "f32", k, v, "f32", bt, np.array([N], np.int32), 0.125,
                                    P, NP)
    spans = []
    for p in range(NP):
        cnt = l[0, 0, p]
        if cnt == 0:
            continue
        assert m[0, 0, p] == 0.0
        assert np.all(o[0, 0, p] == o[0, 0, p, 0])
        t0 = (2 * o[0, 0, p, 0] + 1 - cnt) / 2
        spans.append((int(round(t0)), int(round(t0 + cnt))))
        assert abs(t0 - round(t0)) < 1e-9
    return spans, l[0, 0]


@pytest.mark.parametrize("np_extra", [0, 2])
@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0][0]}_P{c[0][1]}" for c in CASES])
def test_partition_spans(case, np_extra):
    (N, P), want = case
    NP = max(-(-N // P), 1) + np_extra      # extra partitions stay empty
    spans, l = _spans_from_oracle(N, P, NP)
    assert spans == want
    # partitions past the last hold no token
    assert np.all(l[len(want):] == 0)


def test_spans_are_block_aligned_and_equal():
    """Every partition but the last has the same length, a multiple of 16, and
    none is longer than P."""
    for (N, P), want in CASES:
        if len(want) < 2:
            continue
        lens = [t1 - t0 for t0, t1 in want]
        assert len(set(lens[:-1])) == 1 and lens[0] % BS == 0 and lens[0] <= P
        assert 0 < lens[-1] <= lens[0]
        assert len(want) == -(-N // P)
