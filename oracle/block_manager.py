"""Oracle of the paged-KV block manager (plain Python, CPU).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s
``cpu_baseline`` leg, never by the product package; it shares no code with
the native manager in ``libpkv``.

What a block manager must achieve, as the pages define it:

- every sequence's cache is cut into logical blocks of ``block_size`` tokens,
  physical blocks are taken from one global pool only when a sequence needs
  them, and a per-sequence table maps logical block j to a physical block
  ("Efficient AI Lecture 13" notes, section "PagedAttention", its four
  numbered steps; docs.lazyllm.ai lesson 4, section 4.2: per-request page
  table, global block pool with dynamic allocation and release);
- sequences continuing one prompt (parallel sampling, beam search) reuse the
  physical blocks of the prompt they share (lecture 13 notes, the advantages
  listed under "PagedAttention"; juejin "LLM Engineer's Handbook", section
  "optimized attention": memory sharing between outputs of one prompt).

This oracle models only the logical content.  A sequence is the list of the
ids of the tokens it holds, and every token written gets an id never used
before, so two sequences hold the same id at a position only if that token
reached both by sharing (a fork), never by a second write.  Physical sharing
then has a plain definition: logical block j of two sequences can be one
physical block exactly when the two id tuples of block j are equal (same
tokens, nobody wrote into the block after the fork).  The least number of
physical blocks any manager can use is the number of distinct
``(j, ids of block j)`` pairs over the live sequences; a manager that shares
what it may and copies a shared block only when a sequence writes into it
uses exactly that many.  ``blocks_in_use`` returns it.

A sequence that attends through a sliding window (only the most recent
window of its cache is kept: caojiahao2.github.io section 2.3, fixed memory)
may release its positions before some p: whole blocks that end at or before p
leave the physical count (the partly filled last block never does).

Pinned by ``tests/test_oracle_block_manager.py`` against closed forms:
independent sequences use sum(ceil(len / 16)) blocks; n samples of an
L-token prompt, t new tokens each, use floor(L / 16) + n * ceil((L mod 16 +
t) / 16) blocks (t >= 1, L mod 16 > 0); a fork without writes adds nothing;
freeing every sequence leaves nothing; a sequence of N tokens that released
everything before N - W holds ceil(N / 16) - floor((N - W) / 16) blocks.
"""
from __future__ import annotations

from typing import Dict, List


class SequenceSet:
    """Live sequences as lists of globally unique token ids."""

    def __init__(self, block_size: int = 16):
        self.block_size = block_size
        self.seqs: Dict[int, List[int]] = {}
        self.released: Dict[int, int] = {}   # whole blocks released at the front
        self._next_token = 0

    def add(self, seq: int) -> None:
        """A new, empty sequence."""
        if seq in self.seqs:
            raise KeyError(f"sequence {seq} exists")
        self.seqs[seq] = []
        self.released[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        """The child continues from everything the parent holds now."""
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        self.seqs[child] = list(self.seqs[parent])
        self.released[child] = self.released[parent]

    def release_before(self, seq: int, position: int) -> None:
        """Positions before `position` are no longer needed: every whole block
        that ends at or before it (and before the last token) is dropped."""
        full = len(self.seqs[seq]) // self.block_size
        drop = min(max(position, 0) // self.block_size, full)
        self.released[seq] = max(self.released[seq], drop)

    def append(self, seq: int, n: int) -> List[int]:
        """Write n new tokens at the end of seq; returns their ids."""
        ids = list(range(self._next_token, self._next_token + n))
        self._next_token += n
        self.seqs[seq].extend(ids)
        return ids

    def free(self, seq: int) -> None:
        del self.seqs[seq]
        del self.released[seq]

    def tokens(self, seq: int) -> List[int]:
        return self.seqs[seq]

    def blocks_of(self, seq: int) -> int:
        n = len(self.seqs[seq])
        return -(-n // self.block_size)

    def distinct_blocks(self) -> set:
        bs = self.block_size
        out = set()
        for seq, ids in self.seqs.items():
            for j in range(self.released[seq] * bs, len(ids), bs):
                out.add((j // bs, tuple(ids[j:j + bs])))
        return out

    def blocks_in_use(self) -> int:
        """Least number of physical blocks holding every live sequence."""
        return len(self.distinct_blocks())

    def blocks_without_sharing(self) -> int:
        return sum(self.blocks_of(s) - self.released[s] for s in self.seqs)

    def copy(self) -> "SequenceSet":
        c = SequenceSet(self.block_size)
        c.seqs = {k: list(v) for k, v in self.seqs.items()}
        c.released = dict(self.released)
        c._next_token = self._next_token
        return c
