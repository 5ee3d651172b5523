"""Oracle model of the block lifecycle (test infrastructure; see oracle/__init__.py).

Plain Python, written from the pages:

* "PagedAttention: Mathematical Foundations, ..." sec. 4, allocation lifecycle: a prompt
  of N tokens takes ceil(N/B) blocks from the free list; each decoding step appends the
  new token to the last block; when that block is full, one new block is taken from the
  free list and appended to the table; on completion every block loses a reference and
  blocks at zero return to the pool.
* same page, sec. 5, parallel sampling: K samples start from the prompt's blocks with
  reference count K; each writes its new tokens into private blocks; a sample that must
  write into a partially filled shared block copies it into a new block first, the
  shared block loses one reference, and the sample's table points at the copy.
* same page, sec. 7, fusion 3: all copies of one step are done by one batched copy.
* "Pytorch implementation of paper ..." sec. 3: blocks leave the free list from the front
  and return at its back.
* "PagedAttention: Mathematical Foundations, ..." sec. 6, preemption by swapping: the
  blocks of a preempted request are evicted to host RAM and brought back on resume.

Readings: a sequence's next token goes to slot len % B of logical block len // B; when
len % B == 0 that block does not exist yet (overflow: pop one block); otherwise, if the
last block's reference count exceeds 1, it is copied first (copy-on-write).  Appends in
one call are applied in the order given.  A call that would need more blocks than are
free changes nothing.  Swapping moves a gang of sequences (e.g. all samples of a request)
at once: each distinct block of the gang gets one slot on the other side (host slots
from their own FIFO list, ascending initially), in order of first appearance (gang order,
then table order); the old side loses the gang's references.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class _Seq:
    blocks: list
    length: int
    live: bool = True
    swapped: bool = False


@dataclass
class LifecycleOracle:
    num_blocks: int
    block_size: int
    free: list = field(default_factory=list)
    refs: list = field(default_factory=list)
    seqs: list = field(default_factory=list)

    host_free: list = field(default_factory=list)
    host_refs: list = field(default_factory=list)

    @classmethod
    def create(cls, num_blocks, block_size, free_order=None):
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        return cls(num_blocks, block_size, order, [0] * num_blocks, [])

    def host_pool(self, n):
        assert all(r == 0 for r in self.host_refs)
        self.host_free = list(range(n))
        self.host_refs = [0] * n

    def _move(self, handles, out):
        """Swap a gang out (device -> host) or in; returns the (old, new) id pairs or
        None when the other side has too few free ids (nothing changes)."""
        for h in handles:
            assert self.seqs[h].live and self.seqs[h].swapped == (not out)
        assert len(set(handles)) == len(handles)
        order = []
        for h in handles:
            for b in self.seqs[h].blocks:
                if b not in order:
                    order.append(b)
        from_refs, to_refs = (self.refs, self.host_refs) if out else (self.host_refs, self.refs)
        from_free, to_free = (self.free, self.host_free) if out else (self.host_free, self.free)
        if len(order) > len(to_free):
            return None
        new = {}
        for b in order:
            new[b] = to_free.pop(0)
            to_refs[new[b]] = 0
        for h in handles:
            seq = self.seqs[h]
            for j, b in enumerate(seq.blocks):
                from_refs[b] -= 1
                if from_refs[b] == 0:
                    from_free.append(b)
                to_refs[new[b]] += 1
                seq.blocks[j] = new[b]
            seq.swapped = out
        return [(b, new[b]) for b in order]

    def swap_out(self, handles):
        return self._move(list(handles), True)

    def swap_in(self, handles):
        return self._move(list(handles), False)

    # -- allocation of new sequences (same rule as the table builder of oracle.cpp)
    def alloc(self, context_lens, prefix_group=None, prefix_lens=None):
        B = self.block_size
        need = 0
        seen = set()
        for s, n in enumerate(context_lens):
            total = -(-int(n) // B)
            shared = 0
            if prefix_group is not None and prefix_group[s] >= 0:
                g = int(prefix_group[s])
                shared = int(prefix_lens[g]) // B
                if g not in seen:
                    need += shared
                    seen.add(g)
            need += total - shared
        if need > len(self.free):
            return None
        handles = []
        group_blocks = {}
        for s, n in enumerate(context_lens):
            total = -(-int(n) // B)
            blocks = []
            if prefix_group is not None and prefix_group[s] >= 0:
                g = int(prefix_group[s])
                if g not in group_blocks:
                    group_blocks[g] = [self.free.pop(0) for _ in range(int(prefix_lens[g]) // B)]
                blocks = list(group_blocks[g])
            while len(blocks) < total:
                blocks.append(self.free.pop(0))
            for b in blocks:
                self.refs[b] += 1
            self.seqs.append(_Seq(blocks, int(n)))
            handles.append(len(self.seqs) - 1)
        return handles

    def fork(self, parent, n):
        """n new sequences sharing every block of `parent` (parallel sampling)."""
        p = self.seqs[parent]
        assert p.live and not p.swapped
        out = []
        for _ in range(n):
            for b in p.blocks:
                self.refs[b] += 1
            self.seqs.append(_Seq(list(p.blocks), p.length))
            out.append(len(self.seqs) - 1)
        return out

    def append(self, handles):
        """Reserve the next token's slot of every handle, in order.  Returns
        (blocks, slots, copies) or None when the free list is too short (no change)."""
        B = self.block_size
        assert all(self.seqs[h].live and not self.seqs[h].swapped for h in handles)
        # dry run on copies of the counters
        refs = list(self.refs)
        lens = {h: self.seqs[h].length for h in handles}
        blocks = {h: list(self.seqs[h].blocks) for h in handles}
        need = 0
        for h in handles:
            n = lens[h]
            if n % B == 0:
                need += 1
                blocks[h].append(-1)
            else:
                last = blocks[h][n // B]
                if last >= 0 and refs[last] > 1:
                    need += 1
                    refs[last] -= 1
                    blocks[h][n // B] = -1
            lens[h] = n + 1
        if need > len(self.free):
            return None
        out_blocks, out_slots, copies = [], [], []
        for h in handles:
            seq = self.seqs[h]
            j, off = divmod(seq.length, B)
            if off == 0:
                nb = self.free.pop(0)
                self.refs[nb] = 1
                seq.blocks.append(nb)
            else:
                last = seq.blocks[j]
                if self.refs[last] > 1:
                    nb = self.free.pop(0)
                    self.refs[last] -= 1
                    self.refs[nb] = 1
                    copies.append((last, nb))
                    seq.blocks[j] = nb
            out_blocks.append(seq.blocks[j])
            out_slots.append(off)
            seq.length += 1
        return out_blocks, out_slots, copies

    def free_seqs(self, handles):
        for h in handles:
            seq = self.seqs[h]
            assert seq.live
            refs, free = (self.host_refs, self.host_free) if seq.swapped else (self.refs, self.free)
            for b in seq.blocks:
                refs[b] -= 1
                if refs[b] == 0:
                    free.append(b)
            seq.swapped = False
            seq.blocks = []
            seq.live = False

    def table(self, handles, max_blocks):
        t = np.full((len(handles), max_blocks), -1, np.int32)
        lens = np.zeros(len(handles), np.int32)
        for i, h in enumerate(handles):
            b = self.seqs[h].blocks
            t[i, : len(b)] = b
            lens[i] = self.seqs[h].length
        return t, lens


def copy_blocks(cache: np.ndarray, pairs):
    """The batched copy of one step: block dst receives block src, all KV heads."""
    for src, dst in pairs:
        cache[dst] = cache[src]
    return cache
