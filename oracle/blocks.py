"""A plain model of the paged cache's block management (test infrastructure only).

Follows the PagedAttention description on the survey page (section 3, core
principle): physical blocks are taken on demand, one whenever a sequence's
tokens reach a new 16-token page; a block shared by several sequences keeps a
reference count; a sequence that must write into a block others share first
gets its own copy (copy on write); blocks return to the free list when their
last reference goes.  Grants take the lowest free id, so runs are
deterministic.
"""
from __future__ import annotations

BLOCK = 16


class OutOfBlocks(Exception):
    pass


class BlockModel:
    def __init__(self, num_blocks: int):
        self.ref = [0] * num_blocks

    def free_ids(self):
        return [i for i, r in enumerate(self.ref) if r == 0]

    def alloc(self) -> int:
        free = self.free_ids()
        if not free:
            raise OutOfBlocks()
        self.ref[free[0]] = 1
        return free[0]

    def share(self, block: int):
        assert self.ref[block] > 0
        self.ref[block] += 1

    def release(self, block: int):
        assert self.ref[block] > 0
        self.ref[block] -= 1

    def plan_append(self, tables, ctx_lens, num_new):
        """tables: list of per-sequence lists of block ids (logical order);
        returns (slots, copies) and updates tables, ctx_lens and the counts.
        Raises OutOfBlocks (or ValueError) with nothing changed."""
        # dry run on copies: the same steps, so that a failure changes nothing
        saved = (list(self.ref), [list(t) for t in tables], list(ctx_lens))
        try:
            return self._apply(tables, ctx_lens, num_new)
        except (OutOfBlocks, ValueError):
            self.ref[:] = saved[0]
            for t, s in zip(tables, saved[1]):
                t[:] = s
            ctx_lens[:] = saved[2]
            raise

    def _apply(self, tables, ctx_lens, num_new):
        slots, copies = [], []
        for b, n in enumerate(num_new):
            c = ctx_lens[b]
            if n < 0:
                raise ValueError("negative length")
            if n == 0:
                continue
            table = tables[b]
            if c % BLOCK:                                  # partly filled last page
                page = table[c // BLOCK]
                if self.ref[page] > 1:                     # shared: copy on write
                    fresh = self.alloc()
                    copies.append((page, fresh))
                    self.release(page)
                    table[c // BLOCK] = fresh
            for p in range(c, c + n):
                if p % BLOCK == 0:                         # a new page starts
                    block = self.alloc()
                    if p // BLOCK < len(table):
                        table[p // BLOCK] = block
                    else:
                        table.append(block)
                slots.append(table[p // BLOCK] * BLOCK + p % BLOCK)
            ctx_lens[b] = c + n
        return slots, copies
