"""Block sharing with reference counts and copy-on-write.  (Oracle; test
infrastructure only.)

"KV cache, PagedAttention and FlashAttention", Problem 4 ("The idea"):
because a sequence reaches its blocks through its block table, several
sequences can point at the same physical blocks -- parallel samples or
beam-search branches share the prompt's blocks -- and a reference count per
block tracks how many tables name it.  A block is allocated only when the
previous one fills.  Before a sequence writes into a block that another
sequence also names, the block is copied and the writer's table is pointed at
the copy (copy-on-write); the same mechanism serves prefix caching.  "Memory
Management in LLM Serving Systems", "Prefix sharing": a shared prefix is
stored once however many requests use it.

Readings where the pages are silent (listed in the design notes):
  * free blocks are handed out lowest id first, so a sequence of pool
    operations has one deterministic outcome;
  * appending n tokens to a sequence of length L touches its logical blocks
    L // B .. (L + n - 1) // B; a touched block that exists and is shared is
    copied (a new block is allocated before the old reference is dropped),
    a touched block that does not exist yet is allocated;
  * the pool checks that enough free blocks exist before changing anything.
"""
import numpy as np


class PoolExhausted(Exception):
    pass


class BlockPool:
    """Reference counts of num_blocks physical blocks; 0 means free."""

    def __init__(self, num_blocks: int):
        self.ref = [0] * int(num_blocks)

    def free_blocks(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def _lowest_free(self, n: int):
        out = [b for b, r in enumerate(self.ref) if r == 0][:n]
        if len(out) < n:
            raise PoolExhausted(f"{n} blocks wanted, {len(out)} free")
        return out

    def alloc(self, n: int):
        """n fresh blocks, each with one reference, lowest free ids first."""
        ids = self._lowest_free(n)
        for b in ids:
            self.ref[b] = 1
        return ids

    def share(self, ids):
        """One more table names each of ids (a fork)."""
        for b in ids:
            if self.ref[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
        for b in ids:
            self.ref[b] += 1

    def release(self, ids):
        """One table fewer names each of ids; a block with no reference left is free."""
        for b in ids:
            if self.ref[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
        for b in ids:
            self.ref[b] -= 1

    def prepare_append(self, row, seq_len: int, n_new: int, block_size: int):
        """Make the blocks that positions seq_len .. seq_len + n_new - 1 of one
        sequence fall into writable.  Returns (new row, [(src, dst), ...]):
        the row with fresh or copied blocks in place, and the block copies the
        cache needs (copy src into dst before writing)."""
        row = list(row)
        if n_new <= 0:
            return row, []
        have = -(-seq_len // block_size)                      # blocks the sequence owns
        first, last = seq_len // block_size, (seq_len + n_new - 1) // block_size
        shared = [j for j in range(first, min(last + 1, have)) if self.ref[row[j]] > 1]
        fresh = max(0, last + 1 - have)
        if len(shared) + fresh > self.free_blocks():
            raise PoolExhausted("not enough free blocks for the append")
        if last >= len(row):
            raise ValueError("block table row too short")
        copies = []
        for j in range(first, last + 1):
            if j < have:
                if self.ref[row[j]] > 1:
                    (new,) = self.alloc(1)
                    copies.append((row[j], new))
                    self.release([row[j]])
                    row[j] = new
            else:
                (row[j],) = self.alloc(1)
        return row, copies


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs, k_scale=None, v_scale=None):
    """Copy whole blocks (every KV head, every slot) src -> dst, bit for bit,
    for K, V and (fp8) their per-(block, KV head) scales.  Returns new arrays."""
    k, v = k_cache.copy(), v_cache.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    for src, dst in pairs:
        k[dst] = k_cache[src]
        v[dst] = v_cache[src]
        if ks is not None:
            ks[dst] = k_scale[src]
            vs[dst] = v_scale[src]
    return k, v, ks, vs
