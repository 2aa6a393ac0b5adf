"""Block tables, slots, append and gather.  (Oracle; test infrastructure only.)

"KV cache, PagedAttention and FlashAttention", Problem 4 ("The idea"): the KV
pool is split into fixed-size blocks of B tokens; each sequence's block table
maps its logical block p // B to a physical block anywhere in the pool, and
the token sits at offset p % B inside it.  Waste per sequence is at most B - 1
tokens, because only the last block is partly filled.

"Memory Management in LLM Serving Systems", "Method 3: PagedAttention" and
"Walking the table": the same mapping stored as CSR arrays -- request i owns
pages kv_indices[kv_indptr[i]:kv_indptr[i+1]].

Storage layout (one layer): cache[num_blocks, n_kv, B, d]; a flat slot id is
physical_block * B + offset.
"""
import numpy as np


def slot_of(block_table: np.ndarray, seq: int, pos: int, block_size: int) -> int:
    """Flat slot of logical position ``pos`` of sequence ``seq``."""
    physical_block = int(block_table[seq][pos // block_size])
    offset = pos % block_size
    return physical_block * block_size + offset


def slot_mapping(block_table, seq_ids, positions, block_size: int) -> np.ndarray:
    """Slot of each (sequence, position) pair, as int64."""
    out = np.empty(len(seq_ids), dtype=np.int64)
    for t, (s, p) in enumerate(zip(seq_ids, positions)):
        out[t] = slot_of(block_table, int(s), int(p), block_size)
    return out


def kv_append(k_cache: np.ndarray, v_cache: np.ndarray, slots, k_new: np.ndarray, v_new: np.ndarray):
    """Copy each new token's K and V rows (all KV heads) into its slot, bit for bit.

    k_new, v_new: [num_tokens, n_kv, d] in the cache's storage dtype.  A slot
    below zero marks a padding token and is skipped.  Returns new arrays; the
    inputs are not modified.
    """
    k_out, v_out = k_cache.copy(), v_cache.copy()
    block_size = k_cache.shape[2]
    for t, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = slot // block_size, slot % block_size
        k_out[block, :, offset, :] = k_new[t]
        v_out[block, :, offset, :] = v_new[t]
    return k_out, v_out


def gather_sequence(cache: np.ndarray, block_table: np.ndarray, seq: int, seq_len: int) -> np.ndarray:
    """Walk one sequence's block table: returns its rows [seq_len, n_kv, d] in
    logical order, in the cache's storage dtype."""
    block_size = cache.shape[2]
    rows = []
    for p in range(seq_len):
        block = int(block_table[seq][p // block_size])
        rows.append(cache[block, :, p % block_size, :])
    if not rows:
        return np.zeros((0,) + (cache.shape[1], cache.shape[3]), dtype=cache.dtype)
    return np.stack(rows, axis=0)


def gather_scales(scales: np.ndarray, block_table: np.ndarray, seq: int, seq_len: int, block_size: int) -> np.ndarray:
    """Per-token copy of a per-(block, KV head) scale: [seq_len, n_kv]."""
    return np.stack([scales[int(block_table[seq][p // block_size])] for p in range(seq_len)], axis=0) \
        if seq_len else np.zeros((0, scales.shape[1]), dtype=scales.dtype)


def csr_pages(kv_indptr, kv_indices, request: int):
    """Pages owned by ``request`` in a CSR page table."""
    return list(kv_indices[kv_indptr[request]:kv_indptr[request + 1]])


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, bytes_per_value: int) -> int:
    """2 (K and V) x layers x KV heads x head dim x bytes per value."""
    return 2 * n_layers * n_kv_heads * d_head * bytes_per_value


def kv_bytes(n_layers, n_kv_heads, d_head, bytes_per_value, tokens, users=1) -> int:
    return kv_bytes_per_token(n_layers, n_kv_heads, d_head, bytes_per_value) * tokens * users


def waste_tokens(seq_len: int, block_size: int) -> int:
    """Slots allocated but unused for one sequence: blocks are handed out whole."""
    blocks = -(-seq_len // block_size)
    return blocks * block_size - seq_len
