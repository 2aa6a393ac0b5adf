"""Preemption by swap: whole blocks moved to host memory and back.  (Oracle;
test infrastructure only.)

"KV cache, PagedAttention and FlashAttention", Problem 4 ("The idea" and
"Trade-offs"): when memory runs out the scheduler may preempt a sequence,
freeing its blocks and later either recomputing its prefix or swapping the
blocks to CPU memory and back (no recompute, at the cost of host-link
bandwidth and CPU memory).  Because the sequence reaches its blocks only
through its table, the blocks may come back anywhere in the pool.

Reading (the pages give no format): the host image of n swapped blocks is one
byte buffer laid out as
  [K of block 0 .. n-1][V of block 0 .. n-1][K scales][V scales]
where "K of block i" is the whole (every KV head, every slot) K slab of the
i-th listed block, and the scale sections (n x n_kv float32 each) exist only
for FP8 caches.  Swapping in writes the image's i-th block into the i-th
listed device block.
"""
import numpy as np


def _raw(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x).view(np.uint8)


def swap_image(k_cache: np.ndarray, v_cache: np.ndarray, ids, k_scale=None, v_scale=None) -> np.ndarray:
    """The host image of blocks `ids` (a uint8 array)."""
    parts = [_raw(k_cache[int(b)]).reshape(-1) for b in ids]
    parts += [_raw(v_cache[int(b)]).reshape(-1) for b in ids]
    if k_scale is not None:
        parts += [_raw(k_scale[int(b)]).reshape(-1) for b in ids]
        parts += [_raw(v_scale[int(b)]).reshape(-1) for b in ids]
    if not parts:
        return np.zeros(0, dtype=np.uint8)
    return np.concatenate(parts)


def swap_in(k_cache: np.ndarray, v_cache: np.ndarray, image: np.ndarray, ids, k_scale=None, v_scale=None):
    """Write the image's blocks into device blocks `ids`; returns new arrays."""
    k, v = k_cache.copy(), v_cache.copy()
    ks = None if k_scale is None else k_scale.copy()
    vs = None if v_scale is None else v_scale.copy()
    n = len(ids)
    kb = _raw(k_cache[0]).size          # bytes of one block's K (all heads)
    sb = 0 if k_scale is None else _raw(k_scale[0]).size
    off = 0
    for dst, arr, size in ((k, k_cache, kb), (v, v_cache, kb)):
        for i, b in enumerate(ids):
            chunk = image[off + i * size: off + (i + 1) * size]
            dst[int(b)] = chunk.view(arr.dtype).reshape(arr.shape[1:])
        off += n * size
    if ks is not None:
        for dst, arr in ((ks, k_scale), (vs, v_scale)):
            for i, b in enumerate(ids):
                chunk = image[off + i * sb: off + (i + 1) * sb]
                dst[int(b)] = chunk.view(arr.dtype).reshape(arr.shape[1:])
            off += n * sb
    return k, v, ks, vs
