"""FP8 E4M3FN quantisation on append.  (Oracle; test infrastructure only.)

The pages size FP8 KV caches at one byte per value ("KV cache, PagedAttention
and FlashAttention", Problem 3) and name quantising the cached keys and values
as a way to shrink the per-token cost ("Memory Management in LLM Serving
Systems", "Long-context optimization").  They fix neither the scale
granularity nor the rounding.  Here a (block, KV head) carries one fp32 scale,
the block's largest magnitude divided by 448 (the format's largest finite
value), and since the pages do not say what happens to that scale while a
block fills one token at a time, the reading used is:

  * a block's scale only grows: appending rows to a (block, KV head) sets
    scale = max(old scale, max |new values| / 448), the old scale counting
    only if the block already holds rows of this sequence;
  * when the scale grows, the block's existing codes are re-encoded against
    the new scale (value = code * old scale, then / new scale);
  * a new value x is stored as the code nearest to x / scale;
  * a block whose values are all zero keeps scale 0 and codes 0.

Every step that decides a code is done in float32, as the GPU does it: the
division by 448, code * old scale, and x / scale are float32 operations;
encoding picks the nearest E4M3FN value to that float32, ties to the code
with an even mantissa field, magnitudes above 448 saturating to 448 (OCP
8-bit floating point specification: round to nearest even; E4M3FN has no
infinities).
"""
import numpy as np

from .codecs import e4m3fn_to_f64

_F448 = np.float32(448.0)


def _finite_table():
    """Non-negative finite codes 0x00..0x7E and their values, ascending."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return codes, e4m3fn_to_f64(codes)


def encode_e4m3fn(x) -> np.ndarray:
    """Nearest E4M3FN code to each float (ties to an even mantissa field,
    saturating at +-448); the sign of the input is kept, zero included."""
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _finite_table()
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    mag = np.where(vals[hi] == a, codes[hi], mag)
    return np.where(np.signbit(x), mag | np.uint8(0x80), mag).astype(np.uint8)


def append_block_fp8(codes: np.ndarray, scale: np.float32, n_old: int, new_rows_f32: np.ndarray):
    """One (block, KV head) of an fp8 cache: codes [B, d] with rows [0, n_old)
    filled, its scale, and the float32 values of the rows appended after them
    ([n, d], n_old + n <= B).  Returns the new codes and scale."""
    codes = codes.copy()
    new_rows_f32 = np.asarray(new_rows_f32, dtype=np.float32)
    old = np.float32(scale) if n_old > 0 else np.float32(0.0)
    m = np.float32(np.max(np.abs(new_rows_f32))) if new_rows_f32.size else np.float32(0.0)
    new = np.maximum(old, np.float32(m / _F448))
    if new > old and n_old > 0:
        vals = e4m3fn_to_f64(codes[:n_old]).astype(np.float32) * old
        codes[:n_old] = encode_e4m3fn(vals / new)
    n = new_rows_f32.shape[0]
    if new > 0:
        codes[n_old:n_old + n] = encode_e4m3fn(new_rows_f32 / new)
    else:
        codes[n_old:n_old + n] = 0
    return codes, np.float32(new)


def kv_append_fp8(k_cache, v_cache, k_scale, v_scale, block_table, context_lens, cu_new, k_new_f32, v_new_f32,
                  block_size: int):
    """Append each sequence s's rows cu_new[s] .. cu_new[s+1] (float32 values,
    [total, n_kv, d]) at positions context_lens[s] onwards, block by block, with
    the grow-only scale rule.  Returns new caches and scales."""
    k, v = k_cache.copy(), v_cache.copy()
    ks, vs = k_scale.copy(), v_scale.copy()
    B = block_size
    n_kv = k.shape[1]
    for s in range(len(context_lens)):
        ctx, t0, t1 = int(context_lens[s]), int(cu_new[s]), int(cu_new[s + 1])
        n = t1 - t0
        if n <= 0:
            continue
        for j in range(ctx // B, (ctx + n - 1) // B + 1):
            blk = int(block_table[s][j])
            n_old = min(max(ctx - j * B, 0), B)
            lo = max(ctx, j * B) - ctx           # first new row (relative to t0) in block j
            hi = min(ctx + n, (j + 1) * B) - ctx
            for h in range(n_kv):
                k[blk, h], ks[blk, h] = append_block_fp8(k[blk, h], ks[blk, h], n_old, k_new_f32[t0 + lo:t0 + hi, h])
                v[blk, h], vs[blk, h] = append_block_fp8(v[blk, h], vs[blk, h], n_old, v_new_f32[t0 + lo:t0 + hi, h])
    return k, v, ks, vs
