"""Textbook softmax attention over a gathered paged cache.  (Oracle; test
infrastructure only.)

Definition followed:
  * "KV cache, PagedAttention and FlashAttention", Problem 5: S = Q K^T / sqrt(d),
    P = softmax(S), O = P V.  (The scale is an argument; the workloads pass
    1/sqrt(d_head) rounded to float32.)
  * "Memory Management in LLM Serving Systems", "FlashAttention": the
    numerically stable softmax subtracts the row max c before exponentiating;
    causally masked positions get -inf, i.e. they are left out.
  * "Memory Management in LLM Serving Systems", "MHA, MQA, and GQA", and
    "The KV Cache from First Principles", "Implementation": each KV head serves
    a group of G = n_q / n_kv consecutive query heads (repeat_interleave), so
    query head h reads KV head h // G; a head ratio that does not divide is an
    error raised before anything else happens.
  * "The KV Cache from First Principles", "The redundancy": the decode query
    at step t attends positions 1..t including itself, so ``seq_lens`` counts
    the token appended in the same step.
  * Paging changes where rows live, not the result ("KV cache, PagedAttention
    and FlashAttention", Problem 4): rows are gathered through the block table
    first, then attended as a contiguous sequence.

No tiling, no online softmax, no partitions: one softmax per query row over
all of its visible keys, in float64.
"""
import numpy as np

from .codecs import decode_storage
from .paging import gather_sequence, gather_scales


def _check_heads(n_q: int, n_kv: int) -> int:
    """Group size G = n_q / n_kv; every KV head must serve the same whole
    number (at least one) of query heads, checked before any data is read."""
    if n_kv < 1 or n_q < n_kv or n_q % n_kv != 0:
        raise ValueError(f"{n_q} query heads cannot be split evenly over {n_kv} KV heads")
    return n_q // n_kv


def softmax_attention_rows(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                           visible: np.ndarray) -> np.ndarray:
    """Attention for several query rows against one sequence's keys/values.

    q_rows [n, d], keys/values [L, d] (float64); visible[r] = number of leading
    keys query row r may see (keys 0 .. visible[r]-1).  A row that sees no key
    yields zeros.
    """
    out = np.zeros((q_rows.shape[0], values.shape[1]), dtype=np.float64)
    for r in range(q_rows.shape[0]):
        n = int(visible[r])
        if n <= 0:
            continue
        s = (keys[:n] @ q_rows[r]) * scale          # scores of row r
        c = np.max(s)                               # row max, for stability
        e = np.exp(s - c)
        w = e / np.sum(e)                           # softmax weights
        out[r] = w @ values[:n]                     # weighted sum of values
    return out


def _sequence_kv(k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, seq, length):
    """Gathered, decoded K and V of one sequence: [length, n_kv, d] float64."""
    block_size = k_cache.shape[2]
    K = decode_storage(gather_sequence(k_cache, block_table, seq, length), kv_dtype)
    V = decode_storage(gather_sequence(v_cache, block_table, seq, length), kv_dtype)
    if kv_dtype == "fp8":
        K = K * gather_scales(k_scale, block_table, seq, length, block_size).astype(np.float64)[:, :, None]
        V = V * gather_scales(v_scale, block_table, seq, length, block_size).astype(np.float64)[:, :, None]
    return K, V


def decode_one(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, seq_lens,
               n_q, n_kv, scale, seq, heads=None) -> np.ndarray:
    """Decode output of one sequence for the listed query heads: [len(heads), d]."""
    groups = _check_heads(n_q, n_kv)
    heads = list(range(n_q)) if heads is None else list(heads)
    L = int(seq_lens[seq])
    K, V = _sequence_kv(k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, seq, L)
    qs = decode_storage(q[seq], q_dtype)  # [n_q, d]
    out = np.zeros((len(heads), qs.shape[1]), dtype=np.float64)
    for i, h in enumerate(heads):
        kvh = h // groups
        out[i] = softmax_attention_rows(qs[h:h + 1], K[:, kvh, :], V[:, kvh, :], scale, np.array([L]))[0]
    return out


def paged_decode(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, seq_lens,
                 n_q, n_kv, scale) -> np.ndarray:
    """One decode query per sequence against its whole cached sequence.

    q [batch, n_q, d]; caches [num_blocks, n_kv, B, d]; returns [batch, n_q, d].
    """
    _check_heads(n_q, n_kv)
    batch = len(seq_lens)
    d = k_cache.shape[3]
    out = np.zeros((batch, n_q, d), dtype=np.float64)
    for s in range(batch):
        out[s] = decode_one(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table,
                            seq_lens, n_q, n_kv, scale, s)
    return out


def prefill_one(q, q_dtype, cu_q_lens, context_lens, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                block_table, n_q, n_kv, scale, seq, causal=True, rows=None, heads=None) -> np.ndarray:
    """Chunked-prefill output of one sequence: [n_rows, n_heads, d].

    Query i of the chunk sits at absolute position ctx + i.  With ``causal`` it
    sees keys 0 .. ctx + i; without, it sees the whole context plus the whole
    chunk.  The chunk's own rows must already be in the cache.
    """
    groups = _check_heads(n_q, n_kv)
    start, end = int(cu_q_lens[seq]), int(cu_q_lens[seq + 1])
    ctx, q_len = int(context_lens[seq]), end - start
    rows = list(range(q_len)) if rows is None else list(rows)
    heads = list(range(n_q)) if heads is None else list(heads)
    K, V = _sequence_kv(k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, seq, ctx + q_len)
    qs = decode_storage(q[start:end], q_dtype)  # [q_len, n_q, d]
    if causal:
        visible = np.array([ctx + i + 1 for i in rows])
    else:
        visible = np.full(len(rows), ctx + q_len)
    out = np.zeros((len(rows), len(heads), qs.shape[2]), dtype=np.float64)
    for j, h in enumerate(heads):
        kvh = h // groups
        out[:, j, :] = softmax_attention_rows(qs[rows, h, :], K[:, kvh, :], V[:, kvh, :], scale, visible)
    return out


def paged_prefill(q, q_dtype, cu_q_lens, context_lens, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                  block_table, n_q, n_kv, scale, causal=True) -> np.ndarray:
    """All chunk queries of all sequences: q packed [total_q, n_q, d] -> [total_q, n_q, d]."""
    _check_heads(n_q, n_kv)
    total_q, d = q.shape[0], k_cache.shape[3]
    out = np.zeros((total_q, n_q, d), dtype=np.float64)
    for s in range(len(context_lens)):
        a, b = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        if b > a:
            out[a:b] = prefill_one(q, q_dtype, cu_q_lens, context_lens, k_cache, v_cache, kv_dtype,
                                   k_scale, v_scale, block_table, n_q, n_kv, scale, s, causal)
    return out
