"""CPU oracle for attention over a paged KV cache -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy statement of what the paged-attention hot path
computes.  It exists to check the HIP library, and nothing in the product path
may import, call or execute it: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, tables or helpers); the only module both
sides use is ``synth`` (seeded input generation, no attention arithmetic).

Sources (three web pages):
  * "KV cache, PagedAttention and FlashAttention" -- Problem 3 (the per-token
    byte formula), Problem 4 (blocks, block table, logical->physical address),
    Problem 5 (textbook attention S = QK^T/sqrt(d), P = softmax(S), O = PV).
  * "Memory Management in LLM Serving Systems" -- "KV cache sizing",
    "MHA, MQA, and GQA", "Method 3: PagedAttention", "Walking the table",
    "FlashAttention" (numerically stable softmax, causal -inf mask).
    "Prefix sharing" (a shared prefix stored once); Problem 4 of the first
    page for block sharing with reference counts and copy-on-write, and for
    preemption by swapping blocks to CPU memory.
  * "The KV Cache from First Principles" -- "The redundancy" (the query
    attends positions 1..t including itself), "Implementation" (query head h
    uses KV head h // (n_q / n_kv); the head-ratio check runs before the cache
    is touched).

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, library routines and brute force on tiny inputs.
"""
from .codecs import bf16_bits_to_f64, e4m3fn_to_f64, f32_to_f64, decode_storage
from .paging import (slot_of, slot_mapping, kv_append, gather_sequence, csr_pages,
                     kv_bytes_per_token, kv_bytes, waste_tokens)
from .attention import (softmax_attention_rows, paged_decode, paged_prefill,
                        decode_one, prefill_one)
from .sharing import BlockPool, PoolExhausted, copy_blocks
from .quant import encode_e4m3fn, append_block_fp8, kv_append_fp8
from .swap import swap_image, swap_in

__all__ = [
    "bf16_bits_to_f64", "e4m3fn_to_f64", "f32_to_f64", "decode_storage",
    "slot_of", "slot_mapping", "kv_append", "gather_sequence", "csr_pages",
    "kv_bytes_per_token", "kv_bytes", "waste_tokens",
    "softmax_attention_rows", "paged_decode", "paged_prefill",
    "decode_one", "prefill_one",
    "BlockPool", "PoolExhausted", "copy_blocks",
    "encode_e4m3fn", "append_block_fp8", "kv_append_fp8",
    "swap_image", "swap_in",
]
