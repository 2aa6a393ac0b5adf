"""Seeded synthetic workloads for paged-KV attention.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It draws random numbers, encodes them into the storage formats the
caches use (fp32, bf16, OCP E4M3FN + per-(block, KV head) scale), builds block
pools and block tables, and poisons storage that must never be read.  It holds
none of the attention arithmetic: no gather, no softmax, no decoding of stored
values back to numbers.

Workload shapes follow the pages' model shapes (Llama3-8B: 32 query heads,
8 KV heads, head dim 128, "KV cache, PagedAttention and FlashAttention",
Problem 3; the 70B shape: 64 query heads, 8 KV heads) and their block size of
16 tokens ("commonly 16", same page, Problem 4 "The idea").

Seeding: every tensor is drawn from
``Generator(PCG64(SeedSequence([0, config, layer, tensor_id])))`` with
tensor_id 0 = q, 1 = k, 2 = v, 3 = block permutation, 4 = lengths,
5 = new K rows, 6 = new V rows.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_SIZE = 16

# storage codes for the three cache element types
F32, BF16, FP8 = "f32", "bf16", "fp8"
ELEM_BYTES = {F32: 4, BF16: 2, FP8: 1}
STORAGE_DTYPE = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}
# poison patterns for slots that must never influence a result
POISON = {F32: np.float32(np.nan), BF16: np.uint16(0x7FC0), FP8: np.uint8(0x7F)}

T_Q, T_K, T_V, T_PERM, T_LEN, T_KNEW, T_VNEW = range(7)


def rng(config: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, config, layer, tensor_id])))


# ---------------------------------------------------------------------------
# encoders (float32 -> storage bits)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bits, nearest-even; NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    nan = np.isnan(x)
    # finite inputs are <= 0xFF7FFFFF, so adding at most 0x8000 cannot wrap
    u = np.where(nan, np.uint32(0), x.view(np.uint32))
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    r = (u >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


_E4M3_MAX = 448.0


def f32_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    """Encode to OCP FP8 E4M3FN codes: round to nearest even, saturate to +-448.

    E4M3FN has exponent bias 7, 3 mantissa bits, no infinities, and uses
    S.1111.111 for NaN only, so the largest finite magnitude is 448 (OCP 8-bit
    floating point specification).  NaN inputs encode as 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8)
    a = np.abs(x)
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.minimum(a, _E4M3_MAX))
    # quantum: 2^(e-3) for normals (e >= -6), 2^-9 for subnormals
    _, e2 = np.frexp(a)  # a = f * 2^e2 with f in [0.5, 1)
    e = np.maximum(e2 - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    q = np.rint(a / quantum) * quantum  # np.rint rounds half to even
    q = np.minimum(q, _E4M3_MAX)
    # encode q exactly
    _, qe2 = np.frexp(q)
    qe = np.maximum(qe2 - 1, -6)
    is_sub = (q < 2.0 ** -6)
    exp_field = np.where(is_sub, 0, qe + 7)
    man = np.where(is_sub, np.rint(q / 2.0 ** -9), np.rint((q / np.ldexp(1.0, qe) - 1.0) * 8.0))
    code = (sign.astype(np.int64) << 7) | (exp_field.astype(np.int64) << 3) | man.astype(np.int64)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def encode(x_f32: np.ndarray, kind: str) -> np.ndarray:
    if kind == F32:
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    if kind == BF16:
        return f32_to_bf16_bits(x_f32)
    raise ValueError(kind)


def fp8_block_scales(x_f32: np.ndarray, filled: np.ndarray) -> np.ndarray:
    """Per-(block, KV head) scale = max |x| over the block's filled slots / 448.

    x_f32: [num_blocks, n_kv, B, d]; filled: bool [num_blocks, B].  A block
    whose max-abs is 0 (or that holds no filled slot) gets scale 1.0.
    """
    a = np.abs(x_f32).astype(np.float64)
    a = np.where(filled[:, None, :, None], a, 0.0)
    m = a.max(axis=(2, 3))
    s = np.where(m > 0, m / _E4M3_MAX, 1.0)
    return s.astype(np.float32)


def quantize_fp8(x_f32: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes = E4M3FN(x / scale[block, head]), the division done in float64."""
    return f32_to_e4m3fn(x_f32.astype(np.float64) / scales.astype(np.float64)[:, :, None, None])


# ---------------------------------------------------------------------------
# pools and block tables
# ---------------------------------------------------------------------------

def blocks_for(seq_len: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-int(seq_len) // block_size)


def build_tables(seq_lens, num_blocks: int, perm: np.ndarray, block_size: int = BLOCK_SIZE,
                 max_blocks: Optional[int] = None):
    """Sequences take consecutive chunks of a permuted pool, in order.

    Returns block_table int32 [batch, max_blocks] (unused entries -1) and a
    bool [num_blocks, B] map of filled slots.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    need = [blocks_for(L, block_size) for L in seq_lens]
    if max_blocks is None:
        max_blocks = max(max(need), 1)
    assert sum(need) <= num_blocks
    table = np.full((len(seq_lens), max_blocks), -1, dtype=np.int32)
    filled = np.zeros((num_blocks, block_size), dtype=bool)
    cur = 0
    for s, (L, nb) in enumerate(zip(seq_lens, need)):
        ids = perm[cur:cur + nb]
        cur += nb
        table[s, :nb] = ids
        for j, b in enumerate(ids):
            n = min(block_size, int(L) - j * block_size)
            filled[b, :n] = True
    return table, filled


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeCase:
    """One layer of paged decode inputs, in storage form (host arrays)."""
    n_q: int
    n_kv: int
    d: int
    block_size: int
    kv_dtype: str
    q_dtype: str
    q: np.ndarray            # [batch, n_q, d] float32 or bf16 bits
    k_cache: np.ndarray      # [num_blocks, n_kv, B, d] storage
    v_cache: np.ndarray
    k_scale: Optional[np.ndarray]  # fp32 [num_blocks, n_kv] (fp8 only)
    v_scale: Optional[np.ndarray]
    block_table: np.ndarray  # int32 [batch, max_blocks]
    seq_lens: np.ndarray     # int32 [batch]
    scale: float             # softmax scale, a float32 value

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])


@dataclasses.dataclass
class PrefillCase:
    """One layer of chunked-prefill inputs.

    ``k_cache``/``v_cache`` hold the cached context (positions < ctx) and, when
    ``chunk_in_cache`` is true, the chunk's own rows too.  ``k_new``/``v_new``
    hold the chunk's rows ([total_q, n_kv, d]) for appending, ``slots`` their
    flat slot ids, ``seq_ids``/``positions`` the (sequence, position) pairs.
    """
    n_q: int
    n_kv: int
    d: int
    block_size: int
    kv_dtype: str
    q_dtype: str
    q: np.ndarray            # [total_q, n_q, d]
    cu_q_lens: np.ndarray    # int32 [num_seqs + 1]
    context_lens: np.ndarray  # int32 [num_seqs]
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    seq_ids: np.ndarray      # int32 [total_q]
    positions: np.ndarray    # int32 [total_q]
    block_table: np.ndarray
    scale: float
    k_scale: Optional[np.ndarray] = None  # FP8: float32 [num_blocks, n_kv]
    v_scale: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])


def softmax_scale(d: int) -> float:
    """1/sqrt(d) computed in float64 and rounded to float32."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_decode_case(*, config: int, layer: int, n_q: int, n_kv: int, d: int, seq_lens,
                     kv_dtype: str = BF16, q_dtype: Optional[str] = None, num_blocks: Optional[int] = None,
                     block_size: int = BLOCK_SIZE, max_blocks: Optional[int] = None,
                     q_mult: float = 1.0, poison: bool = True) -> DecodeCase:
    """Draw one decode layer: Q, K, V i.i.d. N(0,1) float32, then encoded.

    The pool has ``num_blocks`` blocks (default: exactly the blocks the
    sequences need); sequences take consecutive chunks of a seeded
    permutation.  Unused blocks and the slots past each sequence's length are
    filled with the dtype's NaN pattern.
    """
    if q_dtype is None:
        q_dtype = F32 if kv_dtype == F32 else BF16
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    need = sum(blocks_for(L, block_size) for L in seq_lens)
    if num_blocks is None:
        num_blocks = max(need, 1)
    perm = rng(config, layer, T_PERM).permutation(num_blocks).astype(np.int32)
    table, filled = build_tables(seq_lens, num_blocks, perm, block_size, max_blocks)
    batch = len(seq_lens)
    qf = rng(config, layer, T_Q).standard_normal((batch, n_q, d), dtype=np.float32) * np.float32(q_mult)
    kf = rng(config, layer, T_K).standard_normal((num_blocks, n_kv, block_size, d), dtype=np.float32)
    vf = rng(config, layer, T_V).standard_normal((num_blocks, n_kv, block_size, d), dtype=np.float32)
    k_scale = v_scale = None
    if kv_dtype == FP8:
        k_scale = fp8_block_scales(kf, filled)
        v_scale = fp8_block_scales(vf, filled)
        kc = quantize_fp8(kf, k_scale)
        vc = quantize_fp8(vf, v_scale)
    else:
        kc = encode(kf, kv_dtype)
        vc = encode(vf, kv_dtype)
    if poison:
        mask = ~filled[:, None, :, None]
        mask = np.broadcast_to(mask, kc.shape)
        kc = np.where(mask, POISON[kv_dtype], kc)
        vc = np.where(mask, POISON[kv_dtype], vc)
    q = encode(qf, q_dtype)
    return DecodeCase(n_q=n_q, n_kv=n_kv, d=d, block_size=block_size, kv_dtype=kv_dtype, q_dtype=q_dtype,
                      q=q, k_cache=np.ascontiguousarray(kc), v_cache=np.ascontiguousarray(vc),
                      k_scale=k_scale, v_scale=v_scale, block_table=table, seq_lens=seq_lens,
                      scale=softmax_scale(d))


def make_prefill_case(*, config: int, layer: int, n_q: int, n_kv: int, d: int, context_lens, q_len,
                      kv_dtype: str = BF16, block_size: int = BLOCK_SIZE, chunk_in_cache: bool = True,
                      num_blocks: Optional[int] = None, poison: bool = True) -> PrefillCase:
    """Draw one chunked-prefill layer.

    Each sequence s holds ``context_lens[s]`` cached tokens and brings
    ``q_len[s]`` new query tokens at absolute positions ctx..ctx+q_len-1.  The
    pool holds exactly ceil((ctx + q_len)/B) blocks per sequence.
    """
    context_lens = np.asarray(context_lens, dtype=np.int32)
    q_len = np.broadcast_to(np.asarray(q_len, dtype=np.int32), context_lens.shape).copy()
    total_lens = context_lens + q_len
    need = sum(blocks_for(L, block_size) for L in total_lens)
    if num_blocks is None:
        num_blocks = max(need, 1)
    perm = rng(config, layer, T_PERM).permutation(num_blocks).astype(np.int32)
    table, filled_all = build_tables(total_lens, num_blocks, perm, block_size)
    # which slots hold context (positions < ctx) and which hold chunk rows
    ctx_mask = np.zeros((num_blocks, block_size), dtype=bool)
    seq_ids, positions, slots = [], [], []
    for s in range(len(context_lens)):
        for p in range(int(total_lens[s])):
            b = table[s, p // block_size]
            if p < context_lens[s]:
                ctx_mask[b, p % block_size] = True
            else:
                seq_ids.append(s)
                positions.append(p)
    seq_ids = np.asarray(seq_ids, dtype=np.int32)
    positions = np.asarray(positions, dtype=np.int32)
    cu = np.zeros(len(context_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_len)
    total_q = int(cu[-1])
    qf = rng(config, layer, T_Q).standard_normal((total_q, n_q, d), dtype=np.float32)
    kf = rng(config, layer, T_K).standard_normal((num_blocks, n_kv, block_size, d), dtype=np.float32)
    vf = rng(config, layer, T_V).standard_normal((num_blocks, n_kv, block_size, d), dtype=np.float32)
    # the chunk's new rows are the pool values at their slots
    blk = table[seq_ids, positions // block_size]
    off = positions % block_size
    keep = filled_all if chunk_in_cache else ctx_mask
    k_scale = v_scale = None
    if kv_dtype == FP8:
        # scales over every slot the sequences will hold (context and chunk),
        # so appending the chunk's codes leaves them valid
        k_scale = fp8_block_scales(kf, filled_all)
        v_scale = fp8_block_scales(vf, filled_all)
        kc, vc = quantize_fp8(kf, k_scale), quantize_fp8(vf, v_scale)
    else:
        kc, vc = encode(kf, kv_dtype), encode(vf, kv_dtype)
    k_new_rows, v_new_rows = kc[blk, :, off, :], vc[blk, :, off, :]
    if poison:
        mask = np.broadcast_to(~keep[:, None, :, None], kc.shape)
        kc = np.where(mask, POISON[kv_dtype], kc)
        vc = np.where(mask, POISON[kv_dtype], vc)
    return PrefillCase(n_q=n_q, n_kv=n_kv, d=d, block_size=block_size, kv_dtype=kv_dtype, q_dtype=BF16,
                       q=encode(qf, BF16), cu_q_lens=cu, context_lens=context_lens,
                       k_cache=np.ascontiguousarray(kc), v_cache=np.ascontiguousarray(vc),
                       k_new=np.ascontiguousarray(k_new_rows), v_new=np.ascontiguousarray(v_new_rows),
                       seq_ids=seq_ids, positions=positions, block_table=table, scale=softmax_scale(d),
                       k_scale=k_scale, v_scale=v_scale)


# ---------------------------------------------------------------------------
# the five workload configurations
# ---------------------------------------------------------------------------

def lognormal_lens(config: int, layer: int, batch: int, median: float = 1024.0,
                   sigma: float = math.sqrt(2.0 * math.log(2.0)), lo: int = 16, hi: int = 8192) -> np.ndarray:
    """Lengths rint(median * e^(sigma z)) clipped to [lo, hi]; sigma = sqrt(2 ln 2)
    puts the unclipped mean at 2 * median."""
    z = rng(config, layer, T_LEN).standard_normal(batch)
    return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int32)


# shape/length recipes; the length draw of configs 2, 4 and 5 is shared by all layers
CONFIGS = {
    1: dict(kind="decode", name="tiny paged decode fp32 (b2, 8q/2kv, d64)", n_q=8, n_kv=2, d=64,
            kv_dtype=F32, layers=1),
    2: dict(kind="decode", name="Llama3-8B-shaped decode bf16 (b64, 32q/8kv, d128, L~U[1024,2048])",
            n_q=32, n_kv=8, d=128, kv_dtype=BF16, layers=32),
    3: dict(kind="decode", name="70B-shaped long-context decode bf16 (b8, 64q/8kv, d128, L=32768)",
            n_q=64, n_kv=8, d=128, kv_dtype=BF16, layers=80),
    4: dict(kind="decode", name="70B-shaped fp8-E4M3 KV serving mix (b256, 64q/8kv, d128, log-normal L)",
            n_q=64, n_kv=8, d=128, kv_dtype=FP8, layers=16),
    5: dict(kind="prefill", name="chunked prefill bf16 (16 seqs x 512 new, ctx~U[0,8192], 32q/8kv, d128)",
            n_q=32, n_kv=8, d=128, kv_dtype=BF16, layers=1),
}


def config_seq_lens(config: int) -> np.ndarray:
    """Sequence lengths (decode) or context lengths (prefill) of a configuration."""
    if config == 1:
        return np.array([37, 100], dtype=np.int32)
    if config == 2:
        return rng(2, 0, T_LEN).integers(1024, 2049, size=64).astype(np.int32)
    if config == 3:
        return np.full(8, 32768, dtype=np.int32)
    if config == 4:
        return lognormal_lens(4, 0, 256)
    if config == 5:
        return rng(5, 0, T_LEN).integers(0, 8193, size=16).astype(np.int32)
    raise ValueError(config)


def config_decode_case(config: int, layer: int = 0, **overrides) -> DecodeCase:
    c = CONFIGS[config]
    assert c["kind"] == "decode"
    kw = dict(config=config, layer=layer, n_q=c["n_q"], n_kv=c["n_kv"], d=c["d"],
              seq_lens=config_seq_lens(config), kv_dtype=c["kv_dtype"])
    if config == 1:
        kw["num_blocks"] = 64
    kw.update(overrides)
    return make_decode_case(**kw)


def config_prefill_case(config: int = 5, layer: int = 0, q_len: int = 512, **overrides) -> PrefillCase:
    c = CONFIGS[config]
    kw = dict(config=config, layer=layer, n_q=c["n_q"], n_kv=c["n_kv"], d=c["d"],
              context_lens=config_seq_lens(config), q_len=q_len, kv_dtype=c["kv_dtype"])
    kw.update(overrides)
    return make_prefill_case(**kw)


# ---------------------------------------------------------------------------
# device-side fill for benchmark-sized pools (torch RNG, seeded)
# ---------------------------------------------------------------------------

def device_normal_(t, seed: int, chunk_elems: int = 1 << 27):
    """Fill a CUDA tensor (float32/bfloat16) with seeded N(0,1) values in chunks."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    flat = t.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        n = min(chunk_elems, flat.numel() - s)
        flat[s:s + n].copy_(torch.randn(n, generator=g, device=t.device, dtype=torch.float32))
    return t
