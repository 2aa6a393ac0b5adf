"""Pools whose addresses need more than 32 bits: blocks placed at the top of
a pool past 4 GiB of byte offsets (bf16, d 128: matrix-core decode, prefill,
gather) and past 2^31 rows (fp8, d 64, the smallest row: the vector-unit
decode, whose row indices are unsigned 32-bit).  A compact case is drawn as
usual and its blocks copied to the top of the large pool; the oracle runs on
the compact case, whose table differs only by the id offset."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev, host_bits, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def _lift(small: np.ndarray, kind: str, num_blocks: int, base: int, same=None) -> torch.Tensor:
    """A pool of num_blocks blocks (only blocks base .. base + len(small) - 1
    written) holding the compact pool's blocks there."""
    shape = (num_blocks,) + small.shape[1:]
    big = same if same is not None else torch.empty(shape, dtype=dev(small[:1], kind).dtype, device="cuda")
    big[base:base + small.shape[0]] = dev(small, kind)
    return big


def _lift_table(table: np.ndarray, base: int) -> np.ndarray:
    return np.where(table >= 0, table + base, table).astype(np.int32)


def test_bf16_past_4gib_offsets(pkv):
    torch.cuda.empty_cache()
    nb_big = (1 << 17) + 8192  # 4.56 GB per bf16 cache at 8 KV heads, 16 tokens, d 128
    lens = [1, 17, 300, 1000, 2500]
    c = synth.make_decode_case(config=980, layer=0, n_q=32, n_kv=8, d=128, seq_lens=lens, kv_dtype="bf16")
    base = nb_big - c.num_blocks
    note(f"bf16 pool of {nb_big} blocks, used blocks from id {base} (byte offsets past 4 GiB)")
    k, v = _lift(c.k_cache, "bf16", nb_big, base), _lift(c.v_cache, "bf16", nb_big, base)
    table = dev(_lift_table(c.block_table, base))
    for part in (0, 512):
        out = pkv.paged_attn_decode(dev(c.q, "bf16"), k, v, table, dev(c.seq_lens), c.n_q, c.n_kv, c.d, 16, c.scale,
                                    partition_tokens=part)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy().astype(np.float64), oracle.paged_decode(
            c.q, "bf16", c.k_cache, c.v_cache, "bf16", None, None, c.block_table, c.seq_lens, c.n_q, c.n_kv, c.scale),
            "bf16", f"decode, partitions {part}:")
    # gather walks the same rows
    cu = np.zeros(len(lens) + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    gk, _ = pkv.paged_gather(k, v, table, dev(c.seq_lens), dev(cu), int(cu[-1]))
    torch.cuda.synchronize()
    gk = host_bits(gk)
    for s, L in enumerate(lens):
        assert np.array_equal(gk[cu[s]:cu[s + 1]], oracle.gather_sequence(c.k_cache, c.block_table, s, L))
    del k, v
    # prefill over a large pool
    p = synth.make_prefill_case(config=981, layer=0, n_q=32, n_kv=8, d=128, context_lens=[0, 700, 2000],
                                q_len=[100, 33, 300])
    base = nb_big - p.k_cache.shape[0]
    k, v = _lift(p.k_cache, "bf16", nb_big, base), _lift(p.v_cache, "bf16", nb_big, base)
    ql = int(np.diff(p.cu_q_lens).max())
    out = pkv.paged_attn_prefill_chunk(dev(p.q, "bf16"), dev(p.cu_q_lens), dev(p.context_lens), ql, k, v,
                                       dev(_lift_table(p.block_table, base)), p.n_q, p.n_kv, p.d, 16, p.scale)
    torch.cuda.synchronize()
    want = oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, "bf16", None, None,
                                p.block_table, p.n_q, p.n_kv, p.scale, causal=True)
    assert_parity(out.cpu().numpy().astype(np.float64), want, "bf16", "prefill:")
    del k, v
    torch.cuda.empty_cache()


def test_fp8_rows_past_2_31(pkv):
    """fp8 at d 64 has 64-byte rows; 2^26 + 2^20 blocks of 2 KV heads x 16
    tokens put the used rows above 2^31 (the pool is 138 GB; K and V share it,
    so the oracle takes the same array for both)."""
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    nb_big = (1 << 26) + (1 << 20)
    need = nb_big * 2 * 16 * 64
    if free < need + (8 << 30):
        pytest.skip(f"needs {need / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    lens = [1, 16, 33, 700, 4000]
    c = synth.make_decode_case(config=982, layer=0, n_q=8, n_kv=2, d=64, seq_lens=lens, kv_dtype="fp8")
    base = nb_big - c.num_blocks
    rows0 = base * 2 * 16
    note(f"fp8 d=64 pool of {nb_big} blocks ({need / 1e9:.0f} GB), first used row {rows0} (> 2^31: {rows0 > 2**31})")
    assert rows0 > 2 ** 31
    kv = _lift(c.k_cache, "fp8", nb_big, base)
    ks = torch.ones(nb_big, 2, dtype=torch.float32, device="cuda")
    ks[base:base + c.num_blocks] = dev(c.k_scale)
    table = dev(_lift_table(c.block_table, base))
    want = oracle.paged_decode(c.q, "bf16", c.k_cache, c.k_cache, "fp8", c.k_scale, c.k_scale, c.block_table,
                               c.seq_lens, c.n_q, c.n_kv, c.scale)
    for part in (0, 1024, -1):
        out = pkv.paged_attn_decode(dev(c.q, "bf16"), kv, kv, table, dev(c.seq_lens), c.n_q, c.n_kv, c.d, 16, c.scale,
                                    k_scale=ks, v_scale=ks, partition_tokens=part)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy().astype(np.float64), want, "fp8", f"decode, partitions {part}:")
    del kv, ks
    torch.cuda.empty_cache()
