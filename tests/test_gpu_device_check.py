"""The opt-in device checks (pkv_set_device_checks): with checks on, calls on
valid device data give the same bits as without; calls whose lengths, table
entries or slots are invalid return PKV_ERR_DEVICE_CHECK and leave every
output and cache byte as it was (validate before mutate, "The KV Cache from
First Principles", Implementation).  The bad calls never reach the attention
or append kernels (the check fails first), and no bad call is made with the
checks off."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    yield p
    p.set_device_checks(False)


@pytest.fixture
def checks(pkv):
    pkv.set_device_checks(True)
    assert pkv.device_checks()
    yield pkv
    pkv.set_device_checks(False)


def _expect_check_failure(pkv, fn, what):
    with pytest.raises(pkv.PkvError) as e:
        fn()
    note(f"  {what}: {e.value}")
    assert e.value.status == pkv.ERR_DEVICE_CHECK


def _decode_inputs():
    c = synth.make_decode_case(config=990, layer=0, n_q=32, n_kv=8, d=128, seq_lens=[40, 300, 17], kv_dtype="bf16",
                               max_blocks=24)
    t = dict(q=dev(c.q, "bf16"), k=dev(c.k_cache, "bf16"), v=dev(c.v_cache, "bf16"))
    return c, t


def _decode(pkv, c, t, table, lens, out):
    return pkv.paged_attn_decode(t["q"], t["k"], t["v"], dev(table), dev(lens), c.n_q, c.n_kv, c.d, 16, c.scale,
                                 out=out)


def test_valid_data_same_bits(pkv):
    c, t = _decode_inputs()
    out0 = torch.empty((3, 32, 128), device="cuda")
    _decode(pkv, c, t, c.block_table, c.seq_lens, out0)
    pkv.set_device_checks(True)
    try:
        out1 = torch.empty_like(out0)
        _decode(pkv, c, t, c.block_table, c.seq_lens, out1)
    finally:
        pkv.set_device_checks(False)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int32), out1.view(torch.int32))


def test_decode_bad_tables_rejected(checks):
    pkv = checks
    c, t = _decode_inputs()
    nb = c.k_cache.shape[0]
    out = torch.full((3, 32, 128), 7.0, device="cuda")
    bad_id = c.block_table.copy()
    bad_id[1, 5] = nb                       # entry 5 of a 300-token sequence: used
    _expect_check_failure(pkv, lambda: _decode(pkv, c, t, bad_id, c.seq_lens, out), "block id = num_blocks")
    neg_id = c.block_table.copy()
    neg_id[0, 2] = -1                       # entry 2 of a 40-token sequence: used
    _expect_check_failure(pkv, lambda: _decode(pkv, c, t, neg_id, c.seq_lens, out), "block id -1 in use")
    long = c.seq_lens.copy()
    long[2] = 24 * 16 + 1                   # beyond the row's 24 entries
    _expect_check_failure(pkv, lambda: _decode(pkv, c, t, c.block_table, long, out), "seq_len > capacity")
    neg = c.seq_lens.copy()
    neg[0] = -3
    _expect_check_failure(pkv, lambda: _decode(pkv, c, t, c.block_table, neg, out), "negative seq_len")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "a rejected call must not write its output"
    # an unused entry (past the sequence's blocks) may hold anything
    spare = c.block_table.copy()
    spare[0, 20] = nb + 100
    _decode(pkv, c, t, spare, c.seq_lens, out)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))


def test_csr_offsets_rejected(checks):
    pkv = checks
    c, t = _decode_inputs()
    counts = [synth.blocks_for(int(L)) for L in c.seq_lens]
    indices = np.concatenate([c.block_table[s, :counts[s]] for s in range(3)]).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out = torch.full((3, 32, 128), 7.0, device="cuda")
    call = lambda ip: pkv.paged_attn_decode_csr(t["q"], t["k"], t["v"], dev(ip), dev(indices), 24, dev(c.seq_lens),
                                                32, 8, 128, 16, c.scale, out=out)
    bad = indptr.copy()
    bad[2] = bad[1] - 1                     # decreasing offsets
    _expect_check_failure(pkv, lambda: call(bad), "decreasing CSR offsets")
    short = indptr.copy()
    short[1] = 1                            # sequence 0 (40 tokens) given one page
    _expect_check_failure(pkv, lambda: call(short), "seq_len beyond the CSR row")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    call(indptr)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))


def test_append_bad_slot_rejected(checks):
    pkv = checks
    nb, n_kv, d = 6, 2, 64
    k_cache = torch.zeros((nb, n_kv, 16, d), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros_like(k_cache)
    k = torch.ones((3, n_kv, d), dtype=torch.bfloat16, device="cuda")
    slots = torch.tensor([0, nb * 16, -1], dtype=torch.int64, device="cuda")
    _expect_check_failure(pkv, lambda: pkv.kv_append(k_cache, v_cache, slots, k, k), "slot = num_blocks * B")
    torch.cuda.synchronize()
    assert not torch.any(k_cache.view(torch.int16)) and not torch.any(v_cache.view(torch.int16))
    ok = torch.tensor([0, nb * 16 - 1, -1], dtype=torch.int64, device="cuda")  # -1 is padding
    pkv.kv_append(k_cache, v_cache, ok, k, k)
    torch.cuda.synchronize()
    assert k_cache.view(torch.int16).flatten()[:d].eq(0x3F80).all()


def test_append_positions_bad_entry_rejected(checks):
    """The fused slot indexing + append: a table entry at or past the pool
    fails the check; pairs outside the table and negative entries are padding."""
    pkv = checks
    nb, n_kv, d = 6, 2, 64
    k_cache = torch.zeros((nb, n_kv, 16, d), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros_like(k_cache)
    k = torch.ones((4, n_kv, d), dtype=torch.bfloat16, device="cuda")
    table = dev(np.array([[0, nb], [-1, 5]], np.int32))
    seq = dev(np.array([0, 0, 1, 2], np.int32))
    pos = dev(np.array([3, 20, 4, 0], np.int32))  # (0, 20) -> entry nb: bad; (1, 4) -> -1; seq 2: padding
    _expect_check_failure(pkv, lambda: pkv.kv_append_positions(k_cache, v_cache, table, seq, pos, k, k),
                          "table entry = num_blocks")
    torch.cuda.synchronize()
    assert not torch.any(k_cache.view(torch.int16)) and not torch.any(v_cache.view(torch.int16))
    pos_ok = dev(np.array([3, 5, 4, 0], np.int32))
    pkv.kv_append_positions(k_cache, v_cache, table, seq, pos_ok, k, k)
    torch.cuda.synchronize()
    assert k_cache.view(torch.int16)[0, :, 3].eq(0x3F80).all() and k_cache.view(torch.int16)[0, :, 5].eq(0x3F80).all()
    assert int(torch.count_nonzero(k_cache.view(torch.int16))) == 2 * n_kv * d


def test_prefill_and_fp8_append_rejected(checks):
    pkv = checks
    p = synth.make_prefill_case(config=991, layer=0, n_q=32, n_kv=8, d=128, context_lens=[20, 50], q_len=[10, 30])
    cap = p.block_table.shape[1] * 16
    out = torch.full((40, 32, 128), 7.0, device="cuda")
    q, k, v, tb = dev(p.q, "bf16"), dev(p.k_cache, "bf16"), dev(p.v_cache, "bf16"), dev(p.block_table)
    call = lambda cu, ctx: pkv.paged_attn_prefill_chunk(q, dev(cu), dev(ctx), 30, k, v, tb, 32, 8, 128, 16, p.scale,
                                                        out=out)
    ctx_big = p.context_lens.copy()
    ctx_big[1] = cap                        # context + 30 new tokens beyond the row
    _expect_check_failure(pkv, lambda: call(p.cu_q_lens, ctx_big), "context + chunk > capacity")
    cu_bad = p.cu_q_lens.copy()
    cu_bad[2] = 39                          # last offset != total_q
    _expect_check_failure(pkv, lambda: call(cu_bad, p.context_lens), "cu_q_lens[-1] != total_q")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    call(p.cu_q_lens, p.context_lens)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
    # fp8 append with a negative context length
    nb = 8
    kc = torch.zeros((nb, 8, 16, 128), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.zeros((nb, 8), dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    table = dev(np.arange(nb, dtype=np.int32).reshape(2, 4))
    new = torch.ones((5, 8, 128), dtype=torch.bfloat16, device="cuda")
    cu = dev(np.array([0, 2, 5], np.int32))
    _expect_check_failure(pkv, lambda: pkv.kv_append_fp8(kc, vc, ks, vs, table, dev(np.array([-1, 0], np.int32)), cu,
                                                         3, new, new), "negative context length")
    torch.cuda.synchronize()
    assert not torch.any(kc) and not torch.any(ks)
    pkv.kv_append_fp8(kc, vc, ks, vs, table, dev(np.array([0, 0], np.int32)), cu, 3, new, new)
    torch.cuda.synchronize()
    assert torch.any(kc) and torch.all(ks[0] > 0)
