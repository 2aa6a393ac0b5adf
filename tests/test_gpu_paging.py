"""GPU parity of slot indexing, append and gather: bit-exact against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, host_bits, note

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def test_slot_mapping_worked_example(pkv):
    g = json.load(open(os.path.join(GOLDEN, "csr_walk.json")))
    table = np.full((4, 4), -1, dtype=np.int32)
    for i, pages in enumerate(g["pages_by_request"]):
        table[i, :len(pages)] = pages
    toks = [int(t) for t in g["request2_slots"]]
    note(f"slot_mapping worked example, tokens {toks}")
    out = pkv.slot_mapping(dev(table), dev(np.full(len(toks), 2, np.int32)), dev(np.array(toks, np.int32)), 16)
    assert out.cpu().tolist() == list(g["request2_slots"].values())


def test_slot_mapping_random_and_invalid(pkv):
    r = np.random.default_rng(4)
    lens = r.integers(0, 300, size=37)
    nb = sum(synth.blocks_for(L) for L in lens) + 5
    table, _ = synth.build_tables(lens, nb, r.permutation(nb).astype(np.int32), 16, max_blocks=20)
    seq = r.integers(-2, 39, size=5000).astype(np.int32)
    pos = r.integers(-3, 330, size=5000).astype(np.int32)
    note("slot_mapping random 5000 pairs incl. invalid")
    got = pkv.slot_mapping(dev(table), dev(seq), dev(pos), 16).cpu().numpy()
    want = np.full(5000, -1, dtype=np.int64)
    for i, (s, p) in enumerate(zip(seq, pos)):
        if 0 <= s < 37 and 0 <= p < 20 * 16 and table[s, p // 16] >= 0:
            want[i] = oracle.slot_of(table, int(s), int(p), 16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind,d", [("bf16", 128), ("f32", 64), ("fp8", 128), ("bf16", 64), ("fp8", 64)])
def test_append_whole_pool_bit_exact(pkv, kind, d):
    r = np.random.default_rng(7)
    n_kv, B = 4, 16
    lens = [1, 16, 17, 40, 3]
    nb = 12
    table, _ = synth.build_tables(lens, nb, r.permutation(nb).astype(np.int32), B)
    dt = synth.STORAGE_DTYPE[kind]
    pool_k = r.integers(0, 256, size=(nb, n_kv, B, d * synth.ELEM_BYTES[kind]), dtype=np.uint8).view(dt)
    pool_v = r.integers(0, 256, size=pool_k.shape[:3] + (d * synth.ELEM_BYTES[kind],), dtype=np.uint8).view(dt)
    seq_ids = np.array([s for s, L in enumerate(lens) for _ in range(L)], dtype=np.int32)
    pos = np.array([p for L in lens for p in range(L)], dtype=np.int32)
    T = len(seq_ids)
    kn = r.integers(0, 256, size=(T, n_kv, d * synth.ELEM_BYTES[kind]), dtype=np.uint8).view(dt)
    vn = r.integers(0, 256, size=(T, n_kv, d * synth.ELEM_BYTES[kind]), dtype=np.uint8).view(dt)
    slots = oracle.slot_mapping(table, seq_ids, pos, B)
    slots[5] = -1  # a padding token
    want_k, want_v = oracle.kv_append(pool_k, pool_v, slots, kn, vn)
    note(f"append {kind} d={d} T={T}")
    kc, vc = dev(pool_k, kind), dev(pool_v, kind)
    pkv.kv_append(kc, vc, dev(slots), dev(kn, kind), dev(vn, kind))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kc).view(np.uint8), want_k.view(np.uint8))
    assert np.array_equal(host_bits(vc).view(np.uint8), want_v.view(np.uint8))


def test_append_empty_is_noop(pkv):
    kc = torch.zeros((2, 1, 16, 64), dtype=torch.bfloat16, device="cuda")
    pkv.kv_append(kc, kc.clone(), torch.zeros(0, dtype=torch.int64, device="cuda"),
                  torch.zeros((0, 1, 64), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((0, 1, 64), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert kc.abs().sum().item() == 0


@pytest.mark.parametrize("kind", ["bf16", "f32", "fp8"])
def test_gather_bit_exact(pkv, kind):
    c = synth.make_decode_case(config=200, layer=0, n_q=8, n_kv=2, d=128 if kind != "f32" else 64,
                               seq_lens=[0, 1, 15, 16, 17, 100, 257], kv_dtype=kind, num_blocks=40)
    cu = np.zeros(len(c.seq_lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(c.seq_lens)
    note(f"gather {kind}")
    gk, gv = pkv.paged_gather(dev(c.k_cache, kind), dev(c.v_cache, kind), dev(c.block_table), dev(c.seq_lens),
                              dev(cu), int(cu[-1]))
    torch.cuda.synchronize()
    gk, gv = host_bits(gk), host_bits(gv)
    for s, L in enumerate(c.seq_lens):
        wk = oracle.gather_sequence(c.k_cache, c.block_table, s, int(L))
        wv = oracle.gather_sequence(c.v_cache, c.block_table, s, int(L))
        assert np.array_equal(gk[cu[s]:cu[s + 1]].view(np.uint8), wk.view(np.uint8))
        assert np.array_equal(gv[cu[s]:cu[s + 1]].view(np.uint8), wv.view(np.uint8))


def test_check_tables_counts_bad_entries(pkv):
    table = np.array([[0, 1, -1], [2, 9, 3], [4, 5, 6]], dtype=np.int32)
    lens = np.array([20, 40, 49], dtype=np.int32)  # seq 1 uses block id 9 (>= 8); seq 2 is longer than 3 blocks
    note("check_tables")
    assert pkv.check_tables(dev(table), dev(lens), num_blocks=8) == 2
    assert pkv.check_tables(dev(table[:1]), dev(lens[:1]), num_blocks=8) == 0


@pytest.mark.parametrize("kind,d,B", [("bf16", 128, 16), ("f32", 64, 8), ("fp8", 128, 64), ("bf16", 64, 256)])
def test_append_positions_equals_slot_mapping_then_append(pkv, kind, d, B):
    """The fused slot indexing + append writes the pool the oracle's slot
    mapping + append writes, and the two-call path too, bit for bit; its slot
    output equals the slot mapping's, padding pairs included (ids and
    positions outside the table, negative entries, a table entry past the
    pool)."""
    r = np.random.default_rng(11 + B)
    n_kv = 4
    lens = [1, B, B + 1, 3 * B + 5, 7, 0]
    nb = sum(synth.blocks_for(L, B) for L in lens) + 3
    table, _ = synth.build_tables(lens, nb, r.permutation(nb).astype(np.int32), B)
    table[4, 0] = nb + 2  # an entry past the pool: its slot is computed, its rows are skipped
    dt = synth.STORAGE_DTYPE[kind]
    eb = synth.ELEM_BYTES[kind]
    pool_k = r.integers(0, 256, size=(nb, n_kv, B, d * eb), dtype=np.uint8).view(dt)
    pool_v = r.integers(0, 256, size=(nb, n_kv, B, d * eb), dtype=np.uint8).view(dt)
    seq_ids = [s for s, L in enumerate(lens) for _ in range(L)] + [-1, len(lens), 0, 2]
    pos = [p for L in lens for p in range(L)] + [0, 0, -1, table.shape[1] * B]
    seq_ids, pos = np.array(seq_ids, np.int32), np.array(pos, np.int32)
    T = len(seq_ids)
    kn = r.integers(0, 256, size=(T, n_kv, d * eb), dtype=np.uint8).view(dt)
    vn = r.integers(0, 256, size=(T, n_kv, d * eb), dtype=np.uint8).view(dt)
    slots = np.full(T, -1, np.int64)
    for i, (s, p) in enumerate(zip(seq_ids, pos)):
        if 0 <= s < len(lens) and 0 <= p < table.shape[1] * B and table[s, p // B] >= 0:
            slots[i] = oracle.slot_of(table, int(s), int(p), B)
    live = (slots >= 0) & (slots < nb * B)
    want_k, want_v = oracle.kv_append(pool_k, pool_v, np.where(live, slots, -1), kn, vn)
    note(f"append_positions {kind} d={d} B={B} T={T}")
    tt, ts, tp, tkn, tvn = dev(table), dev(seq_ids), dev(pos), dev(kn, kind), dev(vn, kind)
    kc, vc = dev(pool_k, kind), dev(pool_v, kind)
    out = torch.full((T,), 7, dtype=torch.int64, device="cuda")
    pkv.kv_append_positions(kc, vc, tt, ts, tp, tkn, tvn, slot_mapping_out=out)
    kc2, vc2 = dev(pool_k, kind), dev(pool_v, kind)
    s2 = pkv.slot_mapping(tt, ts, tp, B)
    pkv.kv_append(kc2, vc2, s2, tkn, tvn)
    kc3, vc3 = dev(pool_k, kind), dev(pool_v, kind)
    pkv.kv_append_positions(kc3, vc3, tt, ts, tp, tkn, tvn)  # no slot output
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), slots)
    assert np.array_equal(s2.cpu().numpy(), slots)
    for c, w in ((kc, want_k), (vc, want_v), (kc2, want_k), (vc2, want_v), (kc3, want_k), (vc3, want_v)):
        assert np.array_equal(host_bits(c).view(np.uint8), w.view(np.uint8))
