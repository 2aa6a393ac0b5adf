"""GPU parity of the page-table variants: block sizes 8 .. 256 and CSR page
tables (kv_indptr / kv_indices), for decode (matrix-core and vector kernels,
fixed partitions and the work-queue split), chunked prefill (bf16 and fp8),
quantising append, slot indexing / append / gather, and the CSR expansion.
Expected values come from the oracle, which walks any block size and takes
CSR rows as per-request page lists."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev, host_bits, note, oracle_decode, run_decode

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

LENS = [1, 8, 9, 17, 100, 257, 700, 2500, 5000]
# (kv kind, d, n_q, n_kv): the first two run on the matrix cores, the rest on the vector units
DECODE_KINDS = [("bf16", 128, 32, 8), ("fp8", 128, 64, 8), ("f32", 64, 8, 2), ("bf16", 64, 8, 4), ("fp8", 64, 8, 2)]


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


@pytest.mark.parametrize("B", [8, 32, 64, 256])
@pytest.mark.parametrize("kind,d,n_q,n_kv", DECODE_KINDS)
def test_decode_block_sizes(pkv, kind, d, n_q, n_kv, B):
    c = synth.make_decode_case(config=950, layer=B + d, n_q=n_q, n_kv=n_kv, d=d, seq_lens=LENS, kv_dtype=kind,
                               block_size=B)
    note(f"decode {kind} d={d} {n_q}q/{n_kv}kv B={B}")
    got = run_decode(pkv, c)
    want = oracle_decode(c)
    assert_parity(got, want, kind)


@pytest.mark.parametrize("B", [8, 64])
@pytest.mark.parametrize("kind,d,n_q,n_kv", [("f32", 64, 8, 2), ("bf16", 64, 8, 4), ("fp8", 64, 8, 2)])
def test_decode_queue_split_block_sizes(pkv, kind, d, n_q, n_kv, B):
    c = synth.make_decode_case(config=951, layer=B, n_q=n_q, n_kv=n_kv, d=d, seq_lens=LENS, kv_dtype=kind,
                               block_size=B)
    note(f"decode queue split {kind} d={d} B={B}")
    got = run_decode(pkv, c, partition_tokens=-1)
    want = oracle_decode(c)
    assert_parity(got, want, kind)


def _scatter(rows_per_seq, B, perm):
    """Pool [nb, n_kv, B, d] and table holding each sequence's rows in blocks
    of B taken in order from `perm`; unused slots hold NaN."""
    lens = [r.shape[0] for r in rows_per_seq]
    n_kv, d = rows_per_seq[0].shape[1:]
    need = [synth.blocks_for(L, B) for L in lens]
    nb = sum(need)
    pool = np.full((nb, n_kv, B, d), np.nan, dtype=np.float32)
    table = np.full((len(lens), max(need)), -1, dtype=np.int32)
    cur = 0
    for s, rows in enumerate(rows_per_seq):
        ids = perm[cur:cur + need[s]] % nb
        cur += need[s]
        table[s, :need[s]] = ids
        for p in range(rows.shape[0]):
            pool[ids[p // B], :, p % B, :] = rows[p]
    return pool, table


@pytest.mark.parametrize("kind,d,n_q,n_kv", [("bf16", 128, 32, 8), ("f32", 64, 8, 2)])
def test_decode_bits_do_not_depend_on_block_size(pkv, kind, d, n_q, n_kv):
    """The kernels work in 16-token tiles of two 8-token halves, so the same
    sequences laid out in blocks of 8, 16, 64 or 256 give the same bits (with
    the partition size fixed)."""
    r = synth.rng(952, 0, 0)
    lens = [3, 40, 300, 1500]
    rows = [r.standard_normal((L, 2 * n_kv, d)).astype(np.float32) for L in lens]
    q = r.standard_normal((len(lens), n_q, d)).astype(np.float32)
    outs = []
    for B in (8, 16, 64, 256):
        need = sum(synth.blocks_for(L, B) for L in lens)
        pool, table = _scatter(rows, B, r.permutation(need).astype(np.int32))
        k, v = pool[:, :n_kv], pool[:, n_kv:]
        k = synth.encode(np.ascontiguousarray(k), kind)
        v = synth.encode(np.ascontiguousarray(v), kind)
        qq = synth.encode(q, kind)
        out = pkv.paged_attn_decode(dev(qq, kind), dev(k, kind), dev(v, kind), dev(table),
                                    dev(np.array(lens, np.int32)), n_q, n_kv, d, B, synth.softmax_scale(d),
                                    partition_tokens=1024)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    note(f"decode {kind}: B = 8, 16, 64, 256 give the same bits")
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("B", [8, 32, 256])
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_prefill_block_sizes(pkv, kind, B):
    ctx = [0, 5, 16, 37, 300, 1000]
    ql = [7, 1, 33, 128, 200, 65]
    p = synth.make_prefill_case(config=953, layer=B, n_q=32, n_kv=8, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype=kind, block_size=B)
    note(f"prefill {kind} B={B}")
    q_lens = np.diff(p.cu_q_lens)
    out = pkv.paged_attn_prefill_chunk(
        dev(p.q, "bf16"), dev(p.cu_q_lens), dev(p.context_lens), int(q_lens.max()), dev(p.k_cache, kind),
        dev(p.v_cache, kind), dev(p.block_table), p.n_q, p.n_kv, p.d, B, p.scale, causal=True,
        k_scale=None if p.k_scale is None else dev(p.k_scale), v_scale=None if p.v_scale is None else dev(p.v_scale))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, kind, p.k_scale,
                                p.v_scale, p.block_table, p.n_q, p.n_kv, p.scale, causal=True)
    assert_parity(got, want, kind)


@pytest.mark.parametrize("B", [8, 64, 256])
def test_kv_append_fp8_block_sizes(pkv, B):
    r = synth.rng(954, B, 0)
    n_kv, d = 2, 128
    ctx = np.array([0, 1, 7, 8, 63, 64, 300], np.int32)
    n_new = np.array([1, 9, 1, 30, 2, 70, 5], np.int32)
    max_blocks = max(synth.blocks_for(int(c + n), B) for c, n in zip(ctx, n_new))
    nb = len(ctx) * max_blocks + 3
    table = r.permutation(nb)[:len(ctx) * max_blocks].astype(np.int32).reshape(len(ctx), max_blocks)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    total = int(cu[-1])
    mag = np.repeat(np.array([1, 2, 0.1, 5, 1, 0.5, 30], np.float32), n_new)[:, None, None]
    kb = synth.encode(r.standard_normal((total, n_kv, d)).astype(np.float32) * mag, "bf16")
    vb = synth.encode(r.standard_normal((total, n_kv, d)).astype(np.float32), "bf16")
    k = (r.integers(0, 0x7F, size=(nb, n_kv, B, d), dtype=np.uint8) | (r.integers(0, 2, size=(nb, n_kv, B, d),
                                                                                   dtype=np.uint8) << 7))
    v = k[::-1].copy()
    ks = (r.random((nb, n_kv)) * 0.02 + 1e-3).astype(np.float32)
    vs = ks[::-1].copy()
    tk, tv, tks, tvs = dev(k), dev(v), dev(ks), dev(vs)
    note(f"kv_append_fp8 B={B}")
    pkv.kv_append_fp8(tk, tv, tks, tvs, dev(table), dev(ctx), dev(cu), int(n_new.max()), dev(kb, "bf16"),
                      dev(vb, "bf16"))
    torch.cuda.synchronize()
    wk, wv, wks, wvs = oracle.kv_append_fp8(k, v, ks, vs, table, ctx, cu,
                                            oracle.bf16_bits_to_f64(kb).astype(np.float32),
                                            oracle.bf16_bits_to_f64(vb).astype(np.float32), B)
    assert np.array_equal(tk.cpu().numpy(), wk) and np.array_equal(tv.cpu().numpy(), wv)
    assert np.array_equal(tks.cpu().numpy().view(np.uint32), wks.view(np.uint32))
    assert np.array_equal(tvs.cpu().numpy().view(np.uint32), wvs.view(np.uint32))


@pytest.mark.parametrize("B", [8, 64])
def test_slot_append_gather_block_sizes(pkv, B):
    r = np.random.default_rng(955 + B)
    n_kv, d = 2, 64
    lens = [1, B - 1, B, B + 1, 3 * B + 5, 0]
    nb = sum(synth.blocks_for(L, B) for L in lens) + 2
    table, _ = synth.build_tables(lens, nb, r.permutation(nb).astype(np.int32), B)
    seq_ids = np.array([s for s, L in enumerate(lens) for _ in range(L)], dtype=np.int32)
    pos = np.array([p for L in lens for p in range(L)], dtype=np.int32)
    T = len(seq_ids)
    note(f"slot mapping, append, gather B={B}")
    slots = pkv.slot_mapping(dev(table), dev(seq_ids), dev(pos), B)
    want_slots = oracle.slot_mapping(table, seq_ids, pos, B)
    assert np.array_equal(slots.cpu().numpy(), want_slots)
    pool = np.full((nb, n_kv, B, d), np.nan, dtype=np.float32)
    kn = r.standard_normal((T, n_kv, d)).astype(np.float32)
    vn = r.standard_normal((T, n_kv, d)).astype(np.float32)
    kc, vc = dev(pool), dev(pool)
    pkv.kv_append(kc, vc, slots, dev(kn), dev(vn))
    want_k, want_v = oracle.kv_append(pool, pool.copy(), want_slots, kn, vn)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy().view(np.uint32), want_k.view(np.uint32))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    gk, gv = pkv.paged_gather(kc, vc, dev(table), dev(np.array(lens, np.int32)), dev(cu), T)
    torch.cuda.synchronize()
    assert np.array_equal(gk.cpu().numpy(), kn) and np.array_equal(gv.cpu().numpy(), vn)


def _csr_from_table(table, lens, B):
    pages = [table[s, :synth.blocks_for(int(L), B)] for s, L in enumerate(lens)]
    indptr = np.concatenate([[0], np.cumsum([len(p) for p in pages])]).astype(np.int32)
    indices = np.concatenate(pages).astype(np.int32) if indptr[-1] else np.zeros(0, np.int32)
    return indptr, indices


def test_csr_pages_example(pkv):
    """The pages' CSR table: kv_indptr [0, 2, 3, 6, 10] over 18 pages of 16
    tokens.  Decode through it matches the oracle walking the same pages, the
    expansion to a 2-D table is exact, and decode through the expanded table
    gives the same bits; prefill through it matches the oracle too."""
    g = json.load(open(os.path.join(GOLDEN, "csr_walk.json")))
    indptr = np.array(g["kv_indptr"], np.int32)
    indices = np.array(g["kv_indices"], np.int32)
    B, n_kv, n_q, d = 16, 2, 8, 128
    nb = int(indices.max()) + 1
    counts = np.diff(indptr)
    lens = np.array([c * B - 3 for c in counts], np.int32)  # every request ends inside its last page
    r = synth.rng(956, 0, 0)
    k = synth.encode(r.standard_normal((nb, n_kv, B, d)).astype(np.float32), "bf16")
    v = synth.encode(r.standard_normal((nb, n_kv, B, d)).astype(np.float32), "bf16")
    q = synth.encode(r.standard_normal((len(lens), n_q, d)).astype(np.float32), "bf16")
    rows = [oracle.csr_pages(indptr, indices, i) for i in range(len(lens))]
    scale = synth.softmax_scale(d)
    note("decode through the pages' CSR table")
    tk, tv = dev(k, "bf16"), dev(v, "bf16")
    got = pkv.paged_attn_decode_csr(dev(q, "bf16"), tk, tv, dev(indptr), dev(indices), int(counts.max()),
                                    dev(lens), n_q, n_kv, d, B, scale)
    table = pkv.csr_to_block_table(dev(indptr), dev(indices), int(counts.max()))
    via_table = pkv.paged_attn_decode(dev(q, "bf16"), tk, tv, table, dev(lens), n_q, n_kv, d, B, scale)
    torch.cuda.synchronize()
    want_table = np.full((len(lens), int(counts.max())), -1, np.int32)
    for i, pg in enumerate(rows):
        want_table[i, :len(pg)] = pg
    assert np.array_equal(table.cpu().numpy(), want_table)
    want = oracle.paged_decode(q, "bf16", k, v, "bf16", None, None, rows, lens, n_q, n_kv, scale)
    g64 = got.cpu().numpy().astype(np.float64)
    assert_parity(g64, want, "bf16")
    assert np.array_equal(got.cpu().numpy().view(np.uint32), via_table.cpu().numpy().view(np.uint32))
    # prefill: the last 5 tokens of each request are the chunk
    ql = np.minimum(5, lens).astype(np.int32)
    ctx = (lens - ql).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    qp = synth.encode(r.standard_normal((int(cu[-1]), n_q, d)).astype(np.float32), "bf16")
    out = pkv.paged_attn_prefill_chunk_csr(dev(qp, "bf16"), dev(cu), dev(ctx), int(ql.max()), tk, tv, dev(indptr),
                                           dev(indices), int(counts.max()), n_q, n_kv, d, B, scale)
    torch.cuda.synchronize()
    wantp = oracle.paged_prefill(qp, "bf16", cu, ctx, k, v, "bf16", None, None, rows, n_q, n_kv, scale, causal=True)
    gp = out.cpu().numpy().astype(np.float64)
    assert_parity(gp, wantp, "bf16")


@pytest.mark.parametrize("B", [8, 32])
def test_csr_random_fp8(pkv, B):
    """Random CSR tables over a shuffled pool (fp8 KV): decode and prefill
    match the oracle; requests with no pages decode to zeros."""
    c = synth.make_decode_case(config=957, layer=B, n_q=32, n_kv=8, d=128, seq_lens=[0] + LENS, kv_dtype="fp8",
                               block_size=B)
    indptr, indices = _csr_from_table(c.block_table, c.seq_lens, B)
    rows = [oracle.csr_pages(indptr, indices, i) for i in range(c.batch)]
    max_pages = int(np.diff(indptr).max())
    note(f"decode fp8 CSR B={B}")
    t = dict(q=dev(c.q, "bf16"), k=dev(c.k_cache), v=dev(c.v_cache), ks=dev(c.k_scale), vs=dev(c.v_scale))
    out = pkv.paged_attn_decode_csr(t["q"], t["k"], t["v"], dev(indptr), dev(indices), max_pages, dev(c.seq_lens),
                                    c.n_q, c.n_kv, c.d, B, c.scale, k_scale=t["ks"], v_scale=t["vs"])
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = oracle.paged_decode(c.q, "bf16", c.k_cache, c.v_cache, "fp8", c.k_scale, c.v_scale, rows, c.seq_lens,
                               c.n_q, c.n_kv, c.scale)
    assert_parity(got, want, "fp8")
    assert np.all(got[0] == 0)


def _stale_fp8(table, need, k_scale, v_scale):
    """Blocks no sequence uses get non-finite scales (NaN, +inf, -inf in
    turn: a free block's scale slot may hold anything), and every table entry
    past a sequence's last block names one of them, as a stale or reused table
    row would."""
    nb = k_scale.shape[0]
    unused = np.setdiff1d(np.arange(nb), table[table >= 0])
    assert unused.size > 0
    bad = np.array([np.nan, np.inf, -np.inf], np.float32)
    ks, vs = k_scale.copy(), v_scale.copy()
    ks[unused] = bad[np.arange(unused.size) % 3][:, None]
    vs[unused] = bad[(np.arange(unused.size) + 1) % 3][:, None]
    tb = table.copy()
    for s in range(tb.shape[0]):
        tail = tb.shape[1] - need[s]
        tb[s, need[s]:] = unused[np.arange(tail) % unused.size]
    return tb, ks, vs


@pytest.mark.parametrize("d,n_q,n_kv", [(128, 64, 8), (64, 8, 2)])
def test_fp8_decode_ignores_scales_past_the_sequence(pkv, d, n_q, n_kv):
    """With 8-token blocks a sequence whose length mod 16 is 1..8 ends on a
    16-token tile whose second half lies wholly past it; the kernels must not
    let that half's block scale (here non-finite, through a stale table entry)
    meet the zero weights of its masked keys."""
    B = 8
    lens = [1, 8, 17, 24, 100, 257, 2500, 5000]
    need = [synth.blocks_for(L, B) for L in lens]
    c = synth.make_decode_case(config=956, layer=d, n_q=n_q, n_kv=n_kv, d=d, seq_lens=lens, kv_dtype="fp8",
                               block_size=B, num_blocks=sum(need) + 7, max_blocks=max(need) + 3)
    tb, ks, vs = _stale_fp8(c.block_table, need, c.k_scale, c.v_scale)
    c = dataclasses.replace(c, block_table=tb, k_scale=ks, v_scale=vs)
    want = oracle_decode(c)
    for pt in ((0, 512, -1) if d == 64 else (0, 512)):
        note(f"fp8 decode d={d} B=8, non-finite scales behind stale entries, partition_tokens={pt}")
        got = run_decode(pkv, c, partition_tokens=pt)
        assert np.all(np.isfinite(got))
        assert_parity(got, want, "fp8")


@pytest.mark.parametrize("products", ["widened", "fp8"])
def test_fp8_prefill_ignores_scales_past_the_keys(pkv, products):
    B = 8
    ctx = [0, 3, 17, 40, 300]
    ql = [1, 5, 7, 33, 100]
    p = synth.make_prefill_case(config=957, layer=0, n_q=32, n_kv=8, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype="fp8", block_size=B,
                                num_blocks=sum(synth.blocks_for(c + q, B) for c, q in zip(ctx, ql)) + 7)
    need = [synth.blocks_for(c + q, B) for c, q in zip(ctx, ql)]
    tb, ks, vs = _stale_fp8(p.block_table, need, p.k_scale, p.v_scale)
    q_lens = np.diff(p.cu_q_lens)
    args = (dev(p.q, "bf16"), dev(p.cu_q_lens), dev(p.context_lens), int(q_lens.max()), dev(p.k_cache),
            dev(p.v_cache), dev(tb), p.n_q, p.n_kv, p.d, B, p.scale)
    kw = dict(causal=True, k_scale=dev(ks), v_scale=dev(vs))
    note(f"fp8 prefill ({products} products) B=8, non-finite scales behind stale entries")
    if products == "fp8":
        out = pkv.paged_attn_prefill_chunk_fp8_mma(*args, **kw)
    else:
        out = pkv.paged_attn_prefill_chunk(*args, **kw)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, "fp8", ks, vs, tb,
                                p.n_q, p.n_kv, p.scale, causal=True)
    assert np.all(np.isfinite(got))
    assert_parity(got, want, "fp8")
