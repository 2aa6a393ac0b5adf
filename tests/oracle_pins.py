"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``check_*`` takes the oracle package as an argument so the same checks run
against the real oracle (``test_oracle_pins.py``) and against copies of it with
a planted mistake (``test_oracle_mutations.py``), which must each fail at least
one check.  Nothing here reuses the oracle's own code paths for the expected
value: expected values come from the pages (``tests/golden``), closed forms,
library routines (torch float64 scaled_dot_product_attention, torch's bf16 and
float8_e4m3fn casts) or independent scalar brute force.
"""
import json
import math
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


KiB, MiB, GiB = 2 ** 10, 2 ** 20, 2 ** 30


# ---------------------------------------------------------------------------
# sizing and paging
# ---------------------------------------------------------------------------

def check_sizing(orc):
    for c in _golden("sizing.json")["cases"]:
        L, n_kv, d = c["layers"], c["n_kv"], c["d_head"]
        if "values_per_token" in c:
            # values per token = bytes per token at one byte per value
            assert orc.kv_bytes_per_token(L, n_kv, d, 1) == c["values_per_token"], c["cite"]
            continue
        if "bits_per_value" in c:
            # a 4-bit value is half a byte: count nibbles, then halve
            nibbles = orc.kv_bytes_per_token(L, n_kv, d, 1) * c["bits_per_value"] // 4
            assert nibbles // 2 == c["kib_per_token"] * KiB, c["cite"]
            continue
        if "gib_by_bits" in c:
            for bits, gib in c["gib_by_bits"].items():
                b = orc.kv_bytes(L, n_kv, d, 1, c["tokens"], c["users"]) * int(bits) / 8
                assert b == gib * GiB, c["cite"]
                if "gb_1dp_by_bits" in c:
                    assert round(b / 1e9, 1) == c["gb_1dp_by_bits"][bits], c["cite"]
            continue
        b = c.get("bytes_per_value")
        per_tok = orc.kv_bytes_per_token(L, n_kv, d, b)
        if "bytes_per_token" in c:
            assert per_tok == c["bytes_per_token"], c["cite"]
        if "kib_per_token" in c:
            assert per_tok == c["kib_per_token"] * KiB, c["cite"]
        if "mib_per_token" in c:
            assert per_tok == c["mib_per_token"] * MiB, c["cite"]
        if "gib_total" in c:
            total = orc.kv_bytes(L, n_kv, d, b, c["tokens"], c.get("users", 1))
            assert total == c["gib_total"] * GiB, c["cite"]
        if "gb_total_approx" in c:
            total = orc.kv_bytes(L, n_kv, d, b, c["tokens"], c.get("users", 1))
            assert abs(total / 1e9 - c["gb_total_approx"]) < 1.0, c["cite"]
        if "mib_total" in c:
            assert orc.kv_bytes(L, n_kv, d, b, c["tokens"]) == c["mib_total"] * MiB, c["cite"]
        if "kib_total" in c:
            assert orc.kv_bytes(L, n_kv, d, b, c["tokens"]) == c["kib_total"] * KiB, c["cite"]
        if "kilo_tokens" in c:
            assert c["budget_gib"] * GiB // per_tok == c["kilo_tokens"] * 1024, c["cite"]
        if "gb_approx" in c:
            total = orc.kv_bytes(L, n_kv, d, b, c["tokens"], c["users"])
            assert round(total / 1e9, 2 if c["gb_approx"] < 10 else 1) == c["gb_approx"], c["cite"]


def check_csr_walk(orc):
    g = _golden("csr_walk.json")
    B = g["block_size"]
    for i, pages in enumerate(g["pages_by_request"]):
        assert [int(p) for p in orc.csr_pages(g["kv_indptr"], g["kv_indices"], i)] == pages
    table = np.full((4, 4), -1, dtype=np.int32)
    for i, pages in enumerate(g["pages_by_request"]):
        table[i, :len(pages)] = pages
    for tok, slot in g["request2_slots"].items():
        assert orc.slot_of(table, 2, int(tok), B) == slot, tok
    toks = [int(t) for t in g["request2_slots"]]
    got = orc.slot_mapping(table, [2] * len(toks), toks, B)
    assert got.dtype == np.int64
    assert list(got) == list(g["request2_slots"].values())
    for rng_str, page in g["request2_token_ranges"].items():
        lo, hi = map(int, rng_str.split("-"))
        assert {orc.slot_of(table, 2, p, B) // B for p in range(lo, hi + 1)} == {page}


def check_waste(orc):
    """At most B-1 wasted slots per sequence; over a full period of lengths the
    mean waste is (B-1)/2 ("about B/2")."""
    for B in (1, 8, 16, 64):
        ws = [orc.waste_tokens(L, B) for L in range(1, 4 * B + 1)]
        assert max(ws) == B - 1 and min(ws) == 0
        assert sum(ws[:B]) * 2 == B * (B - 1)
        assert all((L + w) % B == 0 for L, w in zip(range(1, 4 * B + 1), ws))


def check_append_gather(orc):
    """Append every token of three sequences through the slot mapping, then walk
    the tables: each row comes back bit-exact, in logical order, and slots not
    targeted keep their old bytes; a slot of -1 writes nothing."""
    r = np.random.default_rng(5)
    B, n_kv, d, num_blocks = 4, 2, 3, 12
    lens = [5, 1, 9]
    perm = r.permutation(num_blocks).astype(np.int32)
    table, _ = synth.build_tables(lens, num_blocks, perm, B)
    kc = r.integers(0, 2 ** 16, size=(num_blocks, n_kv, B, d)).astype(np.uint16)
    vc = r.integers(0, 2 ** 16, size=(num_blocks, n_kv, B, d)).astype(np.uint16)
    seq_ids = [s for s, L in enumerate(lens) for _ in range(L)]
    pos = [p for L in lens for p in range(L)]
    T = len(seq_ids)
    kn = r.integers(0, 2 ** 16, size=(T + 1, n_kv, d)).astype(np.uint16)
    vn = r.integers(0, 2 ** 16, size=(T + 1, n_kv, d)).astype(np.uint16)
    slots = list(orc.slot_mapping(table, seq_ids, pos, B)) + [-1]
    assert len(set(slots[:-1])) == T, "slots must be distinct"
    k2, v2 = orc.kv_append(kc, vc, slots, kn, vn)
    touched = np.zeros((num_blocks, B), dtype=bool)
    for s in slots[:-1]:
        touched[s // B, s % B] = True
    keep = np.broadcast_to(~touched[:, None, :, None], kc.shape)
    assert np.array_equal(k2[keep], kc[keep]) and np.array_equal(v2[keep], vc[keep])
    t = 0
    for s, L in enumerate(lens):
        gk = orc.gather_sequence(k2, table, s, L)
        gv = orc.gather_sequence(v2, table, s, L)
        assert gk.shape == (L, n_kv, d)
        assert np.array_equal(gk, kn[t:t + L]) and np.array_equal(gv, vn[t:t + L])
        t += L
    # the physical block of each position is the table entry (pages' address rule)
    for s, L in enumerate(lens):
        for p in range(L):
            assert orc.slot_of(table, s, p, B) // B == table[s, p // B]
            assert orc.slot_of(table, s, p, B) % B == p - (p // B) * B


# ---------------------------------------------------------------------------
# codecs
# ---------------------------------------------------------------------------

def check_e4m3(orc):
    g = _golden("e4m3fn_anchors.json")
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.e4m3fn_to_f64(codes)
    for code, v in g["anchors"].items():
        got = vals[int(code, 16)]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), code
    for code in g["nan_codes"]:
        assert np.isnan(vals[int(code, 16)])
    # library cross-check: torch's float8_e4m3fn cast, all 256 codes
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(vals)
    assert np.all(both_nan | (ref == vals))
    # positive finite codes are strictly increasing; negatives mirror them
    assert np.all(np.diff(vals[:127]) > 0)
    assert np.array_equal(vals[128:255], -vals[:127])


def check_bf16(orc):
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0]
    got = orc.bf16_bits_to_f64(bits)
    assert list(got) == want
    r = np.random.default_rng(3).integers(0, 2 ** 16, size=4096).astype(np.uint16)
    r = r[(r & 0x7F80) != 0x7F80]  # drop inf/NaN patterns
    ref = torch.from_numpy(r.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_bits_to_f64(r), ref)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _decode_case(**kw):
    return synth.make_decode_case(**kw)


def _run_decode(orc, c, **over):
    args = dict(q=c.q, q_dtype=c.q_dtype, k_cache=c.k_cache, v_cache=c.v_cache, kv_dtype=c.kv_dtype,
                k_scale=c.k_scale, v_scale=c.v_scale, block_table=c.block_table, seq_lens=c.seq_lens,
                n_q=c.n_q, n_kv=c.n_kv, scale=c.scale)
    args.update(over)
    return orc.paged_decode(**args)


def _contiguous_kv(c):
    """Gather with plain fancy indexing (independent of the oracle's walk)."""
    out = []
    dec = {"f32": lambda x: x.astype(np.float64),
           "bf16": lambda x: torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()}
    for s, L in enumerate(c.seq_lens):
        p = np.arange(L)
        blk = c.block_table[s, p // c.block_size]
        K = dec[c.kv_dtype](c.k_cache[blk, :, p % c.block_size, :])
        V = dec[c.kv_dtype](c.v_cache[blk, :, p % c.block_size, :])
        out.append((K, V))
    return out


def _q64(c):
    if c.q_dtype == "f32":
        return c.q.astype(np.float64)
    return torch.from_numpy(c.q.view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def check_bruteforce_decode(orc):
    """Pure-Python scalar loops on tiny inputs agree to 1e-12."""
    c = _decode_case(config=90, layer=0, n_q=4, n_kv=2, d=3, seq_lens=[5, 9], kv_dtype="f32",
                     block_size=4, num_blocks=6)
    got = _run_decode(orc, c)
    q = c.q.astype(np.float64)
    G = c.n_q // c.n_kv
    for s, L in enumerate(c.seq_lens):
        for h in range(c.n_q):
            kvh = h // G
            scores = []
            for p in range(L):
                blk = int(c.block_table[s][p // 4])
                k = [float(x) for x in c.k_cache[blk, kvh, p % 4]]
                scores.append(sum(q[s, h, i] * k[i] for i in range(c.d)) * c.scale)
            mx = max(scores)
            ex = [math.exp(x - mx) for x in scores]
            tot = sum(ex)
            for i in range(c.d):
                o = 0.0
                for p in range(L):
                    blk = int(c.block_table[s][p // 4])
                    o += ex[p] / tot * float(c.v_cache[blk, kvh, p % 4, i])
                assert abs(got[s, h, i] - o) <= 1e-12, (s, h, i)


def check_sdpa_decode(orc):
    """torch float64 scaled_dot_product_attention on repeat_interleave'd K/V."""
    for kv_dtype, n_q, n_kv in (("bf16", 8, 2), ("f32", 6, 6), ("bf16", 4, 1)):
        c = _decode_case(config=91, layer=n_q, n_q=n_q, n_kv=n_kv, d=16, seq_lens=[1, 17, 40],
                         kv_dtype=kv_dtype, num_blocks=10)
        got = _run_decode(orc, c)
        q = _q64(c)
        for s, (K, V) in enumerate(_contiguous_kv(c)):
            G = n_q // n_kv
            Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
            Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
            qt = torch.from_numpy(q[s])[None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=c.scale)[0, :, 0, :]
            assert np.max(np.abs(got[s] - ref.numpy())) <= 1e-12, (kv_dtype, s)


def check_sdpa_prefill(orc):
    """Chunked prefill == SDPA with the chunk's bottom-right causal mask."""
    p = synth.make_prefill_case(config=92, layer=0, n_q=4, n_kv=2, d=16, context_lens=[0, 5, 21, 32],
                                q_len=[7, 1, 12, 3])
    got = orc.paged_prefill(p.q, p.q_dtype, p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, p.kv_dtype,
                            None, None, p.block_table, p.n_q, p.n_kv, p.scale, causal=True)
    got_nc = orc.paged_prefill(p.q, p.q_dtype, p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, p.kv_dtype,
                               None, None, p.block_table, p.n_q, p.n_kv, p.scale, causal=False)
    qall = torch.from_numpy(p.q.view(np.int16).copy()).view(torch.bfloat16).double()
    for s in range(p.num_seqs):
        ctx = int(p.context_lens[s])
        a, b = int(p.cu_q_lens[s]), int(p.cu_q_lens[s + 1])
        n = b - a
        L = ctx + n
        pos = np.arange(L)
        blk = p.block_table[s, pos // 16]
        K = torch.from_numpy(p.k_cache[blk, :, pos % 16, :].view(np.int16).copy()).view(torch.bfloat16).double()
        V = torch.from_numpy(p.v_cache[blk, :, pos % 16, :].view(np.int16).copy()).view(torch.bfloat16).double()
        G = p.n_q // p.n_kv
        Kt = K.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        Vt = V.permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
        qt = qall[a:b].permute(1, 0, 2)[None]
        mask = torch.arange(L)[None, :] <= (ctx + torch.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=p.scale)
        assert np.max(np.abs(got[a:b] - ref[0].permute(1, 0, 2).numpy())) <= 1e-12, s
        ref_nc = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=p.scale)
        assert np.max(np.abs(got_nc[a:b] - ref_nc[0].permute(1, 0, 2).numpy())) <= 1e-12, s


def check_prefill_reductions(orc):
    """ctx = 0 is causal self-attention; a one-token chunk equals decode with
    seq_len = ctx + 1."""
    p = synth.make_prefill_case(config=93, layer=0, n_q=8, n_kv=2, d=32, context_lens=[0], q_len=[20])
    got = orc.paged_prefill(p.q, p.q_dtype, p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, p.kv_dtype,
                            None, None, p.block_table, p.n_q, p.n_kv, p.scale)
    q = torch.from_numpy(p.q.view(np.int16).copy()).view(torch.bfloat16).double().permute(1, 0, 2)[None]
    pos = np.arange(20)
    blk = p.block_table[0, pos // 16]
    K = torch.from_numpy(p.k_cache[blk, :, pos % 16].view(np.int16).copy()).view(torch.bfloat16).double()
    V = torch.from_numpy(p.v_cache[blk, :, pos % 16].view(np.int16).copy()).view(torch.bfloat16).double()
    Kt = K.permute(1, 0, 2).repeat_interleave(4, dim=0)[None]
    Vt = V.permute(1, 0, 2).repeat_interleave(4, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, is_causal=True, scale=p.scale)
    assert np.max(np.abs(got - ref[0].permute(1, 0, 2).numpy())) <= 1e-12
    # chunk of one token at ctx = 37 vs decode over 38 tokens, same bytes
    p1 = synth.make_prefill_case(config=94, layer=0, n_q=8, n_kv=2, d=32, context_lens=[37], q_len=[1])
    pf = orc.paged_prefill(p1.q, p1.q_dtype, p1.cu_q_lens, p1.context_lens, p1.k_cache, p1.v_cache, p1.kv_dtype,
                           None, None, p1.block_table, p1.n_q, p1.n_kv, p1.scale)
    dec = orc.paged_decode(p1.q, p1.q_dtype, p1.k_cache, p1.v_cache, p1.kv_dtype, None, None, p1.block_table,
                           np.array([38]), p1.n_q, p1.n_kv, p1.scale)
    assert np.array_equal(pf, dec)


def check_paged_equals_contiguous(orc):
    """The same logical rows under a permuted table and under the identity
    table give bitwise-equal outputs."""
    c = _decode_case(config=95, layer=0, n_q=8, n_kv=2, d=32, seq_lens=[3, 16, 33, 70], kv_dtype="bf16",
                     num_blocks=20)
    got = _run_decode(orc, c)
    # re-lay the same rows contiguously: sequence s's block j -> physical block base_s + j
    nb = c.block_table.shape[1]
    kc2 = np.full_like(c.k_cache, synth.POISON["bf16"])
    vc2 = np.full_like(c.v_cache, synth.POISON["bf16"])
    table2 = np.full_like(c.block_table, -1)
    base = 0
    for s, L in enumerate(c.seq_lens):
        n = -(-int(L) // 16)
        for j in range(n):
            kc2[base + j] = c.k_cache[c.block_table[s, j]]
            vc2[base + j] = c.v_cache[c.block_table[s, j]]
            table2[s, j] = base + j
        base += n
    assert not np.array_equal(table2, c.block_table)
    got2 = _run_decode(orc, c, k_cache=kc2, v_cache=vc2, block_table=table2)
    assert np.array_equal(got, got2)
    assert nb >= 5


def check_block_sizes_and_csr(orc):
    """The same sequences paged into blocks of 8, 16 and 64 tokens, through a
    2-D table or as CSR rows, give bitwise-equal decode and prefill outputs
    ([KVP] Problem 4: block = p // B, offset = p % B; [MEM] "Walking the
    table"), equal to attention over the unpaged rows within rounding."""
    r = np.random.default_rng(21)
    n_q, n_kv, d = 4, 2, 8
    lens = [1, 7, 8, 9, 40, 100]
    rows_k = [r.standard_normal((L, n_kv, d)) for L in lens]
    rows_v = [r.standard_normal((L, n_kv, d)) for L in lens]
    q = r.standard_normal((len(lens), n_q, d)).astype(np.float32)
    scale = 0.3
    outs, pre = [], []
    for B in (8, 16, 64):
        need = [-(-L // B) for L in lens]
        nb = sum(need) + 3
        perm = r.permutation(nb)
        k = np.full((nb, n_kv, B, d), np.nan, np.float32)
        v = np.full((nb, n_kv, B, d), np.nan, np.float32)
        table = np.full((len(lens), max(need)), -1, np.int32)
        cur = 0
        for s, L in enumerate(lens):
            ids = perm[cur:cur + need[s]]
            cur += need[s]
            table[s, :need[s]] = ids
            for p in range(L):
                k[ids[p // B], :, p % B] = rows_k[s][p]
                v[ids[p // B], :, p % B] = rows_v[s][p]
        out = orc.paged_decode(q, "f32", k, v, "f32", None, None, table, lens, n_q, n_kv, scale)
        indptr = np.concatenate([[0], np.cumsum(need)]).astype(np.int32)
        indices = np.concatenate([table[s, :need[s]] for s in range(len(lens))]).astype(np.int32)
        csr_rows = [orc.csr_pages(indptr, indices, s) for s in range(len(lens))]
        out_csr = orc.paged_decode(q, "f32", k, v, "f32", None, None, csr_rows, lens, n_q, n_kv, scale)
        assert np.array_equal(out, out_csr)
        outs.append(out)
        # prefill: the last 3 tokens of each sequence as the chunk
        ql = np.minimum(3, lens)
        ctx = np.array(lens) - ql
        cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        qp = np.random.default_rng(5).standard_normal((int(cu[-1]), n_q, d)).astype(np.float32)
        pre.append(orc.paged_prefill(qp, "f32", cu, ctx, k, v, "f32", None, None, csr_rows, n_q, n_kv, scale))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    for o in pre[1:]:
        assert np.array_equal(o, pre[0])
    # and the unpaged computation agrees
    for s, L in enumerate(lens):
        for h in range(n_q):
            kv = h // (n_q // n_kv)
            sc = rows_k[s][:, kv, :].astype(np.float32).astype(np.float64) @ q[s, h].astype(np.float64) * scale
            w = np.exp(sc - sc.max())
            want = (w / w.sum()) @ rows_v[s][:, kv, :].astype(np.float32).astype(np.float64)
            assert np.allclose(outs[0][s, h], want, rtol=1e-12, atol=1e-12)


def check_cache_equals_recompute(orc):
    """T steps of append-then-attend through the paged cache equal full causal
    attention recomputed from all inputs at each step (synthetic projections)."""
    r = np.random.default_rng(11)
    T, dm, n_q, n_kv, d, B = 12, 24, 4, 2, 8, 4
    WQ = r.standard_normal((dm, n_q * d)) / math.sqrt(dm)
    WK = r.standard_normal((dm, n_kv * d)) / math.sqrt(dm)
    WV = r.standard_normal((dm, n_kv * d)) / math.sqrt(dm)
    X = r.standard_normal((T, dm))
    num_blocks = 5
    table = np.array([[3, 0, 4]], dtype=np.int32)
    kc = np.full((num_blocks, n_kv, B, d), np.nan, dtype=np.float32)
    vc = np.full((num_blocks, n_kv, B, d), np.nan, dtype=np.float32)
    scale = 1.0 / math.sqrt(d)
    projections = 0
    Q = (X @ WQ).reshape(T, n_q, d).astype(np.float32)
    Kf = (X @ WK).reshape(T, n_kv, d).astype(np.float32)
    Vf = (X @ WV).reshape(T, n_kv, d).astype(np.float32)
    for t in range(T):
        projections += 1  # one new K/V projection per step with a cache
        slot = orc.slot_mapping(table, [0], [t], B)
        kc, vc = orc.kv_append(kc, vc, slot, Kf[t:t + 1], Vf[t:t + 1])
        out = orc.paged_decode(Q[t:t + 1], "f32", kc, vc, "f32", None, None, table, np.array([t + 1]),
                               n_q, n_kv, scale)
        # recompute from scratch: all t+1 rows, causal self-attention, last row
        qt = torch.from_numpy(Q[:t + 1].astype(np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(Kf[:t + 1].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)[None]
        vt = torch.from_numpy(Vf[:t + 1].astype(np.float64)).permute(1, 0, 2).repeat_interleave(2, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
        assert np.max(np.abs(out[0] - ref[0, :, t, :].numpy())) <= 1e-12, t
    assert projections == T
    demo = _golden("decode_demo.json")["redundancy"]
    Tn = demo["T"]
    assert Tn * (Tn + 1) // 2 - Tn == demo["redundant_projections"]


def check_head_grouping(orc):
    """GQA equals MHA on explicitly repeat_interleave'd K/V; MQA (one KV head)
    equals single-head attention per query head."""
    c = _decode_case(config=96, layer=0, n_q=8, n_kv=2, d=16, seq_lens=[9, 30], kv_dtype="f32", num_blocks=4)
    got = _run_decode(orc, c)
    kc = np.repeat(c.k_cache, 4, axis=1)  # repeat_interleave over the head axis
    vc = np.repeat(c.v_cache, 4, axis=1)
    mha = _run_decode(orc, c, k_cache=kc, v_cache=vc, n_kv=8)
    assert np.array_equal(got, mha)
    # MQA
    m = _decode_case(config=97, layer=0, n_q=4, n_kv=1, d=16, seq_lens=[12], kv_dtype="f32", num_blocks=1)
    gm = _run_decode(orc, m)
    for h in range(4):
        one = _run_decode(orc, m, q=m.q[:, h:h + 1], n_q=1, n_kv=1)
        assert np.array_equal(gm[:, h:h + 1], one)
    # the ratio check fires before any work
    try:
        _run_decode(orc, c, n_q=6, n_kv=4)
    except ValueError:
        pass
    else:
        raise AssertionError("non-multiple head ratio must raise")


def check_special_cases(orc):
    """Closed forms: one key -> V[0]; identical keys or q = 0 -> mean(V);
    q = c * k_j with a large c -> V[j]; huge scores stay finite."""
    c = _decode_case(config=98, layer=0, n_q=2, n_kv=1, d=8, seq_lens=[1, 20], kv_dtype="f32", num_blocks=3)
    got = _run_decode(orc, c)
    b0 = c.block_table[0, 0]
    assert np.array_equal(got[0], np.repeat(c.v_cache[b0, 0, 0][None].astype(np.float64), 2, 0))
    # identical keys
    kc = c.k_cache.copy()
    kc[...] = kc[c.block_table[1, 0], 0, 0]
    got2 = _run_decode(orc, c, k_cache=kc)
    V = np.concatenate([c.v_cache[c.block_table[1, 0], 0, :16], c.v_cache[c.block_table[1, 1], 0, :4]]).astype(np.float64)
    assert np.max(np.abs(got2[1] - V.mean(0)[None])) <= 1e-12
    # q = 0
    got3 = _run_decode(orc, c, q=np.zeros_like(c.q))
    assert np.max(np.abs(got3[1] - V.mean(0)[None])) <= 1e-12
    # dominant key: key 7 = 10 e_0, the others shrunk to 0.1x, q = 100 e_0:
    # the score gap is hundreds, so the output is V[7] to rounding
    j = 7
    kd = c.k_cache.copy()
    for p in range(20):
        kd[c.block_table[1, p // 16], 0, p % 16] *= np.float32(0.1)
    kd[c.block_table[1, 0], 0, j] = 0.0
    kd[c.block_table[1, 0], 0, j, 0] = 10.0
    q = np.zeros_like(c.q)
    q[1, :, 0] = 100.0
    got4 = _run_decode(orc, c, q=q, k_cache=kd)
    assert np.max(np.abs(got4[1] - V[j][None])) <= 1e-12
    # stability: scores of order 1e4 must not overflow
    got5 = _run_decode(orc, c, q=(c.q * np.float32(3000.0)))
    assert np.all(np.isfinite(got5))
    # fp8: values are code * per-(block, head) scale
    f = _decode_case(config=99, layer=0, n_q=2, n_kv=1, d=4, seq_lens=[32], kv_dtype="fp8", num_blocks=2)
    kc8 = np.full_like(f.k_cache, 0x38)        # every key = 1.0 * scale
    vc8 = f.v_cache.copy()
    b0, b1 = f.block_table[0, 0], f.block_table[0, 1]
    vc8[b0] = 0x38                             # 1.0
    vc8[b1] = 0x40                             # 2.0
    ks = np.full_like(f.k_scale, 0.75)
    vs = f.v_scale.copy()
    vs[b0] = 2.0
    vs[b1] = 0.25
    got6 = _run_decode(orc, f, k_cache=kc8, v_cache=vc8, k_scale=ks, v_scale=vs)
    assert np.max(np.abs(got6 - 1.25)) <= 1e-12  # mean of 16 x 2.0 and 16 x 0.5
    # a key scale that differs per block changes scores exactly as code * scale
    ks2 = ks.copy()
    ks2[b1] = 0.0
    qf = np.zeros_like(f.q)
    qf[0, :, 0] = 0x3F80  # q = (1, 0, 0, 0) in bf16
    got7 = _run_decode(orc, f, k_cache=kc8, v_cache=vc8, k_scale=ks2, v_scale=vs, q=qf)
    w0 = math.exp(0.75 * f.scale)  # score of block-0 keys: 1 * 1.0 * 0.75 * scale
    want = (16 * w0 * 2.0 + 16 * 1.0 * 0.5) / (16 * w0 + 16)
    assert np.max(np.abs(got7 - want)) <= 1e-12


def _online_partitioned(q, K, V, scale, P):
    """Test-only FlashAttention-style recurrence: tiles of P keys, running max m
    and sum l, rescale by e^(m - m_new); then merge partitions."""
    parts = []
    for a in range(0, K.shape[0], P):
        m, l, o = -np.inf, 0.0, np.zeros(V.shape[1])
        for t0 in range(a, min(a + P, K.shape[0]), 3):  # inner tiles of 3 keys
            s = K[t0:min(t0 + 3, a + P)] @ q * scale
            m_new = max(m, s.max())
            alpha = math.exp(m - m_new) if m > -np.inf else 0.0
            e = np.exp(s - m_new)
            l = alpha * l + e.sum()
            o = alpha * o + e @ V[t0:t0 + len(s)]
            m = m_new
        parts.append((m, l, o))
    M = max(p[0] for p in parts)
    L = sum(math.exp(p[0] - M) * p[1] for p in parts)
    O = sum(math.exp(p[0] - M) * p[2] for p in parts)
    return O / L


def check_online_softmax(orc):
    """The tiled online softmax and the partition merge reach the textbook
    result to 1e-12 for several partition sizes."""
    c = _decode_case(config=100, layer=0, n_q=2, n_kv=1, d=16, seq_lens=[157], kv_dtype="f32", num_blocks=10)
    got = _run_decode(orc, c, q=(c.q * np.float32(4.0)))
    K, V = _contiguous_kv(c)[0]
    for P in (1, 7, 16, 64, 157, 512):
        for h in range(2):
            o = _online_partitioned(c.q[0, h].astype(np.float64) * 4.0, K[:, 0], V[:, 0], c.scale, P)
            assert np.max(np.abs(o - got[0, h])) <= 1e-12, P


def check_demo_shapes(orc):
    """The five-step decode demo: the cache holds 1..5 rows and every output is
    one vector per head (batch 1, 4 heads, d 64); step 0 returns v_0 exactly."""
    g = _golden("decode_demo.json")
    r = np.random.default_rng(0)
    heads, d, B = g["heads"], g["d_head"], 16
    kc = np.full((1, heads, B, d), np.nan, dtype=np.float32)
    vc = kc.copy()
    table = np.array([[0]], dtype=np.int32)
    for step in range(g["steps"]):
        x = r.standard_normal((1, heads, d)).astype(np.float32)
        kc, vc = orc.kv_append(kc, vc, orc.slot_mapping(table, [0], [step], B), x, x)
        out = orc.paged_decode(x, "f32", kc, vc, "f32", None, None, table, np.array([step + 1]), heads, heads,
                               1.0 / math.sqrt(d))
        rows = int(np.sum(~np.isnan(kc[0, 0, :, 0])))
        assert rows == g["cache_rows_after_step"][step]
        assert (out.shape[0], out.shape[1], 1, out.shape[2]) == tuple(g["output_shape"])
        if step == 0:
            assert np.array_equal(out[0], x[0].astype(np.float64))


def check_poison_ignored(orc):
    """NaN-poisoned tail slots and unused blocks never reach a result."""
    for kv in ("f32", "bf16", "fp8"):
        c = _decode_case(config=101, layer=0, n_q=4, n_kv=2, d=16, seq_lens=[1, 15, 17, 33], kv_dtype=kv,
                         num_blocks=12)
        assert np.isnan(orc.decode_storage(c.k_cache, kv)).any()
        assert np.all(np.isfinite(_run_decode(orc, c)))


ALL_CHECKS = [
    check_sizing, check_csr_walk, check_waste, check_append_gather, check_e4m3, check_bf16,
    check_bruteforce_decode, check_sdpa_decode, check_sdpa_prefill, check_prefill_reductions,
    check_paged_equals_contiguous, check_cache_equals_recompute, check_head_grouping, check_special_cases,
    check_online_softmax, check_demo_shapes, check_poison_ignored, check_block_sizes_and_csr,
]


# ---------------------------------------------------------------------------
# block sharing and copy-on-write
# ---------------------------------------------------------------------------

def _replay_cow(pool, steps, B, width=8):
    """Run the fixture's operations; yields (step, row or None, copies)."""
    rows = {}
    for st in steps:
        row, copies = None, []
        if st["op"] == "prompt":
            n = -(-st["tokens"] // B)
            rows[st["seq"]] = (list(pool.alloc(n)) + [0] * width)[:width]
            row = rows[st["seq"]][:n]
        elif st["op"] == "fork":
            n = len(st["row"])
            pool.share(rows[st["from"]][:n])
            rows[st["seq"]] = list(rows[st["from"]])
            row = rows[st["seq"]][:n]
        elif st["op"] == "append":
            r, copies = pool.prepare_append(rows[st["seq"]], st["seq_len"], st["tokens"], B)
            rows[st["seq"]] = list(r)
            row = list(r)[:-(-(st["seq_len"] + st["tokens"]) // B)]
        elif st["op"] == "release":
            pool.release(rows[st["seq"]][:4])  # the released sequence owns four blocks
        yield st, row, [list(c) for c in copies]


def check_cow_fixture(orc):
    """The fork / append / release walk worked by hand from the page's rules."""
    g = _golden("cow_fork.json")
    pool = orc.BlockPool(g["num_blocks"])
    for st, row, copies in _replay_cow(pool, g["steps"], g["block_size"]):
        if row is not None:
            assert row == st["row"], (st, row)
        if st["op"] == "append":
            assert copies == st["copies"], (st, copies)
        if st["op"] == "release":
            assert pool.free_blocks() == st["free"], st
        assert list(pool.ref) == st["ref"], (st, list(pool.ref))


def check_cow_invariants(orc):
    """Random forks, appends and releases: a block's count equals the number
    of live tables naming it, and after an append every block the new tokens
    fall into is named by that table alone (so writing it touches no other
    sequence)."""
    rng = np.random.default_rng(7)
    B, N = 4, 64
    pool = orc.BlockPool(N)
    live = {}  # seq -> (row, length)
    nxt = 0
    for _ in range(400):
        op = rng.integers(0, 4)
        if op == 0 or not live:
            n = int(rng.integers(1, 10))
            try:
                row, _ = pool.prepare_append([0] * 32, 0, n, B)
            except orc.PoolExhausted:
                continue
            live[nxt] = (row, n)
            nxt += 1
        elif op == 1:
            s = int(rng.choice(list(live)))
            row, L = live[s]
            pool.share(row[:-(-L // B)])
            live[nxt] = (list(row), L)
            nxt += 1
        elif op == 2:
            s = int(rng.choice(list(live)))
            row, L = live[s]
            n = int(rng.integers(1, 7))
            if -(-(L + n) // B) > 32:
                continue
            before = pool.free_blocks()
            try:
                new_row, copies = pool.prepare_append(row, L, n, B)
            except orc.PoolExhausted:
                assert pool.free_blocks() == before  # nothing changed
                continue
            for j in range(L // B, (L + n - 1) // B + 1):
                assert pool.ref[new_row[j]] == 1
            for src, dst in copies:
                assert src in row[:-(-L // B)] and dst not in row[:-(-L // B)]
            live[s] = (new_row, L + n)
        else:
            s = int(rng.choice(list(live)))
            row, L = live.pop(s)
            pool.release(row[:-(-L // B)])
        counts = np.zeros(N, dtype=int)
        for row, L in live.values():
            for b in row[:-(-L // B)]:
                counts[b] += 1
        assert list(counts) == list(pool.ref)
        assert pool.free_blocks() == int(np.sum(counts == 0))


def check_copy_blocks(orc):
    """A copied block equals its source in every head and slot, scales
    included; no other block changes."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((6, 2, 4, 8)).astype(np.float32)
    v = rng.standard_normal((6, 2, 4, 8)).astype(np.float32)
    ks, vs = rng.random((6, 2)).astype(np.float32), rng.random((6, 2)).astype(np.float32)
    k2, v2, ks2, vs2 = orc.copy_blocks(k, v, [(1, 4), (2, 0)], ks, vs)
    for src, dst in [(1, 4), (2, 0)]:
        assert np.array_equal(k2[dst], k[src]) and np.array_equal(v2[dst], v[src])
        assert np.array_equal(ks2[dst], ks[src]) and np.array_equal(vs2[dst], vs[src])
    for b in (1, 2, 3, 5):
        assert np.array_equal(k2[b], k[b]) and np.array_equal(v2[b], v[b]) and np.array_equal(ks2[b], ks[b])


def check_shared_prefix_decode(orc):
    """'Prefix sharing': two sequences whose tables name the same prefix
    blocks attend exactly as two sequences holding private copies."""
    rng = np.random.default_rng(11)
    B, n_kv, d, n_q = 4, 2, 8, 4
    k = rng.standard_normal((10, n_kv, B, d)).astype(np.float32)
    v = rng.standard_normal((10, n_kv, B, d)).astype(np.float32)
    q = rng.standard_normal((2, n_q, d)).astype(np.float32)
    shared = np.array([[0, 1, 2, 0], [0, 1, 3, 0]], dtype=np.int32)     # blocks 0, 1 shared
    private = np.array([[0, 1, 2, 0], [4, 5, 3, 0]], dtype=np.int32)    # 4, 5 copies of 0, 1
    k2, v2 = k.copy(), v.copy()
    k2[4], k2[5], v2[4], v2[5] = k[0], k[1], v[0], v[1]
    lens = np.array([10, 11], dtype=np.int32)
    a = orc.paged_decode(q, "f32", k, v, "f32", None, None, shared, lens, n_q, n_kv, 0.3)
    b = orc.paged_decode(q, "f32", k2, v2, "f32", None, None, private, lens, n_q, n_kv, 0.3)
    assert np.array_equal(a, b)


ALL_CHECKS += [check_cow_fixture, check_cow_invariants, check_copy_blocks, check_shared_prefix_decode]


# ---------------------------------------------------------------------------
# fp8 quantisation on append
# ---------------------------------------------------------------------------

def check_e4m3_encode(orc):
    """Every finite code's value encodes to that code; midpoints go to the even
    code; magnitudes past 448 saturate; random in-range values agree with
    torch's float8_e4m3fn cast."""
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.e4m3fn_to_f64(codes)
    finite = ~np.isnan(vals)
    back = orc.encode_e4m3fn(vals[finite])
    assert np.array_equal(back, codes[finite])
    pos = np.sort(np.unique(vals[finite & (vals >= 0)]))
    mids = (pos[:-1] + pos[1:]) / 2
    enc = orc.encode_e4m3fn(mids)
    lo_codes = orc.encode_e4m3fn(pos[:-1])
    hi_codes = orc.encode_e4m3fn(pos[1:])
    want = np.where(lo_codes % 2 == 0, lo_codes, hi_codes)
    assert np.array_equal(enc, want)
    assert list(orc.encode_e4m3fn(np.array([449.0, 1e9, -500.0]))) == [0x7E, 0x7E, 0xFE]
    x = (np.random.default_rng(5).standard_normal(20000) * np.exp2(np.random.default_rng(6).integers(-12, 9, 20000))
         ).astype(np.float32)
    x = x[np.abs(x) <= 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.encode_e4m3fn(x), t)


def check_fp8_append_fixture(orc):
    g = _golden("fp8_append.json")
    B, d = g["block_size"], 2
    codes = np.zeros((B, d), dtype=np.uint8)
    scale = np.float32(0)
    for st in g["steps"]:
        codes, scale = orc.append_block_fp8(codes, scale, st["n_old"], np.array(st["rows"], dtype=np.float32))
        n = len(st["codes"])
        assert [[hex(c) for c in row] for row in codes[:n]] == [[c if c != "0x00" else "0x0" for c in row]
                                                                for row in st["codes"]], st
        assert scale == np.float32(st["scale_num"]) / np.float32(448.0)


def check_fp8_append_one_shot(orc):
    """A block filled by one append holds exactly the workload's encoding:
    scale = largest magnitude / 448 and codes = x / scale cast to E4M3FN
    (torch's float32 division and cast)."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, 32)) * 3).astype(np.float32)
    codes, scale = orc.append_block_fp8(np.zeros((16, 32), np.uint8), np.float32(0), 0, x)
    tx = torch.from_numpy(x)
    ts = tx.abs().max() / 448.0
    assert scale == np.float32(ts.item())
    assert np.array_equal(codes, (tx / ts).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def check_fp8_append_invariants(orc):
    """Appending token by token: the scale covers every value appended to the
    block (scale * 448 >= max |x|), never shrinks, and every stored value is
    within the rounding of a few E4M3 steps of what was appended."""
    rng = np.random.default_rng(12)
    B, n_kv, d, nb = 4, 2, 8, 6
    k = np.zeros((nb, n_kv, B, d), np.uint8)
    v = np.zeros_like(k)
    ks = np.zeros((nb, n_kv), np.float32)
    vs = np.zeros_like(ks)
    table = np.array([[3, 1, 5], [0, 2, 4]], dtype=np.int32)
    lens = [0, 0]
    hist = {0: [], 1: []}
    for step in range(9):
        n = [int(rng.integers(1, 3)), 1]
        n = [min(n[s], 12 - lens[s]) for s in range(2)]
        if sum(n) == 0:
            break
        kn = (rng.standard_normal((sum(n), n_kv, d)) * rng.choice([0.1, 1, 10])).astype(np.float32)
        vn = (rng.standard_normal((sum(n), n_kv, d))).astype(np.float32)
        cu = [0, n[0], n[0] + n[1]]
        before = ks.copy()
        k, v, ks, vs = orc.kv_append_fp8(k, v, ks, vs, table, lens, cu, kn, vn, B)
        for s in range(2):
            for t in range(n[s]):
                hist[s].append(kn[cu[s] + t])
            lens[s] += n[s]
        touched = ks != before
        assert np.all(ks[touched] > before[touched]) or not touched.any()
        for s in range(2):
            rows = np.array(hist[s])
            for p in range(lens[s]):
                blk = table[s][p // B]
                got = orc.e4m3fn_to_f64(k[blk, :, p % B]) * ks[blk][:, None]
                assert np.all(ks[blk][:, None] * 448 >= np.abs(rows[p]) * (1 - 1e-6))
                # each re-encoding adds at most half a step (1/16 relative) plus subnormal steps
                assert np.all(np.abs(got - rows[p]) <= np.abs(rows[p]) / 8 + ks[blk][:, None] * 2.0 ** -8)


ALL_CHECKS += [check_e4m3_encode, check_fp8_append_fixture, check_fp8_append_one_shot, check_fp8_append_invariants]

# ---------------------------------------------------------------------------
# preemption by swap
# ---------------------------------------------------------------------------

def _swap_fixture_caches():
    k16 = np.zeros((3, 1, 2, 2), np.uint16)
    for b in range(3):
        k16[b, 0] = [[0x0001 + 0x10 * b, 0x0002 + 0x10 * b], [0x0003 + 0x10 * b, 0x0004 + 0x10 * b]]
    v16 = k16 + np.uint16(0x0100)
    k8 = np.zeros((2, 2, 1, 2), np.uint8)
    for b in range(2):
        for h in range(2):
            k8[b, h, 0] = [0x10 * b + 2 * h, 0x10 * b + 2 * h + 1]
    v8 = k8 | np.uint8(0x80)
    ks = np.array([[1, 2], [3, 4]], np.float32)
    vs = np.array([[0.5, 0.25], [8, 16]], np.float32)
    return k16, v16, k8, v8, ks, vs


def check_swap_fixture(orc):
    """Host images of the hand-worked example, byte for byte, and swapping
    them back in restores the blocks."""
    g = _golden("swap_image.json")
    k16, v16, k8, v8, ks, vs = _swap_fixture_caches()
    img = orc.swap_image(k16, v16, g["bf16"]["ids"])
    assert [f"{b:02x}" for b in img] == g["bf16"]["image"]
    img8 = orc.swap_image(k8, v8, g["fp8"]["ids"], ks, vs)
    assert [f"{b:02x}" for b in img8] == g["fp8"]["image"]
    k2, v2, _, _ = orc.swap_in(np.zeros_like(k16), np.zeros_like(v16), img, [0, 1])
    assert np.array_equal(k2[0], k16[2]) and np.array_equal(k2[1], k16[0]) and np.all(k2[2] == 0)
    assert np.array_equal(v2[0], v16[2]) and np.array_equal(v2[1], v16[0])
    k3, v3, ks3, vs3 = orc.swap_in(np.zeros_like(k8), np.zeros_like(v8), img8, [0], np.zeros_like(ks),
                                   np.zeros_like(vs))
    assert np.array_equal(k3[0], k8[1]) and np.array_equal(v3[0], v8[1])
    assert np.array_equal(ks3[0], ks[1]) and np.array_equal(vs3[0], vs[1]) and np.all(ks3[1] == 0)


def check_swap_equals_block_copy(orc):
    """Swapping blocks A out and into blocks B moves exactly what the block
    copy of pairs (A[i], B[i]) moves, for every element type."""
    r = np.random.default_rng(31)
    for kind, d in (("f32", 4), ("bf16", 8), ("fp8", 16)):
        dt = synth.STORAGE_DTYPE[kind]
        nb, n_kv, B = 10, 2, 4
        k = r.integers(0, 256, size=(nb, n_kv, B, d * np.dtype(dt).itemsize), dtype=np.uint8).view(dt)
        v = r.integers(0, 256, size=(nb, n_kv, B, d * np.dtype(dt).itemsize), dtype=np.uint8).view(dt)
        ks = r.random((nb, n_kv)).astype(np.float32) if kind == "fp8" else None
        vs = r.random((nb, n_kv)).astype(np.float32) if kind == "fp8" else None
        src, dst = [7, 2, 5], [0, 9, 3]
        img = orc.swap_image(k, v, src, ks, vs)
        got = orc.swap_in(k, v, img, dst, ks, vs)
        want = orc.copy_blocks(k, v, list(zip(src, dst)), ks, vs)
        for a, b in zip(got, want):
            if a is not None:
                assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def check_swap_preemption_decode(orc):
    """Preempt a sequence (swap its blocks out, let other data overwrite them),
    bring it back into other blocks and point its table there: its decode
    output is bitwise what it was before ([KVP] Problem 4: blocks are reached
    only through the table)."""
    c = _decode_case(config=97, layer=0, n_q=4, n_kv=2, d=16, seq_lens=[5, 40, 23], kv_dtype="fp8", num_blocks=12)
    before = _run_decode(orc, c)
    s = 1
    n = -(-int(c.seq_lens[s]) // 16)
    ids = [int(b) for b in c.block_table[s, :n]]
    img = orc.swap_image(c.k_cache, c.v_cache, ids, c.k_scale, c.v_scale)
    k, v, ks, vs = c.k_cache.copy(), c.v_cache.copy(), c.k_scale.copy(), c.v_scale.copy()
    k[ids] = 0x7F  # the freed blocks are reused: NaN codes
    v[ids] = 0x7F
    used = set(int(b) for b in c.block_table.reshape(-1) if b >= 0)
    fresh = [b for b in range(12) if b not in used][:n]
    assert len(fresh) == n
    k, v, ks, vs = orc.swap_in(k, v, img, fresh, ks, vs)
    table = c.block_table.copy()
    table[s, :n] = fresh
    after = _run_decode(orc, c, k_cache=k, v_cache=v, block_table=table, k_scale=ks, v_scale=vs)
    assert np.array_equal(before, after)


ALL_CHECKS += [check_swap_fixture, check_swap_equals_block_copy, check_swap_preemption_decode]
