"""GPU parity of block sharing: pkv_copy_blocks bit-exact against the oracle,
and a fork-and-diverge walk (prompt shared by two sequences, copy-on-write on
the first divergent append) whose caches stay byte-identical to the oracle's
and whose decode outputs match the oracle's attention over them."""
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


def _raw(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x).view(np.uint8)


@pytest.mark.parametrize("kind,d", [("f32", 64), ("bf16", 128), ("fp8", 128), ("bf16", 64)])
def test_copy_blocks_bit_exact(pkv, kind, d):
    r = synth.rng(900, 0, 1)
    nb, n_kv, B = 40, 4, 16
    dt = synth.STORAGE_DTYPE[synth.FP8 if kind == "fp8" else synth.BF16 if kind == "bf16" else synth.F32]
    # arbitrary bytes, NaN patterns included: the copy must not interpret them
    k = r.integers(0, 256, size=(nb, n_kv, B, d * np.dtype(dt).itemsize), dtype=np.uint8).view(dt)
    v = r.integers(0, 256, size=k.view(np.uint8).shape, dtype=np.uint8).view(dt)
    ks = r.random((nb, n_kv)).astype(np.float32) if kind == "fp8" else None
    vs = r.random((nb, n_kv)).astype(np.float32) if kind == "fp8" else None
    perm = r.permutation(nb)
    src, dst = perm[:12].astype(np.int32), perm[12:24].astype(np.int32)
    # pairs naming blocks outside the pool are skipped
    src_all = np.concatenate([src, np.array([-1, 3], np.int32)])
    dst_all = np.concatenate([dst, np.array([5, nb], np.int32)])
    note(f"copy_blocks {kind} d={d}: 12 pairs + 2 out-of-pool")
    tk = torch.from_numpy(k.view(np.uint8).copy()).cuda()
    tv = torch.from_numpy(v.view(np.uint8).copy()).cuda()
    tk_t = tk.view(torch.float32 if kind == "f32" else torch.bfloat16 if kind == "bf16" else torch.uint8)
    tv_t = tv.view(tk_t.dtype)
    tks = dev(ks) if ks is not None else None
    tvs = dev(vs) if vs is not None else None
    pkv.copy_blocks(tk_t, tv_t, dev(src_all), dev(dst_all), k_scale=tks, v_scale=tvs)
    torch.cuda.synchronize()
    wk, wv, wks, wvs = oracle.copy_blocks(k, v, list(zip(src.tolist(), dst.tolist())), ks, vs)
    assert np.array_equal(tk.cpu().numpy(), _raw(wk))
    assert np.array_equal(tv.cpu().numpy(), _raw(wv))
    if ks is not None:
        assert np.array_equal(tks.cpu().numpy(), wks) and np.array_equal(tvs.cpu().numpy(), wvs)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_fork_and_diverge(pkv, kind):
    """Sequence A holds a 37-token prompt; B forks it (shares its blocks);
    both then append different tokens.  Library and oracle run the same pool
    operations, block copies and appends; the caches must agree byte for byte
    after every step and the decode outputs within the dtype's tolerance."""
    r = synth.rng(901, 0, 2)
    nb, n_kv, n_q, d, B, W = 24, 2, 8, 64, 16, 8
    code = synth.BF16 if kind == "bf16" else synth.F32
    dt = synth.STORAGE_DTYPE[code]
    poison = synth.POISON[code]
    k_host = np.full((nb, n_kv, B, d), poison, dtype=dt)
    v_host = k_host.copy()
    tk, tv = dev(k_host, kind), dev(v_host, kind)
    ours, ref = pkv.BlockPool(nb), oracle.BlockPool(nb)
    rows, lens = {}, {}

    def fresh_rows(n):
        return synth.encode(r.standard_normal((n, n_kv, d)).astype(np.float32), kind)

    def append(seq, n):
        nonlocal k_host, v_host
        row, L = rows[seq], lens[seq]
        got_row, got_c = ours.prepare_append(row, L, n, B)
        want_row, want_c = ref.prepare_append(row, L, n, B)
        assert got_row == want_row and got_c == want_c
        if got_c:
            pkv.copy_blocks(tk, tv, dev(np.array([c[0] for c in got_c], np.int32)),
                            dev(np.array([c[1] for c in got_c], np.int32)))
            k_host, v_host, _, _ = oracle.copy_blocks(k_host, v_host, want_c)
        rows[seq] = got_row
        table = np.array([got_row], dtype=np.int32)
        pos = np.arange(L, L + n, dtype=np.int32)
        slots = pkv.slot_mapping(dev(table), dev(np.zeros(n, np.int32)), dev(pos), B)
        kn, vn = fresh_rows(n), fresh_rows(n)
        pkv.kv_append(tk, tv, slots, dev(kn, kind), dev(vn, kind))
        k_host, v_host = oracle.kv_append(k_host, v_host, oracle.slot_mapping(table, [0] * n, pos, B), kn, vn)
        lens[seq] = L + n
        return got_c

    rows["A"], lens["A"] = [0] * W, 0
    append("A", 37)
    rows["B"], lens["B"] = list(rows["A"]), lens["A"]
    ours.share(rows["A"][:3])
    ref.share(rows["A"][:3])
    copies = []
    for step, (seq, n) in enumerate([("A", 1), ("B", 2), ("A", 12), ("B", 30), ("A", 3), ("B", 1)]):
        c = append(seq, n)
        copies += c
        torch.cuda.synchronize()
        assert np.array_equal(_raw(host_bits(tk)), _raw(k_host)), step
        assert np.array_equal(_raw(host_bits(tv)), _raw(v_host)), step
        table = np.array([rows["A"], rows["B"]], dtype=np.int32)
        sl = np.array([lens["A"], lens["B"]], dtype=np.int32)
        q = synth.encode(r.standard_normal((2, n_q, d)).astype(np.float32), kind)
        note(f"fork {kind} step {step}: {seq} +{n}, lens {sl.tolist()}, copies so far {copies}")
        out = pkv.paged_attn_decode(dev(q, kind), tk, tv, dev(table), dev(sl), n_q, n_kv, d, B, 0.125)
        torch.cuda.synchronize()
        want = oracle.paged_decode(q, kind, k_host, v_host, kind, None, None, table, sl, n_q, n_kv, 0.125)
        assert_parity(out.cpu().numpy().astype(np.float64), want, kind, f"step {step}")
    # the first divergent append copied the shared, partly filled prompt block
    assert copies and copies[0][0] == 2
    assert ours.refcount(0) == 2 and ours.refcount(1) == 2
