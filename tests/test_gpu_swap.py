"""GPU parity of preemption by swap: the host image written by pkv_swap_out
is byte-identical to the oracle's, swap-in writes exactly the oracle's
blocks, and a sequence preempted (its blocks overwritten) and brought back into
other blocks decodes to the same bits as before."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev, note, oracle_decode, run_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def _buffers(pkv, n, kind, n_kv, d, B):
    nbytes = pkv.swap_image_bytes(n, {"f32": pkv.F32, "bf16": pkv.BF16, "fp8": pkv.FP8_E4M3FN}[kind], n_kv, d, B)
    staging = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    host = torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)
    return staging, host


def _raw(x):
    return np.ascontiguousarray(x).view(np.uint8)


@pytest.mark.parametrize("kind,d,B", [("f32", 64, 16), ("bf16", 128, 16), ("fp8", 128, 16), ("bf16", 128, 64),
                                      ("fp8", 64, 8)])
def test_swap_image_and_swap_in_bit_exact(pkv, kind, d, B):
    r = synth.rng(960, d, B)
    nb, n_kv = 30, 4
    dt = synth.STORAGE_DTYPE[kind]
    eb = np.dtype(dt).itemsize
    k = r.integers(0, 256, size=(nb, n_kv, B, d * eb), dtype=np.uint8).view(dt)
    v = r.integers(0, 256, size=(nb, n_kv, B, d * eb), dtype=np.uint8).view(dt)
    ks = r.random((nb, n_kv)).astype(np.float32) if kind == "fp8" else None
    vs = r.random((nb, n_kv)).astype(np.float32) if kind == "fp8" else None
    src = r.permutation(nb)[:11].astype(np.int32)
    tk, tv = dev(_raw(k)), dev(_raw(v))
    tk_t = tk.view(torch.float32 if kind == "f32" else torch.bfloat16 if kind == "bf16" else torch.uint8)
    tk_t = tk_t.view(nb, n_kv, B, d)
    tv_t = tv.view(tk_t.dtype).view(nb, n_kv, B, d)
    tks = dev(ks) if ks is not None else None
    tvs = dev(vs) if vs is not None else None
    staging, host = _buffers(pkv, len(src), kind, n_kv, d, B)
    note(f"swap out {kind} d={d} B={B}: {len(src)} blocks, {host.numel()} bytes")
    pkv.swap_out(tk_t, tv_t, dev(src), staging, host, k_scale=tks, v_scale=tvs)
    torch.cuda.synchronize()
    want = oracle.swap_image(k, v, src, ks, vs)
    assert np.array_equal(host.numpy(), want)
    # swap the image into other blocks (some of them the sources themselves)
    dst = np.concatenate([src[5:], np.setdiff1d(np.arange(nb), src)[:5]]).astype(np.int32)
    assert len(set(dst.tolist())) == len(src)
    staging.fill_(0xEE)
    pkv.swap_in(tk_t, tv_t, dev(dst), staging, host, k_scale=tks, v_scale=tvs)
    torch.cuda.synchronize()
    wk, wv, wks, wvs = oracle.swap_in(k, v, want, dst, ks, vs)
    assert np.array_equal(tk.cpu().numpy(), _raw(wk)) and np.array_equal(tv.cpu().numpy(), _raw(wv))
    if ks is not None:
        assert np.array_equal(tks.cpu().numpy(), wks) and np.array_equal(tvs.cpu().numpy(), wvs)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "f32"])
def test_preempt_and_restore_decodes_the_same_bits(pkv, kind):
    d, n_q, n_kv = (64, 8, 2) if kind == "f32" else (128, 32, 8)
    lens = [100, 1500, 33, 700]
    need = sum(synth.blocks_for(L) for L in lens)
    c = synth.make_decode_case(config=961, layer=0, n_q=n_q, n_kv=n_kv, d=d, seq_lens=lens, kv_dtype=kind,
                               num_blocks=need + 200)
    t = dict(q=dev(c.q, c.q_dtype), k_cache=dev(c.k_cache, c.kv_dtype), v_cache=dev(c.v_cache, c.kv_dtype),
             k_scale=None if c.k_scale is None else dev(c.k_scale),
             v_scale=None if c.v_scale is None else dev(c.v_scale), block_table=dev(c.block_table),
             seq_lens=dev(c.seq_lens))
    before = run_decode(pkv, c, t)
    s = 1
    n = synth.blocks_for(lens[s])
    ids = c.block_table[s, :n].astype(np.int32)
    staging, host = _buffers(pkv, n, kind, n_kv, d, 16)
    note(f"preempt sequence {s} ({n} blocks, {kind}) and restore it elsewhere")
    pkv.swap_out(t["k_cache"], t["v_cache"], dev(ids), staging, host, k_scale=t["k_scale"], v_scale=t["v_scale"])
    # the freed blocks are handed to other work and overwritten
    idx = torch.from_numpy(ids.astype(np.int64)).cuda()
    t["k_cache"].index_fill_(0, idx, float("nan") if kind != "fp8" else 0x7F)
    t["v_cache"].index_fill_(0, idx, float("nan") if kind != "fp8" else 0x7F)
    if t["k_scale"] is not None:
        t["k_scale"].index_fill_(0, idx, 123.0)
    used = set(int(b) for b in c.block_table.reshape(-1) if b >= 0)
    fresh = np.array([b for b in range(need + 200) if b not in used][50:50 + n], np.int32)
    pkv.swap_in(t["k_cache"], t["v_cache"], dev(fresh), staging, host, k_scale=t["k_scale"], v_scale=t["v_scale"])
    table = c.block_table.copy()
    table[s, :n] = fresh
    t["block_table"] = dev(table)
    after = run_decode(pkv, c, t)
    assert np.array_equal(before.view(np.uint64), after.view(np.uint64))
    want = oracle_decode(c)
    assert_parity(after, want, c.kv_dtype)


def test_swap_in_skips_ids_outside_the_pool(pkv):
    nb, n_kv, d, B = 6, 2, 64, 16
    k = torch.arange(nb * n_kv * B * d, dtype=torch.float32, device="cuda").view(nb, n_kv, B, d)
    v = -k
    staging, host = _buffers(pkv, 3, "f32", n_kv, d, B)
    pkv.swap_out(k, v, dev(np.array([0, 1, 2], np.int32)), staging, host)
    k2, v2 = k.clone(), v.clone()
    pkv.swap_in(k2, v2, dev(np.array([5, -1, nb], np.int32)), staging, host)
    torch.cuda.synchronize()
    note("swap in with ids outside the pool")
    assert torch.equal(k2[5], k[0]) and torch.equal(v2[5], v[0])
    assert torch.equal(k2[:5], k[:5]) and torch.equal(v2[:5], v[:5])
