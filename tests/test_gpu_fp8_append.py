"""GPU parity of FP8 quantisation on append (pkv_kv_append_fp8): cache bytes
and per-(block, KV head) scales bit-exact against oracle.kv_append_fp8 on the
same host inputs -- a ragged batch over random prior states (scales that grow
and re-encode, scales that stay), every bf16 value in [-448, 448] and float32
ties through the encoder at scale 1, token-by-token and chunked appends from
an empty cache followed by a decode over the result, and the skip rules."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev, note

pytestmark = pytest.mark.gpu

B = 16


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def _random_codes(r, shape):
    """Finite E4M3FN codes of either sign (no NaN pattern)."""
    mag = r.integers(0, 0x7F, size=shape, dtype=np.uint8)
    return mag | (r.integers(0, 2, size=shape, dtype=np.uint8) << 7)


def _tables(r, batch, max_blocks, nb):
    perm = r.permutation(nb)[:batch * max_blocks].astype(np.int32)
    return perm.reshape(batch, max_blocks)


def _new_rows(r, total, n_kv, d, kind, gains):
    """New K/V rows: normal values times a per-token gain, a few exact zeros
    and negative zeros; returns (device-side storage array, float32 values)."""
    x = r.standard_normal((total, n_kv, d)).astype(np.float32) * gains[:, None, None]
    x.reshape(-1)[r.integers(0, x.size, size=max(x.size // 97, 1))] = 0.0
    x.reshape(-1)[r.integers(0, x.size, size=max(x.size // 89, 1))] = -0.0
    if kind == "bf16":
        bits = synth.encode(x, "bf16")
        return bits, oracle.bf16_bits_to_f64(bits).astype(np.float32)
    return x, x


def _run(pkv, k, v, ks, vs, table, ctx, cu, max_new, kn, vn, kind):
    tk, tv = dev(k), dev(v)
    tks, tvs = dev(ks), dev(vs)
    pkv.kv_append_fp8(tk, tv, tks, tvs, dev(table), dev(ctx), dev(cu), max_new, dev(kn, kind), dev(vn, kind))
    torch.cuda.synchronize()
    return tk.cpu().numpy(), tv.cpu().numpy(), tks.cpu().numpy(), tvs.cpu().numpy()


def _assert_same(got, want):
    gk, gv, gks, gvs = got
    wk, wv, wks, wvs = want
    assert np.array_equal(gks.view(np.uint32), wks.view(np.uint32)), "k scales differ"
    assert np.array_equal(gvs.view(np.uint32), wvs.view(np.uint32)), "v scales differ"
    for name, g, w in (("k", gk, wk), ("v", gv, wv)):
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{name} codes differ at {len(bad)} places, first {bad[:4].tolist()}"


@pytest.mark.parametrize("kind,d,n_kv", [("bf16", 128, 2), ("f32", 128, 8), ("bf16", 64, 4), ("f32", 64, 1)])
def test_append_fp8_ragged_batch(pkv, kind, d, n_kv):
    r = synth.rng(910, d, n_kv)
    ctx = np.array([0, 1, 15, 16, 17, 40, 100, 63, 5], np.int32)
    n_new = np.array([1, 0, 1, 33, 16, 50, 7, 20, 11], np.int32)
    batch, max_blocks = len(ctx), 12
    nb = batch * max_blocks + 7
    table = _tables(r, batch, max_blocks, nb)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    total = int(cu[-1])
    # per-sequence gains: some appends stay under the blocks' scales, some grow them
    gains = np.repeat(np.array([1.0, 1.0, 0.01, 3.0, 0.2, 1.0, 40.0, 0.001, 1.0], np.float32), n_new)
    kn, kf = _new_rows(r, total, n_kv, d, kind, gains)
    vn, vf = _new_rows(r, total, n_kv, d, kind, gains * 0.5)
    k = _random_codes(r, (nb, n_kv, B, d))
    v = _random_codes(r, (nb, n_kv, B, d))
    ks = (r.random((nb, n_kv)) * 0.02 + 1e-4).astype(np.float32)
    vs = (r.random((nb, n_kv)) * 0.02 + 1e-4).astype(np.float32)
    note(f"fp8 append ragged {kind} d={d} n_kv={n_kv} total={total}")
    got = _run(pkv, k, v, ks, vs, table, ctx, cu, int(n_new.max()), kn, vn, kind)
    want = oracle.kv_append_fp8(k, v, ks, vs, table, ctx, cu, kf, vf, B)
    _assert_same(got, want)
    # something happened in both directions: a scale grew, a scale stayed
    grew = got[2] > ks
    assert grew.any() and (got[2] == ks).any()


def _exhaustive_case(values: np.ndarray, n_kv: int, d: int):
    """One sequence with one cached row per KV head at scale 1.0 and 15 new
    rows holding `values` (padded with zeros); every |value| <= 448 keeps the
    scale at 1, so each code is the encoder's answer for the value itself."""
    per = 15 * n_kv * d
    assert values.size <= per
    x = np.zeros(per, np.float32)
    x[:values.size] = values
    x = x.reshape(15, n_kv, d)
    k = np.zeros((2, n_kv, B, d), np.uint8)
    ks = np.ones((2, n_kv), np.float32)
    table = np.array([[1, 0]], np.int32)
    ctx = np.array([1], np.int32)
    cu = np.array([0, 15], np.int32)
    return x, k, ks, table, ctx, cu


def test_encoder_every_bf16_value(pkv):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    bits = bits[keep]
    n_kv, d = 19, 128
    x, k, ks, table, ctx, cu = _exhaustive_case(oracle.bf16_bits_to_f64(bits).astype(np.float32), n_kv, d)
    xb = synth.encode(x, "bf16")
    assert np.array_equal(oracle.bf16_bits_to_f64(xb).astype(np.float32), x)
    note(f"fp8 encoder: {bits.size} bf16 values")
    got = _run(pkv, k, k.copy(), ks, ks.copy(), table, ctx, cu, 15, xb, xb, "bf16")
    want = oracle.kv_append_fp8(k, k.copy(), ks, ks.copy(), table, ctx, cu, x, x, B)
    _assert_same(got, want)
    assert np.all(got[2] == 1.0)


def test_encoder_f32_ties_and_neighbours(pkv):
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = oracle.e4m3fn_to_f64(codes).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1].astype(np.float64) + vals[1:]) / 2)
    cand = np.concatenate([vals, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                           np.nextafter(vals, np.float32(0)), np.nextafter(vals, np.float32(1e9))])
    r = synth.rng(911, 0, 0)
    rand = (r.random(20000) * 448).astype(np.float32) * np.float32(2.0) ** -r.integers(0, 14, 20000).astype(np.float32)
    cand = np.concatenate([cand, rand, np.float32([1e-30, 1e-12, 2.0 ** -10, 2.0 ** -10 * 1.0000001])])
    cand = cand[np.abs(cand) <= 448]
    cand = np.concatenate([cand, -cand]).astype(np.float32)
    n_kv, d = 24, 128
    x, k, ks, table, ctx, cu = _exhaustive_case(cand, n_kv, d)
    note(f"fp8 encoder: {cand.size} float32 values")
    got = _run(pkv, k, k.copy(), ks, ks.copy(), table, ctx, cu, 15, x, x, "f32")
    want = oracle.kv_append_fp8(k, k.copy(), ks, ks.copy(), table, ctx, cu, x, x, B)
    _assert_same(got, want)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_chunked_appends_then_decode(pkv, kind):
    """Three sequences fill an empty FP8 cache in steps of 1 .. 20 tokens
    (token by token for the first); after every step the caches match the
    oracle's bit for bit, and a decode over the final cache matches the
    oracle's attention over its own cache."""
    r = synth.rng(912, 0, 1 if kind == "bf16" else 2)
    n_kv, n_q, d = 2, 8, 128
    batch, max_blocks = 3, 6
    nb = 24
    table = _tables(r, batch, max_blocks, nb)
    k = np.zeros((nb, n_kv, B, d), np.uint8)
    v = k.copy()
    ks = np.zeros((nb, n_kv), np.float32)
    vs = ks.copy()
    tk, tv, tks, tvs = dev(k), dev(v), dev(ks), dev(vs)
    ttable = dev(table)
    lens = np.zeros(batch, np.int32)
    steps = 0
    while steps < 40:
        n_new = np.array([1, r.integers(0, 9), r.integers(1, 21)], np.int32)
        n_new = np.minimum(n_new, max_blocks * B - lens).astype(np.int32)
        if n_new.sum() == 0:
            break
        cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
        total = int(cu[-1])
        # later tokens are larger, so scales keep growing and blocks re-encode
        gains = np.float32(1.0 + 0.05 * steps) * np.ones(total, np.float32)
        kn, kf = _new_rows(r, total, n_kv, d, kind, gains)
        vn, vf = _new_rows(r, total, n_kv, d, kind, gains)
        pkv.kv_append_fp8(tk, tv, tks, tvs, ttable, dev(lens), dev(cu), int(n_new.max()), dev(kn, kind),
                          dev(vn, kind))
        k, v, ks, vs = oracle.kv_append_fp8(k, v, ks, vs, table, lens, cu, kf, vf, B)
        lens = lens + n_new
        steps += 1
    torch.cuda.synchronize()
    note(f"fp8 chunked appends {kind}: {steps} steps, lens {lens.tolist()}")
    _assert_same((tk.cpu().numpy(), tv.cpu().numpy(), tks.cpu().numpy(), tvs.cpu().numpy()), (k, v, ks, vs))
    q = synth.encode(r.standard_normal((batch, n_q, d)).astype(np.float32), "bf16")
    scale = synth.softmax_scale(d)
    out = pkv.paged_attn_decode(dev(q, "bf16"), tk, tv, ttable, dev(lens), n_q, n_kv, d, B, scale, k_scale=tks,
                                v_scale=tvs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want = oracle.paged_decode(q, "bf16", k, v, "fp8", ks, vs, table, lens, n_q, n_kv, scale)
    assert_parity(got, want, "fp8")


def test_skips_and_noops(pkv):
    """A sequence whose table names blocks outside the pool, one with a
    negative context length and one with no new rows change nothing; the valid
    sequence appends as the oracle says; max_new_len == 0 is a no-op."""
    r = synth.rng(913, 0, 0)
    n_kv, d, nb, max_blocks = 2, 64, 16, 4
    k = _random_codes(r, (nb, n_kv, B, d))
    v = _random_codes(r, (nb, n_kv, B, d))
    ks = (r.random((nb, n_kv)) * 0.02 + 1e-4).astype(np.float32)
    vs = ks.copy()
    table = np.array([[3, 7, 9, 2], [-1, nb, nb + 5, -7], [4, 5, 6, 8], [10, 11, 12, 13]], np.int32)
    ctx = np.array([9, 0, -1, 20], np.int32)
    n_new = np.array([20, 12, 5, 0], np.int32)
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    kn, kf = _new_rows(r, int(cu[-1]), n_kv, d, "bf16", np.ones(int(cu[-1]), np.float32))
    vn, vf = _new_rows(r, int(cu[-1]), n_kv, d, "bf16", np.ones(int(cu[-1]), np.float32))
    note("fp8 append skips")
    got = _run(pkv, k, v, ks, vs, table, ctx, cu, 20, kn, vn, "bf16")
    want = oracle.kv_append_fp8(k, v, ks, vs, table[:1], ctx[:1], cu[:2], kf[:20], vf[:20], B)
    _assert_same(got, want)
    got0 = _run(pkv, k, v, ks, vs, table, ctx, cu, 0, kn, vn, "bf16")
    _assert_same(got0, (k, v, ks, vs))
