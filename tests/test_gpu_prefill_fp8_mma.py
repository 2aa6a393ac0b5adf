"""GPU parity of the chunked prefill whose two products run in FP8
(pkv_paged_attn_prefill_chunk_fp8_mma), against the float64 oracle on the
dequantised cache.

split=True (queries and softmax weights each carried as two E4M3 terms, the
remainder's rounding leaving about 2^-8 of each value) is held to the FP8 bar
of the widened path: max-abs 5e-2 and per-row relative error 5e-3.

split=False (one E4M3 term each, FlashAttention-3's FP8 scheme) does not meet
that bar: each query element and each weight is rounded by up to 2^-4 of
itself (rms 2^-4 / sqrt(3) = 3.6e-2 over a binade), and a row's output moves
by about that fraction of its size whatever its length.  Its test checks that
the error is of that size and no larger: median row error <= 5e-2, every row
<= 0.15, max-abs <= 0.25 (a wrong key, scale or mask moves rows by O(1)).

Where the result is fixed exactly (one visible key), both modes give it.  Each
test also prints the error of the widened-bf16 path on the same inputs: the
price of the quantisation."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_parity, dev, err_report, note, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def _inputs(p, k_scale=None, v_scale=None, v_cache=None):
    return dict(q=dev(p.q, "bf16"), cu=dev(p.cu_q_lens), ctx=dev(p.context_lens), k=dev(p.k_cache),
                v=dev(p.v_cache if v_cache is None else v_cache), tb=dev(p.block_table),
                ks=dev(p.k_scale if k_scale is None else k_scale), vs=dev(p.v_scale if v_scale is None else v_scale))


def _run(pkv, p, t, causal=True, mma=True, out_dtype=torch.float32, split=True):
    ql = int(np.diff(p.cu_q_lens).max())
    kw = dict(causal=causal, k_scale=t["ks"], v_scale=t["vs"], out_dtype=out_dtype)
    if mma:
        out = pkv.paged_attn_prefill_chunk_fp8_mma(t["q"], t["cu"], t["ctx"], ql, t["k"], t["v"], t["tb"], p.n_q,
                                                   p.n_kv, p.d, p.block_size, p.scale, split=split, **kw)
    else:
        out = pkv.paged_attn_prefill_chunk(t["q"], t["cu"], t["ctx"], ql, t["k"], t["v"], t["tb"], p.n_q, p.n_kv,
                                           p.d, p.block_size, p.scale, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _oracle(p, causal=True, k_scale=None, v_scale=None, v_cache=None):
    return oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, p.k_cache,
                                p.v_cache if v_cache is None else v_cache, "fp8",
                                p.k_scale if k_scale is None else k_scale, p.v_scale if v_scale is None else v_scale,
                                p.block_table, p.n_q, p.n_kv, p.scale, causal=causal)


def _check(pkv, p, t, want, causal=True, label=""):
    got = _run(pkv, p, t, causal)
    widened = _run(pkv, p, t, causal, mma=False)
    note(f"  {label} widened-bf16 path: {err_report(widened, want)}")
    return assert_parity(got, want, "fp8", f"{label} fp8 products (split):")


def _check_single(got, want, label=""):
    """split=False: errors of the size one E4M3 rounding gives, and no larger."""
    rep = err_report(got, want)
    note(f"  {label} fp8 products (one term): {rep}")
    r = row_rel_err(got, want)
    assert np.all(np.isfinite(got)), rep
    assert float(np.median(r)) <= 5e-2 and float(r.max()) <= 0.15, rep
    assert float(np.max(np.abs(got - want))) <= 0.25, rep


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (16, 2), (8, 1), (64, 8), (128, 1)])
def test_fp8_mma_ragged(pkv, causal, n_q, n_kv):
    ctx = [0, 5, 16, 37, 300, 1000]
    ql = [7, 1, 33, 128, 200, 65]
    p = synth.make_prefill_case(config=420, layer=n_q + n_kv, n_q=n_q, n_kv=n_kv, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype="fp8")
    note(f"fp8 products n_q={n_q} n_kv={n_kv} causal={causal}")
    t, want = _inputs(p), _oracle(p, causal)
    _check(pkv, p, t, want, causal)
    _check_single(_run(pkv, p, t, causal, split=False), want)


@pytest.mark.parametrize("block_size", [8, 32, 256])
def test_fp8_mma_block_sizes(pkv, block_size):
    ctx = [3, 130, 700]
    ql = [40, 129, 17]
    p = synth.make_prefill_case(config=421, layer=block_size, n_q=32, n_kv=8, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype="fp8", block_size=block_size)
    note(f"fp8 products block_size={block_size}")
    _check(pkv, p, _inputs(p), _oracle(p))


def test_fp8_mma_long_context(pkv):
    """A 512-token chunk behind 3.5K tokens of context: many 128-key tiles,
    so the error of the weights' sums over a long row shows."""
    p = synth.make_prefill_case(config=422, layer=0, n_q=64, n_kv=8, d=128, context_lens=[3584, 0], q_len=[512, 300],
                                kv_dtype="fp8")
    note("fp8 products, 3.5K context + 512 chunk")
    _check(pkv, p, _inputs(p), _oracle(p))


def test_fp8_mma_one_key_is_exact(pkv):
    """With no context, the first query token of a causal chunk sees one key:
    its output is that key's dequantised V row (the weights' sum holds the
    quantised weight itself), up to fp32 rounding."""
    p = synth.make_prefill_case(config=423, layer=0, n_q=32, n_kv=8, d=128, context_lens=[0, 0, 0], q_len=[1, 20, 130],
                                kv_dtype="fp8")
    t, want = _inputs(p), _oracle(p)
    first = p.cu_q_lens[:-1]
    for split in (True, False):
        got = _run(pkv, p, t, split=split)
        note(f"one key, split={split}: {err_report(got[first], want[first])}")
        np.testing.assert_allclose(got[first], want[first], rtol=1e-5, atol=1e-6)
    got = _run(pkv, p, t)
    assert_parity(got, want, "fp8", "fp8 products (split):")


def test_fp8_mma_zero_and_small_v_blocks(pkv):
    """Blocks whose V rows are zero (scale 0, zero codes, as the FP8 append
    writes them) and blocks of tiny V (scale 2^-12 of the others): their keys
    carry softmax weight that the row sum must count, though their weights in
    the value product vanish."""
    p = synth.make_prefill_case(config=424, layer=0, n_q=32, n_kv=8, d=128, context_lens=[64, 500], q_len=[64, 100],
                                kv_dtype="fp8")
    vs = p.v_scale.copy()
    vc = p.v_cache.copy()
    used = np.unique(p.block_table[p.block_table >= 0])
    zero_blocks, small_blocks = used[::3], used[1::5]
    vs[zero_blocks] = 0.0
    vc[zero_blocks] = 0
    vs[small_blocks] *= np.float32(2.0 ** -12)
    t = _inputs(p, v_scale=vs, v_cache=vc)
    want = _oracle(p, v_scale=vs, v_cache=vc)
    note(f"{zero_blocks.size} zero V blocks, {small_blocks.size} tiny V blocks")
    _check(pkv, p, t, want)
    _check_single(_run(pkv, p, t, split=False), want)


def test_fp8_mma_bf16_output_and_heads(pkv):
    p = synth.make_prefill_case(config=425, layer=0, n_q=40, n_kv=5, d=128, context_lens=[10, 77], q_len=[50, 3],
                                kv_dtype="fp8")
    t = _inputs(p)
    got = _run(pkv, p, t, out_dtype=torch.bfloat16)
    want = _oracle(p)
    # bf16 output rounding adds up to 2^-9 of each value
    assert_parity(got, want, "fp8", "bf16 out:", rel=1e-2)


def test_fp8_mma_after_fp8_append(pkv):
    """Chunk rows quantised into the cache by kv_append_fp8, then attended
    through the FP8 products; the oracle appends and attends in float64."""
    ctx = [0, 9, 40, 250]
    ql = [20, 64, 3, 130]
    p = synth.make_prefill_case(config=426, layer=0, n_q=32, n_kv=8, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype="fp8", chunk_in_cache=False)
    r = synth.rng(426, 0, 99)
    total = int(p.cu_q_lens[-1])
    kb = synth.encode(r.standard_normal((total, p.n_kv, p.d)).astype(np.float32) * 2, "bf16")
    vb = synth.encode(r.standard_normal((total, p.n_kv, p.d)).astype(np.float32), "bf16")
    kf = oracle.bf16_bits_to_f64(kb).astype(np.float32)
    vf = oracle.bf16_bits_to_f64(vb).astype(np.float32)
    t = _inputs(p)
    pkv.kv_append_fp8(t["k"], t["v"], t["ks"], t["vs"], t["tb"], t["ctx"], t["cu"], int(max(ql)), dev(kb, "bf16"),
                      dev(vb, "bf16"))
    k, v, ks, vs = oracle.kv_append_fp8(p.k_cache, p.v_cache, p.k_scale, p.v_scale, p.block_table, p.context_lens,
                                        p.cu_q_lens, kf, vf, 16)
    torch.cuda.synchronize()
    assert np.array_equal(t["k"].cpu().numpy(), k) and np.array_equal(t["v"].cpu().numpy(), v)
    want = oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, k, v, "fp8", ks, vs, p.block_table, p.n_q,
                                p.n_kv, p.scale, causal=True)
    note("fp8 append then fp8 products")
    _check(pkv, p, t, want)


def test_fp8_mma_many_sequences(pkv):
    """More sequences than the kernel ranks in LDS: plain sequence order."""
    r = np.random.default_rng(428)
    ctx = r.integers(0, 60, size=300).tolist()
    ql = r.integers(1, 12, size=300).tolist()
    p = synth.make_prefill_case(config=428, layer=0, n_q=8, n_kv=2, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype="fp8")
    note("fp8 products over 300 short sequences")
    _check(pkv, p, _inputs(p), _oracle(p))


def test_fp8_mma_rejects_bf16_cache(pkv):
    p = synth.make_prefill_case(config=427, layer=0, n_q=8, n_kv=8, d=128, context_lens=[4], q_len=[4])
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_prefill_chunk_fp8_mma(dev(p.q, "bf16"), dev(p.cu_q_lens), dev(p.context_lens), 4,
                                             dev(p.k_cache, "bf16"), dev(p.v_cache, "bf16"), dev(p.block_table), 8, 8,
                                             128, 16, p.scale, k_scale=None, v_scale=None)
    assert e.value.status == pkv.ERR_UNSUPPORTED
