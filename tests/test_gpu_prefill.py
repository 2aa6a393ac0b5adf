"""GPU parity of chunked prefill (MFMA path) and append-then-attend."""
import dataclasses

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


def _run(pkv, p, causal=True, k_cache=None, v_cache=None, out_dtype=torch.float32):
    kc = dev(p.k_cache, "bf16") if k_cache is None else k_cache
    vc = dev(p.v_cache, "bf16") if v_cache is None else v_cache
    q_lens = np.diff(p.cu_q_lens)
    out = pkv.paged_attn_prefill_chunk(dev(p.q, "bf16"), dev(p.cu_q_lens), dev(p.context_lens), int(q_lens.max()),
                                       kc, vc, dev(p.block_table), p.n_q, p.n_kv, p.d, 16, p.scale, causal=causal,
                                       out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _oracle(p, causal=True):
    return oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, "bf16", None, None,
                                p.block_table, p.n_q, p.n_kv, p.scale, causal=causal)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (8, 8), (16, 2), (8, 1), (64, 1), (128, 1)])
def test_prefill_ragged(pkv, causal, n_q, n_kv):
    ctx = [0, 5, 16, 37, 300, 1000]
    ql = [7, 1, 33, 128, 200, 65]
    p = synth.make_prefill_case(config=400, layer=n_q + n_kv, n_q=n_q, n_kv=n_kv, d=128, context_lens=ctx, q_len=ql)
    note(f"prefill n_q={n_q} n_kv={n_kv} causal={causal}")
    got = _run(pkv, p, causal)
    want = _oracle(p, causal)
    assert_parity(got, want, "bf16")


def test_prefill_long_chunks(pkv):
    """Chunks of thousands of tokens (a whole prompt at once: 86 query tiles of
    one sequence, with and without context before it), where the ordering of
    query tiles and their placement over the XCDs span many workgroups per
    (sequence, KV head)."""
    p = synth.make_prefill_case(config=983, layer=0, n_q=8, n_kv=2, d=128, context_lens=[0, 1000],
                                q_len=[4096, 2000])
    note("prefill chunks of 4096 (no context) and 2000 (after 1000) tokens")
    assert_parity(_run(pkv, p), _oracle(p), "bf16", "long chunks:")


def test_prefill_many_sequences(pkv):
    """More sequences than the kernels rank by length in LDS (256): the work
    order falls back to plain sequence order, with the same results."""
    r = np.random.default_rng(984)
    ctx = r.integers(0, 60, size=300).tolist()
    ql = r.integers(1, 12, size=300).tolist()
    p = synth.make_prefill_case(config=984, layer=0, n_q=8, n_kv=2, d=128, context_lens=ctx, q_len=ql)
    note("prefill over 300 short sequences")
    assert_parity(_run(pkv, p), _oracle(p), "bf16", "300 sequences:")


def test_prefill_chunk_of_one_matches_decode(pkv):
    p = synth.make_prefill_case(config=401, layer=0, n_q=32, n_kv=8, d=128, context_lens=[37, 500, 0], q_len=1)
    got = _run(pkv, p)
    dec = pkv.paged_attn_decode(dev(p.q, "bf16"), dev(p.k_cache, "bf16"), dev(p.v_cache, "bf16"), dev(p.block_table),
                                dev(p.context_lens + 1), p.n_q, p.n_kv, p.d, 16, p.scale)
    torch.cuda.synchronize()
    want = _oracle(p)
    d = dec.float().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - want)) <= 1e-2 and np.max(np.abs(d - want)) <= 1e-2
    assert np.max(np.abs(got - d)) <= 1e-2


def test_append_then_attend(pkv):
    """kv_append writes the chunk's rows (bit-exact), then prefill attends them."""
    p = synth.make_prefill_case(config=402, layer=0, n_q=32, n_kv=8, d=128, context_lens=[0, 100, 1234],
                                q_len=[64, 100, 512], chunk_in_cache=False)
    full = synth.make_prefill_case(config=402, layer=0, n_q=32, n_kv=8, d=128, context_lens=[0, 100, 1234],
                                   q_len=[64, 100, 512], chunk_in_cache=True)
    kc, vc = dev(p.k_cache, "bf16"), dev(p.v_cache, "bf16")
    tb = dev(p.block_table)
    note("append then attend")
    slots = pkv.slot_mapping(tb, dev(p.seq_ids), dev(p.positions), 16)
    pkv.kv_append(kc, vc, slots, dev(p.k_new, "bf16"), dev(p.v_new, "bf16"))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(kc), full.k_cache) and np.array_equal(host_bits(vc), full.v_cache)
    got = _run(pkv, p, k_cache=kc, v_cache=vc)
    want = _oracle(full)
    assert_parity(got, want, "bf16")


def test_prefill_bf16_output(pkv):
    p = synth.make_prefill_case(config=403, layer=0, n_q=32, n_kv=8, d=128, context_lens=[10, 70], q_len=[50, 3])
    want = _oracle(p)
    got = _run(pkv, p, out_dtype=torch.bfloat16)
    assert np.max(np.abs(got - want)) <= 1e-2 + 2 ** -8 * np.max(np.abs(want))


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_wide_score_range(pkv, causal):
    """Scores whose row maxima keep climbing along the keys (q x 4, key rows
    scaled up to 4x with position), so the running reference max moves many
    times mid-sequence and the accumulators are rescaled on those moves."""
    ctx = [3000, 517, 64]
    p = synth.make_prefill_case(config=404, layer=int(causal), n_q=32, n_kv=8, d=128, context_lens=ctx,
                                q_len=[200, 90, 64])
    q = synth.f32_to_bf16_bits((oracle.bf16_bits_to_f64(p.q) * 4.0).astype(np.float32))
    kc = oracle.bf16_bits_to_f64(p.k_cache)
    for s, L in enumerate(np.asarray(ctx) + np.diff(p.cu_q_lens)):
        for j in range(synth.blocks_for(int(L))):
            b = p.block_table[s, j]
            pos = j * 16 + np.arange(16)
            kc[b] *= (1.0 + 3.0 * pos / L)[None, :, None]
    p = dataclasses.replace(p, q=q, k_cache=synth.f32_to_bf16_bits(kc.astype(np.float32)))
    note(f"prefill wide score range causal={causal}")
    got = _run(pkv, p, causal)
    want = _oracle(p, causal)
    assert_parity(got, want, "bf16")


def test_prefill_sequence_without_new_tokens(pkv):
    """A sequence with no new tokens in the chunk leaves no output rows and
    does not disturb its neighbours."""
    p = synth.make_prefill_case(config=405, layer=0, n_q=32, n_kv=8, d=128, context_lens=[40, 300, 7],
                                q_len=[33, 0, 20])
    got = _run(pkv, p)
    want = _oracle(p)
    assert got.shape[0] == 53
    assert_parity(got, want, "bf16")


# ---- FP8 KV (codes widened to bf16 in LDS, per-block K/V scales)

def _run_fp8(pkv, p, causal=True, k_cache=None, v_cache=None, k_scale=None, v_scale=None):
    q_lens = np.diff(p.cu_q_lens)
    out = pkv.paged_attn_prefill_chunk(
        dev(p.q, "bf16"), dev(p.cu_q_lens), dev(p.context_lens), int(q_lens.max()),
        dev(p.k_cache) if k_cache is None else k_cache, dev(p.v_cache) if v_cache is None else v_cache,
        dev(p.block_table), p.n_q, p.n_kv, p.d, 16, p.scale, causal=causal,
        k_scale=dev(p.k_scale) if k_scale is None else k_scale,
        v_scale=dev(p.v_scale) if v_scale is None else v_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (16, 2), (8, 1), (64, 8)])
def test_prefill_fp8_ragged(pkv, causal, n_q, n_kv):
    ctx = [0, 5, 16, 37, 300, 1000]
    ql = [7, 1, 33, 128, 200, 65]
    p = synth.make_prefill_case(config=402, layer=n_q + n_kv, n_q=n_q, n_kv=n_kv, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype="fp8")
    note(f"prefill fp8 n_q={n_q} n_kv={n_kv} causal={causal}")
    got = _run_fp8(pkv, p, causal)
    want = oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, p.k_cache, p.v_cache, "fp8", p.k_scale,
                                p.v_scale, p.block_table, p.n_q, p.n_kv, p.scale, causal=causal)
    assert_parity(got, want, "fp8")


def test_fp8_append_then_prefill(pkv):
    """A chunk of bf16 K/V rows is quantised into an FP8 cache that already
    holds each sequence's context (kv_append_fp8), then attended; the oracle
    runs the same two steps.  Caches must agree bit for bit, outputs within
    the FP8 tolerance."""
    ctx = [0, 9, 40, 250]
    ql = [20, 64, 3, 130]
    p = synth.make_prefill_case(config=403, layer=0, n_q=32, n_kv=8, d=128, context_lens=ctx, q_len=ql,
                                kv_dtype="fp8", chunk_in_cache=False)
    r = synth.rng(403, 0, 99)
    total = int(p.cu_q_lens[-1])
    kb = synth.encode(r.standard_normal((total, p.n_kv, p.d)).astype(np.float32) * 2, "bf16")
    vb = synth.encode(r.standard_normal((total, p.n_kv, p.d)).astype(np.float32), "bf16")
    kf = oracle.bf16_bits_to_f64(kb).astype(np.float32)
    vf = oracle.bf16_bits_to_f64(vb).astype(np.float32)
    tk, tv, tks, tvs = dev(p.k_cache), dev(p.v_cache), dev(p.k_scale), dev(p.v_scale)
    table = dev(p.block_table)
    pkv.kv_append_fp8(tk, tv, tks, tvs, table, dev(p.context_lens), dev(p.cu_q_lens), int(max(ql)), dev(kb, "bf16"),
                      dev(vb, "bf16"))
    k, v, ks, vs = oracle.kv_append_fp8(p.k_cache, p.v_cache, p.k_scale, p.v_scale, p.block_table, p.context_lens,
                                        p.cu_q_lens, kf, vf, 16)
    torch.cuda.synchronize()
    assert np.array_equal(tk.cpu().numpy(), k) and np.array_equal(tv.cpu().numpy(), v)
    assert np.array_equal(tks.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(tvs.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    note("fp8 append then prefill")
    got = _run_fp8(pkv, p, True, tk, tv, tks, tvs)
    want = oracle.paged_prefill(p.q, "bf16", p.cu_q_lens, p.context_lens, k, v, "fp8", ks, vs, p.block_table, p.n_q,
                                p.n_kv, p.scale, causal=True)
    assert_parity(got, want, "fp8")
