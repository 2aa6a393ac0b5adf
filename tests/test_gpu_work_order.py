"""GPU checks of the decode work order: pkv_paged_attn_decode_order writes the
length ranking (pairing long with short, or longest first) or, for a split
with several partitions per sequence, the (sequence, partition) units ranked by
tokens followed by -1s; decode with any such order gives bit-identical outputs
to plain decode."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_parity, dev, note, oracle_decode, upload_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def _expected(lens):
    n = len(lens)
    desc = sorted(range(n), key=lambda t: (-max(int(lens[t]), 0), t))
    half = (n + 1) // 2
    pair = [desc[q] if q < half else desc[n - 1 - (q - half)] for q in range(n)]
    return desc, pair


def _expected_units(lens, n_parts, part_tokens):
    tok = {s * n_parts + p: min(max(int(lens[s]) - p * part_tokens, 0), part_tokens)
           for s in range(len(lens)) for p in range(n_parts)}
    ranked = sorted(tok, key=lambda u: (-tok[u], u))
    return [u if tok[u] > 0 else -1 for u in ranked]


@pytest.mark.parametrize("batch,max_len", [(1, 3000), (2, 3000), (7, 3000), (64, 3000), (256, 3000), (1000, 3000),
                                           (64, 9000), (256, 8192)])
def test_order_is_the_length_ranking(pkv, batch, max_len):
    r = np.random.default_rng(970 + batch + max_len)
    lens = r.integers(0, max_len, size=batch).astype(np.int32)
    lens[::5] = lens[0]  # ties
    mb = max_len // 16 + 1
    note(f"decode order batch={batch} max_len={max_len}")
    got = pkv.paged_attn_decode_order(dev(lens), 32, 8, 128, mb, 16, pkv.BF16).cpu().tolist()
    plan = pkv.paged_attn_decode_plan(batch, 32, 8, 128, mb, 16, pkv.BF16)
    if len(got) == batch:
        desc, pair = _expected(lens)
        assert got == desc or got == pair
    else:
        # several partitions per sequence: the unit order
        assert plan["n_parts"] > 1 and len(got) == batch * plan["n_parts"]
        assert got == _expected_units(lens, plan["n_parts"], plan["partition_tokens"])


@pytest.mark.parametrize("kind,d,n_q,n_kv", [("bf16", 128, 32, 8), ("fp8", 128, 64, 8), ("f32", 64, 8, 2)])
def test_ordered_decode_is_bit_identical(pkv, kind, d, n_q, n_kv):
    lens = [1, 5000, 17, 300, 9000, 2048, 0, 777, 4097, 64]
    c = synth.make_decode_case(config=971, layer=0, n_q=n_q, n_kv=n_kv, d=d, seq_lens=lens, kv_dtype=kind)
    t = upload_decode(c)
    def run(order=None):
        out = pkv.paged_attn_decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"], n_q, n_kv, d,
                                    16, c.scale, k_scale=t["k_scale"], v_scale=t["v_scale"], work_order=order)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    note(f"ordered decode {kind}")
    plain = run()
    lib_order = pkv.paged_attn_decode_order(t["seq_lens"], n_q, n_kv, d, c.block_table.shape[1], 16,
                                            pkv.dtype_code(t["k_cache"]))
    n = lib_order.numel()  # sequences, or (sequence, partition) units
    assert n == len(lens) or n % len(lens) == 0
    rand = torch.from_numpy(np.random.default_rng(5).permutation(n).astype(np.int32)).cuda()
    ident = torch.arange(n, dtype=torch.int32, device="cuda")
    ordered = run(lib_order)
    # the order only moves work between workgroups: the same bits for every
    # permutation (a unit list may name empty units too: they exit)
    for o in (rand, ident):
        assert np.array_equal(run(o).view(np.uint32), ordered.view(np.uint32))
    want = oracle_decode(c)
    assert np.array_equal(plain.view(np.uint32), ordered.view(np.uint32))  # same split, same bits
    for got in (plain, ordered):
        assert_parity(got.astype(np.float64), want, kind)


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_single_long_sequence_fills_the_device(pkv, kind):
    """One 20000-token sequence: the split spreads it over every resident
    workgroup slot (not just a few 4096-token partitions) and still matches
    the oracle."""
    c = synth.make_decode_case(config=972, layer=0, n_q=32, n_kv=8, d=128, seq_lens=[20000], kv_dtype=kind)
    plan = pkv.paged_attn_decode_plan(1, 32, 8, 128, c.block_table.shape[1], 16, pkv.BF16 if kind == "bf16"
                                      else pkv.FP8_E4M3FN)
    note(f"single long sequence {kind}: {plan}")
    assert plan["workgroups"] >= 256 and plan["n_parts"] > 5
    t = upload_decode(c)
    out = pkv.paged_attn_decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"], 32, 8, 128, 16,
                                c.scale, k_scale=t["k_scale"], v_scale=t["v_scale"])
    torch.cuda.synchronize()
    want = oracle_decode(c)
    assert_parity(out.cpu().numpy().astype(np.float64), want, kind, "20000 tokens")


def test_work_order_entries(pkv):
    """Size of the work order on the device: one entry per sequence when each
    sequence is one partition, one per (sequence, partition) unit when the
    matrix-core split cuts sequences into several (up to 8192 units)."""
    lib = pkv.load()
    assert lib.pkv_paged_attn_decode_order_entries(64, 32, 8, 128, 128, 16, pkv.BF16) == 64          # 2048 tokens
    assert lib.pkv_paged_attn_decode_order_entries(256, 64, 8, 128, 512, 16, pkv.FP8_E4M3FN) == 512  # 8192: 2 parts
    assert lib.pkv_paged_attn_decode_order_entries(8, 64, 8, 128, 2048, 16, pkv.BF16) == 64          # 32768: 8 parts
    assert lib.pkv_paged_attn_decode_order_entries(2048, 64, 8, 128, 512, 16, pkv.BF16) == 4096     # 2 parts
    assert lib.pkv_paged_attn_decode_order_entries(8192, 64, 8, 128, 512, 16, pkv.BF16) == 8192     # > 8192 units
    assert lib.pkv_paged_attn_decode_order_entries(4, 6, 4, 128, 8, 16, pkv.BF16) == 0              # head ratio
