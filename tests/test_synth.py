"""The seeded input generators: encoders against library casts, pools,
tables and the five workload recipes.  CPU only."""
import numpy as np
import torch

import oracle
import synth


def test_bf16_encoder_matches_torch_rne():
    x = np.random.default_rng(1).standard_normal(200_000).astype(np.float32) * np.float32(1e3)
    x[:4] = [0.0, -0.0, 3.0e38, 1e-40]
    got = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert synth.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0] == 0x7FC0


def test_e4m3_encoder_matches_torch_and_saturates():
    r = np.random.default_rng(2)
    x = np.concatenate([r.standard_normal(100_000) * 100, r.uniform(-448, 448, 100_000),
                        r.standard_normal(10_000) * 1e-3]).astype(np.float32)
    got = synth.f32_to_e4m3fn(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inside = np.abs(x) < 464  # torch's cast gives NaN above the rounding range; ours saturates
    assert np.array_equal(got[inside], ref[inside])
    assert np.all(got[~inside] & 0x7F == 0x7E)
    assert list(synth.f32_to_e4m3fn(np.array([1e6, -1e6, 464.0, 447.0], dtype=np.float32))) == [0x7E, 0xFE, 0x7E, 0x7E]
    assert synth.f32_to_e4m3fn(np.array([np.nan]))[0] == 0x7F


def test_e4m3_round_trip_and_ties_to_even():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    vals = oracle.e4m3fn_to_f64(codes)
    assert np.array_equal(synth.f32_to_e4m3fn(vals), codes)
    # halfway between 1.0 (0x38) and 1.125 (0x39) -> even mantissa 0x38; 1.1875 -> 0x3A
    assert list(synth.f32_to_e4m3fn(np.array([1.0625, 1.1875]))) == [0x38, 0x3A]
    # subnormal halfway 1.5 * 2^-9 -> 2 * 2^-9 (0x02); 0.5 * 2^-9 -> 0
    assert list(synth.f32_to_e4m3fn(np.array([1.5 * 2 ** -9, 0.5 * 2 ** -9]))) == [0x02, 0x00]


def test_fp8_scales_are_blockwise_maxabs_over_filled_slots():
    x = np.zeros((3, 2, 16, 4), dtype=np.float32)
    x[0, 0, 3, 1] = -896.0
    x[0, 1, 0, 0] = 4.48
    x[1, 0, 15, 3] = 1e9      # an unfilled slot: ignored
    filled = np.zeros((3, 16), dtype=bool)
    filled[0, :] = True
    filled[1, :8] = True
    s = synth.fp8_block_scales(x, filled)
    assert s[0, 0] == np.float32(2.0) and s[0, 1] == np.float32(0.01)
    assert s[1, 0] == 1.0 and s[2, 1] == 1.0
    codes = synth.quantize_fp8(x, s)
    assert codes[0, 0, 3, 1] == 0xFE  # -448


def test_tables_take_consecutive_chunks_of_the_permutation():
    perm = np.array([5, 3, 0, 7, 1, 2, 6, 4], dtype=np.int32)
    table, filled = synth.build_tables([17, 3, 32], 8, perm, 16)
    assert table.tolist() == [[5, 3], [0, -1], [7, 1]]
    assert filled[5].all() and filled[3, :1].all() and not filled[3, 1:].any()
    assert filled[0, :3].all() and not filled[0, 3:].any()
    assert not filled[[2, 6, 4]].any()


def test_workload_recipes():
    c1 = synth.config_decode_case(1)
    assert c1.seq_lens.tolist() == [37, 100] and c1.num_blocks == 64
    assert (c1.block_table >= 0).sum() == 3 + 7
    used = set(c1.block_table[c1.block_table >= 0].tolist())
    unused = [b for b in range(64) if b not in used]
    assert np.isnan(c1.k_cache[unused]).all()
    assert c1.scale == np.float32(1 / 8)
    l2 = synth.config_seq_lens(2)
    assert l2.shape == (64,) and l2.min() >= 1024 and l2.max() <= 2048
    assert 1400 < l2.mean() < 1700
    l4 = synth.config_seq_lens(4)
    assert l4.shape == (256,) and l4.min() >= 16 and l4.max() <= 8192
    assert 700 < np.median(l4) < 1400
    l5 = synth.config_seq_lens(5)
    assert l5.shape == (16,) and l5.min() >= 0 and l5.max() <= 8192


def test_prefill_case_layout():
    p = synth.make_prefill_case(config=7, layer=0, n_q=4, n_kv=2, d=8, context_lens=[0, 21], q_len=[5, 12],
                                chunk_in_cache=False)
    assert p.cu_q_lens.tolist() == [0, 5, 17]
    assert p.positions.tolist() == list(range(5)) + list(range(21, 33))
    assert p.seq_ids.tolist() == [0] * 5 + [1] * 12
    # chunk rows are poisoned in the cache until appended
    b = p.block_table[1, 21 // 16]
    assert (p.k_cache[b, :, 21 % 16] == synth.POISON["bf16"]).all()
    assert not (p.k_cache[b, :, 20 % 16] == synth.POISON["bf16"]).all()
