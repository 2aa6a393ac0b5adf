"""The C-ABI library: it loads, exports every symbol include/pkv.h declares,
and rejects bad arguments on the host before any launch.  No GPU needed: every
call here fails validation (or is host-only arithmetic)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")
LIB = os.path.join(ROOT, "paged_kv_cache_blocks_amd", "libpkv.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpkv.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    return p


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_binding_signatures_cover_the_header(pkv):
    assert set(pkv._SIGS) == set(_declared())


def test_version_and_status_strings(pkv):
    hdr = open(HEADER).read()
    assert pkv.abi_version() == int(re.search(r"#define PKV_ABI_VERSION (\d+)", hdr).group(1))
    lib = pkv.load()
    names = [lib.pkv_status_string(i).decode() for i in range(6)]
    assert names == ["PKV_OK", "PKV_ERR_INVALID_ARG", "PKV_ERR_UNSUPPORTED", "PKV_ERR_WORKSPACE", "PKV_ERR_HIP",
                     "PKV_ERR_NO_BLOCKS"]


def test_bytes_per_token_formula(pkv):
    # 128 KiB (Llama3-8B shape, fp16) and 320 KiB (70B shape, bf16) per token
    assert pkv.kv_bytes_per_token(32, 8, 128, 2) == 128 * 1024
    assert pkv.kv_bytes_per_token(80, 8, 128, 2) == 320 * 1024
    assert pkv.kv_bytes_per_token(80, 8, 128, 1) == 160 * 1024
    assert pkv.kv_bytes_per_token(-1, 8, 128, 2) == -1


def _decode(lib, **kw):
    a = dict(out=0x1000, out_dtype=0, q=0x1000, q_dtype=1, k=0x1000, v=0x1000, kv_dtype=1, ks=None, vs=None,
             table=0x1000, max_blocks=8, seq_lens=0x1000, batch=2, num_blocks=16, n_q=8, n_kv=2, d=128, bs=16,
             scale=0.088, part=0, ws=None, ws_n=0, stream=None)
    a.update(kw)
    return lib.pkv_paged_attn_decode_partitioned(a["out"], a["out_dtype"], a["q"], a["q_dtype"], a["k"], a["v"],
                                                 a["kv_dtype"], a["ks"], a["vs"], a["table"], a["max_blocks"],
                                                 a["seq_lens"], a["batch"], a["num_blocks"], a["n_q"], a["n_kv"],
                                                 a["d"], a["bs"], a["scale"], a["part"], a["ws"], a["ws_n"],
                                                 a["stream"])


def test_decode_validation_before_launch(pkv):
    lib = pkv.load()
    # the head ratio is checked first ("validate before mutate")
    assert _decode(lib, n_q=6, n_kv=4, out=None) == pkv.ERR_INVALID_ARG
    assert b"do not split evenly" in lib.pkv_last_error()
    assert _decode(lib, n_kv=0) == pkv.ERR_INVALID_ARG
    assert _decode(lib, q=None) == pkv.ERR_INVALID_ARG
    assert _decode(lib, d=96) == pkv.ERR_UNSUPPORTED
    assert _decode(lib, bs=24) == pkv.ERR_UNSUPPORTED               # block sizes: powers of two 8 .. 256
    assert _decode(lib, bs=512) == pkv.ERR_UNSUPPORTED
    assert _decode(lib, bs=4) == pkv.ERR_UNSUPPORTED
    assert _decode(lib, q_dtype=0) == pkv.ERR_UNSUPPORTED          # f32 q with bf16 KV
    assert _decode(lib, kv_dtype=2) == pkv.ERR_INVALID_ARG         # fp8 without scales
    assert _decode(lib, scale=0.0) == pkv.ERR_INVALID_ARG
    assert _decode(lib, part=100) == pkv.ERR_INVALID_ARG
    # 8 blocks * 16 = 128 tokens -> a single partition, no workspace; 4096-token tables need one
    need = pkv.paged_attn_decode_workspace(2, 8, 2, 128, 256, 16, pkv.BF16, 256)
    assert need > 0
    assert _decode(lib, max_blocks=256, part=256, ws=0x1000, ws_n=need - 1) == pkv.ERR_WORKSPACE
    assert _decode(lib, max_blocks=256, part=256, ws=0x1001, ws_n=need) == pkv.ERR_INVALID_ARG  # misaligned


def test_csr_entry_points_validate(pkv):
    lib = pkv.load()
    # decode: no indptr; unsupported block size; row space beyond 2^32
    args = [0x1000, 0, 0x2000, 1, 0x3000, 0x4000, 1, None, None, 0x5000, 0x6000, 4, 0x7000, 2, 64, 8, 2, 128, 16,
            0.088, None, 0, None]
    a = list(args); a[9] = None
    assert lib.pkv_paged_attn_decode_csr(*a) == pkv.ERR_INVALID_ARG
    a = list(args); a[18] = 12
    assert lib.pkv_paged_attn_decode_csr(*a) == pkv.ERR_UNSUPPORTED
    a = list(args); a[14] = 1 << 28; a[18] = 256
    assert lib.pkv_paged_attn_decode_csr(*a) == pkv.ERR_UNSUPPORTED
    # prefill: fp8 without scales, block size, empty chunk is a no-op
    pargs = [0x1000, 0, 0x2000, 1, 0x3000, 0x4000, 2, 64, 32, 0x5000, 0x6000, 1, None, None, 0x7000, 0x8000, 4, 32,
             8, 2, 128, 16, 0.088, 1, None]
    a = list(pargs); a[11] = 2
    assert lib.pkv_paged_attn_prefill_chunk_csr(*a) == pkv.ERR_INVALID_ARG
    a = list(pargs); a[21] = 48
    assert lib.pkv_paged_attn_prefill_chunk_csr(*a) == pkv.ERR_UNSUPPORTED
    a = list(pargs); a[7] = 0
    assert lib.pkv_paged_attn_prefill_chunk_csr(*a) == pkv.OK
    # expansion: empty batch is a no-op, null pointers are rejected
    assert lib.pkv_csr_to_block_table(None, None, 0, 4, None, None) == pkv.OK
    assert lib.pkv_csr_to_block_table(None, 0x1000, 2, 4, 0x2000, None) == pkv.ERR_INVALID_ARG
    assert lib.pkv_csr_to_block_table(0x1000, 0x1000, 2, 0, 0x2000, None) == pkv.ERR_INVALID_ARG


def test_swap_entry_points_validate(pkv):
    lib = pkv.load()
    # image: 2 x (n_kv x B x d x bytes) per block, plus 2 x n_kv fp32 scales for FP8
    assert lib.pkv_swap_image_bytes(3, pkv.BF16, 8, 128, 16) == 3 * 2 * 8 * 16 * 128 * 2
    assert lib.pkv_swap_image_bytes(3, pkv.FP8_E4M3FN, 8, 128, 16) == 3 * 2 * (8 * 16 * 128 + 8 * 4)
    assert lib.pkv_swap_image_bytes(-1, pkv.BF16, 8, 128, 16) == 0
    need = lib.pkv_swap_image_bytes(4, pkv.BF16, 2, 64, 16)
    base = [0x1000, 0x2000, pkv.BF16, None, None, 64, 0x3000, 4, 0x4000, need, 0x5000, 2, 64, 16, None]
    for f in (lib.pkv_swap_out, lib.pkv_swap_in):
        a = list(base); a[7] = 0
        assert f(*a) == pkv.OK                          # nothing to move
        a = list(base); a[9] = need - 1
        assert f(*a) == pkv.ERR_WORKSPACE               # staging too small
        a = list(base); a[2] = pkv.FP8_E4M3FN
        assert f(*a) == pkv.ERR_INVALID_ARG             # fp8 without scales
        a = list(base); a[8] = 0x4008
        assert f(*a) == pkv.ERR_INVALID_ARG             # misaligned staging
        a = list(base); a[10] = None
        assert f(*a) == pkv.ERR_INVALID_ARG             # no host image
        a = list(base); a[7] = 70000
        assert f(*a) == pkv.ERR_UNSUPPORTED


def test_work_order_entry_points_validate(pkv):
    lib = pkv.load()
    assert lib.pkv_paged_attn_decode_order(None, 4, 8, 2, 128, 8, 16, pkv.BF16, 0x1000, None) == pkv.ERR_INVALID_ARG
    assert lib.pkv_paged_attn_decode_order(0x1000, 4, 6, 4, 128, 8, 16, pkv.BF16, 0x2000, None) == pkv.ERR_INVALID_ARG
    assert lib.pkv_paged_attn_decode_order(0x1000, 4, 8, 2, 96, 8, 16, pkv.BF16, 0x2000, None) == pkv.ERR_UNSUPPORTED
    args = [0x1000, 0, 0x2000, 1, 0x3000, 0x4000, 1, None, None, 0x5000, 8, 0x6000, 2, 64, 8, 2, 128, 16, 0.088,
            None, None, 0, None]
    assert lib.pkv_paged_attn_decode_ordered(*args) == pkv.ERR_INVALID_ARG   # no order


def test_work_order_entries_need_a_device(pkv):
    """The matrix-core split (bf16 / fp8 KV at d 128) is planned against the
    device's resident workgroups, so without a device the order size (and the
    workspace size) is 0 rather than a guess; invalid arguments give 0 too.
    The sizes themselves are checked on the GPU (test_gpu_work_order.py)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: the GPU test checks the sizes")
    lib = pkv.load()
    assert lib.pkv_paged_attn_decode_order_entries(64, 32, 8, 128, 128, 16, pkv.BF16) == 0
    assert lib.pkv_paged_attn_decode_order_entries(256, 64, 8, 128, 512, 16, pkv.FP8_E4M3FN) == 0
    assert lib.pkv_paged_attn_decode_workspace(8, 64, 8, 128, 2048, 16, pkv.BF16, 0) == 0
    info = (ctypes.c_int32 * 7)()
    assert lib.pkv_paged_attn_decode_plan(8, 64, 8, 128, 2048, 16, pkv.BF16, 0, info) == pkv.ERR_HIP
    assert lib.pkv_paged_attn_decode_order_entries(4, 6, 4, 128, 8, 16, pkv.BF16) == 0              # head ratio
    assert lib.pkv_paged_attn_decode_order_entries(4, 8, 2, 96, 8, 16, pkv.BF16) == 0               # d_head


def test_read_probe_validates(pkv):
    lib = pkv.load()
    f = lib.pkv_read_probe
    assert f(None, 4096, None, 0, 4096, 8, 1, 0x1000, None) == pkv.ERR_INVALID_ARG        # no buffer
    assert f(0x1000, 4096, None, 0, 4096, 8, 1, None, None) == pkv.ERR_INVALID_ARG        # no sink
    assert f(0x1000, 4100, None, 0, 4096, 8, 1, 0x2000, None) == pkv.ERR_INVALID_ARG      # not 16-byte pieces
    assert f(0x1000, 1 << 20, 0x3000, 64, 1000, 8, 1, 0x2000, None) == pkv.ERR_INVALID_ARG  # slab size
    assert f(0x1000, 1 << 20, 0x3000, 4, 4096, 8, 1, 0x2000, None) == pkv.ERR_INVALID_ARG   # fewer slabs than WGs
    assert f(0x1000, 1 << 20, None, 0, 4096, 0, 1, 0x2000, None) == pkv.ERR_INVALID_ARG     # no workgroups


def test_decode_workspace_sizes(pkv):
    # partition mode: one partition -> none; otherwise batch * n_q * parts * (d + 2) floats (d part rounded to 256 B)
    assert pkv.paged_attn_decode_workspace(2, 8, 2, 64, 4, 16, pkv.BF16, 256) == 0
    n = 64 * 32 * 8
    assert pkv.paged_attn_decode_workspace(64, 32, 8, 128, 128, 16, pkv.BF16, 256) == \
        ((n * 128 * 4 + 255) // 256) * 256 + n * 8
    assert pkv.paged_attn_decode_workspace(2, 6, 4, 64, 7, 16, pkv.BF16, 256) == 0  # invalid -> 0


def test_other_entry_points_validate(pkv):
    lib = pkv.load()
    assert lib.pkv_slot_mapping(None, 1, 1, None, None, 0, 16, None, None) == pkv.OK  # empty is a no-op
    assert lib.pkv_slot_mapping(None, 1, 1, 0x1000, 0x1000, 4, 16, 0x1000, None) == pkv.ERR_INVALID_ARG
    assert lib.pkv_kv_append(None, None, 1, 1, None, None, None, 0, 8, 128, 16, None) == pkv.OK
    assert lib.pkv_kv_append(0x1000, 0x1000, 7, 1, 0x1000, 0x1000, 0x1000, 1, 8, 128, 16, None) == pkv.ERR_INVALID_ARG
    assert lib.pkv_kv_append(0x1000, 0x1000, 2, 1, 0x1000, 0x1000, 0x1000, 1, 8, 8, 16, None) == pkv.ERR_UNSUPPORTED
    ap = lib.pkv_kv_append_positions
    good = [0x1000, 0x2000, 1, 4, 0x3000, 2, 8, 0x4000, 0x5000, 0x6000, 0x7000, 3, 8, 128, 16, None, None]
    args = list(good); args[11] = 0
    assert ap(*args) == pkv.OK                       # no tokens: no-op
    args = list(good); args[11] = -1
    assert ap(*args) == pkv.ERR_INVALID_ARG          # negative token count
    args = list(good); args[7] = None
    assert ap(*args) == pkv.ERR_INVALID_ARG          # no sequence ids
    args = list(good); args[4] = None
    assert ap(*args) == pkv.ERR_INVALID_ARG          # no table
    args = list(good); args[2] = 7
    assert ap(*args) == pkv.ERR_INVALID_ARG          # unknown dtype
    args = list(good); args[5] = 0
    assert ap(*args) == pkv.ERR_INVALID_ARG          # no sequences
    args = list(good); args[2] = 2; args[13] = 8
    assert ap(*args) == pkv.ERR_UNSUPPORTED          # 8-byte fp8 rows
    args = list(good); args[6] = 1 << 27
    assert ap(*args) == pkv.ERR_INVALID_ARG          # table wider than 2^30 tokens
    fa = lib.pkv_kv_append_fp8
    good = [0x1000, 0x2000, 0x3000, 0x4000, 8, 0x5000, 2, 0x6000, 0x7000, 1, 4, 0x8000, 0x9000, 1, 2, 128, 16, None]
    args = list(good); args[10] = 0
    assert fa(*args) == pkv.OK                       # max_new_len 0: no-op
    args = list(good); args[13] = 2
    assert fa(*args) == pkv.ERR_UNSUPPORTED          # new rows already FP8
    args = list(good); args[16] = 12
    assert fa(*args) == pkv.ERR_UNSUPPORTED          # block size 12
    args = list(good); args[15] = 96
    assert fa(*args) == pkv.ERR_UNSUPPORTED          # d 96
    args = list(good); args[11] = 0x8004
    assert fa(*args) == pkv.ERR_UNSUPPORTED          # misaligned new K
    args = list(good); args[2] = None
    assert fa(*args) == pkv.ERR_INVALID_ARG          # no scales
    args = list(good); args[9] = -1
    assert fa(*args) == pkv.ERR_INVALID_ARG          # negative batch
    assert lib.pkv_paged_gather(0x1000, 0x1000, 0x1000, 0x1000, 1, 4, 0x1000, 2, 0x1000, 0x1000, 0, 1, 2, 64, 16,
                                None) == pkv.OK
    assert lib.pkv_check_tables(None, 1, None, 1, 1, 16, None, None) == pkv.ERR_INVALID_ARG
    pf = lib.pkv_paged_attn_prefill_chunk
    base = [0x1000, 0, 0x1000, 1, 0x1000, 0x1000, 2, 64, 32, 0x1000, 0x1000, 1, None, None, 0x1000, 8, 32, 32, 8, 128,
            16, 0.088, 1, None, 0, None]
    args = list(base); args[18] = 5
    assert pf(*args) == pkv.ERR_INVALID_ARG          # 32 / 5
    args = list(base); args[19] = 64
    assert pf(*args) == pkv.ERR_UNSUPPORTED          # d 64
    args = list(base); args[11] = 2
    assert pf(*args) == pkv.ERR_INVALID_ARG          # fp8 KV without scales
    args = list(base); args[11] = 0
    assert pf(*args) == pkv.ERR_UNSUPPORTED          # f32 KV
    args = list(base); args[22] = 3
    assert pf(*args) == pkv.ERR_INVALID_ARG          # causal flag
    args = list(base); args[7] = 0
    assert pf(*args) == pkv.OK                       # no queries: no-op
    assert pkv.load().pkv_paged_attn_prefill_workspace(16, 512, 32, 128) == 0


def test_decode_plan_argument_checks(pkv):
    """The plan query validates like the decode call; explicit partitions are
    planned without a device."""
    with pytest.raises(pkv.PkvError):
        pkv.paged_attn_decode_plan(2, 6, 4, 64, 7, 16, pkv.BF16, 256)  # heads not a multiple
    with pytest.raises(pkv.PkvError):
        pkv.paged_attn_decode_plan(2, 8, 2, 64, 7, 16, pkv.BF16, 300)  # partition not a multiple of 256
    p = pkv.paged_attn_decode_plan(3, 32, 8, 128, 256, 16, pkv.BF16, 1024)
    # 3 x 4 (sequence, partition) slots, numbered in eights (one XCD each): 16 slots x 8 KV heads
    assert p == {"split": "partitions", "partition_tokens": 1024, "n_parts": 4, "workgroups": 16 * 8,
                 "merge_pass": True, "heads_per_workgroup": 4, "matrix_cores": True}
    p = pkv.paged_attn_decode_plan(3, 64, 8, 128, 64, 16, pkv.FP8_E4M3FN, 1024)
    assert p["n_parts"] == 1 and not p["merge_pass"] and p["heads_per_workgroup"] == 8 and p["matrix_cores"]
