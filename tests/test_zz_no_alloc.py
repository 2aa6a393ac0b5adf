"""pkv_paged_attn_decode_noalloc, the decode for callers that cannot allocate:
its split keeps partial results in the library's static device scratch.  Two
calls in a row (the second smaller, so it meets the first one's leftovers in
the scratch), for the matrix-core split with a merge pass and for the VALU
work-queue split (whose item counter lives in the scratch): each equals
pkv_paged_attn_decode_partitioned on a caller workspace bit for bit and the
oracle within the parity bar.  A decode too large for the scratch fails before
any launch."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_parity, note, oracle_decode, upload_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def _both(pkv, c, part):
    t = upload_decode(c)
    args = (t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seq_lens"], c.n_q, c.n_kv, c.d, c.block_size,
            c.scale)
    ref = pkv.paged_attn_decode(*args, k_scale=t["k_scale"], v_scale=t["v_scale"], partition_tokens=part)
    out = torch.full_like(ref, float("nan"))
    pkv.paged_attn_decode_noalloc(*args, out=out, k_scale=t["k_scale"], v_scale=t["v_scale"], partition_tokens=part)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("kind,d,n_q,n_kv,part,lens_big,lens_small", [
    ("bf16", 128, 64, 8, 0, [32768, 20000, 5000, 1], [3000, 17, 900]),
    ("fp8", 128, 64, 8, 4096, [9000, 8192, 4097, 300], [5000, 33]),
    ("f32", 64, 8, 2, -1, [3000, 1, 0, 2500, 700, 64] * 20, [40, 9000, 5]),
])
def test_noalloc_matches_workspace_decode(pkv, kind, d, n_q, n_kv, part, lens_big, lens_small):
    for i, lens in enumerate((lens_big, lens_small)):
        c = synth.make_decode_case(config=995, layer=10 * i + d, n_q=n_q, n_kv=n_kv, d=d, seq_lens=lens,
                                   kv_dtype=kind)
        plan = pkv.paged_attn_decode_plan(len(lens), n_q, n_kv, d, c.block_table.shape[1], 16,
                                          {"f32": pkv.F32, "bf16": pkv.BF16, "fp8": pkv.FP8_E4M3FN}[kind], part)
        note(f"noalloc call {i + 1} {kind} batch={len(lens)} plan={plan}")
        assert plan["merge_pass"], "the case must use the scratch"
        got, ref = _both(pkv, c, part)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        assert_parity(got.astype(np.float64), oracle_decode(c), kind, f"call {i + 1}:")


def test_noalloc_rejects_oversize_workspace(pkv):
    """batch 4096 x 64 query heads x two 4096-token partitions needs 272 MB of
    partial results: rejected on the host, nothing launched."""
    batch, n_q, n_kv, d, mb = 4096, 64, 8, 128, 512
    need = pkv.paged_attn_decode_workspace(batch, n_q, n_kv, d, mb, 16, pkv.BF16, 0)
    assert need > 32 << 20
    q = torch.zeros((batch, n_q, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, n_kv, 16, d), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((batch, mb), dtype=torch.int32, device="cuda")
    lens = torch.ones(batch, dtype=torch.int32, device="cuda")
    out = torch.full((batch, n_q, d), 3.0, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_decode_noalloc(q, kc, kc, table, lens, n_q, n_kv, d, 16, 0.088, out=out)
    assert e.value.status == pkv.ERR_WORKSPACE and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
