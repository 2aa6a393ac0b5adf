"""A decode step recorded in a HIP graph (slot mapping, work order, append,
decode of two layers) and replayed several times, with eager library work and
synchronisations between the replays, gives bit for bit the outputs of the same
step run eagerly.  The library's decode path records no memset or allocation,
so nothing in it depends on being launched from the host each time."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import note, upload_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


def _bits(t):
    return t.cpu().numpy().view(np.uint32).copy()


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_graph_replay_matches_eager(pkv, kind):
    n_q, n_kv, d, B = 32, 8, 128, 16
    lens = [300, 17, 1000, 64, 2049]
    cases = [synth.make_decode_case(config=981, layer=l, n_q=n_q, n_kv=n_kv, d=d, seq_lens=lens, kv_dtype=kind)
             for l in range(2)]
    ts = [upload_decode(c) for c in cases]
    batch = len(lens)
    sl = ts[0]["seq_lens"]
    tables = [t["block_table"] for t in ts]  # each layer pages the same sequences into its own pool
    kvd = pkv.BF16 if kind == "bf16" else pkv.FP8_E4M3FN
    seq_ids = torch.arange(batch, dtype=torch.int32, device="cuda")
    positions = (sl - 1).to(torch.int32)
    slots = [torch.empty(batch, dtype=torch.int64, device="cuda") for _ in range(2)]
    order = torch.empty(pkv.paged_attn_decode_order_entries(batch, n_q, n_kv, d, tables[0].shape[1], B, kvd),
                        dtype=torch.int32, device="cuda")
    mb = tables[0].shape[1]
    ws = torch.zeros(max(pkv.paged_attn_decode_workspace(batch, n_q, n_kv, d, mb, B, kvd), 256),
                     dtype=torch.uint8, device="cuda")
    # the current token's K/V rows: the rows already cached at that slot, so the append is idempotent
    knew, vnew = [], []
    for c, t in zip(cases, ts):
        rows = []
        for s, L in enumerate(lens):
            blk = int(c.block_table[s, (L - 1) // B])
            rows.append((blk, (L - 1) % B))
        knew.append(torch.stack([t["k_cache"][b, :, o, :] for b, o in rows]).contiguous())
        vnew.append(torch.stack([t["v_cache"][b, :, o, :] for b, o in rows]).contiguous())
    outs = [torch.empty((batch, n_q, d), dtype=torch.float32, device="cuda") for _ in range(2)]

    def step():
        for l in range(2):
            pkv.slot_mapping(tables[l], seq_ids, positions, B, out=slots[l])
        pkv.paged_attn_decode_order(sl, n_q, n_kv, d, mb, B, kvd, out=order)
        for l in range(2):
            pkv.kv_append(ts[l]["k_cache"], ts[l]["v_cache"], slots[l], knew[l], vnew[l])
        for l in range(2):
            pkv.paged_attn_decode(q=ts[l]["q"], k_cache=ts[l]["k_cache"], v_cache=ts[l]["v_cache"],
                                  block_table=tables[l], seq_lens=sl, n_q_heads=n_q, n_kv_heads=n_kv, d_head=d,
                                  block_size=B, scale=cases[l].scale, k_scale=ts[l]["k_scale"],
                                  v_scale=ts[l]["v_scale"], out=outs[l], workspace=ws, work_order=order)

    step()
    torch.cuda.synchronize()
    want = [_bits(o) for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        # eager library work between replays (an unrelated decode into its own output)
        extra = pkv.paged_attn_decode(ts[0]["q"], ts[0]["k_cache"], ts[0]["v_cache"], tables[0], sl, n_q, n_kv, d, B,
                                      cases[0].scale, k_scale=ts[0]["k_scale"], v_scale=ts[0]["v_scale"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(2):
            assert np.array_equal(_bits(outs[l]), want[l]), f"replay {rep} layer {l} differs from the eager step"
        assert torch.isfinite(extra).all()
    note(f"graph replay {kind}: 3 replays bit-identical to the eager step")
