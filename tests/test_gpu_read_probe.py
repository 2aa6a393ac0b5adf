"""The read probe (a measurement aid beside the attention calls) runs in both
patterns and with both load kinds, and its sink stays untouched for data that
cannot fold to the sink's pattern (all-zero words fold to zero)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_blocks_amd as p
    assert torch.cuda.is_available()
    return p


@pytest.mark.parametrize("nt", [False, True])
def test_read_probe_runs(pkv, nt):
    buf = torch.zeros(8 << 20, dtype=torch.uint8, device="cuda")  # 8 MiB
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    pkv.read_probe(buf, sink, None, 4096, 64, nt)
    perm = torch.from_numpy(np.random.default_rng(3).permutation((8 << 20) // 16384).astype(np.int32)).cuda()
    pkv.read_probe(buf, sink, perm, 16384, 32, nt)
    pkv.read_probe(buf, sink, perm[:40], 4096, 8, nt)  # list shorter than the 4-slab groups times workgroups
    pkv.read_probe(buf, sink, perm, 2048, 32, nt)      # slabs smaller than a workgroup's 4 KiB sweep
    pkv.read_probe(buf, sink, perm[:37], 1024, 4, nt)  # and a remainder of single loads
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
