"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (the benchmark's own workload builder and step: slot mapping,
work order, append, then attention), over whole layers: every sequence and
every query head of the layer, or every token of every sequence of the prefill
chunk, checked against the float64 oracle run on the bytes the device caches
hold after the step.  Bar: max-abs error within the stated tolerance of the KV
type and every output row's relative error within gpu_util.REL."""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench():
    import bench as b
    assert torch.cuda.is_available()
    return b


@pytest.mark.parametrize("workload,layers", [("tiny-f32", 1), ("llama8b-bf16", 2), ("llama70b-32k-bf16", 1),
                                             ("llama70b-fp8-mix", 1)])
def test_decode_fullsize_whole_layers(bench, workload, layers):
    note(f"full-size decode {workload}: building {layers} layer(s)")
    w = bench.DecodeWorkload(bench.WORKLOADS[workload], layers=layers)
    w.step()
    torch.cuda.synchronize()
    note(f"  plan {w.kernel_desc()}; oracle on {bench.cpu_workers()} processes")
    want, secs = bench.oracle_decode_layers(w, range(layers))
    note(f"  oracle {secs:.1f} s for {layers} layer(s) x {w.batch} sequences")
    for layer in range(layers):
        got = w.out[layer].cpu().numpy().astype(np.float64)
        assert_parity(got, want[layer], w.kind, f"layer {layer} (all {w.batch} sequences x {w.n_q} heads):")
        # a sequence's rows are all real outputs: none is left unwritten
        assert np.all(np.abs(got).reshape(w.batch, -1).max(axis=1) > 0)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_fullsize_whole_chunk(bench, kv):
    note(f"full-size chunked prefill, 16 x 512 new tokens, {kv} cache")
    w = bench.PrefillWorkload(5, kv)
    w.step()
    torch.cuda.synchronize()
    seqs = list(range(len(w.ctx)))
    want, secs = bench.oracle_prefill_seqs(w, seqs)
    note(f"  oracle {secs:.1f} s for {len(seqs)} sequences")
    cu = w.cu.cpu().numpy()
    got = w.out.cpu().numpy().astype(np.float64)
    for s in seqs:
        assert_parity(got[cu[s]:cu[s + 1]], want[s], kv, f"seq {s} (ctx={int(w.ctx[s])}):")
    assert_parity(got, np.concatenate([want[s] for s in seqs]), kv, "whole chunk:")
