"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (same workload builder, same calls), on sampled outputs the
oracle computes one sequence at a time from the same device bytes."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, host_bits, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench():
    import bench as b
    assert torch.cuda.is_available()
    return b


def _host(t):
    return None if t is None else host_bits(t)


@pytest.mark.parametrize("workload,layers,seqs", [("tiny-f32", 1, [0, 1]), ("llama8b-bf16", 2, [0, 17, 63]),
                                                  ("llama70b-32k-bf16", 1, [0, 5]),
                                                  ("llama70b-fp8-mix", 1, None)])
def test_decode_fullsize_sampled(bench, workload, layers, seqs):
    note(f"full-size decode {workload}: building {layers} layer(s)")
    w = bench.DecodeWorkload(bench.WORKLOADS[workload], layers=layers)
    w.step()
    torch.cuda.synchronize()
    if seqs is None:  # fp8 mix: the longest, the shortest and a median sequence
        order = np.argsort(w.seq_lens)
        seqs = [int(order[-1]), int(order[0]), int(order[len(order) // 2])]
    q_dtype = "f32" if w.kind == "f32" else "bf16"
    for layer in range(layers):
        q, k, v = host_bits(w.q[layer]), host_bits(w.k[layer]), host_bits(w.v[layer])
        ks, vs = _host(w.ks[layer]), _host(w.vs[layer])
        got = w.out[layer].cpu().numpy().astype(np.float64)
        for s in seqs:
            want = oracle.decode_one(q, q_dtype, k, v, w.kind, ks, vs, w.block_table_np, w.seq_lens, w.n_q, w.n_kv,
                                     w.scale, s)
            err = float(np.max(np.abs(got[s] - want)))
            note(f"  layer {layer} seq {s} (L={w.seq_lens[s]}): max_abs={err:.3e}")
            assert err <= TOL[w.kind]


def test_prefill_fullsize_sampled(bench):
    note("full-size chunked prefill, 16 x 512 new tokens")
    w = bench.PrefillWorkload(5)
    w.step()
    torch.cuda.synchronize()
    q, k, v = host_bits(w.q), host_bits(w.k), host_bits(w.v)
    cu = w.cu.cpu().numpy()
    got = w.out.cpu().numpy().astype(np.float64)
    order = np.argsort(w.ctx)
    for s in [int(order[0]), int(order[-1]), 3]:
        rows = [0, 1, 17, 255, 510, 511]
        want = oracle.prefill_one(q, "bf16", cu, w.ctx, k, v, "bf16", None, None, w.block_table.cpu().numpy(),
                                  w.n_q, w.n_kv, w.scale, s, rows=rows)
        err = float(np.max(np.abs(got[cu[s] + np.array(rows)] - want)))
        note(f"  seq {s} (ctx={w.ctx[s]}): max_abs={err:.3e}")
        assert err <= 1e-2
