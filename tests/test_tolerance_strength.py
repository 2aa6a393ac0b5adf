"""How strong the parity bar is, shown on the oracle itself (CPU only).

With N(0,1) queries and keys and the 1/sqrt(d) scale the softmax is nearly
flat, so a decode output row of a long sequence is small (rms about
sqrt(e / L)) and a max-abs bound alone barely sees a missing piece of the
sequence.  The GPU tests therefore also bound every row's relative rms error
(gpu_util.REL).  This file checks, at the 70B-shaped long-context length
(32768 tokens, d 128), that:
  * dropping one 16-token block, or one 4096-token partition, changes a row by
    more than the relative bound (so the bound catches it), while the
    dropped block's max-abs change stays far below the bf16 max-abs tolerance;
  * rounding every softmax weight to bf16 (what the kernels do) stays well
    inside the relative bound.
"""
import numpy as np
import torch

import oracle
from gpu_util import REL, TOL, row_rel_err

L, D, HEADS = 32768, 128, 4


def _rows(seed):
    r = np.random.default_rng(seed)
    bf = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    K = bf(r.standard_normal((L, D)))
    V = bf(r.standard_normal((L, D)))
    Q = bf(r.standard_normal((HEADS, D)))
    return Q, K, V


def _attend(Q, K, V, keep=None):
    if keep is not None:
        K, V = K[keep], V[keep]
    return oracle.softmax_attention_rows(Q, K, V, 1.0 / np.sqrt(D), np.full(len(Q), len(K)))


def test_relative_bound_catches_a_dropped_block_and_partition():
    Q, K, V = _rows(11)
    want = _attend(Q, K, V)
    keep = np.ones(L, bool)
    keep[20000:20016] = False                  # one 16-token block
    block = _attend(Q, K, V, keep)
    assert row_rel_err(block, want).min() > 2 * REL["bf16"]
    assert np.max(np.abs(block - want)) < TOL["bf16"] / 2   # max-abs alone would pass it
    keep = np.ones(L, bool)
    keep[8192:12288] = False                   # one 4096-token partition
    part = _attend(Q, K, V, keep)
    assert row_rel_err(part, want).min() > 10 * REL["bf16"]


def test_bf16_weights_stay_inside_the_relative_bound():
    """The kernels' bf16 weights: each weight 2^(s - m) (m a running
    reference at most 8 below the true max, in log2 units) rounded to bf16,
    the normaliser summing the same rounded weights."""
    Q, K, V = _rows(12)
    want = _attend(Q, K, V)
    s = (K @ Q.T) / np.sqrt(D) * np.log2(np.e)          # [L, heads], log2 units
    m = s.max(axis=0) - 3.0
    p = torch.from_numpy(np.exp2(s - m)).to(torch.bfloat16).double().numpy()
    got = (p.T @ V) / p.sum(axis=0)[:, None]
    rel = row_rel_err(got, want)
    assert rel.max() < REL["bf16"] / 2, rel
