"""Helpers for the GPU parity tests: upload synth cases as torch tensors and
run the library through its binding.  Expected values always come from the
CPU oracle on the same host bytes."""
import sys

import numpy as np
import torch

import oracle
import synth


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, kind: str = None) -> torch.Tensor:
    """Host array -> CUDA tensor; bf16 bit patterns become torch.bfloat16."""
    x = np.ascontiguousarray(x)
    if kind == "bf16" or (kind is None and x.dtype == np.uint16):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """CUDA tensor -> host array in storage form (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload_decode(c: synth.DecodeCase) -> dict:
    return dict(q=dev(c.q, c.q_dtype), k_cache=dev(c.k_cache, c.kv_dtype), v_cache=dev(c.v_cache, c.kv_dtype),
                k_scale=None if c.k_scale is None else dev(c.k_scale),
                v_scale=None if c.v_scale is None else dev(c.v_scale),
                block_table=dev(c.block_table), seq_lens=dev(c.seq_lens))


def run_decode(pkv, c: synth.DecodeCase, t: dict = None, out_dtype=torch.float32, partition_tokens: int = 0,
               **over) -> np.ndarray:
    t = upload_decode(c) if t is None else t
    args = dict(t)
    args.update(over)
    out = pkv.paged_attn_decode(args["q"], args["k_cache"], args["v_cache"], args["block_table"], args["seq_lens"],
                                c.n_q, c.n_kv, c.d, c.block_size, c.scale, k_scale=args["k_scale"],
                                v_scale=args["v_scale"], out_dtype=out_dtype, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def oracle_decode(c: synth.DecodeCase) -> np.ndarray:
    return oracle.paged_decode(c.q, c.q_dtype, c.k_cache, c.v_cache, c.kv_dtype, c.k_scale, c.v_scale,
                               c.block_table, c.seq_lens, c.n_q, c.n_kv, c.scale)


# Max-abs bound over every output element, per KV element type (the stated
# parity tolerances; fp8 against an oracle fed the same dequantised values).
TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}

# Bound on the relative error of every output row (one sequence or query
# token, one head): rms(got - want) / rms(want) over the row's d values.
# With bf16 or fp8 KV the kernels round each softmax weight to bf16 (relative
# error up to 2^-9, rms 2^-9/sqrt(3) = 1.1e-3), which perturbs a row by about
# that fraction of its size whatever the sequence length (1.2e-3 - 1.9e-3 in a
# float64 simulation at 37 - 32768 tokens); 5e-3 leaves room for that.  Output
# rows shrink like 1/sqrt(L), so the absolute bound alone grows weak with
# length: one 16-token block left out of a 32768-token sequence moves the row
# by about 1.5e-2 of its size (tests/test_tolerance_strength.py) while its
# max-abs change stays near 1e-3.  f32 KV keeps fp32 weights.
REL = {"f32": 1e-5, "bf16": 5e-3, "fp8": 5e-3}


def row_rel_err(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """rms(got - want) / rms(want) over the last axis, for every row whose
    reference is not all zeros (rows that are must match exactly: max-abs)."""
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    w = want.reshape(-1, want.shape[-1]).astype(np.float64)
    num = np.sqrt(np.mean((g - w) ** 2, axis=1))
    den = np.sqrt(np.mean(w ** 2, axis=1))
    live = den > 0
    return num[live] / den[live]


def err_report(got: np.ndarray, want: np.ndarray) -> str:
    d = np.abs(got - want)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    rel = row_rel_err(got, want)
    rel_max = float(rel.max()) if rel.size else 0.0
    return (f"max_abs={d.max():.3e} rms_err={np.sqrt(np.mean(d ** 2)):.3e} out_rms={rms:.3e} "
            f"max_row_rel={rel_max:.3e}")


def assert_parity(got: np.ndarray, want: np.ndarray, kind: str, label: str = "", tol: float = None,
                  rel: float = None) -> str:
    """The parity bar: every output finite, max-abs error <= the stated
    tolerance of the KV type, and every row's relative error <= REL.  Prints
    and returns the figures."""
    tol = TOL[kind] if tol is None else tol
    rel = REL[kind] if rel is None else rel
    rep = err_report(got, want)
    note(f"  {label} {rep}".rstrip())
    assert np.all(np.isfinite(got)), rep
    assert float(np.max(np.abs(got - want))) <= tol, rep
    r = row_rel_err(got, want)
    assert (r.max() if r.size else 0.0) <= rel, rep
    return rep
