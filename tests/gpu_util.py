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


TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}


def err_report(got: np.ndarray, want: np.ndarray) -> str:
    d = np.abs(got - want)
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    return f"max_abs={d.max():.3e} rms_err={np.sqrt(np.mean(d ** 2)):.3e} out_rms={rms:.3e}"
