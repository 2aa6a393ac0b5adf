"""Benchmark of the paged-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch, on inputs already
resident in HBM:
  * decode workloads: slot indexing for the batch's current token, the
    step's work order (the batch ranked by length once, shared by every
    layer), kv_append of that token's K/V rows into every layer's cache (a
    one-layer step indexes and appends in one launch, kv_append_positions),
    then paged decode attention of every layer, back to back (each layer's
    append precedes its attention; with no model between the layers the two
    orders do the same work, and back-to-back calls keep launch gaps out of
    the decode timing);
  * prefill workload: slot indexing and append of the chunk's 8,192 new rows
    (one launch), chunked-prefill attention.
With --fp8-append quantize the FP8 workload's append takes the token's rows
in bf16 and quantises them into the cache (kv_append_fp8: per-block scale
update, re-encoding when a scale grows) instead of copying ready-made codes.
The default workload is the 70B-shaped long-context decode (batch 8, every
sequence 32768 tokens, 64 query heads, 8 KV heads, d 128, 80 layers, bf16 KV:
about 86 GB of cache), the largest of the workloads that fits one GPU;
--workload picks another (the 8B-shaped decode, the fp8 serving mix, the tiny
fp32 case, the prefill chunk).  The tiny and prefill workloads are timed
cold: an untimed 512 MiB write before every step keeps their small working
sets out of the caches, and the medians of per-step events are reported.
Decode steps of several layers are recorded once into two HIP graphs (prep,
attention) after the eager warm-up and replayed in the timed steps, so the
host's launch work is off the clock (--graph off launches every kernel from
Python; a one-layer step does so by default, a graph replay costing more than
its few direct launches); the bounded-sample parity check reads the outputs of
the replayed steps.

Prints one JSON line.  `value` is achieved GB/s (algorithmic bytes / wall
time of the K timed steps; TFLOP/s for prefill); `roofline` describes the
attention call (split-K kernel + merge when split), timed with HIP events on
the launch stream around each step's block of decode calls and divided by the
calls; `cpu_baseline` times the float64 CPU oracle on whole layers of the same
workload on the host cores (and one layer on one core), and `parity` gives the
GPU outputs' errors against it over those layers.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 MFMA
METRIC = "paged GQA decode: achieved HBM GB/s (% of peak) and tokens/s per layer"

# workload name -> synth workload id (the id also namespaces the seeds)
WORKLOADS = {
    "tiny-f32": 1,            # batch 2, 8q/2kv, d 64, lengths {37, 100}, f32, 1 layer
    "llama8b-bf16": 2,        # batch 64, 32q/8kv, d 128, lengths U[1024, 2048], bf16, 32 layers
    "llama70b-32k-bf16": 3,   # batch 8, 64q/8kv, d 128, lengths 32768, bf16, 80 layers
    "llama70b-fp8-mix": 4,    # batch 256, 64q/8kv, d 128, log-normal lengths, fp8 E4M3, 16 layers
    "prefill-chunk-bf16": 5,  # 16 x 512 new tokens over contexts U[0, 8192], 32q/8kv, d 128, bf16
}


# ---------------------------------------------------------------------------
# algorithmic bytes / flops
# ---------------------------------------------------------------------------

def decode_layer_bytes(seq_lens, n_q, n_kv, d, kv_bytes, q_bytes, out_bytes, fp8, block_size=16):
    """Every cached K/V byte read once, plus q, output, scales, table and lengths."""
    L = np.asarray(seq_lens, dtype=np.int64)
    blocks = (L + block_size - 1) // block_size
    b = int((L * n_kv * 2 * d * kv_bytes).sum())
    if fp8:
        b += int((blocks * n_kv * 2 * 4).sum())
    b += len(L) * n_q * d * (q_bytes + out_bytes)
    b += int(blocks.sum()) * 4 + 4 * len(L)
    return b


def append_bytes(tokens, n_kv, d, kv_bytes):
    """Read the new K/V rows and their slots, write them into the pool."""
    return tokens * (n_kv * d * kv_bytes * 2 * 2 + 8)


def append_fp8_bytes(tokens, n_kv, d, in_bytes):
    """Read the new bf16/f32 K/V rows and the (block, KV head) scales, write the
    codes and the scales (the rows of a block whose scale grows are re-read and
    re-written on top; not counted)."""
    return tokens * n_kv * 2 * (d * (in_bytes + 1) + 8) + tokens * 4 * 3


def slot_bytes(tokens, max_blocks):
    return tokens * (4 + 4 + 4 + 8)


def prefill_flops(ctx_lens, q_len, n_q, d):
    """4 d n_q per unmasked (query, key) pair; query i of a chunk sees ctx + i + 1 keys."""
    tot = 0
    for c in ctx_lens:
        tot += sum(int(c) + i + 1 for i in range(q_len))
    return 4 * d * n_q * tot


# ---------------------------------------------------------------------------
# workloads on the device
# ---------------------------------------------------------------------------

class DecodeWorkload:
    def __init__(self, cfg_id: int, layers: int = None, fp8_append: str = "copy", block_size: int = 16,
                 csr: bool = False, shape=None):
        import torch
        import paged_kv_cache_blocks_amd as pkv
        self.pkv, self.torch = pkv, torch
        c = synth.CONFIGS[cfg_id]
        self.cfg_id = cfg_id
        self.name = c["name"]
        self.n_q, self.n_kv, self.d, self.kind = c["n_q"], c["n_kv"], c["d"], c["kv_dtype"]
        self.layers = layers or c["layers"]
        self.quantize_append = self.kind == "fp8" and fp8_append == "quantize"
        self.bs, self.csr = block_size, csr
        B = block_size
        self.seq_lens = synth.config_seq_lens(cfg_id)
        if shape is not None:
            # the workload's heads and element type, with `batch` sequences of
            # `length` tokens each
            batch, length = shape
            self.seq_lens = np.full(batch, length, dtype=np.int32)
            self.name = f"{self.name} at batch {batch} x {length} tokens"
        self.batch = len(self.seq_lens)
        dev = torch.device("cuda")
        need = sum(synth.blocks_for(L, B) for L in self.seq_lens)
        self.num_blocks = 64 if (cfg_id == 1 and B == 16) else need
        perm = synth.rng(cfg_id, 0, synth.T_PERM).permutation(self.num_blocks).astype(np.int32)
        table, filled = synth.build_tables(self.seq_lens, self.num_blocks, perm, B)
        # slots allocated but not holding a token: the tail of each sequence's last block
        self.waste = 1.0 - float(np.sum(self.seq_lens)) / float(need * B)
        self.block_table_np = table
        self.block_table = torch.from_numpy(table).to(dev)
        self.seq_lens_t = torch.from_numpy(self.seq_lens).to(dev)
        self.max_blocks = table.shape[1]
        if csr:
            # the same pages as a CSR table: request s owns kv_indices[kv_indptr[s]:kv_indptr[s+1]]
            counts = np.array([synth.blocks_for(L, B) for L in self.seq_lens], np.int64)
            indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
            indices = np.concatenate([table[s, :counts[s]] for s in range(self.batch)]).astype(np.int32)
            self.kv_indptr = torch.from_numpy(indptr).to(dev)
            self.kv_indices = torch.from_numpy(indices).to(dev)
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[self.kind]
        qdt = torch.float32 if self.kind == "f32" else torch.bfloat16
        shape = (self.num_blocks, self.n_kv, B, self.d)
        filled_t = torch.from_numpy(filled).to(dev)[:, None, :, None]
        self.k, self.v, self.ks, self.vs, self.q, self.k_new, self.v_new = [], [], [], [], [], [], []
        for layer in range(self.layers):
            seed = (cfg_id * 1000 + layer) * 8
            kv = []
            sc = []
            for j in range(2):
                x = torch.empty(shape, dtype=torch.float32, device=dev)
                synth.device_normal_(x, seed + 1 + j)
                if self.kind == "fp8":
                    amax = torch.where(filled_t, x.abs(), torch.zeros((), device=dev)).amax(dim=(2, 3))
                    s = torch.where(amax > 0, amax / 448.0, torch.ones((), device=dev)).float()
                    codes = (x / s[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
                    codes = torch.where(filled_t, codes, torch.full((), 0x7F, dtype=torch.uint8, device=dev))
                    kv.append(codes.contiguous())
                    sc.append(s.contiguous())
                else:
                    y = x.to(tdt)
                    nan = torch.full((), float("nan"), dtype=tdt, device=dev)
                    kv.append(torch.where(filled_t, y, nan).contiguous())
                del x
            self.k.append(kv[0])
            self.v.append(kv[1])
            self.ks.append(sc[0] if sc else None)
            self.vs.append(sc[1] if sc else None)
            qf = torch.empty((self.batch, self.n_q, self.d), dtype=torch.float32, device=dev)
            synth.device_normal_(qf, seed + 3)
            self.q.append(qf.to(qdt).contiguous())
            # the step's new token rows: the rows already at each sequence's last slot
            last = torch.from_numpy(self.seq_lens - 1).to(dev).long()
            blk = self.block_table[torch.arange(self.batch, device=dev), last // B].long()
            if self.quantize_append:
                # the token's rows as the model would hand them over: bf16 values
                # of the codes already there (code x block scale)
                for j, lst in ((0, self.k_new), (1, self.v_new)):
                    vals = kv[j][blk, :, last % B, :].view(torch.float8_e4m3fn).float() * sc[j][blk][:, :, None]
                    lst.append(vals.to(torch.bfloat16).contiguous())
            else:
                self.k_new.append(kv[0][blk, :, last % B, :].contiguous())
                self.v_new.append(kv[1][blk, :, last % B, :].contiguous())
        self.seq_ids = torch.arange(self.batch, dtype=torch.int32, device=dev)
        self.positions = (self.seq_lens_t - 1).to(torch.int32)
        self.slots = torch.empty(self.batch, dtype=torch.int64, device=dev)
        self.cu_new = torch.arange(self.batch + 1, dtype=torch.int32, device=dev)
        # The work order balances the split over the CUs and is paid once per
        # step; a one-layer step of a few sequences (the tiny case: 2) has
        # nothing to balance, and decodes in plain order without its launch.
        self.ordered = not self.csr and (self.layers > 1 or self.batch > 8)
        self.order = torch.empty(pkv.paged_attn_decode_order_entries(self.batch, self.n_q, self.n_kv, self.d,
                                                                     self.max_blocks, B, pkv.dtype_code(self.k[0])),
                                 dtype=torch.int32, device=dev)
        self.out = [torch.empty((self.batch, self.n_q, self.d), dtype=torch.float32, device=dev)
                    for _ in range(self.layers)]
        ws = pkv.paged_attn_decode_workspace(self.batch, self.n_q, self.n_kv, self.d, self.max_blocks, B,
                                             pkv.dtype_code(self.k[0]))
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        self.plan = pkv.paged_attn_decode_plan(self.batch, self.n_q, self.n_kv, self.d, self.max_blocks, B,
                                               pkv.dtype_code(self.k[0]))
        self.scale = synth.softmax_scale(self.d)
        torch.cuda.synchronize()
        kvb = synth.ELEM_BYTES[self.kind]
        qb = 4 if self.kind == "f32" else 2
        self.layer_bytes = decode_layer_bytes(self.seq_lens, self.n_q, self.n_kv, self.d, kvb, qb, 4,
                                              self.kind == "fp8", B)
        app = (append_fp8_bytes(self.batch, self.n_kv, self.d, 2) if self.quantize_append
               else append_bytes(self.batch, self.n_kv, self.d, kvb))
        self.step_bytes = slot_bytes(self.batch, self.max_blocks) + self.layers * (self.layer_bytes + app)

    def decode_call(self, layer):
        if self.csr:
            self.pkv.paged_attn_decode_csr(self.q[layer], self.k[layer], self.v[layer], self.kv_indptr,
                                           self.kv_indices, self.max_blocks, self.seq_lens_t, self.n_q, self.n_kv,
                                           self.d, self.bs, self.scale, k_scale=self.ks[layer],
                                           v_scale=self.vs[layer], out=self.out[layer], workspace=self.ws)
            return
        self.pkv.paged_attn_decode(self.q[layer], self.k[layer], self.v[layer], self.block_table, self.seq_lens_t,
                                   self.n_q, self.n_kv, self.d, self.bs, self.scale, k_scale=self.ks[layer],
                                   v_scale=self.vs[layer], out=self.out[layer], workspace=self.ws,
                                   work_order=self.order if self.ordered else None)

    calls_per_event = property(lambda self: self.layers)

    def prep(self):
        """Slot indexing, work order and every layer's append for the batch's
        current token.  Several layers share one slot mapping, each layer's
        append copying through it; a one-layer step indexes and appends in one
        launch (kv_append_positions, which also stores the slots).  (Measured
        on the 8B-shaped step: the fused call per layer, re-walking the table
        32 times, is 0.6 % slower than one slot mapping; on the one-layer step
        one launch less is 15 % faster.)"""
        pkv = self.pkv
        fused = self.layers == 1 and not self.quantize_append
        if not fused:
            pkv.slot_mapping(self.block_table, self.seq_ids, self.positions, self.bs, out=self.slots)
        if self.ordered:
            # one work order per step, shared by every layer's decode (same batch, same lengths)
            pkv.paged_attn_decode_order(self.seq_lens_t, self.n_q, self.n_kv, self.d, self.max_blocks, self.bs,
                                        pkv.dtype_code(self.k[0]), out=self.order)
        for layer in range(self.layers):
            if self.quantize_append:
                pkv.kv_append_fp8(self.k[layer], self.v[layer], self.ks[layer], self.vs[layer], self.block_table,
                                  self.positions, self.cu_new, 1, self.k_new[layer], self.v_new[layer])
            elif fused:
                pkv.kv_append_positions(self.k[layer], self.v[layer], self.block_table, self.seq_ids, self.positions,
                                        self.k_new[layer], self.v_new[layer], slot_mapping_out=self.slots)
            else:
                pkv.kv_append(self.k[layer], self.v[layer], self.slots, self.k_new[layer], self.v_new[layer])

    def attend(self):
        for layer in range(self.layers):
            self.decode_call(layer)

    def step(self, events=None):
        self.prep()
        if events is not None:
            events[0].record()
        self.attend()
        if events is not None:
            events[1].record()

    def capture(self):
        """Record the step's launches in two HIP graphs (prep, attention), so a
        timed step replays them without per-launch host work.  Every step
        appends the same token into the same slot, so replays compute what the
        eager step computes."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.prep()
            self.attend()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.g_prep, self.g_attend = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_prep):
            self.prep()
        with torch.cuda.graph(self.g_attend):
            self.attend()
        torch.cuda.synchronize()

    def graph_step(self, events=None):
        self.g_prep.replay()
        if events is not None:
            events[0].record()
        self.g_attend.replay()
        if events is not None:
            events[1].record()

    def kernel_desc(self):
        p = self.plan
        if p["split"] == "queue":
            k = f"decode_queue_kernel ({p['workgroups']} workgroups claiming items) + combine_queue_kernel"
        else:
            name = "decode_mfma_kernel" if p.get("matrix_cores") else "decode_kernel"
            k = (f"{name} ({p['n_parts']} partition(s) of {p['partition_tokens']} tokens per (sequence, KV "
                 f"head), {p['workgroups']} workgroups)")
            if p["merge_pass"]:
                k += " + combine_kernel"
        return k

    def describe(self):
        return {"workload": self.name, "batch": self.batch, "n_q_heads": self.n_q, "n_kv_heads": self.n_kv,
                "d_head": self.d, "block_size": self.bs, "layers": self.layers, "kv_dtype": self.kind,
                **({"append": "quantize bf16 -> fp8"} if self.quantize_append else {}),
                **({"page_table": "csr"} if self.csr else {}),
                "tail_waste": round(self.waste, 5),
                "mean_seq_len": float(np.mean(self.seq_lens)), "max_blocks_per_seq": int(self.max_blocks),
                "num_blocks_per_layer": int(self.num_blocks)}


class PrefillWorkload:
    calls_per_event = 1

    def __init__(self, cfg_id: int = 5, kv: str = "bf16"):
        import torch
        import paged_kv_cache_blocks_amd as pkv
        self.pkv, self.torch = pkv, torch
        # "fp8-mma": the FP8 cache attended with both products in FP8, queries
        # and weights as two E4M3 terms ("fp8-mma-single": one term)
        self.mma = kv.startswith("fp8-mma")
        self.split = kv == "fp8-mma"
        self.kind = "fp8" if self.mma else kv
        c = synth.CONFIGS[cfg_id]
        self.name = c["name"]
        self.n_q, self.n_kv, self.d = c["n_q"], c["n_kv"], c["d"]
        self.layers = 1
        self.ctx = synth.config_seq_lens(cfg_id)
        self.q_len = 512
        dev = torch.device("cuda")
        total = self.ctx + self.q_len
        self.num_blocks = sum(synth.blocks_for(L) for L in total)
        perm = synth.rng(cfg_id, 0, synth.T_PERM).permutation(self.num_blocks).astype(np.int32)
        table, _ = synth.build_tables(total, self.num_blocks, perm)
        self.block_table = torch.from_numpy(table).to(dev)
        shape = (self.num_blocks, self.n_kv, 16, self.d)
        self.ks = self.vs = None
        if self.kind == "fp8":
            # codes and per-(block, KV head) scales = max |x| / 448 over the block
            cs = []
            for seed in (5001, 5002):
                x = synth.device_normal_(torch.empty(shape, device=dev), seed)
                sc = (x.abs().amax(dim=(2, 3)) / 448.0).float().contiguous()
                cs.append(((x / sc[:, :, None, None]).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), sc))
                del x
            (self.k, self.ks), (self.v, self.vs) = cs
        else:
            self.k = synth.device_normal_(torch.empty(shape, device=dev), 5001).to(torch.bfloat16)
            self.v = synth.device_normal_(torch.empty(shape, device=dev), 5002).to(torch.bfloat16)
        nq = len(self.ctx) * self.q_len
        self.q = synth.device_normal_(torch.empty((nq, self.n_q, self.d), device=dev), 5003).to(torch.bfloat16)
        self.seq_ids = torch.repeat_interleave(torch.arange(len(self.ctx), dtype=torch.int32), self.q_len).to(dev)
        self.positions = torch.cat([torch.arange(int(cx), int(cx) + self.q_len, dtype=torch.int32)
                                    for cx in self.ctx]).to(dev)
        self.k_new = synth.device_normal_(torch.empty((nq, self.n_kv, self.d), device=dev), 5004).to(torch.bfloat16)
        self.v_new = synth.device_normal_(torch.empty((nq, self.n_kv, self.d), device=dev), 5005).to(torch.bfloat16)
        self.cu = torch.arange(0, nq + 1, self.q_len, dtype=torch.int32, device=dev)
        self.ctx_t = torch.from_numpy(self.ctx).to(dev)
        self.slots = torch.empty(nq, dtype=torch.int64, device=dev)
        self.out = torch.empty((nq, self.n_q, self.d), dtype=torch.float32, device=dev)
        self.scale = synth.softmax_scale(self.d)
        self.flops = prefill_flops(self.ctx, self.q_len, self.n_q, self.d)
        torch.cuda.synchronize()

    def attn_call(self):
        args = (self.q, self.cu, self.ctx_t, self.q_len, self.k, self.v, self.block_table, self.n_q, self.n_kv, self.d,
                16, self.scale)
        if self.mma:
            self.pkv.paged_attn_prefill_chunk_fp8_mma(*args, out=self.out, k_scale=self.ks, v_scale=self.vs,
                                                      split=self.split)
        else:
            self.pkv.paged_attn_prefill_chunk(*args, out=self.out, k_scale=self.ks, v_scale=self.vs)

    def step(self, events=None):
        pkv = self.pkv
        if self.kind == "fp8":
            # the chunk's bf16 rows are quantised into the cache
            pkv.slot_mapping(self.block_table, self.seq_ids, self.positions, 16, out=self.slots)
            pkv.kv_append_fp8(self.k, self.v, self.ks, self.vs, self.block_table, self.ctx_t, self.cu, self.q_len,
                              self.k_new, self.v_new)
        else:
            # slot indexing and append in one launch
            pkv.kv_append_positions(self.k, self.v, self.block_table, self.seq_ids, self.positions, self.k_new,
                                    self.v_new, slot_mapping_out=self.slots)
        if events is not None:
            events[0].record()
        self.attn_call()
        if events is not None:
            events[1].record()

    def describe(self):
        return {"workload": self.name, "num_seqs": len(self.ctx), "q_len": self.q_len, "n_q_heads": self.n_q,
                "n_kv_heads": self.n_kv, "d_head": self.d, "block_size": 16, "kv_dtype": self.kind,
                **({"products": "fp8: q and softmax weights as %s" % ("two E4M3 terms each" if self.split else
                                                                       "one E4M3 term each")} if self.mma else {}),
                "mean_ctx": float(np.mean(self.ctx))}


# ---------------------------------------------------------------------------
# CPU oracle: baseline timing and whole-layer parity (same device bytes)
# ---------------------------------------------------------------------------

_CPU = {}


def cpu_workers() -> int:
    """Worker processes for the oracle: every core this process may run on,
    capped at OMP_NUM_THREADS when that is set (the GPU machine gives one GPU's
    job a 16-thread share of its host and says so there; its affinity mask may
    show more cores than that share)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host(t):
    import torch
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _decode_task(args):
    layer, s = args
    import oracle
    from threadpoolctl import threadpool_limits
    w = _CPU
    with threadpool_limits(limits=1):
        o = oracle.decode_one(w["q"][layer], w["q_dtype"], w["k"][layer], w["v"][layer], w["kind"],
                              w["ks"][layer], w["vs"][layer], w["table"], w["lens"], w["n_q"], w["n_kv"],
                              w["scale"], s)
    return layer, s, o


def _prefill_task(s):
    import oracle
    from threadpoolctl import threadpool_limits
    w = _CPU
    with threadpool_limits(limits=1):
        o = oracle.prefill_one(w["q"], "bf16", w["cu"], w["ctx"], w["k"], w["v"], w["kind"], w["ks"], w["vs"],
                               w["table"], w["n_q"], w["n_kv"], w["scale"], s, causal=True)
    return s, o


def _pool_map(fn, tasks, workers):
    """fn over tasks on a fork pool of `workers` processes (in-process for
    one worker); returns (results, wall seconds of the map)."""
    import multiprocessing as mp
    if workers <= 1:
        t0 = time.perf_counter()
        res = [fn(t) for t in tasks]
        return res, time.perf_counter() - t0
    with mp.get_context("fork").Pool(workers) as pool:
        t0 = time.perf_counter()
        res = pool.map(fn, tasks, chunksize=max(1, len(tasks) // (workers * 4)))
        dt = time.perf_counter() - t0
        pool.close()  # let the workers exit on their own rather than be terminated
        pool.join()
    return res, dt


def _load_decode_layers(w, layers):
    _CPU.clear()
    _CPU.update(dict(q={i: _host(w.q[i]) for i in layers}, k={i: _host(w.k[i]) for i in layers},
                     v={i: _host(w.v[i]) for i in layers}, ks={i: _host(w.ks[i]) for i in layers},
                     vs={i: _host(w.vs[i]) for i in layers}, table=w.block_table_np, lens=w.seq_lens,
                     n_q=w.n_q, n_kv=w.n_kv, scale=w.scale, kind=w.kind,
                     q_dtype="f32" if w.kind == "f32" else "bf16"))


def oracle_decode_layers(w, layers, workers=None):
    """Oracle outputs of whole layers (every sequence, every query head),
    computed from the bytes now in the device caches: {layer: [batch, n_q, d]
    float64}, and the wall seconds of the oracle map."""
    layers = list(layers)
    _load_decode_layers(w, layers)
    tasks = [(i, s) for i in layers for s in range(w.batch)]
    res, dt = _pool_map(_decode_task, tasks, cpu_workers() if workers is None else workers)
    outs = {i: np.zeros((w.batch, w.n_q, w.d)) for i in layers}
    for layer, s, o in res:
        outs[layer][s] = o
    return outs, dt


def _load_prefill(w):
    _CPU.clear()
    _CPU.update(dict(q=_host(w.q), cu=w.cu.cpu().numpy(), ctx=w.ctx, k=_host(w.k), v=_host(w.v), ks=_host(w.ks),
                     vs=_host(w.vs), kind=w.kind, table=w.block_table.cpu().numpy(), n_q=w.n_q, n_kv=w.n_kv,
                     scale=w.scale))


def oracle_prefill_seqs(w, seqs, workers=None):
    """Oracle outputs of whole sequences of the prefill chunk (every query
    token and head), from the bytes now in the device cache (the chunk
    appended): {seq: [q_len, n_q, d]}, and the wall seconds."""
    _load_prefill(w)
    res, dt = _pool_map(_prefill_task, list(seqs), cpu_workers() if workers is None else workers)
    return dict(res), dt


def parity_figures(got, want):
    """max-abs error and the largest per-row relative rms error (rows: one
    sequence or token and one head; rms(err) / rms(reference))."""
    d = got - want
    g = d.reshape(-1, d.shape[-1])
    ref = want.reshape(-1, want.shape[-1])
    den = np.sqrt(np.mean(ref ** 2, axis=1))
    rel = np.sqrt(np.mean(g ** 2, axis=1))[den > 0] / den[den > 0]
    return float(np.max(np.abs(d))), float(rel.max()) if rel.size else 0.0


# whole layers the oracle runs on all cores, by workload id (tiny, 8B, 70B 32K, fp8 mix)
DEFAULT_CPU_LAYERS = {1: 1, 2: 8, 3: 8, 4: 4}


def cpu_baseline(w: DecodeWorkload, sample_layers: int = None):
    """The oracle as it stands, timed on the host: whole layers (every
    sequence and head) on a fork pool of cpu_workers() processes, plus one
    whole layer on one core.  Returns the baseline record and the GPU-vs-oracle
    error figures over the sampled layers."""
    n = min(sample_layers or DEFAULT_CPU_LAYERS.get(w.cfg_id, 2), w.layers)
    workers = cpu_workers()
    layers = list(range(n))
    outs, dt = oracle_decode_layers(w, layers, workers)
    err = rel = 0.0
    for i in layers:
        e, r = parity_figures(w.out[i].cpu().numpy().astype(np.float64), outs[i])
        err, rel = max(err, e), max(rel, r)
    _, dt1 = oracle_decode_layers(w, [0], 1)
    nbytes = n * w.layer_bytes
    model = cpu_model()
    rec = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
           "sample": f"{n} whole layer(s) of the same workload ({w.batch} sequences, all {w.n_q} query heads), "
                     f"float64 NumPy oracle on {workers} processes x 1 BLAS thread, {dt:.2f} s wall; one layer on "
                     f"one core {dt1:.2f} s; CPU: {model}",
           "seconds": round(dt, 3), "seconds_per_layer": round(dt / n, 3), "one_core_seconds_per_layer": round(dt1, 3),
           "tokens_per_s_per_layer": round(w.batch * n / dt, 2), "cpu_model": model}
    return rec, err, rel


def cpu_baseline_prefill(w):
    """The oracle on the whole prefill chunk (all 16 sequences, every token and
    head) on cpu_workers() processes, and on one core for one sequence (the
    median context).  Returns the record and the error figures of the GPU
    output over the whole chunk."""
    workers = cpu_workers()
    seqs = list(range(len(w.ctx)))
    outs, dt = oracle_prefill_seqs(w, seqs, workers)
    got = w.out.cpu().numpy().astype(np.float64)
    cu = w.cu.cpu().numpy()
    want = np.concatenate([outs[s] for s in seqs])
    err, rel = parity_figures(got[cu[0]:cu[-1]], want)
    mid = int(np.argsort(w.ctx)[len(w.ctx) // 2])
    _, dt1 = oracle_prefill_seqs(w, [mid], 1)
    flops1 = prefill_flops([w.ctx[mid]], w.q_len, w.n_q, w.d)
    model = cpu_model()
    rec = {"value": round(w.flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
           "sample": f"the whole chunk ({len(seqs)} sequences x {w.q_len} tokens, all {w.n_q} query heads), float64 "
                     f"NumPy oracle on {workers} processes x 1 BLAS thread, {dt:.2f} s wall; sequence {mid} "
                     f"(context {int(w.ctx[mid])}) on one core {dt1:.2f} s; CPU: {model}",
           "seconds": round(dt, 3), "one_core_seconds_one_sequence": round(dt1, 3),
           "one_core_TFLOP/s": round(flops1 / dt1 / 1e12, 6), "cpu_model": model}
    return rec, err, rel


# ---------------------------------------------------------------------------
# counters from committed rocprofv3 summaries
# ---------------------------------------------------------------------------

def source_hash():
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_mfma.hip", "pkv_device.h"):
        h.update(open(os.path.join(ROOT, "paged_kv_cache_blocks_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload_key):
    """HBM bytes per decode call from the committed counter summary, or None if
    absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload_key}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel source hash:\s*([0-9a-f]+)", text)
    t = re.search(r"HBM bytes per decode call:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_hash():
        return None
    return float(t.group(1))


# ---------------------------------------------------------------------------

def read_probe_bench():
    """Read bandwidth a plain kernel gets on this GPU: a 2 GiB buffer read in
    grid-stride order, and randomly placed slabs (2 KiB: one (block, KV head)
    slab of an fp8 paged cache at 16-token blocks; 4 KiB: the same for bf16;
    16 KiB) of its first 430 MB, the size of one
    8B-shaped decode call, with ordinary and non-temporal loads.  Best of 5
    event-timed launches after one warm-up."""
    import torch
    import paged_kv_cache_blocks_amd as pkv
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    region = 430 * 10 ** 6
    rows = []

    def timed(fn):
        fn()
        best = float("inf")
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
        return best

    for nt in (False, True):
        for wgs in (1024, 2048, 4096):
            t = timed(lambda: pkv.read_probe(buf, sink, None, 4096, wgs, nt))
            rows.append({"pattern": "sequential", "bytes": nbytes, "workgroups": wgs, "nontemporal": nt,
                         "GB/s": round(nbytes / t / 1e9, 1)})
    for slab in (2048, 4096, 16384):
        n = region // slab
        perm = torch.from_numpy(np.random.default_rng(7).permutation(n).astype(np.int32)).cuda()
        for nt in (False, True):
            for wgs in (512, 1024, 1536, 2048):
                per = n // wgs
                t = timed(lambda: pkv.read_probe(buf, sink, perm, slab, wgs, nt))
                rows.append({"pattern": f"random {slab // 1024} KiB slabs", "bytes": per * wgs * slab,
                             "workgroups": wgs, "nontemporal": nt, "GB/s": round(per * wgs * slab / t / 1e9, 1)})
    return {"read_probe": rows, "peak_GB/s": HBM_PEAK_GBS}


def swap_bench(cfg, args):
    """Swap N blocks of one layer of a decode workload out to pinned host
    memory and back (preemption by swap); image bytes / time per direction,
    beside a plain pinned copy of the same size."""
    import torch
    import paged_kv_cache_blocks_amd as pkv
    w = DecodeWorkload(cfg, 1, "copy", args.block_size)
    table = w.block_table_np
    ids_np = table[table >= 0][:args.swap_blocks].astype(np.int32)
    n = len(ids_np)
    ids = torch.from_numpy(ids_np).cuda()
    code = pkv.dtype_code(w.k[0])
    nbytes = pkv.swap_image_bytes(n, code, w.n_kv, w.d, w.bs)
    staging = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    kw = dict(k_scale=w.ks[0], v_scale=w.vs[0])
    k0, v0 = w.k[0].clone(), w.v[0].clone()

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3

    reps = max(args.steps, 5)
    t_out = timed(lambda: pkv.swap_out(w.k[0], w.v[0], ids, staging, host, **kw), reps)
    t_in = timed(lambda: pkv.swap_in(w.k[0], w.v[0], ids, staging, host, **kw), reps)
    t_d2h = timed(lambda: host.copy_(staging, non_blocking=True), reps)
    t_h2d = timed(lambda: staging.copy_(host, non_blocking=True), reps)
    torch.cuda.synchronize()
    # out then in to the same blocks leaves every byte as it was (NaN-poisoned slots included)
    same = bool(torch.equal(w.k[0].view(torch.uint8), k0.view(torch.uint8)) and
                torch.equal(w.v[0].view(torch.uint8), v0.view(torch.uint8)))
    return {"metric": "preemption by swap: host-link GB/s (out, in)", "value": round(nbytes / t_out / 1e9, 2),
            "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
            "config": {"workload": w.name, "blocks": n, "block_size": w.bs, "image_bytes": nbytes,
                       "kv_dtype": w.kind},
            "swap_out_GBps": round(nbytes / t_out / 1e9, 2), "swap_in_GBps": round(nbytes / t_in / 1e9, 2),
            "swap_out_us": round(t_out * 1e6, 1), "swap_in_us": round(t_in * 1e6, 1),
            "plain_copy_d2h_GBps": round(nbytes / t_d2h / 1e9, 2), "plain_copy_h2d_GBps": round(nbytes / t_h2d / 1e9, 2),
            "round_trip_bit_exact": same}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 100 for the cold-cache tiny and prefill workloads, else 30)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama70b-32k-bf16", choices=list(WORKLOADS))
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (profiling only)")
    ap.add_argument("--cpu-sample-layers", type=int, default=None,
                    help="whole layers the CPU oracle runs on all cores (default by workload: 1 tiny, 8 for the 8B "
                         "shape and the 70B 32K decode, 4 for the fp8 mix)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="cold-cache protocol (tiny and prefill workloads): MiB written before every timed step, "
                         "untimed, so no step finds the previous one's data in the L2 / last-level cache")
    ap.add_argument("--fp8-append", choices=["copy", "quantize"], default="copy",
                    help="FP8 workload: copy ready-made codes, or quantise bf16 rows on append")
    ap.add_argument("--swap-blocks", type=int, default=0,
                    help="time swapping this many blocks of one decode layer out to pinned host memory and back")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32, 64, 128, 256],
                    help="decode workloads: tokens per cache block (the same sequences, re-paged)")
    ap.add_argument("--csr", action="store_true", help="decode workloads: pass the page table in CSR form")

    def _shape(text):
        b, _, n = text.partition("x")
        if not (b.isdigit() and n.isdigit() and int(b) > 0 and int(n) > 0):
            raise argparse.ArgumentTypeError("shape is BATCHxTOKENS, e.g. 1x32768")
        return int(b), int(n)
    ap.add_argument("--shape", type=_shape, default=None,
                    help="decode workloads: BATCHxTOKENS sequences of equal length instead of the workload's mix "
                         "(a shape sweep; the line is not the workload's headline)")
    ap.add_argument("--prefill-kv", choices=["bf16", "fp8", "fp8-mma", "fp8-mma-single"], default="bf16",
                    help="prefill workload: KV cache element type (fp8: the chunk is quantised on append and the "
                         "codes widened to bf16 for the products; fp8-mma: the same cache with both products in "
                         "fp8, queries and weights as two E4M3 terms; fp8-mma-single: one term each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="decode workloads: replay each step from HIP graphs (auto: when the step has several "
                         "layers; a graph replay costs more than a few direct launches, so a one-layer step "
                         "launches its kernels directly)")
    ap.add_argument("--read-probe", action="store_true",
                    help="run only the library's read probe: the HBM read bandwidth of a plain kernel, sequential and "
                         "over randomly placed slabs, with ordinary and non-temporal loads")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run only a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)

    if args.read_probe:
        print(json.dumps(read_probe_bench()))
        return

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * 2 ** 20 // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))
        return

    cfg = WORKLOADS[args.workload]
    prefill = synth.CONFIGS[cfg]["kind"] == "prefill"
    if args.steps is None:
        args.steps = 100 if (prefill or args.workload == "tiny-f32") else 30
    if args.swap_blocks:
        print(json.dumps(swap_bench(cfg, args)))
        return
    t_build = time.perf_counter()
    w = (PrefillWorkload(cfg, args.prefill_kv) if prefill
         else DecodeWorkload(cfg, args.layers, args.fp8_append, args.block_size, args.csr, args.shape))
    print(f"[bench] built {args.workload} in {time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    graphs = not prefill and (args.graph == "on" or (args.graph == "auto" and w.layers >= 4))
    step = w.step
    if graphs:
        w.capture()
        for _ in range(args.warmup):
            w.graph_step()
        step = w.graph_step

    # Tiny and prefill workloads use the cold-cache protocol: every timed step
    # is preceded by an untimed write of --flush-mb MiB (more than the 256 MB
    # last-level cache), the step is bracketed by events, and the median step
    # and attention-call times are reported.  Their whole working set would
    # otherwise stay cached from one step to the next.
    cold = prefill or w.name == "tiny-f32"
    flush = torch.empty(args.flush_mb << 18, dtype=torch.float32, device="cuda") if cold else None
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if cold:
            flush.fill_(float(k))
            events[k][2].record()
        step(events[k])
        if cold:
            events[k][3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [ev[0].elapsed_time(ev[1]) / w.calls_per_event for ev in events]
    if cold:
        step_ms = [ev[2].elapsed_time(ev[3]) for ev in events]
        call_s = float(np.median(call_ms)) / 1e3
        step_s = float(np.median(step_ms)) / 1e3
        timing = (f"cold cache: {args.flush_mb} MiB written (untimed) before each of {args.steps} steps; medians of "
                  f"HIP events around each step and each attention call")
    else:
        call_s = float(np.mean(call_ms)) / 1e3
        step_s = wall / args.steps
        timing = None
    avg_call_s = call_s
    ms_per_step = step_s * 1e3

    if prefill:
        tflops = w.flops / step_s / 1e12
        achieved = w.flops / avg_call_s / 1e12
        peak = MFMA_FP8_PEAK_TFLOPS if w.mma else MFMA_BF16_PEAK_TFLOPS
        rec = {"metric": "chunked prefill over a paged cache: achieved TFLOP/s (%s MFMA)" % ("fp8" if w.mma else "bf16"),
               "value": round(tflops, 3),
               "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
               "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "fp8" if w.mma else "bf16",
               "data": "synthetic: seeded N(0,1) q/k/v, random-permutation block tables (no weights or datasets)",
               "config": w.describe(), "timing": timing, "wall_s_with_flushes": round(wall, 4),
               "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                            "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                            "kernel": ("prefill_fp8_kernel<%s>" % ("true" if w.split else "false")) if w.mma
                            else "prefill_kernel",
                            "avg_call_us": round(avg_call_s * 1e6, 2), "flops_per_call": w.flops},
               "new_tokens_per_s": round(len(w.ctx) * w.q_len / step_s, 1)}
        print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step (median)", file=sys.stderr, flush=True)
        if not args.no_cpu_baseline:
            base, err, rel = cpu_baseline_prefill(w)
            rec["cpu_baseline"] = base
            rec["parity"] = {"max_abs_err": err, "max_row_rel_err": rel,
                             "over": "the whole chunk: every sequence, token and head"}
        print(json.dumps(rec))
        return

    gbs = w.step_bytes / step_s / 1e9
    achieved = w.layer_bytes / avg_call_s / 1e9
    traffic = traffic_from_profile(args.workload)
    rec = {"metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": w.kind,
           "data": "synthetic: seeded N(0,1) q/k/v, random-permutation block tables (no weights or datasets)",
           "config": w.describe(),
           "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
           "tokens_per_s_per_layer": round(w.batch / (step_s / w.layers), 1),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                        "kernel": w.kernel_desc(),
                        "timing": timing or (f"HIP events around each step's {w.layers} back-to-back decode calls"
                                             + (" (replayed from a HIP graph)" if graphs else "") + f", / {w.layers}"),
                        "avg_call_us": round(avg_call_s * 1e6, 3), "bytes_per_call": w.layer_bytes}}
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        base, err, rel = cpu_baseline(w, args.cpu_sample_layers)
        rec["cpu_baseline"] = base
        n = min(args.cpu_sample_layers or DEFAULT_CPU_LAYERS.get(w.cfg_id, 2), w.layers)
        rec["parity"] = {"max_abs_err": err, "max_row_rel_err": rel,
                         "over": f"{n} whole layer(s): every sequence and query head"}
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
