"""Python binding of libpkv (attention over a paged KV cache, MI355X / gfx950).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every computation runs in the HIP kernels of ``libpkv.so``.  The
entry points carry the C ABI's names without the ``pkv_`` prefix.  The first
call into the library fails loudly (ImportError) if it has not been built
(``python -m paged_kv_cache_blocks_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the same library (the sanitizer build of
# the host code loads this way)
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(_HERE, "libpkv.so")

_lib = None

# status codes and element types (include/pkv.h)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_NO_BLOCKS, ERR_DEVICE_CHECK = range(7)
F32, BF16, FP8_E4M3FN = 0, 1, 2

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "pkv_abi_version": ([], ctypes.c_int),
    "pkv_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_kv_bytes_per_token": ([_i32, _i32, _i32, _i32], _i64),
    "pkv_set_device_checks": ([ctypes.c_int], None),
    "pkv_device_checks": ([], ctypes.c_int),
    "pkv_slot_mapping": ([_vp, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp], ctypes.c_int),
    "pkv_kv_append": ([_vp, _vp, ctypes.c_int, _i64, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "pkv_kv_append_positions": ([_vp, _vp, ctypes.c_int, _i64, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _vp, _vp], ctypes.c_int),
    "pkv_kv_append_fp8": ([_vp, _vp, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, ctypes.c_int, _i32,
                           _i32, _i32, _vp], ctypes.c_int),
    "pkv_paged_gather": ([_vp, _vp, _vp, _vp, ctypes.c_int, _i64, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _i32, _i32,
                          _vp],
                         ctypes.c_int),
    "pkv_check_tables": ([_vp, _i32, _vp, _i32, _i64, _i32, _vp, _vp], ctypes.c_int),
    "pkv_read_probe": ([_vp, _i64, _vp, _i32, _i32, _i32, _i32, _vp, _vp], ctypes.c_int),
    "pkv_paged_attn_decode": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i32, _vp,
                               _i32, _i64, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp], ctypes.c_int),
    "pkv_paged_attn_decode_partitioned": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                           _i32, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp],
                                          ctypes.c_int),
    "pkv_paged_attn_decode_noalloc": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                       _i32, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32, _i32, _vp], ctypes.c_int),
    "pkv_paged_attn_decode_ordered": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                       _i32, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _sz, _vp],
                                      ctypes.c_int),
    "pkv_paged_attn_decode_order": ([_vp, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _vp, _vp], ctypes.c_int),
    "pkv_paged_attn_decode_order_entries": ([_i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int], _i32),
    "pkv_paged_attn_decode_workspace": ([_i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _i32], _sz),
    "pkv_paged_attn_decode_plan": ([_i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _i32, _vp], ctypes.c_int),
    "pkv_paged_attn_prefill_chunk": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                                      ctypes.c_int, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32, _i32, _vp,
                                      _sz, _vp], ctypes.c_int),
    "pkv_paged_attn_prefill_workspace": ([_i32, _i32, _i32, _i32], _sz),
    "pkv_paged_attn_decode_csr": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                   _i32, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp], ctypes.c_int),
    "pkv_paged_attn_prefill_chunk_csr": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                                          ctypes.c_int, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                                          _i32, _vp], ctypes.c_int),
    "pkv_paged_attn_prefill_chunk_fp8_mma": ([_vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _i32, _i32, _i32, _vp,
                                              _vp, ctypes.c_int, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32,
                                              _f32, _i32, _i32, _vp], ctypes.c_int),
    "pkv_csr_to_block_table": ([_vp, _vp, _i32, _i32, _vp, _vp], ctypes.c_int),
    "pkv_swap_image_bytes": ([_i32, ctypes.c_int, _i32, _i32, _i32], _sz),
    "pkv_swap_out": ([_vp, _vp, ctypes.c_int, _vp, _vp, _i64, _vp, _i32, _vp, _sz, _vp, _i32, _i32, _i32, _vp],
                     ctypes.c_int),
    "pkv_swap_in": ([_vp, _vp, ctypes.c_int, _vp, _vp, _i64, _vp, _i32, _vp, _sz, _vp, _i32, _i32, _i32, _vp],
                    ctypes.c_int),
    "pkv_pool_create": ([_i64, _vp], ctypes.c_int),
    "pkv_pool_destroy": ([_vp], None),
    "pkv_pool_free_blocks": ([_vp], _i64),
    "pkv_pool_refcount": ([_vp, _i32], _i32),
    "pkv_pool_alloc": ([_vp, _i32, _vp], ctypes.c_int),
    "pkv_pool_share": ([_vp, _vp, _i32], ctypes.c_int),
    "pkv_pool_release": ([_vp, _vp, _i32], ctypes.c_int),
    "pkv_pool_prepare_append": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "pkv_copy_blocks": ([_vp, _vp, ctypes.c_int, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
}


def load():
    """The loaded libpkv.so (ctypes.CDLL); raises ImportError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libpkv.so is not built ({LIB_PATH}); run `python -m paged_kv_cache_blocks_amd.build`")
        cdll = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(cdll, name)
            fn.argtypes = args
            fn.restype = res
        _lib = cdll
    return _lib


def __getattr__(name):
    if name == "lib":
        return load()
    raise AttributeError(name)


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{load().pkv_status_string(status).decode()}: {message}")
        self.status = status


def _check(status: int):
    if status != OK:
        raise PkvError(status, load().pkv_last_error().decode())


def abi_version() -> int:
    return load().pkv_abi_version()


def set_device_checks(enable: bool) -> None:
    """Turn the library's device-data checks on or off (process-wide)."""
    load().pkv_set_device_checks(1 if enable else 0)


def device_checks() -> bool:
    return bool(load().pkv_device_checks())


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, d_head: int, bytes_per_value: int) -> int:
    return load().pkv_kv_bytes_per_token(n_layers, n_kv_heads, d_head, bytes_per_value)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def slot_mapping(block_table: torch.Tensor, seq_ids: torch.Tensor, positions: torch.Tensor, block_size: int = 16,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _need(block_table, torch.int32, "block_table")
    _need(seq_ids, torch.int32, "seq_ids")
    _need(positions, torch.int32, "positions")
    n = seq_ids.numel()
    if positions.numel() != n:
        raise ValueError("seq_ids and positions differ in length")
    if out is None:
        out = torch.empty(n, dtype=torch.int64, device=seq_ids.device)
    _need(out, torch.int64, "out")
    _check(load().pkv_slot_mapping(_ptr(block_table), block_table.shape[0], block_table.shape[1], _ptr(seq_ids),
                                _ptr(positions), n, block_size, _ptr(out), _stream(stream)))
    return out


def kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor, k: torch.Tensor,
              v: torch.Tensor, stream=None) -> None:
    """Copy k[t], v[t] ([num_tokens, n_kv, d]) into their slots of one layer's caches."""
    _need(slot_mapping, torch.int64, "slot_mapping")
    nb, n_kv, bs, d = k_cache.shape
    if k.dtype != k_cache.dtype or v.dtype != v_cache.dtype or v_cache.shape != k_cache.shape:
        raise TypeError("k/v must match the caches")
    if k.shape != (slot_mapping.numel(), n_kv, d) or v.shape != k.shape:
        raise ValueError("k, v must be [num_tokens, n_kv, d]")
    _check(load().pkv_kv_append(_ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), nb, _ptr(slot_mapping), _ptr(k),
                             _ptr(v), slot_mapping.numel(), n_kv, d, bs, _stream(stream)))


def kv_append_positions(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                        seq_ids: torch.Tensor, positions: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        slot_mapping_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """Slot indexing and append in one launch: k[t], v[t] ([num_tokens, n_kv, d])
    go to position positions[t] of sequence seq_ids[t] through block_table;
    the slots are also stored in slot_mapping_out (int64) when given."""
    _need(block_table, torch.int32, "block_table")
    _need(seq_ids, torch.int32, "seq_ids")
    _need(positions, torch.int32, "positions")
    n = seq_ids.numel()
    if positions.numel() != n:
        raise ValueError("seq_ids and positions differ in length")
    nb, n_kv, bs, d = k_cache.shape
    if k.dtype != k_cache.dtype or v.dtype != v_cache.dtype or v_cache.shape != k_cache.shape:
        raise TypeError("k/v must match the caches")
    if k.shape != (n, n_kv, d) or v.shape != k.shape:
        raise ValueError("k, v must be [num_tokens, n_kv, d]")
    if slot_mapping_out is not None:
        _need(slot_mapping_out, torch.int64, "slot_mapping_out")
        if slot_mapping_out.numel() < n:
            raise ValueError("slot_mapping_out holds fewer than num_tokens entries")
    _check(load().pkv_kv_append_positions(_ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), nb, _ptr(block_table),
                                       block_table.shape[0], block_table.shape[1], _ptr(seq_ids), _ptr(positions),
                                       _ptr(k), _ptr(v), n, n_kv, d, bs,
                                       None if slot_mapping_out is None else _ptr(slot_mapping_out), _stream(stream)))


def kv_append_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                  block_table: torch.Tensor, context_lens: torch.Tensor, cu_new_lens: torch.Tensor, max_new_len: int,
                  k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """Quantise and append each sequence's new rows ([total_new, n_kv, d], bf16
    or f32) to one layer's FP8 caches at positions context_lens[s] onwards,
    updating the per-(block, KV head) scales (``pkv_kv_append_fp8``)."""
    nb, n_kv, bs, d = k_cache.shape
    if dtype_code(k_cache) != FP8_E4M3FN or v_cache.shape != k_cache.shape or dtype_code(v_cache) != FP8_E4M3FN:
        raise TypeError("k_cache and v_cache must be matching FP8 caches")
    _need(k_scale, torch.float32, "k_scale")
    _need(v_scale, torch.float32, "v_scale")
    if k_scale.shape != (nb, n_kv) or v_scale.shape != (nb, n_kv):
        raise ValueError("scales must be [num_blocks, n_kv]")
    _need(block_table, torch.int32, "block_table")
    _need(context_lens, torch.int32, "context_lens")
    _need(cu_new_lens, torch.int32, "cu_new_lens")
    batch = context_lens.numel()
    if cu_new_lens.numel() != batch + 1 or block_table.shape[0] != batch:
        raise ValueError("cu_new_lens must hold batch + 1 entries and block_table batch rows")
    if k_new.dtype != v_new.dtype or k_new.shape != v_new.shape or k_new.dim() != 3 or k_new.shape[1:] != (n_kv, d):
        raise ValueError("k_new, v_new must be [total_new, n_kv, d] of one dtype")
    _check(load().pkv_kv_append_fp8(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), nb,
                                    _ptr(block_table), block_table.shape[1], _ptr(context_lens), _ptr(cu_new_lens),
                                    batch, int(max_new_len), _ptr(k_new), _ptr(v_new), dtype_code(k_new), n_kv, d, bs,
                                    _stream(stream)))


def paged_gather(k_cache, v_cache, block_table, seq_lens, cu_seq_lens, total_tokens: int, stream=None):
    """Rows of every sequence in logical order: returns (k, v) [total_tokens, n_kv, d]."""
    nb, n_kv, bs, d = k_cache.shape
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(cu_seq_lens, torch.int64, "cu_seq_lens")
    k_out = torch.empty((total_tokens, n_kv, d), dtype=k_cache.dtype, device=k_cache.device)
    v_out = torch.empty_like(k_out)
    if total_tokens == 0:
        return k_out, v_out
    _check(load().pkv_paged_gather(_ptr(k_out), _ptr(v_out), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), nb,
                                _ptr(block_table), block_table.shape[1], _ptr(seq_lens), _ptr(cu_seq_lens),
                                int(total_tokens), block_table.shape[0], n_kv, d, bs, _stream(stream)))
    return k_out, v_out


def check_tables(block_table, seq_lens, num_blocks: int, block_size: int = 16, stream=None) -> int:
    """Number of invalid table entries / lengths (synchronises)."""
    err = torch.zeros(1, dtype=torch.int32, device=block_table.device)
    _check(load().pkv_check_tables(_ptr(block_table), block_table.shape[1], _ptr(seq_lens), block_table.shape[0],
                                num_blocks, block_size, _ptr(err), _stream(stream)))
    return int(err.item())


class BlockPool:
    """Host-side block pool of libpkv: reference counts, lowest-id-first
    allocation and copy-on-write bookkeeping for appends (``pkv_pool_*``).
    Ids are plain ints; rows are lists of int."""

    def __init__(self, num_blocks: int):
        h = ctypes.c_void_p()
        _check(load().pkv_pool_create(int(num_blocks), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            load().pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def free_blocks(self) -> int:
        return load().pkv_pool_free_blocks(self._h)

    def refcount(self, block: int) -> int:
        return load().pkv_pool_refcount(self._h, int(block))

    @staticmethod
    def _ids(ids):
        arr = (ctypes.c_int32 * max(1, len(ids)))(*[int(b) for b in ids])
        return arr, len(ids)

    def alloc(self, n: int) -> list:
        arr = (ctypes.c_int32 * max(1, n))()
        _check(load().pkv_pool_alloc(self._h, int(n), ctypes.cast(arr, ctypes.c_void_p)))
        return list(arr[:n])

    def share(self, ids) -> None:
        arr, n = self._ids(ids)
        _check(load().pkv_pool_share(self._h, ctypes.cast(arr, ctypes.c_void_p), n))

    def release(self, ids) -> None:
        arr, n = self._ids(ids)
        _check(load().pkv_pool_release(self._h, ctypes.cast(arr, ctypes.c_void_p), n))

    def prepare_append(self, row, seq_len: int, n_new: int, block_size: int = 16):
        """Returns (new row, [(src, dst)]) -- the copies to run before the append."""
        arr, n = self._ids(row)
        src, dst, nc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(load().pkv_pool_prepare_append(self._h, ctypes.cast(arr, ctypes.c_void_p), n, int(seq_len), int(n_new),
                                              int(block_size), ctypes.byref(src), ctypes.byref(dst), ctypes.byref(nc)))
        return list(arr[:n]), [(src.value, dst.value)] if nc.value else []


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src: torch.Tensor, dst: torch.Tensor, *,
                k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """Copy whole blocks src[i] -> dst[i] (int32 device tensors) of one layer's caches, scales included."""
    _need(src, torch.int32, "src")
    _need(dst, torch.int32, "dst")
    if src.numel() != dst.numel():
        raise ValueError("src and dst differ in length")
    nb, n_kv, bs, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise TypeError("k_cache and v_cache must match")
    _check(load().pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale), nb,
                                  _ptr(src), _ptr(dst), src.numel(), n_kv, d, bs, _stream(stream)))


def swap_image_bytes(n_blocks: int, cache_dtype: int, n_kv_heads: int, d_head: int, block_size: int) -> int:
    return int(load().pkv_swap_image_bytes(n_blocks, cache_dtype, n_kv_heads, d_head, block_size))


def _swap_args(k_cache, v_cache, block_ids, staging, host_image, k_scale, v_scale):
    _need(block_ids, torch.int32, "block_ids")
    if not host_image.is_pinned():
        raise ValueError("host_image must be pinned host memory")
    if not host_image.is_contiguous() or staging.dtype != torch.uint8 or host_image.dtype != torch.uint8:
        raise TypeError("staging and host_image must be contiguous uint8 tensors")
    nb, n_kv, bs, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise TypeError("k_cache and v_cache must match")
    return nb, n_kv, bs, d


def swap_out(k_cache, v_cache, block_ids, staging, host_image, *, k_scale=None, v_scale=None, stream=None) -> None:
    """Pack blocks block_ids into the device staging buffer and copy the image
    to host_image (a pinned uint8 tensor of swap_image_bytes(...) bytes)."""
    nb, n_kv, bs, d = _swap_args(k_cache, v_cache, block_ids, staging, host_image, k_scale, v_scale)
    _check(load().pkv_swap_out(_ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale), nb,
                               _ptr(block_ids), block_ids.numel(), _ptr(staging), staging.numel(),
                               host_image.data_ptr(), n_kv, d, bs, _stream(stream)))


def swap_in(k_cache, v_cache, block_ids, staging, host_image, *, k_scale=None, v_scale=None, stream=None) -> None:
    """Copy host_image to the staging buffer and write its blocks into block_ids."""
    nb, n_kv, bs, d = _swap_args(k_cache, v_cache, block_ids, staging, host_image, k_scale, v_scale)
    _check(load().pkv_swap_in(_ptr(k_cache), _ptr(v_cache), dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale), nb,
                              _ptr(block_ids), block_ids.numel(), _ptr(staging), staging.numel(),
                              host_image.data_ptr(), n_kv, d, bs, _stream(stream)))


def paged_attn_decode_plan(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size=16,
                           kv_dtype: int = BF16, partition_tokens=0) -> dict:
    """How the decode call splits its work on the current device."""
    info = (ctypes.c_int32 * 7)()
    _check(load().pkv_paged_attn_decode_plan(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size,
                                             kv_dtype, partition_tokens, ctypes.cast(info, ctypes.c_void_p)))
    return {"split": "queue" if info[0] else "partitions", "partition_tokens": info[1], "n_parts": info[2],
            "workgroups": info[3], "merge_pass": bool(info[4]), "heads_per_workgroup": info[5],
            "matrix_cores": bool(info[6])}


def paged_attn_decode_workspace(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size=16,
                                kv_dtype: int = BF16, partition_tokens=0) -> int:
    return load().pkv_paged_attn_decode_workspace(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq,
                                                  block_size, kv_dtype, partition_tokens)


def paged_attn_decode(q, k_cache, v_cache, block_table, seq_lens, n_q_heads, n_kv_heads, d_head, block_size, scale,
                      *, k_scale=None, v_scale=None, out=None, out_dtype=torch.float32, workspace=None,
                      partition_tokens: int = 0, work_order=None, stream=None) -> torch.Tensor:
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over the seq_lens[s] cached tokens of sequence s.
    work_order (from paged_attn_decode_order) only changes which workgroup takes which sequence."""
    batch = q.shape[0]
    nb = k_cache.shape[0]
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    if out is None:
        out = torch.empty((batch, n_q_heads, d_head), dtype=out_dtype, device=q.device)
    ws_bytes = paged_attn_decode_workspace(batch, n_q_heads, n_kv_heads, d_head, block_table.shape[1], block_size,
                                           dtype_code(k_cache), partition_tokens)
    if workspace is None and ws_bytes:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)  # the item counter starts at 0
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if work_order is not None:
        _need(work_order, torch.int32, "work_order")
        n = paged_attn_decode_order_entries(batch, n_q_heads, n_kv_heads, d_head, block_table.shape[1], block_size,
                                            dtype_code(k_cache))
        if partition_tokens != 0 or work_order.numel() != n:
            raise ValueError(f"work_order takes the library's split and {n} entries (paged_attn_decode_order)")
        _check(load().pkv_paged_attn_decode_ordered(
            _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache),
            _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1], _ptr(seq_lens), batch, nb,
            n_q_heads, n_kv_heads, d_head, block_size, float(scale), _ptr(work_order), ws_ptr, ws_n, _stream(stream)))
        return out
    _check(load().pkv_paged_attn_decode_partitioned(
        _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1], _ptr(seq_lens), batch, nb, n_q_heads,
        n_kv_heads, d_head, block_size, float(scale), int(partition_tokens), ws_ptr, ws_n, _stream(stream)))
    return out


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, n_q_heads, n_kv_heads, d_head, block_size,
                              scale, *, out, k_scale=None, v_scale=None, partition_tokens: int = 0,
                              stream=None) -> torch.Tensor:
    """paged_attn_decode without a workspace: the library's static device
    scratch holds the split's partial results (pkv_paged_attn_decode_noalloc).
    `out` must be given: nothing is allocated."""
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _check(load().pkv_paged_attn_decode_noalloc(
        _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1], _ptr(seq_lens), q.shape[0],
        k_cache.shape[0], n_q_heads, n_kv_heads, d_head, block_size, float(scale), int(partition_tokens),
        _stream(stream)))
    return out


def paged_attn_decode_order_entries(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size=16,
                                    kv_dtype: int = BF16) -> int:
    """int32 entries of the work order for these arguments (batch, or batch x partitions)."""
    n = load().pkv_paged_attn_decode_order_entries(batch, n_q_heads, n_kv_heads, d_head, int(max_blocks_per_seq),
                                                   block_size, kv_dtype)
    if n <= 0:
        raise PkvError(ERR_INVALID_ARG, "no work order for these arguments: " + load().pkv_last_error().decode())
    return n


def paged_attn_decode_order(seq_lens, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size=16,
                            kv_dtype: int = BF16, out=None, stream=None) -> torch.Tensor:
    """Work order for the decode calls of one step: the sequences ranked by
    length, or, when the split has several partitions per sequence, the
    (sequence, partition) units ranked by tokens followed by -1s."""
    _need(seq_lens, torch.int32, "seq_lens")
    batch = seq_lens.numel()
    n = paged_attn_decode_order_entries(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size,
                                        kv_dtype)
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=seq_lens.device)
    elif out.numel() != n or out.dtype != torch.int32:
        raise ValueError(f"the work order takes {n} int32 entries")
    _check(load().pkv_paged_attn_decode_order(_ptr(seq_lens), batch, n_q_heads, n_kv_heads, d_head,
                                              int(max_blocks_per_seq), block_size, kv_dtype, _ptr(out),
                                              _stream(stream)))
    return out


def paged_attn_decode_csr(q, k_cache, v_cache, kv_indptr, kv_indices, max_pages_per_seq, seq_lens, n_q_heads,
                          n_kv_heads, d_head, block_size, scale, *, k_scale=None, v_scale=None, out=None,
                          out_dtype=torch.float32, workspace=None, stream=None) -> torch.Tensor:
    """Decode with a CSR page table: request s owns kv_indices[kv_indptr[s]:kv_indptr[s+1]]."""
    batch = q.shape[0]
    nb = k_cache.shape[0]
    _need(kv_indptr, torch.int32, "kv_indptr")
    _need(kv_indices, torch.int32, "kv_indices")
    _need(seq_lens, torch.int32, "seq_lens")
    if kv_indptr.numel() != batch + 1:
        raise ValueError("kv_indptr must hold batch + 1 entries")
    if out is None:
        out = torch.empty((batch, n_q_heads, d_head), dtype=out_dtype, device=q.device)
    ws_bytes = paged_attn_decode_workspace(batch, n_q_heads, n_kv_heads, d_head, max_pages_per_seq, block_size,
                                           dtype_code(k_cache), 0)
    if workspace is None and ws_bytes:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pkv_paged_attn_decode_csr(
        _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(kv_indptr), _ptr(kv_indices), int(max_pages_per_seq), _ptr(seq_lens),
        batch, nb, n_q_heads, n_kv_heads, d_head, block_size, float(scale), ws_ptr, ws_n, _stream(stream)))
    return out


def csr_to_block_table(kv_indptr, kv_indices, max_blocks_per_seq: int, out=None, stream=None) -> torch.Tensor:
    """2-D block table [batch, max_blocks_per_seq] (padded with -1) from a CSR page table."""
    _need(kv_indptr, torch.int32, "kv_indptr")
    _need(kv_indices, torch.int32, "kv_indices")
    batch = kv_indptr.numel() - 1
    if out is None:
        out = torch.empty((batch, max_blocks_per_seq), dtype=torch.int32, device=kv_indptr.device)
    _check(load().pkv_csr_to_block_table(_ptr(kv_indptr), _ptr(kv_indices), batch, int(max_blocks_per_seq), _ptr(out),
                                         _stream(stream)))
    return out


def paged_attn_prefill_chunk_csr(q, cu_q_lens, context_lens, max_q_len, k_cache, v_cache, kv_indptr, kv_indices,
                                 max_pages_per_seq, n_q_heads, n_kv_heads, d_head, block_size, scale, *,
                                 causal: bool = True, out=None, out_dtype=torch.float32, k_scale=None, v_scale=None,
                                 stream=None) -> torch.Tensor:
    """Chunked prefill with a CSR page table."""
    total_q = q.shape[0]
    _need(cu_q_lens, torch.int32, "cu_q_lens")
    _need(context_lens, torch.int32, "context_lens")
    _need(kv_indptr, torch.int32, "kv_indptr")
    _need(kv_indices, torch.int32, "kv_indices")
    if out is None:
        out = torch.empty((total_q, n_q_heads, d_head), dtype=out_dtype, device=q.device)
    _check(load().pkv_paged_attn_prefill_chunk_csr(
        _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(cu_q_lens), _ptr(context_lens),
        context_lens.numel(), total_q, int(max_q_len), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(kv_indptr), _ptr(kv_indices), int(max_pages_per_seq), k_cache.shape[0],
        n_q_heads, n_kv_heads, d_head, block_size, float(scale), 1 if causal else 0, _stream(stream)))
    return out


def paged_attn_prefill_chunk(q, cu_q_lens, context_lens, max_q_len, k_cache, v_cache, block_table, n_q_heads,
                             n_kv_heads, d_head, block_size, scale, *, causal: bool = True, out=None,
                             out_dtype=torch.float32, k_scale=None, v_scale=None, stream=None) -> torch.Tensor:
    """Packed chunk queries [total_q, n_q, d] against cached context + chunk (already appended);
    FP8 caches take their per-(block, KV head) scales in k_scale / v_scale."""
    total_q = q.shape[0]
    _need(cu_q_lens, torch.int32, "cu_q_lens")
    _need(context_lens, torch.int32, "context_lens")
    _need(block_table, torch.int32, "block_table")
    if out is None:
        out = torch.empty((total_q, n_q_heads, d_head), dtype=out_dtype, device=q.device)
    _check(load().pkv_paged_attn_prefill_chunk(
        _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(cu_q_lens), _ptr(context_lens),
        context_lens.numel(), total_q, int(max_q_len), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), block_table.shape[1], k_cache.shape[0], n_q_heads, n_kv_heads, d_head, block_size,
        float(scale), 1 if causal else 0, None, 0, _stream(stream)))
    return out


def paged_attn_prefill_chunk_fp8_mma(q, cu_q_lens, context_lens, max_q_len, k_cache, v_cache, block_table,
                                     n_q_heads, n_kv_heads, d_head, block_size, scale, *, k_scale, v_scale,
                                     causal: bool = True, split: bool = True, out=None,
                                     out_dtype=torch.float32, stream=None) -> torch.Tensor:
    """Chunked prefill over an FP8 cache with both products in FP8: queries
    and softmax weights in E4M3, as two terms each (split=True, within the FP8
    tolerance) or one (split=False, faster, row errors of a few percent)."""
    total_q = q.shape[0]
    _need(cu_q_lens, torch.int32, "cu_q_lens")
    _need(context_lens, torch.int32, "context_lens")
    _need(block_table, torch.int32, "block_table")
    if out is None:
        out = torch.empty((total_q, n_q_heads, d_head), dtype=out_dtype, device=q.device)
    _check(load().pkv_paged_attn_prefill_chunk_fp8_mma(
        _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(cu_q_lens), _ptr(context_lens),
        context_lens.numel(), total_q, int(max_q_len), _ptr(k_cache), _ptr(v_cache), dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1], k_cache.shape[0], n_q_heads,
        n_kv_heads, d_head, block_size, float(scale), 1 if causal else 0, 1 if split else 0, _stream(stream)))
    return out


def read_probe(buf: torch.Tensor, sink: torch.Tensor, slab_list: Optional[torch.Tensor] = None, slab_bytes: int = 4096,
               workgroups: int = 512, nontemporal: bool = True, stream=None) -> None:
    """Stream buf (grid-stride, or the listed slabs) with 16-byte loads: a
    measurement aid for the read bandwidth a plain kernel gets."""
    nbytes = buf.numel() * buf.element_size()
    n_list = 0
    if slab_list is not None:
        _need(slab_list, torch.int32, "slab_list")
        n_list = slab_list.numel()
    _check(load().pkv_read_probe(_ptr(buf), nbytes, _ptr(slab_list), n_list, slab_bytes, workgroups,
                                 1 if nontemporal else 0, _ptr(sink), _stream(stream)))
