// Block-table plumbing on the device: slot indexing, append (scatter of new
// K/V rows into their slots), gather (walk a table into contiguous rows) and a
// table validity check.
//
// Slot indexing follows "KV cache, PagedAttention and FlashAttention",
// Problem 4 ("The idea"): logical position p of a sequence lives in logical
// block p / B at offset p % B, and the block table maps the logical block to a
// physical block.  A flat slot id is physical_block * B + offset.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void slot_mapping_kernel(const int32_t* __restrict__ table, int32_t batch,
                                                           int32_t max_blocks, const int32_t* __restrict__ seq_ids,
                                                           const int32_t* __restrict__ positions, int32_t n,
                                                           int32_t block_size, int64_t* __restrict__ out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int s = seq_ids[t];
  const int p = positions[t];
  int64_t slot = -1;
  if (s >= 0 && s < batch && p >= 0 && p < max_blocks * block_size) {
    const int blk = table[(int64_t)s * max_blocks + p / block_size];
    if (blk >= 0) slot = (int64_t)blk * block_size + p % block_size;
  }
  out[t] = slot;
}

// One thread moves 16 bytes; a row of one KV head is row_bytes (a multiple of
// 16).  Grid: x over (token, head, 16-byte piece), y = 0 for K, 1 for V.
__global__ __launch_bounds__(256) void kv_append_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                        int64_t num_slots, const int64_t* __restrict__ slots,
                                                        const char* __restrict__ k, const char* __restrict__ v,
                                                        int32_t n, int32_t n_kv, int32_t row_bytes,
                                                        int32_t block_size) {
  const int pieces = row_bytes / 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)n * n_kv * pieces;
  if (i >= total) return;
  const int piece = (int)(i % pieces);
  const int h = (int)((i / pieces) % n_kv);
  const int t = (int)(i / ((int64_t)pieces * n_kv));
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size, off = slot % block_size;
  const int64_t dst = ((blk * n_kv + h) * block_size + off) * row_bytes + piece * 16;
  const int64_t src = ((int64_t)t * n_kv + h) * row_bytes + piece * 16;
  if (blockIdx.y == 0) st16(k_cache + dst, ld16(k + src));
  else st16(v_cache + dst, ld16(v + src));
}

// Grid: x = logical block of the sequence, y = sequence.  The workgroup copies
// the block's filled rows for every KV head, K and V.
__global__ __launch_bounds__(256) void gather_kernel(char* __restrict__ k_out, char* __restrict__ v_out,
                                                     const char* __restrict__ k_cache,
                                                     const char* __restrict__ v_cache, int64_t num_blocks,
                                                     const int32_t* __restrict__ table, int32_t max_blocks,
                                                     const int32_t* __restrict__ seq_lens,
                                                     const int64_t* __restrict__ cu, int64_t total_rows,
                                                     int32_t n_kv, int32_t row_bytes, int32_t block_size) {
  const int j = blockIdx.x, s = blockIdx.y;
  int L = seq_lens[s];
  L = min(max(L, 0), max_blocks * block_size);
  const int first = j * block_size;
  if (first >= L) return;
  const int rows = min(block_size, L - first);
  int blk = table[(int64_t)s * max_blocks + j];
  blk = (int)min(max((int64_t)blk, (int64_t)0), num_blocks - 1);
  const int pieces = row_bytes / 16;
  const int total = rows * n_kv * pieces;
  const int64_t out_row0 = cu[s] + first;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int piece = i % pieces;
    const int h = (i / pieces) % n_kv;
    const int r = i / (pieces * n_kv);
    if (out_row0 + r < 0 || out_row0 + r >= total_rows) continue;  // never write outside k_out / v_out
    const int64_t src = (((int64_t)blk * n_kv + h) * block_size + r) * row_bytes + piece * 16;
    const int64_t dst = ((out_row0 + r) * n_kv + h) * row_bytes + piece * 16;
    st16(k_out + dst, ld16(k_cache + src));
    st16(v_out + dst, ld16(v_cache + src));
  }
}

__global__ __launch_bounds__(256) void check_tables_kernel(const int32_t* __restrict__ table, int32_t max_blocks,
                                                           const int32_t* __restrict__ seq_lens, int32_t batch,
                                                           int64_t num_blocks, int32_t block_size,
                                                           int32_t* __restrict__ err) {
  const int s = blockIdx.x;
  if (s >= batch) return;
  const int L = seq_lens[s];
  int bad = 0;
  if (threadIdx.x == 0 && (L < 0 || (int64_t)L > (int64_t)max_blocks * block_size)) bad = 1;
  const int nb = min(max(L, 0), max_blocks * block_size);
  const int used = (nb + block_size - 1) / block_size;
  for (int j = threadIdx.x; j < used; j += blockDim.x) {
    const int blk = table[(int64_t)s * max_blocks + j];
    if (blk < 0 || (int64_t)blk >= num_blocks) ++bad;
  }
  if (bad) atomicAdd(err, bad);
}

// Copy-on-write copy: whole blocks src -> dst of the K and V pools.  One
// thread moves 16 bytes; grid x over the block's 16-byte pieces, y = pair,
// z = 0 for K, 1 for V.  The first n_kv threads of each (pair, K/V) also copy
// the block's scales when there are any.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                          float* __restrict__ k_scale, float* __restrict__ v_scale,
                                                          int64_t num_blocks, const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int64_t block_bytes,
                                                          int32_t n_kv) {
  const int64_t piece = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t s = src[blockIdx.y], d = dst[blockIdx.y];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  char* const cache = blockIdx.z == 0 ? k_cache : v_cache;
  if (piece * 16 < block_bytes) st16(cache + d * block_bytes + piece * 16, ld16(cache + s * block_bytes + piece * 16));
  float* const scale = blockIdx.z == 0 ? k_scale : v_scale;
  if (scale != nullptr && piece < n_kv) scale[d * n_kv + piece] = scale[s * n_kv + piece];
}

hipError_t launch_slot_mapping(const int32_t* table, int32_t batch, int32_t max_blocks, const int32_t* seq_ids,
                               const int32_t* positions, int32_t n, int32_t block_size, int64_t* out,
                               hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, table, batch, max_blocks,
                     seq_ids, positions, n, block_size, out);
  return hipGetLastError();
}

hipError_t launch_kv_append(void* k_cache, void* v_cache, int64_t num_blocks, const int64_t* slots, const void* k,
                            const void* v, int32_t n, int32_t n_kv, int32_t row_bytes, int32_t block_size,
                            hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t total = (int64_t)n * n_kv * (row_bytes / 16);
  dim3 grid((unsigned)((total + 255) / 256), 2);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(256), 0, stream, (char*)k_cache, (char*)v_cache,
                     num_blocks * block_size, slots, (const char*)k, (const char*)v, n, n_kv, row_bytes,
                     block_size);
  return hipGetLastError();
}

hipError_t launch_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache, int64_t num_blocks,
                         const int32_t* table, int32_t max_blocks, const int32_t* seq_lens, const int64_t* cu,
                         int64_t total_rows, int32_t batch, int32_t n_kv, int32_t row_bytes, int32_t block_size,
                         hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3(max_blocks, batch), dim3(256), 0, stream, (char*)k_out, (char*)v_out,
                     (const char*)k_cache, (const char*)v_cache, num_blocks, table, max_blocks, seq_lens, cu,
                     total_rows, n_kv, row_bytes, block_size);
  return hipGetLastError();
}

hipError_t launch_check_tables(const int32_t* table, int32_t max_blocks, const int32_t* seq_lens, int32_t batch,
                               int64_t num_blocks, int32_t block_size, int32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(batch), dim3(256), 0, stream, table, max_blocks, seq_lens, batch,
                     num_blocks, block_size, err);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                              const int32_t* src, const int32_t* dst, int32_t n_pairs, int64_t block_bytes,
                              int32_t n_kv, hipStream_t stream) {
  if (n_pairs == 0) return hipSuccess;
  const int64_t pieces = block_bytes / 16;
  const int64_t gx = ((pieces > n_kv ? pieces : (int64_t)n_kv) + 255) / 256;
  if (gx > 0x7fffffff || n_pairs > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)n_pairs, 2), dim3(256), 0, stream,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), k_scale, v_scale, num_blocks, src, dst,
                     block_bytes, n_kv);
  return hipGetLastError();
}

}  // namespace pkv
