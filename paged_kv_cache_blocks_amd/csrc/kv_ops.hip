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

// Slot of (sequence s, position p), or -1 (padding) for a pair outside the
// table or a negative table entry.
__device__ __forceinline__ int64_t slot_of(const int32_t* __restrict__ table, int32_t batch, int32_t max_blocks,
                                           int s, int p, int32_t block_size) {
  int64_t slot = -1;
  if (s >= 0 && s < batch && p >= 0 && p < max_blocks * block_size) {
    const int blk = table[(int64_t)s * max_blocks + p / block_size];
    if (blk >= 0) slot = (int64_t)blk * block_size + p % block_size;
  }
  return slot;
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(const int32_t* __restrict__ table, int32_t batch,
                                                           int32_t max_blocks, const int32_t* __restrict__ seq_ids,
                                                           const int32_t* __restrict__ positions, int32_t n,
                                                           int32_t block_size, int64_t* __restrict__ out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  out[t] = slot_of(table, batch, max_blocks, seq_ids[t], positions[t], block_size);
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

// Slot indexing and append in one pass: each thread finds its token's slot
// through the table (as slot_mapping_kernel) and moves its 16 bytes (as
// kv_append_kernel); the threads of piece 0, head 0 of K also store the slot
// when slots_out is given.  Same grid as kv_append_kernel.
__global__ __launch_bounds__(256) void kv_append_positions_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache, int64_t num_slots, const int32_t* __restrict__ table,
    int32_t batch, int32_t max_blocks, const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions,
    const char* __restrict__ k, const char* __restrict__ v, int32_t n, int32_t n_kv, int32_t row_bytes,
    int32_t block_size, int64_t* __restrict__ slots_out) {
  const int pieces = row_bytes / 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)n * n_kv * pieces;
  if (i >= total) return;
  const int piece = (int)(i % pieces);
  const int h = (int)((i / pieces) % n_kv);
  const int t = (int)(i / ((int64_t)pieces * n_kv));
  const int64_t slot = slot_of(table, batch, max_blocks, seq_ids[t], positions[t], block_size);
  if (slots_out && blockIdx.y == 0 && h == 0 && piece == 0) slots_out[t] = slot;
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

// ---- fp8 E4M3FN quantisation on append ----
// float -> E4M3FN code: nearest value, ties to an even mantissa field,
// magnitudes above 448 saturating to 448 (OCP 8-bit floating point: round to
// nearest even, E4M3FN has no infinities).  Inputs are finite.
__device__ __forceinline__ uint32_t f32_to_e4m3fn(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.f);  // subnormals: m * 2^-9 (8 is the smallest normal, 0x08)
  } else {
    const uint32_t ab = __float_as_uint(a);
    int e = (int)(ab >> 23) - 127;  // -6 .. 8
    const uint32_t man = ab & 0x7FFFFFu;
    uint32_t m = man >> 20;
    const uint32_t rem = man & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    if (m == 8u) {
      m = 0u;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | m;  // at most (15, 6): 448
  }
  return sign | code;
}

// E4M3FN code (not NaN) -> its exact float value
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// D / 64 consecutive values of one row, widened to float
template <typename TIn, int N>
__device__ __forceinline__ void load_row_part(const TIn* p, float (&x)[N]) {
  if constexpr (sizeof(TIn) == 2) {
    if constexpr (N == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      x[0] = __uint_as_float(w << 16);
      x[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      x[0] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(p) << 16);
    }
  } else {
    if constexpr (N == 2) {
      const float2 w = *reinterpret_cast<const float2*>(p);
      x[0] = w.x;
      x[1] = w.y;
    } else {
      x[0] = *reinterpret_cast<const float*>(p);
    }
  }
}

template <int N>
__device__ __forceinline__ void store_codes(uint8_t* p, const uint32_t (&c)[N]) {
  if constexpr (N == 2)
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)(c[0] | (c[1] << 8));
  else
    *p = (uint8_t)c[0];
}

// Workgroup per (sequence, logical block touched by the append), one wave per
// (KV head, K|V) pair.  The block's new scale is max(old scale, max |new
// values| / 448) (the old one only if the block already holds rows of the
// sequence); when it grows, the existing rows are re-encoded (code * old /
// new); the new rows are encoded as x / scale.  A wave walks the block's rows
// with lane l holding values l * D/64 ...: a first pass over the new rows
// finds their largest magnitude, a second encodes them (the first row's
// values stay in registers, later rows are read again from cache).
template <int D, typename TIn>
__global__ __launch_bounds__(1024) void kv_append_fp8_kernel(uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                            float* __restrict__ k_scale, float* __restrict__ v_scale,
                                                            int64_t num_blocks, const int32_t* __restrict__ table,
                                                            int32_t max_blocks, const int32_t* __restrict__ ctx_lens,
                                                            const int32_t* __restrict__ cu_new,
                                                            const TIn* __restrict__ k_new,
                                                            const TIn* __restrict__ v_new, int32_t n_kv,
                                                            int32_t log2_bs) {
  constexpr int VPL = D / kWave;
  const int B = 1 << log2_bs;
  const int lane = threadIdx.x & (kWave - 1);
  const int pair = (int)blockIdx.z * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  if (pair >= 2 * n_kv) return;
  const int h = pair >> 1, is_v = pair & 1, s = blockIdx.y;
  const int ctx = ctx_lens[s], t0 = cu_new[s], n = cu_new[s + 1] - t0;
  if (ctx < 0 || n <= 0) return;
  const int j = (ctx >> log2_bs) + (int)blockIdx.x;  // logical block
  if (j * B >= ctx + n || j >= max_blocks) return;
  const int32_t raw = table[(int64_t)s * max_blocks + j];
  if (raw < 0 || raw >= num_blocks) return;
  const int64_t blk = raw;
  const int n_old = max(min(ctx - j * B, B), 0);  // rows the block already holds
  const int lo = max(ctx, j * B) - ctx;           // first new row of the block, relative to t0
  const int cnt = min(ctx + n, (j + 1) * B) - ctx - lo;
  uint8_t* const codes = (is_v ? v_cache : k_cache) + (blk * n_kv + h) * B * D + lane * VPL;
  float* const sc = (is_v ? v_scale : k_scale) + blk * n_kv + h;
  const float sc_in = *sc;
  const int64_t stride = (int64_t)n_kv * D;
  const TIn* const src = (is_v ? v_new : k_new) + ((int64_t)(t0 + lo) * n_kv + h) * D + lane * VPL;

  float x0[VPL];
  load_row_part(src, x0);
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < VPL; ++e) m = fmaxf(m, fabsf(x0[e]));
  for (int i = 1; i < cnt; ++i) {
    float x[VPL];
    load_row_part(src + i * stride, x);
#pragma unroll
    for (int e = 0; e < VPL; ++e) m = fmaxf(m, fabsf(x[e]));
  }
  m = group_max<kWave>(m);
  const float old = n_old > 0 ? sc_in : 0.f;
  const float nw = fmaxf(old, m / 448.f);
  if (nw > old) {
    for (int r = 0; r < n_old; ++r) {
      uint32_t c[VPL];
      if constexpr (VPL == 2) {
        const uint32_t w = *reinterpret_cast<const uint16_t*>(codes + r * D);
        c[0] = f32_to_e4m3fn((e4m3fn_to_f32(w & 0xFFu) * old) / nw);
        c[1] = f32_to_e4m3fn((e4m3fn_to_f32(w >> 8) * old) / nw);
      } else {
        c[0] = f32_to_e4m3fn((e4m3fn_to_f32(codes[r * D]) * old) / nw);
      }
      store_codes(codes + r * D, c);
    }
  }
  {
    uint32_t c[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) c[e] = nw > 0.f ? f32_to_e4m3fn(x0[e] / nw) : 0u;
    store_codes(codes + n_old * D, c);
  }
  for (int i = 1; i < cnt; ++i) {
    float x[VPL];
    load_row_part(src + i * stride, x);
    uint32_t c[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) c[e] = nw > 0.f ? f32_to_e4m3fn(x[e] / nw) : 0u;
    store_codes(codes + (n_old + i) * D, c);
  }
  if (lane == 0) *sc = nw;
}

// CSR page table -> 2-D table: row s holds kv_indices[kv_indptr[s] ..
// kv_indptr[s+1]) followed by -1 up to max_blocks entries (a row with more
// pages keeps its first max_blocks).  Grid: x over entries, y = sequence.
__global__ __launch_bounds__(256) void csr_to_table_kernel(const int32_t* __restrict__ indptr,
                                                           const int32_t* __restrict__ indices, int32_t max_blocks,
                                                           int32_t* __restrict__ table) {
  const int s = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= max_blocks) return;
  const int b = indptr[s], n = indptr[s + 1] - b;
  table[(int64_t)s * max_blocks + j] = j < n ? indices[b + j] : -1;
}

// Swap image of n listed blocks: [K slabs][V slabs][K scales][V scales] (the
// scale sections for FP8 only), block i of the list at position i of each
// section.  Pack (to_image = 1) copies listed blocks into the image, unpack
// the image into listed blocks; a listed id outside the pool is skipped.
// One thread moves 16 bytes; grid x over a slab's 16-byte pieces, y = list
// position, z = 0 for K, 1 for V; the first n_kv threads of x-block 0 move
// the block's scales.
__global__ __launch_bounds__(256) void swap_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                                                   float* __restrict__ k_scale, float* __restrict__ v_scale,
                                                   int64_t num_blocks, const int32_t* __restrict__ ids, int32_t n,
                                                   char* __restrict__ image, int64_t block_bytes, int32_t n_kv,
                                                   int32_t to_image) {
  const int i = blockIdx.y, z = blockIdx.z;
  const int id = ids[i];
  if (id < 0 || id >= num_blocks) return;
  char* const cache = z ? v_cache : k_cache;
  char* const slab = cache + (int64_t)id * block_bytes;
  char* const img = image + ((int64_t)z * n + i) * block_bytes;
  const int64_t piece = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (piece * 16 < block_bytes) {
    if (to_image) st16(img + piece * 16, ld16(slab + piece * 16));
    else st16(slab + piece * 16, ld16(img + piece * 16));
  }
  if (k_scale && blockIdx.x == 0 && (int)threadIdx.x < n_kv) {
    float* const sc = (z ? v_scale : k_scale) + (int64_t)id * n_kv + threadIdx.x;
    float* const isc = reinterpret_cast<float*>(image + 2 * (int64_t)n * block_bytes) + ((int64_t)z * n + i) * n_kv +
                       threadIdx.x;
    if (to_image) *isc = *sc;
    else *sc = *isc;
  }
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

hipError_t launch_kv_append_positions(void* k_cache, void* v_cache, int64_t num_blocks, const int32_t* table,
                                      int32_t batch, int32_t max_blocks, const int32_t* seq_ids,
                                      const int32_t* positions, const void* k, const void* v, int32_t n, int32_t n_kv,
                                      int32_t row_bytes, int32_t block_size, int64_t* slots_out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t total = (int64_t)n * n_kv * (row_bytes / 16);
  dim3 grid((unsigned)((total + 255) / 256), 2);
  hipLaunchKernelGGL(kv_append_positions_kernel, grid, dim3(256), 0, stream, (char*)k_cache, (char*)v_cache,
                     num_blocks * block_size, table, batch, max_blocks, seq_ids, positions, (const char*)k,
                     (const char*)v, n, n_kv, row_bytes, block_size, slots_out);
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

hipError_t launch_kv_append_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                                 const int32_t* table, int32_t max_blocks, const int32_t* ctx_lens,
                                 const int32_t* cu_new, int32_t batch, int32_t max_new, const void* k_new,
                                 const void* v_new, int32_t new_bytes, int32_t n_kv, int32_t d, int32_t log2_bs,
                                 hipStream_t stream) {
  if (batch == 0 || max_new == 0) return hipSuccess;
  // n consecutive rows starting anywhere in a block of B touch at most (n + B - 2) / B + 1 blocks
  const int B = 1 << log2_bs;
  const int gx = (max_new + B - 2) / B + 1;
  const int pairs = 2 * n_kv, waves = pairs < 16 ? pairs : 16;
  const dim3 grid((unsigned)gx, (unsigned)batch, (unsigned)((pairs + waves - 1) / waves));
  const dim3 block((unsigned)(waves * kWave));
  auto* kc = static_cast<uint8_t*>(k_cache);
  auto* vc = static_cast<uint8_t*>(v_cache);
#define PKV_APPEND_FP8(DD, T)                                                                                   \
  hipLaunchKernelGGL((kv_append_fp8_kernel<DD, T>), grid, block, 0, stream, kc, vc, k_scale, v_scale,          \
                     num_blocks, table, max_blocks, ctx_lens, cu_new, static_cast<const T*>(k_new),             \
                     static_cast<const T*>(v_new), n_kv, log2_bs)
  if (d == 128 && new_bytes == 2) PKV_APPEND_FP8(128, uint16_t);
  else if (d == 128) PKV_APPEND_FP8(128, float);
  else if (new_bytes == 2) PKV_APPEND_FP8(64, uint16_t);
  else PKV_APPEND_FP8(64, float);
#undef PKV_APPEND_FP8
  return hipGetLastError();
}

hipError_t launch_csr_to_table(const int32_t* indptr, const int32_t* indices, int32_t batch, int32_t max_blocks,
                               int32_t* table, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const dim3 grid((unsigned)((max_blocks + 255) / 256), (unsigned)batch);
  hipLaunchKernelGGL(csr_to_table_kernel, grid, dim3(256), 0, stream, indptr, indices, max_blocks, table);
  return hipGetLastError();
}

hipError_t launch_swap(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                       const int32_t* ids, int32_t n, void* image, int64_t block_bytes, int32_t n_kv, int to_image,
                       hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t pieces = block_bytes / 16;
  const dim3 grid((unsigned)((pieces + 255) / 256), (unsigned)n, 2u);
  hipLaunchKernelGGL(swap_kernel, grid, dim3(256), 0, stream, static_cast<char*>(k_cache), static_cast<char*>(v_cache),
                     k_scale, v_scale, num_blocks, ids, n, static_cast<char*>(image), block_bytes, n_kv, to_image);
  return hipGetLastError();
}

// ---- read probe (measurement aid, not part of the attention path) ----
// Streams a buffer with 16-byte loads and keeps only a token of what it read,
// so its duration gives the read bandwidth the memory system delivers to a
// plain kernel: either every 16-byte piece in grid-stride order, or slabs of
// slab_bytes (a multiple of 4 KiB) named by a list, each workgroup reading its
// share of the list one slab after another (the access pattern of one
// (block, KV head) slab of a paged cache).  nt selects non-temporal loads.
template <int NT>
__device__ __forceinline__ u32x4 probe_ld(const char* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

template <int NT>
__global__ __launch_bounds__(256) void read_probe_kernel(const char* __restrict__ buf, int64_t bytes,
                                                         const int32_t* __restrict__ slabs, int32_t per_wg,
                                                         int32_t slab_bytes, int64_t n_slabs,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  if (!slabs) {
    const int64_t n16 = bytes / 16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
      const u32x4 v = probe_ld<NT>(buf + i * 16);
      acc ^= v[0] ^ v[3];
    }
  } else {
    const int32_t* my = slabs + (int64_t)blockIdx.x * per_wg;
    auto slab_at = [&](int j) { return buf + min(max((int64_t)my[j], (int64_t)0), n_slabs - 1) * slab_bytes; };
    if (slab_bytes >= 4096) {
      // four slabs at a time, so each thread keeps four loads in flight
      int j = 0;
      for (; j + 4 <= per_wg; j += 4) {
        const char* sp[4] = {slab_at(j), slab_at(j + 1), slab_at(j + 2), slab_at(j + 3)};
        for (int o = threadIdx.x * 16; o < slab_bytes; o += 256 * 16) {
          u32x4 v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = probe_ld<NT>(sp[q] + o);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc ^= v[q][0] ^ v[q][3];
        }
      }
      for (; j < per_wg; ++j) {
        const char* slab = slab_at(j);
        for (int o = threadIdx.x * 16; o < slab_bytes; o += 256 * 16) {
          const u32x4 v = probe_ld<NT>(slab + o);
          acc ^= v[0] ^ v[3];
        }
      }
    } else {
      // slabs of 1 or 2 KiB: one 4 KiB sweep of the workgroup covers `per`
      // slabs, thread t reading slab t * 16 / slab_bytes of the sweep at byte
      // t * 16 % slab_bytes; four sweeps at a time keep four loads in flight
      const int per = 4096 / slab_bytes;
      const int sub = (int)(threadIdx.x * 16) / slab_bytes, o = (int)(threadIdx.x * 16) % slab_bytes;
      int j = 0;
      for (; j + 4 * per <= per_wg; j += 4 * per) {
        u32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = probe_ld<NT>(slab_at(j + q * per + sub) + o);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc ^= v[q][0] ^ v[q][3];
      }
      for (; j + sub < per_wg; j += per) {
        const u32x4 v = probe_ld<NT>(slab_at(j + sub) + o);
        acc ^= v[0] ^ v[3];
      }
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never stores
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, const int32_t* slabs, int32_t n_list, int32_t slab_bytes,
                             int32_t workgroups, int32_t nt, uint32_t* sink, hipStream_t stream) {
  const int32_t per_wg = slabs ? n_list / workgroups : 0;
  const int64_t n_slabs = slab_bytes > 0 ? bytes / slab_bytes : 0;
  const char* b = reinterpret_cast<const char*>(buf);
  if (nt)
    hipLaunchKernelGGL(read_probe_kernel<1>, dim3(workgroups), dim3(256), 0, stream, b, bytes, slabs, per_wg,
                       slab_bytes, n_slabs, sink);
  else
    hipLaunchKernelGGL(read_probe_kernel<0>, dim3(workgroups), dim3(256), 0, stream, b, bytes, slabs, per_wg,
                       slab_bytes, n_slabs, sink);
  return hipGetLastError();
}

}  // namespace pkv
