// Opt-in device-data checks: the block ids, lengths and slots the attention
// and append calls would use, counted on the device before those calls touch
// anything ("The KV Cache from First Principles", Implementation: the inputs
// are validated before the cache is mutated).  The fast paths never check
// these (ids outside the pool are clamped into it, bad slots skipped), so a
// bad table gives a meaningless result there; with checks on, the call fails
// instead and changes nothing.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

// One workgroup per sequence: its request (decode length, or context plus new
// tokens) must fit its table row, and every table entry the request covers
// must name a block of the pool.
__global__ __launch_bounds__(256) void check_seqs_kernel(SeqCheck c, int32_t* __restrict__ err) {
  const int s = blockIdx.x;
  if (s >= c.batch) return;
  int bad = 0;
  const bool lead = threadIdx.x == 0;
  const int32_t* ids = c.table + (int64_t)s * c.max_blocks;
  int n = c.max_blocks;
  bool row_ok = true;
  if (c.indptr) {
    // CSR: offsets nondecreasing from 0; a sequence whose offsets are not is
    // counted and its entries are not read
    const int b = c.indptr[s], e = c.indptr[s + 1];
    row_ok = b >= 0 && e >= b && (s > 0 || b == 0);
    if (lead && !row_ok) ++bad;
    ids = c.table + (row_ok ? b : 0);
    n = row_ok ? min(e - b, c.max_blocks) : 0;
  }
  int64_t need;
  if (c.mode == SeqCheck::kDecode) {
    const int L = c.lens[s];
    if (lead && L < 0) ++bad;
    need = L;
  } else {
    // context lengths plus the new tokens cu[s] .. cu[s+1]
    const int ctx = c.lens[s];
    const int qb = c.cu[s], qe = c.cu[s + 1];
    const int q = qe - qb;
    if (lead && (ctx < 0 || q < 0 || q > c.max_new || (s == 0 && qb != 0))) ++bad;
    if (lead && c.mode == SeqCheck::kPrefill && s == c.batch - 1 && qe != c.total) ++bad;
    need = (int64_t)max(ctx, 0) + max(q, 0);
  }
  const int64_t cap = (int64_t)n << c.log2_bs;
  if (lead && need > cap) ++bad;
  const int64_t covered = min(max(need, (int64_t)0), cap);
  const int used = (int)((covered + (1 << c.log2_bs) - 1) >> c.log2_bs);
  for (int j = threadIdx.x; j < used; j += blockDim.x) {
    const int id = ids[j];
    if (id < 0 || (int64_t)id >= c.num_blocks) ++bad;
  }
  if (bad) atomicAdd(err, bad);
}

// Slots of an append: negative is padding (allowed); anything at or past the
// pool's end is counted.
__global__ __launch_bounds__(256) void check_slots_kernel(const int64_t* __restrict__ slots, int32_t n, int64_t limit,
                                                          int32_t* __restrict__ err) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int bad = (t < n && slots[t] >= limit) ? 1 : 0;
  const uint64_t m = __builtin_amdgcn_ballot_w64(bad != 0);
  if (m && (threadIdx.x & 63) == __builtin_ctzll(m)) atomicAdd(err, (int)__builtin_popcountll(m));
}

// Slots an append through the table would write: one per (sequence id,
// position) pair, computed as the slot indexing does; a slot at or past
// `limit` counts as bad (-1, padding, does not).
__global__ __launch_bounds__(256) void check_positions_kernel(const int32_t* __restrict__ table, int32_t batch,
                                                              int32_t max_blocks, const int32_t* __restrict__ seq_ids,
                                                              const int32_t* __restrict__ positions, int32_t n,
                                                              int32_t block_size, int64_t limit,
                                                              int32_t* __restrict__ err) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  int bad = 0;
  if (t < n) {
    const int s = seq_ids[t], p = positions[t];
    if (s >= 0 && s < batch && p >= 0 && p < max_blocks * block_size) {
      const int blk = table[(int64_t)s * max_blocks + p / block_size];
      bad = (blk >= 0 && (int64_t)blk * block_size + p % block_size >= limit) ? 1 : 0;
    }
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(bad != 0);
  if (m && (threadIdx.x & 63) == __builtin_ctzll(m)) atomicAdd(err, (int)__builtin_popcountll(m));
}

// Clears n 32-bit words: a kernel rather than a memset, so that a stream
// being captured into a graph records a kernel node.
__global__ __launch_bounds__(256) void zero_words_kernel(int32_t* __restrict__ p, int32_t n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) p[t] = 0;
}

}  // namespace

hipError_t launch_check_seqs(const SeqCheck& c, int32_t* err, hipStream_t stream) {
  if (c.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_seqs_kernel, dim3((unsigned)c.batch), dim3(256), 0, stream, c, err);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t* slots, int32_t n, int64_t limit, int32_t* err, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_slots_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, slots, n, limit,
                     err);
  return hipGetLastError();
}

hipError_t launch_check_positions(const int32_t* table, int32_t batch, int32_t max_blocks, const int32_t* seq_ids,
                                  const int32_t* positions, int32_t n, int32_t block_size, int64_t limit, int32_t* err,
                                  hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_positions_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, table, batch,
                     max_blocks, seq_ids, positions, n, block_size, limit, err);
  return hipGetLastError();
}

hipError_t launch_zero_words(int32_t* p, int32_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace pkv
