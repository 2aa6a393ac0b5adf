// Host-side launch interfaces shared by the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// the queue decode mode keeps per-sequence item prefix sums in LDS (4 bytes each)
constexpr int kDecodeMaxQueueBatch = 4096;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;  // 2-D [batch][max_blocks], or CSR page ids when indptr is set
  const int32_t* indptr;       // CSR: sequence s owns block_table[indptr[s] .. indptr[s+1])
  const int32_t* seq_lens;
  float* ws_o;    // [batch][n_q][n_parts][d] partial outputs (unnormalised)
  float* ws_ml;   // [batch][n_q][n_parts][2] running max (log2 units) and sum
                  // (queue mode: [item][heads per workgroup][d] and [...][2])
  int* split_info;  // queue mode: int4 per (sequence, KV head chunk): first and last item
  unsigned* dyn_counter;  // queue mode: item counter, zero before the call and rewound to zero by it
  int32_t n_wg;     // queue mode: workgroups (0 = partition mode)
  int32_t merge_splits;  // queue mode: merge workgroups per pair (divides the heads per workgroup)
  int32_t n_slots;       // queue mode: partial-state slots in the workspace
  int32_t items_per_wg;  // queue mode: items the batch is cut into per workgroup
  int64_t num_blocks;
  int32_t batch;
  int32_t max_blocks;   // table row width (CSR: bound on the pages of one sequence)
  int32_t log2_bs;      // tokens per cache block = 1 << log2_bs (8 .. 256)
  int32_t n_q;
  int32_t n_kv;
  int32_t group;        // n_q / n_kv
  int32_t head_chunks;  // group / heads per workgroup
  int32_t part_tokens;
  int32_t n_parts;
  int32_t out_bf16;
  int32_t use_mfma;     // partition mode: the matrix-core split kernel (decode_mfma.hip)
  const int32_t* work_order;  // partition mode: sequence slot -> sequence (a permutation), or null
  int32_t order_units;        // work_order is a unit list (entry i: sequence * n_parts + partition, or -1)
  float scale_log2;     // softmax scale * log2(e)
};

// decode: kv_kind 0 f32 / 1 bf16 / 2 fp8; returns hipSuccess or the launch error
int decode_heads_per_wg(int group);
int decode_chunk_blocks(int heads_per_wg);
int decode_partition_wgs_per_cu(int kv_kind, int d, int heads_per_wg);
int decode_queue_lds_bytes(int batch);  // dynamic LDS of the queue kernel
int decode_queue_items_per_wg();           // items the queue kernel aims for per workgroup
int decode_queue_max_item_blocks();      // largest item the queue kernel makes
int decode_queue_wgs_per_cu(int kv_kind, int d, int heads_per_wg, int batch);
hipError_t launch_decode(const DecodeArgs& a, int kv_kind, int d, hipStream_t stream);
// order[slot] = sequence: sequences ranked by length (longer first, ties by
// index); pair != 0 puts the k-th longest and the k-th shortest in slots s
// and s + ceil(batch / 2)
hipError_t launch_decode_order(const int32_t* seq_lens, int32_t batch, int32_t pair, int32_t* order,
                               hipStream_t stream);
// order[rank] = unit (sequence * n_parts + partition) by token count, more
// first; units without tokens rank last as -1
hipError_t launch_decode_unit_order(const int32_t* seq_lens, int32_t batch, int32_t n_parts, int32_t part_tokens,
                                    int32_t* order, hipStream_t stream);
// matrix-core decode (partition mode only): bf16 / fp8 KV, d = 128, 4, 8 or 16 heads per workgroup
bool decode_mfma_supported(int kv_kind, int d, int heads_per_wg);
int decode_mfma_wgs_per_cu(int kv_kind, int heads_per_wg);
hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_kind, hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* table, int32_t batch, int32_t max_blocks, const int32_t* seq_ids,
                               const int32_t* positions, int32_t n, int32_t block_size, int64_t* out,
                               hipStream_t stream);
hipError_t launch_kv_append(void* k_cache, void* v_cache, int64_t num_blocks, const int64_t* slots, const void* k,
                            const void* v, int32_t n, int32_t n_kv, int32_t row_bytes, int32_t block_size,
                            hipStream_t stream);
hipError_t launch_kv_append_positions(void* k_cache, void* v_cache, int64_t num_blocks, const int32_t* table,
                                      int32_t batch, int32_t max_blocks, const int32_t* seq_ids,
                                      const int32_t* positions, const void* k, const void* v, int32_t n, int32_t n_kv,
                                      int32_t row_bytes, int32_t block_size, int64_t* slots_out, hipStream_t stream);
hipError_t launch_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache, int64_t num_blocks,
                         const int32_t* table, int32_t max_blocks, const int32_t* seq_lens, const int64_t* cu,
                         int64_t total_rows, int32_t batch, int32_t n_kv, int32_t row_bytes, int32_t block_size,
                         hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                              const int32_t* src, const int32_t* dst, int32_t n_pairs, int64_t block_bytes,
                              int32_t n_kv, hipStream_t stream);
hipError_t launch_kv_append_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                                 const int32_t* table, int32_t max_blocks, const int32_t* ctx_lens,
                                 const int32_t* cu_new, int32_t batch, int32_t max_new, const void* k_new,
                                 const void* v_new, int32_t new_bytes, int32_t n_kv, int32_t d, int32_t log2_bs,
                                 hipStream_t stream);
hipError_t launch_swap(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                       const int32_t* ids, int32_t n, void* image, int64_t block_bytes, int32_t n_kv, int to_image,
                       hipStream_t stream);
hipError_t launch_csr_to_table(const int32_t* indptr, const int32_t* indices, int32_t batch, int32_t max_blocks,
                               int32_t* table, hipStream_t stream);
hipError_t launch_read_probe(const void* buf, int64_t bytes, const int32_t* slabs, int32_t n_list, int32_t slab_bytes,
                             int32_t workgroups, int32_t nt, uint32_t* sink, hipStream_t stream);
hipError_t launch_check_tables(const int32_t* table, int32_t max_blocks, const int32_t* seq_lens, int32_t batch,
                               int64_t num_blocks, int32_t block_size, int32_t* err, hipStream_t stream);

// Device-data check of one call's sequences (device_check.hip): each
// sequence's request must fit its table row and every entry it covers must
// name a pool block.
struct SeqCheck {
  enum Mode : int32_t { kDecode = 0, kPrefill = 1, kAppend = 2 };
  const int32_t* table;   // 2-D [batch][max_blocks], or CSR page ids
  const int32_t* indptr;  // CSR offsets [batch + 1], or null
  const int32_t* lens;    // decode: seq_lens; prefill / append: context lengths
  const int32_t* cu;      // prefill / append: new-token offsets [batch + 1]
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t batch;
  int32_t log2_bs;
  int32_t mode;
  int32_t max_new;        // prefill: max_q_len; append: max_new_len
  int32_t total;          // prefill: total_q (cu[batch] must equal it)
};
hipError_t launch_check_seqs(const SeqCheck& c, int32_t* err, hipStream_t stream);
hipError_t launch_check_slots(const int64_t* slots, int32_t n, int64_t limit, int32_t* err, hipStream_t stream);
hipError_t launch_check_positions(const int32_t* table, int32_t batch, int32_t max_blocks, const int32_t* seq_ids,
                                  const int32_t* positions, int32_t n, int32_t block_size, int64_t limit, int32_t* err,
                                  hipStream_t stream);
hipError_t launch_zero_words(int32_t* p, int32_t n, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_q;
  const int32_t* ctx_lens;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;  // FP8 KV: per (block, KV head)
  const float* v_scale;
  const int32_t* block_table;  // as in DecodeArgs
  const int32_t* indptr;
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_q_len;
  int32_t max_blocks;
  int32_t log2_bs;
  int32_t n_q;
  int32_t n_kv;
  int32_t group;
  int32_t causal;
  int32_t out_bf16;
  int32_t kv_fp8;
  float scale_log2;
};
hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t stream);
// both products in FP8 (prefill_fp8.hip): FP8 KV, d = 128, group divides 128;
// split: queries and weights carried as two E4M3 terms each
hipError_t launch_prefill_fp8_mma(const PrefillArgs& a, bool split, hipStream_t stream);
bool prefill_supported_group(int group);


// ---- page-table walk shared by the attention kernels ----
// A sequence's blocks: a row of the 2-D table, or its CSR slice (at most
// max_blocks entries).  The kernels work in 16-token tiles made of two 8-token
// halves; half h of tile q holds tokens 16 q + 8 h .. + 7, all in one cache
// block for every block size from 8 to 256.
struct PageRow {
  const int32_t* ids;
  int32_t n;  // entries of the row
};

template <class A>
__device__ __forceinline__ PageRow page_row(const A& a, int s) {
  if (a.indptr) {
    const int b = a.indptr[s], e = a.indptr[s + 1];
    return {a.block_table + b, min(max(e - b, 0), a.max_blocks)};
  }
  return {a.block_table + (int64_t)s * a.max_blocks, a.max_blocks};
}

// Block id of the block holding sequence token `tok`: entries past the row and
// ids outside the pool are clamped into it (the rows they lead to are masked).
template <class A>
__device__ __forceinline__ int page_block(const A& a, const PageRow& r, int tok) {
  const int j = tok >> a.log2_bs;
  const int id = j < r.n ? r.ids[j] : 0;
  return min(max(id, 0), (int)(a.num_blocks - 1));
}

// Row index of token `tok` in the [num_blocks][n_kv][B] row space of KV head
// kvh, block `id` (the host keeps num_blocks * n_kv * B below 2^32).
template <class A>
__device__ __forceinline__ uint32_t page_row_index(const A& a, int id, int kvh, int tok) {
  return (((uint32_t)id * (uint32_t)a.n_kv + (uint32_t)kvh) << a.log2_bs) | (uint32_t)(tok & ((1 << a.log2_bs) - 1));
}

}  // namespace pkv
