/*
 * pkv.h -- C ABI of libpkv: attention over a paged KV cache on AMD MI355X
 * (gfx950).
 *
 * The operations follow three web pages:
 *   [KVP] "KV cache, PagedAttention and FlashAttention"
 *   [MEM] "Memory Management in LLM Serving Systems"
 *   [FP ] "The KV Cache from First Principles"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked (device) must point to GPU memory of the current HIP
 *    device; pointers marked (host) to host memory.  The caller owns every
 *    buffer, including workspaces, whose sizes the *_workspace() calls give.
 *    The library allocates no device memory and keeps no state between
 *    calls beyond cached device properties, the device-check switch and its
 *    counter (a small file-scope device array per GPU); the host-side block
 *    pool object below is created and destroyed by the caller.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it and the call returns without synchronising.
 *  - Cache layout, one layer: cache[num_blocks][n_kv_heads][block_size][d_head],
 *    row-major, so one (block, KV head) slab of block_size x d_head values is
 *    contiguous.  A flat slot id is physical_block * block_size + offset.
 *    One block table serves every layer: a physical block id names the same
 *    token range in each layer's pool ([KVP] Problem 4, "The idea": a block
 *    holds a fixed number of tokens across the layers' heads).
 *  - block_table is int32 [batch][max_blocks_per_seq], row-major; entry j of
 *    row s is the physical block of sequence s's logical block j.
 *  - Errors: every argument is checked on the host before anything is
 *    launched, so a call that returns an error has changed nothing on the
 *    device (validate before mutate: [FP] "Implementation" checks the head
 *    ratio before the cache is touched).  pkv_last_error() then describes
 *    the failure (thread-local).  Device data (block ids, lengths, slots) is
 *    not validated by the attention calls: ids outside [0, num_blocks) are
 *    clamped into the pool so no access leaves it, but such a result is
 *    meaningless; pkv_set_device_checks() turns on a checked mode that
 *    validates it on the device first (PKV_ERR_DEVICE_CHECK).
 *  - Slots past a sequence's length and blocks no table names may hold any
 *    bytes, NaN included; they never affect a result.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 3

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad head ratio */
  PKV_ERR_UNSUPPORTED = 2, /* valid but not implemented (d_head, block_size, dtype combination) */
  PKV_ERR_WORKSPACE = 3,   /* workspace smaller than the *_workspace() size */
  PKV_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  PKV_ERR_NO_BLOCKS = 5,   /* a block pool has too few free blocks for the request */
  PKV_ERR_DEVICE_CHECK = 6 /* device checks on: a length, block id or slot on the device is invalid */
} pkv_status;

/* Element types. FP8 is OCP E4M3FN (bias 7, max 448, S.1111.111 = NaN), with
 * one fp32 scale per (block, KV head): value = e4m3fn(byte) * scale.  The two
 * range markers are no element types: they make every int32 value a value of
 * the type in C++ as in C, so a call given an unknown code rejects it
 * (PKV_ERR_INVALID_ARG) rather than receive a value outside the enumeration. */
typedef enum {
  PKV_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3FN = 2,
  PKV_DTYPE_RANGE_MAX_ = 2147483647
} pkv_dtype;

int pkv_abi_version(void);
const char* pkv_status_string(int status);
/* Message for the last error returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Device checks (opt-in, for debugging; [FP] "Implementation" validates the
 * inputs before the cache is mutated).  The attention and append calls do not
 * read their device-resident inputs on the host, and their kernels do not
 * validate them: block ids outside the pool are clamped into it, bad slots
 * skipped, lengths capped at the table row, so a bad table gives a
 * meaningless result, never an access outside the pool.  With checks on
 * (process-wide switch, off by default), every call of pkv_kv_append,
 * pkv_kv_append_fp8, the pkv_paged_attn_decode* and the
 * pkv_paged_attn_prefill_chunk* calls first counts on the device, on the
 * caller's stream:
 *   - decode: seq_lens[s] < 0 or > the row's capacity (entries x B);
 *   - prefill / fp8 append: context_lens[s] < 0, a new-token count < 0 or
 *     above max_q_len / max_new_len, cu_*[0] != 0, cu_q_lens[num_seqs] !=
 *     total_q, context + new tokens > the row's capacity;
 *   - every table entry the request covers outside [0, num_blocks); CSR
 *     offsets that decrease or do not start at 0;
 *   - kv_append: a slot >= num_blocks * B (negative slots are padding);
 * then waits for the stream (so calls are synchronous and cannot be captured
 * into a graph) and, if anything was counted, returns PKV_ERR_DEVICE_CHECK
 * without launching the call's work: nothing is changed.  The counter is a
 * file-scope device array of the library, one per GPU; checks from several
 * threads are serialised.  CSR offsets must still index kv_indices (the
 * check reads the entries they name). */
void pkv_set_device_checks(int enable);
/* 1 if device checks are on, else 0. */
int pkv_device_checks(void);

/* Per-token KV-cache bytes: 2 (K and V) x n_layers x n_kv_heads x d_head x
 * bytes_per_value ([KVP] Problem 3, "The concepts"; [MEM] "KV cache sizing").
 * Returns -1 if an argument is negative. Host-only arithmetic. */
int64_t pkv_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t d_head, int32_t bytes_per_value);

/* Slot indexing ([KVP] Problem 4, "The idea": block = p // B, offset = p % B,
 * address = block_table[seq][block] * block_bytes + offset * token_bytes;
 * [MEM] "Walking the table"):
 *   slot[t] = block_table[seq_ids[t]][positions[t] / B] * B + positions[t] % B
 * seq_ids, positions: (device) int32 [num_tokens]; slot_mapping_out: (device)
 * int64 [num_tokens].  A pair with seq_id outside [0, batch), position outside
 * [0, max_blocks_per_seq * B) or a negative table entry yields slot -1
 * (padding).  num_tokens == 0 is a no-op. */
pkv_status pkv_slot_mapping(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                            const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                            int32_t block_size, int64_t* slot_mapping_out, void* stream);

/* Append ([FP] "Deriving the cache": compute a token's key and value once and
 * keep them; [KVP] Problem 4: blocks are filled as tokens arrive):
 *   k_cache[slot / B][h][slot % B][:] = k[t][h][:]  (and v), for every KV head h.
 * A bit copy in the cache's element type (FP8 bytes must be pre-quantised).
 * k, v: (device) [num_tokens][n_kv_heads][d_head]; slot_mapping: (device)
 * int64 [num_tokens]; a slot < 0 or >= num_blocks * B is skipped.  Two tokens
 * with the same slot race (the result is one of them). */
pkv_status pkv_kv_append(void* k_cache, void* v_cache, pkv_dtype cache_dtype, int64_t num_blocks,
                         const int64_t* slot_mapping, const void* k, const void* v, int32_t num_tokens,
                         int32_t n_kv_heads, int32_t d_head, int32_t block_size, void* stream);

/* Slot indexing and append in one launch: for every token t,
 *   slot = block_table[seq_ids[t]][positions[t] / B] * B + positions[t] % B
 * exactly as pkv_slot_mapping computes it (-1 for a pair outside the table or
 * a negative entry), then its K and V rows are copied as pkv_kv_append copies
 * them (a slot < 0 or >= num_blocks * B is skipped).  The result equals
 * pkv_slot_mapping followed by pkv_kv_append, bit for bit; the pages' append
 * step ([FP] "Deriving the cache"; [KVP] Problem 4, "The idea") with the
 * table walk inside.  slot_mapping_out: (device) int64 [num_tokens] receiving
 * the slots, or NULL.  Other arguments as pkv_slot_mapping and pkv_kv_append.
 * num_tokens == 0 is a no-op. */
pkv_status pkv_kv_append_positions(void* k_cache, void* v_cache, pkv_dtype cache_dtype, int64_t num_blocks,
                                   const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                                   const int32_t* seq_ids, const int32_t* positions, const void* k, const void* v,
                                   int32_t num_tokens, int32_t n_kv_heads, int32_t d_head, int32_t block_size,
                                   int64_t* slot_mapping_out, void* stream);

/* Append with FP8 quantisation ([KVP] Problem 3: an FP8 cache takes half the
 * bytes of a 16-bit one; [MEM] "Long-context optimization": quantising the
 * cached keys and values shrinks the per-token cost).  The pages fix neither
 * the scale granularity nor how a scale evolves while a block fills token by
 * token; this library keeps one fp32 scale per (block, KV head) (the FP8
 * format above) and its rule is:
 *   - appending rows to (block, KV head) sets
 *     scale = max(old scale, max |new values| / 448), the old scale counting
 *     only if the block already holds rows of the sequence;
 *   - if the scale grew, the block's existing rows are re-encoded:
 *     code = nearest(e4m3fn(code) * old / new);
 *   - a new value x is stored as nearest(x / scale); a block whose scale is 0
 *     (all values zero) stores code 0.
 * nearest() picks the closest E4M3FN value, ties to an even mantissa field,
 * magnitudes above 448 saturating to 448, the sign kept (zero included); every
 * product, quotient and the division by 448 is one fp32 operation.
 * Sequence s appends its rows cu_new_lens[s] .. cu_new_lens[s+1] - 1 of
 * k_new / v_new at positions context_lens[s] onwards, through its table row.
 *   k_cache, v_cache: (device) FP8 [num_blocks][n_kv_heads][B][d_head];
 *   k_scale, v_scale: (device) f32 [num_blocks][n_kv_heads], read and written;
 *   block_table: (device) int32 [batch][max_blocks_per_seq];
 *   context_lens: (device) int32 [batch], tokens already cached;
 *   cu_new_lens: (device) int32 [batch + 1], nondecreasing, starting at 0;
 *     each cu_new_lens[s+1] - cu_new_lens[s] <= max_new_len (more is not
 *     appended past the first max_new_len / B + 1 blocks);
 *   k_new, v_new: (device) new_dtype (BF16 or F32) [total_new][n_kv_heads][d_head].
 * A sequence with a negative context length, positions past
 * max_blocks_per_seq * B and table entries outside [0, num_blocks) are
 * skipped.  The blocks appended to must be named by one sequence only (a
 * shared block is copied first: pkv_pool_prepare_append); two sequences
 * writing one block race.  Supported: block_size 8, 16, 32, 64, 128 or 256;
 * d_head 64 or 128; pointers 16-byte aligned.  batch == 0 or max_new_len == 0 is a no-op. */
pkv_status pkv_kv_append_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                             const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                             const int32_t* cu_new_lens, int32_t batch, int32_t max_new_len, const void* k_new,
                             const void* v_new, pkv_dtype new_dtype, int32_t n_kv_heads, int32_t d_head,
                             int32_t block_size, void* stream);

/* Gather (test/debug export of the block-table walk of [MEM] "Walking the
 * table"): k_out[cu_seq_lens[s] + p][h][:] = k_cache[block_table[s][p / B]][h][p % B][:]
 * for p < seq_lens[s]; same for v.  k_out, v_out: (device)
 * [total_tokens][n_kv_heads][d_head] with total_tokens = sum(seq_lens);
 * seq_lens (device) int32 [batch]; cu_seq_lens (device) int64 [batch + 1]
 * (exclusive prefix sums).  Rows that would land outside [0, total_tokens)
 * are not written. */
pkv_status pkv_paged_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                            int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int64_t* cu_seq_lens, int64_t total_tokens,
                            int32_t batch, int32_t n_kv_heads, int32_t d_head, int32_t block_size, void* stream);

/* Read probe, a measurement aid outside the attention path: the bandwidth a
 * plain kernel gets from HBM, to set beside the decode figures.  Reads the
 * device buffer buf (bytes, a multiple of 16) with 16-byte loads on
 * `workgroups` workgroups of 256 threads: with slab_list == NULL every byte in
 * grid-stride order; otherwise the slabs of slab_bytes (1024, 2048 or a multiple of 4096)
 * named by slab_list (device int32 [n_list], entries clamped into the buffer),
 * workgroup w reading entries w * (n_list / workgroups) onward one slab after
 * another, the pattern of one (block, KV head) slab of a paged cache.
 * nontemporal != 0 sets the nt bit on the loads.  sink (device uint32) is
 * written only in the practically impossible case that the folded data equals
 * a fixed pattern.  Errors: INVALID_ARG for null pointers, sizes out of range
 * or fewer list entries than workgroups; HIP for launch failures. */
pkv_status pkv_read_probe(const void* buf, int64_t bytes, const int32_t* slab_list, int32_t n_list,
                          int32_t slab_bytes, int32_t workgroups, int32_t nontemporal, uint32_t* sink, void* stream);

/* Device-side table check, asynchronous and for a 2-D table (the device
 * checks above do the same per call, synchronously): counts, into
 * *error_count (device int32, which the caller zeroes first), every sequence
 * with seq_lens[s] < 0 or > max_blocks_per_seq * B and every table entry a
 * sequence uses (logical block < ceil(seq_len / B)) that lies outside
 * [0, num_blocks). */
pkv_status pkv_check_tables(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t batch, int64_t num_blocks, int32_t block_size, int32_t* error_count,
                            void* stream);

/* ---- Block sharing: reference counts and copy-on-write ----
 * [KVP] Problem 4, "The idea": blocks are handed out only when a sequence's
 * previous block fills; because sequences reach blocks through their tables,
 * several can name the same physical blocks -- parallel samples and beam
 * branches share the prompt's blocks -- with a reference count per block, and
 * a block named by more than one table is copied before it is written
 * (copy-on-write); [MEM] "Prefix sharing" stores a shared prefix once.
 *
 * pkv_block_pool is host bookkeeping only (reference counts and the free
 * list; it never touches the device).  Free blocks are handed out lowest id
 * first, so a sequence of operations has one outcome.  Each call locks the
 * pool, so pools may be used from several threads.  Calls that fail change
 * nothing. */
typedef struct pkv_block_pool pkv_block_pool;

/* Creates a pool of num_blocks (1 .. 2^31 - 1) free blocks in *pool_out. */
pkv_status pkv_pool_create(int64_t num_blocks, pkv_block_pool** pool_out);
void pkv_pool_destroy(pkv_block_pool* pool);
/* Free blocks, or -1 for a NULL pool. */
int64_t pkv_pool_free_blocks(pkv_block_pool* pool);
/* How many tables name `block` (0 = free), or -1 if it is not in the pool. */
int32_t pkv_pool_refcount(pkv_block_pool* pool, int32_t block);
/* n fresh blocks, each named once, into ids_out (host int32 [n]);
 * PKV_ERR_NO_BLOCKS if fewer than n are free. */
pkv_status pkv_pool_alloc(pkv_block_pool* pool, int32_t n, int32_t* ids_out);
/* One more table names each of ids (host int32 [n]): a fork.  Every id must
 * be allocated (else PKV_ERR_INVALID_ARG). */
pkv_status pkv_pool_share(pkv_block_pool* pool, const int32_t* ids, int32_t n);
/* One table fewer names each of ids; a block no table names is free again.
 * Every id must be allocated, counted with multiplicity. */
pkv_status pkv_pool_release(pkv_block_pool* pool, const int32_t* ids, int32_t n);
/* Before appending n_new tokens to a sequence of seq_len tokens whose table
 * row (host int32 [max_blocks_per_seq], entries < ceil(seq_len / block_size)
 * valid) names blocks of this pool: makes every block that positions
 * seq_len .. seq_len + n_new - 1 fall into writable by this sequence alone.
 * A logical block past the row's last is allocated; an existing one named by
 * other tables too (only the partly filled last block can be one) is
 * replaced in the row by a fresh block, whose contents must be copied from
 * the old one before the append: *n_copies (0 or 1) gets the count and
 * *copy_src / *copy_dst the pair, for pkv_copy_blocks.  The row is updated
 * in place.  PKV_ERR_NO_BLOCKS if the pool cannot supply the blocks;
 * PKV_ERR_INVALID_ARG if the row is too short or names a block outside the
 * pool or not allocated. */
pkv_status pkv_pool_prepare_append(pkv_block_pool* pool, int32_t* table_row, int32_t max_blocks_per_seq,
                                   int32_t seq_len, int32_t n_new, int32_t block_size, int32_t* copy_src,
                                   int32_t* copy_dst, int32_t* n_copies);

/* Copies whole blocks src[i] -> dst[i] of one layer's K and V pools (every KV
 * head and slot, bit for bit) and, when k_scale / v_scale are given (FP8
 * caches), their per-(block, KV head) scales: the copy of copy-on-write.
 * src, dst: (device) int32 [n_pairs]; a pair naming a block outside
 * [0, num_blocks) is skipped.  No dst may equal a src of the same call. */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, pkv_dtype cache_dtype, float* k_scale, float* v_scale,
                           int64_t num_blocks, const int32_t* src, const int32_t* dst, int32_t n_pairs,
                           int32_t n_kv_heads, int32_t d_head, int32_t block_size, void* stream);

/* ---- Preemption by swap ([KVP] Problem 4, "The idea" and "Trade-offs": when
 * memory runs out a sequence's blocks can be moved to CPU memory and brought
 * back later instead of recomputed; a sequence reaches its blocks only
 * through its table, so they may come back into any free blocks).
 * Host image of n listed blocks: [K of block 0 .. n-1][V of block 0 .. n-1]
 * [K scales][V scales], a block's K (or V) being its whole slab
 * (n_kv_heads x block_size x d_head elements) and the scale sections
 * (n x n_kv_heads fp32 each) present for FP8 caches only. */

/* Bytes of the host image (and of the staging buffer) for n_blocks blocks;
 * 0 for invalid arguments. */
size_t pkv_swap_image_bytes(int32_t n_blocks, pkv_dtype cache_dtype, int32_t n_kv_heads, int32_t d_head,
                            int32_t block_size);

/* Swap out: packs blocks block_ids[0 .. n_blocks) (device int32; an id
 * outside [0, num_blocks) leaves its image slot unwritten) into `staging`
 * (device, 16-byte aligned, >= pkv_swap_image_bytes, else
 * PKV_ERR_WORKSPACE), then copies the image to `host_image` (host memory the
 * caller allocated pinned, e.g. hipHostMalloc, for the copy to run
 * asynchronously on the DMA engines; pageable memory works but the copy may
 * block), both on `stream`.  The image is complete once the stream reaches
 * this point; staging and host_image must not be reused before.  The blocks
 * themselves are unchanged (freeing them is the caller's pool operation).
 * k_scale / v_scale: given exactly for FP8 caches.  n_blocks == 0 is a
 * no-op; at most 65535 blocks per call. */
pkv_status pkv_swap_out(const void* k_cache, const void* v_cache, pkv_dtype cache_dtype, const float* k_scale,
                        const float* v_scale, int64_t num_blocks, const int32_t* block_ids, int32_t n_blocks,
                        void* staging, size_t staging_bytes, void* host_image, int32_t n_kv_heads, int32_t d_head,
                        int32_t block_size, void* stream);

/* Swap in: copies `host_image` (as written by pkv_swap_out for n_blocks
 * blocks) to `staging`, then writes its i-th block (K, V and FP8 scales) into
 * device block block_ids[i]; ids outside the pool are skipped.  The listed
 * blocks may differ from the ones swapped out; the caller points the
 * sequence's table at them.  Arguments as pkv_swap_out. */
pkv_status pkv_swap_in(void* k_cache, void* v_cache, pkv_dtype cache_dtype, float* k_scale, float* v_scale,
                       int64_t num_blocks, const int32_t* block_ids, int32_t n_blocks, void* staging,
                       size_t staging_bytes, const void* host_image, int32_t n_kv_heads, int32_t d_head,
                       int32_t block_size, void* stream);

/* Paged decode attention: one query per sequence attends every cached token
 * of its sequence, the current one included ([FP] "The redundancy"; [KVP]
 * Problem 5, "Serving note": decode reads K and V once):
 *   out[s][h] = sum_p softmax_p(scale * q[s][h] . K_s[p]) V_s[p],  p < seq_lens[s],
 * with K_s/V_s the rows of KV head h / (n_q_heads / n_kv_heads) gathered
 * through block_table ([MEM] "MHA, MQA, and GQA"; [FP] "Grouped-query
 * attention").  Computed FlashAttention-style ([KVP] Problem 5, "Tiling",
 * "Online softmax"; [MEM] "FlashAttention-2"): the sequence is split across
 * workgroups, each keeping a running max and sum, and the pieces are merged;
 * scores never reach memory.  With bf16 or fp8 KV, d_head 128 and 4, 8 or
 * 16 query heads per KV head (or per chunk of them) the split kernel does the
 * dot products on the matrix cores, always in fixed partitions of at most
 * 4096 tokens; otherwise the split is the library's choice: fixed
 * partitions per (sequence, KV head) when equal partitions of at most 4096
 * tokens give one resident workgroup each, otherwise the work-queue split:
 * each (sequence, KV head) is cut into items of equal block counts, a
 * resident set of workgroups claims items from a counter in the workspace,
 * and a merge pass combines the items of each sequence (any length mix,
 * batch <= 4096).  pkv_paged_attn_decode_partitioned picks either one
 * explicitly.
 *   q: (device) [batch][n_q_heads][d_head]; out: (device) same shape.
 *   k_cache, v_cache: (device) [num_blocks][n_kv_heads][block_size][d_head].
 *   k_scale, v_scale: (device) fp32 [num_blocks][n_kv_heads] for FP8, else NULL.
 *   seq_lens: (device) int32 [batch], 0 <= seq_lens[s] <= max_blocks_per_seq * B;
 *   a sequence of length 0 yields zeros.
 * Supported: d_head in {64, 128}; block_size 8, 16, 32, 64, 128 or 256
 * ([KVP] Problem 4, "Trade-offs": small blocks waste less, large ones read
 * more contiguously); num_blocks * n_kv_heads * block_size <= 2^32; (q, kv)
 * in {(F32, F32), (BF16, BF16), (BF16, FP8_E4M3FN)}; out F32 or BF16;
 * n_q_heads a multiple of n_kv_heads.  workspace: (device) at least
 * pkv_paged_attn_decode_workspace(...) bytes, 256-byte aligned.  It must be
 * zero-filled before its first use: the work-queue split keeps its item
 * counter there, and every call leaves the counter at zero again, so a
 * workspace reused call after call (graph replays included) needs no further
 * clearing.  The rest is scratch for the call.  Calls that share one
 * workspace must be ordered (same stream).  The result is deterministic: the
 * same inputs and launch give the same bits, whichever workgroup ran which
 * item.
 * Accumulation is fp32; with bf16/fp8 KV the softmax weights are rounded to
 * bf16 before the value product and the normaliser sums the same rounded
 * weights. */
pkv_status pkv_paged_attn_decode(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                 const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                 const float* k_scale, const float* v_scale, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                 int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                 int32_t block_size, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Same as pkv_paged_attn_decode with an explicit split: partition_tokens > 0
 * gives fixed partitions of that many tokens per (sequence, KV head), one
 * workgroup each, and must be a multiple of 256 (of 64 * the chunk of the
 * head group) up to 4096; -1 asks for the work-queue split (batch <= 4096,
 * else PKV_ERR_UNSUPPORTED); 0 is the library's choice.  Used to test that
 * results do not depend on the split and to tune it. */
pkv_status pkv_paged_attn_decode_partitioned(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                             const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                             const float* k_scale, const float* v_scale,
                                             const int32_t* block_table, int32_t max_blocks_per_seq,
                                             const int32_t* seq_lens, int32_t batch, int64_t num_blocks,
                                             int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                             int32_t block_size, float scale, int32_t partition_tokens,
                                             void* workspace, size_t workspace_bytes, void* stream);

/* Decode for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): as
 * pkv_paged_attn_decode_partitioned (partition_tokens: 0 = the library's
 * split, > 0 fixed partitions, -1 the work-queue split), without a workspace
 * argument.  The partial results of a split call (and the work-queue split's
 * item counter) go to a static scratch array of the library, 32 MiB in each
 * GPU's memory, held from the call's first use on that GPU until the process
 * ends; this call allocates nothing.  A decode whose workspace
 * (pkv_paged_attn_decode_workspace) exceeds 32 MiB fails with
 * PKV_ERR_WORKSPACE before any launch (the 70B-shaped 32K decode needs about
 * 2 MB, batch 256 of 8192 tokens with 64 query heads about 17 MB).  Every
 * call on one GPU shares that GPU's scratch, which keeps the last call's
 * bytes (the item counter is cleared by each call): two such calls whose
 * work overlaps in time on one GPU (different streams, or threads) race and
 * give wrong results; order them on one stream.  Results equal
 * pkv_paged_attn_decode_partitioned's bit for bit.  Other arguments and
 * errors as pkv_paged_attn_decode. */
pkv_status pkv_paged_attn_decode_noalloc(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                         const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                         int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                         int32_t block_size, float scale, int32_t partition_tokens, void* stream);

/* Workspace bytes the decode call needs on the current device (partition_tokens
 * as above, 0 = the library's choice).  Returns 0 for invalid arguments, or
 * when the split depends on the device and no device is present. */
size_t pkv_paged_attn_decode_workspace(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                       int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype kv_dtype,
                                       int32_t partition_tokens);

/* How the decode call with these arguments splits its work on the current
 * device (partition_tokens as for pkv_paged_attn_decode_partitioned).  info:
 * (host) int32[7], filled with {split: 0 fixed partitions / 1 work queue,
 * partition tokens (0 for the queue), partitions per (sequence, KV head)
 * (0 for the queue), workgroups of the split kernel, 1 if a merge pass
 * follows else 0, query heads per workgroup, 1 if the split kernel is the
 * matrix-core one else 0}.  Errors as for the decode
 * call's argument checks; PKV_ERR_HIP when the split needs a device and none
 * is present. */
pkv_status pkv_paged_attn_decode_plan(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                      int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype kv_dtype,
                                      int32_t partition_tokens, int32_t* info);

/* Work order for the decode calls of one step (every layer decodes the same
 * batch), the order pkv_paged_attn_decode_ordered takes; work_order_out is
 * device int32 with pkv_paged_attn_decode_order_entries() entries.
 *  - When the library's split gives each sequence one partition (or the work
 *    queue), the entries are a permutation of 0 .. batch - 1: the sequences
 *    ranked by length (longer first, ties by index).  When every split
 *    workgroup is resident at once (workgroups i and i + half the grid share
 *    a CU) the k-th longest sequence is paired with the k-th shortest;
 *    otherwise the longest come first, so the short ones fill the end.
 *  - When the split has several partitions per sequence (and at most 8192
 *    (sequence, partition) units), the entries list the units u = sequence *
 *    n_parts + partition, ranked by their token counts (more first, ties by
 *    index), followed by -1 for every unit without tokens: a long sequence's
 *    later partitions then start with the other long work, and the empty
 *    units come last.
 * Balancing is this library's addition to the pages' split of a sequence
 * across thread blocks ([KVP] Problem 5, serving note).  Arguments as
 * pkv_paged_attn_decode_plan; one launch of about entries^2 comparisons,
 * meant to run once per step. */
pkv_status pkv_paged_attn_decode_order(const int32_t* seq_lens, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t d_head, int32_t max_blocks_per_seq, int32_t block_size,
                                       pkv_dtype kv_dtype, int32_t* work_order_out, void* stream);

/* Entries of the work order for these arguments (host call): batch, or batch
 * * partitions per sequence when the order lists (sequence, partition) units;
 * 0 for invalid arguments or when the split needs a device and none is
 * present. */
int32_t pkv_paged_attn_decode_order_entries(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                            int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype kv_dtype);

/* Decode as pkv_paged_attn_decode (the library's split) with the split
 * grid's work taken in work_order (device int32, as pkv_paged_attn_decode_order
 * writes it: a permutation of the sequences, or the list of (sequence,
 * partition) units followed by -1s; entries are clamped into range, so
 * anything else computes some work twice and leaves other outputs unwritten
 * or unmerged).  Every (sequence, head, partition) is computed the same way
 * whichever workgroup takes it, so the output is bit-identical to
 * pkv_paged_attn_decode's for any such order.  The work-queue split ignores
 * the order. */
pkv_status pkv_paged_attn_decode_ordered(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                         const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                         int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                         int32_t block_size, float scale, const int32_t* work_order,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- CSR page tables ([MEM] "Method 3: PagedAttention", "Walking the
 * table"): request s owns pages kv_indices[kv_indptr[s] .. kv_indptr[s+1]),
 * its token p sits in page kv_indices[kv_indptr[s] + p / B] at offset p % B.
 *   kv_indptr: (device) int32 [batch + 1], nondecreasing, kv_indptr[0] = 0;
 *   kv_indices: (device) int32 [kv_indptr[batch]];
 *   max_pages_per_seq: a bound on kv_indptr[s+1] - kv_indptr[s] (it sizes
 *   the split like max_blocks_per_seq; pages past it are not read). */

/* Decode over a CSR page table: as pkv_paged_attn_decode (library's split)
 * with the table given as above; seq_lens[s] <= its page count * B (longer
 * sequences are cut there).  Workspace as pkv_paged_attn_decode_workspace
 * with max_blocks_per_seq = max_pages_per_seq. */
pkv_status pkv_paged_attn_decode_csr(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                     const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                     const float* k_scale, const float* v_scale, const int32_t* kv_indptr,
                                     const int32_t* kv_indices, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                     int32_t batch, int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t d_head, int32_t block_size, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Expands a CSR page table into the 2-D table the other calls take: row s of
 * block_table_out (device, int32 [batch][max_blocks_per_seq]) gets request
 * s's pages, then -1 (a request with more pages keeps its first
 * max_blocks_per_seq).  batch == 0 is a no-op. */
pkv_status pkv_csr_to_block_table(const int32_t* kv_indptr, const int32_t* kv_indices, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t* block_table_out, void* stream);

/* Chunked prefill attention: each sequence s brings q_len = cu_q_lens[s+1] -
 * cu_q_lens[s] new query tokens at absolute positions context_lens[s] + i.
 * With causal = 1, query i attends keys 0 .. context_lens[s] + i; with
 * causal = 0, every key of the context and the chunk ([MEM] "FlashAttention":
 * masked positions get -inf and fully masked blocks are skipped).  The chunk's
 * own K/V must already be appended to the cache (pkv_kv_append or
 * pkv_kv_append_fp8).  Computed with bf16 MFMA tiles, fp32 accumulation and an
 * online softmax per query row; the softmax weights enter the value product as
 * bf16.  FP8 caches ([KVP] Problem 3) are widened to bf16 exactly; a key's K
 * scale multiplies its score and its V scale its weight in the value product
 * (k_scale, v_scale: (device) f32 [num_blocks][n_kv_heads], required for FP8,
 * ignored otherwise).
 *   q, out: (device) packed [total_q][n_q_heads][d_head];
 *   cu_q_lens: (device) int32 [num_seqs + 1], cu_q_lens[0] = 0, nondecreasing,
 *   cu_q_lens[num_seqs] = total_q, each q_len <= max_q_len;
 *   context_lens: (device) int32 [num_seqs];
 *   context_lens[s] + q_len <= max_blocks_per_seq * B.
 * Supported: d_head 128; block_size 8, 16, 32, 64, 128 or 256; num_blocks *
 * n_kv_heads * block_size <= 2^32; q BF16; KV BF16 or FP8; out F32 or BF16.
 * workspace: pkv_paged_attn_prefill_workspace(...) bytes (may be 0, then the
 * pointer may be NULL). */
pkv_status pkv_paged_attn_prefill_chunk(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                        const int32_t* cu_q_lens, const int32_t* context_lens, int32_t num_seqs,
                                        int32_t total_q, int32_t max_q_len, const void* k_cache,
                                        const void* v_cache, pkv_dtype kv_dtype, const float* k_scale,
                                        const float* v_scale, const int32_t* block_table,
                                        int32_t max_blocks_per_seq, int64_t num_blocks, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t d_head, int32_t block_size, float scale,
                                        int32_t causal, void* workspace, size_t workspace_bytes, void* stream);

size_t pkv_paged_attn_prefill_workspace(int32_t num_seqs, int32_t max_q_len, int32_t n_q_heads, int32_t d_head);

/* Chunked prefill over a CSR page table (see "CSR page tables" above): as
 * pkv_paged_attn_prefill_chunk; context_lens[s] + q_len <= the request's page
 * count * B.  Needs no workspace. */
pkv_status pkv_paged_attn_prefill_chunk_csr(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                            const int32_t* cu_q_lens, const int32_t* context_lens, int32_t num_seqs,
                                            int32_t total_q, int32_t max_q_len, const void* k_cache,
                                            const void* v_cache, pkv_dtype kv_dtype, const float* k_scale,
                                            const float* v_scale, const int32_t* kv_indptr,
                                            const int32_t* kv_indices, int32_t max_pages_per_seq, int64_t num_blocks,
                                            int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                            int32_t block_size, float scale, int32_t causal, void* stream);

/* Chunked prefill over an FP8 cache with both products in FP8 on the matrix
 * cores (the FP8 attention of FlashAttention-3, [KVP] Problem 5, over the FP8
 * cache of [MEM] "long context"): the K and V codes enter the products as
 * stored; each query row is scaled by its own max |q| / 448 and each softmax
 * weight carries its block's V scale and one factor per workgroup, and both
 * enter the products in E4M3.  The row sum adds the quantised weights
 * themselves (each over its V scale), so every output row is a convex
 * combination of the dequantised V rows and a single visible key returns its
 * V row exactly; keys of blocks whose V scale is below 2^-3 of what the
 * weights can use count unquantised weights instead.
 *   split = 1: queries and weights are each carried as two E4M3 terms, the
 *     nearest value plus the nearest value to the remainder (relative error
 *     about 2^-8), at two products per tile pair: within the FP8 tolerance of
 *     pkv_paged_attn_prefill_chunk's result (about 3e-3 max-abs on N(0,1)
 *     data).
 *   split = 0: one E4M3 term each, as FlashAttention-3 does, at half the
 *     products: faster, with row errors of a few percent (a rounding of up to
 *     2^-4 per query element and weight); it does not meet the FP8 tolerance.
 * Arguments as pkv_paged_attn_prefill_chunk (2-D block table, no workspace),
 * with kv_dtype PKV_FP8_E4M3FN only (else PKV_ERR_UNSUPPORTED); k_scale and
 * v_scale are required, non-negative and finite (as pkv_kv_append_fp8 writes
 * them), and a block whose scale is 0 holds zero codes.  Supported: d_head
 * 128; block_size 8 .. 256; n_q_heads / n_kv_heads divides 128; q BF16; out
 * F32 or BF16. */
pkv_status pkv_paged_attn_prefill_chunk_fp8_mma(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                                const int32_t* cu_q_lens, const int32_t* context_lens,
                                                int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                                const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                                const float* k_scale, const float* v_scale,
                                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                                int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                                                int32_t d_head, int32_t block_size, float scale, int32_t causal,
                                                int32_t split, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
