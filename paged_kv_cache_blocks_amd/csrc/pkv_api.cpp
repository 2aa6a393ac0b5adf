// C ABI of libpkv: argument validation, launch-shape choice, error reporting,
// and the host-side block pool.  Every check runs before any launch, so a
// failing call leaves the device untouched.  No device allocation.  State
// beyond the thread-local message: cached device properties, the device-check
// switch, and a small file-scope device array per GPU (the device-check
// counter), located once per device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <atomic>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

thread_local char g_err[512] = "";

pkv_status fail(pkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

pkv_status ok() {
  g_err[0] = '\0';
  return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(pkv_dtype t) {
  switch (t) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3FN: return 1;
    default: return 0;
  }
}

bool valid_dtype(int t) { return t == PKV_F32 || t == PKV_BF16 || t == PKV_FP8_E4M3FN; }

// Longest partition: the matrix-core kernel keeps the row indices of a
// partition's tiles in its waves' lanes (4 waves x 32 chunks x 32 tokens).
constexpr int kMaxPartition = 4096;

// log2 of a supported block size (8, 16, 32, 64, 128, 256), else -1
int log2_block_size(int32_t bs) {
  for (int l = 3; l <= 8; ++l)
    if (bs == (1 << l)) return l;
  return -1;
}

// the attention kernels address cache rows of one KV head with 32-bit indices
pkv_status check_row_space(int64_t num_blocks, int32_t n_kv, int32_t block_size) {
  if ((double)num_blocks * n_kv * block_size > 4294967296.0)
    return fail(PKV_ERR_UNSUPPORTED, "num_blocks x n_kv_heads x block_size beyond 2^32 rows");
  return PKV_OK;
}
constexpr int kQueueMaxWgsPerCu = 2;
constexpr int kQueueSplit = -1;  // partition_tokens value that asks for the work-queue split

// heads ratio check, shared by the attention calls
pkv_status check_heads(int32_t n_q, int32_t n_kv) {
  if (n_kv < 1 || n_q < 1) return fail(PKV_ERR_INVALID_ARG, "head counts must be positive (n_q=%d, n_kv=%d)", n_q, n_kv);
  if (n_q % n_kv != 0) return fail(PKV_ERR_INVALID_ARG, "%d query heads do not split evenly over %d KV heads", n_q, n_kv);
  return PKV_OK;
}

struct DecodePlan {
  int32_t head_chunks;
  int32_t use_mfma;     // partition mode on the matrix-core kernel
  int32_t part_tokens;  // partition mode
  int32_t n_parts;      // partition mode
  int32_t n_wg;         // queue mode: workgroups (0 = partition mode)
  int32_t merge_splits;  // queue mode: merge workgroups per pair
  int32_t n_slots;       // queue mode: partial-state slots
  int32_t items_per_wg;
  size_t ws_o_off, ws_ml_off, split_off, counter_off;
  size_t ws_bytes;
};

// Compute units of the current device and workgroups per CU of the decode
// kernels: fixed properties of the device and the code object, looked up once
// per (device, kernel variant).  Any thread may fill an entry; all compute the
// same value, so a relaxed atomic load / store per entry is enough.
constexpr int kMaxDevices = 64;
using Cached = std::atomic<int>;

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

template <class F>
int cached(Cached& slot, F compute) {
  int v = slot.load(std::memory_order_relaxed);
  if (v == 0) {
    v = compute();
    if (v > 0) slot.store(v, std::memory_order_relaxed);
  }
  return v;
}

int device_cus() {
  static Cached cus[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return 0;
  return cached(cus[dev], [dev] {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  });
}

int partition_wgs_per_cu(int kind, int d, int gw) {
  static Cached cache[kMaxDevices][3][2][9];
  const int dev = current_device();
  if (dev < 0) return 0;
  return cached(cache[dev][kind][d == 128][gw], [&] { return pkv::decode_partition_wgs_per_cu(kind, d, gw); });
}

int mfma_wgs_per_cu(int kind, int gw) {
  static Cached cache[kMaxDevices][3][17];
  const int dev = current_device();
  if (dev < 0) return 0;
  return cached(cache[dev][kind][gw], [&] { return pkv::decode_mfma_wgs_per_cu(kind, gw); });
}

int queue_wgs_per_cu(int kind, int d, int gw, int batch) {
  // keyed by the batch rounded up to 256 sequences (1 KiB of prefix sums)
  constexpr int kBuckets = pkv::kDecodeMaxQueueBatch / 256;
  static Cached cache[kMaxDevices][3][2][9][kBuckets];
  const int dev = current_device();
  if (dev < 0) return 0;
  const int bucket = (batch + 255) / 256 - 1;
  return cached(cache[dev][kind][d == 128][gw][bucket],
                [&] { return pkv::decode_queue_wgs_per_cu(kind, d, gw, (bucket + 1) * 256); });
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- opt-in device-data checks (pkv_set_device_checks) ----
// The counter the check kernels add to: one int per GPU, in a file-scope
// device array.  Its device address is looked up once per device with
// hipGetSymbolAddress (the array's name is not a device address in host code).
__device__ __align__(256) int32_t g_check_count[1];

std::atomic<int> g_device_checks{0};
std::mutex g_check_mu;                         // one check sequence at a time
std::atomic<int32_t*> g_count_ptr[kMaxDevices];  // per device, once found

pkv_status count_ptr(int32_t** out) {
  const int dev = current_device();
  if (dev < 0) return fail(PKV_ERR_HIP, "no HIP device for the device checks");
  int32_t* p = g_count_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(g_check_count));
    if (e != hipSuccess) return hip_status(e, "locating the device-check counter");
    p = static_cast<int32_t*>(addr);
    g_count_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PKV_OK;
}

// Runs `launch_checks(counter)` on the stream between a clear of the counter
// and a copy of it back, waits for the stream, and returns
// PKV_ERR_DEVICE_CHECK if anything was counted.  Called before the checked
// call launches its own work, so a failing call changes nothing.
template <class F>
pkv_status run_device_check(hipStream_t stream, const char* what, F launch_checks) {
  std::lock_guard<std::mutex> lock(g_check_mu);
  int32_t* cnt = nullptr;
  pkv_status st = count_ptr(&cnt);
  if (st != PKV_OK) return st;
  hipError_t e = pkv::launch_zero_words(cnt, 1, stream);
  if (e == hipSuccess) e = launch_checks(cnt);
  int32_t host = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&host, cnt, sizeof host, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e, "device check");
  if (host != 0) return fail(PKV_ERR_DEVICE_CHECK, "%s: %d bad device entries (lengths, block ids or slots)", what, host);
  return PKV_OK;
}

bool device_checks_on() { return g_device_checks.load(std::memory_order_relaxed) != 0; }

// ---- decode without a caller workspace (pkv_paged_attn_decode_noalloc) ----
// The split kernels' partial results, and the work-queue split's counter, go
// to this file-scope device array instead of a caller's workspace: 32 MiB per
// GPU, held until the process ends (the 70B-shaped 32K decode needs 2.1 MB,
// the fp8 serving mix 17 MB).  Host code never passes the array's name to a
// kernel: its device address is looked up once per device.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

pkv_status scratch_ptr(void** out) {
  const int dev = current_device();
  if (dev < 0) return fail(PKV_ERR_HIP, "no HIP device for the static scratch");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      // with device `dev` current: its own copy of the array
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "locating the static scratch");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PKV_OK;
}

pkv_status plan_decode(int32_t batch, int32_t n_q, int32_t n_kv, int32_t d, int32_t max_blocks, int32_t block_size,
                       int kv_dtype, int32_t partition_tokens, DecodePlan* plan) {
  pkv_status st = check_heads(n_q, n_kv);
  if (st != PKV_OK) return st;
  if (!valid_dtype(kv_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown dtype");
  if (batch < 1 || max_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "batch and max_blocks_per_seq must be positive");
  if (log2_block_size(block_size) < 0)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (8, 16, 32, 64, 128 or 256)", block_size);
  if (d != 64 && d != 128) return fail(PKV_ERR_UNSUPPORTED, "d_head %d unsupported (64 or 128)", d);
  const int group = n_q / n_kv;
  const int gw = pkv::decode_heads_per_wg(group);
  const int quantum = 64 * pkv::decode_chunk_blocks(gw);
  const int64_t max_tokens = (int64_t)max_blocks * block_size;
  if (max_tokens > (1 << 30)) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  plan->head_chunks = group / gw;
  const int64_t hk = (int64_t)n_kv * plan->head_chunks;
  // bf16 and fp8 KV at d = 128 run their fixed partitions on the matrix-core
  // kernel: with fp8 the VALU kernel's dot products, not HBM, set its pace
  // (1.7x slower on the fp8 serving mix), and with bf16 the two kernels
  // stream at the same rate or the matrix-core one faster
  const bool mfma = pkv::decode_mfma_supported(kv_dtype, d, gw);
  plan->use_mfma = 0;
  int32_t part = partition_tokens;
  if (part == 0 && mfma) {
    // Fewest equal partitions of at most kMaxPartition tokens, but at least
    // enough that every CU gets a workgroup (a single long sequence otherwise
    // left most CUs idle).  One per CU, not one per resident slot: on
    // few long sequences the longer per-wave streams and the shorter merge
    // measured 2-12 % faster than twice the workgroups.  The matrix-core
    // kernel has no work-queue form.  The split depends on the device, so
    // planning needs one.
    int64_t n_parts = (max_tokens + kMaxPartition - 1) / kMaxPartition;
    const int cus = device_cus();
    if (cus <= 0) return fail(PKV_ERR_HIP, "no HIP device to plan the decode launch for");
    const int64_t pairs = (int64_t)batch * hk;
    n_parts = std::max<int64_t>(n_parts, std::min<int64_t>((cus + pairs - 1) / pairs, (max_tokens + 255) / 256));
    // partitions in whole 32-token chunks, the matrix-core kernel's unit
    part = (int32_t)(((max_tokens + n_parts - 1) / n_parts + 31) / 32 * 32);
  } else if (part == 0) {
    // Library's choice.  Cut each (sequence, KV head chunk) into the fewest
    // equal partitions of at most kMaxPartition tokens; if all of those
    // workgroups are resident at once, use them (long per-wave streams, no
    // cross-sequence bookkeeping).  Otherwise the work-queue split, which
    // keeps every workgroup busy until the batch is done whatever the length
    // mix and however fast each XCD runs.
    const int cus = device_cus();
    if (cus <= 0) return fail(PKV_ERR_HIP, "no HIP device to plan the decode launch for");
    const int64_t resident = (int64_t)cus * partition_wgs_per_cu(kv_dtype, d, gw);
    const int64_t step = quantum > 256 ? quantum : 256;
    const int64_t n_parts = (max_tokens + kMaxPartition - 1) / kMaxPartition;
    if ((int64_t)batch * hk * n_parts <= resident)
      part = (int32_t)(((max_tokens + n_parts - 1) / n_parts + step - 1) / step * step);
    if (part == 0 && batch > pkv::kDecodeMaxQueueBatch) part = kMaxPartition;
  } else if (part == kQueueSplit) {
    if (batch > pkv::kDecodeMaxQueueBatch)
      return fail(PKV_ERR_UNSUPPORTED, "the work-queue split takes at most %d sequences", pkv::kDecodeMaxQueueBatch);
    part = 0;
  } else if (part < 0 || part % 256 != 0 || part % quantum != 0 || part > kMaxPartition) {
    return fail(PKV_ERR_INVALID_ARG, "partition_tokens %d must be -1, 0 or a multiple of %d in (0, %d]", part,
                quantum > 256 ? quantum : 256, kMaxPartition);
  }
  if (part == 0) {
    // work-queue mode: as many workgroups as the device keeps resident (at
    // least 8 blocks each), items claimed dynamically
    const int cus = device_cus();
    if (cus <= 0) return fail(PKV_ERR_HIP, "no HIP device to plan the decode launch for");
    // at most two workgroups per CU: measured faster than three on both the
    // 8B- and 70B-shaped decodes (more waves in flight only add contention)
    const int occ = std::min(queue_wgs_per_cu(kv_dtype, d, gw, batch), kQueueMaxWgsPerCu);
    const int64_t resident = (int64_t)cus * occ;
    const int64_t pairs = (int64_t)batch * hk;
    const int64_t max_blocks_total = pairs * ((max_tokens + 15) / 16);  // 16-token tiles
    int64_t n_wg = std::min(resident, (max_blocks_total + 7) / 8);
    if (n_wg < 1) n_wg = 1;
    plan->n_wg = (int32_t)n_wg;
    plan->part_tokens = 0;
    plan->n_parts = 0;
    // items <= F / U + pairs, and U >= F / (n_wg * items per wg) unless U hits
    // its cap, so this many partial slots always suffice
    const int64_t per_wg = pkv::decode_queue_items_per_wg();
    plan->items_per_wg = (int32_t)per_wg;
    const int64_t cap = pkv::decode_queue_max_item_blocks();
    const int64_t slots = std::max(n_wg * per_wg, (max_blocks_total + cap - 1) / cap) + pairs;
    // merge workgroups per pair: one per head when pairs hold many items
    int splits = 1;
    while (splits < gw && n_wg * per_wg / pairs / splits > 8) splits *= 2;
    plan->merge_splits = splits;
    if (slots > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "decode too large for the work-queue split");
    plan->n_slots = (int32_t)slots;
    plan->ws_o_off = 0;
    plan->ws_ml_off = align256((size_t)slots * gw * d * sizeof(float));
    plan->split_off = plan->ws_ml_off + align256((size_t)slots * gw * 2 * sizeof(float));
    plan->counter_off = plan->split_off + align256((size_t)pairs * 16);
    plan->ws_bytes = plan->counter_off + 256;
    return PKV_OK;
  }
  plan->n_wg = 0;
  plan->use_mfma = mfma ? 1 : 0;
  plan->merge_splits = 1;
  plan->n_slots = 0;
  plan->items_per_wg = 0;
  plan->counter_off = 0;
  plan->part_tokens = part;
  plan->n_parts = (int32_t)((max_tokens + part - 1) / part);
  plan->ws_o_off = 0;
  plan->split_off = 0;
  if (plan->n_parts == 1) {
    plan->ws_ml_off = 0;
    plan->ws_bytes = 0;
  } else {
    const size_t n = (size_t)batch * n_q * plan->n_parts;
    plan->ws_ml_off = align256(n * d * sizeof(float));
    plan->ws_bytes = plan->ws_ml_off + n * 2 * sizeof(float);
  }
  return PKV_OK;
}

// A split call's work order lists its (sequence, partition) units, longest
// first (a unit order), when it has several partitions per sequence and few
// enough units for the order kernel's all-pairs ranking; otherwise it lists
// the sequences.
constexpr int64_t kMaxOrderUnits = 8192;
bool order_units(const DecodePlan& p, int32_t batch) {
  return !p.n_wg && p.n_parts > 1 && (int64_t)batch * p.n_parts <= kMaxOrderUnits;
}

const float kLog2e = 1.4426950408889634f;

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_NO_BLOCKS: return "PKV_ERR_NO_BLOCKS";
    case PKV_ERR_DEVICE_CHECK: return "PKV_ERR_DEVICE_CHECK";
  }
  return "PKV_ERR_UNKNOWN";
}

const char* pkv_last_error(void) { return g_err; }

void pkv_set_device_checks(int enable) { g_device_checks.store(enable ? 1 : 0, std::memory_order_relaxed); }

int pkv_device_checks(void) { return device_checks_on() ? 1 : 0; }

int64_t pkv_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t d_head, int32_t bytes_per_value) {
  if (n_layers < 0 || n_kv_heads < 0 || d_head < 0 || bytes_per_value < 0) return -1;
  return (int64_t)2 * n_layers * n_kv_heads * d_head * bytes_per_value;
}

pkv_status pkv_slot_mapping(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                            const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                            int32_t block_size, int64_t* slot_mapping_out, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) return ok();
  if (!block_table || !seq_ids || !positions || !slot_mapping_out) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (batch < 1 || max_blocks_per_seq < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "batch, max_blocks_per_seq and block_size must be positive");
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return fail(PKV_ERR_INVALID_ARG, "table too wide");
  return hip_status(pkv::launch_slot_mapping(block_table, batch, max_blocks_per_seq, seq_ids, positions, num_tokens,
                                             block_size, slot_mapping_out, (hipStream_t)stream),
                    "slot_mapping launch");
}

pkv_status pkv_kv_append(void* k_cache, void* v_cache, pkv_dtype cache_dtype, int64_t num_blocks,
                         const int64_t* slot_mapping, const void* k, const void* v, int32_t num_tokens,
                         int32_t n_kv_heads, int32_t d_head, int32_t block_size, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (!valid_dtype(cache_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown cache dtype %d", (int)cache_dtype);
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !slot_mapping || !k || !v) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (num_blocks < 1 || n_kv_heads < 1 || d_head < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  const int row_bytes = d_head * elem_bytes(cache_dtype);
  if (row_bytes % 16) return fail(PKV_ERR_UNSUPPORTED, "a row of %d bytes is not a multiple of 16", row_bytes);
  if (device_checks_on()) {
    const pkv_status st = run_device_check((hipStream_t)stream, "kv_append", [&](int32_t* cnt) {
      return pkv::launch_check_slots(slot_mapping, num_tokens, num_blocks * block_size, cnt, (hipStream_t)stream);
    });
    if (st != PKV_OK) return st;
  }
  return hip_status(pkv::launch_kv_append(k_cache, v_cache, num_blocks, slot_mapping, k, v, num_tokens, n_kv_heads,
                                          row_bytes, block_size, (hipStream_t)stream),
                    "kv_append launch");
}

pkv_status pkv_kv_append_positions(void* k_cache, void* v_cache, pkv_dtype cache_dtype, int64_t num_blocks,
                                   const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                                   const int32_t* seq_ids, const int32_t* positions, const void* k, const void* v,
                                   int32_t num_tokens, int32_t n_kv_heads, int32_t d_head, int32_t block_size,
                                   int64_t* slot_mapping_out, void* stream) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (!valid_dtype(cache_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown cache dtype %d", (int)cache_dtype);
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !block_table || !seq_ids || !positions || !k || !v)
    return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (num_blocks < 1 || batch < 1 || max_blocks_per_seq < 1 || n_kv_heads < 1 || d_head < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return fail(PKV_ERR_INVALID_ARG, "table too wide");
  const int row_bytes = d_head * elem_bytes(cache_dtype);
  if (row_bytes % 16) return fail(PKV_ERR_UNSUPPORTED, "a row of %d bytes is not a multiple of 16", row_bytes);
  if (device_checks_on()) {
    const pkv_status st = run_device_check((hipStream_t)stream, "kv_append_positions", [&](int32_t* cnt) {
      return pkv::launch_check_positions(block_table, batch, max_blocks_per_seq, seq_ids, positions, num_tokens,
                                         block_size, num_blocks * block_size, cnt, (hipStream_t)stream);
    });
    if (st != PKV_OK) return st;
  }
  return hip_status(pkv::launch_kv_append_positions(k_cache, v_cache, num_blocks, block_table, batch,
                                                    max_blocks_per_seq, seq_ids, positions, k, v, num_tokens,
                                                    n_kv_heads, row_bytes, block_size, slot_mapping_out,
                                                    (hipStream_t)stream),
                    "kv_append_positions launch");
}

pkv_status pkv_kv_append_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, int64_t num_blocks,
                             const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                             const int32_t* cu_new_lens, int32_t batch, int32_t max_new_len, const void* k_new,
                             const void* v_new, pkv_dtype new_dtype, int32_t n_kv_heads, int32_t d_head,
                             int32_t block_size, void* stream) {
  if (batch < 0 || max_new_len < 0) return fail(PKV_ERR_INVALID_ARG, "batch and max_new_len must be >= 0");
  if (new_dtype != PKV_BF16 && new_dtype != PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "new K/V must be BF16 or F32 (got dtype %d)", (int)new_dtype);
  if (batch == 0 || max_new_len == 0) return ok();
  if (!k_cache || !v_cache || !k_scale || !v_scale || !block_table || !context_lens || !cu_new_lens || !k_new ||
      !v_new)
    return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || n_kv_heads < 1 || d_head < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  const int log2_bs = log2_block_size(block_size);
  if (log2_bs < 0) return fail(PKV_ERR_UNSUPPORTED, "block_size %d (supported: 8, 16, 32, 64, 128, 256)", block_size);
  if (d_head != 64 && d_head != 128) return fail(PKV_ERR_UNSUPPORTED, "d_head %d (supported: 64, 128)", d_head);
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return fail(PKV_ERR_INVALID_ARG, "table too wide");
  if (batch > 65535 || 2 * n_kv_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)k_new | (uintptr_t)v_new) & 15)
    return fail(PKV_ERR_UNSUPPORTED, "caches and new K/V must be 16-byte aligned");
  if (device_checks_on()) {
    pkv::SeqCheck c{block_table, nullptr, context_lens, cu_new_lens, num_blocks, max_blocks_per_seq, batch, log2_bs,
                    pkv::SeqCheck::kAppend, max_new_len, 0};
    const pkv_status st = run_device_check((hipStream_t)stream, "kv_append_fp8", [&](int32_t* cnt) {
      return pkv::launch_check_seqs(c, cnt, (hipStream_t)stream);
    });
    if (st != PKV_OK) return st;
  }
  return hip_status(pkv::launch_kv_append_fp8(k_cache, v_cache, k_scale, v_scale, num_blocks, block_table,
                                              max_blocks_per_seq, context_lens, cu_new_lens, batch, max_new_len,
                                              k_new, v_new, new_dtype == PKV_BF16 ? 2 : 4, n_kv_heads, d_head,
                                              log2_bs, (hipStream_t)stream),
                    "kv_append_fp8 launch");
}

size_t pkv_swap_image_bytes(int32_t n_blocks, pkv_dtype cache_dtype, int32_t n_kv_heads, int32_t d_head,
                            int32_t block_size) {
  if (n_blocks < 0 || n_kv_heads < 1 || d_head < 1 || block_size < 1 || !valid_dtype(cache_dtype)) return 0;
  const size_t block_bytes = (size_t)n_kv_heads * block_size * d_head * elem_bytes(cache_dtype);
  const size_t scales = cache_dtype == PKV_FP8_E4M3FN ? (size_t)n_kv_heads * sizeof(float) : 0;
  return (size_t)n_blocks * 2 * (block_bytes + scales);
}

}  // extern "C"

namespace {

// checks shared by swap out and swap in
pkv_status check_swap(const void* k_cache, const void* v_cache, pkv_dtype cache_dtype, const float* k_scale,
                      const float* v_scale, int64_t num_blocks, const int32_t* block_ids, int32_t n_blocks,
                      const void* staging, size_t staging_bytes, const void* host_image, int32_t n_kv_heads,
                      int32_t d_head, int32_t block_size, int64_t* block_bytes) {
  if (n_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks must be >= 0");
  if (!valid_dtype(cache_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown dtype");
  if (!k_cache || !v_cache || !block_ids || !staging || !host_image) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (num_blocks < 1 || n_kv_heads < 1 || d_head < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  if ((cache_dtype == PKV_FP8_E4M3FN) != (k_scale != nullptr) || (k_scale != nullptr) != (v_scale != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale are given exactly for FP8 caches");
  *block_bytes = (int64_t)n_kv_heads * block_size * d_head * elem_bytes(cache_dtype);
  if (*block_bytes % 16 != 0) return fail(PKV_ERR_UNSUPPORTED, "a block must be a multiple of 16 bytes");
  if (n_blocks > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 blocks per call");
  if (((uintptr_t)staging) & 15) return fail(PKV_ERR_INVALID_ARG, "staging must be 16-byte aligned");
  const size_t need = pkv_swap_image_bytes(n_blocks, cache_dtype, n_kv_heads, d_head, block_size);
  if (staging_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "staging of %zu bytes needed, %zu given", need, staging_bytes);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_swap_out(const void* k_cache, const void* v_cache, pkv_dtype cache_dtype, const float* k_scale,
                        const float* v_scale, int64_t num_blocks, const int32_t* block_ids, int32_t n_blocks,
                        void* staging, size_t staging_bytes, void* host_image, int32_t n_kv_heads, int32_t d_head,
                        int32_t block_size, void* stream) {
  if (n_blocks == 0) return ok();
  int64_t block_bytes = 0;
  pkv_status st = check_swap(k_cache, v_cache, cache_dtype, k_scale, v_scale, num_blocks, block_ids, n_blocks,
                             staging, staging_bytes, host_image, n_kv_heads, d_head, block_size, &block_bytes);
  if (st != PKV_OK) return st;
  const size_t bytes = pkv_swap_image_bytes(n_blocks, cache_dtype, n_kv_heads, d_head, block_size);
  st = hip_status(pkv::launch_swap(const_cast<void*>(k_cache), const_cast<void*>(v_cache), const_cast<float*>(k_scale),
                                   const_cast<float*>(v_scale), num_blocks, block_ids, n_blocks, staging, block_bytes,
                                   n_kv_heads, 1, (hipStream_t)stream),
                  "swap pack launch");
  if (st != PKV_OK) return st;
  return hip_status(hipMemcpyAsync(host_image, staging, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream),
                    "swap copy to host");
}

pkv_status pkv_swap_in(void* k_cache, void* v_cache, pkv_dtype cache_dtype, float* k_scale, float* v_scale,
                       int64_t num_blocks, const int32_t* block_ids, int32_t n_blocks, void* staging,
                       size_t staging_bytes, const void* host_image, int32_t n_kv_heads, int32_t d_head,
                       int32_t block_size, void* stream) {
  if (n_blocks == 0) return ok();
  int64_t block_bytes = 0;
  pkv_status st = check_swap(k_cache, v_cache, cache_dtype, k_scale, v_scale, num_blocks, block_ids, n_blocks,
                             staging, staging_bytes, host_image, n_kv_heads, d_head, block_size, &block_bytes);
  if (st != PKV_OK) return st;
  const size_t bytes = pkv_swap_image_bytes(n_blocks, cache_dtype, n_kv_heads, d_head, block_size);
  st = hip_status(hipMemcpyAsync(staging, host_image, bytes, hipMemcpyHostToDevice, (hipStream_t)stream),
                  "swap copy to device");
  if (st != PKV_OK) return st;
  return hip_status(pkv::launch_swap(k_cache, v_cache, k_scale, v_scale, num_blocks, block_ids, n_blocks, staging,
                                     block_bytes, n_kv_heads, 0, (hipStream_t)stream),
                    "swap unpack launch");
}

pkv_status pkv_csr_to_block_table(const int32_t* kv_indptr, const int32_t* kv_indices, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t* block_table_out, void* stream) {
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch == 0) return ok();
  if (!kv_indptr || !kv_indices || !block_table_out) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  return hip_status(pkv::launch_csr_to_table(kv_indptr, kv_indices, batch, max_blocks_per_seq, block_table_out,
                                             (hipStream_t)stream),
                    "csr_to_table launch");
}

pkv_status pkv_paged_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                            int64_t num_blocks, const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int64_t* cu_seq_lens, int64_t total_tokens, int32_t batch,
                            int32_t n_kv_heads, int32_t d_head, int32_t block_size, void* stream) {
  if (!valid_dtype(kv_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown cache dtype %d", (int)kv_dtype);
  if (!k_out || !v_out || !k_cache || !v_cache || !block_table || !seq_lens || !cu_seq_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (batch < 1 || num_blocks < 1 || max_blocks_per_seq < 1 || n_kv_heads < 1 || d_head < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  if (total_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "total_tokens must be >= 0");
  if (total_tokens == 0) return ok();
  if (max_blocks_per_seq > 65535 || batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  const int row_bytes = d_head * elem_bytes(kv_dtype);
  if (row_bytes % 16) return fail(PKV_ERR_UNSUPPORTED, "a row of %d bytes is not a multiple of 16", row_bytes);
  return hip_status(pkv::launch_gather(k_out, v_out, k_cache, v_cache, num_blocks, block_table, max_blocks_per_seq,
                                       seq_lens, cu_seq_lens, total_tokens, batch, n_kv_heads, row_bytes, block_size,
                                       (hipStream_t)stream),
                    "gather launch");
}

pkv_status pkv_read_probe(const void* buf, int64_t bytes, const int32_t* slab_list, int32_t n_list,
                          int32_t slab_bytes, int32_t workgroups, int32_t nontemporal, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (bytes < 16 || bytes % 16 != 0 || workgroups < 1) return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  if (slab_list) {
    if (!(slab_bytes == 1024 || slab_bytes == 2048 || (slab_bytes >= 4096 && slab_bytes % 4096 == 0)) ||
        slab_bytes > bytes)
      return fail(PKV_ERR_INVALID_ARG, "slab_bytes must be 1024, 2048 or a multiple of 4096 within the buffer");
    if (n_list < workgroups) return fail(PKV_ERR_INVALID_ARG, "fewer slabs than workgroups");
  }
  return hip_status(pkv::launch_read_probe(buf, bytes, slab_list, n_list, slab_bytes, workgroups, nontemporal ? 1 : 0,
                                           sink, (hipStream_t)stream),
                    "read probe launch");
}

pkv_status pkv_check_tables(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            int32_t batch, int64_t num_blocks, int32_t block_size, int32_t* error_count,
                            void* stream) {
  if (!block_table || !seq_lens || !error_count) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (batch < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  return hip_status(pkv::launch_check_tables(block_table, max_blocks_per_seq, seq_lens, batch, num_blocks,
                                             block_size, error_count, (hipStream_t)stream),
                    "check_tables launch");
}

size_t pkv_paged_attn_decode_workspace(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                       int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype kv_dtype,
                                       int32_t partition_tokens) {
  DecodePlan plan;
  if (plan_decode(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size, (int)kv_dtype,
                  partition_tokens, &plan) != PKV_OK)
    return 0;
  return plan.ws_bytes;
}

pkv_status pkv_paged_attn_decode_plan(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                      int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype kv_dtype,
                                      int32_t partition_tokens, int32_t* info) {
  if (!info) return fail(PKV_ERR_INVALID_ARG, "info is NULL");
  DecodePlan plan;
  pkv_status st = plan_decode(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size, (int)kv_dtype,
                              partition_tokens, &plan);
  if (st != PKV_OK) return st;
  const int64_t pairs = (int64_t)batch * n_kv_heads * plan.head_chunks;
  info[0] = plan.n_wg ? 1 : 0;
  info[1] = plan.part_tokens;
  info[2] = plan.n_parts;
  // (the matrix-core kernel numbers its unit slots in eights, one XCD each)
  const int64_t slots = (int64_t)batch * plan.n_parts;
  const int64_t split_wgs = plan.use_mfma ? (slots + 7) / 8 * 8 * (pairs / batch) : pairs * plan.n_parts;
  info[3] = plan.n_wg ? plan.n_wg : (int32_t)std::min<int64_t>(split_wgs, 0x7fffffff);
  info[4] = (plan.n_wg || plan.n_parts > 1) ? 1 : 0;
  info[5] = (n_q_heads / n_kv_heads) / plan.head_chunks;
  info[6] = plan.use_mfma;
  return ok();
}

}  // extern "C"

namespace {

// decode over a 2-D table (indptr == nullptr) or CSR rows
pkv_status decode_impl(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const void* k_cache,
                       const void* v_cache, pkv_dtype kv_dtype, const float* k_scale, const float* v_scale,
                       const int32_t* block_table, const int32_t* indptr, int32_t max_blocks_per_seq,
                       const int32_t* seq_lens, int32_t batch, int64_t num_blocks, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t d_head, int32_t block_size, float scale, int32_t partition_tokens,
                       const int32_t* work_order, void* workspace, size_t workspace_bytes, void* stream,
                       bool static_scratch = false) {
  // head ratio first, before anything else (validate before mutate)
  pkv_status st = check_heads(n_q_heads, n_kv_heads);
  if (st != PKV_OK) return st;
  if (!out || !q || !k_cache || !v_cache || !block_table || !seq_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (!valid_dtype(out_dtype) || !valid_dtype(q_dtype) || !valid_dtype(kv_dtype))
    return fail(PKV_ERR_INVALID_ARG, "unknown dtype");
  if (num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be positive");
  if (num_blocks > (int64_t)1 << 31) return fail(PKV_ERR_UNSUPPORTED, "num_blocks beyond int32 block ids");
  if (batch < 1 || max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "batch and max_blocks_per_seq must be positive");
  const int log2_bs = log2_block_size(block_size);
  if (log2_bs < 0) return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (8, 16, 32, 64, 128 or 256)", block_size);
  if (d_head != 64 && d_head != 128) return fail(PKV_ERR_UNSUPPORTED, "d_head %d unsupported (64 or 128)", d_head);
  st = check_row_space(num_blocks, n_kv_heads, block_size);
  if (st != PKV_OK) return st;
  const bool combo_ok = (q_dtype == PKV_F32 && kv_dtype == PKV_F32) || (q_dtype == PKV_BF16 && kv_dtype == PKV_BF16) ||
                        (q_dtype == PKV_BF16 && kv_dtype == PKV_FP8_E4M3FN);
  if (!combo_ok) return fail(PKV_ERR_UNSUPPORTED, "(q, kv) dtype combination (%d, %d) unsupported", q_dtype, kv_dtype);
  if (out_dtype == PKV_FP8_E4M3FN) return fail(PKV_ERR_UNSUPPORTED, "fp8 output unsupported");
  if (kv_dtype == PKV_FP8_E4M3FN && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID_ARG, "fp8 caches need k_scale and v_scale");
  const int group = n_q_heads / n_kv_heads;
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(PKV_ERR_INVALID_ARG, "scale must be positive and finite");
  DecodePlan plan;
  st = plan_decode(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size, (int)kv_dtype,
                   partition_tokens, &plan);
  if (st != PKV_OK) return st;
  if (batch > 65535 || (int64_t)batch * n_kv_heads * plan.head_chunks > 0x7fffffff)
    return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  if (static_scratch && plan.ws_bytes > 0) {
    if (plan.ws_bytes > kScratchBytes)
      return fail(PKV_ERR_WORKSPACE, "this decode needs %zu bytes of workspace; the library's static scratch holds %zu",
                  plan.ws_bytes, kScratchBytes);
    st = scratch_ptr(&workspace);
    if (st != PKV_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) & 255) return fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.indptr = indptr;
  a.seq_lens = seq_lens;
  char* wsp = reinterpret_cast<char*>(workspace);
  a.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(wsp + plan.ws_o_off) : nullptr;
  a.ws_ml = plan.ws_bytes ? reinterpret_cast<float*>(wsp + plan.ws_ml_off) : nullptr;
  a.split_info = plan.n_wg ? reinterpret_cast<int*>(wsp + plan.split_off) : nullptr;
  a.n_wg = plan.n_wg;
  a.merge_splits = plan.merge_splits;
  a.n_slots = plan.n_slots;
  a.items_per_wg = plan.items_per_wg;
  a.dyn_counter = plan.n_wg ? reinterpret_cast<unsigned*>(wsp + plan.counter_off) : nullptr;
  a.num_blocks = num_blocks;
  a.batch = batch;
  a.max_blocks = max_blocks_per_seq;
  a.log2_bs = log2_bs;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.group = group;
  a.head_chunks = plan.head_chunks;
  a.use_mfma = plan.use_mfma;
  a.work_order = work_order;
  a.order_units = (work_order && order_units(plan, batch)) ? 1 : 0;
  a.part_tokens = plan.part_tokens;
  a.n_parts = plan.n_parts;
  a.out_bf16 = out_dtype == PKV_BF16;
  a.scale_log2 = scale * kLog2e;
  if (device_checks_on()) {
    pkv::SeqCheck c{block_table, indptr, seq_lens, nullptr, num_blocks, max_blocks_per_seq, batch, log2_bs,
                    pkv::SeqCheck::kDecode, 0, 0};
    st = run_device_check((hipStream_t)stream, "decode", [&](int32_t* cnt) {
      return pkv::launch_check_seqs(c, cnt, (hipStream_t)stream);
    });
    if (st != PKV_OK) return st;
  }
  if (static_scratch && plan.n_wg) {
    // the scratch keeps the previous call's bytes: the work-queue split's item
    // counter must start at zero (a kernel, not a memset, so that captured
    // streams record a kernel node)
    const hipError_t e = pkv::launch_zero_words(reinterpret_cast<int32_t*>(a.dyn_counter), 1, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "scratch counter clear");
  }
  return hip_status(pkv::launch_decode(a, (int)kv_dtype, d_head, (hipStream_t)stream), "decode launch");
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attn_decode_partitioned(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                             const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                             const float* k_scale, const float* v_scale,
                                             const int32_t* block_table, int32_t max_blocks_per_seq,
                                             const int32_t* seq_lens, int32_t batch, int64_t num_blocks,
                                             int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                             int32_t block_size, float scale, int32_t partition_tokens,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, nullptr,
                     max_blocks_per_seq, seq_lens, batch, num_blocks, n_q_heads, n_kv_heads, d_head, block_size,
                     scale, partition_tokens, nullptr, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attn_decode_ordered(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                         const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                         int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                         int32_t block_size, float scale, const int32_t* work_order,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!work_order) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  return decode_impl(out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, nullptr,
                     max_blocks_per_seq, seq_lens, batch, num_blocks, n_q_heads, n_kv_heads, d_head, block_size,
                     scale, 0, work_order, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attn_decode_order(const int32_t* seq_lens, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t d_head, int32_t max_blocks_per_seq, int32_t block_size,
                                       pkv_dtype kv_dtype, int32_t* work_order_out, void* stream) {
  if (!seq_lens || !work_order_out) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  DecodePlan plan;
  pkv_status st = plan_decode(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size, (int)kv_dtype, 0,
                              &plan);
  if (st != PKV_OK) return st;
  if (order_units(plan, batch))
    return hip_status(pkv::launch_decode_unit_order(seq_lens, batch, plan.n_parts, plan.part_tokens, work_order_out,
                                                    (hipStream_t)stream),
                      "decode order launch");
  // All split workgroups resident at once: workgroups i and i + half the grid
  // share a CU, so pair the k-th longest sequence with the k-th shortest.
  // Otherwise workgroups start as others finish: the longest first.
  int pair = 0;
  if (!plan.n_wg) {
    const int cus = device_cus();
    if (cus <= 0) return fail(PKV_ERR_HIP, "no HIP device to plan the decode launch for");
    const int gw = (n_q_heads / n_kv_heads) / plan.head_chunks;
    const int per_cu = plan.use_mfma ? mfma_wgs_per_cu(kv_dtype, gw) : partition_wgs_per_cu(kv_dtype, d_head, gw);
    const int64_t wgs = (int64_t)batch * n_kv_heads * plan.head_chunks * plan.n_parts;
    pair = wgs <= (int64_t)cus * per_cu ? 1 : 0;
  }
  return hip_status(pkv::launch_decode_order(seq_lens, batch, pair, work_order_out, (hipStream_t)stream),
                    "decode order launch");
}

int32_t pkv_paged_attn_decode_order_entries(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                            int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype kv_dtype) {
  DecodePlan plan;
  if (plan_decode(batch, n_q_heads, n_kv_heads, d_head, max_blocks_per_seq, block_size, (int)kv_dtype, 0, &plan) !=
      PKV_OK)
    return 0;
  return order_units(plan, batch) ? batch * plan.n_parts : batch;
}

pkv_status pkv_paged_attn_decode_csr(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                     const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                     const float* k_scale, const float* v_scale, const int32_t* kv_indptr,
                                     const int32_t* kv_indices, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                     int32_t batch, int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t d_head, int32_t block_size, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!kv_indptr) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  return decode_impl(out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, kv_indices, kv_indptr,
                     max_pages_per_seq, seq_lens, batch, num_blocks, n_q_heads, n_kv_heads, d_head, block_size, scale,
                     0, nullptr, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attn_decode(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                 const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                 const float* k_scale, const float* v_scale, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                 int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                 int32_t block_size, float scale, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return pkv_paged_attn_decode_partitioned(out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                           block_table, max_blocks_per_seq, seq_lens, batch, num_blocks, n_q_heads,
                                           n_kv_heads, d_head, block_size, scale, 0, workspace, workspace_bytes,
                                           stream);
}

pkv_status pkv_paged_attn_decode_noalloc(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                         const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                         int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                         int32_t block_size, float scale, int32_t partition_tokens, void* stream) {
  return decode_impl(out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_table, nullptr,
                     max_blocks_per_seq, seq_lens, batch, num_blocks, n_q_heads, n_kv_heads, d_head, block_size,
                     scale, partition_tokens, nullptr, nullptr, 0, stream, true);
}

size_t pkv_paged_attn_prefill_workspace(int32_t num_seqs, int32_t max_q_len, int32_t n_q_heads, int32_t d_head) {
  (void)num_seqs;
  (void)max_q_len;
  (void)n_q_heads;
  (void)d_head;
  return 0;
}

}  // extern "C"

namespace {

pkv_status prefill_impl(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype, const int32_t* cu_q_lens,
                        const int32_t* context_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                        const void* k_cache, const void* v_cache, pkv_dtype kv_dtype, const float* k_scale,
                        const float* v_scale, const int32_t* block_table, const int32_t* indptr,
                        int32_t max_blocks_per_seq, int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t d_head, int32_t block_size, float scale, int32_t causal, void* stream,
                        int fp8_mma = -1) {
  pkv_status st = check_heads(n_q_heads, n_kv_heads);
  if (st != PKV_OK) return st;
  if (!valid_dtype(out_dtype) || !valid_dtype(q_dtype) || !valid_dtype(kv_dtype))
    return fail(PKV_ERR_INVALID_ARG, "unknown dtype");
  if (num_seqs < 1 || total_q < 0 || max_q_len < 0) return fail(PKV_ERR_INVALID_ARG, "bad sequence counts");
  if (total_q == 0 || max_q_len == 0) return ok();
  if (!out || !q || !cu_q_lens || !context_lens || !k_cache || !v_cache || !block_table)
    return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (num_blocks < 1 || max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  if (num_blocks > (int64_t)1 << 31) return fail(PKV_ERR_UNSUPPORTED, "num_blocks beyond int32 block ids");
  const int log2_bs = log2_block_size(block_size);
  if (log2_bs < 0) return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (8, 16, 32, 64, 128 or 256)", block_size);
  if (d_head != 128) return fail(PKV_ERR_UNSUPPORTED, "prefill supports d_head 128 only");
  st = check_row_space(num_blocks, n_kv_heads, block_size);
  if (st != PKV_OK) return st;
  if (q_dtype != PKV_BF16 || kv_dtype == PKV_F32)
    return fail(PKV_ERR_UNSUPPORTED, "prefill needs bf16 q and bf16 or fp8 KV");
  if (kv_dtype == PKV_FP8_E4M3FN && (!k_scale || !v_scale))
    return fail(PKV_ERR_INVALID_ARG, "fp8 caches need k_scale and v_scale");
  if (fp8_mma >= 0 && kv_dtype != PKV_FP8_E4M3FN)
    return fail(PKV_ERR_UNSUPPORTED, "fp8 products need an FP8 cache");
  if (out_dtype == PKV_FP8_E4M3FN) return fail(PKV_ERR_UNSUPPORTED, "fp8 output unsupported");
  const int group = n_q_heads / n_kv_heads;
  if (!pkv::prefill_supported_group(group))
    return fail(PKV_ERR_UNSUPPORTED, "prefill needs n_q / n_kv to divide 128 (got %d)", group);
  if (causal != 0 && causal != 1) return fail(PKV_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(PKV_ERR_INVALID_ARG, "scale must be positive and finite");
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return fail(PKV_ERR_INVALID_ARG, "table too wide");
  if (num_seqs > 65535 || n_kv_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  pkv::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.cu_q = cu_q_lens;
  a.ctx_lens = context_lens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.indptr = indptr;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_blocks = max_blocks_per_seq;
  a.log2_bs = log2_bs;
  a.n_q = n_q_heads;
  a.n_kv = n_kv_heads;
  a.group = group;
  a.causal = causal;
  a.out_bf16 = out_dtype == PKV_BF16;
  a.kv_fp8 = kv_dtype == PKV_FP8_E4M3FN;
  a.scale_log2 = scale * kLog2e;
  if (device_checks_on()) {
    pkv::SeqCheck c{block_table, indptr, context_lens, cu_q_lens, num_blocks, max_blocks_per_seq, num_seqs, log2_bs,
                    pkv::SeqCheck::kPrefill, max_q_len, total_q};
    st = run_device_check((hipStream_t)stream, "prefill", [&](int32_t* cnt) {
      return pkv::launch_check_seqs(c, cnt, (hipStream_t)stream);
    });
    if (st != PKV_OK) return st;
  }
  if (fp8_mma >= 0)
    return hip_status(pkv::launch_prefill_fp8_mma(a, fp8_mma != 0, (hipStream_t)stream), "prefill launch");
  return hip_status(pkv::launch_prefill(a, d_head, (hipStream_t)stream), "prefill launch");
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attn_prefill_chunk(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                        const int32_t* cu_q_lens, const int32_t* context_lens, int32_t num_seqs,
                                        int32_t total_q, int32_t max_q_len, const void* k_cache,
                                        const void* v_cache, pkv_dtype kv_dtype, const float* k_scale,
                                        const float* v_scale, const int32_t* block_table,
                                        int32_t max_blocks_per_seq, int64_t num_blocks, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t d_head, int32_t block_size, float scale,
                                        int32_t causal, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return prefill_impl(out, out_dtype, q, q_dtype, cu_q_lens, context_lens, num_seqs, total_q, max_q_len, k_cache,
                      v_cache, kv_dtype, k_scale, v_scale, block_table, nullptr, max_blocks_per_seq, num_blocks,
                      n_q_heads, n_kv_heads, d_head, block_size, scale, causal, stream);
}

pkv_status pkv_paged_attn_prefill_chunk_csr(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                            const int32_t* cu_q_lens, const int32_t* context_lens, int32_t num_seqs,
                                            int32_t total_q, int32_t max_q_len, const void* k_cache,
                                            const void* v_cache, pkv_dtype kv_dtype, const float* k_scale,
                                            const float* v_scale, const int32_t* kv_indptr,
                                            const int32_t* kv_indices, int32_t max_pages_per_seq, int64_t num_blocks,
                                            int32_t n_q_heads, int32_t n_kv_heads, int32_t d_head,
                                            int32_t block_size, float scale, int32_t causal, void* stream) {
  if (!kv_indptr && total_q > 0 && max_q_len > 0) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  return prefill_impl(out, out_dtype, q, q_dtype, cu_q_lens, context_lens, num_seqs, total_q, max_q_len, k_cache,
                      v_cache, kv_dtype, k_scale, v_scale, kv_indices, kv_indptr, max_pages_per_seq, num_blocks,
                      n_q_heads, n_kv_heads, d_head, block_size, scale, causal, stream);
}

pkv_status pkv_paged_attn_prefill_chunk_fp8_mma(void* out, pkv_dtype out_dtype, const void* q, pkv_dtype q_dtype,
                                                const int32_t* cu_q_lens, const int32_t* context_lens,
                                                int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                                const void* k_cache, const void* v_cache, pkv_dtype kv_dtype,
                                                const float* k_scale, const float* v_scale,
                                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                                int64_t num_blocks, int32_t n_q_heads, int32_t n_kv_heads,
                                                int32_t d_head, int32_t block_size, float scale, int32_t causal,
                                                int32_t split, void* stream) {
  if (split != 0 && split != 1) return fail(PKV_ERR_INVALID_ARG, "split must be 0 or 1");
  return prefill_impl(out, out_dtype, q, q_dtype, cu_q_lens, context_lens, num_seqs, total_q, max_q_len, k_cache,
                      v_cache, kv_dtype, k_scale, v_scale, block_table, nullptr, max_blocks_per_seq, num_blocks,
                      n_q_heads, n_kv_heads, d_head, block_size, scale, causal, stream, split);
}


// ---- block pool: reference counts, lowest-id-first allocation, copy-on-write
// ("KV cache, PagedAttention and FlashAttention", Problem 4, "The idea")

}  // extern "C"

struct pkv_block_pool {
  std::mutex mu;
  std::vector<int32_t> ref;  // tables naming each block; 0 = free
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_ids;  // lowest id on top

  int32_t take() {  // caller checked that a block is free
    const int32_t b = free_ids.top();
    free_ids.pop();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_ids.push(b);
  }
  bool allocated(int32_t b) const { return b >= 0 && b < (int32_t)ref.size() && ref[b] > 0; }
};

extern "C" {

pkv_status pkv_pool_create(int64_t num_blocks, pkv_block_pool** pool_out) {
  if (!pool_out) return fail(PKV_ERR_INVALID_ARG, "pool_out is NULL");
  if (num_blocks < 1 || num_blocks > 0x7fffffff) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be in [1, 2^31)");
  auto* p = new pkv_block_pool;
  p->ref.assign((size_t)num_blocks, 0);
  std::vector<int32_t> ids((size_t)num_blocks);
  for (int64_t i = 0; i < num_blocks; ++i) ids[(size_t)i] = (int32_t)i;
  p->free_ids = decltype(p->free_ids)(std::greater<int32_t>(), std::move(ids));
  *pool_out = p;
  return ok();
}

void pkv_pool_destroy(pkv_block_pool* pool) { delete pool; }

int64_t pkv_pool_free_blocks(pkv_block_pool* pool) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> g(pool->mu);
  return (int64_t)pool->free_ids.size();
}

int32_t pkv_pool_refcount(pkv_block_pool* pool, int32_t block) {
  if (!pool) return -1;
  std::lock_guard<std::mutex> g(pool->mu);
  if (block < 0 || block >= (int32_t)pool->ref.size()) return -1;
  return pool->ref[block];
}

pkv_status pkv_pool_alloc(pkv_block_pool* pool, int32_t n, int32_t* ids_out) {
  if (!pool || (n > 0 && !ids_out)) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  std::lock_guard<std::mutex> g(pool->mu);
  if ((size_t)n > pool->free_ids.size())
    return fail(PKV_ERR_NO_BLOCKS, "%d blocks wanted, %zu free", n, pool->free_ids.size());
  for (int32_t i = 0; i < n; ++i) ids_out[i] = pool->take();
  return ok();
}

pkv_status pkv_pool_share(pkv_block_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool || (n > 0 && !ids)) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  std::lock_guard<std::mutex> g(pool->mu);
  for (int32_t i = 0; i < n; ++i)
    if (!pool->allocated(ids[i])) return fail(PKV_ERR_INVALID_ARG, "block %d is not allocated", ids[i]);
  for (int32_t i = 0; i < n; ++i) ++pool->ref[ids[i]];
  return ok();
}

pkv_status pkv_pool_release(pkv_block_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool || (n > 0 && !ids)) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  std::lock_guard<std::mutex> g(pool->mu);
  // every reference released must exist, counting repeats in ids
  std::vector<int32_t> sorted(ids, ids + n);
  std::sort(sorted.begin(), sorted.end());
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    while (j < n && sorted[j] == sorted[i]) ++j;
    const int32_t b = sorted[i];
    if (!pool->allocated(b) || pool->ref[b] < j - i)
      return fail(PKV_ERR_INVALID_ARG, "block %d released more often than it is named", b);
    i = j;
  }
  for (int32_t i = 0; i < n; ++i) pool->drop(ids[i]);
  return ok();
}

pkv_status pkv_pool_prepare_append(pkv_block_pool* pool, int32_t* table_row, int32_t max_blocks_per_seq,
                                   int32_t seq_len, int32_t n_new, int32_t block_size, int32_t* copy_src,
                                   int32_t* copy_dst, int32_t* n_copies) {
  if (!pool || !table_row || !copy_src || !copy_dst || !n_copies) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (seq_len < 0 || n_new < 0 || block_size < 1 || max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID_ARG, "seq_len and n_new must be >= 0, block_size and max_blocks positive");
  *n_copies = 0;
  if (n_new == 0) return ok();
  const int64_t have = ((int64_t)seq_len + block_size - 1) / block_size;  // blocks the sequence owns
  const int64_t first = seq_len / block_size, last = ((int64_t)seq_len + n_new - 1) / block_size;
  if (last >= max_blocks_per_seq) return fail(PKV_ERR_INVALID_ARG, "block table row too short");
  std::lock_guard<std::mutex> g(pool->mu);
  for (int64_t j = 0; j < have; ++j)
    if (!pool->allocated(table_row[j]))
      return fail(PKV_ERR_INVALID_ARG, "row entry %lld names block %d, which is not allocated", (long long)j,
                  table_row[j]);
  // only the partly filled last block can exist already
  const bool cow = first < have && pool->ref[table_row[first]] > 1;
  const int64_t need = (cow ? 1 : 0) + (last + 1 - std::max(have, first));
  if ((size_t)need > pool->free_ids.size())
    return fail(PKV_ERR_NO_BLOCKS, "the append needs %lld blocks, %zu free", (long long)need, pool->free_ids.size());
  for (int64_t j = first; j <= last; ++j) {
    if (j < have) {
      if (cow) {
        const int32_t fresh = pool->take();
        *copy_src = table_row[j];
        *copy_dst = fresh;
        *n_copies = 1;
        pool->drop(table_row[j]);
        table_row[j] = fresh;
      }
    } else {
      table_row[j] = pool->take();
    }
  }
  return ok();
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, pkv_dtype cache_dtype, float* k_scale, float* v_scale,
                           int64_t num_blocks, const int32_t* src, const int32_t* dst, int32_t n_pairs,
                           int32_t n_kv_heads, int32_t d_head, int32_t block_size, void* stream) {
  if (n_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "n_pairs must be >= 0");
  if (n_pairs == 0) return ok();
  if (!k_cache || !v_cache || !src || !dst) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (!valid_dtype(cache_dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown dtype");
  if (num_blocks < 1 || n_kv_heads < 1 || d_head < 1 || block_size < 1)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be positive");
  if ((cache_dtype == PKV_FP8_E4M3FN) != (k_scale != nullptr) || (k_scale != nullptr) != (v_scale != nullptr))
    return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale are given exactly for FP8 caches");
  const int64_t block_bytes = (int64_t)n_kv_heads * block_size * d_head * elem_bytes(cache_dtype);
  if (block_bytes % 16 != 0) return fail(PKV_ERR_UNSUPPORTED, "a block must be a multiple of 16 bytes");
  if (n_pairs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 pairs per call");
  return hip_status(pkv::launch_copy_blocks(k_cache, v_cache, k_scale, v_scale, num_blocks, src, dst, n_pairs,
                                            block_bytes, n_kv_heads, (hipStream_t)stream),
                    "copy_blocks launch");
}

}  // extern "C"
