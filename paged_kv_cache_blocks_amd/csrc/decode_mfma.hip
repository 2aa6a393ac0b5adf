// Paged GQA decode on the matrix cores (d = 128, bf16 or fp8 E4M3 KV).
//
// Same method as the VALU decode kernel ("KV cache, PagedAttention and
// FlashAttention", Problem 5: tiles of K and V, running max and sum, deferred
// division; "Memory Management in LLM Serving Systems", MHA/MQA/GQA: the G
// query heads of a group share every K and V element), with the two dot
// products done by v_mfma_f32_16x16x32_bf16.  A KV head's G query heads are
// the 16 columns of the MFMA tile (columns G..15 are zero queries whose
// results are dropped), so one K or V fragment read from LDS feeds all G
// heads.  With fp8 KV the VALU work per byte (two bf16 dot products per
// element and head) is what limits the VALU kernel; here the products cost
// 16 MFMAs per 32 tokens and the vector units only convert, stage and run the
// softmax.
//
// Work decomposition (as the VALU kernel's partition mode): one workgroup per
// (sequence, KV head chunk, partition), in the caller's work order if given
// (sequences, or (sequence, partition) units), the KV head chunks of one
// (sequence, partition) on one XCD; its four waves take 32-token chunks
// (two 16-token tiles) round robin and keep their own running state, merged
// at the end through LDS.  Each tile is two 8-token halves, each inside one
// cache block whatever the block size (8 .. 256) and table format.  Per chunk
// a wave:
//   loads the K and V rows of its two tiles with coalesced, non-temporal
//   16-byte loads (issued one chunk ahead, from a scalar base per half),
//   and writes them into its own LDS region in a swizzled row layout: K as
//   bf16 (fp8 codes widened, exactly), V as bf16 or as the fp8 codes, which
//   the value product widens as it reads them (on a partition's last chunk,
//   V rows past its end are written as zeros: their zero weights must not
//   meet a NaN, and only that chunk masks scores);
//   S^T = K q^T: 2 token tiles x 4 d steps, K fragments from LDS, q^T in
//   registers; the fp8 K scale of each half's block multiplies its scores;
//   online softmax per head column (in-lane max over the lane's 8 tokens,
//   then across the four lane rows); weights rounded to bf16, the running sum
//   adds the same rounded weights, and with fp8 each half's V scale
//   multiplies its weights before the value product;
//   O^T += V^T P^T: 8 d tiles, V^T fragments read with ds_read_b64_tr_b16
//   (bf16) or ds_read_b64_tr_b8 and widened (fp8).
// With fp8 KV a wave's LDS region is 12 KiB (bf16: 16 KiB), which with 160
// VGPRs lets three workgroups share a CU: measured 2% faster on the serving
// mix than two workgroups with two chunks in flight per wave.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int D = 128;
constexpr int kB = 16;                 // tokens per tile
constexpr int kCT = 32;                // tokens per wave chunk (two tiles)
constexpr int kW = 4;                  // waves per workgroup
constexpr int kTileB = kCT * 256;      // one K or V chunk in LDS (bf16 rows of 256 bytes)
constexpr int kTile8B = kCT * 128;     // one V chunk of fp8 codes (rows of 128 bytes)
// LDS per wave: the K chunk as bf16, then the V chunk as bf16 (bf16 KV) or as
// the cache's fp8 codes (fp8 KV, widened as the value product reads them)
template <int KIND> constexpr int wave_lds_bytes() { return kTileB + (KIND == KIND_FP8 ? kTile8B : kTileB); }
constexpr int kMaxHeads = 16;          // MFMA columns
constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)
constexpr float kSlack = 8.f;          // log2 units: the running max moves only past this

template <int KIND> struct Slab;
// bf16: a tile is 16 rows x 256 bytes; load i, lane l brings row 4 i + l / 16,
// piece l % 16 (loads 0, 1: the first half, 2, 3: the second)
template <> struct Slab<KIND_BF16> {
  static constexpr int row_bytes = 256;
  static constexpr int loads = 4;
};
// fp8: 16 rows x 128 bytes; load i, lane l brings row 8 i + l / 8, fp8 piece
// l % 8 (16 codes = bf16 pieces 2 (l % 8) and 2 (l % 8) + 1); load i is half i
template <> struct Slab<KIND_FP8> {
  static constexpr int row_bytes = 128;
  static constexpr int loads = 2;
};

__device__ __forceinline__ int seq_len_of(const DecodeArgs& a, const PageRow& pr, int s) {
  return min(max(a.seq_lens[s], 0), pr.n << a.log2_bs);
}

// Block id of the block holding token tok (as page_block), read without a
// branch: an entry past the table row reads the valid word `spare` instead
// and is replaced by block 0.  A guarded load would make the wave wait for it
// where the branch rejoins; this one is waited for only where it is used.
__device__ __forceinline__ int page_block_nowait(const DecodeArgs& a, const PageRow& r, int tok,
                                                 const int32_t* spare) {
  const int j = tok >> a.log2_bs;
  const bool in = j < r.n;
  const int v = *(in ? r.ids + j : spare);
  return min(max(in ? v : 0, 0), (int)(a.num_blocks - 1));
}

__device__ __forceinline__ void put_out(const DecodeArgs& a, int64_t idx, float v) {
  if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[idx] = (__bf16)v;
  else reinterpret_cast<float*>(a.out)[idx] = v;
}

}  // namespace

// The decode's LDS tile layout: as swz (pkv_device.h), with the permutation
// f = (r1 ^ r3, r0, r1, r2 ^ r3 in bits 0..3): besides the K and V reads it
// serves the bf16 staging writes (one row per 16 lanes) and the fp8 K staging
// writes (eight pieces 2j, or 2j + 1, of two consecutive rows per 16 lanes)
// without bank conflicts under the 16-byte access rule given there.
__device__ __forceinline__ int dswz(int row, int piece) {
  const int r = row & 15;
  const int f = ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 1) ^ (r >> 3)) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 3);
  return row * 256 + ((piece ^ f) << 4);
}

// Slot permutation of the fp8 V chunk's 128-byte rows (eight 16-byte pieces,
// piece p of row r in slot p ^ f8(r)): the transposing reads take one piece of
// rows {4g .. 4g + 3, 16 + 4g .. 16 + 4g + 3} for g = 0, 1 (or 2, 3) at once,
// the staging writes eight pieces of two consecutive rows; rows of one parity
// share a bank half, and f8 is one-to-one over the eight even (and the eight
// odd) rows of each read.
__device__ __forceinline__ int f8_slot(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
// ds_read_b64_tr_b8: lane L of a 16-lane group receives byte L of the eight
// 16-byte rows its lane pairs (2 r, 2 r + 1: bytes 0-7, 8-15 of row r) read
__device__ __forceinline__ v2i ds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(__attribute__((address_space(3))) char*)(p));
}

// FP8 KV: three workgroups per CU (48 KiB of LDS each, three waves per SIMD),
// so a workgroup that starts and waits for its first loads leaves two others
// streaming; bf16 KV: two.
template <int KIND, int GW>
__global__ __launch_bounds__(256, KIND == KIND_FP8 ? 3 : 2) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(GW >= 1 && GW <= kMaxHeads, "heads per workgroup");
  using SL = Slab<KIND>;
  constexpr int kWaveB = wave_lds_bytes<KIND>();
  __shared__ __align__(16) char smem[kW * kWaveB];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = lane & 15, g = lane >> 4;
  const int hk = a.n_kv * a.head_chunks;
  // Workgroup -> (unit slot, KV head chunk): the dispatcher deals workgroups
  // to the eight XCDs in turn (workgroup b to XCD b % 8), so the hk workgroups
  // of one unit slot are numbered 8 apart and share an XCD and its L2: the
  // sequence's table entries and, with fp8, each block's line of per-head
  // scales are then read from memory once per XCD instead of once per KV
  // head.  The grid rounds the slots up to a multiple of 8.  (8 is MI355X's
  // XCD count in its single-partition mode; with another count only the L2
  // sharing is lost, never a result.)
  const int xcd = blockIdx.x % 8, jx = blockIdx.x / 8;
  const int kvc = jx % hk;
  const int slot = (jx / hk) * 8 + xcd;
  if (slot >= a.batch * a.n_parts) return;
  // The unit (sequence, partition) of this workgroup; results do not depend
  // on which workgroup takes which unit.  With a unit order (split calls,
  // pkv_paged_attn_decode_order) entry `slot` names the unit, longest first,
  // and -1 marks a unit without tokens, so real second partitions start early
  // and the empty ones come last.  Otherwise the slots run partition by
  // partition, mapped through the caller's sequence order if any (long
  // sequences paired with short ones on a CU, or the longest first).
  int s, part;
  if (a.work_order && a.order_units) {
    const int u = __builtin_amdgcn_readfirstlane(a.work_order[slot]);
    if (u < 0) return;
    const int uc = min(u, a.batch * a.n_parts - 1);
    s = uc / a.n_parts;
    part = uc % a.n_parts;
  } else {
    s = slot % a.batch;
    if (a.work_order) s = __builtin_amdgcn_readfirstlane(min(max(a.work_order[s], 0), a.batch - 1));
    part = slot / a.batch;
  }
  const int kvh = kvc / a.head_chunks;
  const int h0 = kvh * a.group + (kvc % a.head_chunks) * GW;
  const int p0 = part * a.part_tokens;
  const PageRow pr = page_row(a, s);

  // Where this wave's tiles live: lane i holds tile (i & 1) of the wave's
  // chunk i >> 1 (partition chunk w + 4 (i >> 1)), so a partition has at most
  // 4 x 32 chunks of 32 tokens (the host caps it at 4096), as the cache row index of
  // each half's first row; fp8 scales of each half's block ride along.  A
  // tile past the partition keeps row 0: it is loaded all the same, so the
  // loads need no branch, and its rows, being past the end, are masked (K)
  // or staged as zeros (V).
  // The table entries of every lane's tiles are read before the sequence's
  // length is known (an entry past the table row reads as block 0), and so
  // are the queries: neither waits for the other, nor for the length.
  const int len_raw = a.seq_lens[s];
  const int pb = (w + kW * (lane >> 1)) * 2 + (lane & 1);
  int id_of[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) id_of[h] = page_block_nowait(a, pr, p0 + kB * pb + 8 * h, a.seq_lens + s);

  // q^T fragments (B operand): lane (n, g) holds head n, d = 32 ks + 8 g .. + 7
  u32x4 qf[4];
  {
    const bool real = n < GW;
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)s * a.n_q + h0 + (real ? n : 0)) * D * 2;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 v = ld16(qrow + (32 * ks + 8 * g) * 2);
      qf[ks] = real ? v : u32x4{0, 0, 0, 0};
    }
  }

  // the loads above stay above the branch below (the compiler would sink
  // them past it, behind the length's latency); nothing waits for their data
  asm volatile("" ::: "memory");
  const int L = min(max(len_raw, 0), pr.n << a.log2_bs);
  if (a.n_parts > 1 && p0 >= L) return;
  const int plen = max(0, min(a.part_tokens, L - p0));  // tokens of this partition
  const int nblk = (plen + kB - 1) / kB;
  const int n_chunks = (nblk + 1) / 2;
  const int n_my = n_chunks > w ? (n_chunks - w + kW - 1) / kW : 0;

  // Rows and scales of this lane's tiles, without branches (a branch around a
  // load makes the wave wait for it where the paths rejoin): the scale reads
  // use the clamped block id, always inside the pool.  A half wholly past the
  // partition keeps row 0 and scale 1: its table entry may be clamped or
  // stale, its scale anything (NaN included), and the zero weights of its
  // masked tokens must not meet it.
  uint32_t my_row[2];
  float my_ks[2] = {1.f, 1.f}, my_vs[2] = {1.f, 1.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tok = p0 + kB * pb + 8 * h;
    const int id = id_of[h];
    my_row[h] = pb < nblk ? page_row_index(a, id, kvh, tok) : 0u;
    if constexpr (KIND == KIND_FP8) {
      const bool live = pb < nblk && tok < p0 + plen;
      const float ks = a.k_scale[(int64_t)id * a.n_kv + kvh];
      const float vs = a.v_scale[(int64_t)id * a.n_kv + kvh];
      my_ks[h] = live ? ks : 1.f;
      my_vs[h] = live ? vs : 1.f;
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  char* const k_lds = smem + w * kWaveB;
  char* const v_lds = k_lds + kTileB;
  const char* const kc = reinterpret_cast<const char*>(a.k_cache);
  const char* const vc = reinterpret_cast<const char*>(a.v_cache);

  u32x4 bk[2][SL::loads], bv[2][SL::loads];
  // Loads take a scalar base (the half's first row, read from its lane) plus
  // this lane's 32-bit offset, so the per-load address work is scalar.
  const uint32_t lane_off = (uint32_t)lane * 16;
  auto issue = [&](int c) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint64_t half0 = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(my_row[0], 2 * c + b) * SL::row_bytes;
      const uint64_t half1 = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(my_row[1], 2 * c + b) * SL::row_bytes;
#pragma unroll
      for (int i = 0; i < SL::loads; ++i) {
        constexpr int LH = SL::loads / 2;  // loads per half
        const uint64_t h = i < LH ? half0 : half1;
        const uint32_t off = (uint32_t)((i % LH) * kWave * 16) + lane_off;
        bk[b][i] = ld16_stream(kc + h + off);
        bv[b][i] = ld16_stream(vc + h + off);
      }
    }
  };

  // Stage the chunk's K and V rows into LDS (bf16 rows, swizzled).  Only a
  // chunk that runs past the partition's end (TAIL) writes its V rows there
  // as zeros; the others store every row as loaded.
  auto stage = [&](int t0, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < SL::loads; ++i) {
        if constexpr (KIND == KIND_BF16) {
          const int r = kB * b + 4 * i + (lane >> 4);  // chunk row
          const int pc = lane & 15;
          const bool live = !TAIL || t0 + r < plen;
          st16(k_lds + dswz(r, pc), bk[b][i]);
          st16(v_lds + dswz(r, pc), live ? bv[b][i] : u32x4{0, 0, 0, 0});
        } else {
          const int r = kB * b + 8 * i + (lane >> 3);
          const int p8 = lane & 7;
          const bool live = !TAIL || t0 + r < plen;
          // Lane p8 widens its 16 codes into bf16 pieces 2 p8 and 2 p8 + 1;
          // lanes 4-7 of each eight store the odd piece first, so each store
          // instruction's eight lanes (one pass) cover all eight 16-byte bank
          // groups of a 128-byte pass
          const bool odd_first = p8 >= 4;
          const u32x4 c = bk[b][i];
          const uint32_t c0 = odd_first ? c[2] : c[0], c1 = odd_first ? c[3] : c[1];
          const uint32_t c2 = odd_first ? c[0] : c[2], c3 = odd_first ? c[1] : c[3];
          uint32_t kb[8];
          fp8x4_to_bf16x4(c0, kb[0], kb[1]);
          fp8x4_to_bf16x4(c1, kb[2], kb[3]);
          fp8x4_to_bf16x4(c2, kb[4], kb[5]);
          fp8x4_to_bf16x4(c3, kb[6], kb[7]);
          const int pc0 = 2 * p8 + (odd_first ? 1 : 0);
          st16(k_lds + dswz(r, pc0), u32x4{kb[0], kb[1], kb[2], kb[3]});
          st16(k_lds + dswz(r, pc0 ^ 1), u32x4{kb[4], kb[5], kb[6], kb[7]});
          // V codes as loaded (zero codes past the partition: +0)
          st16(v_lds + r * 128 + ((p8 ^ f8_slot(r)) << 4), live ? bv[b][i] : u32x4{0, 0, 0, 0});
        }
      }
    }
  };

  const float sl = a.scale_log2;
  if (n_my > 0) issue(0);
  for (int c = 0; c < n_my; ++c) {
    const int t0 = (w + kW * c) * kCT;  // first token of the chunk (partition-relative)
    const bool tail = t0 + kCT > plen;  // wave-uniform: only a partition's last chunk

    wave_lds_sync();  // this wave's reads of the previous chunk are done
    if (tail) stage(t0, std::true_type{});
    else stage(t0, std::false_type{});
    // the registers are free again: fetch the next chunk while this one computes
    if (c + 1 < n_my) issue(c + 1);
    wave_lds_sync();

    // ---- S^T = K q^T: token tiles t (block t of the chunk) x 4 d steps ----
    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) st[t] = mfma_bf16(ld16(k_lds + dswz(16 * t + n, 4 * ks + g)), qf[ks], st[t]);
    }

    // ---- online softmax for head column n over tokens t0 + 16 t + 4 g + j ----
    float sc[2][4];
    float mx = -INFINITY;
    auto scores = [&](auto tail_tag) {
      constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // this lane's tokens 4 g .. 4 g + 3 of tile t lie in half g / 2
        float kscale = 1.f;
        if constexpr (KIND == KIND_FP8) {
          const float k0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_ks[0]), 2 * c + t));
          const float k1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_ks[1]), 2 * c + t));
          kscale = g < 2 ? k0 : k1;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tok = t0 + 16 * t + 4 * g + j;
          sc[t][j] = (!TAIL || tok < plen) ? st[t][j] * (sl * kscale) : -INFINITY;
          mx = fmaxf(mx, sc[t][j]);
        }
      }
    };
    if (tail) scores(std::true_type{});
    else scores(std::false_type{});
    mx = max_xor32(max_xor16(mx));
    const float m_new = (mx > m_run + kSlack) ? mx : m_run;  // m_run = -inf takes mx
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    uint32_t pw[2][2];  // weights for the value product (fp8: times the block's V scale)
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = exp2_fast(sc[t][j] - m_use);
      const uint32_t r0 = pack_bf16(p[0], p[1]), r1 = pack_bf16(p[2], p[3]);
      ls = dot2_bf16(r1, kOnes, dot2_bf16(r0, kOnes, ls));  // the sum adds the rounded weights
      if constexpr (KIND == KIND_FP8) {
        const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_vs[0]), 2 * c + t));
        const float v1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_vs[1]), 2 * c + t));
        const float vscale = g < 2 ? v0 : v1;
        pw[t][0] = pack_bf16(p[0] * vscale, p[1] * vscale);
        pw[t][1] = pack_bf16(p[2] * vscale, p[3] * vscale);
      } else {
        pw[t][0] = r0;
        pw[t][1] = r1;
      }
    }
    l_run = l_run * alpha + ls;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }

    // ---- O^T += V^T P^T: lane group g's weights are tokens {4g..4g+3,
    // 16+4g..16+4g+3}; the transposing reads fetch V rows in that order ----
    const u32x4 pf = u32x4{pw[0][0], pw[0][1], pw[1][0], pw[1][1]};
    if constexpr (KIND == KIND_FP8) {
      // lane pair (2 b, 2 b + 1) of group g reads the row of the group's token
      // b (4 g + b, then 16 + 4 g + b - 4), so lane m receives the eight codes
      // V[token b][16 dt + m], b = 0..7, in the order of its weights
      const int b = n >> 1;
      const int key = (b < 4 ? 4 * g + b : 16 + 4 * g + b - 4);
      const char* row = v_lds + key * 128 + 8 * (n & 1);
      const int fs = f8_slot(key);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v2i c = ds_read_tr8(row + ((dt ^ fs) << 4));
        uint32_t v0, v1, v2, v3;
        fp8x4_to_bf16x4((uint32_t)c[0], v0, v1);
        fp8x4_to_bf16x4((uint32_t)c[1], v2, v3);
        o[dt] = mfma_bf16(u32x4{v0, v1, v2, v3}, pf, o[dt]);
      }
    } else {
      const int jj = (lane >> 2) & 3, qq = lane & 3;
      const int key_a = 4 * g + jj, key_b = key_a + 16;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int pc = 2 * dt + (qq >> 1), half = (qq & 1) * 8;
        const u32x2 lo = ds_read_tr(v_lds + dswz(key_a, pc) + half);
        const u32x2 hi = ds_read_tr(v_lds + dswz(key_b, pc) + half);
        o[dt] = mfma_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, o[dt]);
      }
    }
  }

  // ---- merge the four waves: lane (n, g) holds O^T[16 dt + 4 g + j][head n] ----
  const float l_head = sum_xor32(sum_xor16(l_run));
  __syncthreads();  // every wave is done with its LDS region
  // rows of kMoRow floats: the eight lanes a 16-byte store serves together
  // (heads n .. n + 7) start 16 bytes apart modulo the 128 bytes of a pass (a
  // 128-float row would put them on one bank group, 136 on every other)
  constexpr int kMoRow = D + 4;
  float* mo = reinterpret_cast<float*>(smem);     // [wave][head][kMoRow]
  float* mml = mo + kW * kMaxHeads * kMoRow;      // [wave][head][2]
  if (g == 0) {
    mml[(w * kMaxHeads + n) * 2 + 0] = m_run;
    mml[(w * kMaxHeads + n) * 2 + 1] = l_head;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<f32x4*>(mo + (w * kMaxHeads + n) * kMoRow + 16 * dt + 4 * g) = o[dt];
  __syncthreads();
  for (int idx = threadIdx.x; idx < GW * D; idx += 256) {
    const int h = idx / D, col = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) M = fmaxf(M, mml[(ww * kMaxHeads + h) * 2]);
    float lsum = 0.f, osum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) {
        const float mw = mml[(ww * kMaxHeads + h) * 2];
        const float e = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
        lsum = fmaf(e, mml[(ww * kMaxHeads + h) * 2 + 1], lsum);
        osum = fmaf(e, mo[(ww * kMaxHeads + h) * kMoRow + col], osum);
      }
    }
    const int hq = h0 + h;
    if (a.n_parts == 1 || L <= a.part_tokens) {  // the sequence's only partition: final output
      put_out(a, ((int64_t)s * a.n_q + hq) * D + col, lsum > 0.f ? osum / lsum : 0.f);
    } else {
      const int64_t pi = ((int64_t)s * a.n_q + hq) * a.n_parts + part;
      a.ws_o[pi * D + col] = osum;
      if (col == 0) {
        a.ws_ml[pi * 2 + 0] = M;
        a.ws_ml[pi * 2 + 1] = lsum;
      }
    }
  }
}

bool decode_mfma_supported(int kv_kind, int d, int heads_per_wg) {
  return (kv_kind == KIND_BF16 || kv_kind == KIND_FP8) && d == D &&
         (heads_per_wg == 16 || heads_per_wg == 8 || heads_per_wg == 4);
}

template <int KIND, int GW>
static int mfma_wgs_per_cu() {
  int nwg = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nwg, decode_mfma_kernel<KIND, GW>, 256, 0) != hipSuccess) return 1;
  return nwg > 0 ? nwg : 1;
}

// uncached: the C-ABI layer caches it per device
int decode_mfma_wgs_per_cu(int kv_kind, int heads_per_wg) {
  if (kv_kind == KIND_BF16)
    return heads_per_wg == 16 ? mfma_wgs_per_cu<KIND_BF16, 16>()
           : heads_per_wg == 8 ? mfma_wgs_per_cu<KIND_BF16, 8>() : mfma_wgs_per_cu<KIND_BF16, 4>();
  return heads_per_wg == 16 ? mfma_wgs_per_cu<KIND_FP8, 16>()
         : heads_per_wg == 8 ? mfma_wgs_per_cu<KIND_FP8, 8>() : mfma_wgs_per_cu<KIND_FP8, 4>();
}

template <int KIND>
static hipError_t launch_kind(const DecodeArgs& a, unsigned wgs, hipStream_t stream) {
  switch (a.group / a.head_chunks) {
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<KIND, 16>), dim3(wgs), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<KIND, 8>), dim3(wgs), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<KIND, 4>), dim3(wgs), dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_kind, hipStream_t stream) {
  // unit slots rounded up to a multiple of 8, each with its KV head chunks
  const int64_t wgs = ((int64_t)a.n_parts * a.batch + 7) / 8 * 8 * a.n_kv * a.head_chunks;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  return kv_kind == KIND_FP8 ? launch_kind<KIND_FP8>(a, (unsigned)wgs, stream)
                             : launch_kind<KIND_BF16>(a, (unsigned)wgs, stream);
}

}  // namespace pkv
