// Chunked-prefill attention over a paged KV cache on gfx950 bf16 MFMA.
//
// Method ("KV cache, PagedAttention and FlashAttention", Problem 5: tiles of
// Q, K, V in on-chip memory, online softmax with running max and sum, one
// fused kernel; "Memory Management in LLM Serving Systems", FlashAttention:
// masked positions are -inf and fully masked blocks are skipped, GQA lets the
// query heads of a group share each K/V tile; FlashAttention-2: Q is split
// across waves while every wave sees the whole K/V tile, and the division by
// the row sum waits until the end).
//
// Work decomposition
//   1-D grid over (query tile, KV head, sequence) work items, placed so the
//   query tiles of one (sequence, KV head) share an XCD; 256 threads = 4 waves.
//   A workgroup owns 64 NT packed query rows of one sequence and one KV head
//   (NT = 2 or 3): row r = (token r / G, head r % G), so the G heads that
//   share the KV head reuse every K/V tile.  Each wave owns 16 NT rows (NT
//   16-row MFMA tiles).
//   Per 64-key tile (eight 8-key halves, each inside one cache block of 8 ..
//   256 tokens, looked up in the 2-D or CSR table):
//     K and V slabs -> LDS (16-byte loads, issued one tile ahead);
//     S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (K from LDS, Q in registers),
//     so each lane holds four keys of one query row;
//     causal mask only on tiles that cross the diagonal; online softmax per
//     row (in-lane max over 16 keys + two cross-lane steps);
//     P^T (bf16) is already in the B-operand layout of the next product, so
//     O^T += V^T P^T uses V^T fragments read with ds_read_b64_tr_b16.
//   FP8 KV: each wave brings its block's codes (half the bytes) into a
//   double-buffered staging area and, once the previous tile is consumed,
//   widens them to bf16 (exact) into the same single tile layout; each
//   16-key score tile is one cache block, so its K scale multiplies that
//   tile's scores, and the V scale of a key's block multiplies the key's
//   softmax weight as it is packed for the value product (the row sum takes
//   the weights unscaled).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int D = 128;
constexpr int BS = 16;          // keys per wave part of a tile (two 8-key halves, each in one cache block)
constexpr int KT = 64;          // keys per tile
constexpr int ROWS = 128;       // packed query rows per workgroup with two row tiles per wave
constexpr int ROWB = D * 2;      // bytes of one bf16 K or V row
constexpr int TILE_B = KT * ROWB;  // one K (or V) tile in LDS
constexpr int STAGE_B = 2 * TILE_B;  // K tile then V tile
constexpr int kStages = 2;      // tiles in flight through LDS
constexpr int kXcds = 8;        // XCDs the dispatcher spreads workgroup ids over
constexpr int kMaxSortSeqs = 256;  // batches up to this size are ordered longest first
constexpr int BLK8_B = BS * D;     // FP8 codes of one wave part (16 keys) of K or V
constexpr int STG8_B = (KT / BS) * 2 * BLK8_B;  // one tile's K and V codes
static_assert(STAGE_B + 2 * STG8_B <= kStages * STAGE_B, "FP8 tile + staging must fit the bf16 stages");

// LDS tiles use the swizzled row layout of swz() (pkv_device.h): rows unpadded, since the
// direct global->LDS loads write 1 KiB of consecutive LDS each.


constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // bf16 pair (1, 1)
constexpr float kRescaleSlack = 8.f;           // log2 units: weights stay <= 256

// Keeps a rarely taken branch a branch: without it the compiler may turn the
// body into selects executed on every tile.
__device__ __forceinline__ void no_if_conversion() { asm volatile("" ::: "memory"); }

}  // namespace

template <bool FP8, int NT>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  // bf16 KV: kStages tiles (K then V).  FP8 KV: one bf16 tile at the start,
  // then two staging buffers of codes, per wave [K block][V block].
  __shared__ __align__(16) char smem[kStages * STAGE_B];
  __shared__ float blk_scale[2][2 * KT / BS];  // FP8: K and V scale of each 8-token half of the tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
  const int G = a.group;
  const int tq = 64 * NT / G;           // tokens per workgroup (64 NT packed rows)
  // Work order.  Sequences are taken longest first (most keys: context plus
  // chunk), so the long workgroups start early and short ones fill the end;
  // within a sequence the later query tiles, which see more keys, go first.
  // Workgroup ids go round-robin over the 8 XCDs, each with its own L2: id i
  // runs on XCD i % 8 and takes query tile (i / 8) % q_tiles of pair
  // p = ((i / 8) / q_tiles) * 8 + i % 8 in that order, pair p = (sequence
  // rank p / n_kv, KV head p % n_kv).  So every query tile of a pair, all
  // reading the same K/V tiles, runs on one XCD and shares its L2, while the
  // pairs of a sequence spread over the XCDs and keep their loads even.
  // (Pair counts that are not a multiple of 8 keep the XCD-blind order.)
  __shared__ int seq_key[kMaxSortSeqs], seq_at_rank[kMaxSortSeqs];
  const bool sorted = a.num_seqs <= kMaxSortSeqs;
  if (sorted) {
    const int t = threadIdx.x;
    if (t < a.num_seqs) {
      const int cs = min(max(a.ctx_lens[t], 0), page_row(a, t).n << a.log2_bs);
      const int qb = min(max(a.cu_q[t], 0), a.total_q), qe = min(max(a.cu_q[t + 1], qb), a.total_q);
      seq_key[t] = cs + (qe - qb);
    }
    __syncthreads();
    if (t < a.num_seqs) {
      const int k = seq_key[t];
      int rank = 0;
      for (int u = 0; u < a.num_seqs; ++u) {
        const int ku = seq_key[u];
        rank += (ku > k) || (ku == k && u < t);
      }
      seq_at_rank[rank] = t;
    }
    __syncthreads();
  }
  const int q_tiles = (a.max_q_len + tq - 1) / tq;
  const int n_pairs = a.n_kv * a.num_seqs;
  const int id = blockIdx.x;
  int qt, pair;
  if (n_pairs % kXcds == 0) {
    const int j = id / kXcds;
    qt = j % q_tiles;
    pair = (j / q_tiles) * kXcds + id % kXcds;
  } else {
    qt = id % q_tiles;
    pair = id / q_tiles;
  }
  qt = q_tiles - 1 - qt;
  const int kvh = pair % a.n_kv;
  const int s = __builtin_amdgcn_readfirstlane(sorted ? seq_at_rank[pair / a.n_kv] : pair / a.n_kv);
  const int q0 = qt * tq;               // first chunk token of the tile
  // a packed-query range outside [0, total_q) is clipped so no access leaves q or out
  const int qs = min(max(a.cu_q[s], 0), a.total_q);
  const int q_len = min(a.cu_q[s + 1], a.total_q) - qs;
  if (q0 >= q_len) return;
  const PageRow prow = page_row(a, s);
  // context and keys are capped at the table row's capacity, so no tile
  // reaches past the row (callers keep ctx + q_len within it)
  const int cap = prow.n << a.log2_bs;
  const int ctx = min(max(a.ctx_lens[s], 0), cap);
  const int total = min(ctx + q_len, cap);  // keys that exist for this sequence
  const int last_q = min(q0 + tq, q_len) - 1;
  // keys any row of the tile sees (none when the table row is empty)
  const int kv_end = prow.n == 0 ? 0 : a.causal ? min(ctx + last_q + 1, total) : total;
  const int n_tiles = (kv_end + KT - 1) / KT;
  const int diag0 = ctx + q0;           // keys >= diag0 are masked for some row

  const int n = lane & 15;   // column (query row within a 16-row tile)
  const int g = lane >> 4;   // lane group

  // ---- Q^T fragments (B operand): row = (w*NT + nt)*16 + n, d = 32*ds + 8g + e
  u32x4 qf[NT][4];
  int row_tok[NT], row_head[NT], row_lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = (w * NT + nt) * 16 + n;
    const int tok = q0 + r / G;
    row_tok[nt] = tok;
    row_head[nt] = kvh * G + r % G;
    row_lim[nt] = a.causal ? min(ctx + tok, total - 1) : total - 1;  // last visible key
    const bool ok = tok < q_len;
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(qs + (ok ? tok : 0)) * a.n_q + row_head[nt]) * D * 2;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const u32x4 v = ld16(qrow + (32 * ds + 8 * g) * 2);
      qf[nt][ds] = ok ? v : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 o[8][NT];  // O^T[16*dt + 4g + j][row n]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  // ---- tile loads: wave w brings keys 16 w .. 16 w + 15 of the tile straight
  // into LDS, 4 KiB of K and 4 KiB of V in four 1-KiB instructions each; the
  // block ids of its two halves are fetched one tile ahead of the loads
  const char* const kc = reinterpret_cast<const char*>(a.k_cache);
  const char* const vc = reinterpret_cast<const char*>(a.v_cache);

  const int n_lblocks = (kv_end + BS - 1) / BS;  // 16-key parts any row of the workgroup sees
  // The raw table entry is fetched one tile ahead and checked only when its
  // loads are issued, so nothing waits on the fetch in between.
  // A tile part (16 keys) is two 8-key halves, each inside one cache block.
  // Only the entry index is clamped here (to the row, which is not empty when
  // there are tiles); the ids are checked when their loads are issued, so the
  // wave does not wait on this fetch in between.
  auto fetch_id = [&](int kt) {
    const int tok = (kt * (KT / BS) + w) * BS;
    const int last = prow.n - 1;
    return int2{prow.ids[min(tok >> a.log2_bs, last)], prow.ids[min((tok + 8) >> a.log2_bs, last)]};
  };
  // Per-lane source offsets inside a block, one per instruction k: lane l
  // brings key row r = 4k + l / 16 and the global piece that lands in slot
  // l % 16 of that row (r < 16, so the swizzle takes r as is).
  // (Instructions 0, 1 bring the first half's rows, 2, 3 the second's;
  // offsets are relative to the half's first row.)
  uint32_t src_off[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 4 * k + (lane >> 4);
    src_off[k] = (r & 7) * ROWB + (((lane & 15) ^ swz_f(r)) << 4);
  }
  const uint32_t lds0 = lds_addr(smem) + BS * w * ROWB;  // this wave's first tile row
  // FP8: this wave's staging slot and the scales of the block it loads
  const uint32_t stg0 = lds_addr(smem) + STAGE_B + w * 2 * BLK8_B;
  float ks_load[2] = {0.f, 0.f}, vs_load[2] = {0.f, 0.f};  // scales of the halves last issued (0 when none)
  auto issue = [&](int kt, int2 raw_id) {
    const int lb = kt * (KT / BS) + w;
    if (FP8) {
      ks_load[0] = ks_load[1] = vs_load[0] = vs_load[1] = 0.f;
    }
    if (lb >= n_lblocks) return;  // nothing to load for this wave
    const int nb1 = (int)(a.num_blocks - 1);
    const int id[2] = {min(max(__builtin_amdgcn_readfirstlane(raw_id.x), 0), nb1),
                       min(max(__builtin_amdgcn_readfirstlane(raw_id.y), 0), nb1)};
    int64_t half[2];  // byte offset of each half's first row (KV head kvh)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      half[h] = (int64_t)page_row_index(a, id[h], kvh, lb * BS + 8 * h) * (FP8 ? D : ROWB);
    if (FP8) {
      const uint32_t dst = stg0 + (kt & 1) * STG8_B;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        lds_dma16(kc + half[k], 16 * lane, dst + k * 1024);
        lds_dma16(vc + half[k], 16 * lane, dst + BLK8_B + k * 1024);
      }
      // a half wholly past the keys the workgroup sees keeps scale 0: its
      // table entry may be clamped or stale and its scale anything (NaN
      // included), which the zero weights of its masked keys must not meet
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool live = lb * BS + 8 * h < kv_end;
        ks_load[h] = live ? a.k_scale[(int64_t)id[h] * a.n_kv + kvh] : 0.f;
        vs_load[h] = live ? a.v_scale[(int64_t)id[h] * a.n_kv + kvh] : 0.f;
      }
    } else {
      const uint32_t dst = lds0 + (kt % kStages) * STAGE_B;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lds_dma16(kc + half[k >> 1], src_off[k], dst + 4 * k * ROWB);
        lds_dma16(vc + half[k >> 1], src_off[k], dst + TILE_B + 4 * k * ROWB);
      }
    }
  };
  int2 id_next = int2{0, 0};
  if (n_tiles > 0) {
    issue(0, fetch_id(0));
    if (n_tiles > 1) id_next = fetch_id(1);
  }

  const float sl = a.scale_log2;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const char* const k_lds = smem + (FP8 ? 0 : (kt % kStages) * STAGE_B);
    const char* const v_lds = k_lds + TILE_B;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of tile kt have landed
    // FP8: scales of this wave's halves of tile kt
    const float ks_tile0 = ks_load[0], ks_tile1 = ks_load[1], vs_tile0 = vs_load[0], vs_tile1 = vs_load[1];
    if (!FP8 && kt * KT + KT > kv_end) {
      // the keys this workgroup sees end inside this tile: V rows past them
      // (rows no load wrote, or past the sequence end) may hold anything, NaN
      // included, and the zero weights every real row gives them must not
      // meet a NaN.  K rows need no clearing: their scores are masked.
      no_if_conversion();
      for (int idx = lane; idx < BS * 16; idx += kWave) {
        const int r = BS * w + idx / 16;
        if (kt * KT + r >= kv_end) st16(const_cast<char*>(v_lds) + r * ROWB + (idx % 16) * 16, u32x4{0, 0, 0, 0});
      }
    }
    __syncthreads();  // tile kt is in LDS; every wave is done with tile kt - 1
    if (kt + 1 < n_tiles) {
      issue(kt + 1, id_next);
      if (kt + 2 < n_tiles) id_next = fetch_id(kt + 2);
    }
    // FP8: this lane's K and V scale per 16-key part t of the tile: its keys
    // 4 g .. 4 g + 3 of each part lie in the part's half g / 2
    float ksc[KT / BS], vsc[KT / BS];
    if (FP8) {
      // widen this wave's block of codes into rows 16w .. 16w+15 of the bf16
      // tile: lane l converts row l / 4, values 32 (l % 4) .. +31; V rows past
      // the keys the tile sees become zeros (their weights are zero, and a
      // zero weight must not meet a NaN)
      const char* stg = smem + STAGE_B + (kt & 1) * STG8_B + w * 2 * BLK8_B;
      const int r = lane >> 2, c = (lane & 3) * 32;
      const int row = BS * w + r;
      const bool live = kt * KT + row < kv_end;
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        const u32x4 c0 = ld16(stg + kv * BLK8_B + r * D + c);
        const u32x4 c1 = ld16(stg + kv * BLK8_B + r * D + c + 16);
        const uint32_t cw[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        uint32_t bw[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) fp8x4_to_bf16x4(cw[i], bw[2 * i], bw[2 * i + 1]);
        const bool keep = kv == 0 || live;
        char* dst = smem + kv * TILE_B;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st16(dst + swz(row, (lane & 3) * 4 + i),
               keep ? u32x4{bw[4 * i], bw[4 * i + 1], bw[4 * i + 2], bw[4 * i + 3]} : u32x4{0, 0, 0, 0});
      }
      if (lane == 0) {
        blk_scale[0][2 * w] = ks_tile0;
        blk_scale[0][2 * w + 1] = ks_tile1;
        blk_scale[1][2 * w] = vs_tile0;
        blk_scale[1][2 * w + 1] = vs_tile1;
      }
      __syncthreads();  // the bf16 tile and its scales are complete
      const int hs = g >> 1;
#pragma unroll
      for (int t = 0; t < KT / BS; ++t) {
        const float k0 = blk_scale[0][2 * t], k1 = blk_scale[0][2 * t + 1];
        const float v0 = blk_scale[1][2 * t], v1 = blk_scale[1][2 * t + 1];
        ksc[t] = hs ? k1 : k0;
        vsc[t] = hs ? v1 : v0;
      }
    }

    // ---- S^T = K Q^T : four 16-key tiles x NT row tiles.  Wave priority by
    // phase: the two waves sharing a SIMD come from different workgroups and
    // drift in and out of step; a wave in a product phase is preferred at
    // issue (value products most), so the matrix core keeps its queue while
    // the other wave's softmax fills the VALU slots between (measured 4-6 %
    // faster than equal priorities).
    __builtin_amdgcn_s_setprio(1);
    f32x4 st_[4][NT];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st_[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments of the next 32-wide d step are read while this step's
    // MFMAs run (two groups of four fragments in flight)
    if constexpr (NT == 2) {
      u32x4 kf[2][4];
#pragma unroll
      for (int t = 0; t < 4; ++t) kf[0][t] = ld16(k_lds + swz(16 * t + n, g));
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        if (ds + 1 < 4) {
#pragma unroll
          for (int t = 0; t < 4; ++t) kf[(ds + 1) & 1][t] = ld16(k_lds + swz(16 * t + n, 4 * (ds + 1) + g));
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's MFMAs
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) st_[t][nt] = mfma_bf16(kf[ds & 1][t], qf[nt][ds], st_[t][nt]);
      }
    } else {
      // more row tiles: one fragment (16 keys x 32 d) ahead, fewer registers
      u32x4 kf[2];
      kf[0] = ld16(k_lds + swz(n, g));
#pragma unroll
      for (int i = 0; i < 16; ++i) {  // i = 4 ds + t
        const int ds = i >> 2, t = i & 3;
        if (i + 1 < 16) kf[(i + 1) & 1] = ld16(k_lds + swz(16 * ((i + 1) & 3) + n, 4 * ((i + 1) >> 2) + g));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st_[t][nt] = mfma_bf16(kf[i & 1], qf[nt][ds], st_[t][nt]);
      }
    }

    if (FP8) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st_[t][nt] *= ksc[t];
    }

    // ---- mask, online softmax, P^T fragments.  The reference max m is kept
    // in log2 units (scale * log2 e folded in), so each weight is one FMA and
    // one exp2.  m moves only when a row's max exceeds it by more than
    // kRescaleSlack: weights up to 2^kRescaleSlack are exact in the same way
    // (the final division by l cancels any common reference), and the output
    // accumulators are rescaled only on those rare moves.
    __builtin_amdgcn_s_setprio(0);
    const bool need_mask = (a.causal && kt * KT + KT - 1 > diag0) || (kt * KT + KT > total);
    u32x4 pf[2][NT];  // B operand per 32-key step
    if (need_mask) {
      no_if_conversion();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kt * KT + 16 * t + 4 * g + j;
            st_[t][nt][j] = (key <= row_lim[nt]) ? st_[t][nt][j] : -INFINITY;
          }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          mx = fmaxf(mx, st_[t][nt][j]);
        }
      mx = max_xor32(max_xor16(mx));
      const float mt = mx * sl;
      const float m_new = (mt > m_run[nt] + kRescaleSlack) ? mt : m_run[nt];  // m_run = -inf takes mt
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run[nt] - m_use);
      m_run[nt] = m_new;
      uint32_t pk[4][2];
      float ls = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float p4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p4[j] = exp2_fast(fmaf(st_[t][nt][j], sl, -m_use));
        if (FP8) {
          // weights enter the value product scaled by their block's V scale
          ls += (p4[0] + p4[1]) + (p4[2] + p4[3]);
          const float vs = vsc[t];
          pk[t][0] = pack_bf16(p4[0] * vs, p4[1] * vs);
          pk[t][1] = pack_bf16(p4[2] * vs, p4[3] * vs);
        } else {
          pk[t][0] = pack_bf16(p4[0], p4[1]);
          pk[t][1] = pack_bf16(p4[2], p4[3]);
          // the row sum takes the same bf16-rounded weights the product uses
          ls = dot2_bf16(pk[t][0], kOnesBf16x2, ls);
          ls = dot2_bf16(pk[t][1], kOnesBf16x2, ls);
        }
      }
      l_run[nt] = l_run[nt] * alpha + ls;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pf[ks][nt] = u32x4{pk[2 * ks][0], pk[2 * ks][1], pk[2 * ks + 1][0], pk[2 * ks + 1][1]};
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
        no_if_conversion();
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt][nt] *= alpha;
      }
    }

    // ---- O^T += V^T P^T
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int jj = (lane >> 2) & 3;  // which of the four keys this lane's read supplies
      const int qq = lane & 3;         // which 4-column group
      const int key_a = 32 * ks + 4 * g + jj;
      const int key_b = key_a + 16;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int pc = 2 * dt + (qq >> 1), half = (qq & 1) * 8;  // bytes (16 dt + 4 qq) * 2
        const u32x2 lo = ds_read_tr(v_lds + swz(key_a, pc) + half);
        const u32x2 hi = ds_read_tr(v_lds + swz(key_b, pc) + half);
        const u32x4 vf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[dt][nt] = mfma_bf16(vf, pf[ks][nt], o[dt][nt]);
      }
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- normalise and store: lane (n, g) holds d = 16*dt + 4g + j of row n
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_run[nt];
    l = sum_xor32(sum_xor16(l));
    if (row_tok[nt] >= q_len) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t obase = ((int64_t)(qs + row_tok[nt]) * a.n_q + row_head[nt]) * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d0 = 16 * dt + 4 * g;
      const f32x4 v = o[dt][nt] * inv;
      if (a.out_bf16) {
        *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(a.out) + obase + d0) =
            u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + obase + d0) = v;
      }
    }
  }
}

bool prefill_supported_group(int group) {
  return group >= 1 && group <= ROWS && (ROWS % group) == 0;
}

// Rows per wave.  Each 1-KiB K or V fragment read from LDS feeds one product
// per 16-row tile the wave owns.  Three row tiles (48 rows per wave, 192 per
// workgroup; the group size must divide 192) cut the fragment reads per
// product by a third and still fit two waves per SIMD (256 registers, a few
// spilled outside the key loop).  Measured on the 16 x 512-token chunk with
// both builds called in alternation in one process: 425 against 462 us for
// two row tiles.  FP8 caches keep two tiles (their conversion pass needs the
// registers).
static bool three_row_tiles(const PrefillArgs& a) {
  return !a.kv_fp8 && (192 % a.group) == 0;
}

hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t stream) {
  (void)d;
  const int nt = three_row_tiles(a) ? 3 : 2;
  const int tq = 64 * nt / a.group;
  const int64_t n_work = (int64_t)((a.max_q_len + tq - 1) / tq) * a.n_kv * a.num_seqs;
  if (n_work == 0) return hipSuccess;
  if (n_work > 0x7fffffff) return hipErrorInvalidValue;
  if (a.kv_fp8)
    hipLaunchKernelGGL((prefill_kernel<true, 2>), dim3((unsigned)n_work), dim3(256), 0, stream, a);
  else if (nt == 3)
    hipLaunchKernelGGL((prefill_kernel<false, 3>), dim3((unsigned)n_work), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<false, 2>), dim3((unsigned)n_work), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
