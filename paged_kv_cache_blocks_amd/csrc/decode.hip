// Paged decode attention for gfx950: split-K over the sequence with a
// FlashAttention-style online softmax per wave, merged per workgroup, and a
// merge pass for sequences that several workgroups share.
//
// Method ("KV cache, PagedAttention and FlashAttention", Problem 5: tiling,
// online softmax with a running max m and sum l rescaled by e^(m - m_new),
// kernel fusion, and the serving note that decode reads K and V once and
// splits a long sequence across thread blocks; "Memory Management in LLM
// Serving Systems", FlashAttention-2: rescale once per block, divide by l at
// the very end, parallelise over the sequence as well as batch and head; GQA:
// the query heads of a group are processed against the same K/V block).
//
// A workgroup (4 waves) serves GW query heads that share one KV head.  Its
// waves take the 16-token tiles of a range round-robin in chunks of CB tiles;
// a tile is two 8-token halves, each inside one cache block whatever the
// block size (8 .. 256) and table format; per chunk a wave
//   1. has the chunk's K and V rows in registers (coalesced 16-byte loads,
//      issued while the previous chunk computed; the table is walked once per
//      range, one tile per lane);
//   2. stages K into LDS as bf16 rows (fp8 converted here, once per element)
//      and V as bf16 token *pairs* interleaved per column, so the value
//      product runs on v_dot2c_f32_bf16;
//   3. scores: lane (head h, token t, d-half) holds half of q[h] in registers
//      and reads half of the K row from LDS; a DPP add joins the halves.
//      Every K element is fetched from HBM once and serves all GW heads;
//   4. online softmax over the chunk with DPP lane-group reductions; the
//      weights go to LDS as bf16 pairs (fp8: times their half's V scale);
//   5. values: lane c owns output columns (2c, 2c+1) for all GW heads and
//      accumulates dot2(weight pair, value pair) in f32.
// f32 caches take the same path with f32 rows and fma in place of dot2.
//
// Work split.  Partition mode: fixed-size token partitions per (sequence,
// KV head) on a 1-D grid, then a merge of each sequence's partitions.
// Work-queue mode: each (sequence, KV head) is cut into items of equal block
// counts; a resident set of workgroups takes two items each and then claims
// the rest from a counter, so faster XCDs take more; a merge kernel combines
// each sequence's items.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kBlock = 16;  // tokens per tile (two 8-token halves; a cache block holds 8 .. 256 tokens)
constexpr int kWaves = 4;   // waves per workgroup
constexpr int kSegBlocks = kWaves * kWave;  // blocks one id load covers (one id per lane per wave)

constexpr int align16(int x) { return (x + 15) & ~15; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int KIND, int D>
struct Geo {
  static constexpr int esize = KindBytes<KIND>::v;
  static constexpr int row_bytes = D * esize;           // one token row of one KV head in HBM
  static constexpr int LW = row_bytes >= 128 ? 16 : 8;   // bytes per lane per load
  static constexpr int LPR = row_bytes / LW;             // lanes per row
  static constexpr int RPI = kWave / LPR;                // rows per load instruction
  static constexpr int NLK = kBlock / RPI;               // load instructions per tile
  static constexpr int EPL = LW / esize;                 // elements per lane per load
  static_assert(LPR <= kWave && NLK >= 2 && NLK % 2 == 0, "slab geometry");
};

template <int LW> struct LoadVec;
template <> struct LoadVec<16> { typedef u32x4 T; };
template <> struct LoadVec<8> { typedef u32x2 T; };

// Compile-time layout of one (element kind, head dim, heads per workgroup).
template <int KIND, int D, int GW>
struct Lay {
  using Gm = Geo<KIND, D>;
  using LV = typename LoadVec<Gm::LW>::T;
  static constexpr bool F32P = (KIND == KIND_F32);
  // score layout: each (token, head) score is split over QS adjacent lanes
  // that each hold 1/QS of q[head] (fewer registers, more waves per SIMD)
  static constexpr int QS = 2;
  static constexpr int TG = kWave / GW;                 // lanes per head group
  static constexpr int T = TG / QS;                     // tokens per score round
  // blocks per chunk: a round must fit in a chunk, and fp8 takes two blocks
  // so a chunk still moves 8 KiB of K+V per wave
  static constexpr int CB = (T > kBlock ? T / kBlock : 1) * (KIND == KIND_FP8 ? 2 : 1);
  static constexpr int CT = CB * kBlock;                // tokens per chunk
  static constexpr int R = CT / T;                      // score rounds per chunk
  static constexpr int ES = F32P ? 4 : 2;               // bytes per element in LDS
  static constexpr int KROW = D * ES + 16;              // padded K row in LDS
  static constexpr int VROW = D * 4 + 16;               // f32 V row, or one bf16-pair row
  static constexpr int NPAIR = kBlock / 2;              // token pairs per block
  static constexpr int K_BYTES = CT * KROW;
  static constexpr int V_BYTES = F32P ? CT * VROW : CB * NPAIR * VROW;
  static constexpr int P_BYTES = F32P ? CT * GW * 4 : CB * NPAIR * GW * 4;
  static constexpr int A_BYTES = align16(GW * 4);
  static constexpr int WAVE_BYTES = align16(K_BYTES + V_BYTES + P_BYTES + A_BYTES);
  static constexpr int MERGE_BYTES = kWaves * GW * D * 4 + kWaves * GW * 2 * 4;
  static constexpr int SMEM = cmax(kWaves * WAVE_BYTES, MERGE_BYTES);
  // value-product layout
  static constexpr int PVL = F32P ? kWave : D / 2;      // lanes covering one row
  static constexpr int PVG = kWave / PVL;               // row groups (bf16 path, d = 64)
  static constexpr int COLS = F32P ? D / kWave : 2;     // output columns per lane
  static constexpr int QV = (F32P ? D / 4 : D / 8) / QS;  // 16-byte pieces of q per lane
  static_assert(COLS >= 1 && PVG >= 1 && R >= 1 && CT % T == 0, "layout");
};

// Per-wave running state: q slice, running max (log2 units), this lane's share
// of the running sum, and the output accumulators.
template <int KIND, int D, int GW>
struct WaveState {
  using Ly = Lay<KIND, D, GW>;
  u32x4 qv[Ly::QV];
  float m_run, l_run;
  float o[GW][Ly::COLS];
};

template <int KIND, int D, int GW>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int s, int h0, int lane, WaveState<KIND, D, GW>& ws) {
  using Ly = Lay<KIND, D, GW>;
  const int sh = lane / Ly::TG, qh = lane % Ly::QS;
  const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)s * a.n_q + h0 + sh) * D * Ly::ES;
#pragma unroll
  for (int j = 0; j < Ly::QV; ++j) ws.qv[j] = ld16(qrow + (qh * Ly::QV + j) * 16);
}

template <int KIND, int D, int GW>
__device__ __forceinline__ void reset_state(WaveState<KIND, D, GW>& ws) {
  ws.m_run = -INFINITY;
  ws.l_run = 0.f;
#pragma unroll
  for (int h = 0; h < GW; ++h)
#pragma unroll
    for (int k = 0; k < Lay<KIND, D, GW>::COLS; ++k) ws.o[h][k] = 0.f;
}

// Where this wave's 16-token tiles [blk_begin, blk_begin + nblk) (nblk <=
// kSegBlocks) of sequence s live, one tile per lane: lane i <-> tile (i % CB)
// of the wave's chunk i / CB (= range chunk w + 4 * (i / CB)), as the cache
// row index (KV head kvh) of the first row of each 8-token half; block ids
// outside the pool or the table row are clamped into the pool, and tiles past
// the range keep row 0 (loaded all the same, then masked).  fp8: the K and V
// scales of each half's block ride along.
struct BlockIds {
  uint32_t row[2];
  float ks[2], vs[2];
};

template <int KIND, int D, int GW>
__device__ __forceinline__ BlockIds load_ids(const DecodeArgs& a, int s, int kvh, int blk_begin, int nblk, int w,
                                             int lane) {
  constexpr int CB = Lay<KIND, D, GW>::CB;
  BlockIds r{{0u, 0u}, {1.f, 1.f}, {1.f, 1.f}};
  const int pb_lane = (w + kWaves * (lane / CB)) * CB + lane % CB;
  if (pb_lane < nblk) {
    const PageRow pr = page_row(a, s);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tok = (blk_begin + pb_lane) * kBlock + 8 * h;
      const int id = page_block(a, pr, tok);
      r.row[h] = page_row_index(a, id, kvh, tok);
      if constexpr (KIND == KIND_FP8) {
        r.ks[h] = a.k_scale[(int64_t)id * a.n_kv + kvh];
        r.vs[h] = a.v_scale[(int64_t)id * a.n_kv + kvh];
      }
    }
  }
  return r;
}

// Chunks of a range this wave takes (chunks go round-robin over the waves).
template <int KIND, int D, int GW>
__device__ __forceinline__ int wave_chunks(int nblk, int w) {
  constexpr int CB = Lay<KIND, D, GW>::CB;
  const int n_chunks = (nblk + CB - 1) / CB;
  return n_chunks > w ? (n_chunks - w + kWaves - 1) / kWaves : 0;
}

// The K and V slabs of one chunk in flight (registers).
template <int KIND, int D, int GW>
struct SlabRegs {
  using Ly = Lay<KIND, D, GW>;
  typename Ly::LV bk[Ly::CB][Ly::Gm::NLK], bv[Ly::CB][Ly::Gm::NLK];
};

// Issue the 16-byte loads of the wave's chunk c (rows from load_ids): load
// instruction i covers rows RPI i .. RPI i + RPI - 1 of a tile, so the first
// NLK / 2 fall in the first half and the rest in the second.
template <int KIND, int D, int GW>
__device__ __forceinline__ void issue_chunk(const DecodeArgs& a, const BlockIds& ids, int c, int lane,
                                            SlabRegs<KIND, D, GW>& r) {
  using Ly = Lay<KIND, D, GW>;
  using Gm = typename Ly::Gm;
  using LV = typename Ly::LV;
  constexpr int LH = Gm::NLK / 2;
  const char* const kc = reinterpret_cast<const char*>(a.k_cache);
  const char* const vc = reinterpret_cast<const char*>(a.v_cache);
#pragma unroll
  for (int b = 0; b < Ly::CB; ++b) {
    // row indices are unsigned 32-bit (the row space reaches 2^32): widen
    // them without sign extension
    const int64_t half0 = (int64_t)(uint32_t)__builtin_amdgcn_readlane(ids.row[0], c * Ly::CB + b) * Gm::row_bytes;
    const int64_t half1 = (int64_t)(uint32_t)__builtin_amdgcn_readlane(ids.row[1], c * Ly::CB + b) * Gm::row_bytes;
#pragma unroll
    for (int i = 0; i < Gm::NLK; ++i) {
      const int64_t off = (i < LH ? half0 : half1) + (int64_t)((i % LH) * kWave + lane) * Gm::LW;
      // read once: non-temporal loads (see ld16_stream)
      r.bk[b][i] = __builtin_nontemporal_load(reinterpret_cast<const LV*>(kc + off));
      r.bv[b][i] = __builtin_nontemporal_load(reinterpret_cast<const LV*>(vc + off));
    }
  }
}

// Blocks [blk_begin, blk_begin + nblk) (nblk <= kSegBlocks) of sequence s,
// KV head kvh; the four waves interleave chunks.  Tokens at or past L, or past
// the range, are masked.  Accumulates into this wave's state.  On entry the
// loads of the wave's first chunk are in flight in `slabs` (if it has one).
// first_staged() runs once, right after the wave's first chunk is staged;
// after_stage() runs once the wave's last chunk is staged and the registers
// are free (the caller may start the next range's loads there);
// after_scores() once the last chunk's scores are done and q is free.
template <int KIND, int D, int GW, class FirstStaged, class AfterStage, class AfterScores>
__device__ __forceinline__ void run_blocks(const DecodeArgs& a, int s, int kvh, int blk_begin, int nblk, int L,
                                           int w, int lane, char* wbase, WaveState<KIND, D, GW>& ws,
                                           SlabRegs<KIND, D, GW>& slabs, const BlockIds& ids,
                                           FirstStaged first_staged, AfterStage after_stage,
                                           AfterScores after_scores) {
  using Ly = Lay<KIND, D, GW>;
  using Gm = typename Ly::Gm;
  constexpr bool F32P = Ly::F32P;
  constexpr int T = Ly::T, TG = Ly::TG, QS = Ly::QS, CB = Ly::CB, CT = Ly::CT, R = Ly::R, ES = Ly::ES;
  constexpr int KROW = Ly::KROW, VROW = Ly::VROW, NPAIR = Ly::NPAIR, PVL = Ly::PVL, PVG = Ly::PVG;
  constexpr int COLS = Ly::COLS, QV = Ly::QV;

  const int n_my = wave_chunks<KIND, D, GW>(nblk, w);
  if (n_my == 0) return;
  // a chunk may extend past the range (nblk not a multiple of CB): tokens
  // there belong to another range even when the sequence goes on
  L = min(L, (blk_begin + nblk) * kBlock);
  const int sh = lane / TG, st = (lane % TG) / QS, qh = lane % QS;
  const int tok0 = blk_begin * kBlock;  // sequence position of the range's first token

  char* const k_lds = wbase;
  char* const v_lds = wbase + Ly::K_BYTES;
  char* const p_lds = v_lds + Ly::V_BYTES;
  float* const a_lds = reinterpret_cast<float*>(p_lds + Ly::P_BYTES);
  auto& bk = slabs.bk;
  auto& bv = slabs.bv;

  for (int c = 0; c < n_my; ++c) {
    set_priority_for_progress(c, n_my);
    const int ct0 = (w + kWaves * c) * CT;      // first token of the chunk (range-relative)
    const int nvalid = L - (tok0 + ct0);        // tokens of the chunk that exist (may exceed CT)
    float kscale[2 * CB], vscale[2 * CB];  // per 8-token half of the chunk
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        kscale[2 * b + h] = vscale[2 * b + h] = 1.f;
        // a half wholly past the range keeps scale 1: its block id may be a
        // clamped or stale table entry whose scale is anything (NaN included),
        // and its zero weights must not meet it
        if constexpr (KIND == KIND_FP8) {
          if (8 * (2 * b + h) < nvalid) {
            kscale[2 * b + h] =
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ids.ks[h]), c * CB + b));
            vscale[2 * b + h] =
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ids.vs[h]), c * CB + b));
          }
        }
      }

    wave_lds_sync();
    // ---- stage K rows (bf16 or f32) and V (bf16 pairs or f32 rows) into LDS ----
#pragma unroll
    for (int b = 0; b < CB; ++b) {
#pragma unroll
      for (int i = 0; i < Gm::NLK; ++i) {
        const int r = lane / Gm::LPR + Gm::RPI * i;
        const int c0 = (lane % Gm::LPR) * Gm::EPL;
        char* dst = k_lds + (b * kBlock + r) * KROW + c0 * ES;
        if constexpr (KIND == KIND_FP8) {
          constexpr int NW = Gm::LW / 4;
          uint32_t wv[NW];
          __builtin_memcpy(wv, &bk[b][i], Gm::LW);
          uint32_t bw[2 * NW];
#pragma unroll
          for (int e = 0; e < NW; ++e) fp8x4_to_bf16x4(wv[e], bw[2 * e], bw[2 * e + 1]);
#pragma unroll
          for (int e = 0; e < NW / 2; ++e) st16(dst + e * 16, u32x4{bw[4 * e], bw[4 * e + 1], bw[4 * e + 2], bw[4 * e + 3]});
        } else {
          st16(dst, bk[b][i]);
        }
      }
      const bool tail = nvalid < (b + 1) * kBlock;  // some rows of this block are past the end
      if constexpr (F32P) {
#pragma unroll
        for (int i = 0; i < Gm::NLK; ++i) {
          const int r = lane / Gm::LPR + Gm::RPI * i;
          const int c0 = (lane % Gm::LPR) * Gm::EPL;
          u32x4 v = bv[b][i];
          if (tail && b * kBlock + r >= nvalid) v = u32x4{0, 0, 0, 0};
          st16(v_lds + (b * kBlock + r) * VROW + c0 * 4, v);
        }
      } else {
#pragma unroll
        for (int i = 0; i < Gm::NLK; i += 2) {
          const int g = lane / Gm::LPR;
          const int r0 = g + Gm::RPI * i, r1 = r0 + Gm::RPI;
          const int pq = g + Gm::RPI * (i / 2);
          const int c0 = (lane % Gm::LPR) * Gm::EPL;
          constexpr int NB = Gm::EPL / 2;  // bf16 dwords per row piece
          uint32_t A[NB], Bv[NB];
          if constexpr (KIND == KIND_FP8) {
            constexpr int NW = Gm::LW / 4;
            uint32_t wa[NW], wb[NW];
            __builtin_memcpy(wa, &bv[b][i], Gm::LW);
            __builtin_memcpy(wb, &bv[b][i + 1], Gm::LW);
#pragma unroll
            for (int e = 0; e < NW; ++e) {
              fp8x4_to_bf16x4(wa[e], A[2 * e], A[2 * e + 1]);
              fp8x4_to_bf16x4(wb[e], Bv[2 * e], Bv[2 * e + 1]);
            }
          } else {
            __builtin_memcpy(A, &bv[b][i], Gm::LW);
            __builtin_memcpy(Bv, &bv[b][i + 1], Gm::LW);
          }
          uint32_t pr[2 * NB];
#pragma unroll
          for (int e = 0; e < NB; ++e) {
            pr[2 * e] = pair_lo(A[e], Bv[e]);
            pr[2 * e + 1] = pair_hi(A[e], Bv[e]);
          }
          if (tail) {
            // rows past the end may hold NaN: clear their half of every pair
            const uint32_t keep = (b * kBlock + r0 < nvalid ? 0x0000ffffu : 0u) |
                                  (b * kBlock + r1 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
            for (int e = 0; e < 2 * NB; ++e) pr[e] &= keep;
          }
          char* dst = v_lds + (b * NPAIR + pq) * VROW + c0 * 4;
#pragma unroll
          for (int e = 0; e < NB / 2; ++e) st16(dst + e * 16, u32x4{pr[4 * e], pr[4 * e + 1], pr[4 * e + 2], pr[4 * e + 3]});
        }
      }
    }
    if (c == 0) first_staged();
    // the registers are free again: fetch the next chunk while this one computes
    if (c + 1 < n_my) issue_chunk<KIND, D, GW>(a, ids, c + 1, lane, slabs);
    else after_stage();
    wave_lds_sync();

    // ---- scores and online softmax ----
    float sc[R];
    float cmax_ = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int tau = r * T + st;  // token within the chunk
      const char* krow = k_lds + tau * KROW + qh * QV * 16;
      float acc0, acc1, acc2, acc3;
      if constexpr (F32P) {
        acc0 = acc1 = acc2 = acc3 = 0.f;
#pragma unroll
        for (int j = 0; j < QV; ++j) {
          const u32x4 kp = ld16(krow + j * 16);
          acc0 = fmaf(__uint_as_float(ws.qv[j][0]), __uint_as_float(kp[0]), acc0);
          acc1 = fmaf(__uint_as_float(ws.qv[j][1]), __uint_as_float(kp[1]), acc1);
          acc2 = fmaf(__uint_as_float(ws.qv[j][2]), __uint_as_float(kp[2]), acc2);
          acc3 = fmaf(__uint_as_float(ws.qv[j][3]), __uint_as_float(kp[3]), acc3);
        }
      } else {
        const u32x4 k0 = ld16(krow);
        acc0 = dot2_bf16(ws.qv[0][0], k0[0], 0.f);
        acc1 = dot2_bf16(ws.qv[0][1], k0[1], 0.f);
        acc2 = dot2_bf16(ws.qv[0][2], k0[2], 0.f);
        acc3 = dot2_bf16(ws.qv[0][3], k0[3], 0.f);
#pragma unroll
        for (int j = 1; j < QV; ++j) {
          const u32x4 kp = ld16(krow + j * 16);
          acc0 = dot2_bf16(ws.qv[j][0], kp[0], acc0);
          acc1 = dot2_bf16(ws.qv[j][1], kp[1], acc1);
          acc2 = dot2_bf16(ws.qv[j][2], kp[2], acc2);
          acc3 = dot2_bf16(ws.qv[j][3], kp[3], acc3);
        }
      }
      float dot = (acc0 + acc1) + (acc2 + acc3);
      dot += dpp_f<DPP_QUAD_XOR1>(dot);  // the other d-half of this (token, head)
      float ksc = kscale[0];
#pragma unroll
      for (int hb = 1; hb < 2 * CB; ++hb) ksc = (tau / 8 == hb) ? kscale[hb] : ksc;
      const float sv = dot * (a.scale_log2 * ksc);
      sc[r] = (tau < nvalid) ? sv : -INFINITY;
      cmax_ = fmaxf(cmax_, sc[r]);
    }
    if (c + 1 == n_my) after_scores();
    cmax_ = group_max<TG>(cmax_);
    const float m_new = fmaxf(ws.m_run, cmax_);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(ws.m_run - m_use);
    ws.m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int tau = r * T + st;
      float p = exp2_fast(sc[r] - m_use);
      if constexpr (F32P) {
        if (qh == 0) reinterpret_cast<float*>(p_lds)[tau * GW + sh] = p;
      } else {
        p = round_bf16(p);
        const int b = tau / kBlock, t = tau % kBlock;
        const int i = t / Gm::RPI, g = t % Gm::RPI;
        const int pq = g + Gm::RPI * (i / 2);
        // fp8: the weight enters the value product times its half's V scale
        float pv = p;
        if constexpr (KIND == KIND_FP8) {
          float vsc = vscale[0];
#pragma unroll
          for (int hb = 1; hb < 2 * CB; ++hb) vsc = (tau / 8 == hb) ? vscale[hb] : vsc;
          pv = p * vsc;
        }
        if (qh == 0) reinterpret_cast<__bf16*>(p_lds)[((b * NPAIR + pq) * GW + sh) * 2 + (i & 1)] = (__bf16)pv;
      }
      lsum += (qh == 0) ? p : 0.f;
    }
    ws.l_run = ws.l_run * alpha + lsum;
    // alpha is exactly 1 for a head whose running max did not move
    const bool rescale = __builtin_amdgcn_ballot_w64(alpha != 1.f) != 0;
    if (rescale && st == 0 && qh == 0) a_lds[sh] = alpha;
    wave_lds_sync();

    // ---- rescale and accumulate P V ----
    if (rescale) {
      float al[GW];
#pragma unroll
      for (int h = 0; h < GW; ++h) al[h] = a_lds[h];
#pragma unroll
      for (int h = 0; h < GW; ++h)
#pragma unroll
        for (int k = 0; k < COLS; ++k) ws.o[h][k] *= al[h];
    }
    if constexpr (F32P) {
      const int col = lane * COLS;
#pragma unroll 4
      for (int tau = 0; tau < CT; ++tau) {
        float pp[GW];
#pragma unroll
        for (int h = 0; h < GW; ++h) pp[h] = reinterpret_cast<const float*>(p_lds)[tau * GW + h];
        const float* vr = reinterpret_cast<const float*>(v_lds + tau * VROW) + col;
        float vv[COLS];
#pragma unroll
        for (int k = 0; k < COLS; ++k) vv[k] = vr[k];
#pragma unroll
        for (int h = 0; h < GW; ++h)
#pragma unroll
          for (int k = 0; k < COLS; ++k) ws.o[h][k] = fmaf(pp[h], vv[k], ws.o[h][k]);
      }
    } else {
      const int pg = lane / PVL;
      const int dcol = (lane % PVL) * 2;
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        float t[GW][2];
#pragma unroll
        for (int h = 0; h < GW; ++h) {
          t[h][0] = ws.o[h][0];
          t[h][1] = ws.o[h][1];
        }
#pragma unroll
        for (int qq = 0; qq < NPAIR / PVG; ++qq) {
          const int pq = qq * PVG + pg;
          uint32_t pp[GW];
          const uint32_t* prow = reinterpret_cast<const uint32_t*>(p_lds) + (b * NPAIR + pq) * GW;
#pragma unroll
          for (int h = 0; h < GW; ++h) pp[h] = prow[h];
          const u32x2 vv = *reinterpret_cast<const u32x2*>(v_lds + (b * NPAIR + pq) * VROW + dcol * 4);
#pragma unroll
          for (int h = 0; h < GW; ++h) {
            t[h][0] = dot2_bf16(pp[h], vv[0], t[h][0]);
            t[h][1] = dot2_bf16(pp[h], vv[1], t[h][1]);
          }
        }
#pragma unroll
        for (int h = 0; h < GW; ++h) {
          ws.o[h][0] = t[h][0];
          ws.o[h][1] = t[h][1];
        }
      }
    }
  }
}

// Merge the four waves' states in LDS.  emit(h, col, M, l, o) is called once
// per (head, column) of the workgroup, spread over the 256 threads; M is in
// log2 units and (l, o) are unnormalised.  All threads must call it.
template <int KIND, int D, int GW, class Emit>
__device__ __forceinline__ void merge_waves(char* smem, int w, int lane, WaveState<KIND, D, GW>& ws, Emit emit) {
  using Ly = Lay<KIND, D, GW>;
  constexpr int COLS = Ly::COLS, PVL = Ly::PVL, PVG = Ly::PVG, TG = Ly::TG, QS = Ly::QS;
  const int sh = lane / TG, st = (lane % TG) / QS, qh = lane % QS;
  const float l_head = group_sum<TG>(ws.l_run);
  if constexpr (!Ly::F32P && PVG > 1) {
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
      for (int k = 0; k < COLS; ++k) ws.o[h][k] += __shfl_xor(ws.o[h][k], 32);
  }
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);  // [wave][head][d]
  float* mml = mo + kWaves * GW * D;            // [wave][head][2]
  if (st == 0 && qh == 0) {
    mml[(w * GW + sh) * 2 + 0] = ws.m_run;
    mml[(w * GW + sh) * 2 + 1] = l_head;
  }
  if (lane < PVL) {
    const int col = Ly::F32P ? lane * COLS : (lane % PVL) * 2;
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
      for (int k = 0; k < COLS; ++k) mo[(w * GW + h) * D + col + k] = ws.o[h][k];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GW * D; idx += 256) {
    const int h = idx / D, col = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, mml[(ww * GW + h) * 2]);
    float lsum = 0.f, osum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = mml[(ww * GW + h) * 2];
        const float e = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
        lsum = fmaf(e, mml[(ww * GW + h) * 2 + 1], lsum);
        osum = fmaf(e, mo[(ww * GW + h) * D + col], osum);
      }
    }
    emit(h, col, M, lsum, osum);
  }
  __syncthreads();  // the LDS is reused by whatever runs next
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t idx, float v) {
  if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[idx] = (__bf16)v;
  else reinterpret_cast<float*>(a.out)[idx] = v;
}

// tokens of sequence s: its length, capped by what its table row can hold
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int s) {
  return min(max(a.seq_lens[s], 0), page_row(a, s).n << a.log2_bs);
}

// ---------------------------------------------------------------------------
// Partition mode: 1-D grid, KV head (x head chunk) fastest, then sequence, then
// partition, so consecutive workgroups go to different XCDs and every XCD
// sees the same mix of heads, sequences and partitions.
// ---------------------------------------------------------------------------
template <int KIND, int D, int GW>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  using Ly = Lay<KIND, D, GW>;
  __shared__ __align__(16) char smem[Ly::SMEM];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int hk = a.n_kv * a.head_chunks;
  const int kvc = blockIdx.x % hk;
  int s, part;  // the unit this workgroup serves: see the matrix-core kernel
  if (a.work_order && a.order_units) {
    const int u = __builtin_amdgcn_readfirstlane(a.work_order[blockIdx.x / hk]);
    if (u < 0) return;
    const int uc = min(u, a.batch * a.n_parts - 1);
    s = uc / a.n_parts;
    part = uc % a.n_parts;
  } else {
    s = (blockIdx.x / hk) % a.batch;  // sequence slot -> sequence (the caller's work order, if any)
    if (a.work_order) s = __builtin_amdgcn_readfirstlane(min(max(a.work_order[s], 0), a.batch - 1));
    part = blockIdx.x / (hk * a.batch);
  }
  const int kvh = kvc / a.head_chunks;
  const int h0 = kvh * a.group + (kvc % a.head_chunks) * GW;
  const int p0 = part * a.part_tokens;

  // the length, the q rows and the partition's block ids are fetched together
  // (ids for every table entry the partition could use, whatever the length),
  // so the first K/V loads wait on two dependent fetches, not three
  const int nb_cap = a.part_tokens / kBlock;
  const BlockIds ids = load_ids<KIND, D, GW>(a, s, kvh, p0 / kBlock, nb_cap, w, lane);
  WaveState<KIND, D, GW> ws;
  load_q(a, s, h0, lane, ws);
  const int L = clamp_len(a, s);
  if (a.n_parts > 1 && p0 >= L) return;
  const int plen = max(0, min(a.part_tokens, L - p0));
  const int nb_part = (plen + kBlock - 1) / kBlock;
  reset_state(ws);
  SlabRegs<KIND, D, GW> slabs;
  if (wave_chunks<KIND, D, GW>(nb_part, w) > 0) issue_chunk<KIND, D, GW>(a, ids, 0, lane, slabs);
  run_blocks<KIND, D, GW>(a, s, kvh, p0 / kBlock, nb_part, L, w, lane, smem + w * Ly::WAVE_BYTES, ws, slabs, ids,
                          [] {}, [] {}, [] {});
  merge_waves<KIND, D, GW>(smem, w, lane, ws, [&](int h, int col, float M, float l, float o) {
    const int hq = h0 + h;
    if (a.n_parts == 1 || L <= a.part_tokens) {  // the sequence's only partition: final output
      store_out(a, ((int64_t)s * a.n_q + hq) * D + col, l > 0.f ? o / l : 0.f);
    } else {
      const int64_t pi = ((int64_t)s * a.n_q + hq) * a.n_parts + part;
      a.ws_o[pi * D + col] = o;
      if (col == 0) {
        a.ws_ml[pi * 2 + 0] = M;
        a.ws_ml[pi * 2 + 1] = l;
      }
    }
  });
}

// Merge the partitions of one (sequence, query head): the rescale rule of the
// online softmax applied to whole partitions.  One wave per (sequence, head),
// up to kCombineHeads heads of one sequence per workgroup (a sequence with a
// single partition costs one small workgroup, not one per head): lane j takes
// partition j of each group of 64 for the max and the weights, and every lane
// accumulates its output columns over the partitions with each weight
// broadcast from its lane.
constexpr int kCombineHeads = 16;
template <int D>
__global__ __launch_bounds__(kWave * kCombineHeads) void combine_kernel(DecodeArgs a) {
  constexpr int COLS = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int hq = blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int s = blockIdx.y;
  const int L = clamp_len(a, s);
  const int nv = (L + a.part_tokens - 1) / a.part_tokens;
  if (nv == 1 || hq >= a.n_q) return;  // one partition: the split kernel wrote this sequence's output itself
  const int64_t base = ((int64_t)s * a.n_q + hq) * a.n_parts;
  const float* ml = a.ws_ml + base * 2;
  const float* op = a.ws_o + base * D;
  float M = -INFINITY;
  for (int j0 = 0; j0 < nv; j0 += kWave)
    if (j0 + lane < nv) M = fmaxf(M, ml[2 * (j0 + lane)]);
  M = group_max<kWave>(M);
  float den = 0.f, num[COLS];
#pragma unroll
  for (int k = 0; k < COLS; ++k) num[k] = 0.f;
  if (M != -INFINITY) {
    for (int j0 = 0; j0 < nv; j0 += kWave) {
      float wj = 0.f, lj = 0.f;
      if (j0 + lane < nv) {
        const float m = ml[2 * (j0 + lane)];
        lj = ml[2 * (j0 + lane) + 1];
        wj = (m == -INFINITY) ? 0.f : exp2_fast(m - M);
      }
      den += group_sum<kWave>(wj * lj);
      const int cnt = min(kWave, nv - j0);
      int j = 0;
      for (; j + 4 <= cnt; j += 4) {
        float x[4][COLS], e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          e[u] = __shfl(wj, j + u);
#pragma unroll
          for (int k = 0; k < COLS; ++k) x[u][k] = op[(int64_t)(j0 + j + u) * D + lane + k * kWave];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int k = 0; k < COLS; ++k) num[k] = fmaf(e[u], x[u][k], num[k]);
      }
      for (; j < cnt; ++j) {
        const float e = __shfl(wj, j);
#pragma unroll
        for (int k = 0; k < COLS; ++k) num[k] = fmaf(e, op[(int64_t)(j0 + j) * D + lane + k * kWave], num[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < COLS; ++k)
    store_out(a, ((int64_t)s * a.n_q + hq) * D + lane + k * kWave, den > 0.f ? num[k] / den : 0.f);
}

// ---------------------------------------------------------------------------
// Work-queue mode.  Every (sequence, KV head chunk) pair is cut into items of
// U consecutive blocks (the last one shorter), with U chosen on the device so
// that the batch makes about items_per_wg items per workgroup.  Items are
// numbered pair by pair: item = kvc * NI + pre[s] + j, where pre[s] counts the
// items of the sequences before s.  Workgroup g takes items g and g + n_wg,
// then claims further items from a counter in the workspace until none is
// left, so workgroups on faster XCDs simply take more items.  The claim for
// the item after next is made one item ahead, and the next item's block ids,
// q rows and first K/V chunk are fetched while the current item finishes, so
// switching items does not drain the loads in flight.  An item that covers a
// whole pair writes the output; otherwise it writes its partial (m, l, o) to
// slot `item` and the merge kernel combines the pair's consecutive items.
// Results depend only on the item boundaries, never on which workgroup ran an
// item: the output is deterministic.
// ---------------------------------------------------------------------------
constexpr int kItemsPerWg = 8;  // items per workgroup the planner asks for
constexpr int kMinItemBlocks = 8;

struct Item {
  int kvc, s, j0, nblk;  // pair, first block, blocks
};

template <int KIND, int D, int GW>
__global__ __launch_bounds__(256) void decode_queue_kernel(DecodeArgs a) {
  using Ly = Lay<KIND, D, GW>;
  __shared__ __align__(16) char smem[Ly::SMEM];
  extern __shared__ __align__(16) int pre[];  // [batch + 1] item prefix sums (dynamic LDS)
  __shared__ int red[kWaves];
  __shared__ int next_item;
  // q rows of the next item, fetched at the start of the current one and
  // parked in LDS at its end (double buffered by item parity)
  constexpr int QB = GW * D * Ly::ES;  // bytes of q for one item's heads
  constexpr int QN = (QB / 8 + 255) / 256;
  __shared__ __align__(16) char q_lds[2][QB];
  u32x2 qn[QN];
  WaveState<KIND, D, GW> ws;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int hk = a.n_kv * a.head_chunks;

  // block-wide sum of v over the 256 threads
  auto block_sum = [&](int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[w] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) t += red[ww];
    __syncthreads();
    return t;
  };
  // total blocks over the batch, then the item size
  int nb_tot = 0;
  for (int base = 0; base < a.batch; base += 256) {
    const int s = base + threadIdx.x;
    nb_tot += s < a.batch ? (clamp_len(a, s) + kBlock - 1) / kBlock : 0;
  }
  nb_tot = block_sum(nb_tot);
  const int64_t F = (int64_t)hk * nb_tot;
  const int64_t want = (F + (int64_t)a.n_wg * a.items_per_wg - 1) / ((int64_t)a.n_wg * a.items_per_wg);
  const int U = (int)min<int64_t>(max<int64_t>(want, kMinItemBlocks), kSegBlocks);
  // exclusive prefix sums of the items per sequence, 256 sequences per pass
  {
    int carry = 0;
    for (int base = 0; base <= a.batch; base += 256) {
      const int s = base + threadIdx.x;
      const int ni = s < a.batch ? ((clamp_len(a, s) + kBlock - 1) / kBlock + U - 1) / U : 0;
      int incl = ni;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane == kWave - 1) red[w] = incl;
      __syncthreads();
      int run = carry + incl - ni;
      int tot = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        if (ww < w) run += red[ww];
        tot += red[ww];
      }
      if (s <= a.batch) pre[s] = run;
      carry += tot;
      __syncthreads();
    }
  }
  const int NI = pre[a.batch];
  const int n_items = hk * NI;
  if (n_items > a.n_slots) return;  // cannot happen with the planner's workspace; never write past it
  const int n_static = min(n_items, 2 * a.n_wg);

  auto locate = [&](int item) {
    Item it;
    it.kvc = item / NI;
    const int rem = item - it.kvc * NI;
    int lo = 0, hi = a.batch - 1;  // largest s with pre[s] <= rem
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= rem) lo = mid;
      else hi = mid - 1;
    }
    it.s = lo;
    it.j0 = (rem - pre[lo]) * U;
    const int nb = (clamp_len(a, lo) + kBlock - 1) / kBlock;
    it.nblk = min(U, nb - it.j0);
    return it;
  };
  auto head0 = [&](const Item& it) { return (it.kvc / a.head_chunks) * a.group + (it.kvc % a.head_chunks) * GW; };
  auto q_fetch = [&](const Item& it) {  // the item's GW consecutive q rows are contiguous
    const char* src = reinterpret_cast<const char*>(a.q) + ((int64_t)it.s * a.n_q + head0(it)) * D * Ly::ES;
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < QB / 8) qn[i] = *reinterpret_cast<const u32x2*>(src + idx * 8);
    }
  };
  auto q_park = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int idx = threadIdx.x + 256 * i;
      if (idx < QB / 8) *reinterpret_cast<u32x2*>(q_lds[buf] + idx * 8) = qn[i];
    }
  };
  auto q_from_lds = [&](int buf) {
    const int sh = lane / Ly::TG, qh = lane % Ly::QS;
    const char* row = q_lds[buf] + sh * D * Ly::ES;
#pragma unroll
    for (int j = 0; j < Ly::QV; ++j) ws.qv[j] = ld16(row + (qh * Ly::QV + j) * 16);
  };

  int cur = blockIdx.x;
  if (cur >= n_items) return;
  int parity = 0;  // item count of this workgroup, mod 2
  const unsigned n_dyn = (unsigned)(n_items - n_static);
  const int second = cur + a.n_wg < n_static ? cur + a.n_wg : n_items;  // static second item

  SlabRegs<KIND, D, GW> slabs;
  Item ic = locate(cur);
  BlockIds ids_c = load_ids<KIND, D, GW>(a, ic.s, ic.kvc / a.head_chunks, ic.j0, ic.nblk, w, lane);
  load_q(a, ic.s, head0(ic), lane, ws);
  if (wave_chunks<KIND, D, GW>(ic.nblk, w) > 0)
    issue_chunk<KIND, D, GW>(a, ids_c, 0, lane, slabs);

  for (int k = 0;; ++k) {
    // The next item: the static second one after the first, then an item
    // claimed at the start of this one and published right after every wave
    // has staged its first chunk of this one (a barrier each wave reaches
    // exactly once per item), early enough to prefetch its block ids, q rows
    // and first chunk before this item ends.
    unsigned claimed = 0;
    if (threadIdx.x == 0 && k >= 1 && n_dyn > 0) claimed = atomicAdd(a.dyn_counter, 1u);
    int nxt = n_items;
    Item in_{0, 0, 0, 0};
    BlockIds ids_n{{0u, 0u}, {1.f, 1.f}, {1.f, 1.f}};
    int nmy_next = 0;
    auto publish_next = [&] {
      if (threadIdx.x == 0)
        next_item = (k == 0) ? second : (claimed < n_dyn ? n_static + (int)claimed : n_items);
      __syncthreads();
      nxt = next_item;
      if (nxt < n_items) {
        in_ = locate(nxt);
        ids_n = load_ids<KIND, D, GW>(a, in_.s, in_.kvc / a.head_chunks, in_.j0, in_.nblk, w, lane);
        nmy_next = wave_chunks<KIND, D, GW>(in_.nblk, w);
        q_fetch(in_);
      }
    };
    const int kvh = ic.kvc / a.head_chunks;
    const int h0 = head0(ic);
    const int L = clamp_len(a, ic.s);
    const int nb = (L + kBlock - 1) / kBlock;
    reset_state(ws);
    if (wave_chunks<KIND, D, GW>(ic.nblk, w) == 0) {
      // nothing of this item for this wave: go straight to the next one
      publish_next();
      if (nmy_next > 0) issue_chunk<KIND, D, GW>(a, ids_n, 0, lane, slabs);
    } else {
      run_blocks<KIND, D, GW>(
          a, ic.s, kvh, ic.j0, ic.nblk, L, w, lane, smem + w * Ly::WAVE_BYTES, ws, slabs, ids_c, publish_next,
          [&] {
            if (nmy_next > 0) issue_chunk<KIND, D, GW>(a, ids_n, 0, lane, slabs);
          },
          [] {});
    }
    const bool have_next = nxt < n_items;
    if (have_next) q_park(parity ^ 1);  // read after the merge's barriers
    // the merge below reads the states of all four waves
    const bool whole = (ic.j0 == 0 && ic.nblk == nb);
    const int item = cur;
    merge_waves<KIND, D, GW>(smem, w, lane, ws, [&](int h, int col, float M, float l, float o) {
      if (whole) {
        store_out(a, ((int64_t)ic.s * a.n_q + h0 + h) * D + col, l > 0.f ? o / l : 0.f);
      } else {
        const int64_t pi = (int64_t)item * GW + h;
        a.ws_o[pi * D + col] = o;
        if (col == 0) {
          a.ws_ml[pi * 2 + 0] = M;
          a.ws_ml[pi * 2 + 1] = l;
        }
      }
    });
    if (ic.j0 == 0 && threadIdx.x == 0) {
      int4 info;
      info.x = cur;
      info.y = cur + (nb + U - 1) / U - 1;  // the pair's items are consecutive
      info.z = 0;
      info.w = 0;
      reinterpret_cast<int4*>(a.split_info)[(int64_t)ic.s * hk + ic.kvc] = info;
    }
    if (!have_next) break;
    cur = nxt;
    ic = in_;
    ids_c = ids_n;
    parity ^= 1;
    q_from_lds(parity);
  }
}

// Merge the items of the pairs that several items cover: the rescale rule of
// the online softmax applied to whole items.  grid = (pairs, GW / HPW): a
// workgroup takes HPW heads of one pair, E = HPW * D output elements.  With
// E >= 256 each thread folds all items of its elements; with fewer elements
// KS = 256 / E threads share an element, each folding every KS-th item, and
// meet in LDS.  Items are folded eight per batch of independent loads.  Empty
// pairs get zeros here.  Block (0, 0) also rewinds the item counter for the
// next call (the decode kernel has finished by now).
template <int D, int GW>
__global__ __launch_bounds__(256) void combine_queue_kernel(DecodeArgs a, int hpw) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.dyn_counter = 0u;
  constexpr int NB = 8;  // items per batch of loads
  __shared__ float red_m[256], red_l[256], red_o[256];
  const int hk = a.n_kv * a.head_chunks;
  const int kvc = blockIdx.x % hk;
  const int s = blockIdx.x / hk;
  const int kvh = kvc / a.head_chunks;
  const int h0 = kvh * a.group + (kvc % a.head_chunks) * GW;
  const int L = clamp_len(a, s);
  const int hb = blockIdx.y * hpw;
  const int E = hpw * D;
  if (L == 0) {
    for (int idx = threadIdx.x; idx < E; idx += 256)
      store_out(a, ((int64_t)s * a.n_q + h0 + hb + idx / D) * D + idx % D, 0.f);
    return;
  }
  const int4 info = reinterpret_cast<const int4*>(a.split_info)[(int64_t)s * hk + kvc];
  if (info.y <= info.x) return;
  const int n = info.y - info.x + 1;
  const int KS = E >= 256 ? 1 : 256 / E;  // threads per element (E and 256 are powers of two)
  const int ks = threadIdx.x / (256 / KS), e0 = threadIdx.x % (256 / KS);
  for (int e = e0; e < E; e += 256 / KS) {
    const int h = hb + e / D, col = e % D;
    float M = -INFINITY, l = 0.f, o = 0.f;
    for (int k0 = ks; k0 < n; k0 += KS * NB) {
      float mk[NB], lk[NB], ok[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int k = k0 + j * KS;
        mk[j] = -INFINITY;
        lk[j] = ok[j] = 0.f;
        if (k < n) {
          const int64_t pi = (int64_t)(info.x + k) * GW + h;
          mk[j] = a.ws_ml[pi * 2];
          lk[j] = a.ws_ml[pi * 2 + 1];
          ok[j] = a.ws_o[pi * D + col];
        }
      }
      float Mb = M;
#pragma unroll
      for (int j = 0; j < NB; ++j) Mb = fmaxf(Mb, mk[j]);
      if (Mb == -INFINITY) continue;
      const float e_old = exp2_fast(M - Mb);  // 0 while M is still -inf
      l *= e_old;
      o *= e_old;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float ej = (mk[j] == -INFINITY) ? 0.f : exp2_fast(mk[j] - Mb);
        l = fmaf(ej, lk[j], l);
        o = fmaf(ej, ok[j], o);
      }
      M = Mb;
    }
    const int64_t oi = ((int64_t)s * a.n_q + h0 + h) * D + col;
    if (KS == 1) {
      store_out(a, oi, l > 0.f ? o / l : 0.f);
    } else {
      // E < 256: this is the only pass of the element loop
      red_m[threadIdx.x] = M;
      red_l[threadIdx.x] = l;
      red_o[threadIdx.x] = o;
      __syncthreads();
      if (ks == 0) {
        float Mt = -INFINITY;
        for (int j = 0; j < KS; ++j) Mt = fmaxf(Mt, red_m[j * E + e]);
        float lt = 0.f, ot = 0.f;
        if (Mt != -INFINITY) {
          for (int j = 0; j < KS; ++j) {
            const float mj = red_m[j * E + e];
            const float w = (mj == -INFINITY) ? 0.f : exp2_fast(mj - Mt);
            lt = fmaf(w, red_l[j * E + e], lt);
            ot = fmaf(w, red_o[j * E + e], ot);
          }
        }
        store_out(a, oi, lt > 0.f ? ot / lt : 0.f);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int decode_heads_per_wg(int group) {
  for (int g : {8, 4, 2, 1})
    if (group % g == 0) return g;
  return 1;
}

int decode_chunk_blocks(int heads_per_wg) {
  const int t = kWave / heads_per_wg / 2;  // tokens per score round (d split over two lanes)
  return t > kBlock ? t / kBlock : 1;
}

template <int KIND, int D, int GW>
static int queue_wgs_per_cu(int batch) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_queue_kernel<KIND, D, GW>, 256,
                                                   decode_queue_lds_bytes(batch)) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

template <int KIND, int D>
static int queue_wgs_gw(int gw, int batch) {
  switch (gw) {
    case 8: return queue_wgs_per_cu<KIND, D, 8>(batch);
    case 4: return queue_wgs_per_cu<KIND, D, 4>(batch);
    case 2: return queue_wgs_per_cu<KIND, D, 2>(batch);
    default: return queue_wgs_per_cu<KIND, D, 1>(batch);
  }
}

template <int KIND, int D, int GW>
static int partition_wgs_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<KIND, D, GW>, 256, 0) != hipSuccess) return 1;
  return n > 0 ? n : 1;
}

template <int KIND, int D>
static int partition_wgs_gw(int gw) {
  switch (gw) {
    case 8: return partition_wgs_per_cu<KIND, D, 8>();
    case 4: return partition_wgs_per_cu<KIND, D, 4>();
    case 2: return partition_wgs_per_cu<KIND, D, 2>();
    default: return partition_wgs_per_cu<KIND, D, 1>();
  }
}

int decode_partition_wgs_per_cu(int kv_kind, int d, int heads_per_wg) {
  if (kv_kind == KIND_F32)
    return d == 64 ? partition_wgs_gw<KIND_F32, 64>(heads_per_wg) : partition_wgs_gw<KIND_F32, 128>(heads_per_wg);
  if (kv_kind == KIND_BF16)
    return d == 64 ? partition_wgs_gw<KIND_BF16, 64>(heads_per_wg) : partition_wgs_gw<KIND_BF16, 128>(heads_per_wg);
  return d == 64 ? partition_wgs_gw<KIND_FP8, 64>(heads_per_wg) : partition_wgs_gw<KIND_FP8, 128>(heads_per_wg);
}

int decode_queue_lds_bytes(int batch) { return ((batch + 1) * 4 + 255) / 256 * 256; }
int decode_queue_items_per_wg() { return kItemsPerWg; }
int decode_queue_max_item_blocks() { return kSegBlocks; }

int decode_queue_wgs_per_cu(int kv_kind, int d, int heads_per_wg, int batch) {
  if (kv_kind == KIND_F32)
    return d == 64 ? queue_wgs_gw<KIND_F32, 64>(heads_per_wg, batch)
                   : queue_wgs_gw<KIND_F32, 128>(heads_per_wg, batch);
  if (kv_kind == KIND_BF16)
    return d == 64 ? queue_wgs_gw<KIND_BF16, 64>(heads_per_wg, batch)
                   : queue_wgs_gw<KIND_BF16, 128>(heads_per_wg, batch);
  return d == 64 ? queue_wgs_gw<KIND_FP8, 64>(heads_per_wg, batch)
                 : queue_wgs_gw<KIND_FP8, 128>(heads_per_wg, batch);
}

template <int KIND, int D, int GW>
static hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  if (a.n_wg > 0) {
    hipLaunchKernelGGL((decode_queue_kernel<KIND, D, GW>), dim3(a.n_wg), dim3(256),
                       decode_queue_lds_bytes(a.batch), stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t pairs = (int64_t)a.batch * a.n_kv * a.head_chunks;
    const int hpw = GW / a.merge_splits;
    hipLaunchKernelGGL((combine_queue_kernel<D, GW>), dim3((unsigned)pairs, (unsigned)a.merge_splits), dim3(256), 0,
                       stream, a, hpw);
    return hipGetLastError();
  }
  const int64_t wgs = (int64_t)a.n_parts * a.n_kv * a.head_chunks * a.batch;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e;
  if (a.use_mfma) {
    e = launch_decode_mfma(a, KIND, stream);
  } else {
    hipLaunchKernelGGL((decode_kernel<KIND, D, GW>), dim3((unsigned)wgs), dim3(256), 0, stream, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess || a.n_parts == 1) return e;
  const int heads = a.n_q < kCombineHeads ? a.n_q : kCombineHeads;
  hipLaunchKernelGGL((combine_kernel<D>), dim3((a.n_q + heads - 1) / heads, a.batch), dim3(kWave * heads), 0, stream,
                     a);
  return hipGetLastError();
}

template <int KIND, int D>
static hipError_t launch_gw(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group / a.head_chunks) {
    case 8: return launch_one<KIND, D, 8>(a, stream);
    case 4: return launch_one<KIND, D, 4>(a, stream);
    case 2: return launch_one<KIND, D, 2>(a, stream);
    default: return launch_one<KIND, D, 1>(a, stream);
  }
}

hipError_t launch_decode(const DecodeArgs& a, int kv_kind, int d, hipStream_t stream) {
  if (kv_kind == KIND_F32) return d == 64 ? launch_gw<KIND_F32, 64>(a, stream) : launch_gw<KIND_F32, 128>(a, stream);
  if (kv_kind == KIND_BF16) return d == 64 ? launch_gw<KIND_BF16, 64>(a, stream) : launch_gw<KIND_BF16, 128>(a, stream);
  return d == 64 ? launch_gw<KIND_FP8, 64>(a, stream) : launch_gw<KIND_FP8, 128>(a, stream);
}

// Work order of a batch: thread t ranks sequence t by length against every
// other (longer first, ties by index; the loads of the whole length array are
// shared by the wave), then writes t into the slot of its rank.
__global__ __launch_bounds__(256) void decode_order_kernel(const int32_t* __restrict__ seq_lens, int32_t batch,
                                                           int32_t pair, int32_t* __restrict__ order) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= batch) return;
  const int lt = max(seq_lens[t], 0);
  int r = 0;
#pragma unroll 8
  for (int u = 0; u < batch; ++u) {
    const int lu = max(seq_lens[u], 0);
    r += (lu > lt) | ((lu == lt) & (u < t));
  }
  const int half = (batch + 1) / 2;
  const int slot = (!pair || r < half) ? r : half + (batch - 1 - r);
  order[slot] = t;
}

// Unit order of a split decode: thread t ranks unit t = (sequence t / n_parts,
// partition t % n_parts) by its token count against every other unit (more
// tokens first, ties by index) and writes t into the slot of its rank, or -1
// when the unit has no tokens (those rank last).
__global__ __launch_bounds__(256) void decode_unit_order_kernel(const int32_t* __restrict__ seq_lens, int32_t batch,
                                                                int32_t n_parts, int32_t part_tokens,
                                                                int32_t* __restrict__ order) {
  const int n = batch * n_parts;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  auto tokens = [&](int u) {
    const int L = max(seq_lens[u / n_parts], 0);
    return min(max(L - (u % n_parts) * part_tokens, 0), part_tokens);
  };
  const int lt = tokens(t);
  int r = 0;
#pragma unroll 4
  for (int u = 0; u < n; ++u) {
    const int lu = tokens(u);
    r += (lu > lt) | ((lu == lt) & (u < t));
  }
  order[r] = lt > 0 ? t : -1;
}

hipError_t launch_decode_unit_order(const int32_t* seq_lens, int32_t batch, int32_t n_parts, int32_t part_tokens,
                                    int32_t* order, hipStream_t stream) {
  const int n = batch * n_parts;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_unit_order_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, seq_lens,
                     batch, n_parts, part_tokens, order);
  return hipGetLastError();
}

hipError_t launch_decode_order(const int32_t* seq_lens, int32_t batch, int32_t pair, int32_t* order,
                               hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_order_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, stream, seq_lens, batch,
                     pair, order);
  return hipGetLastError();
}

}  // namespace pkv
