// Chunked prefill over an FP8 (E4M3) paged cache with both matrix products in
// fp8 on the matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, twice the rate
// of the bf16 products): attention's products run in FP8 as in
// FlashAttention-3's FP8 path ("KV cache, PagedAttention and FlashAttention",
// Problem 5), over the quantised cache of "Memory Management in LLM Serving
// Systems" (long context: FP8 KV).  The cache's K and V codes enter the
// products as stored; the queries and the softmax weights are brought to
// E4M3 here.
//
//   S = (q / qs) K_codes^T * qs * ks * scale    qs = max|q row| / 448 per query
//        row, ks the K scale of each key's (block, KV head); one 16 x 16 x 128
//        product per 16 keys x 16 rows covers the whole d = 128
//   p = 2^(S log2 e - m)                        online softmax, m a running
//        reference within kSlack of the row max, so p <= 2^kSlack
//   w = e4m3(p * vs * c)                        vs the V scale of the key's
//        block, c = 440 / (2^kSlack max vs) one factor for the workgroup, so
//        every weight fits E4M3 and all keys of a tile share one product
//   O = sum_k w_k V_codes_k / sum_k w_k / vs_k
// The denominator adds exactly the quantised weights the numerator uses (each
// over its V scale; c cancels), so a row is a convex combination of the
// dequantised V rows and one visible key gives its V row exactly.  Keys whose
// block has a V scale too small for its weights to keep precision
// (vs c < 2^-3, zero included) enter the denominator with p c instead: their
// V rows are near zero, and their weight must still count.
//
// Precision.  One E4M3 rounding moves a value by up to 2^-4 of itself, and a
// row's output by about that fraction of its size, whatever its length.  With
// SPLIT, q / qs and w are each carried as two E4M3 terms, the nearest value
// and the nearest value to the remainder (exact in fp32), leaving about 2^-8:
// every product is issued twice (hi, then lo into the same accumulator).
//
// Layout.  A workgroup of 4 waves owns 128 packed query rows (32 per wave, two
// 16-row tiles) of one sequence and one KV head; 128-key tiles pass through two
// LDS stages (16 KiB of K codes, 16 KiB of V codes), each wave bringing 32 keys
// (four 8-key halves, each inside one cache block) straight into LDS.  A row of
// 128 bytes is eight 16-byte pieces, piece p of row r in slot p ^ f(r).
//   Scores: the A operand of 16-key tile t = 2 b + o takes row 4 q + j from key
//   32 b + 8 q + j + 4 o, so lane (n, g) of the two results of block b holds
//   keys 32 b + 8 g .. + 7 of query row n.
//   Values: O^T += V^T W^T with k-slot 32 g + 8 b + e <-> key 32 b + 8 g + e,
//   so the weights are B operands as they lie in the lanes, and each lane's
//   eight V^T bytes per block come from one ds_read_b64_tr_b8 (lane L of a
//   16-lane group receives byte L of the eight 16-byte rows its lane pairs
//   read).
//   Denominator: one more product per row tile, A the 0/1 matrix selecting the
//   eight k-slots of group 4 g + b, gives each lane the sums of its own four
//   groups' weights.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr int D = 128;
constexpr int KT = 128;               // keys per tile
constexpr int ROWB = D;               // bytes of one fp8 K or V row
constexpr int TILE_B = KT * ROWB;     // 16 KiB
constexpr int STAGE_B = 2 * TILE_B;   // K codes, then V codes
constexpr int ROWS = 128;             // packed query rows per workgroup
constexpr int NT = 2;                 // 16-row tiles per wave
constexpr int kXcds = 8;
constexpr int kMaxSortSeqs = 256;
constexpr float kSlack = 2.f;         // log2 units
constexpr float kWeightTop = 440.f;   // largest weight before exp2's rounding (E4M3 tops out at 448)
constexpr float kWeakBlock = 0.125f;  // vs c below this: denominator takes p c
constexpr uint32_t kOneE4m3x4 = 0x38383838u;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// Slot permutation of a 128-byte row.  The score reads take one piece of the
// 16 rows {0..3, 8..11, 16..19, 24..27} + 4 o of a 32-key block, the value
// reads one piece of 16 consecutive aligned rows; rows of one parity share a
// bank half, so f must be one-to-one over the eight even (and the eight odd)
// rows of either set: f = (r1, r3, r2 ^ r4) is, for each.
__device__ __forceinline__ int slot_f(int r) {
  return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | ((((r >> 2) ^ (r >> 4)) & 1) << 2);
}
__device__ __forceinline__ int piece_at(int row, int piece) { return row * ROWB + ((piece ^ slot_f(row)) << 4); }

__device__ __forceinline__ v2i ds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(__attribute__((address_space(3))) char*)(p));
}

// D (16x16 fp32) += A (16x128 E4M3) B (128x16 E4M3): lane (n, g) supplies
// A[n][32 g .. + 31] and B[32 g .. + 31][n] and holds D[4 g .. + 3][n]
__device__ __forceinline__ f32x4 mfma_fp8(v8i a, v8i b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// four floats -> four E4M3 codes (bytes 0..3), round to nearest even; the
// inputs lie within +-448
__device__ __forceinline__ uint32_t pack_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
// bytes 0-1 (hi = false) or 2-3 (hi = true) of four E4M3 codes -> two floats (exact)
__device__ __forceinline__ f32x2v unpack_e4m3(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true) : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
}

// x ~ hi + lo as two E4M3 words of four codes: hi the nearest codes, lo the
// nearest codes to the remainder (exact in fp32); |x| <= 448
template <bool SPLIT>
__device__ __forceinline__ void split_e4m3(const float x[4], uint32_t& hi, uint32_t& lo) {
  hi = pack_e4m3(x[0], x[1], x[2], x[3]);
  if constexpr (SPLIT) {
    const f32x2v a = unpack_e4m3(hi, false), b = unpack_e4m3(hi, true);
    lo = pack_e4m3(x[0] - a[0], x[1] - a[1], x[2] - b[0], x[3] - b[1]);
  } else {
    lo = 0u;
  }
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ __forceinline__ void no_if_conversion() { asm volatile("" ::: "memory"); }

}  // namespace

template <bool SPLIT>
__global__ __launch_bounds__(256, 2) void prefill_fp8_kernel(PrefillArgs a) {
  __shared__ __align__(16) char smem[2 * STAGE_B];
  __shared__ float blk_scale[2][2][KT / 8];  // [stage][K, V][8-key half]
  __shared__ int seq_key[kMaxSortSeqs], seq_at_rank[kMaxSortSeqs];
  __shared__ float red[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group;
  const int tq = ROWS / G;

  // Work order as in the bf16 kernel: sequences longest first, later query
  // tiles first, the query tiles of one (sequence, KV head) on one XCD.
  const bool sorted = a.num_seqs <= kMaxSortSeqs;
  if (sorted) {
    if (tid < a.num_seqs) {
      const int cs = min(max(a.ctx_lens[tid], 0), page_row(a, tid).n << a.log2_bs);
      const int qb = min(max(a.cu_q[tid], 0), a.total_q), qe = min(max(a.cu_q[tid + 1], qb), a.total_q);
      seq_key[tid] = cs + (qe - qb);
    }
    __syncthreads();
    if (tid < a.num_seqs) {
      const int k = seq_key[tid];
      int rank = 0;
      for (int u = 0; u < a.num_seqs; ++u) {
        const int ku = seq_key[u];
        rank += (ku > k) || (ku == k && u < tid);
      }
      seq_at_rank[rank] = tid;
    }
    __syncthreads();
  }
  const int q_tiles = (a.max_q_len + tq - 1) / tq;
  const int n_pairs = a.n_kv * a.num_seqs;
  int qt, pair;
  if (n_pairs % kXcds == 0) {
    const int jb = blockIdx.x / kXcds;
    qt = jb % q_tiles;
    pair = (jb / q_tiles) * kXcds + blockIdx.x % kXcds;
  } else {
    qt = blockIdx.x % q_tiles;
    pair = blockIdx.x / q_tiles;
  }
  qt = q_tiles - 1 - qt;
  const int kvh = pair % a.n_kv;
  const int s = __builtin_amdgcn_readfirstlane(sorted ? seq_at_rank[pair / a.n_kv] : pair / a.n_kv);
  const int q0 = qt * tq;
  const int qs0 = min(max(a.cu_q[s], 0), a.total_q);
  const int q_len = min(a.cu_q[s + 1], a.total_q) - qs0;
  if (q0 >= q_len) return;  // uniform over the workgroup
  const PageRow prow = page_row(a, s);
  const int cap = prow.n << a.log2_bs;
  const int ctx = min(max(a.ctx_lens[s], 0), cap);
  const int total = min(ctx + q_len, cap);
  const int last_q = min(q0 + tq, q_len) - 1;
  const int kv_end = prow.n == 0 ? 0 : a.causal ? min(ctx + last_q + 1, total) : total;
  const int n_tiles = (kv_end + KT - 1) / KT;
  const int diag_w = ctx + q0 + (32 * w) / G;  // keys above this are masked for some row of the wave
  const int nb1 = (int)(a.num_blocks - 1);

  // ---- c from the largest V scale of the blocks the workgroup reads
  {
    const int n_blk = (kv_end + (1 << a.log2_bs) - 1) >> a.log2_bs;  // <= prow.n
    float vmax = 0.f;
    for (int j = tid; j < n_blk; j += 256) {
      const int id = min(max(prow.ids[j], 0), nb1);
      vmax = fmaxf(vmax, a.v_scale[(int64_t)id * a.n_kv + kvh]);
    }
    vmax = max_xor32(max_xor16(vmax));
    vmax = group_max<16>(vmax);
    if (lane == 0) red[w] = vmax;
  }
  __syncthreads();
  const float vs_max = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float c_w = vs_max > 0.f ? kWeightTop / (exp2f(kSlack) * vs_max) : 1.f;

  const int nn = lane & 15, g = lane >> 4;

  // ---- queries in E4M3: lane (nn, g) holds row 32 w + 16 nt + nn, d = 32 g ..
  // + 31 (the B operand of the score products), every lane its row's scale
  v8i qb[NT], qb_lo[NT];  // SPLIT: q / qs = qb + qb_lo
  float rsl[NT];  // qs * scale * log2(e)
  int row_tok[NT], row_head[NT], row_lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 32 * w + 16 * nt + nn;
    const int tok = q0 + r / G;
    row_tok[nt] = tok;
    row_head[nt] = kvh * G + r % G;
    row_lim[nt] = a.causal ? min(ctx + tok, total - 1) : total - 1;
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(qs0 + (tok < q_len ? tok : 0)) * a.n_q + row_head[nt]) * D * 2;
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = ld16(qrow + (32 * g + 8 * i) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * i + 2 * e] = bf16_lo(v[e]);
        x[8 * i + 2 * e + 1] = bf16_hi(v[e]);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = max_xor32(max_xor16(amax));
    const float qsc = amax > 0.f ? amax / 448.f : 1.f;
    const float inv = 1.f / qsc;
    rsl[nt] = qsc * a.scale_log2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[4 * i + e] * inv, -448.f), 448.f);
      uint32_t h, l;
      split_e4m3<SPLIT>(y, h, l);
      qb[nt][i] = (int)h;
      qb_lo[nt][i] = (int)l;
    }
  }

  // the 0/1 selector of the denominator product: lane (i, g') supplies row i =
  // group 4 g + b, ones exactly in k-slots 32 g + 8 b .. + 7
  v8i ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (g == (nn >> 2) && (i >> 1) == (nn & 3)) ? (int)kOneE4m3x4 : 0;

  f32x4 o[8][NT];  // O^T[16 dt + 4 g + j][row nn of tile nt]
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

  // ---- tile loads: wave w brings keys 32 w .. 32 w + 31 of the tile, four
  // 8-key halves with one 1-KiB instruction each for K and for V: lane l
  // brings row l / 8 of the half and the global piece stored in slot l % 8.
  // Block ids are fetched one tile ahead of the loads that use them.  Halves
  // past the keys the workgroup sees are not loaded.
  const char* const kc = reinterpret_cast<const char*>(a.k_cache);
  const char* const vc = reinterpret_cast<const char*>(a.v_cache);
  uint32_t src_off[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int row = 32 * w + 8 * h + (lane >> 3);
    src_off[h] = (lane >> 3) * ROWB + (((lane & 7) ^ slot_f(row)) << 4);
  }
  const uint32_t lds_base = lds_addr(smem) + 32 * w * ROWB;
  auto fetch_ids = [&](int t) {
    const int tok = t * KT + 32 * w;
    const int last = prow.n - 1;
    return int4{prow.ids[min(tok >> a.log2_bs, last)], prow.ids[min((tok + 8) >> a.log2_bs, last)],
                prow.ids[min((tok + 16) >> a.log2_bs, last)], prow.ids[min((tok + 24) >> a.log2_bs, last)]};
  };
  // scales of this wave's halves of the tile last issued: a half past the
  // keys takes 1 for both (its keys are masked and its V rows zeroed, and a
  // table entry past the keys may be stale, its scales anything)
  float ks_load[4], vs_load[4];
  auto issue = [&](int t, int4 raw) {
    const int rid[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int tok = t * KT + 32 * w + 8 * h;
      ks_load[h] = vs_load[h] = 1.f;
      if (tok < kv_end) {
        const int id = min(max(__builtin_amdgcn_readfirstlane(rid[h]), 0), nb1);
        const int64_t off = (int64_t)page_row_index(a, id, kvh, tok) * ROWB;
        const uint32_t dst = lds_base + (t & 1) * STAGE_B + 8 * h * ROWB;
        lds_dma16(kc + off, src_off[h], dst);
        lds_dma16(vc + off, src_off[h], dst + TILE_B);
        ks_load[h] = a.k_scale[(int64_t)id * a.n_kv + kvh];
        vs_load[h] = a.v_scale[(int64_t)id * a.n_kv + kvh];
      }
    }
  };
  int4 id_next = int4{0, 0, 0, 0};
  if (n_tiles > 0) {
    issue(0, fetch_ids(0));
    if (n_tiles > 1) id_next = fetch_ids(1);
  }

  for (int t = 0; t < n_tiles; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of tile t have landed
    char* const k_lds = smem + (t & 1) * STAGE_B;
    char* const v_lds = k_lds + TILE_B;
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        blk_scale[t & 1][0][4 * w + h] = ks_load[h];
        blk_scale[t & 1][1][4 * w + h] = vs_load[h];
      }
    }
    if (t * KT + KT > kv_end) {
      // V rows of this wave's part past the keys (not loaded, or loaded past
      // the sequence) may hold anything, NaN included: zero weights must not
      // meet them.  K rows past the keys are masked.
      no_if_conversion();
      const int row = 32 * w + (lane >> 1);
      if (t * KT + row >= kv_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st16(v_lds + row * ROWB + (lane & 1) * 64 + 16 * i, u32x4{0, 0, 0, 0});
      }
    }
    __syncthreads();  // tile t and its scales are in LDS; every wave is done with tile t - 1
    if (t + 1 < n_tiles) {
      issue(t + 1, id_next);
      if (t + 2 < n_tiles) id_next = fetch_ids(t + 2);
    }
    // this lane's blocks b = 0..3: keys 32 b + 8 g .. + 7, half 4 b + g
    float ksc[4], lvc[4], inv_vs[4];
    bool weak = false;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      ksc[b] = blk_scale[t & 1][0][4 * b + g];
      const float vcw = blk_scale[t & 1][1][4 * b + g] * c_w;
      lvc[b] = __builtin_amdgcn_logf(vcw);  // log2; -inf for a zero scale
      const bool wk = !(vcw >= kWeakBlock);
      weak |= wk;
      inv_vs[b] = wk ? 0.f : c_w / vcw;  // 1 / vs
    }

    // ---- S^T: eight 16-key tiles x two row tiles, one product each.  A wave
    // in a product phase is preferred at issue over one in its softmax (value
    // products most), so the matrix core keeps its queue while the other
    // wave on the SIMD quantises weights in the slots between (measured 3-5 %
    // faster than equal priorities)
    __builtin_amdgcn_s_setprio(1);
    f32x4 sc[8][NT];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int key = 32 * (tt >> 1) + 8 * (nn >> 2) + (nn & 3) + 4 * (tt & 1);
      const u32x4 lo = ld16(k_lds + piece_at(key, 2 * g));
      const u32x4 hi = ld16(k_lds + piece_at(key, 2 * g + 1));
      const v8i ka = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                         (int)hi[3]};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        sc[tt][nt] = mfma_fp8(ka, qb[nt], f32x4{0.f, 0.f, 0.f, 0.f});
        if constexpr (SPLIT) sc[tt][nt] = mfma_fp8(ka, qb_lo[nt], sc[tt][nt]);
      }
    }

    // ---- mask, online softmax, quantised weights
    __builtin_amdgcn_s_setprio(0);
    const int kb = t * KT;
    if ((a.causal && kb + KT - 1 > diag_w) || (kb + KT > total)) {
      no_if_conversion();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = kb + 32 * (tt >> 1) + 8 * g + 4 * (tt & 1) + e;
            sc[tt][nt][e] = (key <= row_lim[nt]) ? sc[tt][nt][e] : -INFINITY;
          }
    }
    v8i wb[NT], wb_lo[NT];  // B operands of the value product: byte 8 b + e <-> k-slot 32 g + 8 b + e
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // raw scores -> log2 units with f = qs * ks * scale * log2 e per block;
      // f is kept positive so a masked -inf stays -inf
      float f[4], mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f[b] = fmaxf(rsl[nt] * ksc[b], 1.17549435e-38f);
        const f32x4 u = sc[2 * b][nt], v = sc[2 * b + 1][nt];
        const float mb = fmaxf(max3(u[0], u[1], u[2]), max3(u[3], v[0], fmaxf(v[1], fmaxf(v[2], v[3]))));
        mx = fmaxf(mx, mb * f[b]);
      }
      mx = max_xor32(max_xor16(mx));
      const float m_new = (mx > m_run[nt] + kSlack) ? mx : m_run[nt];  // m_run = -inf takes mx
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run[nt] - m_use);
      m_run[nt] = m_new;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float off = lvc[b] - m_use;
        float p[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = exp2_fast(fmaf(sc[2 * b][nt][e], f[b], off));
          p[4 + e] = exp2_fast(fmaf(sc[2 * b + 1][nt][e], f[b], off));
        }
        uint32_t h0, l0, h1, l1;
        split_e4m3<SPLIT>(p, h0, l0);
        split_e4m3<SPLIT>(p + 4, h1, l1);
        wb[nt][2 * b] = (int)h0;
        wb[nt][2 * b + 1] = (int)h1;
        wb_lo[nt][2 * b] = (int)l0;
        wb_lo[nt][2 * b + 1] = (int)l1;
      }
      // denominator: per group the sum of its quantised weights over vs
      f32x4 gsum = mfma_fp8(ones, wb[nt], f32x4{0.f, 0.f, 0.f, 0.f});
      if constexpr (SPLIT) gsum = mfma_fp8(ones, wb_lo[nt], gsum);
      float ls = gsum[0] * inv_vs[0] + gsum[1] * inv_vs[1] + gsum[2] * inv_vs[2] + gsum[3] * inv_vs[3];
      if (__builtin_amdgcn_ballot_w64(weak) != 0) {
        // weak blocks count p c (their weights add nothing above)
        no_if_conversion();
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (inv_vs[b] == 0.f) {
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ps += exp2_fast(fmaf(sc[2 * b][nt][e], f[b], -m_use));
              ps += exp2_fast(fmaf(sc[2 * b + 1][nt][e], f[b], -m_use));
            }
            ls += ps * c_w;
          }
        }
      }
      l_run[nt] = l_run[nt] * alpha + ls;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
        no_if_conversion();
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt][nt] *= alpha;
      }
    }

    __builtin_amdgcn_s_setprio(2);
    // ---- O^T += V^T W^T: per 16-d tile dt, lane (m, g) needs the bytes
    // V[32 b + 8 g + e][16 dt + m], four transposing reads of the eight keys
    // 32 b + 8 g .. + 7 (lane L of the group reads row L / 2, bytes
    // 8 (L % 2) .. + 7 of piece dt)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      v8i va;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const v2i r = ds_read_tr8(v_lds + piece_at(32 * b + 8 * g + (nn >> 1), dt) + 8 * (nn & 1));
        va[2 * b] = r[0];
        va[2 * b + 1] = r[1];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        o[dt][nt] = mfma_fp8(va, wb[nt], o[dt][nt]);
        if constexpr (SPLIT) o[dt][nt] = mfma_fp8(va, wb_lo[nt], o[dt][nt]);
      }
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- normalise and store: lane (nn, g) holds d = 16 dt + 4 g + j of its row
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = sum_xor32(sum_xor16(l_run[nt]));
    if (row_tok[nt] >= q_len) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t obase = ((int64_t)(qs0 + row_tok[nt]) * a.n_q + row_head[nt]) * D;
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

hipError_t launch_prefill_fp8_mma(const PrefillArgs& a, bool split, hipStream_t stream) {
  const int tq = ROWS / a.group;
  const int64_t n_work = (int64_t)((a.max_q_len + tq - 1) / tq) * a.n_kv * a.num_seqs;
  if (n_work == 0) return hipSuccess;
  if (n_work > 0x7fffffff) return hipErrorInvalidValue;
  if (split)
    hipLaunchKernelGGL(prefill_fp8_kernel<true>, dim3((unsigned)n_work), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_fp8_kernel<false>, dim3((unsigned)n_work), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
