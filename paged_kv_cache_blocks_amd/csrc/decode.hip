// Paged decode attention for gfx950: split-K over the sequence, FlashAttention
// style online softmax inside each partition, and a partition-combine pass.
//
// Method ("KV cache, PagedAttention and FlashAttention", Problem 5: tiling,
// online softmax with a running max m and sum l rescaled by e^(m - m_new),
// kernel fusion, and the serving note that decode reads K and V once and
// splits a long sequence across thread blocks; "Memory Management in LLM
// Serving Systems", FlashAttention-2: rescale once per block, divide by l at
// the very end, parallelise over the sequence as well as batch and head; GQA:
// the query heads of a group are processed against the same K/V block).
//
// Work decomposition
//   grid = (partitions, KV heads x head chunks, sequences), 256 threads.
//   A workgroup owns one partition of one sequence for GW query heads that
//   share one KV head.  Its 4 waves take the partition's blocks round-robin in
//   chunks of CB blocks and run independent online softmaxes; the 4 states are
//   merged once at the end through LDS.
//   Per chunk a wave:
//     1. reads the chunk's K and V slabs from HBM with coalesced 16-byte loads
//        (issued one chunk ahead; block ids come from the table once per wave)
//     2. stages K into LDS as bf16 rows (fp8 converted here, once per element)
//        and V as bf16 token *pairs* interleaved per column, so the value
//        product runs on v_dot2c_f32_bf16;
//     3. scores: lane (head h, token t) holds q[h] in registers and reads the
//        whole K row from LDS -- every K element is fetched from HBM once and
//        serves all GW heads of the group;
//     4. online softmax over the chunk with DPP lane-group reductions;
//        weights go to LDS as bf16 pairs;
//     5. values: lane c owns output columns (2c, 2c+1) for all GW heads and
//        accumulates dot2(p pair, v pair) in f32.
//   f32 caches take the same path with f32 rows and fma in place of dot2.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kBlock = 16;  // tokens per cache block
constexpr int kWaves = 4;   // waves per workgroup

constexpr int align16(int x) { return (x + 15) & ~15; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int KIND, int D>
struct Geo {
  static constexpr int esize = KindBytes<KIND>::v;
  static constexpr int row_bytes = D * esize;           // one token row of one KV head in HBM
  static constexpr int slab_bytes = kBlock * row_bytes;  // one (block, KV head) slab
  static constexpr int LW = row_bytes >= 128 ? 16 : 8;   // bytes per lane per load
  static constexpr int LPR = row_bytes / LW;             // lanes per row
  static constexpr int RPI = kWave / LPR;                // rows per load instruction
  static constexpr int NLK = kBlock / RPI;               // load instructions per slab
  static constexpr int EPL = LW / esize;                 // elements per lane per load
  static_assert(LPR <= kWave && NLK >= 2 && NLK % 2 == 0, "slab geometry");
};

template <int LW> struct LoadVec;
template <> struct LoadVec<16> { typedef u32x4 T; };
template <> struct LoadVec<8> { typedef u32x2 T; };

template <int KIND, int D, int GW>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  using Gm = Geo<KIND, D>;
  using LV = typename LoadVec<Gm::LW>::T;
  constexpr bool F32P = (KIND == KIND_F32);
  constexpr int T = kWave / GW;                      // token slots per head group (score layout)
  constexpr int CB = T > kBlock ? T / kBlock : 1;    // blocks per chunk
  constexpr int R = T < kBlock ? kBlock / T : 1;     // score rounds per chunk
  constexpr int CT = CB * kBlock;                    // tokens per chunk
  constexpr int ES = F32P ? 4 : 2;                   // bytes per element in LDS
  constexpr int KROW = D * ES + 16;                  // padded K row in LDS
  constexpr int VROW = D * 4 + 16;                   // f32 V row, or one bf16-pair row
  constexpr int NPAIR = kBlock / 2;                  // token pairs per block
  constexpr int K_BYTES = CT * KROW;
  constexpr int V_BYTES = F32P ? CT * VROW : CB * NPAIR * VROW;
  constexpr int P_BYTES = F32P ? CT * GW * 4 : CB * NPAIR * GW * 4;
  constexpr int A_BYTES = align16(GW * 4);
  constexpr int WAVE_BYTES = align16(K_BYTES + V_BYTES + P_BYTES + A_BYTES);
  constexpr int MERGE_BYTES = kWaves * GW * D * 4 + kWaves * GW * 2 * 4;
  constexpr int SMEM = cmax(kWaves * WAVE_BYTES, MERGE_BYTES);
  // value-product layout: columns per lane and lane groups per pair row
  constexpr int PVL = F32P ? kWave : D / 2;          // lanes covering one row
  constexpr int PVG = kWave / PVL;                   // row groups (bf16 path, d = 64)
  constexpr int COLS = F32P ? D / kWave : 2;         // output columns per lane
  static_assert(COLS >= 1 && PVG >= 1, "value layout");

  __shared__ __align__(16) char smem[SMEM];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const int part = blockIdx.x;
  const int s = blockIdx.z;
  const int kvh = blockIdx.y / a.head_chunks;
  const int h0 = kvh * a.group + (blockIdx.y % a.head_chunks) * GW;

  int L = a.seq_lens[s];
  L = min(max(L, 0), a.max_blocks * kBlock);
  const int p0 = part * a.part_tokens;
  if (a.n_parts > 1 && p0 >= L) return;
  const int plen = max(0, min(a.part_tokens, L - p0));
  const int nb_part = (plen + kBlock - 1) / kBlock;
  const int n_chunks = (nb_part + CB - 1) / CB;
  const int n_my = n_chunks > w ? (n_chunks - w + kWaves - 1) / kWaves : 0;

  // this wave's block ids, one per lane: lane i <-> block (i % CB) of the
  // wave's chunk i / CB (= partition chunk w + 4 * (i / CB))
  int my_id = 0;
  {
    const int pb = (w + kWaves * (lane / CB)) * CB + lane % CB;
    if (pb < nb_part) {
      const int id = a.block_table[(int64_t)s * a.max_blocks + p0 / kBlock + pb];
      my_id = min(max(id, 0), (int)(a.num_blocks - 1));
    }
  }

  char* const wbase = smem + w * WAVE_BYTES;
  char* const k_lds = wbase;
  char* const v_lds = wbase + K_BYTES;
  char* const p_lds = v_lds + V_BYTES;
  float* const a_lds = reinterpret_cast<float*>(p_lds + P_BYTES);

  // score layout: lane = sh * T + st  (head sh of the group, token slot st)
  const int sh = lane / T;
  const int st = lane % T;

  // q row of head h0 + sh, kept in registers for the whole partition
  constexpr int QV = F32P ? D / 4 : D / 8;
  u32x4 qv[QV];
  {
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)s * a.n_q + h0 + sh) * D * (F32P ? 4 : 2);
#pragma unroll
    for (int j = 0; j < QV; ++j) qv[j] = ld16(qrow + j * 16);
  }

  float m_run = -INFINITY;  // running max of this lane's head (log2 units)
  float l_run = 0.f;        // this lane's share of the running sum
  float o[GW][COLS];
#pragma unroll
  for (int h = 0; h < GW; ++h)
#pragma unroll
    for (int k = 0; k < COLS; ++k) o[h][k] = 0.f;

  const char* const kc = reinterpret_cast<const char*>(a.k_cache);
  const char* const vc = reinterpret_cast<const char*>(a.v_cache);
  LV kreg[CB][Gm::NLK], vreg[CB][Gm::NLK];

  auto issue_loads = [&](int c) {
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      const int id = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(my_id, c * CB + b));
      const int64_t slab = ((int64_t)id * a.n_kv + kvh) * Gm::slab_bytes;
#pragma unroll
      for (int i = 0; i < Gm::NLK; ++i) {
        const int64_t off = slab + (int64_t)(i * kWave + lane) * Gm::LW;
        kreg[b][i] = *reinterpret_cast<const LV*>(kc + off);
        vreg[b][i] = *reinterpret_cast<const LV*>(vc + off);
      }
    }
  };

  if (n_my > 0) issue_loads(0);

  for (int c = 0; c < n_my; ++c) {
    const int ct0 = (w + kWaves * c) * CT;  // first token of the chunk (partition-relative)
    const int nvalid = plen - ct0;         // tokens of the chunk that exist (may exceed CT)
    float kscale[CB], vscale[CB];
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      kscale[b] = vscale[b] = 1.f;
      if constexpr (KIND == KIND_FP8) {
        const int id = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(my_id, c * CB + b));
        kscale[b] = a.k_scale[(int64_t)id * a.n_kv + kvh];
        vscale[b] = a.v_scale[(int64_t)id * a.n_kv + kvh];
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
          __builtin_memcpy(wv, &kreg[b][i], Gm::LW);
          uint32_t bw[2 * NW];
#pragma unroll
          for (int e = 0; e < NW; ++e) fp8x4_to_bf16x4(wv[e], bw[2 * e], bw[2 * e + 1]);
#pragma unroll
          for (int e = 0; e < NW / 2; ++e) st16(dst + e * 16, u32x4{bw[4 * e], bw[4 * e + 1], bw[4 * e + 2], bw[4 * e + 3]});
        } else {
          st16(dst, kreg[b][i]);
        }
      }
      const bool tail = nvalid < (b + 1) * kBlock;  // some rows of this block are past the end
      if constexpr (F32P) {
#pragma unroll
        for (int i = 0; i < Gm::NLK; ++i) {
          const int r = lane / Gm::LPR + Gm::RPI * i;
          const int c0 = (lane % Gm::LPR) * Gm::EPL;
          u32x4 v = vreg[b][i];
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
            __builtin_memcpy(wa, &vreg[b][i], Gm::LW);
            __builtin_memcpy(wb, &vreg[b][i + 1], Gm::LW);
#pragma unroll
            for (int e = 0; e < NW; ++e) {
              fp8x4_to_bf16x4(wa[e], A[2 * e], A[2 * e + 1]);
              fp8x4_to_bf16x4(wb[e], Bv[2 * e], Bv[2 * e + 1]);
            }
          } else {
            __builtin_memcpy(A, &vreg[b][i], Gm::LW);
            __builtin_memcpy(Bv, &vreg[b][i + 1], Gm::LW);
          }
          if (tail) {
            if (b * kBlock + r0 >= nvalid) {
#pragma unroll
              for (int e = 0; e < NB; ++e) A[e] = 0;
            }
            if (b * kBlock + r1 >= nvalid) {
#pragma unroll
              for (int e = 0; e < NB; ++e) Bv[e] = 0;
            }
          }
          uint32_t pr[2 * NB];
#pragma unroll
          for (int e = 0; e < NB; ++e) {
            pr[2 * e] = pair_lo(A[e], Bv[e]);
            pr[2 * e + 1] = pair_hi(A[e], Bv[e]);
          }
          char* dst = v_lds + (b * NPAIR + pq) * VROW + c0 * 4;
#pragma unroll
          for (int e = 0; e < NB / 2; ++e) st16(dst + e * 16, u32x4{pr[4 * e], pr[4 * e + 1], pr[4 * e + 2], pr[4 * e + 3]});
        }
      }
    }
    // the registers are free again: fetch the next chunk while this one computes
    if (c + 1 < n_my) issue_loads(c + 1);
    wave_lds_sync();

    // ---- scores and online softmax ----
    float sc[R];
    float cmax_ = -INFINITY;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int tau = r * T + st;  // token within the chunk
      const char* krow = k_lds + tau * KROW;
      float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
      if constexpr (F32P) {
#pragma unroll
        for (int j = 0; j < QV; ++j) {
          const u32x4 kp = ld16(krow + j * 16);
          acc0 = fmaf(__uint_as_float(qv[j][0]), __uint_as_float(kp[0]), acc0);
          acc1 = fmaf(__uint_as_float(qv[j][1]), __uint_as_float(kp[1]), acc1);
          acc2 = fmaf(__uint_as_float(qv[j][2]), __uint_as_float(kp[2]), acc2);
          acc3 = fmaf(__uint_as_float(qv[j][3]), __uint_as_float(kp[3]), acc3);
        }
      } else {
#pragma unroll
        for (int j = 0; j < QV; ++j) {
          const u32x4 kp = ld16(krow + j * 16);
          acc0 = dot2_bf16(qv[j][0], kp[0], acc0);
          acc1 = dot2_bf16(qv[j][1], kp[1], acc1);
          acc2 = dot2_bf16(qv[j][2], kp[2], acc2);
          acc3 = dot2_bf16(qv[j][3], kp[3], acc3);
        }
      }
      float ksc = kscale[0];
      if constexpr (CB > 1) {
#pragma unroll
        for (int b = 1; b < CB; ++b) ksc = (tau / kBlock == b) ? kscale[b] : ksc;
      }
      const float sv = ((acc0 + acc1) + (acc2 + acc3)) * (a.scale_log2 * ksc);
      sc[r] = (tau < nvalid) ? sv : -INFINITY;
      cmax_ = fmaxf(cmax_, sc[r]);
    }
    cmax_ = group_max<T>(cmax_);
    const float m_new = fmaxf(m_run, cmax_);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int tau = r * T + st;
      float p = exp2_fast(sc[r] - m_use);
      if constexpr (F32P) {
        reinterpret_cast<float*>(p_lds)[tau * GW + sh] = p;
      } else {
        p = round_bf16(p);
        const int b = tau / kBlock, t = tau % kBlock;
        const int i = t / Gm::RPI, g = t % Gm::RPI;
        const int pq = g + Gm::RPI * (i / 2);
        reinterpret_cast<__bf16*>(p_lds)[((b * NPAIR + pq) * GW + sh) * 2 + (i & 1)] = (__bf16)p;
      }
      lsum += p;
    }
    l_run = l_run * alpha + lsum;
    if (st == 0) a_lds[sh] = alpha;
    wave_lds_sync();

    // ---- rescale and accumulate P V ----
    float al[GW];
#pragma unroll
    for (int h = 0; h < GW; ++h) al[h] = a_lds[h];
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
      for (int k = 0; k < COLS; ++k) o[h][k] *= al[h];

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
          for (int k = 0; k < COLS; ++k) o[h][k] = fmaf(pp[h], vv[k], o[h][k]);
      }
    } else {
      const int pg = lane / PVL;
      const int dcol = (lane % PVL) * 2;
#pragma unroll
      for (int b = 0; b < CB; ++b) {
        float t[GW][2];
#pragma unroll
        for (int h = 0; h < GW; ++h) t[h][0] = t[h][1] = 0.f;
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
          o[h][0] = fmaf(vscale[b], t[h][0], o[h][0]);
          o[h][1] = fmaf(vscale[b], t[h][1], o[h][1]);
        }
      }
    }
  }

  // ---- merge the four waves' states ----
  const float l_head = group_sum<T>(l_run);
  if constexpr (!F32P && PVG > 1) {
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
      for (int k = 0; k < COLS; ++k) o[h][k] += __shfl_xor(o[h][k], 32);
  }
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);  // [wave][head][d]
  float* mml = mo + kWaves * GW * D;            // [wave][head][2]
  if (st == 0) {
    mml[(w * GW + sh) * 2 + 0] = m_run;
    mml[(w * GW + sh) * 2 + 1] = l_head;
  }
  if (lane < PVL) {
    const int col = F32P ? lane * COLS : (lane % PVL) * 2;
#pragma unroll
    for (int h = 0; h < GW; ++h)
#pragma unroll
      for (int k = 0; k < COLS; ++k) mo[(w * GW + h) * D + col + k] = o[h][k];
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
    const int hq = h0 + h;
    if (a.n_parts == 1) {
      const float val = lsum > 0.f ? osum / lsum : 0.f;
      const int64_t oi = ((int64_t)s * a.n_q + hq) * D + col;
      if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[oi] = (__bf16)val;
      else reinterpret_cast<float*>(a.out)[oi] = val;
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

// Merge the partitions of one (sequence, query head): the rescale rule of the
// online softmax applied to whole partitions.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs a) {
  constexpr int COLS = D / kWave;
  const int hq = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  int L = a.seq_lens[s];
  L = min(max(L, 0), a.max_blocks * kBlock);
  const int nv = (L + a.part_tokens - 1) / a.part_tokens;
  const int64_t base = ((int64_t)s * a.n_q + hq) * a.n_parts;
  const float* ml = a.ws_ml + base * 2;
  const float* op = a.ws_o + base * D;
  float M = -INFINITY;
  for (int j = 0; j < nv; ++j) M = fmaxf(M, ml[2 * j]);
  float den = 0.f, num[COLS];
#pragma unroll
  for (int k = 0; k < COLS; ++k) num[k] = 0.f;
  if (M != -INFINITY) {
    for (int j = 0; j < nv; ++j) {
      const float m = ml[2 * j];
      if (m == -INFINITY) continue;
      const float e = exp2_fast(m - M);
      den = fmaf(e, ml[2 * j + 1], den);
#pragma unroll
      for (int k = 0; k < COLS; ++k) num[k] = fmaf(e, op[(int64_t)j * D + lane + k * kWave], num[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < COLS; ++k) {
    const float val = den > 0.f ? num[k] / den : 0.f;
    const int64_t oi = ((int64_t)s * a.n_q + hq) * D + lane + k * kWave;
    if (a.out_bf16) reinterpret_cast<__bf16*>(a.out)[oi] = (__bf16)val;
    else reinterpret_cast<float*>(a.out)[oi] = val;
  }
}

int decode_heads_per_wg(int group) {
  for (int g : {8, 4, 2, 1})
    if (group % g == 0) return g;
  return 1;
}

int decode_chunk_blocks(int heads_per_wg) {
  const int t = kWave / heads_per_wg;
  return t > kBlock ? t / kBlock : 1;
}

template <int KIND, int D, int GW>
static hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_parts, a.n_kv * a.head_chunks, a.batch);
  hipLaunchKernelGGL((decode_kernel<KIND, D, GW>), grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_parts == 1) return e;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(a.n_q, a.batch), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int KIND, int D>
static hipError_t launch_gw(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group / a.head_chunks) {
    case 8: return launch_one<KIND, D, 8>(a, stream);
    case 4: return launch_one<KIND, D, 4>(a, stream);
    case 2: return launch_one<KIND, D, 2>(a, stream);
    default:
      // one query head per KV head with f32 rows of 128 would need more LDS than a CU has
      if constexpr (KIND == KIND_F32 && D == 128) return hipErrorInvalidValue;
      else return launch_one<KIND, D, 1>(a, stream);
  }
}

bool decode_supported(int kv_kind, int d, int heads_per_wg) {
  return !(kv_kind == KIND_F32 && d == 128 && heads_per_wg == 1);
}

hipError_t launch_decode(const DecodeArgs& a, int kv_kind, int d, hipStream_t stream) {
  if (kv_kind == KIND_F32) return d == 64 ? launch_gw<KIND_F32, 64>(a, stream) : launch_gw<KIND_F32, 128>(a, stream);
  if (kv_kind == KIND_BF16) return d == 64 ? launch_gw<KIND_BF16, 64>(a, stream) : launch_gw<KIND_BF16, 128>(a, stream);
  return d == 64 ? launch_gw<KIND_FP8, 64>(a, stream) : launch_gw<KIND_FP8, 128>(a, stream);
}

}  // namespace pkv
