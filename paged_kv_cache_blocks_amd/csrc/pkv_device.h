// Device helpers for the gfx950 (CDNA4) paged-attention kernels: 16-byte
// vector types, bf16 / OCP-E4M3FN conversions, and wave64 lane-group
// reductions built from DPP row operations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// cache element kinds (mirror the C-ABI dtype codes)
enum Kind : int { KIND_F32 = 0, KIND_BF16 = 1, KIND_FP8 = 2 };

template <int K> struct KindBytes;
template <> struct KindBytes<KIND_F32> { static constexpr int v = 4; };
template <> struct KindBytes<KIND_BF16> { static constexpr int v = 2; };
template <> struct KindBytes<KIND_FP8> { static constexpr int v = 1; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// low / high bf16 of a packed dword, widened to f32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// f32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// bf16 rounding of one value, returned widened to f32
__device__ __forceinline__ float round_bf16(float x) { return __bf16(x); }

// interleave the low halves / high halves of two packed bf16 dwords:
// lo_pair = (a.lo, b.lo), hi_pair = (a.hi, b.hi)
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// dot of two bf16 pairs accumulated in f32 (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// four OCP E4M3FN bytes -> two packed bf16 dwords (exact: every E4M3FN value
// is a bf16 value).  gfx950 converts the OCP encoding in hardware.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  // v_cvt_scalef32_pk_bf16_fp8 with scale 1: every E4M3 value is a bf16 value,
  // so the conversion is exact (NaN stays NaN)
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// --- lane-group reductions over G consecutive lanes (G a power of two) ---
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int G>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (G >= 2) x = fmaxf(x, dpp_f<DPP_QUAD_XOR1>(x));
  if constexpr (G >= 4) x = fmaxf(x, dpp_f<DPP_QUAD_XOR2>(x));
  if constexpr (G >= 8) x = fmaxf(x, dpp_f<DPP_ROW_HALF_MIRROR>(x));
  if constexpr (G >= 16) x = fmaxf(x, dpp_f<DPP_ROW_MIRROR>(x));
  if constexpr (G >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (G >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp_f<DPP_QUAD_XOR1>(x);
  if constexpr (G >= 4) x += dpp_f<DPP_QUAD_XOR2>(x);
  if constexpr (G >= 8) x += dpp_f<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (G >= 16) x += dpp_f<DPP_ROW_MIRROR>(x);
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  if constexpr (G >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Exchanges across 16-lane rows without going through LDS: v_permlane16_swap
// and v_permlane32_swap (gfx950 VALU ops) swap rows between two registers.
// Given the same value in both, the two results of a lane are its own value and
// that of lane ^ 16 (resp. lane ^ 32), so max or sum of the pair reduces over
// the partner lanes in every lane.
__device__ __forceinline__ float max_xor16(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order LDS traffic between lanes of one wave: LDS instructions of a wave
// execute in order, so a compiler-level barrier with wavefront-scope fences is
// enough for one lane to read what another lane of the same wave wrote.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave issue priority from the fraction of its own chunks a wave has done:
// 3 below half, 2 below 80%, 1 below 95%, then 0.  Two workgroups share each
// CU and the SIMD arbiter otherwise favours the older wave, so the workgroup
// dispatched first streams faster and finishes early while its neighbour
// still runs, leaving the CU half busy at the end.  With this rule a wave
// that gets ahead drops below its neighbour and the one behind catches up at
// every step, so co-resident workgroups finish together (in proportion to
// their work when it differs).  Only the issue order changes, not what is
// computed.
// s_setprio is a scalar instruction that ignores the exec mask, so the level
// is made wave-uniform first: only scalar branches may choose which one runs.
__device__ __forceinline__ void set_priority_for_progress(int done, int total) {
  const int level = 20 * done < 10 * total ? 3 : 20 * done < 16 * total ? 2 : 20 * done < 19 * total ? 1 : 0;
  switch (__builtin_amdgcn_readfirstlane(level)) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// ---- matrix-core tiles (d = 128, bf16) ----
// LDS layout of a K or V tile: row r (one token) is 256 bytes (all 64 banks),
// its 16 pieces of 16 bytes with piece c stored in slot c ^ f(r % 16), f a
// permutation of 0..15 (linear over GF(2)).  Measured on gfx950 (a lane-pair probe
// under rocprofv3's bank-conflict counter): a 16-byte LDS access serves its 64
// lanes in four passes of 16, pass = (lane >> 5, parity of (lane >> 2) & 7),
// e.g. lanes 0-3, 12-15 and 20-27 together; an 8-byte access (the transposing
// reads included) in two passes of 32 consecutive lanes.  Under that rule the
// patterns to serve are:
//   the score MFMAs' K reads, one piece per 16 lanes of 16 consecutive rows
//   (lane (n, g) reads row n, piece 4 s + g): f must map rows {0..3, 12..15}
//   and {4..11} each onto whole slot pairs {2j, 2j + 1};
//   the transposing V reads, pieces {2j, 2j + 1} of rows 0..7 (and 8..15):
//   f >> 1 one-to-one on each;
//   the prefill's FP8 widening writes (lane l: row l / 4, pieces 4 (l % 4) + i).
// The prefill's direct-to-LDS loads apply the permutation to global addresses
// and are fast only if bit 0 of f is the same for the four rows one load
// instruction brings (a variant without that ran 62 % slower).  The function
// below keeps that, and leaves 2-way conflicts on the K reads (a third of the
// prefill's LDS-active cycles): the conflict-free permutation (r0, r1, r2 ^ r3
// in bits 1, 2, 3 and r2 in bit 0) measured zero conflict cycles and ran 1-3 %
// slower in same-box runs (449.6 and 457.1 us against 444.5 and 444.3 us),
// the prefill not being bound by LDS.  The decode, which stages from
// registers and writes two consecutive fp8 rows per 16 lanes, uses its own
// conflict-free permutation (dswz in decode_mfma.hip).
__device__ __forceinline__ int swz_f(int r) { return ((r & 7) << 1) | (((r >> 2) ^ (r >> 3)) & 1); }
__device__ __forceinline__ int swz(int row, int piece) { return row * 256 + ((piece ^ swz_f(row & 15)) << 4); }

// D (16x16, fp32) += A (16x32, bf16) B (32x16, bf16): lane l supplies
// A[l % 16][8 (l / 16) .. +7] and B[8 (l / 16) .. +7][l % 16] and holds
// D[4 (l / 16) .. +3][l % 16].
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
// ds_read_b64_tr_b16: 8 bytes per lane, transposed across the lanes of a
// 16-lane row group (the A/B fragment of a product over the rows read).
__device__ __forceinline__ u32x2 ds_read_tr(const char* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// 16-byte load marked non-temporal (the nt bit: a streaming access whose
// lines the caches need not keep), for K/V bytes a kernel reads exactly once.
// Measured on MI355X (pkv_read_probe): 512-1024 workgroups reading randomly
// placed 4-16 KiB pieces of a 430 MB region stream at 6.28-6.50 TB/s this way
// against 5.33-5.82 TB/s with ordinary loads.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---- direct global -> LDS loads (prefill kernels) ----
// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (global_load_lds_dwordx4, scalar-base form: address = base + off, with the
// base and the LDS address the same in every lane and the LDS address in M0).
// Issued from inline assembly on purpose: the compiler, unable to tell which
// LDS bytes such a load writes, would otherwise wait for it before every later
// LDS read, including reads of the other stage, and expose the load latency on
// every tile.  The caller waits for these loads itself (vmcnt) before the
// barrier that hands the stage to the readers.  An LDS-DMA load needs one wait
// state after a scalar write of M0; the compiler inserts it for loads it
// generates but cannot see into this string, hence the s_nop.  The compiler keeps nothing in
// M0 across these statements in the prefill kernels (checked in their assembly).
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}


}  // namespace pkv
