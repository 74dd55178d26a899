// gdn_device.h -- device helpers for the gfx950 kernels of libgdn.
//
// bf16 handling, 128-bit vector types, the matrix-core (MFMA) tile
// primitive, wave-level reductions and the fp32 exponential the
// convolution uses.
//
// MFMA operand layout on gfx950 (64-lane wave), for D(16x16) += A(16xK) B(Kx16):
//   A: lane l holds row (l % 16), k = kb + KPL*(l / 16) + e, e < KPL
//   B: lane l holds col (l % 16), k = kb + KPL*(l / 16) + e
//   D: lane l holds col (l % 16), rows 4*(l / 16) + e, e < 4
// with KPL = 8 (v_mfma_f32_16x16x32_bf16, K step 32) or KPL = 1
// (v_mfma_f32_16x16x4_f32, K step 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// c + a.lo b.lo + a.hi b.hi for two packed bf16 pairs, in fp32, one
// instruction (sums of squares for the q/k norms).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two fp32 -> packed bf16 pair with the gfx950 convert instruction (round to
// nearest even).  Used on the tolerance-checked paths; the bit-exact
// convolution keeps its own rounding above.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element traits: storage type of q/k/v/o and of the MFMA operands.
struct BF16 {
  typedef uint16_t store_t;
  static constexpr int KPL = 8;    // operand elements per lane
  static constexpr int KSTEP = 32; // K covered by one MFMA
  typedef bf16x8 frag_t;
  __device__ __forceinline__ static float to_f32(store_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static store_t from_f32(float f) { return f32_to_bf16(f); }
};

struct F32 {
  typedef float store_t;
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 4;
  typedef float frag_t;
  __device__ __forceinline__ static float to_f32(store_t v) { return v; }
  __device__ __forceinline__ static store_t from_f32(float f) { return f; }
};

// Load one MFMA operand fragment: KPL consecutive elements starting at p
// (p must be 16-byte aligned for bf16).
__device__ __forceinline__ bf16x8 load_frag(const uint16_t* p, BF16) {
  u32x4 w = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ float load_frag(const float* p, F32) { return *p; }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D += A[row0.., k0..k0+K) * B[k0..k0+K), col0..) where A is row-major with
// leading dimension lda and B is given TRANSPOSED (BT row-major [col][k],
// leading dimension ldb) -- both operands then read KPL contiguous elements.
// fp32 operands (K a multiple of 16): the 16 k of four consecutive 16x16x4
// steps are regrouped so that each lane's four values sit side by side
// (step i, lane (r, q) takes k = kb + 4q + i), so each operand is one
// 16-byte read per four steps instead of one 4-byte read per step.  Every k
// is used exactly once, by the same lane of A and B.  Rows of A and BT must
// be 16-byte aligned.  BATCH: every read in flight before the first product
// (left to itself, the compiler waits on each pair right after issuing it;
// batching costs 8 VGPRs per 16 k).
template <int K, bool BATCH>
__device__ __forceinline__ f32x4 tile_mma_f32(f32x4 acc, const float* A, int lda, const float* BT, int ldb,
                                              int lane) {
  static_assert(K % 16 == 0, "K must be a multiple of 16");
  const int r = lane & 15, kq = (lane >> 4) * 4;
  const float* pa = A + r * lda + kq;
  const float* pb = BT + r * ldb + kq;
  f32x4 a4[K / 16], b4[K / 16];
#pragma unroll
  for (int j = 0; j < K / 16; j++) {
    a4[j] = *reinterpret_cast<const f32x4*>(pa + 16 * j);
    b4[j] = *reinterpret_cast<const f32x4*>(pb + 16 * j);
  }
  if constexpr (BATCH) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < K / 16; j++)
#pragma unroll
    for (int i = 0; i < 4; i++) acc = mfma16(a4[j][i], b4[j][i], acc);
  return acc;
}

template <class E, int K, bool BATCH = false>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const typename E::store_t* A, int lda,
                                          const typename E::store_t* BT, int ldb, int lane) {
  if constexpr (E::KSTEP == 4 && K % 16 == 0) return tile_mma_f32<K, BATCH>(acc, A, lda, BT, ldb, lane);
  const int r = lane & 15, kq = (lane >> 4) * E::KPL;
  const typename E::store_t* pa = A + r * lda + kq;
  const typename E::store_t* pb = BT + r * ldb + kq;
#pragma unroll
  for (int kb = 0; kb < K; kb += E::KSTEP) {
    acc = mfma16(load_frag(pa + kb, E()), load_frag(pb + kb, E()), acc);
  }
  return acc;
}

// ---------------------------------------------------------- reductions

// v plus the value of the lane 16 (or 32) apart, in every lane, through the
// row swaps v_permlane16_swap / v_permlane32_swap (odd 16- or 32-lane rows of
// the first operand traded with even rows of the second), with no trip
// through the LDS.  Each lane adds its own value and its partner's; the sum
// is the same either way round.
__device__ __forceinline__ float add_lane_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_lane_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32 or 64), every lane
// of a group receiving the group's sum.  Within 16-lane rows the exchange
// uses DPP lane swizzles, across rows the row swaps (no LDS traffic).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v += __builtin_amdgcn_update_dpp(0.f, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  if (N >= 4) v += __builtin_amdgcn_update_dpp(0.f, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if (N >= 8) v += __builtin_amdgcn_update_dpp(0.f, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  if (N >= 16) v += __builtin_amdgcn_update_dpp(0.f, v, 0x140, 0xF, 0xF, false); // row_mirror
  if (N >= 32) v = add_lane_xor16(v);
  if (N >= 64) v = add_lane_xor32(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Index of the calling wave in its workgroup, as a value the compiler knows
// to be uniform across the wave: index arithmetic and loops that depend on
// it then run on the scalar unit instead of costing vector instructions.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Workgroup barrier for LDS traffic: every wave's earlier LDS writes are
// visible to every wave's later LDS reads.  Unlike __syncthreads(), whose
// workgroup fence also covers global memory and so makes each wave wait
// until all of its global loads have returned and its global stores have
// been acknowledged, this orders LDS only: global stores keep draining and
// prefetched loads stay in flight across the barrier.  For workgroups whose
// waves exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Make this wave's earlier LDS writes visible to its later LDS reads
// (other lanes of the same wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------- fixed fp32 exponential
//
// e^x by Cody & Waite's method ("Software Manual for the Elementary
// Functions", 1980): x = n ln2 + r, n = rint(x / ln2), r = (x - n C1) - n C2
// with C1 = ln2 cut to 16 significant bits (n C1 exact for |n| < 256) and
// C2 = fp32(ln2 - C1); e^r by its Taylor series through r^7 in Horner form
// with fused multiply-adds; then scaled by 2^n.  Inputs above 88.5 give
// +inf, below -86 give 0, so every finite result is a normal number; NaN
// gives itself.  The operation order is fixed so that the convolution's
// output is a function of its inputs alone, reproducible bit for bit by any
// IEEE fp32 machine that follows the same steps.  The three special ranges
// are selected at the end rather than branched on, so a wave never splits.
__device__ __forceinline__ float exp_cw(float x) {
  const float c1 = 0.693145751953125f;          // 45426 / 65536
  const float c2 = (float)(0.69314718055994530942 - 0.693145751953125);
  const float inv_ln2 = (float)(1.0 / 0.69314718055994530942);
  float n = __builtin_rintf(x * inv_ln2);
  float r = __builtin_fmaf(-n, c1, x);
  r = __builtin_fmaf(-n, c2, r);
  float p = (float)(1.0 / 5040.0);
  p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  // in range |n| <= 128; the clamp only keeps the integer conversion defined
  // for inputs whose result is replaced below
  float e = __builtin_ldexpf(p, (int)__builtin_fminf(__builtin_fmaxf(n, -200.0f), 200.0f));
  e = x > 88.5f ? __builtin_inff() : e;
  e = x < -86.0f ? 0.0f : e;
  return x != x ? x : e;
}

// ------------------------------------------------- MFMA fragment helpers
//
// A 16x16 fp32 accumulator tile (lane (c, g) holds rows 4g..4g+3 of column
// c) becomes half of a bf16 operand fragment when packed: two stacked tiles
// give, per lane, the 8 values at k = {4g+e} and {16+4g+e} of one 32-wide
// k step.  The other operand, read from LDS, must present the same k order;
// LDS copies of row-major operands therefore store each 32-column block with
// logical column 4g+e at 8g+e and 16+4g+e at 8g+4+e (perm_lo below), so a
// fragment is one 16-byte read.

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

__device__ __forceinline__ u32x2 pack4_bf16(f32x4 v) { return u32x2{cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3])}; }

__device__ __forceinline__ bf16x8 frag2(u32x2 lo, u32x2 hi) {
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Operand fragment from two stacked accumulator tiles.
__device__ __forceinline__ bf16x8 frag_acc(f32x4 lo, f32x4 hi) { return frag2(pack4_bf16(lo), pack4_bf16(hi)); }

__device__ __forceinline__ bf16x8 ld_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane L supplies the address of 4 consecutive bf16; lane i receives element
// i % 4 of the loads of lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.  With
// lane L pointing at row r0 + L / 4, column c0 + 4 (L % 4) of a row-major
// tile, lane i gets rows r0..r0+3 of column c0 + i.
__device__ __forceinline__ u32x2 ld_tr(const uint16_t* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ f32x4 bf4_to_f32(u32x2 w) {
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
               __uint_as_float(w[1] & 0xffff0000u)};
}

// Position in the LDS operand layout of the first 4 of the 8 logical columns
// 8v..8v+7 (the other 4 go 8 further on).
__device__ __forceinline__ int perm_lo(int v) { return 32 * (v >> 2) + 16 * (v & 1) + 4 * ((v >> 1) & 1); }

}  // namespace gdn
