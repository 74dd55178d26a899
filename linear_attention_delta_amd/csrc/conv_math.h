// conv_math.h -- the arithmetic of the causal depthwise conv1d + SiLU that
// produces q, k, v (Vallmo.jl README, "What's here"), shared by the
// stand-alone convolution kernel and the prefill kernel that convolves its
// chunk on the fly, so both give the same bits.
//
// One output: acc = bias (or 0); acc = fma(w_j, x_j, acc) for j = 0..W-1 in
// tap order (tap W-1 multiplies the current token); y = acc / (1 +
// exp_cw(-acc)); a bf16 output is rounded to nearest even with NaN -> 0x7fc0.
// Contraction is switched off inside every function here so the compiler
// adds or removes no fused multiply-adds.
#pragma once

#include <type_traits>

#include "gdn_device.h"

namespace gdn {

__device__ __forceinline__ float silu_exact(float a) {
#pragma clang fp contract(off)
  return a / (1.0f + exp_cw(-a));
}

// SiLU for an output that is rounded to bf16.  The fp32 value of
// a * (1 + 2^(-a log2 e))^-1 from the hardware exponential and reciprocal is
// within a few ulp of silu_exact(a) for every fp32 a > -8, so both round to
// the same bf16 unless a bf16 rounding midpoint lies within that distance.  Results whose low 16 bits are within
// 16 of the midpoint pattern 0x8000, and every a <= -8 (where the relative
// error of the exponential grows with |a|), take the exact path instead:
// the rounded output is that of silu_exact, bit for bit, at a fraction of
// its cost.  NaN stays NaN on both paths (the store canonicalises it).
// The convolution test drives every one of the 2^32 fp32 pre-activations
// through the kernel and finds each rounded output equal to the exact
// definition's, bit for bit.
__device__ __forceinline__ float silu_fast(float a);
__device__ __forceinline__ bool silu_needs_exact(float a, float q);
__device__ __forceinline__ float silu_for_bf16(float a) {
  const float q = silu_fast(a);
  return silu_needs_exact(a, q) ? silu_exact(a) : q;
}

template <class E>
__device__ __forceinline__ float silu(float a) {
  if constexpr (std::is_same<E, BF16>::value) return silu_for_bf16(a);
  return silu_exact(a);
}

// True where the fast form of silu_for_bf16 may round differently from
// silu_exact (and for NaN).
__device__ __forceinline__ bool silu_needs_exact(float a, float q) {
  const uint32_t low = __float_as_uint(q) & 0xffffu;
  return !(a > -8.0f) || low - (0x8000u - 16u) <= 32u;
}

__device__ __forceinline__ float silu_fast(float a) {
#pragma clang fp contract(off)
  const float e = __builtin_amdgcn_exp2f(-a * 1.44269504088896341f);
  return a * __builtin_amdgcn_rcpf(1.0f + e);
}

// Eight SiLU outputs of a 16-byte bf16 word, each equal to silu<BF16> of its
// input: the fast form for all eight, then one branch that redoes the
// flagged ones exactly.  The test for the branch is done for the word as a
// whole, with few vector instructions (the kernel is bound by them): the
// a > -8 compares combine as lane masks on the scalar unit, and the
// distances of the eight results' low halves to the midpoint pattern are
// formed two at a time in 16-bit lanes and reduced to their minimum.  Only
// a taken branch (any of 64 lanes asking) tests the elements one by one.
typedef unsigned short conv_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void silu8_for_bf16(float (&v)[8]) {
  float q[8];
  bool neg = false;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    q[i] = silu_fast(v[i]);
    neg |= !(v[i] > -8.0f);
  }
  conv_u16x2 d[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    // low 16 bits of q[2k] and q[2k+1] side by side, less (0x8000 - 16)
    const uint32_t w = __builtin_amdgcn_perm(__float_as_uint(q[2 * k + 1]), __float_as_uint(q[2 * k]), 0x05040100u);
    d[k] = __builtin_bit_cast(conv_u16x2, w) - conv_u16x2{0x8000 - 16, 0x8000 - 16};
  }
  const conv_u16x2 m01 = __builtin_elementwise_min(d[0], d[1]), m23 = __builtin_elementwise_min(d[2], d[3]);
  const conv_u16x2 m = __builtin_elementwise_min(m01, m23);
  const bool band = (m.x < m.y ? m.x : m.y) <= 32;
  if (neg || band) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (silu_needs_exact(v[i], q[i])) {
        // NaN can only arise here (every NaN or -inf input is flagged): make
        // it the canonical quiet NaN, so the rounding below needs no check
        const float e = silu_exact(v[i]);
        q[i] = e != e ? __uint_as_float(0x7fc00000u) : e;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = q[i];
}

// One convolution output from the W inputs in tap order.
template <class E, int W, bool ACT>
__device__ __forceinline__ float conv_point(float bias, const float (&w)[W], const float (&xv)[W]) {
#pragma clang fp contract(off)
  float acc = bias;
#pragma unroll
  for (int j = 0; j < W; j++) acc = __builtin_fmaf(w[j], xv[j], acc);
  return ACT ? silu<E>(acc) : acc;
}

// The pre-activation sum alone (the same fma chain as conv_point).
template <int W>
__device__ __forceinline__ float conv_sum(float bias, const float (&w)[W], const float (&xv)[W]) {
#pragma clang fp contract(off)
  float acc = bias;
#pragma unroll
  for (int j = 0; j < W; j++) acc = __builtin_fmaf(w[j], xv[j], acc);
  return acc;
}

// Eight outputs rounded to bf16 with the hardware conversion (nearest even),
// for values that are finite, infinite or the canonical quiet NaN (which
// converts to 0x7fc0): the outputs of silu8_for_bf16.
__device__ __forceinline__ u32x4 conv_pack_bf16x8_canonical(const float* v) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; i++) w[i] = cvt_bf16x2(v[2 * i], v[2 * i + 1]);
  return w;
}

// Eight outputs rounded to bf16 (nearest even with the hardware conversion;
// a NaN is first made the canonical quiet NaN so that it converts to 0x7fc0).
__device__ __forceinline__ u32x4 conv_pack_bf16x8(const float* v) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float lo = v[2 * i] != v[2 * i] ? __uint_as_float(0x7fc00000u) : v[2 * i];
    const float hi = v[2 * i + 1] != v[2 * i + 1] ? __uint_as_float(0x7fc00000u) : v[2 * i + 1];
    w[i] = cvt_bf16x2(lo, hi);
  }
  return w;
}

}  // namespace gdn
