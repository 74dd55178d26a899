// gated_norm.hip -- the gated RMS norm on the layer's output, the step
// between the recurrence and the output projection (oxydllm 0.0.0-alpha.12.2
// release notes, "Performance": the Gated DeltaNet's gated norm runs as one
// fused kernel over the whole token batch; "New Features", GGUF qwen35: its
// weight is used as stored, with no plus-one).  Per (token, v-head) row of
// d_v values:
//   y_j = w_j * o_j / sqrt(mean_i o_i^2 + eps) * silu(z_j)
//
// HBM-bound: o and z are read once and y written once.  A thread owns one
// 16-byte word of a row (8 bf16 or 4 fp32); the LPR = d_v / 8 (or / 4) lanes
// of a row reduce its sum of squares with lane shuffles, so no LDS and no
// barrier are needed.  Consecutive threads touch consecutive words, and a
// thread reads its word before writing the same place, so y may be o.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <class E>
struct Word;
template <>
struct Word<BF16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const void* p, float* v) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  // y is not read again by this kernel: streaming stores (2 us less at the
  // 4096-token layer)
  __device__ __forceinline__ static void store(void* p, const float* v) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = cvt_bf16x2(v[2 * i], v[2 * i + 1]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  }
};
template <>
struct Word<F32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const void* p, float* v) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = w[i];
  }
  __device__ __forceinline__ static void store(void* p, const float* v) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
  }
};

// silu(z) = z / (1 + e^-z) on the hardware exponential and reciprocal
// (relative error a few fp32 ulp, far inside the layer's tolerance).
__device__ __forceinline__ float silu_gate(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// R rows per thread, spaced a workgroup's row count apart: all 2R loads are
// issued before the first row's reduction, so a wave keeps R times more
// bytes in flight.
template <class E, int DV, int R>
__global__ void __launch_bounds__(256) k_gated_norm(NormArgs a) {
  constexpr int V = Word<E>::N;
  constexpr int LPR = DV / V;  // lanes per row: 8, 16 or 32, inside one wave
  static_assert(LPR >= 2 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row width");
  constexpr int RPB = 256 / LPR;  // rows per workgroup and round
  typedef typename E::store_t T;
  const int part = threadIdx.x % LPR;
  const long row0 = (long)blockIdx.x * (RPB * R) + threadIdx.x / LPR;
  // All loads are issued before any is used and none sits in a branch (the
  // compiler drains every load in flight where a branch around one
  // rejoins): rows past the end read the last row and are zeroed.
  float w[V];
#pragma unroll
  for (int i = 0; i < V; i++) w[i] = a.weight[part * V + i];
  float o[R][V], z[R][V];
  long t[R];
  int h[R];
#pragma unroll
  for (int k = 0; k < R; k++) {
    const long row = row0 + k * RPB;
    // every lane of a row stays through the shuffles below; rows past the
    // end contribute zeros and store nothing
    const long rr = row < a.rows ? row : a.rows - 1;
    if (a.rows <= 0xffffffffL) {  // 32-bit division where it suffices
      const uint32_t r32 = (uint32_t)rr, tq = r32 / (uint32_t)a.heads;
      t[k] = tq;
      h[k] = (int)(r32 - tq * (uint32_t)a.heads);
    } else {
      t[k] = rr / a.heads;
      h[k] = (int)(rr - t[k] * a.heads);
    }
    const long col = (long)h[k] * DV + part * V;
    Word<E>::load(reinterpret_cast<const T*>(a.o) + t[k] * a.stride_o + col, o[k]);
    Word<E>::load(reinterpret_cast<const T*>(a.z) + t[k] * a.stride_z + col, z[k]);
  }
#pragma unroll
  for (int k = 0; k < R; k++) {
    // z is used only by the store below; this empty statement takes it as
    // an input so that the compiler cannot sink its load past the row
    // reduction (it would then be a second round trip after the first)
#pragma unroll
    for (int i = 0; i < V; i++) asm volatile("" ::"v"(z[k][i]));
    if (row0 + k * RPB >= a.rows) {
#pragma unroll
      for (int i = 0; i < V; i++) o[k][i] = z[k][i] = 0.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < R; k++) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < V; i++) ss += o[k][i] * o[k][i];
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv_rms = 1.0f / sqrtf(ss * (1.0f / DV) + a.eps);
    if (row0 + k * RPB < a.rows) {
      float y[V];
#pragma unroll
      for (int i = 0; i < V; i++) y[i] = w[i] * o[k][i] * inv_rms * silu_gate(z[k][i]);
      Word<E>::store(reinterpret_cast<T*>(a.y) + t[k] * a.stride_y + (long)h[k] * DV + part * V, y);
    }
  }
}

constexpr int kNormRows = 1;  // rows per thread (2, 4, 8 and 16 measured slower)

template <class E>
hipError_t launch_e(const NormArgs& a, hipStream_t s) {
  const int V = Word<E>::N;
  const long rows_per_block = 256 / (a.dv / V) * kNormRows;
  const long blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(256);
  if (a.dv == 128) hipLaunchKernelGGL((k_gated_norm<E, 128, kNormRows>), grid, block, 0, s, a);
  else if (a.dv == 64) hipLaunchKernelGGL((k_gated_norm<E, 64, kNormRows>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_norm(const NormArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  return a.dtype == 1 ? launch_e<BF16>(a, s) : launch_e<F32>(a, s);
}

}  // namespace gdn
