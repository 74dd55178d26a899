// conv1d.hip -- causal depthwise conv1d (+SiLU) for the Gated DeltaNet
// layer: the short convolution that produces q, k, v (Vallmo.jl README,
// "What's here"; the oxydllm 0.0.0-alpha.12.2 notes, "New Features", keep
// its window as per-sequence state).
//
// Bandwidth-bound: every input element is read once (plus a W-1 halo per
// run of tokens) and every output written once.  A thread owns one 16-byte
// vector of channels (8 bf16 or 4 fp32) and walks a run of TOK tokens with
// the last W-1 inputs in registers, so rows are read with 128-bit loads and
// consecutive threads touch consecutive 16-byte words.
//
// Bit-exact arithmetic: acc = bias (or 0); acc = fma(w_j, x_j, acc) for
// j = 0..W-1; y = acc / (1 + exp_cw(-acc)); bf16 output rounded to nearest
// even (NaN -> 0x7fc0).  For bf16 outputs the SiLU is evaluated on a fast
// path that provably rounds to the same bf16 (silu_for_bf16 in conv_math.h), since
// the exact exponential and division dominate the kernel's ALU time.
// Contraction is switched off in this file so the compiler adds or removes
// no fused multiply-adds.
#pragma clang fp contract(off)

#include <type_traits>

#include "conv_math.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <class E>
struct Vec;  // 16 bytes of channels
template <>
struct Vec<BF16> {
  static constexpr int N = 8;
  typedef u32x4 raw_t;
  // inputs are read once (the halo rows a second time, from L2): streaming loads
  __device__ __forceinline__ static raw_t load_raw(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ static void cvt(raw_t w, float* out) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float* out) { cvt(load_raw(p), out); }
  __device__ __forceinline__ static void store(uint16_t* p, const float* v) {
    *reinterpret_cast<u32x4*>(p) = conv_pack_bf16x8(v);
  }
};
template <>
struct Vec<F32> {
  static constexpr int N = 4;
  typedef f32x4 raw_t;
  __device__ __forceinline__ static raw_t load_raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ static void cvt(raw_t w, float* out) {
#pragma unroll
    for (int i = 0; i < 4; i++) out[i] = w[i];
  }
  __device__ __forceinline__ static void load(const float* p, float* out) { cvt(load_raw(p), out); }
  __device__ __forceinline__ static void store(float* p, const float* v) {
    f32x4 w = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p) = w;
  }
};

// Sequence containing token t: the last s with cu[s] <= t.
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seq, int t) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <class E, int W, int TOK, int RUN, bool ACT>
__global__ void __launch_bounds__(256) k_conv1d(ConvArgs a) {
  typedef typename E::store_t T;
  constexpr int V = Vec<E>::N;
  constexpr int SPAN = TOK * RUN;  // tokens per thread
  // One-dimensional grid of (token span, channel block) pairs, span-major.
  // Workgroups go to the 8 XCDs round-robin by id; each XCD is given one
  // contiguous run of token spans (all channel blocks of each), i.e. one
  // contiguous stretch of rows, so the W-1 halo rows a span reads were
  // fetched into that XCD's L2 by its predecessor.
  // Channel blocks of 256 groups (the launch's block size); with a power of
  // two of them (8192 channels: 4) the index splits by shifts, since an
  // integer division here delays every address, hence every first load.
  const int ncb = (a.channels / V + 255) >> 8;
  int L = blockIdx.x;
  if ((gridDim.x & 7) == 0) L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  int span_idx, cb;
  if ((ncb & (ncb - 1)) == 0) {
    span_idx = L >> __builtin_ctz(ncb);
    cb = L & (ncb - 1);
  } else {
    span_idx = L / ncb;
    cb = L - span_idx * ncb;
  }
  const int cg = cb * 256 + threadIdx.x;  // channel group
  const int c0 = cg * V;
  if (c0 >= a.channels) return;
  const int t_begin = span_idx * SPAN;
  if (t_begin >= a.total_tokens) return;
  const int t_end = min(t_begin + SPAN, a.total_tokens);

  // Every load below is unconditional: an optional operand is read from a
  // valid stand-in address and masked to +0 afterwards.  A load inside a
  // branch makes the compiler drain all loads in flight where the branch
  // rejoins, i.e. one full memory round trip per optional operand.
  float w[V][W];
  float bias[V];
  const float* bsrc = a.bias ? a.bias : a.weight;
  const uint32_t bmask = a.bias ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < V; i++) {
#pragma unroll
    for (int j = 0; j < W; j++) w[i][j] = a.weight[(long)(c0 + i) * W + j];
    bias[i] = __uint_as_float(__float_as_uint(bsrc[c0 + i]) & bmask);
  }
  const T* x = reinterpret_cast<const T*>(a.x);
  T* y = reinterpret_cast<T*>(a.y);
  const T* win = reinterpret_cast<const T*>(a.conv_state);

  int seq, seq_start, seq_end;
  if (a.seqlen > 0) {
    seq = a.num_seqs == 1 ? 0 : t_begin / a.seqlen;
    seq_start = seq * a.seqlen;
    seq_end = seq_start + a.seqlen;
  } else {
    seq = find_seq(a.cu_seqlens, a.num_seqs, t_begin);
    seq_start = a.cu_seqlens[seq];
    seq_end = a.cu_seqlens[seq + 1];
  }

  // Fast path: a span inside one sequence.  The span is walked in RUN
  // blocks of TOK rows; the rows of block r + 1 are in flight while block r
  // is computed, and the last W inputs stay converted to fp32 in a sliding
  // register window, so no row is read twice.  Halo rows before the
  // sequence's first token come from its window (or are zero).  Spans at a
  // sequence start and the ragged last span take this path too: the grid is
  // resident all at once, so a workgroup on the token-by-token path below
  // would set the kernel's duration.  The ragged span runs its own copy of
  // the walk (RAGGED: row addresses clamped into the span, rows past its end
  // computed and not stored); in the full span's code the guards cost
  // 2.5 us at the 4096-token layer.
  typedef typename Vec<E>::raw_t raw_t;
  auto walk = [&](auto ragged) {
    constexpr bool RAGGED = decltype(ragged)::value;
    auto row_at = [&](int t) { return RAGGED ? min(t, t_end - 1) : t; };
    raw_t halo[W - 1], cur[TOK];
#pragma unroll
    for (int j = 0; j < W - 1; j++) {
      // from x inside the sequence, else slot (W-1) + (pos - seq_start) of
      // the sequence's window, else zero (a row of x read and masked)
      const int pos = t_begin - (W - 1) + j;
      const bool in_seq = pos >= seq_start;
      const T* src = in_seq ? x + (long)pos * a.stride_x + c0
                     : win  ? win + ((long)seq * (W - 1) + (W - 1) + (pos - seq_start)) * a.channels + c0
                            : x + (long)t_begin * a.stride_x + c0;
      halo[j] = Vec<E>::load_raw(src);
      if (!in_seq && !win) halo[j] = raw_t{};
    }
#pragma unroll
    for (int j = 0; j < TOK; j++) cur[j] = Vec<E>::load_raw(x + (long)row_at(t_begin + j) * a.stride_x + c0);
    float wv[W][V];
#pragma unroll
    for (int j = 0; j < W - 1; j++) Vec<E>::cvt(halo[j], wv[j]);
#pragma unroll
    for (int r = 0; r < RUN; r++) {
      raw_t nxt[TOK];
      if (r + 1 < RUN) {
#pragma unroll
        for (int j = 0; j < TOK; j++)
          nxt[j] = Vec<E>::load_raw(x + (long)row_at(t_begin + (r + 1) * TOK + j) * a.stride_x + c0);
      }
#pragma unroll
      for (int tt = 0; tt < TOK; tt++) {
        const int p = r * TOK + tt;  // wv[(p + j) % W] holds input p - (W-1) + j
        Vec<E>::cvt(cur[tt], wv[(p + W - 1) % W]);
        float out[V];
#pragma unroll
        for (int i = 0; i < V; i++) {
          float xv[W];
#pragma unroll
          for (int j = 0; j < W; j++) xv[j] = wv[(p + j) % W][i];
          if constexpr (ACT && std::is_same<E, BF16>::value) out[i] = conv_sum<W>(bias[i], w[i], xv);
          else out[i] = conv_point<E, W, ACT>(bias[i], w[i], xv);
        }
        const bool keep = !RAGGED || t_begin + p < t_end;
        if constexpr (ACT && std::is_same<E, BF16>::value) {
          silu8_for_bf16(out);
          if (keep) *reinterpret_cast<u32x4*>(y + (long)(t_begin + p) * a.stride_y + c0) = conv_pack_bf16x8_canonical(out);
        } else {
          if (keep) Vec<E>::store(y + (long)(t_begin + p) * a.stride_y + c0, out);
        }
      }
      if (r + 1 < RUN) {
#pragma unroll
        for (int j = 0; j < TOK; j++) cur[j] = nxt[j];
      }
    }
  };
  if (t_end <= seq_end) {
    if (t_end - t_begin == SPAN) walk(std::false_type{});
    else walk(std::true_type{});
    return;
  }

  // General path (a sequence starts inside the span).  Rows are fetched TOK
  // at a time, the next block's in flight while a block runs, each address
  // clamped into the span so that no load sits in a branch; tokens then run
  // one by one, and a sequence start reloads that sequence's context.
  // hist[j] = input at position t - (W-1) + j for the token t about to run
  typedef typename Vec<E>::raw_t raw_t;
  float hist[W][V];
  auto fill_context = [&](int t) {  // positions t-(W-1) .. t-1 of sequence seq
#pragma unroll
    for (int j = 0; j < W - 1; j++) {
      const int pos = t - (W - 1) + j;
      const bool in_seq = pos >= seq_start;
      const T* src = in_seq ? x + (long)pos * a.stride_x + c0
                     : win  ? win + ((long)seq * (W - 1) + (W - 1) + (pos - seq_start)) * a.channels + c0
                            : x + (long)t * a.stride_x + c0;
      raw_t v = Vec<E>::load_raw(src);
      if (!in_seq && !win) v = raw_t{};
      Vec<E>::cvt(v, hist[j]);
    }
  };
  auto row = [&](int t) { return Vec<E>::load_raw(x + (long)min(t, t_end - 1) * a.stride_x + c0); };
  raw_t rows[TOK];
#pragma unroll
  for (int j = 0; j < TOK; j++) rows[j] = row(t_begin + j);
  fill_context(t_begin);

  for (int tb = t_begin; tb < t_end; tb += TOK) {
    raw_t nrows[TOK];
#pragma unroll
    for (int j = 0; j < TOK; j++) nrows[j] = row(tb + TOK + j);
#pragma unroll
    for (int j = 0; j < TOK; j++) {
      const int t = tb + j;
      if (t < t_end) {
        if (t == seq_end) {  // next sequence: fresh context
          seq++;
          if (a.seqlen > 0) {
            seq_start = t;
            seq_end = t + a.seqlen;
          } else {
            while (a.cu_seqlens[seq + 1] <= t) seq++;  // skip empty sequences
            seq_start = a.cu_seqlens[seq];
            seq_end = a.cu_seqlens[seq + 1];
          }
          fill_context(t);
        }
        Vec<E>::cvt(rows[j], hist[W - 1]);
        float out[V];
#pragma unroll
        for (int i = 0; i < V; i++) {
          float xv[W];
#pragma unroll
          for (int k = 0; k < W; k++) xv[k] = hist[k][i];
          out[i] = conv_point<E, W, ACT>(bias[i], w[i], xv);
        }
        Vec<E>::store(y + (long)t * a.stride_y + c0, out);
#pragma unroll
        for (int k = 0; k < W - 1; k++)
#pragma unroll
          for (int i = 0; i < V; i++) hist[k][i] = hist[k + 1][i];
      }
    }
#pragma unroll
    for (int j = 0; j < TOK; j++) rows[j] = nrows[j];
  }
}

// New window = last W-1 raw inputs of (old window ++ sequence).  One thread
// per (sequence, 16-byte channel group); it reads everything it needs before
// writing, so the update is in place.  Runs after k_conv1d on the stream.
template <class E, int W>
__global__ void __launch_bounds__(256) k_conv_window(ConvArgs a) {
  typedef typename E::store_t T;
  constexpr int V = Vec<E>::N;
  const int cg = blockIdx.y * blockDim.x + threadIdx.x;
  const int c0 = cg * V;
  const int seq = blockIdx.x;
  if (c0 >= a.channels || seq >= a.num_seqs) return;
  int s0, s1;
  if (a.seqlen > 0) {
    s0 = seq * a.seqlen;
    s1 = s0 + a.seqlen;
  } else {
    s0 = a.cu_seqlens[seq];
    s1 = a.cu_seqlens[seq + 1];
  }
  const int len = s1 - s0;
  if (len == 0) return;
  const T* x = reinterpret_cast<const T*>(a.x);
  T* win = reinterpret_cast<T*>(a.conv_state);
  T* mywin = win + (long)seq * (W - 1) * a.channels + c0;
  float nw[W - 1][V];
#pragma unroll
  for (int i = 0; i < W - 1; i++) {
    int pos = len - (W - 1) + i;  // position in the sequence
    if (pos >= 0)
      Vec<E>::load(x + (long)(s0 + pos) * a.stride_x + c0, nw[i]);
    else
      Vec<E>::load(mywin + (long)((W - 1) + pos) * a.channels, nw[i]);
  }
#pragma unroll
  for (int i = 0; i < W - 1; i++) Vec<E>::store(mywin + (long)i * a.channels, nw[i]);
}

// One token per sequence (decode): read window + token, write y and the
// shifted window.  Same arithmetic as k_conv1d.
template <class E, int W>
__global__ void __launch_bounds__(256) k_conv_step(ConvArgs a) {
  typedef typename E::store_t T;
  constexpr int V = Vec<E>::N;
  const int cg = blockIdx.y * blockDim.x + threadIdx.x;
  const int c0 = cg * V;
  const int seq = blockIdx.x;
  if (c0 >= a.channels || seq >= a.num_seqs) return;
  const T* x = reinterpret_cast<const T*>(a.x);
  T* y = reinterpret_cast<T*>(a.y);
  T* win = reinterpret_cast<T*>(a.conv_state);
  // Every load is issued before any value is used, with no load under a
  // branch: a missing window reads this token's row in its place and a
  // missing bias reads the weights, both masked to zero afterwards.
  const bool has_win = win != nullptr, has_bias = a.bias != nullptr;
  const T* xrow = x + (long)seq * a.stride_x + c0;
  typename Vec<E>::raw_t raw[W];
#pragma unroll
  for (int j = 0; j < W - 1; j++)
    raw[j] = Vec<E>::load_raw(has_win ? win + ((long)seq * (W - 1) + j) * a.channels + c0 : xrow);
  raw[W - 1] = Vec<E>::load_raw(xrow);
  const float* bsrc = has_bias ? a.bias : a.weight;
  float bias[V], wj[V][W];
#pragma unroll
  for (int i = 0; i < V; i++) {
    bias[i] = bsrc[c0 + i];
#pragma unroll
    for (int j = 0; j < W; j++) wj[i][j] = a.weight[(long)(c0 + i) * W + j];
  }
  float hist[W][V];
#pragma unroll
  for (int j = 0; j < W; j++) {
    Vec<E>::cvt(raw[j], hist[j]);
    if (j < W - 1)
#pragma unroll
      for (int i = 0; i < V; i++) hist[j][i] = has_win ? hist[j][i] : 0.0f;
  }
  float out[V];
#pragma unroll
  for (int i = 0; i < V; i++) {
    float xv[W];
#pragma unroll
    for (int j = 0; j < W; j++) xv[j] = hist[j][i];
    const float b = has_bias ? bias[i] : 0.0f;
    out[i] = a.activation ? conv_point<E, W, true>(b, wj[i], xv) : conv_point<E, W, false>(b, wj[i], xv);
  }
  Vec<E>::store(y + (long)seq * a.stride_y + c0, out);
  if (win) {
#pragma unroll
    for (int j = 0; j < W - 1; j++)
      Vec<E>::store(win + ((long)seq * (W - 1) + j) * a.channels + c0, hist[j + 1]);
  }
}

// rows per block and blocks per thread (one halo per 16 rows; the next
// block's loads in flight while a block is computed).  At the 4096-token
// layer (bf16, 8192 channels, N(0, 1) inputs, one call after another):
// 4 x 4 28.9 us, 4 x 8 31.9.  With the exact SiLU branch never taken
// (constant inputs) 4 x 8 led: 25.7 against 26.6, then 2 x 8 27.2,
// 4 x 16 27.0, 8 x 4 28.5, 8 x 2 28.6, 2 x 16 29.2, 4 x 2 32.0, 8 x 1 32.1,
// 2 x 4 33.7; with real data the kernel is near VALU-bound and the four
// workgroups per CU of 4 x 4 hide more of it.
constexpr int kConvTok = 4;
constexpr int kConvRun = 4;

template <class E, int W>
hipError_t launch_w(const ConvArgs& a, hipStream_t s) {
  constexpr int V = Vec<E>::N;
  const int groups = a.channels / V;
  dim3 block(256);
  if (a.seqlen == 1) {
    dim3 grid(a.num_seqs, (groups + 255) / 256);
    if (a.num_seqs > 0) hipLaunchKernelGGL((k_conv_step<E, W>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (a.total_tokens > 0) {
    constexpr int span = kConvTok * kConvRun;
    const long nblk = (long)((a.total_tokens + span - 1) / span) * ((groups + 255) / 256);
    if (nblk > 0x7fffffffL) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)nblk);
    if (a.activation)
      hipLaunchKernelGGL((k_conv1d<E, W, kConvTok, kConvRun, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_conv1d<E, W, kConvTok, kConvRun, false>), grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.conv_state && a.num_seqs > 0) {
    dim3 grid(a.num_seqs, (groups + 255) / 256);
    hipLaunchKernelGGL((k_conv_window<E, W>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_e(const ConvArgs& a, hipStream_t s) {
  switch (a.width) {
    case 2: return launch_w<E, 2>(a, s);
    case 3: return launch_w<E, 3>(a, s);
    case 4: return launch_w<E, 4>(a, s);
    case 5: return launch_w<E, 5>(a, s);
    case 6: return launch_w<E, 6>(a, s);
    case 7: return launch_w<E, 7>(a, s);
    case 8: return launch_w<E, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s) {
  return a.dtype == 1 ? launch_e<BF16>(a, s) : launch_e<F32>(a, s);
}

}  // namespace gdn
