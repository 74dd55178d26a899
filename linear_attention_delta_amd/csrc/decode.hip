// decode.hip -- the O(1) recurrent decode step of the gated delta rule
// (oxydllm 0.0.0-alpha.12.2 release notes, "New Features": one recurrent
// step per generated token on a 32x128x128 fp32 memory per sequence).
//
// Per (sequence b, v-head h), with S the d_k x d_v fp32 state:
//   kv = S^T k_hat, qs = S^T q_hat          (one pass over S)
//   u  = beta (v - alpha kv)
//   o  = alpha qs + (k_hat . q_hat) u
//   S <- alpha S + k_hat u^T                (written back in place)
// which equals decay -> delta -> write -> read of the token recurrence.
//
// The step is a pure read-modify-write of the state: 2 * d_k * d_v * 4 bytes
// per (b, h), everything else is noise.  One 256-thread workgroup owns one
// (b, h) state; thread (rg, cg) holds rows rg, rg+RG, ... of the 4-column
// group cg in registers, so a wave streams whole 512-byte rows with 128-bit
// loads and stores; the column sums are reduced across row groups in LDS.
//
// k_decode_conv also runs the layer's short convolution for the token (the
// Vallmo.jl README, "What's here"): it reads the raw projected row and the
// per-sequence conv window instead of q, k, v, so the convolved values never
// go through memory.
#include <type_traits>

#include "conv_math.h"
#include "gate_math.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr float kL2Eps = 1e-6f;

template <class E>
__device__ __forceinline__ float load_elem(const void* p, long i) {
  return E::to_f32(reinterpret_cast<const typename E::store_t*>(p)[i]);
}

// Thread layout of one 256-thread team working on one (b, h) state.
template <int DK, int DV>
struct Team {
  static constexpr int CG = DV / 4;    // 4-column groups
  static constexpr int RG = 256 / CG;  // row groups
  static constexpr int RPT = DK / RG;  // rows per thread
  static_assert(RPT >= 1 && RG * RPT == DK, "shape");
};

// The pieces below are shared by the plain step and the step that also
// runs the convolution, so that both compute the same bits.

// Stream the state in: thread (rg, cg) holds rows rg, rg+RG, ... of columns
// 4cg .. 4cg+3; every load is independent.
template <int DK, int DV>
__device__ __forceinline__ void load_state(const float* S, int rg, int cg, f32x4* s) {
  typedef Team<DK, DV> T;
#pragma unroll
  for (int m = 0; m < T::RPT; m++)
    s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rg + m * T::RG) * DV + 4 * cg));
}

// Per-wave partial sums of |k|^2, |q|^2 and k.q (the team's first d_k threads
// hold k_i and q_i, the others 0) into part[wave][0..2].
__device__ __forceinline__ void qk_partials(float kv_, float qv_, int lane, int wave, float (*part)[3]) {
  const float kk = wave_sum(kv_ * kv_), qq = wave_sum(qv_ * qv_), kq = wave_sum(kv_ * qv_);
  if (lane == 0) {
    part[wave][0] = kk;
    part[wave][1] = qq;
    part[wave][2] = kq;
  }
}

struct QKFactors {
  float rk, rq, kq;  // 1/|k|, scale/|q| (1 and scale without the norm), raw k.q
};

__device__ __forceinline__ QKFactors qk_factors(const float (*part)[3], int l2norm, float scale) {
  const float kk = part[0][0] + part[1][0] + part[2][0] + part[3][0];
  const float qq = part[0][1] + part[1][1] + part[2][1] + part[3][1];
  QKFactors f;
  f.kq = part[0][2] + part[1][2] + part[2][2] + part[3][2];
  f.rk = l2norm ? 1.0f / sqrtf(kk + kL2Eps) : 1.0f;
  f.rq = scale * (l2norm ? 1.0f / sqrtf(qq + kL2Eps) : 1.0f);
  return f;
}

// The rest of the step for one (b, h): column sums S^T k, S^T q reduced
// across row groups in red (one LDS barrier inside), then o and the new
// state.  ks, qs: the raw k and q in LDS; vv: v at this thread's 4 columns.
template <class E, int DK, int DV>
__device__ __forceinline__ void head_step(f32x4* s, const float* ks, const float* qs, const float (&vv)[4],
                                          float g, float beta, QKFactors f, f32x4 (*red)[DV / 4][2], int rg,
                                          int cg, typename E::store_t* op, float* S) {
  typedef Team<DK, DV> T;
  const float alpha = expf(g);
  // partial column sums over this thread's rows (raw q, k; scaled below)
  f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < T::RPT; m++) {
    const int i = rg + m * T::RG;
    pk += s[m] * ks[i];
    pq += s[m] * qs[i];
  }
  red[rg][cg][0] = pk;
  red[rg][cg][1] = pq;
  lds_barrier();
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < T::RG; r++) {
    sk += red[r][cg][0];
    sq += red[r][cg][1];
  }
  const float khq = f.kq * f.rk * f.rq;  // k_hat . q_hat
  f32x4 u, o;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    u[j] = beta * (vv[j] - alpha * f.rk * sk[j]);
    o[j] = alpha * f.rq * sq[j] + khq * u[j];
  }
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 4; j++) op[4 * cg + j] = E::from_f32(o[j]);
  }
#pragma unroll
  for (int m = 0; m < T::RPT; m++) {
    const int i = rg + m * T::RG;
    f32x4 nv = alpha * s[m] + (f.rk * ks[i]) * u;
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + i * DV + 4 * cg));
  }
}

template <class E, int DK, int DV>
__global__ void __launch_bounds__(256) k_decode(ScanArgs a) {
  typedef Team<DK, DV> T;
  const int h = blockIdx.x % a.hv;
  const int b = blockIdx.x / a.hv;
  const int tid = threadIdx.x;
  const int cg = tid % T::CG, rg = tid / T::CG;
  const int lane = tid & 63, wave = wave_id();
  typedef typename E::store_t ST;
  ST* op = reinterpret_cast<ST*>(a.o) + ((long)b * a.hv + h) * DV;

  const int slot = a.state_slots ? a.state_slots[b] : b;
  if (slot < 0 || slot >= a.num_slots) {  // bad slot: flag the output, leave every state alone
    if (tid < DV) op[tid] = E::from_f32(__builtin_nanf(""));
    return;
  }
  float* S = a.state + ((long)slot * a.hv + h) * (DK * DV);

  __shared__ float ks[DK], qs[DK];
  __shared__ float part[4][3];
  __shared__ f32x4 red[T::RG][T::CG][2];

  // The token's q, k, v first, then the state stream: the load counter
  // retires in order, so the q/k norms wait only for the loads before the
  // stream and run while it arrives.  Every thread loads (threads past DK
  // a clamped element, zeroed): a load inside a branch would make the
  // compiler drain every load in flight where the branch rejoins.
  const int hk = a.tiled ? (h % a.hk) : (h / (a.hv / a.hk));
  const int ti = tid < DK ? tid : tid % DK;
  float kv_ = load_elem<E>(a.k, (long)b * a.stride_k + (long)hk * DK + ti);
  float qv_ = load_elem<E>(a.q, (long)b * a.stride_q + (long)hk * DK + ti);
  float vv[4];
#pragma unroll
  for (int j = 0; j < 4; j++) vv[j] = load_elem<E>(a.v, (long)b * a.stride_v + (long)h * DV + 4 * cg + j);
  const float g = a.g[(long)b * a.hv + h];
  const float beta = a.beta[(long)b * a.hv + h];
  f32x4 s[T::RPT];
  load_state<DK, DV>(S, rg, cg, s);
  if (tid >= DK) kv_ = qv_ = 0.f;
  if (tid < DK) {
    ks[tid] = kv_;
    qs[tid] = qv_;
  }
  qk_partials(kv_, qv_, lane, wave, part);
  lds_barrier();
  head_step<E, DK, DV>(s, ks, qs, vv, g, beta, qk_factors(part, a.l2norm, a.scale), red, rg, cg, op, S);
}

// A convolution output rounded to the element type, as the stand-alone
// convolution stores it (bf16: nearest even, NaN -> 0x7fc0) and the plain
// step reads it back.
template <class E>
__device__ __forceinline__ float as_stored(float y) {
  if constexpr (std::is_same<E, BF16>::value) {
    const float c = y != y ? __uint_as_float(0x7fc00000u) : y;
    return bf16_to_f32((uint16_t)(cvt_bf16x2(c, c) & 0xffffu));
  }
  return y;
}

// A raw input as the stand-alone convolution keeps it in the window (a bf16
// NaN becomes the canonical 0x7fc0).
template <class E>
__device__ __forceinline__ typename E::store_t window_entry(typename E::store_t v) {
  if constexpr (std::is_same<E, BF16>::value) return (v & 0x7fffu) > 0x7f80u ? (uint16_t)0x7fc0u : v;
  return v;
}

// One channel of the decode-time convolution, in two phases so that its
// loads can be issued ahead of the state stream: load() reads the W-1
// window inputs, the token's raw input xr[ch], the taps and the bias;
// finish() runs the causal conv + SiLU (conv_math.h), advances the
// channel's window by one token and returns the output as stored.  Each
// channel is read and written by exactly one thread of the grid.
template <class E, int W>
struct ConvChannel {
  typedef typename E::store_t ST;
  ST raw[W];
  float wj[W], bias;
  ST* win;
  long ch, cc;
  __device__ __forceinline__ void load(const ST* xr, ST* win_, long cc_, const float* weight, const float* bias_,
                                       long ch_) {
    win = win_;
    cc = cc_;
    ch = ch_;
#pragma unroll
    for (int j = 0; j < W - 1; j++) raw[j] = win[j * cc + ch];
    raw[W - 1] = xr[ch];
#pragma unroll
    for (int j = 0; j < W; j++) wj[j] = weight[ch * W + j];
    // no load in a branch (the compiler would drain every load in flight
    // where it rejoins): a missing bias reads a tap and is masked to +0
    const float bl = (bias_ ? bias_ : weight)[ch];
    bias = __uint_as_float(__float_as_uint(bl) & (bias_ ? ~0u : 0u));
  }
  // the output as the stand-alone convolution stores it
  __device__ __forceinline__ float value() const {
    float xv[W];
#pragma unroll
    for (int j = 0; j < W; j++) xv[j] = E::to_f32(raw[j]);
    return as_stored<E>(conv_point<E, W, true>(bias, wj, xv));
  }
  // the window advanced by the token (by the channel's owner only)
  __device__ __forceinline__ void write_window() const {
#pragma unroll
    for (int j = 0; j < W - 1; j++) win[j * cc + ch] = window_entry<E>(raw[j + 1]);
  }
  __device__ __forceinline__ float finish() {
    const float y = value();
    write_window();
    return y;
  }
};

// The decode step fused with the convolution that produces its q, k, v from
// the layer's raw projected row (channels [q | k | v]).  One workgroup per
// (sequence b, q/k head hk) with one 256-thread team per v-head of the
// group (at most 4): q and k are convolved once for the whole group, so
// their window is advanced by one workgroup alone, and each team convolves
// its own head's v.  Every value that reaches the recurrence is the one the
// stand-alone convolution would have stored, so the result equals the two
// separate calls bit for bit.
template <class E, int DK, int DV, int W, bool GATED>
__global__ void __launch_bounds__(1024) k_decode_conv(ScanArgs a, ConvArgs c) {
  typedef Team<DK, DV> T;
  typedef typename E::store_t ST;
  const int hk = blockIdx.x % a.hk;
  const int b = blockIdx.x / a.hk;
  const int team = threadIdx.x >> 8, tid = threadIdx.x & 255;
  const int cg = tid % T::CG, rg = tid / T::CG;
  const int lane = tid & 63, wave = wave_id() & 3;
  const int h = a.tiled ? hk + team * a.hk : hk * (a.hv / a.hk) + team;  // this team's v-head
  ST* op = reinterpret_cast<ST*>(a.o) + ((long)b * a.hv + h) * DV;

  const int slot = a.state_slots ? a.state_slots[b] : b;
  if (slot < 0 || slot >= a.num_slots) {  // bad slot: flag the outputs, leave every state and window alone
    if (tid < DV) op[tid] = E::from_f32(__builtin_nanf(""));
    return;
  }
  __shared__ float ks[DK], qs[DK];
  __shared__ float vs[4][DV];
  __shared__ float part[4][3];
  __shared__ f32x4 red[4][T::RG][T::CG][2];

  // the convolution's inputs first: the load counter retires in order, so
  // loads issued behind the state stream wait for all of it (wide windows
  // with 128 x 128 heads load after the state instead: early, they spill)
  constexpr bool kEarly = W <= 5 || DK * DV < 128 * 128;
  float* S = a.state + ((long)slot * a.hv + h) * (DK * DV);
  f32x4 s[T::RPT];
  if constexpr (!kEarly) load_state<DK, DV>(S, rg, cg, s);
  const long cc = c.channels;
  const ST* xr = reinterpret_cast<const ST*>(c.x) + (long)b * c.stride_x;
  ST* win = reinterpret_cast<ST*>(c.conv_state) + (long)slot * (W - 1) * cc;
  // q and k of head hk on the first team (thread i < d_k takes channel i of
  // both), each team's own v
  const bool qk = team == 0 && tid < DK;
  const long chq = hk * DK + tid, chk = (a.hk + hk) * DK + tid, chv = 2 * a.hk * DK + h * DV + tid;
  ConvChannel<E, W> cq, ck, cv;
  if constexpr (kEarly) {
    // every thread loads (threads that own no channel a clamped one, whose
    // value is computed and dropped): loads inside the ownership branches
    // were drained where those rejoined, one round trip before the state
    // stream went out
    const int tq = tid % DK, tv = tid % DV;
    cq.load(xr, win, cc, c.weight, c.bias, hk * DK + tq);
    ck.load(xr, win, cc, c.weight, c.bias, (a.hk + hk) * DK + tq);
    cv.load(xr, win, cc, c.weight, c.bias, 2 * a.hk * DK + h * DV + tv);
  }
  // the gates: two instantiations rather than a branch, whose loads the
  // compiler drained before the state stream went out
  float g, beta;
  if constexpr (GATED) {
    gates_from_raw<E>(a, b, h, g, beta);
  } else {
    g = a.g[(long)b * a.hv + h];
    beta = a.beta[(long)b * a.hv + h];
  }
  if constexpr (kEarly) load_state<DK, DV>(S, rg, cg, s);

  if constexpr (kEarly) {
    // the values for every thread, unconditionally, so that the loads above
    // stay ahead of the state stream; only the owners keep them
    const float qv0 = cq.value(), kv0 = ck.value(), vv0 = cv.value();
    if (team == 0) {
      const float kv_ = qk ? kv0 : 0.f, qv_ = qk ? qv0 : 0.f;
      if (qk) {
        cq.write_window();
        ck.write_window();
        ks[tid] = kv_;
        qs[tid] = qv_;
      }
      qk_partials(kv_, qv_, lane, wave, part);
    }
    if (tid < DV) {
      cv.write_window();
      vs[team][tid] = vv0;
    }
  } else {
    // late loads go one channel at a time, to keep fewer values live
    if (team == 0) {
      float kv_ = 0.f, qv_ = 0.f;
      if (qk) {
        cq.load(xr, win, cc, c.weight, c.bias, chq);
        qv_ = cq.finish();
        ck.load(xr, win, cc, c.weight, c.bias, chk);
        kv_ = ck.finish();
        ks[tid] = kv_;
        qs[tid] = qv_;
      }
      qk_partials(kv_, qv_, lane, wave, part);
    }
    if (tid < DV) {
      cv.load(xr, win, cc, c.weight, c.bias, chv);
      vs[team][tid] = cv.finish();
    }
  }
  lds_barrier();
  float vv[4];
#pragma unroll
  for (int i = 0; i < 4; i++) vv[i] = vs[team][4 * cg + i];
  head_step<E, DK, DV>(s, ks, qs, vv, g, beta, qk_factors(part, a.l2norm, a.scale), red[team], rg, cg, op, S);
}

template <class E>
hipError_t launch_e(const ScanArgs& a, hipStream_t st) {
  dim3 grid(a.hv * a.num_seqs), block(256);
  if (a.dk == 128 && a.dv == 128) hipLaunchKernelGGL((k_decode<E, 128, 128>), grid, block, 0, st, a);
  else if (a.dk == 128 && a.dv == 64) hipLaunchKernelGGL((k_decode<E, 128, 64>), grid, block, 0, st, a);
  else if (a.dk == 64 && a.dv == 128) hipLaunchKernelGGL((k_decode<E, 64, 128>), grid, block, 0, st, a);
  else if (a.dk == 64 && a.dv == 64) hipLaunchKernelGGL((k_decode<E, 64, 64>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <class E, int DK, int DV>
hipError_t launch_conv_dims(const ScanArgs& a, const ConvArgs& c, hipStream_t st) {
  // one team per v-head of the group
  const int group = a.hv / a.hk;
  if (group > 4) return hipErrorInvalidValue;
  dim3 grid(a.hk * a.num_seqs), block(256 * group);
  const bool gated = a.gate_a != nullptr;
#define GDN_DECODE_CONV_W(WW)                                                                   \
  case WW:                                                                                     \
    if (gated) hipLaunchKernelGGL((k_decode_conv<E, DK, DV, WW, true>), grid, block, 0, st, a, c); \
    else hipLaunchKernelGGL((k_decode_conv<E, DK, DV, WW, false>), grid, block, 0, st, a, c);      \
    break;
  switch (c.width) {
    GDN_DECODE_CONV_W(2)
    GDN_DECODE_CONV_W(3)
    GDN_DECODE_CONV_W(4)
    GDN_DECODE_CONV_W(5)
    GDN_DECODE_CONV_W(6)
    GDN_DECODE_CONV_W(7)
    GDN_DECODE_CONV_W(8)
    default: return hipErrorInvalidValue;
  }
#undef GDN_DECODE_CONV_W
  return hipGetLastError();
}

template <class E>
hipError_t launch_conv_e(const ScanArgs& a, const ConvArgs& c, hipStream_t st) {
  if (a.dk == 128 && a.dv == 128) return launch_conv_dims<E, 128, 128>(a, c, st);
  if (a.dk == 128 && a.dv == 64) return launch_conv_dims<E, 128, 64>(a, c, st);
  if (a.dk == 64 && a.dv == 128) return launch_conv_dims<E, 64, 128>(a, c, st);
  if (a.dk == 64 && a.dv == 64) return launch_conv_dims<E, 64, 64>(a, c, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const ScanArgs& a, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  return a.dtype == 1 ? launch_e<BF16>(a, s) : launch_e<F32>(a, s);
}

hipError_t launch_decode_conv(const ScanArgs& a, const ConvArgs& c, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  return a.dtype == 1 ? launch_conv_e<BF16>(a, c, s) : launch_conv_e<F32>(a, c, s);
}

}  // namespace gdn
