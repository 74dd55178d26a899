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
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr float kL2Eps = 1e-6f;

template <class E>
__device__ __forceinline__ float load_elem(const void* p, long i) {
  return E::to_f32(reinterpret_cast<const typename E::store_t*>(p)[i]);
}

template <class E, int DK, int DV>
__global__ void __launch_bounds__(256) k_decode(ScanArgs a) {
  constexpr int CG = DV / 4;      // 4-column groups
  constexpr int RG = 256 / CG;    // row groups
  constexpr int RPT = DK / RG;    // rows per thread
  static_assert(RPT >= 1 && RG * RPT == DK, "shape");
  const int h = blockIdx.x % a.hv;
  const int b = blockIdx.x / a.hv;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int lane = tid & 63, wave = wave_id();

  const int slot = a.state_slots ? a.state_slots[b] : b;
  if (slot < 0 || slot >= a.num_slots) {  // bad slot: flag the output, leave every state alone
    typedef typename E::store_t T;
    if (tid < DV) reinterpret_cast<T*>(a.o)[((long)b * a.hv + h) * DV + tid] = E::from_f32(__builtin_nanf(""));
    return;
  }
  float* S = a.state + ((long)slot * a.hv + h) * (DK * DV);

  // stream the state in first: every load is independent
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; m++)
    s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rg + m * RG) * DV + 4 * cg));

  __shared__ float ks[DK], qs[DK];
  __shared__ float part[4][3];
  __shared__ f32x4 red[RG][CG][2];

  const int hk = a.tiled ? (h % a.hk) : (h / (a.hv / a.hk));
  float kv_ = 0.f, qv_ = 0.f;
  if (tid < DK) {
    kv_ = load_elem<E>(a.k, (long)b * a.stride_k + (long)hk * DK + tid);
    qv_ = load_elem<E>(a.q, (long)b * a.stride_q + (long)hk * DK + tid);
    ks[tid] = kv_;
    qs[tid] = qv_;
  }
  float kk = wave_sum(kv_ * kv_), qq = wave_sum(qv_ * qv_), kq = wave_sum(kv_ * qv_);
  if (lane == 0) {
    part[wave][0] = kk;
    part[wave][1] = qq;
    part[wave][2] = kq;
  }
  const float g = a.g[(long)b * a.hv + h];
  const float beta = a.beta[(long)b * a.hv + h];
  float vv[4];
#pragma unroll
  for (int j = 0; j < 4; j++) vv[j] = load_elem<E>(a.v, (long)b * a.stride_v + (long)h * DV + 4 * cg + j);
  lds_barrier();
  kk = part[0][0] + part[1][0] + part[2][0] + part[3][0];
  qq = part[0][1] + part[1][1] + part[2][1] + part[3][1];
  kq = part[0][2] + part[1][2] + part[2][2] + part[3][2];
  const float rk = a.l2norm ? 1.0f / sqrtf(kk + kL2Eps) : 1.0f;
  const float rq = a.scale * (a.l2norm ? 1.0f / sqrtf(qq + kL2Eps) : 1.0f);
  const float alpha = expf(g);

  // partial column sums over this thread's rows (raw q, k; scaled below)
  f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; m++) {
    const int i = rg + m * RG;
    pk += s[m] * ks[i];
    pq += s[m] * qs[i];
  }
  red[rg][cg][0] = pk;
  red[rg][cg][1] = pq;
  lds_barrier();
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RG; r++) {
    sk += red[r][cg][0];
    sq += red[r][cg][1];
  }
  const float khq = kq * rk * rq;  // k_hat . q_hat
  f32x4 u, o;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    u[j] = beta * (vv[j] - alpha * rk * sk[j]);
    o[j] = alpha * rq * sq[j] + khq * u[j];
  }
  if (rg == 0) {
    typedef typename E::store_t T;
    T* op = reinterpret_cast<T*>(a.o) + ((long)b * a.hv + h) * DV + 4 * cg;
#pragma unroll
    for (int j = 0; j < 4; j++) op[j] = E::from_f32(o[j]);
  }
#pragma unroll
  for (int m = 0; m < RPT; m++) {
    const int i = rg + m * RG;
    f32x4 nv = alpha * s[m] + (rk * ks[i]) * u;
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + i * DV + 4 * cg));
  }
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

}  // namespace

hipError_t launch_decode(const ScanArgs& a, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  return a.dtype == 1 ? launch_e<BF16>(a, s) : launch_e<F32>(a, s);
}

}  // namespace gdn
