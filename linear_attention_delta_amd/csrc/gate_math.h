// gate_math.h -- the per-token gates from the layer's raw projections
// (oxydllm 0.0.0-alpha.12.2 release notes, "Performance": the beta and decay
// projections; "New Features", GGUF qwen35: the decay rate is the negated
// exponential of A_log), shared by the stand-alone gating kernel and the
// kernels that compute the gates where they consume them, so all give the
// same bits:
//   g = -exp(A_log) * softplus(a + dt_bias),  beta = 1 / (1 + exp(-b))
// softplus(x) = max(x, 0) + log1p(e^-|x|): no overflow, no lost tail.
#pragma once

#include "gdn_device.h"

namespace gdn {

__device__ __forceinline__ float gate_decay(float a_raw, float A_log, float dt_bias) {
#pragma clang fp contract(off)
  const float x = a_raw + dt_bias;
  const float sp = fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
  return -expf(A_log) * sp;
}

__device__ __forceinline__ float gate_beta(float b_raw) {
#pragma clang fp contract(off)
  return 1.0f / (1.0f + expf(-b_raw));
}

// g and beta of token t, v-head h from the raw projections in ScanArgs-like
// argument blocks (fields gate_a, gate_b, stride_ga, stride_gb, A_log, dt_bias).
template <class E, class Args>
__device__ __forceinline__ void gates_from_raw(const Args& a, long t, int h, float& g, float& beta) {
  typedef typename E::store_t T;
  g = gate_decay(E::to_f32(reinterpret_cast<const T*>(a.gate_a)[t * a.stride_ga + h]), a.A_log[h], a.dt_bias[h]);
  beta = gate_beta(E::to_f32(reinterpret_cast<const T*>(a.gate_b)[t * a.stride_gb + h]));
}

}  // namespace gdn
