// gating.hip -- the per-token gates of the layer from its small raw
// projections (oxydllm 0.0.0-alpha.12.2 release notes, "Performance": the
// beta and decay projections; "New Features", GGUF qwen35: the per-head
// decay rate is the negated exponential of A_log, and the scalar parameters
// stay fp32).  Per token t and v-head h:
//   g    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])
//   beta = 1 / (1 + exp(-b[t][h]))
// (gate_math.h).  One thread per (t, h); the work is a few transcendental
// functions per 8-12 bytes, so a launch is all it costs: the prefill and the
// decode step can compute the gates where they read them instead.
#include "gate_math.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <class E>
__global__ void __launch_bounds__(256) k_gating(GatingArgs a) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.rows * a.heads) return;
  const long t = i / a.heads;
  const int h = (int)(i % a.heads);
  gates_from_raw<E>(a, t, h, a.g[i], a.beta[i]);
}

}  // namespace

hipError_t launch_gating(const GatingArgs& a, hipStream_t s) {
  const long n = a.rows * a.heads;
  if (n == 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (a.dtype == 1) hipLaunchKernelGGL((k_gating<BF16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_gating<F32>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
