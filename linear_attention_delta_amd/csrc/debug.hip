// debug.hip -- GDN_DEBUG support: count NaN/Inf values in an output buffer,
// a per-stage non-finite probe like the one the oxydllm 0.0.0-alpha.12.2
// notes list under "GDN debug aids".
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__global__ void __launch_bounds__(256) k_nonfinite(const void* p, long n, int dtype, int* count) {
  int bad = 0;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    float v = dtype == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i])
                         : reinterpret_cast<const float*>(p)[i];
    bad += !__builtin_isfinite(v);
  }
  bad = (int)wave_sum((float)bad);
  if ((threadIdx.x & 63) == 0 && bad) atomicAdd(count, bad);
}

}  // namespace

hipError_t launch_nonfinite_probe(const void* p, long n, int dtype, int* count, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_nonfinite, dim3((unsigned)blocks), dim3(256), 0, s, p, n, dtype, count);
  return hipGetLastError();
}

}  // namespace gdn
