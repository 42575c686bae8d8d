// Range check of the gated delta rule's gates (a debugging aid): counts the
// (b, t, h) whose decay alpha lies outside (0, 1] or whose write strength
// beta lies outside [0, beta_max] (NaN counts as outside).  In the Kairos
// paper (arXiv 2606.16533, HTML v3) both gates are sigmoids (Sec. 2.2.1,
// Eq. 1 and Eq. 4), and the long-horizon bound (Sec. 2.3.2, Remark 2, Eq. 18)
// rests on the update being a contraction, which holds for alpha <= 1 and,
// with unit keys, 0 <= beta <= 1; the kernels also take log2 alpha, which
// needs alpha > 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace kairos {

__global__ __launch_bounds__(64) void zero_count_kernel(uint32_t* count) {
  if (threadIdx.x == 0) *count = 0u;
}

__global__ __launch_bounds__(256) void gate_range_count_kernel(const float* __restrict__ alpha,
                                                               const float* __restrict__ beta, long n,
                                                               float beta_max, uint32_t* count) {
  uint32_t bad = 0;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const float a = alpha[i], b = beta[i];
    bad += (!(a > 0.f && a <= 1.f) || !(b >= 0.f && b <= beta_max)) ? 1u : 0u;
  }
  // wave sum, then one atomic per wave that saw a value out of range
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_down(bad, off, 64);
  if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(count, bad);
}

hipError_t launch_gate_check(const float* alpha, const float* beta, long n, float beta_max, uint32_t* count,
                             hipStream_t stream) {
  zero_count_kernel<<<1, 64, 0, stream>>>(count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  const long blocks = std::min<long>((n + 255) / 256, 2048);
  gate_range_count_kernel<<<(unsigned)blocks, 256, 0, stream>>>(alpha, beta, n, beta_max, count);
  return hipGetLastError();
}

}  // namespace kairos
