// Stand-alone clamp fix-up kernel: per clip, one workgroup per unit of
// fixup_group (lm_fixup.h), then one per segment of each band row that the
// main kernel left unwritten (fixup_empty_row).
#include <algorithm>

#include "lm_fixup.h"

namespace lm {

constexpr int kFixThreads = 256;

template <typename OUT>
__global__ void __launch_bounds__(kFixThreads) clamp_fixup_kernel(FixupArgs a) {
  __shared__ float s_red[kFixThreads / 64];
  __shared__ int s_f0[kFixEntries], s_m0[kFixEntries];
  __shared__ int s_n;
  const int G = a.groups_per_clip, U = G + a.n_empty * a.empty_units;
  const int64_t b = blockIdx.x / U;
  const int u = (int)(blockIdx.x - b * U);
  if (u < G) {
    fixup_group<OUT, kFixThreads>(a, b, u, s_f0, s_m0, &s_n, s_red);
  } else {
    const int e = (u - G) / a.empty_units;
    fixup_empty_row<OUT, kFixThreads>(a, b, e, u - G - e * a.empty_units, s_red);
  }
}

hipError_t launch_fixup(FixupArgs a, hipStream_t s, const LaunchTiming *tm) {
  prepare_fixup(a);
  const int64_t units = a.n_clips * ((int64_t)a.groups_per_clip + (int64_t)a.n_empty * a.empty_units);
  if (units > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)units), block(kFixThreads);
  if (a.out_f16) LM_LAUNCH(tm, clamp_fixup_kernel<__half>, grid, block, 0, s, a);
  else LM_LAUNCH(tm, clamp_fixup_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) zero_u64_kernel(uint64_t *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0;
}

hipError_t launch_zero_u64(uint64_t *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_u64_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace lm
