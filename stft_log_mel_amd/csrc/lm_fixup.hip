// Stand-alone clamp fix-up kernel: one workgroup per (clip, group) unit of
// fixup_group (lm_fixup.h).
#include "lm_fixup.h"

namespace lm {

constexpr int kFixThreads = 256;

template <typename OUT>
__global__ void __launch_bounds__(kFixThreads) clamp_fixup_kernel(FixupArgs a) {
  __shared__ float s_red[kFixThreads / 64];
  __shared__ int s_f0[kFixEntries], s_m0[kFixEntries];
  __shared__ int s_n;
  const int G = a.groups_per_clip;
  const int64_t b = blockIdx.x / G;
  fixup_group<OUT, kFixThreads>(a, b, (int)(blockIdx.x - b * G), s_f0, s_m0, &s_n, s_red);
}

hipError_t launch_fixup(FixupArgs a, hipStream_t s, const LaunchTiming *tm) {
  prepare_fixup(a);
  const dim3 grid((unsigned)(a.n_clips * a.groups_per_clip)), block(kFixThreads);
  if (a.out_f16) LM_LAUNCH(tm, clamp_fixup_kernel<__half>, grid, block, 0, s, a);
  else LM_LAUNCH(tm, clamp_fixup_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lm
