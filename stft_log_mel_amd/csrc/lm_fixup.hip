// Per-clip floor: out = max(out, (hi_b - 8 + 4) / 4) (KBench task page
// "audio-mel-spectrogram-fused", section "spec_md": the floor is per clip,
// at the clip's largest log value minus 8).
//
// The main kernels have already written (L + 4) / 4 for every value and
// recorded, per clip, the largest mel value (hi_bits) and, per tile, the
// smallest L.  Since (x + 4) / 4 and the cast to the output type are both
// monotone, max(rescale(L), rescale(hi - 8)) is exactly
// rescale(max(L, hi - 8)); so only tiles whose smallest L lies below
// hi - 8 are touched, and on typical speech none are.  One workgroup per
// clip; it also clears the clip's maximum for the next call.
#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

constexpr int kFixThreads = 256;

template <typename OUT>
__global__ void __launch_bounds__(kFixThreads) clamp_fixup_kernel(FixupArgs a) {
  __shared__ float s_floor;
  const int64_t b = blockIdx.x;
  if (threadIdx.x == 0) s_floor = log10_pos(__uint_as_float(a.hi_bits[b])) - 8.0f;
  __syncthreads();
  const float floorL = s_floor;
  float fo = rescale(floorL);
  if (sizeof(OUT) == 2) fo = __half2float(__float2half_rn(fo));
  OUT *out = reinterpret_cast<OUT *>(a.out);
  const int NM = a.n_mels;
  const int64_t F = a.n_frames;
  for (int t = 0; t < a.tiles_per_clip; ++t) {
    if (!(a.tile_min[b * a.tiles_per_clip + t] < floorL)) continue;
    const int64_t f0 = (int64_t)t * a.frames_per_tile;
    const int nfr = (int)min((int64_t)a.frames_per_tile, F - f0);
    const int n = nfr * NM;
    for (int i = threadIdx.x; i < n; i += kFixThreads) {
      OUT *p;
      if (a.mel_major) {
        const int m = i / nfr, fl = i - m * nfr;
        p = out + (b * NM + m) * F + f0 + fl;
      } else {
        p = out + (b * F + f0) * NM + i;
      }
      if (load_out(p) < fo) store_out(p, fo);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.hi_bits[b] = 0u;
}

hipError_t launch_fixup(const FixupArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_clips), block(kFixThreads);
  if (a.out_f16) hipLaunchKernelGGL(clamp_fixup_kernel<__half>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(clamp_fixup_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lm
