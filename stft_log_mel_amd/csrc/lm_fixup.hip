// Per-clip floor: out = max(out, (hi_b - 8 + 4) / 4) (KBench task page
// "audio-mel-spectrogram-fused", section "spec_md": the floor is per clip,
// at the clip's largest log value minus 8).
//
// The main kernels have already written (L + 4) / 4 for every value and
// recorded, per tile or sub-tile, the largest mel value and the smallest L.
// Since (x + 4) / 4 and the cast to the output type are both monotone, max(rescale(L), rescale(hi - 8)) is exactly
// rescale(max(L, hi - 8)); so only tiles whose smallest L lies below
// hi - 8 are read, and only values below the floor are rewritten.  hi is
// log10 of the largest mel value, with the same log10 the main kernels use,
// so the largest output is exactly (hi + 4) / 4.
#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

constexpr int kFixThreads = 256;
constexpr int kFixWaves = kFixThreads / 64;
constexpr int kFixUnroll = 8;
constexpr int kFixMaxGroups = 64;   // workgroups per clip (each reads all of the clip's maxima)

// Statistics hold R entries per tile.  Mel-major output: entry r covers
// every band over the tile's r-th sub-tile of frames_per_tile / R frames
// (R = 1: the whole tile).  Frame-major output: R = 1, the whole tile.
// Workgroup (clip b, group g) first reduces the clip's per-entry maxima to
// the clip maximum hi (so no cross-workgroup atomics or resets are needed:
// every call overwrites all entries), then each of its waves takes entries
// g*EPG + wave, + 4, ... and rewrites the region of any whose smallest log
// value lies below hi - 8.
template <typename OUT>
__global__ void __launch_bounds__(kFixThreads) clamp_fixup_kernel(FixupArgs a) {
  __shared__ float s_red[kFixWaves];
  const int G = a.groups_per_clip, R = a.rows_per_tile, EPG = a.entries_per_group;
  const int64_t b = blockIdx.x / G;
  const int g = (int)(blockIdx.x - b * G);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n_ent = a.tiles_per_clip * R;
  const float *cmax = a.tile_max + b * (int64_t)n_ent;
  const float *cmin = a.tile_min + b * (int64_t)n_ent;
  float hi = 0.0f;
  for (int e = threadIdx.x; e < n_ent; e += kFixThreads) hi = fmaxf(hi, cmax[e]);
  hi = wave_max(hi);
  if (lane == 0) s_red[wv] = hi;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kFixWaves; ++i) hi = fmaxf(hi, s_red[i]);
  const float floorL = log10_pos(fmaxf(hi, 1e-10f)) - 8.0f;
  float fo = rescale(floorL);
  if (sizeof(OUT) == 2) fo = __half2float(__float2half_rn(fo));
  OUT *out = reinterpret_cast<OUT *>(a.out);
  const int NM = a.n_mels;
  const int64_t F = a.n_frames;
  const int e_end = min(n_ent, (g + 1) * EPG);
  for (int e = g * EPG + wv; e < e_end; e += kFixWaves) {
    if (!(cmin[e] < floorL)) continue;
    const int t = e / R, r = e - t * R;
    const int sub = a.frames_per_tile / R;
    const int64_t f0 = (int64_t)t * a.frames_per_tile + (int64_t)r * sub;
    const int nfr = (int)min((int64_t)sub, F - f0);
    // region: nseg runs of len elements, stride apart, from base
    int64_t base, stride = F;
    int nseg, len;
    if (a.mel_major) {
      base = b * NM * F + f0;
      nseg = NM;
      len = nfr;
    } else {
      base = (b * F + f0) * NM;
      nseg = 1;
      len = nfr * NM;
    }
    const int n = nseg * len;
    for (int i0 = lane; i0 < n; i0 += 64 * kFixUnroll) {
      OUT *p[kFixUnroll];
      float v[kFixUnroll];
#pragma unroll
      for (int u = 0; u < kFixUnroll; ++u) {
        const int i = i0 + u * 64;
        p[u] = nullptr;
        if (i < n) {
          const int sg = nseg > 1 ? i / len : 0;
          p[u] = out + base + sg * stride + (i - sg * len);
          v[u] = load_out(p[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kFixUnroll; ++u)
        if (p[u] && v[u] < fo) store_out(p[u], fo);
    }
  }
}

hipError_t launch_fixup(FixupArgs a, hipStream_t s) {
  const int n_ent = a.tiles_per_clip * a.rows_per_tile;
  int epg = (n_ent + kFixMaxGroups - 1) / kFixMaxGroups;
  epg = ((epg + kFixWaves - 1) / kFixWaves) * kFixWaves;
  if (epg < kFixWaves) epg = kFixWaves;
  a.entries_per_group = epg;
  a.groups_per_clip = (n_ent + epg - 1) / epg;
  const dim3 grid((unsigned)(a.n_clips * a.groups_per_clip)), block(kFixThreads);
  if (a.out_f16) hipLaunchKernelGGL(clamp_fixup_kernel<__half>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(clamp_fixup_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lm
