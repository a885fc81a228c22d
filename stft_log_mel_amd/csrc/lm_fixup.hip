// Per-clip floor: out = max(out, (hi_b - 8 + 4) / 4) (KBench task page
// "audio-mel-spectrogram-fused", section "spec_md": the floor is per clip,
// at the clip's largest log value minus 8).
//
// The main kernels have already written (L + 4) / 4 for every value and
// recorded the largest mel value per tile and the smallest L per region of
// the tile (a frame range times a band range).  Since (x + 4) / 4 and the
// cast to the output type are both monotone, max(rescale(L), rescale(hi -
// 8)) equals rescale(max(L, hi - 8)); so only regions whose smallest L lies
// below hi - 8 are read, and only values below the floor are rewritten.
// hi is log10 of the largest mel value, with the same log10 the main
// kernels use, so the largest output is exactly (hi + 4) / 4.
#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

constexpr int kFixThreads = 256;
constexpr int kFixWaves = kFixThreads / 64;
constexpr int kFixUnroll = 8;
constexpr int kFixEntries = 512;   // minimum entries one workgroup scans

// Workgroup (clip b, group gi): reduce the clip's maxima to hi (every
// group of the clip does this itself, so no cross-workgroup atomics or
// resets are needed), list the entries of its range whose smallest log
// value lies below hi - 8, then let each wave rewrite listed regions.
template <typename OUT>
__global__ void __launch_bounds__(kFixThreads) clamp_fixup_kernel(FixupArgs a) {
  __shared__ float s_red[kFixWaves];
  __shared__ int s_list[kFixEntries];
  __shared__ int s_n;
  const int G = a.groups_per_clip;
  const int64_t b = blockIdx.x / G;
  const int gi = (int)(blockIdx.x - b * G);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const StatLayout st = a.st;
  const int ept = st.min_per_tile();
  const int n_ent = a.tiles_per_clip * ept, n_max = a.tiles_per_clip * st.max_per_tile;
  const float *cmax = a.tile_max + b * (int64_t)n_max;
  const float *cmin = a.tile_min + b * (int64_t)n_ent;
  if (tid == 0) s_n = 0;
  float hi = 0.0f;
  for (int e = tid; e < n_max; e += kFixThreads) hi = fmaxf(hi, cmax[e]);
  hi = wave_max(hi);
  if (lane == 0) s_red[wv] = hi;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kFixWaves; ++i) hi = fmaxf(hi, s_red[i]);
  const float floorL = log10_pos(fmaxf(hi, 1e-10f)) - 8.0f;
  const int e0 = gi * a.entries_per_group, e1 = min(n_ent, e0 + a.entries_per_group);
  for (int e = e0 + tid; e < e1; e += kFixThreads)
    if (cmin[e] < floorL) s_list[atomicAdd(&s_n, 1)] = e;
  __syncthreads();
  const int n_flag = s_n;
  if (n_flag == 0) return;

  float fo = rescale(floorL);
  if (sizeof(OUT) == 2) fo = __half2float(__float2half_rn(fo));
  OUT *out = reinterpret_cast<OUT *>(a.out);
  const int NM = a.n_mels;
  const int64_t F = a.n_frames;
  const int sub_frames = st.frames_per_tile / st.sub_per_tile;
  for (int i = wv; i < n_flag; i += kFixWaves) {
    const int e = s_list[i];
    const int t = e / ept, rem = e - t * ept;
    const int sub = rem / st.blk_per_sub, blk = rem - sub * st.blk_per_sub;
    const int64_t f0 = (int64_t)t * st.frames_per_tile + (int64_t)sub * sub_frames;
    const int nfr = (int)min((int64_t)sub_frames, F - f0);
    const int m0 = blk * st.band_h, nb = min(st.band_h, NM - m0);
    if (nfr <= 0 || nb <= 0) continue;
    // region: nseg runs of len elements, stride apart, from base
    int64_t base, stride;
    int nseg, len;
    if (a.mel_major) {
      base = (b * NM + m0) * F + f0;
      stride = F;
      nseg = nb;
      len = nfr;
    } else {
      base = (b * F + f0) * NM + m0;
      stride = NM;
      nseg = nfr;
      len = nb;
    }
    const int n = nseg * len;
    for (int i0 = lane; i0 < n; i0 += 64 * kFixUnroll) {
      OUT *p[kFixUnroll];
      float v[kFixUnroll];
#pragma unroll
      for (int u = 0; u < kFixUnroll; ++u) {
        const int k = i0 + u * 64;
        p[u] = nullptr;
        if (k < n) {
          const int sg = k / len;
          p[u] = out + base + sg * stride + (k - sg * len);
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
  const int n_ent = a.tiles_per_clip * a.st.min_per_tile();
  a.entries_per_group = kFixEntries;
  a.groups_per_clip = (n_ent + kFixEntries - 1) / kFixEntries;
  const dim3 grid((unsigned)(a.n_clips * a.groups_per_clip)), block(kFixThreads);
  if (a.out_f16) hipLaunchKernelGGL(clamp_fixup_kernel<__half>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(clamp_fixup_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lm
