// Per-clip floor: out = max(out, (hi_b - 8 + 4) / 4) (KBench task page
// "audio-mel-spectrogram-fused", section "spec_md": the floor is per clip,
// at the clip's largest log value minus 8).
//
// The main kernels have already written (L + 4) / 4 for every value and
// recorded, per clip, the largest mel value (hi_bits) and, per tile, the
// smallest L.  Since (x + 4) / 4 and the cast to the output type are both
// monotone, max(rescale(L), rescale(hi - 8)) is exactly
// rescale(max(L, hi - 8)); so only tiles whose smallest L lies below
// hi - 8 are read, and only values below the floor are rewritten.
#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

constexpr int kFixThreads = 256;
constexpr int kFixUnroll = 8;
constexpr int kFixEntries = 2048;   // minimum entries scanned per workgroup

// tile_min holds R entries per tile: R == 1, the smallest log value of the
// whole tile; R > 1 (mel-major output only), entry r covers the band rows
// m = r, r + R, r + 2R, ... of the tile (each a contiguous run of the
// tile's frames).  Workgroup (clip b, group g) scans a group of tiles'
// entries in parallel, lists those below the floor, and rewrites the listed
// regions with unrolled loads.  The last workgroup of a clip to finish (an
// agent-scope acq_rel counter) clears the clip's maximum and the counter,
// so both are zero for the next call.
template <typename OUT>
__global__ void __launch_bounds__(kFixThreads) clamp_fixup_kernel(FixupArgs a) {
  __shared__ float s_floor;
  __shared__ int s_n, s_list[kFixEntries];
  const int G = a.groups_per_clip, R = a.rows_per_tile;
  const int64_t b = blockIdx.x / G;
  const int g = (int)(blockIdx.x - b * G);
  const int t0 = g * a.tiles_per_group;
  const int t1 = min(a.tiles_per_clip, t0 + a.tiles_per_group);
  const int n_ent = (t1 - t0) * R;                        // <= kFixEntries
  const float *tmin = a.tile_min + (b * a.tiles_per_clip + t0) * (int64_t)R;
  float mins[kFixEntries / kFixThreads];
#pragma unroll
  for (int u = 0; u < kFixEntries / kFixThreads; ++u) {
    const int e = threadIdx.x + u * kFixThreads;
    mins[u] = e < n_ent ? tmin[e] : __builtin_huge_valf();
  }
  if (threadIdx.x == 0) {
    const uint32_t bits = __hip_atomic_load(a.hi_bits + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_floor = log10_pos(__uint_as_float(bits)) - 8.0f;
    s_n = 0;
  }
  __syncthreads();
  const float floorL = s_floor;
#pragma unroll
  for (int u = 0; u < kFixEntries / kFixThreads; ++u)
    if (mins[u] < floorL) s_list[atomicAdd(&s_n, 1)] = threadIdx.x + u * kFixThreads;
  __syncthreads();
  const int nflag = s_n;
  float fo = rescale(floorL);
  if (sizeof(OUT) == 2) fo = __half2float(__float2half_rn(fo));
  OUT *out = reinterpret_cast<OUT *>(a.out);
  const int NM = a.n_mels;
  const int64_t F = a.n_frames;
  for (int q = 0; q < nflag; ++q) {
    const int e = s_list[q];
    const int t = t0 + e / R, row = e % R;
    const int64_t f0 = (int64_t)t * a.frames_per_tile;
    const int nfr = (int)min((int64_t)a.frames_per_tile, F - f0);
    // region: `nseg` runs of `len` elements, `stride` apart, from `base`
    int64_t base, stride = F;
    int nseg, len;
    if (R > 1) {
      base = (b * NM + row) * F + f0;
      stride = (int64_t)R * F;
      nseg = (NM - row + R - 1) / R;
      len = nfr;
    } else if (a.mel_major) {
      base = b * NM * F + f0;
      nseg = NM;
      len = nfr;
    } else {
      base = (b * F + f0) * NM;
      nseg = 1;
      len = nfr * NM;
    }
    const int n = nseg * len;
    for (int i0 = threadIdx.x; i0 < n; i0 += kFixThreads * kFixUnroll) {
      OUT *p[kFixUnroll];
      float v[kFixUnroll];
#pragma unroll
      for (int u = 0; u < kFixUnroll; ++u) {
        const int i = i0 + u * kFixThreads;
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
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.done + b, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (uint32_t)(G - 1)) {
      __hip_atomic_store(a.hi_bits + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.done + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_fixup(FixupArgs a, hipStream_t s) {
  const int R = a.rows_per_tile;
  // about 8 to 16 entries per workgroup: flagged entries are rewritten one after the other
  a.tiles_per_group = R == 1 ? 16 : (8 / R > 0 ? 8 / R : 1);
  a.groups_per_clip = (a.tiles_per_clip + a.tiles_per_group - 1) / a.tiles_per_group;
  const dim3 grid((unsigned)(a.n_clips * a.groups_per_clip)), block(kFixThreads);
  if (a.out_f16) hipLaunchKernelGGL(clamp_fixup_kernel<__half>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(clamp_fixup_kernel<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace lm
