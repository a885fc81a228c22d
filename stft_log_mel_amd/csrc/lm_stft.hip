// Complex STFT -> log-mel (KBench task page "audio-mel-spectrogram-fused",
// sections "reference_src", "spec_md", "contract_md", "perf_md").
//
// The source is read exactly once.  A workgroup owns TF consecutive frames
// of one clip; those frames are one contiguous run of TF*NF complex64
// values, streamed with 16-byte non-temporal loads (two bins per load) and
// turned into power re^2 + im^2 straight into an LDS tile.  Each (frame,
// band) output is then the packed triangular mel sum over that tile, log10
// after the 1e-10 floor, (L+4)/4, stored frame-major so a tile's outputs
// are one contiguous run.  The tile's largest mel value and smallest log
// value go to per-tile slots; the clamp fix-up kernel reduces them per clip
// and completes the per-clip floor.
#include <climits>

#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

constexpr int kStftThreads = 256;
constexpr int kStftLoadUnroll = 8;
constexpr int kStftCsrLds = 2048;   // packed weights staged in LDS up to this count

struct StftKernelArgs {
  const float2 *stft;
  int64_t F;
  int NF, NM, TF, tiles_per_clip;
  const int32_t *csr_start, *csr_width, *csr_off;
  const float *csr_w;
  int w_len;
  void *out;
  float *tile_min, *tile_max;
};

__device__ __forceinline__ float pw(float2 v) { return __builtin_fmaf(v.x, v.x, v.y * v.y); }

typedef float v4f __attribute__((ext_vector_type(4)));

template <typename OUT, bool VEC16>
__global__ void __launch_bounds__(kStftThreads) stft_logmel_kernel(StftKernelArgs a) {
  extern __shared__ float s_dyn[];      // [TF*NF power tile][kStftCsrLds weights]
  __shared__ int32_t s_start[256], s_width[256], s_off[256];
  __shared__ float s_red[2 * kStftThreads / 64];

  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t b = tile / a.tiles_per_clip;
  const int t = (int)(tile - b * a.tiles_per_clip);
  const int64_t f0 = (int64_t)t * a.TF;
  const int nfr = (int)min((int64_t)a.TF, a.F - f0);
  const int NF = a.NF, NM = a.NM;
  float *P = s_dyn;
  float *s_w = s_dyn + a.TF * NF;

  // 1. power tile: elements [e0, e0 + n) of the flat complex array
  const int64_t e0 = (b * a.F + f0) * NF;
  const int n = nfr * NF;
  if (VEC16) {
    const int head = (int)(e0 & 1);                  // element e0 is 16-byte aligned iff even
    const int npairs = (n - head) >> 1;
    const v4f *src = reinterpret_cast<const v4f *>(a.stft + e0 + head);
    for (int q0 = tid; q0 < npairs; q0 += kStftLoadUnroll * kStftThreads) {
      v4f v[kStftLoadUnroll];
#pragma unroll
      for (int u = 0; u < kStftLoadUnroll; ++u) {
        const int q = q0 + u * kStftThreads;
        if (q < npairs) v[u] = __builtin_nontemporal_load(src + q);
      }
#pragma unroll
      for (int u = 0; u < kStftLoadUnroll; ++u) {
        const int q = q0 + u * kStftThreads;
        if (q < npairs) {
          P[head + 2 * q] = __builtin_fmaf(v[u].x, v[u].x, v[u].y * v[u].y);
          P[head + 2 * q + 1] = __builtin_fmaf(v[u].z, v[u].z, v[u].w * v[u].w);
        }
      }
    }
    if (tid == 0 && head) P[0] = pw(a.stft[e0]);
    if (tid == kStftThreads - 1 && ((n - head) & 1)) P[n - 1] = pw(a.stft[e0 + n - 1]);
  } else {
    for (int i = tid; i < n; i += kStftThreads) P[i] = pw(a.stft[e0 + i]);
  }

  // packed filterbank -> LDS (ends with a barrier, which also covers the power tile)
  const int nnz = stage_filters<kStftThreads>(NM, a.csr_start, a.csr_width, a.csr_off, a.csr_w, a.w_len, s_start,
                                              s_width, s_off, s_w, kStftCsrLds);
  const bool w_in_lds = nnz <= kStftCsrLds;

  // 2. mel sums, log10, rescale, frame-major store
  OUT *__restrict__ out = reinterpret_cast<OUT *>(a.out) + (b * a.F + f0) * NM;
  float vmax = 0.0f, lmin = __builtin_huge_valf();
  int m = tid % NM, f = tid / NM;
  const int dm = kStftThreads % NM, df = kStftThreads / NM;
  for (int o = tid; o < nfr * NM; o += kStftThreads) {
    const int st = s_start[m], wd = s_width[m];
    const float *pr = P + f * NF + st;
    float acc = 0.0f;
    const float *wr = (w_in_lds ? s_w : a.csr_w) + s_off[m];
    for (int j = 0; j < wd; ++j) acc = __builtin_fmaf(wr[j], pr[j], acc);
    const float v = fmaxf(acc, 1e-10f);
    const float L = log10_pos(v);
    vmax = fmaxf(vmax, v);
    lmin = fminf(lmin, L);
    store_out_nt(out + o, rescale(L));
    m += dm;
    f += df;
    if (m >= NM) {
      m -= NM;
      f += 1;
    }
  }

  // 3. tile statistics
  block_maxmin<kStftThreads>(vmax, lmin, s_red);
  if (tid == 0) {
    a.tile_max[tile] = vmax;
    a.tile_min[tile] = lmin;
  }
}

int stft_frames_per_tile(int n_bins, int n_mels) {
  (void)n_mels;
  int tf = 6144 / n_bins;
  if (tf > 64) tf = 64;
  if (tf < 1) tf = 1;
  return tf;
}

hipError_t launch_stft(const StftArgs &a, hipStream_t s) {
  StftKernelArgs k;
  k.stft = a.stft;
  k.F = a.n_frames;
  k.NF = a.n_bins;
  k.NM = a.n_mels;
  k.TF = a.frames_per_tile;
  k.tiles_per_clip = a.tiles_per_clip;
  k.csr_start = a.csr_start;
  k.csr_width = a.csr_width;
  k.csr_off = a.csr_off;
  k.csr_w = a.csr_w;
  k.w_len = a.w_len;
  k.out = a.out;
  k.tile_min = a.tile_min;
  k.tile_max = a.tile_max;
  const size_t lds = sizeof(float) * ((size_t)a.frames_per_tile * a.n_bins + kStftCsrLds);
  const dim3 grid((unsigned)(a.n_clips * a.tiles_per_clip)), block(kStftThreads);
  const bool vec16 = (reinterpret_cast<uintptr_t>(a.stft) & 15) == 0;
  if (a.out_f16) {
    if (vec16) hipLaunchKernelGGL((stft_logmel_kernel<__half, true>), grid, block, lds, s, k);
    else hipLaunchKernelGGL((stft_logmel_kernel<__half, false>), grid, block, lds, s, k);
  } else {
    if (vec16) hipLaunchKernelGGL((stft_logmel_kernel<float, true>), grid, block, lds, s, k);
    else hipLaunchKernelGGL((stft_logmel_kernel<float, false>), grid, block, lds, s, k);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense (NM, NF) device filterbank -> packed rows (start, width, off, w),
// the same layout as a plan's own table.  One workgroup of 16 waves: each
// wave issues the loads of all its rows at once and reduces each row's
// first and last non-zero; wave 0 lays out the offsets; then each wave
// copies its rows' [first, last] weights.
// ---------------------------------------------------------------------------

constexpr int kPackThreads = 1024;
constexpr int kPackWaves = kPackThreads / 64;
constexpr int kPackRowsPerWave = 256 / kPackWaves;   // NM <= 256

__global__ void __launch_bounds__(kPackThreads)
pack_filters_kernel(const float *__restrict__ dense, int NM, int NF, int32_t *start, int32_t *width,
                    int32_t *off, float *w) {
  __shared__ int s_first[256], s_last[256], s_off[256];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int first[kPackRowsPerWave], last[kPackRowsPerWave];
#pragma unroll
  for (int r = 0; r < kPackRowsPerWave; ++r) {
    first[r] = INT_MAX;
    last[r] = -1;
  }
  for (int k0 = 0; k0 < NF; k0 += 64) {
    const int k = k0 + lane;
    float v[kPackRowsPerWave];
#pragma unroll
    for (int r = 0; r < kPackRowsPerWave; ++r) {
      const int m = wv + r * kPackWaves;
      v[r] = (m < NM && k < NF) ? dense[(size_t)m * NF + k] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < kPackRowsPerWave; ++r)
      if (v[r] != 0.0f) {
        first[r] = min(first[r], k);
        last[r] = max(last[r], k);
      }
  }
#pragma unroll
  for (int r = 0; r < kPackRowsPerWave; ++r) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      first[r] = min(first[r], __shfl_xor(first[r], o, 64));
      last[r] = max(last[r], __shfl_xor(last[r], o, 64));
    }
    const int m = wv + r * kPackWaves;
    if (lane == 0 && m < NM) {
      s_first[m] = first[r];
      s_last[m] = last[r];
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int tid = threadIdx.x;
    int wd[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * tid + i;
      wd[i] = (m < NM && s_last[m] >= 0) ? s_last[m] - s_first[m] + 1 : 0;
      sum += wd[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (tid >= o) incl += t;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * tid + i;
      if (m < NM) {
        s_off[m] = run;
        start[m] = wd[i] ? s_first[m] : 0;
        width[m] = wd[i];
        off[m] = run;
      }
      run += wd[i];
    }
  }
  __syncthreads();
  for (int m = wv; m < NM; m += kPackWaves) {
    if (s_last[m] < 0) continue;
    const int st = s_first[m], wd = s_last[m] - st + 1, o = s_off[m];
    for (int j = lane; j < wd; j += 64) w[o + j] = dense[(size_t)m * NF + st + j];
  }
}

hipError_t launch_pack(const float *dense, int n_mels, int n_bins, void *ws, hipStream_t s) {
  int32_t *start = reinterpret_cast<int32_t *>(ws);
  int32_t *width = start + n_mels;
  int32_t *off = width + n_mels;
  float *w = reinterpret_cast<float *>(off + n_mels);
  hipLaunchKernelGGL(pack_filters_kernel, dim3(1), dim3(kPackThreads), 0, s, dense, n_mels, n_bins, start, width,
                     off, w);
  return hipGetLastError();
}

}  // namespace lm
