// Complex STFT -> log-mel (KBench task page "audio-mel-spectrogram-fused",
// sections "reference_src", "spec_md", "contract_md", "perf_md").
//
// The source is read exactly once.  A tile is TF consecutive frames of one
// clip; those frames are one contiguous run of TF*NF complex64 values,
// streamed with 16-byte non-temporal loads (two bins per load) and turned
// into power re^2 + im^2 straight into an LDS tile.  Workgroups are
// persistent (a few per compute unit) and take tiles in turn.  Each (frame,
// band) output is then the packed triangular mel sum over that tile, log10
// after the 1e-10 floor, (L+4)/4, stored frame-major so a tile's outputs
// are one contiguous run.  The tile's largest and smallest mel values go to
// per-tile slots; the clamp fix-up kernel reduces them per clip
// and completes the per-clip floor.
#include <climits>

#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

// Workgroup size: 256 threads, four resident per CU, when the call has at
// least that many tiles (the streaming regime: 300 us at 256 threads
// against 350 us at 512 on 256 clips); 512 threads when fewer tiles than
// that (latency-bound: a one-clip call's kernel takes 7.5 us instead of
// 10 us at 256).
constexpr int kStftThreadsBig = 256, kStftThreadsSmall = 512;
constexpr int kStftLoadUnroll = 8;
constexpr int kStftWLds = 2048;     // LDS floats for the staged filter weights
constexpr int kStftWgPerCu = 4;     // resident workgroups per compute unit
constexpr int kStftMinTile = 4;     // frames per tile at least

struct StftKernelArgs {
  const float2 *stft;
  int64_t F;
  int NF, NM, TF, tiles_per_clip;
  int64_t n_tiles;
  const int32_t *f_start, *f_width, *f_off;
  const float *f_w;
  int f_stride;
  void *out;
  int mel_out;   // 1: store the mel values themselves (no log tail)
  float *tile_min, *tile_max;
};

__device__ __forceinline__ float pw(float2 v) { return __builtin_fmaf(v.x, v.x, v.y * v.y); }

typedef float v4f __attribute__((ext_vector_type(4)));

// One tile: power of TF frames into P (LDS), then the mel sums, log10,
// rescale, frame-major store and the tile's statistics.  `wsrc` + s_off[m]
// is band m's first weight, in LDS or in global memory.
template <typename OUT, bool VEC16, int kStftThreads>
__device__ __forceinline__ void stft_tile(const StftKernelArgs &a, int64_t tile, float *P, const float *wsrc,
                                          const int32_t *s_start, const int32_t *s_width, const int32_t *s_off,
                                          float *s_red) {
  const int tid = threadIdx.x;
  const int64_t b = tile / a.tiles_per_clip;
  const int t = (int)(tile - b * a.tiles_per_clip);
  const int64_t f0 = (int64_t)t * a.TF;
  const int nfr = (int)min((int64_t)a.TF, a.F - f0);
  const int NF = a.NF, NM = a.NM;

  // 1. power tile: elements [e0, e0 + n) of the flat complex array.  The
  //    workgroups of a CU are at different phases; the one issuing its
  //    loads goes first (wave priority 1 here, 0 for the mel sums below), so
  //    more of the CU's loads are in flight at a time (256-clip batch: main
  //    kernel 300.0 -> 293.5 us)
  __builtin_amdgcn_s_setprio(1);
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
  __syncthreads();

  // 2. mel sums, log10, rescale, frame-major store
  __builtin_amdgcn_s_setprio(0);
  OUT *__restrict__ out = reinterpret_cast<OUT *>(a.out) + (b * a.F + f0) * NM;
  float vmax = 0.0f, vmin = __builtin_huge_valf();
  int m = tid % NM, f = tid / NM;
  const int dm = kStftThreads % NM, df = kStftThreads / NM;
  for (int o = tid; o < nfr * NM; o += kStftThreads) {
    const int st = s_start[m], wd = s_width[m];
    const float *pr = P + f * NF + st;
    const float *wr = wsrc + s_off[m];
    float acc = 0.0f;
    for (int j = 0; j < wd; ++j) acc = __builtin_fmaf(wr[j], pr[j], acc);
    if (a.mel_out) {
      store_out_nt(out + o, acc);
    } else {
      const float v = fmaxf(acc, 1e-10f);
      const float ov = logmel_of(v);
      vmax = fmaxf(vmax, v);
      vmin = fminf(vmin, v);
      store_out_nt(out + o, ov);
    }
    m += dm;
    f += df;
    if (m >= NM) {
      m -= NM;
      f += 1;
    }
  }

  // 3. tile statistics (the barrier inside also ends every read of P)
  block_maxmin<kStftThreads>(vmax, vmin, s_red);
  if (tid == 0) {
    a.tile_max[tile] = vmax;
    a.tile_min[tile] = vmin;
  }
  __syncthreads();
}

// Persistent: each workgroup stages the filter rows once, then takes tiles
// blockIdx.x, + gridDim.x, ...
template <typename OUT, bool VEC16, int kStftThreads>
__global__ void __launch_bounds__(kStftThreads) stft_logmel_kernel(StftKernelArgs a) {
  constexpr int kStftNW = kStftThreads / 64;
  extern __shared__ float s_dyn[];      // [TF*NF power tile][kStftWLds weights]
  __shared__ int32_t s_start[256], s_width[256], s_off[256];
  __shared__ int32_t s_scan[kStftNW];
  __shared__ float s_red[2 * kStftNW];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int NM = a.NM;
  float *P = s_dyn;
  float *s_w = s_dyn + a.TF * a.NF;

  // filter rows: start, width; offsets by a block scan of the widths (NM <= 256 = threads)
  int st = 0, wd = 0;
  if (tid < NM) {
    st = a.f_start[tid];
    wd = a.f_width[tid];
  }
  int incl = wd;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_scan[wv] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kStftNW; ++w) {
    const int v = s_scan[w];
    if (w < wv) base += v;
    total += v;
  }
  const bool in_lds = total <= kStftWLds;
  int src = 0, off = 0;
  if (tid < NM) {
    src = a.f_stride ? tid * a.f_stride + st : a.f_off[tid];
    off = base + incl - wd;
    s_start[tid] = st;
    s_width[tid] = wd;
    s_off[tid] = in_lds ? off : src;
  }
  if (in_lds) {
    // a row's weights kCopy at a time with their loads in flight together
    constexpr int kCopy = 8;
    for (int j0 = 0; j0 < wd; j0 += kCopy) {
      float v[kCopy];
#pragma unroll
      for (int u = 0; u < kCopy; ++u) v[u] = j0 + u < wd ? a.f_w[src + j0 + u] : 0.0f;
#pragma unroll
      for (int u = 0; u < kCopy; ++u)
        if (j0 + u < wd) s_w[off + j0 + u] = v[u];
    }
  }
  __syncthreads();

  // one copy of the tile loop per weight source (see stft_tile)
  if (in_lds) {
    for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x)
      stft_tile<OUT, VEC16, kStftThreads>(a, tile, P, s_w, s_start, s_width, s_off, s_red);
  } else {
    for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x)
      stft_tile<OUT, VEC16, kStftThreads>(a, tile, P, a.f_w, s_start, s_width, s_off, s_red);
  }
}

int stft_frames_per_tile(int n_bins, int n_mels, int64_t total_frames, int n_cu) {
  (void)n_mels;
  int tf = 6144 / n_bins;
  if (tf > 64) tf = 64;
  if (tf < 1) tf = 1;
  // a call with fewer tiles than resident workgroups runs one workgroup per
  // tile and is latency-bound: smaller tiles, about one per CU, spread it
  // over more of the chip
  if (n_cu > 0 && (total_frames + tf - 1) / tf < (int64_t)n_cu * kStftWgPerCu) {
    const int64_t per_cu = (total_frames + n_cu - 1) / n_cu;
    if (per_cu < tf) tf = (int)(per_cu < kStftMinTile ? kStftMinTile : per_cu);
  }
  return tf;
}

hipError_t launch_stft(const StftArgs &a, hipStream_t s, const LaunchTiming *tm) {
  StftKernelArgs k;
  k.stft = a.stft;
  k.F = a.n_frames;
  k.NF = a.n_bins;
  k.NM = a.n_mels;
  k.TF = a.frames_per_tile;
  k.tiles_per_clip = a.tiles_per_clip;
  k.n_tiles = a.n_clips * a.tiles_per_clip;
  k.f_start = a.f_start;
  k.f_width = a.f_width;
  k.f_off = a.f_off;
  k.f_w = a.f_w;
  k.f_stride = a.f_stride;
  k.out = a.out;
  k.mel_out = a.mel_out;
  k.tile_min = a.tile_min;
  k.tile_max = a.tile_max;
  const size_t lds = sizeof(float) * ((size_t)a.frames_per_tile * a.n_bins + kStftWLds);
  const int64_t cap = (int64_t)a.n_cu * kStftWgPerCu;
  const bool small = k.n_tiles < cap;
  const dim3 grid((unsigned)(small ? k.n_tiles : cap)), block(small ? kStftThreadsSmall : kStftThreadsBig);
  const bool vec16 = (reinterpret_cast<uintptr_t>(a.stft) & 15) == 0;
#define LM_STFT(OUT, V, T) LM_LAUNCH(tm, (stft_logmel_kernel<OUT, V, T>), grid, block, lds, s, k)
  if (small) {
    if (a.out_f16) {
      if (vec16) LM_STFT(__half, true, kStftThreadsSmall);
      else LM_STFT(__half, false, kStftThreadsSmall);
    } else {
      if (vec16) LM_STFT(float, true, kStftThreadsSmall);
      else LM_STFT(float, false, kStftThreadsSmall);
    }
  } else {
    if (a.out_f16) {
      if (vec16) LM_STFT(__half, true, kStftThreadsBig);
      else LM_STFT(__half, false, kStftThreadsBig);
    } else {
      if (vec16) LM_STFT(float, true, kStftThreadsBig);
      else LM_STFT(float, false, kStftThreadsBig);
    }
  }
#undef LM_STFT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense (NM, NF) device filterbank -> per-row first non-zero bin and width
// (0 for an all-zero row).  One wave per row; the weights stay in the dense
// matrix, which the STFT kernel reads at row m * NF + start[m].
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) filter_rows_kernel(const float *__restrict__ dense, int NM, int NF,
                                                          int32_t *start, int32_t *width) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= NM) return;
  const float *row = dense + (size_t)m * NF;
  int first = INT_MAX, last = -1;
  for (int k0 = 0; k0 < NF; k0 += 256) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + 64 * u + lane;
      v[u] = k < NF ? row[k] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (v[u] != 0.0f) {
        first = min(first, k0 + 64 * u + lane);
        last = max(last, k0 + 64 * u + lane);
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    first = min(first, __shfl_xor(first, o, 64));
    last = max(last, __shfl_xor(last, o, 64));
  }
  if (lane == 0) {
    start[m] = last >= 0 ? first : 0;
    width[m] = last >= 0 ? last - first + 1 : 0;
  }
}

hipError_t launch_pack(const float *dense, int n_mels, int n_bins, int32_t *start_width, hipStream_t s,
                       const LaunchTiming *tm) {
  LM_LAUNCH(tm, filter_rows_kernel, dim3((unsigned)((n_mels + 3) / 4)), dim3(256), 0, s, dense, n_mels, n_bins,
                     start_width, start_width + n_mels);
  return hipGetLastError();
}

}  // namespace lm
