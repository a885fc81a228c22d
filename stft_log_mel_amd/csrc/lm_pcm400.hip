// PCM -> log-mel for n_fft = 400 (the speech front end: 25 ms frames at
// 16 kHz), using the matrix cores for the first FFT stage.
//
// Chain per frame (flashmel page, "How it works"; KBench task page
// "audio-mel-spectrogram-fused", "spec_md"):
//   fold the 400 windowed samples to z[n] = w[2n]x[2n] + i w[2n+1]x[2n+1],
//   n < 200; 200 = 25 * 8 with n = n1 + 25 n2 and bin k = 8 k1 + k2:
//     Z[8 k1 + k2] = sum_n1 W25^(n1 k1) [ sum_n2 z[n1+25n2] W200^(k2 (n1+25n2)) ]
//   The inner bracket (window, 8-point DFT and twiddle) is, for each n1, one
//   real 16x16 matrix applied to 16 frames at once on the matrix cores
//   (v_mfma_f32_16x16x4f32, four per n1).  Its output layout leaves lane
//   (frame c, group g) with two whole frequency classes k2 over all n1, so
//   the 25-point DFTs over n1 run in registers (5 x 5, Winograd 5-point
//   modules).  The classes are paired (1,7), (2,6), (3,5), (0,4) so that
//   the split into the real spectrum,
//     2 X[k] = (Z[k] + Z*[200-k]) - i W400^k (Z[k] - Z*[200-k]),
//   needs only the lane's own registers.  |X|^2 goes to an LDS power tile
//   (row stride 201, odd), then each wave forms 1/4 of the mel bands for all
//   64 frames of the tile: packed filter weights are wave-uniform (scalar
//   loads), 64 consecutive frames make one 256-byte store per band
//   (mel-major output), log10 after the 1e-10 floor, (L+4)/4.
// Each wave's largest mel value and smallest log value go to per-sub-tile
// slots; the clamp fix-up kernel reduces them per clip and finishes the
// per-clip floor.
#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTileFrames = 64;               // frames per workgroup
constexpr int kThreads = 256;                 // 4 waves, 16 frames each in the FFT
constexpr int kRow = 201;                     // power-tile row stride (odd: no bank conflicts)
constexpr int kLdsFloats = kTileFrames * kRow;
constexpr int kMelWLds = 4096;                // blocked filter weights staged in LDS up to this count

// compile-time cos/sin of 2 pi j / N for N a multiple of 8 (octant reduction
// in integers, Taylor series on [0, pi/4]); evaluated in double, rounded once
constexpr double kPi = 3.14159265358979323846264338327950288;
constexpr double ct_sin(double x) {
  double t = x, s = x;
  for (int i = 1; i < 14; ++i) {
    t *= -x * x / ((2.0 * i) * (2.0 * i + 1));
    s += t;
  }
  return s;
}
constexpr double ct_cos(double x) {
  double t = 1, s = 1;
  for (int i = 1; i < 14; ++i) {
    t *= -x * x / ((2.0 * i - 1) * (2.0 * i));
    s += t;
  }
  return s;
}
struct Cs {
  double c, s;
};
constexpr Cs cs2pi(long j, long N) {
  j = ((j % N) + N) % N;
  double ss = 1, sc = 1;
  if (2 * j > N) {
    j = N - j;
    ss = -1;
  }
  if (4 * j > N) {
    j = N / 2 - j;
    sc = -1;
  }
  Cs r{0, 0};
  if (8 * j > N) {
    const double a = 2 * kPi * (double)(N / 4 - j) / (double)N;
    r = {ct_sin(a), ct_cos(a)};
  } else {
    const double a = 2 * kPi * (double)j / (double)N;
    r = {ct_cos(a), ct_sin(a)};
  }
  return {sc * r.c, ss * r.s};
}
// exp(-2 pi i j / N) as float2
template <int N>
struct Wtab {
  float c[N], s[N];
  constexpr Wtab() : c(), s() {
    for (int j = 0; j < N; ++j) {
      const Cs v = cs2pi(j, N);
      c[j] = (float)v.c;
      s[j] = (float)-v.s;
    }
  }
};
constexpr Wtab<400> kW400{};

__device__ __forceinline__ float2 w400(int j) { return make_float2(kW400.c[j], kW400.s[j]); }
__device__ __forceinline__ float2 w25(int j) { return w400(16 * (j % 25)); }

// 25-point DFT of a[n1], n1 = p + 5q, as 5-point transforms over q, the
// twiddle W25^(p u), then 5-point transforms over p: out[u + 5 v].
__device__ __forceinline__ void dft25(float2 (&a)[25]) {
  float2 c[5][5];
#pragma unroll
  for (int p = 0; p < 5; ++p) {
    float2 t[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) t[q] = a[p + 5 * q];
    dft5(t);
#pragma unroll
    for (int u = 0; u < 5; ++u) c[p][u] = (p && u) ? cmul(t[u], w25(p * u)) : t[u];
  }
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    float2 t[5];
#pragma unroll
    for (int p = 0; p < 5; ++p) t[p] = c[p][u];
    dft5(t);
#pragma unroll
    for (int v = 0; v < 5; ++v) a[u + 5 * v] = t[v];
  }
}

struct Args {
  const void *pcm;
  int64_t T, F;
  int tiles_per_clip;
  int hop, pad, pad_mode;
  float power, mel_scale, pre_scale;
  int n_mels, n_melblk;
  const v4f *amat;   // [25][64] operand table of the matrix-core stage
  void *out;
  float *tile_max;
  int melw_lds;   // blocked filter weights staged in LDS (count <= kMelWLds), else 0
};

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(int16_t v) { return (float)(int)v; }

template <typename IN>
__device__ __forceinline__ float padded(const IN *__restrict__ x, int64_t j, int64_t T, int mode) {
  if (j < 0 || j >= T) {
    if (mode == LM_PAD_CONSTANT) return 0.0f;
    if (mode == LM_PAD_REFLECT) j = j < 0 ? -j : 2 * (T - 1) - j;
    else if (mode == LM_PAD_REPLICATE) j = j < 0 ? 0 : T - 1;
    else j = ((j % T) + T) % T;
  }
  return to_f(x[j]);
}

// LDS layout of the staged span, in dwords: int16 sample pairs with one
// pad dword after every 32, or float samples with two pad dwords after every
// 64 (sample pairs stay 8-byte aligned).  Frame starts are multiples of
// hop/2 (or hop) dwords, which would put the 16 frames a wave reads at once
// on two banks; the padding spreads them over all of them.
template <typename IN>
__device__ __forceinline__ int skew(int d) {
  return sizeof(IN) == 2 ? d + (d >> 5) : d + 2 * (d >> 6);
}

constexpr int kStageUnroll = 4;

// Stage samples [s_begin, s_begin + span) of the clip (padding resolved by
// index; positions past the end of the clip's last frame read as 0) into
// LDS as dwords.  Interior spans with a 16-byte aligned start are copied
// with 16-byte loads, kStageUnroll in flight per thread.
template <typename IN>
__device__ __forceinline__ void stage_span(const IN *__restrict__ x, int64_t T, int64_t s_begin, int span,
                                           int64_t s_limit, int mode, uint32_t *lds) {
  const int tid = threadIdx.x;
  constexpr int PER_DW = 4 / sizeof(IN);                 // samples per dword
  const int ndw = span / PER_DW;                          // span is a multiple of PER_DW
  const IN *src = x + s_begin;
  const bool interior = s_begin >= 0 && s_begin + span <= T;
  if (interior && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4 *s4 = reinterpret_cast<const u4 *>(src);
    const int n4 = ndw >> 2;
    for (int q0 = tid; q0 < n4; q0 += kStageUnroll * kThreads) {
      u4 v[kStageUnroll];
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u)
        if (q0 + u * kThreads < n4) v[u] = s4[q0 + u * kThreads];
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u)
        if (q0 + u * kThreads < n4) {
          uint32_t *dst = lds + skew<IN>(4 * (q0 + u * kThreads));   // 4 dwords never straddle a pad
          dst[0] = v[u].x;
          dst[1] = v[u].y;
          dst[2] = v[u].z;
          dst[3] = v[u].w;
        }
    }
    const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
    for (int d = 4 * n4 + tid; d < ndw; d += kThreads) lds[skew<IN>(d)] = s32[d];
  } else if (interior && (reinterpret_cast<uintptr_t>(src) & 3) == 0) {
    const uint32_t *s32 = reinterpret_cast<const uint32_t *>(src);
    for (int d0 = tid; d0 < ndw; d0 += kStageUnroll * kThreads) {
      uint32_t v[kStageUnroll];
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u)
        if (d0 + u * kThreads < ndw) v[u] = s32[d0 + u * kThreads];
#pragma unroll
      for (int u = 0; u < kStageUnroll; ++u)
        if (d0 + u * kThreads < ndw) lds[skew<IN>(d0 + u * kThreads)] = v[u];
    }
  } else {
    for (int d = tid; d < ndw; d += kThreads) {
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < PER_DW; ++e) {
        const int64_t j = s_begin + (int64_t)d * PER_DW + e;
        const float v = j < s_limit ? padded(x, j, T, mode) : 0.0f;
        if (sizeof(IN) == 2) w |= (uint32_t)(uint16_t)(int16_t)(int)v << (16 * e);
        else w = __float_as_uint(v);
      }
      lds[skew<IN>(d)] = w;
    }
  }
}

template <typename IN, typename OUT>
__global__ void __launch_bounds__(kThreads, 2)
pcm400_kernel(Args a, const int32_t *__restrict__ melblk_meta, const float *__restrict__ melblk_w,
              OUT *__restrict__ out_base, float *__restrict__ tile_min) {
  // staged span, then the power tile; 4 zero floats after it are read (with
  // weight 0) by a filter chunk that runs past the last frame's row
  __shared__ __attribute__((aligned(16))) float s_lds[kLdsFloats + 4];
  __shared__ float s_melw[kMelWLds];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int64_t tile = blockIdx.x;
  const int64_t b = tile / a.tiles_per_clip;
  const int64_t f0 = (tile - b * a.tiles_per_clip) * (int64_t)kTileFrames;
  const int64_t T = a.T, F = a.F;
  const int hop = a.hop;
  const IN *__restrict__ x = reinterpret_cast<const IN *>(a.pcm) + b * T;

  // 1. the tile's sample span into LDS
  const int64_t s_begin = f0 * hop - a.pad;
  const int span = (kTileFrames - 1) * hop + 400;
  const int64_t s_limit = (F - 1) * (int64_t)hop - a.pad + 400;   // end of the last frame of the clip
  if (tid < 4) s_lds[kLdsFloats + tid] = 0.0f;
  for (int i = tid; i < a.melw_lds; i += kThreads) s_melw[i] = melblk_w[i];
  stage_span<IN>(x, T, s_begin, span, s_limit, a.pad_mode, reinterpret_cast<uint32_t *>(s_lds));
  __syncthreads();

  // 2. window + 8-point DFT + twiddle on the matrix cores: D[n1] = M_n1 * B_n1
  const int c = lane & 15, g = lane >> 4;
  const int fl = 16 * wv + c;                   // frame within the tile
  v4f D[25];
#pragma unroll
  for (int n1 = 0; n1 < 25; ++n1) {
    const int s0 = fl * hop + 2 * n1 + 50 * g;  // samples s0, s0+1 (n2 = g) and s0+200, s0+201 (n2 = g+4)
    float xe0, xo0, xe1, xo1;
    if (sizeof(IN) == 2) {
      const uint32_t *d32 = reinterpret_cast<const uint32_t *>(s_lds);
      const uint32_t p0 = d32[skew<IN>(s0 >> 1)], p1 = d32[skew<IN>((s0 >> 1) + 100)];
      xe0 = (float)(int16_t)(p0 & 0xffffu);
      xo0 = (float)((int32_t)p0 >> 16);
      xe1 = (float)(int16_t)(p1 & 0xffffu);
      xo1 = (float)((int32_t)p1 >> 16);
    } else {
      const float2 q0 = *reinterpret_cast<const float2 *>(s_lds + skew<IN>(s0));
      const float2 q1 = *reinterpret_cast<const float2 *>(s_lds + skew<IN>(s0 + 200));
      xe0 = q0.x;
      xo0 = q0.y;
      xe1 = q1.x;
      xo1 = q1.y;
    }
    const v4f m = a.amat[n1 * 64 + lane];
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(m[0], xe0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(m[1], xe1, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(m[2], xo0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(m[3], xo1, acc, 0, 0, 0);
    D[n1] = acc;
  }
  __syncthreads();   // every wave is done with the span; the LDS becomes the power tile

  // 3. two 25-point DFTs per lane: classes a (rows 4g, 4g+1) and b (4g+2, 4g+3)
  float2 Za[25], Zb[25];
#pragma unroll
  for (int n1 = 0; n1 < 25; ++n1) {
    Za[n1] = make_float2(D[n1][0], D[n1][1]);
    Zb[n1] = make_float2(D[n1][2], D[n1][3]);
  }
  dft25(Za);
  dft25(Zb);

  // 4. split into the real spectrum and power.  Slot i pairs Z[k] with
  // Z[200 - k]; for groups 0..2 (classes a, 8-a): k = 8i + a, partner
  // Zb[24 - i].  Group 3 holds the self-paired classes 0 and 4, laid out
  // into the same slot pattern: slots 0..12 are class 0 (k = 8i, partner
  // Z0[(25 - i) mod 25]), slots 13..24 class 4 (k = 8i - 100, partner
  // Z4[37 - i]); bin 100 (Z4[12] with itself) is one extra slot.
  const bool g3 = g == 3;
  const int d1 = g3 ? 0 : g + 1, d2 = g3 ? -100 : g + 1;
  // per-lane factor of the split twiddle W400^k = W400^(8i) * c
  const float2 wa = g == 0 ? w400(1) : (g == 1 ? w400(2) : w400(3));
  const float2 c1 = g3 ? make_float2(1.0f, 0.0f) : wa;
  const float2 c2 = g3 ? make_float2(0.0f, 1.0f) : wa;
  float *P = s_lds + fl * kRow;
#pragma unroll
  for (int i = 0; i < 25; ++i) {
    float2 zk = Za[i];
    if (i >= 13 && g3) zk = Zb[i - 13];
    const int j = 24 - i;
    float2 zm = Zb[j];
    if (g3) zm = j < 12 ? Zb[13 + j] : (j < 24 ? Za[1 + j] : Za[0]);
    const float2 zc = cconj(zm);
    const float2 Y = cadd(zk, zc), Dd = csub(zk, zc);
    const float2 W = cmul(w400(8 * i), i < 13 ? c1 : c2);
    const float2 V = cmul(W, Dd);
    const float pk = (Y.x + V.y) * (Y.x + V.y) + (Y.y - V.x) * (Y.y - V.x);
    const float pm = (Y.x - V.y) * (Y.x - V.y) + (Y.y + V.x) * (Y.y + V.x);
    const int k = 8 * i + (i < 13 ? d1 : d2);
    P[k] = pk;
    P[200 - k] = pm;
  }
  if (g3) {   // bin 100: 2 X[100] = 2 conj(Z[100]), |.|^2 = 4 |Z[100]|^2
    const float2 z = Zb[12];
    P[100] = 4.0f * (z.x * z.x + z.y * z.y);
  }
  __syncthreads();   // power rows complete (each wave reads its own frames' rows)
  if (a.power != 2.0f) {
    // |X|^p = (|X|^2)^(p/2), in place over the wave's own 16 rows (kept out
    // of the unrolled split above so the power-2 path stays compact)
    float *rows = s_lds + 16 * wv * kRow;
    const float pe = 0.5f * a.power;
    for (int i = lane; i < 16 * kRow; i += 64) rows[i] = powf(rows[i] * a.pre_scale, pe);
  }

  // 5. mel sums on the matrix cores, for the wave's own 16 frames: bands in
  // blocks of 16, each block only over the 4-bin chunks its filters touch.
  // A = blocked filter weights (lane order), B = P[frame c][bin klo+4ch+g],
  // D = 16 bands x 16 frames; lane (c, g) gets bands 16j+4g .. 16j+4g+3 of
  // frame c.  Then log10 after the 1e-10 floor, (L+4)/4, mel-major store.
  const int NM = a.n_mels;
  const int64_t fr = f0 + fl;
  const bool valid = fr < F;
  const float *pb0 = s_lds + fl * kRow + g;
  OUT *__restrict__ ocol = out_base + b * (int64_t)NM * F + fr;
  float vmax = 0.0f, lmin = __builtin_huge_valf();
  for (int j = 0; j < 16; ++j) {
    if (j >= a.n_melblk) break;
    const int klo = melblk_meta[3 * j], nch = melblk_meta[3 * j + 1], toff = melblk_meta[3 * j + 2];
    const float *wt = (a.melw_lds ? s_melw : melblk_w) + toff + lane;
    const float *pb = pb0 + klo;
    v4f acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
    int ch = 0;
    for (; ch + 1 < nch; ch += 2) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(wt[64 * ch], pb[4 * ch], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(wt[64 * ch + 64], pb[4 * ch + 4], acc1, 0, 0, 0);
    }
    if (ch < nch) acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(wt[64 * ch], pb[4 * ch], acc0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * j + 4 * g + r;
      const float v = fmaxf((acc0[r] + acc1[r]) * a.mel_scale, 1e-10f);
      const float L = log10_pos(v);
      if (valid && m < NM) {
        vmax = fmaxf(vmax, v);
        lmin = fminf(lmin, L);
        store_out_nt(ocol + (int64_t)m * F, rescale(L));
      }
    }
  }

  // 6. statistics of the wave's 16-frame sub-tile: smallest log value and
  // largest mel value to entry tile * 4 + wave
  lmin = wave_min(lmin);
  vmax = wave_max(vmax);
  if (lane == 0) {
    tile_min[tile * (kThreads / 64) + wv] = lmin;
    a.tile_max[tile * (kThreads / 64) + wv] = vmax;
  }
}

}  // namespace

// The n_fft = 400 path needs an even hop (sample pairs stay aligned) and a
// staged span that fits the power tile's LDS.
bool pcm400_supported(const lm_plan *p, bool in_i16) {
  if (p->n_fft != 400 || (p->hop & 1) || !p->dt.mfma400 || p->n_mels > 256) return false;
  const int span = (kTileFrames - 1) * p->hop + 400;
  const int ndw = in_i16 ? span / 2 : span;
  return (in_i16 ? ndw + (ndw >> 5) : ndw + 2 * (ndw >> 6)) + 2 <= kLdsFloats;
}

int pcm400_frames_per_tile() { return kTileFrames; }
int pcm400_min_rows_per_tile(const lm_plan *) { return kThreads / 64; }

hipError_t launch_pcm400(const lm_plan *p, const PcmArgs &pa, hipStream_t s) {
  Args k;
  k.pcm = pa.pcm;
  k.T = pa.n_samples;
  k.F = pa.n_frames;
  k.tiles_per_clip = pa.tiles_per_clip;
  k.hop = p->hop;
  k.pad = p->center ? 200 : 0;
  k.pad_mode = p->pad_mode;
  k.power = p->power;
  const float in_scale2 = pa.in_i16 ? 1.0f / 1073741824.0f : 1.0f;   // 2^-30
  if (p->power == 2.0f) {
    k.mel_scale = 0.25f * in_scale2;
    k.pre_scale = 1.0f;
  } else {
    k.mel_scale = 1.0f;
    k.pre_scale = 0.25f * in_scale2;
  }
  k.n_mels = p->n_mels;
  k.n_melblk = p->dt.n_melblk;
  k.amat = reinterpret_cast<const v4f *>(p->dt.mfma400);
  k.out = pa.out;
  k.tile_max = pa.tile_max;
  k.melw_lds = p->melblk_w.size() <= (size_t)kMelWLds ? (int)p->melblk_w.size() : 0;
  const dim3 grid((unsigned)(pa.n_clips * pa.tiles_per_clip)), block(kThreads);
  const bool f16 = p->out_dtype == LM_F16;
  const int32_t *bm = p->dt.melblk_meta;
  const float *bw = p->dt.melblk_w;
  float *tm = pa.tile_min;
  if (!pa.in_i16 && !f16)
    hipLaunchKernelGGL((pcm400_kernel<float, float>), grid, block, 0, s, k, bm, bw, (float *)pa.out, tm);
  else if (!pa.in_i16 && f16)
    hipLaunchKernelGGL((pcm400_kernel<float, __half>), grid, block, 0, s, k, bm, bw, (__half *)pa.out, tm);
  else if (pa.in_i16 && !f16)
    hipLaunchKernelGGL((pcm400_kernel<int16_t, float>), grid, block, 0, s, k, bm, bw, (float *)pa.out, tm);
  else
    hipLaunchKernelGGL((pcm400_kernel<int16_t, __half>), grid, block, 0, s, k, bm, bw, (__half *)pa.out, tm);
  return hipGetLastError();
}

}  // namespace lm
