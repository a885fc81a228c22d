// PCM -> log-mel, one fused kernel per (n_fft, input type, output type).
//
// A workgroup owns a tile of FPB consecutive frames of one clip and runs
// the whole chain on it in LDS (flashmel page, "How it works"):
//   1. frame samples are read straight from the clip with the signal's
//      zero padding and the center padding done as index arithmetic
//      (nothing padded is stored), paired
//      as z[n] = w[2n] x[2n] + i w[2n+1] x[2n+1] (periodic Hann);
//   2. an M = n_fft/2 point complex FFT of z, as Stockham autosort passes
//      of radix 16/8/5/4/2 through one LDS buffer;
//   3. the split into the n_fft-point real spectrum,
//        2 X[k] = (Z[k] + Z*[M-k]) - i e^{-2 pi i k/n_fft} (Z[k] - Z*[M-k]),
//      and |X|^p written back over the same buffer as a power tile with an
//      odd row stride M+1;
//   4. the packed triangular mel sum per (band, frame), log10 after the
//      1e-10 floor (KBench task page, "spec_md"), the (L+4)/4 rescale and a
//      mel-major store (flashmel page, "Usage": (..., n_mels, n_frames));
//   5. the tile's largest and smallest mel values go to per-tile
//      slots; the clamp fix-up kernel reduces them per clip and finishes the
//      per-clip floor.
// int16 input is converted to float without its 1/32768 scale; the mel
// values are scaled by 2^-30 instead (exact), together with the 1/4 of
// the split above.
#include <cstdio>
#include <type_traits>

#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

template <int... R>
struct Radices {};

template <int NFFT>
struct PcmCfg;
// FPB frames per tile, THREADS per workgroup, radix sequence of M = NFFT/2,
// WLDS floats of LDS for staged filter weights (weights past that count
// are read from global memory).  512 threads measured 7-27% faster than
// 256 at every size (more waves to hide each pass's LDS round trips at the
// same LDS per workgroup); 1024, or twice or half the frames, were slower.
template <> struct PcmCfg<400>   { static constexpr int FPB = 16,  THREADS = 512, WLDS = 4096; using Rad = Radices<8, 5, 5>; };
template <> struct PcmCfg<64>    { static constexpr int FPB = 128, THREADS = 512, WLDS = 4096; using Rad = Radices<16, 2>; };
template <> struct PcmCfg<128>   { static constexpr int FPB = 64,  THREADS = 512, WLDS = 4096; using Rad = Radices<16, 4>; };
template <> struct PcmCfg<256>   { static constexpr int FPB = 32,  THREADS = 512, WLDS = 4096; using Rad = Radices<16, 8>; };
template <> struct PcmCfg<512>   { static constexpr int FPB = 16,  THREADS = 512, WLDS = 4096; using Rad = Radices<16, 16>; };
template <> struct PcmCfg<1024>  { static constexpr int FPB = 8,   THREADS = 512, WLDS = 4096; using Rad = Radices<8, 8, 8>; };
template <> struct PcmCfg<2048>  { static constexpr int FPB = 4,   THREADS = 512, WLDS = 4096; using Rad = Radices<16, 16, 4>; };
template <> struct PcmCfg<4096>  { static constexpr int FPB = 2,   THREADS = 512, WLDS = 4096; using Rad = Radices<16, 16, 8>; };
// n_fft 8192 and 16384 (one frame per tile) run in pcm_big_kernel below
template <> struct PcmCfg<8192>  { static constexpr int FPB = 1; };
template <> struct PcmCfg<16384> { static constexpr int FPB = 1; };

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(int16_t v) { return (float)(int)v; }


// One Stockham radix-R pass over FPB frames of M points held in `buf`.
// Butterfly j of a frame (j < M/R, k = j mod Ns) reads a[t] = in[j + t M/R],
// multiplies a[t] by exp(-2 pi i t k / (Ns R)), transforms, and writes
// b[s] to ((j / Ns) Ns R + k + s Ns).  After the last pass the frame holds
// its DFT in natural order.
// LDS position of point i of the FFT buffer: with PAD > 0 one spare
// float2 follows every 2^PAD points, so that the strided accesses of the
// early passes fall on distinct banks.
template <int PAD>
__device__ __forceinline__ int lds_pos(int i) { return PAD ? i + (i >> PAD) : i; }
// lds_pos(b + d) - lds_pos(b) for a compile-time step d, valid wherever b
// and b + d lie in the same 2^PAD block or d is a multiple of 2^PAD
template <int PAD>
constexpr int lds_step(int d) { return PAD ? d + (d >> PAD) : d; }
constexpr bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

template <int R, int M, int FPB, int THREADS, int Ns, int PAD, typename TW>
__device__ __forceinline__ void fft_pass(float2 *buf, TW tw, int tid) {
  constexpr int NBF = M / R;                 // butterflies per frame
  constexpr int NB = FPB * NBF;
  constexpr int BPT = (NB + THREADS - 1) / THREADS;
  constexpr int TW_STEP = M / (Ns * R);
  // Padded positions from one base per butterfly and compile-time steps
  // where that is exact: reads b + t NBF with NBF a multiple of 2^PAD;
  // writes o + s Ns with everything a power of two (then either Ns is a
  // multiple of 2^PAD, or o's offset in its 2^PAD block is below Ns and
  // the butterfly's outputs cross blocks only at multiples of 2^PAD)
  constexpr int P2 = 1 << PAD;
  constexpr bool kReadStep = PAD == 0 || NBF % P2 == 0 || (is_pow2(M) && M <= P2);
  constexpr bool kWriteStep =
      PAD == 0 || (is_pow2(M) && M % P2 == 0 && is_pow2(Ns) && is_pow2(R) && (Ns % P2 == 0 || P2 % Ns == 0));
  float2 v[BPT][R];
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int q = tid + i * THREADS;
    if (NB % THREADS == 0 || q < NB) {
      const int f = q / NBF, j = q - f * NBF;
      if constexpr (kReadStep) {
        const float2 *rb = buf + lds_pos<PAD>(f * M + j);
#pragma unroll
        for (int t = 0; t < R; ++t) v[i][t] = rb[lds_step<PAD>(t * NBF)];
      } else {
#pragma unroll
        for (int t = 0; t < R; ++t) v[i][t] = buf[lds_pos<PAD>(f * M + j + t * NBF)];
      }
      if (Ns > 1) {
        const int k = j % Ns;
        float2 w[R];
        tw.template powers<TW_STEP, R>(k, w);
#pragma unroll
        for (int t = 1; t < R; ++t) v[i][t] = cmul(v[i][t], w[t]);
      }
      dft<R>(v[i]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    const int q = tid + i * THREADS;
    if (NB % THREADS == 0 || q < NB) {
      const int f = q / NBF, j = q - f * NBF;
      const int k = j % Ns;
      const int o = f * M + (j / Ns) * Ns * R + k;
      if constexpr (kWriteStep) {
        float2 *wb = buf + lds_pos<PAD>(o);
#pragma unroll
        for (int s = 0; s < R; ++s) wb[lds_step<PAD>(s * Ns)] = v[i][s];
      } else {
#pragma unroll
        for (int s = 0; s < R; ++s) buf[lds_pos<PAD>(o + s * Ns)] = v[i][s];
      }
    }
  }
  __syncthreads();
}

template <int M, int FPB, int THREADS, int Ns, int PAD, typename TW, int R, int... Rest>
__device__ __forceinline__ void fft_passes(float2 *buf, TW tw, int tid) {
  fft_pass<R, M, FPB, THREADS, Ns, PAD>(buf, tw, tid);
  if constexpr (sizeof...(Rest) > 0) fft_passes<M, FPB, THREADS, Ns * R, PAD, TW, Rest...>(buf, tw, tid);
}

// A twiddle source for fft_pass: at<STEP>(q) returns exp(-2 pi i q STEP / M)
// (0 <= q STEP < M) from a function of the table index j = q STEP.
template <typename F>
struct TwFn {
  F f;
  template <int STEP>
  __device__ __forceinline__ float2 at(int q) const { return f(q * STEP); }
  // w[t] = at<STEP>(t k) for 1 <= t < R: from one table read (R <= 5), two
  // (R = 8: w and w^4) or three (R = 16: w, w^4, w^8), the other powers as
  // products of at most four table values
  template <int STEP, int R>
  __device__ __forceinline__ void powers(int k, float2 (&w)[R]) const {
    if constexpr (R == 2) {
      w[1] = at<STEP>(k);
    } else if constexpr (R <= 5) {
      w[1] = at<STEP>(k);
      w[2] = cmul(w[1], w[1]);
      if constexpr (R > 3) w[3] = cmul(w[2], w[1]);
      if constexpr (R > 4) w[4] = cmul(w[2], w[2]);
    } else if constexpr (R == 8 || R == 16) {
      w[1] = at<STEP>(k);
      w[4] = at<STEP>(4 * k);
      w[2] = cmul(w[1], w[1]);
      w[3] = cmul(w[2], w[1]);
      w[5] = cmul(w[4], w[1]);
      w[6] = cmul(w[4], w[2]);
      w[7] = cmul(w[4], w[3]);
      if constexpr (R == 16) {
        w[8] = at<STEP>(8 * k);
#pragma unroll
        for (int t = 9; t < 16; ++t) w[t] = cmul(w[8], w[t - 8]);
      }
    } else {
#pragma unroll
      for (int t = 1; t < R; ++t) w[t] = at<STEP>(t * k);
    }
  }
};
template <typename F>
__device__ __forceinline__ TwFn<F> tw_fn(F f) { return TwFn<F>{f}; }

// `tw.at<STEP>(q)` returns exp(-2 pi i q STEP / M); `tid` is the thread's
// index in the workgroup; point i of frame f sits at lds_pos<PAD>(f M + i)
template <int M, int FPB, int THREADS, int PAD, typename TW, int... R>
__device__ __forceinline__ void run_fft(float2 *buf, TW tw, Radices<R...>, int tid) {
  fft_passes<M, FPB, THREADS, 1, PAD, TW, R...>(buf, tw, tid);
}

struct PcmKernelArgs {
  const void *pcm;
  int64_t T, F;
  int tiles_per_clip;
  int hop, pad, pad_mode;   // pad: center padding plus the signal's zero padding
  int sig_pad;             // the signal's zero padding (zeros before and after each clip)
  float power;          // exponent p; 2 takes the fast path
  float mel_scale;      // exact power-of-two scale of the mel sums
  float pre_scale;      // scale of |2X|^2 before a general power
  int mel_out;          // 1: store the mel values themselves (no log tail)
  int skip_empty;       // 1: leave bands without weights unwritten (the fix-up writes them)
  int n_mels;
  const float *window;
  const float2 *twiddle, *untangle;
  const float2 *tw2;    // n_fft >= 8192: exp(-2 pi i 128 h / n_fft) for h < n_fft / 128, then exp(-2 pi i l / n_fft), l < 128
  const int32_t *mel_lanes;   // n_fft >= 8192: the mel stage's lane table (band | h << 8 | log2 L << 16, or -1)
  int hann_tw;          // n_fft >= 8192: 1 if the window is the full-length periodic Hann (derived from tw2)
  const int32_t *csr_start, *csr_width, *csr_off;
  const float *csr_w;
  int nnz;
  void *out;
  float *tile_min, *tile_max;
};


// exp(-2 pi i / 400): the odd twiddles of the paired 400-point transform
// come from the 200-point table times this (double-rounded once to fp32)
constexpr float kW400_1c = 0.99987663248166059f, kW400_1s = -0.015707317311820675f;

// PAIRED (n_fft = 400 only; the FFT-variant comparison): instead of folding
// each real frame into a 200-point complex sequence, two frames a, b form
// one 400-point complex sequence z = y_a + i y_b, transformed by radix
// 16/5/5 passes and split as 2 X_a[k] = Z[k] + Z*[400-k], 2 X_b[k] =
// -i (Z[k] - Z*[400-k]).
// Tile of workgroup id b in a grid of n workgroups, one tile each.
// Neighbouring tiles share n_fft - hop input samples, and workgroup ids go
// to the chip's XCDs (each with its own L2) in turn, so every run of
// kXcds * K ids is dealt such that each XCD takes K consecutive tiles and
// the shared samples come from its L2; ids past the last whole run keep
// their own tile.  A permutation of [0, n).
template <int K>
__device__ __forceinline__ int64_t xcd_dealt_tile(int64_t b, int64_t n) {
  constexpr int64_t C = (int64_t)kXcds * K;
  if (b >= n / C * C) return b;
  const int64_t c = b / C;
  const int r = (int)(b - c * C);
  return c * C + (int64_t)(r % kXcds) * K + r / kXcds;
}

template <int NFFT, typename IN, typename OUT, bool PAIRED = false>
__global__ void __launch_bounds__(PcmCfg<NFFT>::THREADS) pcm_logmel_kernel(PcmKernelArgs a) {
  static_assert(!PAIRED || NFFT == 400, "the paired transform is built for n_fft = 400");
  constexpr int M = NFFT / 2;
  constexpr int FPB = PcmCfg<NFFT>::FPB;
  constexpr int THREADS = PcmCfg<NFFT>::THREADS;
  constexpr int NW = THREADS / 64;
  constexpr int PAD = 5;   // one spare point per 32 (lds_pos): the strided first pass stays conflict-free
  __shared__ float2 s_buf[FPB * M + ((FPB * M) >> PAD)];   // also FPB / 2 sequences of NFFT points when PAIRED
  constexpr int WLDS = PcmCfg<NFFT>::WLDS;
  __shared__ int32_t s_start[256], s_width[256], s_off[256];
  __shared__ float s_w[WLDS > 0 ? WLDS : 1];
  __shared__ float s_red[2 * NW];

  const int tid = threadIdx.x;
  const int64_t tile = xcd_dealt_tile<32>(blockIdx.x, gridDim.x);
  const int64_t b = tile / a.tiles_per_clip;
  const int t = (int)(tile - b * a.tiles_per_clip);
  const int64_t f0 = (int64_t)t * FPB;
  const int64_t T = a.T, F = a.F;
  const IN *__restrict__ x = reinterpret_cast<const IN *>(a.pcm) + b * T;

  // packed filterbank -> LDS
  const int NM = a.n_mels;
  const int nnz = stage_filters<THREADS>(NM, a.csr_start, a.csr_width, a.csr_off, a.csr_w, a.nnz, s_start, s_width,
                                         s_off, s_w, WLDS);
  const bool w_in_lds = WLDS > 0 && nnz <= WLDS;

  if constexpr (PAIRED) {
    // 1'. frames 2 l and 2 l + 1 of the tile as one complex sequence
    constexpr int NP = FPB / 2;
    constexpr int IPT = (NP * NFFT + THREADS - 1) / THREADS;
    float xa[IPT], xb[IPT], wv[IPT];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int i = tid + u * THREADS;
      const int pl = i / NFFT, n = i - pl * NFFT;
      const int64_t fa = f0 + 2 * pl;
      xa[u] = xb[u] = wv[u] = 0.0f;
      if (i < NP * NFFT && fa < F) {
        const int64_t j = fa * a.hop - a.pad + n;
        const int64_t sa = signal_source(j, T, a.sig_pad, a.pad_mode);
        const int64_t sb = fa + 1 < F ? signal_source(j + a.hop, T, a.sig_pad, a.pad_mode) : -1;
        xa[u] = sa >= 0 ? to_f(x[sa]) : 0.0f;
        xb[u] = sb >= 0 ? to_f(x[sb]) : 0.0f;
        wv[u] = a.window[n];
      }
    }
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int i = tid + u * THREADS;
      if (i < NP * NFFT) s_buf[lds_pos<PAD>(i)] = make_float2(xa[u] * wv[u], xb[u] * wv[u]);
    }
    __syncthreads();
    // 2'. 400-point complex FFT per pair: exp(-2 pi i j / 400) from the
    //     200-point table, times exp(-2 pi i / 400) for odd j
    const float2 *__restrict__ twt = a.twiddle;
    run_fft<NFFT, NP, THREADS, PAD>(
        s_buf,
        tw_fn([=](int j) {
          const float2 t = twt[j >> 1];
          return (j & 1) ? cmul(t, make_float2(kW400_1c, kW400_1s)) : t;
        }),
        Radices<16, 5, 5>{}, tid);
    // 3'. split into the two frames' spectra, |2 X|^2 in the power tile
    constexpr int NK = NFFT / 2 + 1;
    constexpr int UPT = (NP * NK + THREADS - 1) / THREADS;
    float pa[UPT], pb[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + u * THREADS;
      pa[u] = pb[u] = 0.0f;
      if (q < NP * NK) {
        const int pl = q / NK, k = q - pl * NK;
        const float2 zk = s_buf[lds_pos<PAD>(pl * NFFT + k)];
        const float2 zc = cconj(s_buf[lds_pos<PAD>(pl * NFFT + (k == 0 ? 0 : NFFT - k))]);
        const float2 A = cadd(zk, zc), Bm = csub(zk, zc);   // 2 X_a, and i 2 X_b
        pa[u] = A.x * A.x + A.y * A.y;
        pb[u] = Bm.x * Bm.x + Bm.y * Bm.y;
      }
    }
    __syncthreads();
    float *P = reinterpret_cast<float *>(s_buf);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + u * THREADS;
      if (q < NP * NK) {
        const int pl = q / NK, k = q - pl * NK;
        P[(2 * pl) * (M + 1) + k] = pa[u];
        P[(2 * pl + 1) * (M + 1) + k] = pb[u];
      }
    }
    __syncthreads();
  } else {
  // 1. windowed, padded frame samples as M complex points per frame; every
  //    load of the thread is issued before any is used.  A tile whose
  //    frames all lie inside the clip, with an even first sample (so that a
  //    sample pair is one aligned 8- or 4-byte word), loads each point's two
  //    samples with one load and no padding arithmetic.
  const float2 *__restrict__ win2 = reinterpret_cast<const float2 *>(a.window);
  constexpr int IPT = (FPB * M + THREADS - 1) / THREADS;
  float xs[IPT][2];
  float2 ws[IPT];
  const int64_t j_first = f0 * a.hop - a.pad;
  const bool direct = j_first >= 0 && f0 + FPB <= F && (f0 + FPB - 1) * a.hop - a.pad + NFFT <= T &&
                      (((uintptr_t)(x + j_first) | (uintptr_t)(sizeof(IN) * a.hop)) % (2 * sizeof(IN))) == 0;
  if (direct) {   // uniform
    typedef typename std::conditional<sizeof(IN) == 2, uint32_t, float2>::type Pair;
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int i = tid + u * THREADS;
      const int fl = i / M, n = i - fl * M;
      ws[u] = make_float2(0.0f, 0.0f);
      xs[u][0] = xs[u][1] = 0.0f;
      if ((FPB * M) % THREADS == 0 || i < FPB * M) {
        const Pair v = reinterpret_cast<const Pair *>(x + j_first + (int64_t)fl * a.hop)[n];
        if constexpr (sizeof(IN) == 2) {
          xs[u][0] = (float)(int16_t)(v & 0xffffu);
          xs[u][1] = (float)(int16_t)(v >> 16);
        } else {
          xs[u][0] = v.x;
          xs[u][1] = v.y;
        }
        ws[u] = win2[n];
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int i = tid + u * THREADS;
      const int fl = i / M, n = i - fl * M;
      const int64_t fr = f0 + fl;
      ws[u] = make_float2(0.0f, 0.0f);
      xs[u][0] = xs[u][1] = 0.0f;
      if ((FPB * M) % THREADS == 0 || i < FPB * M) {
        if (fr < F) {
          const int64_t j = fr * a.hop - a.pad + 2 * n;
          const int64_t s0 = signal_source(j, T, a.sig_pad, a.pad_mode), s1 = signal_source(j + 1, T, a.sig_pad, a.pad_mode);
          xs[u][0] = s0 >= 0 ? to_f(x[s0]) : 0.0f;
          xs[u][1] = s1 >= 0 ? to_f(x[s1]) : 0.0f;
          ws[u] = win2[n];
        }
      }
    }
  }
  static_assert(THREADS % (1 << PAD) == 0, "whole 2^PAD blocks per thread stride");
  float2 *const wb = s_buf + lds_pos<PAD>(tid);
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const int i = tid + u * THREADS;
    if ((FPB * M) % THREADS == 0 || i < FPB * M)
      wb[lds_step<PAD>(u * THREADS)] = make_float2(xs[u][0] * ws[u].x, xs[u][1] * ws[u].y);
  }
  __syncthreads();

  // the split's twiddles, loaded before the FFT so that their latency
  // hides behind it (up to n_fft 1024: above, the registers they hold
  // through the FFT would cost a workgroup of occupancy)
  constexpr int NU = M / 2 + 1;              // pairs (k, M-k), k = 0..M/2
  constexpr int UPT = (FPB * NU + THREADS - 1) / THREADS;
  constexpr bool kPreUt = M <= 512;
  float2 ut[UPT];
  if constexpr (kPreUt) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + u * THREADS;
      const int fl = q / NU, k = q - fl * NU;
      ut[u] = q < FPB * NU ? a.untangle[k] : make_float2(0.0f, 0.0f);
    }
  }

  // 2. M-point complex FFT per frame
  const float2 *__restrict__ twt = a.twiddle;
  run_fft<M, FPB, THREADS, PAD>(s_buf, tw_fn([=](int j) { return twt[j]; }), typename PcmCfg<NFFT>::Rad{}, tid);

  // 3. split into the real spectrum; power tile over the same LDS
  float pk[UPT], pmk[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + u * THREADS;
    pk[u] = pmk[u] = 0.0f;
    if (q < FPB * NU) {
      const int fl = q / NU, k = q - fl * NU;
      const float2 zk = s_buf[lds_pos<PAD>(fl * M + k)];
      const float2 zc = cconj(s_buf[lds_pos<PAD>(fl * M + (k == 0 ? 0 : M - k))]);
      const float2 Y = cadd(zk, zc), D = csub(zk, zc);
      const float2 V = cmul(kPreUt ? ut[u] : a.untangle[k], D);
      pk[u] = (Y.x + V.y) * (Y.x + V.y) + (Y.y - V.x) * (Y.y - V.x);
      pmk[u] = (Y.x - V.y) * (Y.x - V.y) + (Y.y + V.x) * (Y.y + V.x);
    }
  }
  __syncthreads();
  float *P = reinterpret_cast<float *>(s_buf);
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + u * THREADS;
    if (q < FPB * NU) {
      const int fl = q / NU, k = q - fl * NU;
      P[fl * (M + 1) + k] = pk[u];
      if (k != M / 2) P[fl * (M + 1) + M - k] = pmk[u];
    }
  }
  __syncthreads();
  }   // folded (not PAIRED)
  float *P = reinterpret_cast<float *>(s_buf);
  if (a.power != 2.0f) {
    // |X|^p = (|X|^2)^(p/2) in place, outside the unrolled split above
    const float e = 0.5f * a.power;
    for (int i = tid; i < FPB * (M + 1); i += THREADS) P[i] = powf(P[i] * a.pre_scale, e);
    __syncthreads();
  }

  // 4. mel sums, log10, rescale, mel-major store
  float vmax = 0.0f, vmin = __builtin_huge_valf();
  OUT *__restrict__ out = reinterpret_cast<OUT *>(a.out) + b * (int64_t)NM * F;
  // one copy of the loop per weight source, so LDS weights are read with LDS
  // instructions (a pointer that may point either way would make every
  // weight load a flat load that waits for all outstanding global loads)
  // L lanes per (band, frame) output when the tile has fewer outputs than
  // threads (L a power of two, at most 16): lane h of a group sums bins h,
  // h + L, ... in two chains and the group adds its partial sums by xor
  // shuffles (every lane of a group has the same trip count; DPP row steps
  // instead measured 1-6% slower)
  int L = 1;
  while (L < 16 && 2 * L * NM * FPB <= THREADS) L *= 2;
  const int h = tid & (L - 1);
  auto mel = [&](const float *wsrc) {
    for (int o = tid / L; o < NM * FPB; o += THREADS / L) {
      const int fl = o % FPB, m = o / FPB;
      const int64_t fr = f0 + fl;
      const int st = s_start[m], wd = s_width[m];
      const float *pr = P + fl * (M + 1) + st;
      const float *wr = wsrc + s_off[m];
      float acc0 = 0.0f, acc1 = 0.0f;
      int j = h;
      for (; j + L < wd; j += 2 * L) {
        acc0 = __builtin_fmaf(wr[j], pr[j], acc0);
        acc1 = __builtin_fmaf(wr[j + L], pr[j + L], acc1);
      }
      if (j < wd) acc0 = __builtin_fmaf(wr[j], pr[j], acc0);
      float acc = acc0 + acc1;
      for (int s2 = L >> 1; s2 > 0; s2 >>= 1) acc += __shfl_xor(acc, s2, 64);
      if (h != 0 || fr >= F) continue;
      if (wd == 0 && a.skip_empty) continue;   // log10(1e-10) everywhere: written by the fix-up
      if (a.mel_out) {
        store_out(out + (int64_t)m * F + fr, acc * a.mel_scale);
        continue;
      }
      const float v = floor_1e10(acc * a.mel_scale);
      const float ov = logmel_of(v);
      vmax = fmaxf(vmax, v);
      vmin = fminf(vmin, v);
      store_out(out + (int64_t)m * F + fr, ov);
    }
  };
  if (w_in_lds) mel(s_w);
  else mel(a.csr_w);

  // 5. tile statistics
  block_maxmin<THREADS>(vmax, vmin, s_red);
  if (tid == 0) {
    a.tile_max[tile] = vmax;
    a.tile_min[tile] = vmin;
  }
}

// ---------------------------------------------------------------------------
// n_fft >= 8192: one frame fills a workgroup's FFT buffer, so the kernel is
// persistent instead: WGS workgroups per compute unit stage the packed
// filterbank (where it fits their LDS share) and a two-level twiddle table
// in LDS once, then walk frames gridDim.x apart (so the padded first and
// last frames of the clips, which take the slower index path, spread over
// the workgroups).  Per frame the phases are those above (windowed load,
// folded complex FFT, split and power, mel, statistics), with no global
// memory access between the load and the store: every twiddle is the
// product of two LDS entries, exp(-2 pi i j / N) = W[j / 128] W'[j % 128].
// At 16384 (one 1024-thread workgroup per CU) the next frame's samples are
// loaded into registers while the mel sums of the current one run; at 8192
// two 512-thread workgroups share a CU, each loading its frame at the
// frame's start, and either one's barriers and loads overlap the other's
// work (48 against 69 us per sweep step with one 1024-thread workgroup).
// The mel gives every band a group of L consecutive lanes (a power of two,
// at most 64, from the plan's lane table, which widens the groups of the
// bands with the most bins per lane), which stride over the band's bins in
// pairs of adjacent bins and add their partial sums at the group's first
// lane (DPP row shifts, one swizzle, one permute), so no band waits on
// another band's reduction.
// ---------------------------------------------------------------------------
template <int NFFT>
struct BigCfg;
// THREADS per workgroup, WGS workgroups per CU, PREFETCH: load the next
// frame's samples during the current frame's mel sums
// TAB_STEP, TAB_NS: the radix-8 pass whose twiddles come from an LDS table
// of their seven powers (its twiddle step and its Ns; 0 for none), where the
// workgroup's LDS has room for it
template <> struct BigCfg<8192> {
  static constexpr int THREADS = big_threads(8192), WGS = 2;
  static constexpr bool PREFETCH = false;
  static constexpr int TAB_STEP = 0, TAB_NS = 0;
  using Rad = Radices<8, 8, 8, 8>;
};
template <> struct BigCfg<16384> {
  static constexpr int THREADS = big_threads(16384), WGS = 1;
  static constexpr bool PREFETCH = true;
  static constexpr int TAB_STEP = 8, TAB_NS = 128;   // the third pass: 8192 / (128 * 8)
  using Rad = Radices<16, 8, 8, 8>;
};

constexpr int kTwLo = 128;   // entries of the low twiddle table
constexpr int kBigPad = 5;   // FFT buffer: one spare point per 32

// Twiddles of the one-frame kernel's M-point FFT from the two-level LDS
// table: exp(-2 pi i q STEP / M) = exp(-2 pi i j / N) with j = 2 q STEP =
// 128 h + l, the product of hi[h] and lo[l]; where every j of a pass is a
// multiple of 128 (the early passes) the low factor is exactly 1 and the
// twiddle is one table entry.
template <int THI, int TSTEP = 0, int TNS = 0>
struct BigTw {
  const float2 *s_tw;   // THI entries exp(-2 pi i 128 h / N), then kTwLo entries exp(-2 pi i l / N)
  const float2 *s_tab;  // TSTEP > 0: at<TSTEP>(t k) for 1 <= t < 8, k < TNS, at [(t - 1) TNS + k]
  template <int STEP>
  __device__ __forceinline__ float2 at(int q) const {
    constexpr int S = 2 * STEP;
    const int j = q * S;
    if constexpr (S % kTwLo == 0) return s_tw[j / kTwLo];
    else return cmul(s_tw[j >> 7], s_tw[THI + (j & (kTwLo - 1))]);
  }
  // w[t] = at<STEP>(t k) for 1 <= t < R.  Where each twiddle would be a
  // product of two table entries, a radix-8 butterfly instead reads w and
  // w^4 (four entries) and forms the other five powers by products of at
  // most three factors (w^7 = w^4 w^2 w), the same number of complex
  // products as before and 4 instead of 14 LDS reads.
  template <int STEP, int R>
  __device__ __forceinline__ void powers(int k, float2 (&w)[R]) const {
    if constexpr (TSTEP > 0 && STEP == TSTEP && R == 8) {
      // seven table reads, no products (the table holds each power as one
      // product of two entries of s_tw)
#pragma unroll
      for (int t = 1; t < R; ++t) w[t] = s_tab[(t - 1) * TNS + k];
    } else if constexpr ((2 * STEP) % kTwLo == 0 || R != 8) {
#pragma unroll
      for (int t = 1; t < R; ++t) w[t] = at<STEP>(t * k);
    } else {
      w[1] = at<STEP>(k);
      w[4] = at<STEP>(4 * k);
      w[2] = cmul(w[1], w[1]);
      w[3] = cmul(w[2], w[1]);
      w[5] = cmul(w[4], w[1]);
      w[6] = cmul(w[4], w[2]);
      w[7] = cmul(w[4], w[3]);
    }
  }
};

template <int NFFT>
constexpr int big_wlds() {
  // LDS floats left for filter weights next to the FFT buffer (M float2),
  // the twiddle tables and the row tables, within one workgroup's share of
  // the CU's 160 KB
  return (160 * 1024 / BigCfg<NFFT>::WGS - (NFFT / 2 + (NFFT >> (kBigPad + 1))) * 8 - (NFFT / kTwLo + kTwLo) * 8 -
          7 * BigCfg<NFFT>::TAB_NS * 8 - 3 * 256 * 4 - 1024) / 4;
}

// A frame that reaches into the padding (the first and last few of a
// clip), windowed into the FFT buffer with every sample by index
// arithmetic, all loads of a thread in flight together.  Kept out of line:
// inlined, its per-sample padding logic enlarged the frame loop and its
// scalar register pressure for the few frames that take it.
template <typename IN, int M, int THREADS>
__device__ __attribute__((noinline)) void big_padded_frame(const IN *__restrict__ x, const float2 *__restrict__ win2,
                                                           int64_t j0, int64_t T, int sig_pad, int pad_mode, int tid,
                                                           float2 *buf) {
  constexpr int IPT = M / THREADS;
  float ys[IPT][2];
  float2 ws[IPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const int n = tid + u * THREADS;
    const int64_t s0 = signal_source(j0 + 2 * n, T, sig_pad, pad_mode),
                  s1 = signal_source(j0 + 2 * n + 1, T, sig_pad, pad_mode);
    ys[u][0] = s0 >= 0 ? to_f(x[s0]) : 0.0f;
    ys[u][1] = s1 >= 0 ? to_f(x[s1]) : 0.0f;
    ws[u] = win2[n];
  }
  float2 *const wb = buf + lds_pos<kBigPad>(tid);
#pragma unroll
  for (int u = 0; u < IPT; ++u) wb[lds_step<kBigPad>(u * THREADS)] = make_float2(ys[u][0] * ws[u].x, ys[u][1] * ws[u].y);
}

template <int NFFT, typename IN, typename OUT>
__global__ void __launch_bounds__(BigCfg<NFFT>::THREADS, BigCfg<NFFT>::THREADS / 256 * BigCfg<NFFT>::WGS)
    pcm_big_kernel(PcmKernelArgs a, int64_t n_tiles) {
  constexpr int M = NFFT / 2;
  constexpr int THREADS = BigCfg<NFFT>::THREADS;
  constexpr int NW = THREADS / 64;
  constexpr int WLDS = big_wlds<NFFT>();
  constexpr int THI = NFFT / kTwLo;
  __shared__ float2 s_buf[M + (M >> kBigPad)];
  __shared__ float2 s_tw[THI + kTwLo];   // exp(-2 pi i 128 h / N), then exp(-2 pi i l / N)
  constexpr int TSTEP = BigCfg<NFFT>::TAB_STEP, TNS = BigCfg<NFFT>::TAB_NS;
  __shared__ float2 s_tab[TNS > 0 ? 7 * TNS : 1];
  __shared__ int32_t s_start[256], s_width[256], s_off[256];
  __shared__ float s_w[WLDS];
  __shared__ float s_red[2 * NW];

  const int NM = a.n_mels;
  for (int i = threadIdx.x; i < THI + kTwLo; i += THREADS) s_tw[i] = a.tw2[i];
  if constexpr (TNS > 0) {
    // the tabulated pass's twiddle powers at<TSTEP>(t k) = exp(-2 pi i j / N),
    // j = 2 TSTEP t k, each the product of its two entries of the two-level
    // table (read here from global memory; the barrier in stage_filters
    // orders these stores before the first frame)
    static_assert((TNS & (TNS - 1)) == 0 && 2 * TSTEP * 7 * (TNS - 1) < NFFT, "table within one turn");
    for (int i = threadIdx.x; i < 7 * TNS; i += THREADS) {
      const int j = 2 * TSTEP * (i / TNS + 1) * (i & (TNS - 1));
      s_tab[i] = cmul(a.tw2[j >> 7], a.tw2[THI + (j & (kTwLo - 1))]);
    }
  }
  const int nnz = stage_filters<THREADS>(NM, a.csr_start, a.csr_width, a.csr_off, a.csr_w, a.nnz, s_start, s_width,
                                         s_off, s_w, WLDS);
  const bool w_in_lds = nnz <= WLDS;
  // this thread's place in the mel stage: band, position h in the band's
  // group of Lb lanes (or none)
  const int lane_ent = a.mel_lanes[threadIdx.x];
  const int perm32 = (((int)threadIdx.x + 32) & 63) << 2;   // ds_bpermute address of lane + 32 in the wave
  const int64_t T = a.T, F = a.F;
  constexpr int IPT = M / THREADS;   // complex points per thread
  static_assert(M % THREADS == 0, "whole points per thread");
  // A thread's points n = tid + THREADS u share their low table entries:
  // 2 THREADS and THREADS are multiples of kTwLo, so for every u the index j
  // = 2n (window) or n (split) has the same j mod kTwLo and its high index
  // advances by a compile-time step.
  static_assert(THREADS % kTwLo == 0, "low twiddle entry shared by a thread's points");

  // samples of an interior frame (no padding) of clip b at frame fr, all
  // loads in flight together; thread tid takes points n = tid + THREADS u
  float xs[IPT][2];
  auto load_interior = [&](int b, int fr, int tid) {
    // one uniform base per u and the thread's 32-bit byte offset, so that
    // the loads take a scalar base and a vector offset (no 64-bit address
    // arithmetic per load)
    const char *__restrict__ xb =
        reinterpret_cast<const char *>(reinterpret_cast<const IN *>(a.pcm) + b * T + ((int64_t)fr * a.hop - a.pad));
    const uint32_t o = (uint32_t)tid * (uint32_t)(2 * sizeof(IN));
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      // opaque, so that the compiler keeps it a scalar base; global address
      // space, so that the loads stay global loads
      uint64_t bu = reinterpret_cast<uint64_t>(xb) + (uint64_t)u * (THREADS * 2 * sizeof(IN));
      asm volatile("" : "+s"(bu));
      const __attribute__((address_space(1))) IN *p =
          reinterpret_cast<const __attribute__((address_space(1))) IN *>(bu + o);
      xs[u][0] = to_f(p[0]);
      xs[u][1] = to_f(p[1]);
    }
  };
  auto interior = [&](int fr) {
    const int64_t j0 = (int64_t)fr * a.hop - a.pad;
    return j0 >= 0 && j0 + NFFT <= T;
  };
  // Neighbouring frames share n_fft - hop samples (three quarters at hop
  // n_fft/4).  Workgroups go to the chip's 8 XCDs in turn and each XCD has
  // its own L2, so tiles are dealt such that the workgroups of one XCD take
  // consecutive frames in each round: the shared samples then come from
  // that XCD's L2 instead of once more from HBM per XCD.
  const int G = gridDim.x;
  const int first = G % kXcds == 0 ? (int)(blockIdx.x % kXcds) * (G / kXcds) + (int)(blockIdx.x / kXcds)
                                   : (int)blockIdx.x;
  constexpr bool PREFETCH = BigCfg<NFFT>::PREFETCH;
  // (clip, frame) of the tile, stepped by G tiles per frame without a
  // division: G = gq clips + gr frames
  const int tpc = a.tiles_per_clip;
  const int gq = G / tpc, gr = G - gq * tpc;
  int cb = first / tpc, cfr = first - cb * tpc;
  bool have = false;
  if constexpr (PREFETCH) {
    have = first < n_tiles && interior(cfr);
    if (have) load_interior(cb, cfr, threadIdx.x);
  }

  for (int64_t tile = first; tile < n_tiles; tile += G) {
    // the window pointer and the thread index are made opaque per frame so
    // that per-thread addresses are not kept live across the whole loop
    const float2 *win2 = reinterpret_cast<const float2 *>(a.window);
    asm volatile("" : "+s"(win2));
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int64_t b = cb;
    const int fr = cfr;   // one frame per tile
    int nb = cb + gq, nfr = cfr + gr;   // the tile G further on
    if (nfr >= tpc) {
      nfr -= tpc;
      ++nb;
    }
    if constexpr (!PREFETCH) {
      have = interior(fr);
      if (have) load_interior(cb, fr, tid);
    }
    // wave priorities: the frame's load and window and its mel sums at 1,
    // the FFT passes at 0, so that where two workgroups share a CU (n_fft
    // 8192) the one in its load or mel phase issues first and the other's
    // passes fill its waits (sweep 8192: main kernel 45.0 -> 43.1 us;
    // 16384, one workgroup per CU, unchanged)
    __builtin_amdgcn_s_setprio(1);
    // 1. windowed samples z[n] = (w[2n] x[2n], w[2n+1] x[2n+1])
    if (have && a.hann_tw) {
      // periodic Hann w[n] = 1/2 - 1/2 cos(2 pi n / N), the cosine from the
      // twiddle table in LDS (no global load at the start of the frame)
      // (samples 2n and 2n + 1 share the high entry of index (2n) >> 7, which
      // advances by 2 THREADS / kTwLo per u; their low entries are those of
      // 2 tid and 2 tid + 1 for every u)
      float2 *const wb = s_buf + lds_pos<kBigPad>(tid);
      const float2 *const hb = s_tw + ((2 * tid) >> 7);
      const float2 l0 = s_tw[THI + ((2 * tid) & (kTwLo - 1))], l1 = s_tw[THI + ((2 * tid + 1) & (kTwLo - 1))];
#pragma unroll
      for (int u = 0; u < IPT; ++u) {
        const float2 h = hb[u * (2 * THREADS / kTwLo)];
        const float c0 = __builtin_fmaf(h.x, l0.x, -h.y * l0.y), c1 = __builtin_fmaf(h.x, l1.x, -h.y * l1.y);
        wb[lds_step<kBigPad>(u * THREADS)] = make_float2(xs[u][0] * __builtin_fmaf(-0.5f, c0, 0.5f),
                                                         xs[u][1] * __builtin_fmaf(-0.5f, c1, 0.5f));
      }
    } else if (have) {
      float2 ws[IPT];
#pragma unroll
      for (int u = 0; u < IPT; ++u) {   // global loads (win2 is opaque, so its address space is restated)
        const __attribute__((address_space(1))) float *wf =
            reinterpret_cast<const __attribute__((address_space(1))) float *>(reinterpret_cast<uint64_t>(win2));
        ws[u] = make_float2(wf[2 * (tid + u * THREADS)], wf[2 * (tid + u * THREADS) + 1]);
      }
      float2 *const wb = s_buf + lds_pos<kBigPad>(tid);
#pragma unroll
      for (int u = 0; u < IPT; ++u) wb[lds_step<kBigPad>(u * THREADS)] = make_float2(xs[u][0] * ws[u].x, xs[u][1] * ws[u].y);
    } else {
      big_padded_frame<IN, M, THREADS>(reinterpret_cast<const IN *>(a.pcm) + b * T, win2, (int64_t)fr * a.hop - a.pad, T,
                                       a.sig_pad, a.pad_mode, tid, s_buf);
    }
    __syncthreads();

    // 2. M-point complex FFT: exp(-2 pi i j / M) = exp(-2 pi i 2j / N)
    __builtin_amdgcn_s_setprio(0);
    run_fft<M, 1, THREADS, kBigPad>(s_buf, BigTw<THI, TSTEP, TNS>{s_tw, s_tab}, typename BigCfg<NFFT>::Rad{}, tid);

    // 3. split into the real spectrum; power over the same LDS
    constexpr int NU = M / 2 + 1;
    constexpr int UPT = (NU + THREADS - 1) / THREADS;
    // point k = tid + THREADS u: Z[k] and Z[M - k] at one base each plus a
    // compile-time step (THREADS is a multiple of 2^kBigPad); the twiddle
    // exp(-2 pi i k / N) is hi[k >> 7] lo[tid mod kTwLo]
    float pk[UPT], pmk[UPT];
    const float2 *const zkb = s_buf + lds_pos<kBigPad>(tid);
    const float2 *const zcb = s_buf + lds_pos<kBigPad>(M - tid);   // one past the buffer's points for tid = 0
    const float2 *const wh = s_tw + (tid >> 7);
    const float2 wl = s_tw[THI + (tid & (kTwLo - 1))];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int k = tid + u * THREADS;
      pk[u] = pmk[u] = 0.0f;
      if (k < NU) {
        const float2 zk = zkb[lds_step<kBigPad>(u * THREADS)];
        const float2 zc = cconj(k == 0 ? s_buf[0] : zcb[-lds_step<kBigPad>(u * THREADS)]);
        const float2 Y = cadd(zk, zc), D = csub(zk, zc);
        const float2 V = cmul(cmul(wh[u * (THREADS / kTwLo)], wl), D);
        pk[u] = (Y.x + V.y) * (Y.x + V.y) + (Y.y - V.x) * (Y.y - V.x);
        pmk[u] = (Y.x - V.y) * (Y.x - V.y) + (Y.y + V.x) * (Y.y + V.x);
      }
    }
    __syncthreads();
    float *P = reinterpret_cast<float *>(s_buf);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int k = tid + u * THREADS;
      if (k < NU) {
        P[k] = pk[u];
        if (k != M / 2) P[M - k] = pmk[u];
      }
    }
    __syncthreads();
    if (a.power != 2.0f) {
      const float e = 0.5f * a.power;
      for (int i = tid; i <= M; i += THREADS) P[i] = powf(P[i] * a.pre_scale, e);
      __syncthreads();
    }

    __builtin_amdgcn_s_setprio(1);
    // the next frame's samples, in flight during the mel sums
    if constexpr (PREFETCH) {
      have = tile + G < n_tiles && interior(nfr);
      if (have) load_interior(nb, nfr, tid);
    }

    // 4. mel: each band's group of Lb lanes strides over its bins in pairs
    //    of adjacent bins; the group's partial sums meet at its first lane.
    //    The frame's largest and smallest mel values are kept on their bit
    //    patterns (positive floats order as unsigned integers).
    uint32_t vmaxb = 0u, vminb = 0x7f800000u;
    OUT *__restrict__ out = reinterpret_cast<OUT *>(a.out) + b * (int64_t)NM * F;
    auto mel = [&](const float *wsrc) {
      const int m = lane_ent & 255, h = (lane_ent >> 8) & 255, Lb = lane_ent >= 0 ? 1 << (lane_ent >> 16) : 1;
      float acc0 = 0.0f, acc1 = 0.0f;
      if (lane_ent >= 0) {
        // pairs of adjacent bins 2h + 2 Lb t and the next one, in two
        // chains: both reads of a chain's step come off one pointer (an
        // immediate offset for the second), and the pointers step by 2 Lb;
        // an odd band's last bin is the single one at the end
        const int wd = s_width[m];
        const float *pr = P + s_start[m] + 2 * h;
        const float *wr = wsrc + s_off[m] + 2 * h;
        int j = 2 * h;
        for (; j + 1 < wd; j += 2 * Lb) {
          acc0 = __builtin_fmaf(wr[0], pr[0], acc0);
          acc1 = __builtin_fmaf(wr[1], pr[1], acc1);
          wr += 2 * Lb;
          pr += 2 * Lb;
        }
        if (j < wd) acc0 = __builtin_fmaf(wr[0], pr[0], acc0);
      }
      // the group's partial sums meet at its first lane (h = 0): step o
      // adds the partial sum of lane + o -- a DPP row shift within the
      // 16-lane row for o <= 8, a swizzle within 32 lanes for 16, a permute
      // across the wave for 32 -- and adds nothing where o >= Lb (the
      // partner belongs to another group)
      float acc = acc0 + acc1;
      auto from_plus = [&](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xf, 0xf, true));
      };
      {
        float t;
        t = from_plus(acc, std::integral_constant<int, 0x101>{});   // row_shl:1
        acc = 1 < Lb ? acc + t : acc;
        t = from_plus(acc, std::integral_constant<int, 0x102>{});   // row_shl:2
        acc = 2 < Lb ? acc + t : acc;
        t = from_plus(acc, std::integral_constant<int, 0x104>{});   // row_shl:4
        acc = 4 < Lb ? acc + t : acc;
        t = from_plus(acc, std::integral_constant<int, 0x108>{});   // row_shl:8
        acc = 8 < Lb ? acc + t : acc;
        t = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(acc), (16 << 10) | 0x1f));   // lane ^ 16
        acc = 16 < Lb ? acc + t : acc;
        t = __int_as_float(__builtin_amdgcn_ds_bpermute(perm32, __float_as_int(acc)));   // lane + 32
        acc = 32 < Lb ? acc + t : acc;
      }
      if (lane_ent >= 0 && h == 0) {
        if (a.mel_out) {
          store_out(out + (int64_t)m * F + fr, acc * a.mel_scale);
        } else {
          const float v = floor_1e10(acc * a.mel_scale);
          const float o = logmel_of(v);
          vmaxb = max(vmaxb, __float_as_uint(v));
          vminb = min(vminb, __float_as_uint(v));
          store_out(out + (int64_t)m * F + fr, o);
        }
      }
    };
    if (w_in_lds) mel(s_w);
    else mel(a.csr_w);

    // 5. frame statistics: each wave's extremes to LDS; the barrier (which
    //    also keeps the next frame's samples out of the power tile until
    //    every band has read it) lets thread 0 combine them while the others
    //    go on to the next frame (s_red is next written at that frame's end)
    {
      const uint32_t wmx = wave_umax(vmaxb), wmn = wave_umin(vminb);
      if ((tid & 63) == 0) {
        s_red[tid >> 6] = __uint_as_float(wmx);
        s_red[NW + (tid >> 6)] = __uint_as_float(wmn);
      }
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t mx = 0u, mn = 0x7f800000u;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        mx = max(mx, __float_as_uint(s_red[i]));
        mn = min(mn, __float_as_uint(s_red[NW + i]));
      }
      a.tile_max[tile] = __uint_as_float(mx);
      a.tile_min[tile] = __uint_as_float(mn);
    }
    cb = nb;
    cfr = nfr;
  }
}

template <int NFFT>
static hipError_t launch_big(const PcmKernelArgs &k, bool i16, bool f16, int64_t n_tiles, int n_cu, hipStream_t s,
                             const LaunchTiming *tm) {
  constexpr int THREADS = BigCfg<NFFT>::THREADS;
  const int64_t slots = (int64_t)n_cu * BigCfg<NFFT>::WGS;
  const int64_t n_wg = n_tiles < slots ? n_tiles : slots;
  const dim3 grid((unsigned)n_wg), block(THREADS);
  if (!i16 && !f16) LM_LAUNCH(tm, (pcm_big_kernel<NFFT, float, float>), grid, block, 0, s, k, n_tiles);
  else if (!i16 && f16) LM_LAUNCH(tm, (pcm_big_kernel<NFFT, float, __half>), grid, block, 0, s, k, n_tiles);
  else if (i16 && !f16) LM_LAUNCH(tm, (pcm_big_kernel<NFFT, int16_t, float>), grid, block, 0, s, k, n_tiles);
  else LM_LAUNCH(tm, (pcm_big_kernel<NFFT, int16_t, __half>), grid, block, 0, s, k, n_tiles);
  return hipGetLastError();
}

template <int NFFT, bool PAIRED = false>
static hipError_t launch_n(const PcmKernelArgs &k, bool i16, bool f16, int64_t n_tiles, hipStream_t s,
                           const LaunchTiming *tm) {
  constexpr int THREADS = PcmCfg<NFFT>::THREADS;
  const dim3 grid((unsigned)n_tiles), block(THREADS);
  if (!i16 && !f16) LM_LAUNCH(tm, (pcm_logmel_kernel<NFFT, float, float, PAIRED>), grid, block, 0, s, k);
  else if (!i16 && f16) LM_LAUNCH(tm, (pcm_logmel_kernel<NFFT, float, __half, PAIRED>), grid, block, 0, s, k);
  else if (i16 && !f16) LM_LAUNCH(tm, (pcm_logmel_kernel<NFFT, int16_t, float, PAIRED>), grid, block, 0, s, k);
  else LM_LAUNCH(tm, (pcm_logmel_kernel<NFFT, int16_t, __half, PAIRED>), grid, block, 0, s, k);
  return hipGetLastError();
}

static int generic_frames_per_tile(int n_fft) {
  switch (n_fft) {
    case 400: return PcmCfg<400>::FPB;
    case 64: return PcmCfg<64>::FPB;
    case 128: return PcmCfg<128>::FPB;
    case 256: return PcmCfg<256>::FPB;
    case 512: return PcmCfg<512>::FPB;
    case 1024: return PcmCfg<1024>::FPB;
    case 2048: return PcmCfg<2048>::FPB;
    case 4096: return PcmCfg<4096>::FPB;
    case 8192: return PcmCfg<8192>::FPB;
    case 16384: return PcmCfg<16384>::FPB;
    default: return 0;
  }
}

static bool use_pcm400(const lm_plan *p, bool in_i16) {
  return (p->fft_variant == LM_FFT_AUTO || p->fft_variant == LM_FFT_SPLIT_MFMA) && pcm400_supported(p, in_i16);
}

std::string pcm_kernel_summary(const lm_plan *p, bool in_i16) {
  if (use_pcm400(p, in_i16)) return pcm400_summary(p);
  char buf[256];
  if (p->n_fft >= 8192) {
    std::snprintf(buf, sizeof buf,
                  "pcm_big_kernel<%d>: one frame per step of a %d-thread workgroup, %d persistent workgroup%s per "
                  "compute unit walking frames; mel on lane groups of up to 64 per band",
                  p->n_fft, big_threads(p->n_fft), p->n_fft == 8192 ? BigCfg<8192>::WGS : BigCfg<16384>::WGS,
                  (p->n_fft == 8192 ? BigCfg<8192>::WGS : BigCfg<16384>::WGS) > 1 ? "s" : "");
  } else if (p->n_fft == 400) {
    std::snprintf(buf, sizeof buf, "pcm_logmel_kernel<400>%s: %d frames per workgroup of 512 threads, %s",
                  p->fft_variant == LM_FFT_PAIRED ? " (paired)" : "", PcmCfg<400>::FPB,
                  p->fft_variant == LM_FFT_PAIRED ? "two frames per 400-point complex FFT"
                                                  : "200-point complex FFT per frame (8 x 5 x 5) and untangle");
  } else {
    std::snprintf(buf, sizeof buf,
                  "pcm_logmel_kernel<%d>: %d frames per workgroup of 512 threads, %d-point complex FFT per frame "
                  "in LDS passes and untangle; mel on split lanes",
                  p->n_fft, generic_frames_per_tile(p->n_fft), p->n_fft / 2);
  }
  return buf;
}

StatLayout pcm_stat_layout(const lm_plan *p, bool in_i16) {
  if (use_pcm400(p, in_i16)) return pcm400_stat_layout(p);
  StatLayout st;   // one entry per tile over all bands
  st.frames_per_tile = generic_frames_per_tile(p->n_fft);
  st.band_h = p->n_mels;
  return st;
}

bool pcm_skips_empty_bands(const lm_plan *p, bool in_i16) {
  return !use_pcm400(p, in_i16) && p->n_fft < 8192 && p->output == LM_OUTPUT_LOGMEL && p->dt.n_empty > 0;
}

hipError_t launch_pcm(const lm_plan *p, const PcmArgs &a, hipStream_t s, const LaunchTiming *tm) {
  if (use_pcm400(p, a.in_i16)) return launch_pcm400(p, a, s, tm);
  PcmKernelArgs k;
  k.pcm = a.pcm;
  k.T = a.n_samples;
  k.F = a.n_frames;
  k.tiles_per_clip = a.tiles_per_clip;
  k.hop = p->hop;
  k.pad = (p->center ? p->n_fft / 2 : 0) + (int)p->sig_pad;
  k.sig_pad = (int)p->sig_pad;
  k.pad_mode = p->pad_mode;
  k.power = p->power;
  // |2X|^2 = 4 |X|^2; int16 samples carry a 2^15 factor per |X|
  // (the normalisation's factor on |X|^2 joins them)
  const double in_scale2 = (a.in_i16 ? 1.0 / 1073741824.0 : 1.0) * power_scale2(p);   // 2^-30
  if (p->power == 2.0f) {
    k.mel_scale = (float)(0.25 * in_scale2);
    k.pre_scale = 1.0f;
  } else {
    k.mel_scale = 1.0f;
    k.pre_scale = (float)(0.25 * in_scale2);
  }
  k.mel_out = p->output == LM_OUTPUT_MEL;
  k.skip_empty = pcm_skips_empty_bands(p, a.in_i16);
  k.n_mels = p->n_mels;
  k.window = p->dt.window;
  k.twiddle = p->dt.twiddle;
  k.untangle = p->dt.untangle;
  k.tw2 = p->dt.tw2;
  k.mel_lanes = p->dt.mel_lanes;
  k.hann_tw = p->win_length == p->n_fft;
  k.csr_start = p->dt.csr_start;
  k.csr_width = p->dt.csr_width;
  k.csr_off = p->dt.csr_off;
  k.csr_w = p->dt.csr_w;
  k.nnz = p->dt.nnz;
  k.out = a.out;
  k.tile_min = a.tile_min;
  k.tile_max = a.tile_max;
  const int64_t n_tiles = a.n_clips * a.tiles_per_clip;
  const bool f16 = p->out_dtype == LM_F16;
  switch (p->n_fft) {
    case 400:
      if (p->fft_variant == LM_FFT_PAIRED) return launch_n<400, true>(k, a.in_i16, f16, n_tiles, s, tm);
      return launch_n<400>(k, a.in_i16, f16, n_tiles, s, tm);
    case 64: return launch_n<64>(k, a.in_i16, f16, n_tiles, s, tm);
    case 128: return launch_n<128>(k, a.in_i16, f16, n_tiles, s, tm);
    case 256: return launch_n<256>(k, a.in_i16, f16, n_tiles, s, tm);
    case 512: return launch_n<512>(k, a.in_i16, f16, n_tiles, s, tm);
    case 1024: return launch_n<1024>(k, a.in_i16, f16, n_tiles, s, tm);
    case 2048: return launch_n<2048>(k, a.in_i16, f16, n_tiles, s, tm);
    case 4096: return launch_n<4096>(k, a.in_i16, f16, n_tiles, s, tm);
    case 8192: return launch_big<8192>(k, a.in_i16, f16, n_tiles, p->n_cu, s, tm);
    case 16384: return launch_big<16384>(k, a.in_i16, f16, n_tiles, p->n_cu, s, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lm
