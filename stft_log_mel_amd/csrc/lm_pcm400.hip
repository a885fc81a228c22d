// PCM -> log-mel for n_fft = 400 (the speech front end: 25 ms frames at
// 16 kHz), using the matrix cores for the first FFT stage.
//
// Chain per frame (flashmel page, "How it works"; KBench task page
// "audio-mel-spectrogram-fused", "spec_md"): the windowed frame y[n] =
// w[n] x[n], n < 400, is split as n = n1 + 25 n2 (n1 < 25, n2 < 16) with bins
// k = 16 k1 + k2, so that
//   X[16 k1 + k2] = sum_n1 W25^(n1 k1) [ sum_n2 y[n1 + 25 n2] W400^(k2 (n1 + 25 n2)) ].
// The bracket (window, 16-point DFT and twiddle) is, for each n1, one real
// 16x16 matrix applied to 16 frames at once on the matrix cores
// (v_mfma_f32_16x16x32_f16, two per n1: the samples as two fp16 planes
// whose sum carries them exactly (int16) or to about 22 bits (float, with a
// per-sub-tile power-of-two scale), against the matrix as fp16 hi + lo
// parts, accumulated in fp32).  Since y is real, classes k2 and
// 16 - k2 are conjugate mirrors, so the matrix rows hold classes 1..7
// (real and imaginary parts) plus the two sums of y over even and over odd
// n2 -- from which classes 0 and 8, the bins that are multiples of 8, are a
// 50-point real DFT.  The output layout leaves lane (frame c, group g) with
// whole classes over all n1: group g < 3 holds classes g + 1 and 7 - g,
// group 3 holds class 4 and the even/odd sums.  The 25-point DFTs over n1
// then run in registers (5 x 5, Winograd 5-point modules); the 50-point
// real DFT is the 25-point complex DFT of z[m] = s[2m] + i s[2m+1] followed
// by its split into real-input bins.  |X|^2 goes to the wave's own power
// rows in LDS; the mel sums run on 4x4x1 matrix blocks (4 bands x 4 frames
// per bin, 16 blocks per instruction) over the bins each quad of bands
// touches; log10 after the 1e-10 floor, (L+4)/4, mel-major store (16
// consecutive frames per band).
//
// One workgroup of 8 waves per compute unit walks a contiguous range of
// 16-frame sub-tiles; its waves take every 8th one and never wait for each
// other (one barrier after the operand tables are staged).  Each wave
// fetches the next sub-tile's samples into registers while it computes the
// current one.  Per sub-tile it records the largest mel value of each of
// its four lane groups and, per 4-band group of every band block, the
// smallest mel value, for the clamp fix-up kernel.
#include <cstdio>
#include <type_traits>

#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSub = 16;                  // frames per wave step (the matrix-core N)
constexpr int kRow = kPcm400Row;          // power row stride
constexpr int kRegion = kSub * kRow;      // floats of LDS per wave: staged samples, then power rows
constexpr int kAmatH = 25 * 2 * 2 * 16;   // first-stage operands (8 fp16 each): [n1][part][g % 2][row]
constexpr int kLoff = 1694;               // dword offset of the second (low) fp16 plane in the region
constexpr int kMelWLds = 5632;            // LDS floats for the mel step weights
constexpr int kMelBatMax = kMelWLds / (16 * kMelBatch);   // mel batches that fit
// With the 25-point stage on the matrix cores its operand table (20 KB)
// takes LDS from the mel weights: up to 1920 of them (128 Slaney bands
// over 0-8 kHz need 1280).
constexpr int kA2Tab = 4 * 5 * 64;         // second-stage operands (8 fp16 each): [mt][step][lane]
constexpr int kMelWLds2 = 1920;
constexpr float kS2In = 0.0009765625f;     // 2^-10: first-stage values into fp16 range
constexpr int kStoreChunks = 13;           // 16-byte chunks of one (class, frame) second-stage input
// Wave priorities (s_setprio) of the phases of a sub-tile.  The two waves of
// a SIMD run different phases at a time; the staging, the first stage and
// the mel sums are chains of LDS reads, matrix products and stores, the
// 25-point DFTs long runs of independent VALU work.  With the DFTs at the
// lower priority, the SIMD issues the chain phases' instructions as soon as
// they are ready and fills their waits with the other wave's DFT work
// (main kernel -2.1% on the int16 headline batch; the reverse order +3.8%,
// the mel phase at the lower priority +3%).
constexpr int kPrioChain = 1, kPrioDft = 0;
constexpr int kPfI16 = 6, kPfF32 = 11;    // 16-byte sample loads per lane held for the next sub-tile

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

// four consecutive outputs (4-byte alignment suffices for a 16-byte store)
typedef float v4f_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ void store_out4(float *p, const float (&o)[4]) {
  *reinterpret_cast<v4f_a4 *>(p) = v4f_a4{o[0], o[1], o[2], o[3]};
}
__device__ __forceinline__ void store_out4(__half *p, const float (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) store_out(p + i, o[i]);
}

struct Args {
  const void *pcm;
  int64_t T, F;
  int S;                 // 16-frame sub-tiles per clip
  int64_t n_sub;         // sub-tiles of the whole call
  int per_wg;            // sub-tiles per workgroup
  int hop, pad, pad_mode;   // pad: center padding plus the signal's zero padding
  int sig_pad;             // the signal's zero padding (zeros before and after each clip)
  float power, pre_scale, mel_scale;
  int n_mels, n_melblk;
  int melw_n;            // mel step weight count (at most kMelWLds)
  int mel_batches;       // batches of kMelBatch steps over all band blocks
  uint64_t end_mask[2];  // bit b: batch b is the last of its band block
  int mel_out;           // 1: store the mel values themselves (no log tail)
  const v4f *a2;         // second-stage operands (the matrix-core 25-point form only)
  float *tile_max;
  // single pass only: this call's tag of the clip maxima, the parity of its
  // grid barrier counter, and the slots ([0], [1] barrier counters, [2 + b]
  // clip b's maximum), see grid_barrier
  uint32_t epoch;
  int parity;
  uint64_t *sync;
};

// Polls of the grid barrier before a workgroup gives up (about 0.1 s):
// with every workgroup resident (cooperative launch) the last one arrives
// within microseconds, so this bound only ends a wait that cannot succeed.
constexpr int kBarrierPolls = 1 << 20;

// Grid barrier of one call; one thread per workgroup.  The plan's calls
// alternate between two arrival counters (the host passes the parity), and
// each call zeroes the other counter once every workgroup has arrived, for
// the call after it (calls on one slot buffer never overlap: they are
// stream-ordered).  Arrivals are plain atomic adds, which the memory side
// performs without retries.  Every atomic here is relaxed: no plain store
// precedes the barrier, and the clip maxima are themselves atomics that
// have completed (their old values were consumed) before any arrival, so
// no release fence -- on this chip a write-back of the XCD's L2 -- is
// needed.  Returns false if the wait ran out of polls.
__device__ bool grid_barrier(uint64_t *cnt, int parity, uint32_t n) {
  const uint64_t before = __hip_atomic_fetch_add(cnt + parity, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (before + 1 >= n) {   // the last arrival
    __hip_atomic_store(cnt + (parity ^ 1), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  for (int i = 0; i < kBarrierPolls; ++i) {
    if (__hip_atomic_load(cnt + parity, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(int16_t v) { return (float)(int)v; }

// LDS layout of the staged span, two fp16 planes (below) in which samples
// 2d and 2d + 1 share dword d.  With SK (hop = 160 samples = 80 dwords), 4
// pad dwords follow every hop, so the 16 frame starts of a wave, 84 dwords
// apart, fall on distinct bank quads; without, the span is dense.  A hop is
// a multiple of 4 dwords, so 16-byte chunks never straddle a pad.
template <bool SK>
__device__ __forceinline__ int span_dw(int d) {
  return SK ? d + 4 * (d / 80) : d;
}

// int16 samples are staged as two fp16 planes with the dword layout above:
// H holds h = (x - (x mod 64)) / 64 in [-512, 511] and L holds (x mod 64) /
// 64, so x / 64 = h + l / 64 exactly.  A dword of two samples converts with
// integer masks into the fp16 bit patterns 1024 + (h + 512) and 1024 + l
// (exponent 10, integer mantissa), then one packed fp16 operation each.
// kLoff is 2 mod 4 dwords, so the two planes' readers use different bank
// quads.
__device__ __forceinline__ void split_i16(uint32_t x, uint32_t &H, uint32_t &L) {
  const uint32_t hb = (((x ^ 0x80008000u) >> 6) & 0x03ff03ffu) | 0x64006400u;
  const uint32_t lb = (x & 0x003f003fu) | 0x64006400u;
  const h2 hv = __builtin_bit_cast(h2, hb) + h2{(_Float16)-1536.0f, (_Float16)-1536.0f};
  const h2 lv = __builtin_bit_cast(h2, lb) * h2{(_Float16)0.015625f, (_Float16)0.015625f} +
                h2{(_Float16)-16.0f, (_Float16)-16.0f};
  H = __builtin_bit_cast(uint32_t, hv);
  L = __builtin_bit_cast(uint32_t, lv);
}

// float samples go to the same two planes, scaled per sub-tile by an exact
// 2^e that puts the span's largest magnitude in [256, 512) (the range of
// x / 64 for int16): H holds the nearest fp16 of x 2^e and L the nearest
// fp16 of the remainder, so H + L = x 2^e to about 22 significant bits
// (2^-24 absolute for the smallest samples).  The mel sums take the exact
// 2^-2e back.
__device__ __forceinline__ void split_f32(float x0, float x1, float sc, uint32_t &H, uint32_t &L) {
  const float a = x0 * sc, b = x1 * sc;
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  const h2 hv{ha, hb}, lv{(_Float16)(a - (float)ha), (_Float16)(b - (float)hb)};
  H = __builtin_bit_cast(uint32_t, hv);
  L = __builtin_bit_cast(uint32_t, lv);
}

// e with 256 <= m 2^e < 512 for the largest magnitude m of a span (0 for a
// silent or non-finite span), kept within [-100, 100]
__device__ __forceinline__ int scale_exponent(float m) {
  if (!(m > 0.0f) || !(m < __builtin_huge_valf())) return 0;
  const int ex = __builtin_amdgcn_frexp_expf(m);   // m = f 2^ex, 1/2 <= f < 1
  return min(100, max(-100, 9 - ex));
}

template <typename IN>
struct Prefetch {
  static constexpr int N = sizeof(IN) == 2 ? kPfI16 : kPfF32;
  u4 v[N];
  int q_lo, q_hi;   // 16-byte chunks [q_lo, q_hi) of the span were loaded (uniform)
};

// Where sub-tile gs reads: clip b, samples [s_begin, s_begin + span) of it
// (s_begin < 0 or past the end: padding).
struct SubTile {
  int64_t b, s;
  int64_t s_begin;
};
__device__ __forceinline__ SubTile locate(const Args &a, int64_t gs) {
  SubTile t;
  t.b = gs / a.S;
  t.s = gs - t.b * a.S;
  t.s_begin = t.s * kSub * a.hop - a.pad;
  return t;
}
// The sub-tile n places after t (uniform; no division: at most n clip steps)
__device__ __forceinline__ SubTile advance(const Args &a, SubTile t, int n) {
  t.s += n;
  while (t.s >= a.S) {
    t.s -= a.S;
    ++t.b;
  }
  t.s_begin = t.s * kSub * a.hop - a.pad;
  return t;
}

// Issue the 16-byte loads of every chunk of the span that lies inside the
// clip (the span must start 16-byte aligned); false if it does not, then
// the whole span takes the padded path.
template <typename IN>
__device__ __forceinline__ bool prefetch(const Args &a, const IN *__restrict__ pcm, const SubTile &t, int span,
                                         Prefetch<IN> &pf) {
  constexpr int PER = 16 / sizeof(IN);   // samples per chunk
  const int n4 = (span + PER - 1) / PER;
  const IN *src = pcm + t.b * a.T + t.s_begin;
  if (n4 > 64 * Prefetch<IN>::N || (reinterpret_cast<uintptr_t>(src) & 15)) return false;
  // chunks q with 0 <= s_begin + PER q and s_begin + PER (q + 1) <= T
  const int64_t lo = t.s_begin < 0 ? (-t.s_begin + PER - 1) / PER : 0;
  const int64_t hi = (a.T - t.s_begin) / PER;
  pf.q_lo = (int)min(lo, (int64_t)n4);
  pf.q_hi = (int)max((int64_t)pf.q_lo, min(hi, (int64_t)n4));
  const u4 *s4 = reinterpret_cast<const u4 *>(src);
  const int lane = threadIdx.x & 63;
  // one opaque uniform base per 4 KB of chunks: every load is then that base
  // plus 16 lane plus an immediate offset below 4 KB, and none needs a
  // freshly computed address register (which the compiler takes from a
  // load destination and guards with a wait for all memory accesses)
  typedef const u4 __attribute__((address_space(1))) *gptr;
  gptr base[(Prefetch<IN>::N + 3) / 4];
#pragma unroll
  for (int h = 0; h < (Prefetch<IN>::N + 3) / 4; ++h) {
    base[h] = (gptr)(s4 + 256 * h);
    asm volatile("" : "+s"(base[h]));
  }
#pragma unroll
  for (int i = 0; i < Prefetch<IN>::N; ++i) {
    const int q = lane + 64 * i;
    if (q >= pf.q_lo && q < pf.q_hi) pf.v[i] = base[i >> 2][lane + 64 * (i & 3)];
  }
  return true;
}

constexpr int kPadBatch = 8;   // dwords per lane with loads in flight together

// Padded path for plane dwords [d_begin, d_end) of the span (samples 2d,
// 2d + 1): each sample by index arithmetic (positions past the end of the
// clip's last frame read as 0), kPadBatch dwords per lane with all their
// loads issued before any is used.  Float samples are scaled by 2^e.
template <typename IN, bool SK>
__device__ __forceinline__ void stage_padded(const Args &a, const IN *__restrict__ pcm, const SubTile &t, int d_begin,
                                             int d_end, float *R, int e) {
  const IN *x = pcm + t.b * a.T;
  const int64_t s_limit = (a.F - 1) * (int64_t)a.hop - a.pad + 400;
  uint32_t *d32 = reinterpret_cast<uint32_t *>(R);
  const float sc = __builtin_amdgcn_ldexpf(1.0f, e);
  const int lane = threadIdx.x & 63;
  for (int d0 = d_begin + lane; d0 < d_end; d0 += 64 * kPadBatch) {
    float v[kPadBatch][2];
#pragma unroll
    for (int u = 0; u < kPadBatch; ++u)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int64_t j = t.s_begin + (int64_t)(d0 + 64 * u) * 2 + k;
        const int64_t src = (d0 + 64 * u < d_end && j < s_limit) ? signal_source(j, a.T, a.sig_pad, a.pad_mode) : -1;
        v[u][k] = src >= 0 ? to_f(x[src]) : 0.0f;
      }
#pragma unroll
    for (int u = 0; u < kPadBatch; ++u) {
      if (d0 + 64 * u >= d_end) break;
      uint32_t H, L;
      if (sizeof(IN) == 2) {
        const uint32_t w = (uint32_t)(uint16_t)(int16_t)(int)v[u][0] | ((uint32_t)(uint16_t)(int16_t)(int)v[u][1] << 16);
        split_i16(w, H, L);
      } else {
        split_f32(v[u][0], v[u][1], sc, H, L);
      }
      const int o = span_dw<SK>(d0 + 64 * u);
      d32[o] = H;
      d32[kLoff + o] = L;
    }
  }
}

// Largest magnitude of the lane's samples among plane dwords [d_begin,
// d_end) of the span, by the padded path's index arithmetic (float input).
template <typename IN>
__device__ __forceinline__ float padded_absmax(const Args &a, const IN *__restrict__ pcm, const SubTile &t, int d_begin,
                                               int d_end) {
  const IN *x = pcm + t.b * a.T;
  const int64_t s_limit = (a.F - 1) * (int64_t)a.hop - a.pad + 400;
  float m = 0.0f;
  for (int d = d_begin + (threadIdx.x & 63); d < d_end; d += 64)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t j = t.s_begin + (int64_t)d * 2 + k;
      const int64_t src = j < s_limit ? signal_source(j, a.T, a.sig_pad, a.pad_mode) : -1;
      if (src >= 0) m = fmaxf(m, fabsf(to_f(x[src])));
    }
  return m;
}

// The prefetched chunks into the wave's region, then the span's dwords
// outside them by the padded path; returns the scale exponent e of float
// input (0 for int16).
template <typename IN, bool SK>
__device__ __forceinline__ int put_prefetch(const Args &a, const IN *__restrict__ pcm, const SubTile &t,
                                            const Prefetch<IN> &pf, int span, float *R) {
  constexpr bool kI16 = sizeof(IN) == 2;
  constexpr int DPC = 8 / sizeof(IN);   // plane dwords per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int ndw = span / 2;
  const int lo_end = min(DPC * pf.q_lo, ndw), hi_begin = DPC * pf.q_hi;
  u4 *d4 = reinterpret_cast<u4 *>(R);
  u2 *h2p = reinterpret_cast<u2 *>(R);
  u2 *l2p = reinterpret_cast<u2 *>(R + kLoff);
  // every prefetch register is retired here, also those the predicated
  // writes below skip, so no load stays in flight into the next prefetch
#pragma unroll
  for (int i = 0; i < Prefetch<IN>::N; ++i) asm volatile("" ::"v"(pf.v[i]));
  int e = 0;
  if constexpr (!kI16) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < Prefetch<IN>::N; ++i) {
      const int q = lane + 64 * i;
      if (q >= pf.q_lo && q < pf.q_hi)
#pragma unroll
        for (int k = 0; k < 4; ++k) m = fmaxf(m, fabsf(__uint_as_float(pf.v[i][k])));
    }
    if (pf.q_lo > 0) m = fmaxf(m, padded_absmax<IN>(a, pcm, t, 0, lo_end));
    if (hi_begin < ndw) m = fmaxf(m, padded_absmax<IN>(a, pcm, t, hi_begin, ndw));
    e = scale_exponent(__uint_as_float(wave_umax(__float_as_uint(m))));   // m >= 0
  }
  const float sc = __builtin_amdgcn_ldexpf(1.0f, e);
#pragma unroll
  for (int i = 0; i < Prefetch<IN>::N; ++i) {
    const int q = lane + 64 * i;
    if (q >= pf.q_lo && q < pf.q_hi) {
      const int o = span_dw<SK>(DPC * q);
      if constexpr (kI16) {
        u4 H, L;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t hh, ll;
          split_i16(pf.v[i][k], hh, ll);
          H[k] = hh;
          L[k] = ll;
        }
        d4[o / 4] = H;
        l2p[o / 2] = u2{L[0], L[1]};
        l2p[o / 2 + 1] = u2{L[2], L[3]};
      } else {
        uint32_t H0, L0, H1, L1;
        split_f32(__uint_as_float(pf.v[i][0]), __uint_as_float(pf.v[i][1]), sc, H0, L0);
        split_f32(__uint_as_float(pf.v[i][2]), __uint_as_float(pf.v[i][3]), sc, H1, L1);
        h2p[o / 2] = u2{H0, H1};
        l2p[o / 2] = u2{L0, L1};
      }
    }
  }
  if (pf.q_lo > 0) stage_padded<IN, SK>(a, pcm, t, 0, lo_end, R, e);
  if (hi_begin < ndw) stage_padded<IN, SK>(a, pcm, t, hi_begin, ndw, R, e);
  return e;
}

// Rank of workgroup id w among G workgroups when consecutive ids are dealt
// to the kXcds XCDs in turn: XCD x = w mod kXcds holds ranks [start_x,
// start_x + count_x), so each XCD's workgroups take consecutive ranks.
__device__ __forceinline__ int xcd_rank(int w, int G) {
  const int x = w % kXcds, j = w / kXcds;
  const int q = G / kXcds, r = G % kXcds;   // XCDs below r hold q + 1 workgroups
  return x * q + min(x, r) + j;
}

template <typename IN, typename OUT, bool SK, bool RES, bool S2>
__global__ void __launch_bounds__(kThreads, 1)
pcm400_kernel(Args a, const v4f *__restrict__ amat, const int32_t *__restrict__ melblk_meta,
              const float *__restrict__ melblk_w, OUT *__restrict__ out, float *__restrict__ tile_min) {
  static_assert(!(S2 && RES), "the single pass keeps the register 25-point form");
  constexpr bool kI16 = sizeof(IN) == 2;
  constexpr int kTab = kAmatH;
  constexpr int kMelW = S2 ? kMelWLds2 : kMelWLds;
  constexpr int kBatMax = kMelW / (16 * kMelBatch);
  constexpr int kTab2 = S2 ? kA2Tab : 0;
  __shared__ v4f s_amat[kAmatH];   // fp16 operands, 8 per entry
  __shared__ v4f s_a2[S2 ? kA2Tab : 1];   // second-stage fp16 operands
  __shared__ float2 s_w50[16];            // W50^q, q < 16 (the 50-point split)
  __shared__ __attribute__((aligned(16))) float s_melw[kMelW];
  __shared__ __attribute__((aligned(16))) float s_reg[kWaves * kRegion];
  __shared__ int s_bat[4 * kBatMax];   // per mel batch and quad: first bin

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const IN *__restrict__ pcm = reinterpret_cast<const IN *>(a.pcm);
  float *R = s_reg + wv * kRegion;
  const int hop = a.hop;
  const int span = (kSub - 1) * hop + 400;
  const int c = lane & 15, g = lane >> 4;
  const bool g3 = g == 3;
  const int NM = a.n_mels, NB = a.n_melblk;
  const int64_t F = a.F;

  // workgroup ids go to the XCDs in turn (each with its own L2); dealing the
  // sub-tile ranges so that each XCD's workgroups take consecutive ranges
  // keeps the output lines shared by neighbouring ranges (a 16-frame run is
  // 64 bytes of a band row) and the input overlap in one L2
  const int64_t wg0 = (int64_t)xcd_rank(blockIdx.x, gridDim.x) * a.per_wg;
  const int64_t wg_end = min(wg0 + a.per_wg, a.n_sub);
  // the waves start on sub-tiles wg0 + wv and then claim the range's next
  // ones from one LDS counter, so that a wave that runs ahead (the older wave
  // of a SIMD wins the issue slots both want) takes more of them and the
  // waves of a compute unit end together
  __shared__ int s_next;
  int64_t gs = wg0 + wv;
  SubTile tc = locate(a, gs);   // the sub-tile gs (clip, index, first sample)
  Prefetch<IN> pf;
  bool have;
  {
    // every table load and the first sub-tile's samples in flight at once
    // (one round trip before the first barrier)
    constexpr int PER = (kTab + kThreads - 1) / kThreads;
    constexpr int PER2 = (kTab2 + kThreads - 1) / kThreads;
    constexpr int WPT = (kMelW + kThreads - 1) / kThreads;
    static_assert(4 * kBatMax <= kThreads, "one batch-table entry per thread");
    v4f v[PER], v2[PER2 > 0 ? PER2 : 1];
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (tid + u * kThreads < kTab) v[u] = amat[tid + u * kThreads];
#pragma unroll
    for (int u = 0; u < PER2; ++u)
      if (tid + u * kThreads < kTab2) v2[u] = a.a2[tid + u * kThreads];
    const int bat = tid < 4 * a.mel_batches ? melblk_meta[tid] : 0;
    float w[WPT];
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int i = tid + u * kThreads;
      w[u] = i < a.melw_n ? melblk_w[i] : 0.0f;
    }
    have = gs < wg_end && prefetch<IN>(a, pcm, tc, span, pf);
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (tid + u * kThreads < kTab) s_amat[tid + u * kThreads] = v[u];
    if constexpr (S2) {
#pragma unroll
      for (int u = 0; u < PER2; ++u)
        if (tid + u * kThreads < kTab2) s_a2[tid + u * kThreads] = v2[u];
      if (tid < 16) s_w50[tid] = w400(8 * tid);
    }
    if (tid < 4 * a.mel_batches) s_bat[tid] = bat & 0xffff;
    if (tid == 0) s_next = kWaves;
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
      const int i = tid + u * kThreads;
      if (i < a.melw_n) s_melw[i] = w[u] * a.mel_scale;
    }
    __syncthreads();
  }

  // single pass (RES): each wave has at most one sub-tile.  It stores its
  // log-mel values as they come, publishes its largest mel value and meets
  // the other workgroups at the grid barrier; its power rows stay in its LDS
  // region meanwhile, so a wave holding a value below its clip's floor runs
  // the mel sums again from them and overwrites its values floored.
  __shared__ int s_ok;
  __shared__ int64_t s_clip[kWaves];
  __shared__ uint32_t s_max[kWaves];
  auto res_sync = [&](uint32_t vmaxb, int64_t b) -> float {
    // the wave's largest mel value, then one atomic per (workgroup, clip):
    // the first wave of each run of waves on the same clip (a workgroup's
    // sub-tiles are consecutive) takes the run's maximum to the clip's slot
    uint32_t m = 0u;
    if (b >= 0) {
      m = row_max16(vmaxb);
      m = max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
              max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
    }
    if (lane == 0) {
      s_clip[wv] = b;
      s_max[wv] = m;
    }
    __syncthreads();
    if (tid < kWaves) {
      const int64_t cb_ = s_clip[tid];
      if (cb_ >= 0 && (tid == 0 || s_clip[tid - 1] != cb_)) {
        uint32_t mm = s_max[tid];
        for (int w = tid + 1; w < kWaves && s_clip[w] == cb_; ++w) mm = max(mm, s_max[w]);
        // (epoch, bits) orders a stale slot of an earlier call below every value of this one
        const uint64_t prev = __hip_atomic_fetch_max(a.sync + 2 + cb_, ((uint64_t)a.epoch << 32) | mm,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // consuming the old value makes the wave wait until the atomic has
        // been performed, before the barrier below lets any arrival go out
        asm volatile("" ::"v"((uint32_t)prev));
      }
    }
    __syncthreads();
    if (tid == 0) s_ok = grid_barrier(a.sync, a.parity, gridDim.x) ? 1 : 0;
    __syncthreads();
    if (b < 0) return 0.0f;
    const uint64_t w = __hip_atomic_load(a.sync + 2 + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the clip's floor in output units; a barrier that ran out of polls gives NaN
    return s_ok ? logmel_of(fmaxf(__uint_as_float((uint32_t)w), 1e-10f)) - 2.0f : __builtin_nanf("");
  };
  bool res_done = false;

  int64_t gs_next = wg_end;
  for (; gs < wg_end; gs = gs_next) {
    if constexpr (!S2) __builtin_amdgcn_s_setprio(kPrioChain);
    // 0. claim the wave's next sub-tile (the LDS atomic's return overlaps the
    //    staging below); the single pass keeps one sub-tile per wave
    int claim = 0;
    if constexpr (!RES) {
      if (lane == 0) claim = atomicAdd(&s_next, 1);
    }
    // 1. this sub-tile's samples into the wave's region (LDS operations of
    //    one wave complete in order, so no barrier is needed around them)
    int esc;   // float input: the sub-tile's scale exponent (uniform)
    if (have) {
      esc = put_prefetch<IN, SK>(a, pcm, tc, pf, span, R);
    } else {
      // no prefetch load is in flight on this path (prefetch returned false),
      // which the compiler cannot tell: retire the registers here as well
#pragma unroll
      for (int i = 0; i < Prefetch<IN>::N; ++i) asm volatile("" ::"v"(pf.v[i]));
      esc = kI16 ? 0 : scale_exponent(__uint_as_float(wave_umax(__float_as_uint(padded_absmax<IN>(a, pcm, tc, 0, span / 2)))));
      stage_padded<IN, SK>(a, pcm, tc, 0, span / 2, R, esc);
    }
    esc = __builtin_amdgcn_readfirstlane(esc);
    // (the single pass has one sub-tile per wave: nothing to prefetch)
    const SubTile t = tc;
    gs_next = RES ? wg_end : wg0 + __builtin_amdgcn_readfirstlane(claim);
    // the next sub-tile's samples: loads issued here, before the transform
    // (the matrix-core 25-point form issues them after its second stage,
    // where its registers are free again)
    auto issue_prefetch = [&]() {
      if (gs_next < wg_end) {
        const int64_t n = gs_next - gs;   // >= 1 (uniform)
        tc = n <= a.S ? advance(a, tc, (int)n) : locate(a, gs_next);
        have = prefetch<IN>(a, pcm, tc, span, pf);
      } else {
        have = false;
      }
    };
    issue_prefetch();

    // 2. window + 16-point DFT + twiddle on the matrix cores: D[n1] = A[n1] x[n1],
    //    per n1 two fp16 products (matrix hi and lo parts) over k-slots e of
    //    lane (c, g): sample n1 + 25 n2 of frame c, n2 = 4 (e / 2) + e % 2 +
    //    2 (g % 2), from plane H (groups 0, 3) or L (groups 1, 2).  The run of
    //    group g % 2 = 1 starts 50 samples (25 dwords) later; in the skewed
    //    layout it is another 4 dwords later where the samples of the two
    //    groups lie on different sides of a hop boundary.
    v4f D[25];
#pragma unroll
    for (int n1 = 0; n1 < 25; ++n1) D[n1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    {
      const int h = g & 1;
      const _Float16 *pl = reinterpret_cast<const _Float16 *>(R + ((g == 0 || g == 3) ? 0 : kLoff));
      const _Float16 *p0 = pl + 2 * ((SK ? 84 * c : (c * hop) >> 1) + 25 * h);
      const _Float16 *p1 = p0 + 8 * h;
      const v8h *tab = reinterpret_cast<const v8h *>(s_amat) + 16 * h + (lane & 15);
#pragma unroll
      for (int n1 = 0; n1 < 25; ++n1) {
        v8h B;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r0 = n1 + 25 * (4 * (e >> 1) + (e & 1));   // sample within the frame for g % 2 = 0
          const int pad0 = SK ? 4 * ((r0 >= 160) + (r0 >= 320)) : 0;
          const bool cross = SK && ((r0 < 160 && r0 + 50 >= 160) || (r0 < 320 && r0 + 50 >= 320));
          const int off = 2 * ((r0 >> 1) + pad0) + (r0 & 1);
          B[e] = (cross ? p1 : p0)[off];
        }
        const v8h Ah = tab[(n1 * 2 + 0) * 32], Al = tab[(n1 * 2 + 1) * 32];
        D[n1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, B, D[n1], 0, 0, 0);
        D[n1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, B, D[n1], 0, 0, 0);
      }
    }

    float *Rc = R + c * kRow;
    if constexpr (S2) {
      // 3'. The 25-point DFTs over n1 on the matrix cores, in two rounds.
      //     Round 0 takes each lane's rows 4g, 4g+1 (class g + 1), round 1
      //     its rows 4g+2, 4g+3 (class 7 - g), or for g = 3 the sequence
      //     s[i] = s[n1 + 25 e] (rows 14, 15) in natural order, so that
      //     z[m] = s[2m] + i s[2m+1].  A lane stores its class's 50 inputs
      //     (times 2^-10, into fp16 range) as fp16 hi and lo parts, 13
      //     chunks of 16 bytes, in the wave's region; the region's staged
      //     span has been read by then (one wave's LDS operations complete
      //     in order).  Then each of the round's four class jobs runs as
      //     products with the (job, frame) chunks as B operand (column =
      //     frame) against the DFT matrix (64 rows x five 32-wide steps,
      //     see the plan's table): lane (c, g) ends with quad q = 4 mt + g,
      //     i.e. Z[q] and Z[25 - q], of every job for frame c.
      asm volatile("" ::: "memory");
      const u4 *st = reinterpret_cast<const u4 *>(R);
      u4 *mine = reinterpret_cast<u4 *>(R) + (g * 16 + c) * kStoreChunks;
      const int cbase = c * kStoreChunks;
      const int f4 = g < 2 ? 4 + g : (g == 2 ? 12 : 0);   // the last step's chunk (g = 3: any, A is zero)
      float *rq = Rc + 16 * g, *rs = Rc + 8 * g, *rm = Rc - 8 * g;
      auto put_quad = [&](int r, int jb, int mt, float p0, float p1) {
        if (mt == 3 && g != 0) return;   // quads 13..15 hold nothing
        if (r == 1 && jb == 3) {
          rs[32 * mt] = p0;
          rm[200 - 32 * mt] = p1;
        } else {
          const int k = r == 0 ? jb + 1 : 7 - jb;
          rq[64 * mt + k] = p0;
          if (mt > 0 || g > 0) rq[64 * mt - k] = p1;
        }
      };
      // the lane's class values of round r in K order, as fp16 hi / lo
      // dwords, stored chunk by chunk (few of them live at a time)
      auto convert_store = [&](int r) {
        auto pair = [&](int n, uint32_t &H, uint32_t &L) {
          float x0, x1;
          if (r == 0) {
            x0 = D[n][0];
            x1 = D[n][1];
          } else {
            const int i0 = 2 * n, i1 = 2 * n + 1;
            const float s0 = i0 < 25 ? D[i0][2] : D[i0 - 25][3];
            const float s1 = i1 < 25 ? D[i1][2] : D[i1 - 25][3];
            x0 = g3 ? s0 : D[n][2];
            x1 = g3 ? s1 : D[n][3];
          }
          split_f32(x0, x1, kS2In, H, L);
        };
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          uint32_t H[4], L[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) pair(4 * j + k, H[k], L[k]);
          mine[j] = u4{H[0], H[1], H[2], H[3]};
          mine[6 + j] = u4{L[0], L[1], L[2], L[3]};
        }
        uint32_t H, L;
        pair(24, H, L);
        mine[12] = u4{H, L, H, 0u};
      };
      // The products of round r in two halves of the output rows (mt 0, 1
      // and 2, 3), operands one step ahead; `done` takes each (job, mt)
      // result.
      auto products = [&](int r, auto done) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          v4f acc[4][2];
#pragma unroll
          for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int i = 0; i < 2; ++i) acc[jb][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          v8h Bv[1][4], Av[1][2];
          auto load_step = [&](int t, v8h (&B)[4], v8h (&A)[2]) {
            // B chunk of lane group g at step t (the plan's pairing): hi
            // 0..5, lo 6..11, the inputs-48/49 tail 12
            const int f = t < 3 ? 4 * t + g : (t == 3 ? g : f4);
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) B[jb] = __builtin_bit_cast(v8h, st[jb * 16 * kStoreChunks + cbase + f]);
#pragma unroll
            for (int i = 0; i < 2; ++i) A[i] = __builtin_bit_cast(v8h, s_a2[((2 * hf + i) * 5 + t) * 64 + lane]);
          };
#pragma unroll
          for (int t = 0; t < 5; ++t) {
            load_step(t, Bv[0], Av[0]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int jb = 0; jb < 4; ++jb)
                acc[jb][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av[0][i], Bv[0][jb], acc[jb][i], 0, 0, 0);
            asm volatile("" ::: "memory");   // at most two steps' operands in registers
          }
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) done(jb, 2 * hf + i, i, acc[jb][i]);
        }
      };
      // 4'. |X|^2 of the lane's quads (4 |X|^2 as in the register form: the
      //     class rows carry a factor 2, the split gives 2 S).  Job 3 of
      //     round 1 is the 50-point real split: with u = Z[q], v = Z[25 - q],
      //     A = u + v*, B = u - v* and W = W50^q, 2 S[q] = A - i W B (bin 8 q)
      //     and conj(2 S[25 - q]) = A + i W B (bin 200 - 8 q).
      auto power2 = [&](bool split, int mt, const v4f &z, float &p0, float &p1) {
        if (split) {
          const float2 W = s_w50[4 * mt + g];
          const float Ax = z[0] + z[2], Ay = z[1] - z[3], Bx = z[0] - z[2], By = z[1] + z[3];
          const float p = __builtin_fmaf(W.x, Bx, -W.y * By), q = __builtin_fmaf(W.x, By, W.y * Bx);
          const float X1x = Ax + q, X1y = Ay - p, X2x = Ax - q, X2y = Ay + p;
          p0 = __builtin_fmaf(X1x, X1x, X1y * X1y);
          p1 = __builtin_fmaf(X2x, X2x, X2y * X2y);
        } else {
          p0 = __builtin_fmaf(z[0], z[0], z[1] * z[1]);
          p1 = __builtin_fmaf(z[2], z[2], z[3] * z[3]);
        }
      };
      convert_store(0);
      asm volatile("" ::: "memory");
      // round 0's power values wait in registers until round 1's operand
      // reads are done, since the power rows overwrite the operand chunks
      float pw0[4][4][2];
      products(0, [&](int jb, int mt, int, const v4f &z) { power2(false, mt, z, pw0[jb][mt][0], pw0[jb][mt][1]); });
      asm volatile("" ::: "memory");
      convert_store(1);
      asm volatile("" ::: "memory");
      float pw1[4][2][2];   // round 1's first half, written after the second half's reads
      products(1, [&](int jb, int mt, int i, const v4f &z) {
        float p0, p1;
        power2(jb == 3, mt, z, p0, p1);
        if (mt < 2) {
          pw1[jb][i][0] = p0;
          pw1[jb][i][1] = p1;
        } else {
          put_quad(1, jb, mt, p0, p1);
          put_quad(1, jb, i, pw1[jb][i][0], pw1[jb][i][1]);
          put_quad(0, jb, mt, pw0[jb][mt][0], pw0[jb][mt][1]);
          put_quad(0, jb, i, pw0[jb][i][0], pw0[jb][i][1]);
        }
      });
      asm volatile("" ::: "memory");
    } else {
      __builtin_amdgcn_s_setprio(kPrioDft);
      // 3. 25-point DFTs over n1.  Za: class g + 1 (rows 4g, 4g+1).  Zb: class
      //    7 - g (rows 4g+2, 4g+3) for g < 3; for g = 3, z[m] = s[2m] + i s[2m+1]
      //    with s[n1 + 25 e] the sum over n2 of parity e (rows 14, 15).
      float2 Za[25], Zb[25];
#pragma unroll
      for (int n1 = 0; n1 < 25; ++n1) Za[n1] = make_float2(D[n1][0], D[n1][1]);
#pragma unroll
      for (int m = 0; m < 25; ++m) {
        const int e = 2 * m, o = 2 * m + 1;
        const float se = e < 25 ? D[e][2] : D[e - 25][3];
        const float so = o < 25 ? D[o][2] : D[o - 25][3];
        Zb[m] = make_float2(g3 ? se : D[m][2], g3 ? so : D[m][3]);
      }
      dft25(Za);
      dft25(Zb);

      // 4. power rows (every value is 4 |X[k]|^2: the class rows are scaled by
      //    2 in the matrix).  Za output k1 is bin 16 k1 + (g+1), or its mirror
      //    400 - that for k1 > 12.  Zb outputs of groups 0..2 are bins 16 k1 +
      //    7 - g and mirrors alike; they are taken in pairs (j, 25 - j), bins
      //    16 j + 7 - g and 16 j - 7 + g, so that group 3 can share the loop:
      //    there, with u = Zb[j], v = Zb[25 - j], A = u + v*, B = u - v* and W =
      //    W50^j, the 50-point real DFT gives 2 S[j] = A - i W B (bin 8 j) and
      //    conj(2 S[25 - j]) = A + i W B (bin 200 - 8 j).  The complex values
      //    are formed before squaring, so a weak bin is not the difference of
      //    two large squares.
      {
        float *pa = Rc + (g + 1), *pb = Rc + (15 - g);
#pragma unroll
        for (int k1 = 0; k1 < 25; ++k1) {
          const float p = __builtin_fmaf(Za[k1].x, Za[k1].x, Za[k1].y * Za[k1].y);
          if (k1 <= 12) pa[16 * k1] = p;
          else pb[16 * (24 - k1)] = p;
        }
        const int kb = 7 - g;
        float *q1 = Rc + (g3 ? 0 : kb), *q2 = Rc + (g3 ? 200 : -kb);
        const int st1 = g3 ? 8 : 16, st2 = g3 ? -8 : 16;
#pragma unroll
        for (int j = 0; j < 13; ++j) {
          const float2 u = Zb[j], v = Zb[(25 - j) % 25];
          const float2 A = make_float2(u.x + v.x, u.y - v.y), B = make_float2(u.x - v.x, u.y + v.y);
          const float wx = kW400.c[8 * j], wy = kW400.s[8 * j];
          const float p = __builtin_fmaf(wx, B.x, -wy * B.y), q = __builtin_fmaf(wx, B.y, wy * B.x);   // W B
          const float2 X1 = g3 ? make_float2(A.x + q, A.y - p) : u;
          const float2 X2 = g3 ? make_float2(A.x - q, A.y + p) : v;
          q1[st1 * j] = __builtin_fmaf(X1.x, X1.x, X1.y * X1.y);
          const float p2 = __builtin_fmaf(X2.x, X2.x, X2.y * X2.y);
          if (j == 0) Rc[g3 ? 200 : kb] = p2;
          else q2[st2 * j] = p2;
        }
      }
    }
    // zero the pad columns 201..211 of the lane's row, which the last chunks read
    static_assert(kRow == 213, "pad columns below assume 12 of them");
    Rc[201 + g] = 0.0f;
    Rc[205 + g] = 0.0f;
    Rc[209 + g] = 0.0f;
    if (a.power != 2.0f) {
      // |X|^p = (|X|^2)^(p/2) in place over the wave's rows (float input:
      // the sub-tile's 2^-2e first)
      const float pe = 0.5f * a.power;
      for (int i = lane; i < kRegion; i += 64) R[i] = powf(__builtin_amdgcn_ldexpf(R[i] * a.pre_scale, -2 * esc), pe);
    }
    // float input at power 2: the mel sums carry 2^2e (exact power of two)
    const int mel_e = (kI16 || a.power != 2.0f) ? 0 : -2 * esc;

    {
      // the next sub-tile's samples have arrived by now (their loads went
      // out before this sub-tile's first stage): retiring the registers
      // here, before this sub-tile's stores, spares the next staging a wait
      // for them
#pragma unroll
      for (int i = 0; i < Prefetch<IN>::N; ++i) asm volatile("" ::"v"(pf.v[i]));
    }
    // 5. mel sums on 4x4x1 matrix blocks (16 per instruction): block (quad
    //    g, frame quad c / 4) of step s multiplies the power of 4 frames at
    //    bin qs_g + s by the weights of the 4 bands of quad 4 jb + g there,
    //    so a step advances every quad of the 16-band block jb by one bin.
    //    A = P[frame c][qs_g + s], B = weight of band 16 jb + 4 g + c % 4:
    //    lane (c, g) gets that band for the frames 4 (c / 4) + i, i < 4,
    //    which are consecutive in the output.  The steps of all blocks run
    //    as one sequence of batches of kMelBatch steps (every block has at
    //    least one); a batch's operands are loaded three batches ahead,
    //    each step reading first the table entry that the load two steps
    //    later needs (LDS reads complete in order, so a wait for an entry
    //    never waits for the operand loads issued after it).
    asm volatile("" ::: "memory");   // keep the table reads below out of the transform's register peak
    if constexpr (!S2) __builtin_amdgcn_s_setprio(kPrioChain);
    const int64_t f0 = t.s * kSub + 4 * (c >> 2);
    const bool sub_full = t.s * kSub + kSub <= F;   // uniform: every frame of the sub-tile exists
    OUT *orow = out + t.b * (int64_t)NM * F + (int64_t)(4 * g + (c & 3)) * F + f0;   // block 0's band
    // mel values are >= 1e-10 > 0, so their float order is the order of
    // their bit patterns: the maximum and the minimum are kept as unsigned
    uint32_t vmaxb = 0u;
    const int NBT = a.mel_batches;
    const float *wl = s_melw + 16 * g + 4 * (c & 3);
    float wR[4][kMelBatch], pR[4][kMelBatch];
    int eR[4];
    bool endR[4];
    auto entry = [&](int bt) { return s_bat[4 * min(bt, NBT - 1) + g]; };
    const uint64_t endm0 = a.end_mask[0], endm1 = a.end_mask[1];
    auto load = [&](auto slot, int bt) {
      constexpr int S = decltype(slot)::value;
      const v4f w4 = *reinterpret_cast<const v4f *>(wl + 16 * kMelBatch * min(bt, NBT - 1));
      const float *pq = Rc + eR[S];
#pragma unroll
      for (int u = 0; u < kMelBatch; ++u) {
        wR[S][u] = w4[u];
        pR[S][u] = pq[u];
      }
      endR[S] = ((bt < 64 ? endm0 : endm1) >> (bt & 63)) & 1;   // uniform: scalar instructions only
    };
    int cb = 0;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    int res_pass = 0;           // single pass: 1 stores and finds the maximum, 2 floors and stores again
    float res_fl = 0.0f;        // single pass: the clip's floor in output units
    bool res_ok = true;         // single pass: the grid barrier completed
    float res_min = __builtin_huge_valf();   // single pass: the lane's smallest output
    OUT *const orow0 = orow;
    (void)orow0;
    auto compute = [&](auto slot) {
      constexpr int S = decltype(slot)::value;
#pragma unroll
      for (int u = 0; u < kMelBatch; ++u) acc = __builtin_amdgcn_mfma_f32_4x4x1f32(pR[S][u], wR[S][u], acc, 0, 0, 0);
      if (!endR[S]) return;
      if (!kI16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_ldexpf(acc[i], mel_e);
      }
      // block cb complete: log10, rescale, store, statistics
      if constexpr (RES) {
        const bool band_ok = 16 * cb + 4 * g + (c & 3) < NM;
        float o[4];
        if (res_pass == 1) {   // uniform: store, and keep the maximum and the lane's minimum
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = floor_1e10(acc[i]);
            o[i] = logmel_of(v);
            if (band_ok && f0 + i < F) {
              vmaxb = max(vmaxb, __float_as_uint(v));
              res_min = fminf(res_min, o[i]);
            }
          }
        } else {               // the floor is known: floor, store again
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = res_ok ? fmaxf(logmel_of(floor_1e10(acc[i])), res_fl) : res_fl;
        }
        {
          if (sub_full && 16 * cb + 16 <= NM) {
            store_out4(orow, o);
          } else if (band_ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (f0 + i < F) store_out(orow + i, o[i]);
          }
        }
        acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        ++cb;
        orow += 16 * F;
        return;
      }
      uint32_t vminb = 0x7f800000u;   // +inf: no value
      if (a.mel_out) {   // uniform: mel values as they are, no statistics
        const bool band_ok = 16 * cb + 4 * g + (c & 3) < NM;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (band_ok && f0 + i < F) store_out(orow + i, acc[i]);
      } else if (sub_full && 16 * cb + 16 <= NM) {   // uniform: every lane's band and frames exist
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = floor_1e10(acc[i]);
          vmaxb = max(vmaxb, __float_as_uint(v));
          vminb = min(vminb, __float_as_uint(v));
          o[i] = logmel_of(v);
        }
        store_out4(orow, o);
      } else {
        const bool band_ok = 16 * cb + 4 * g + (c & 3) < NM;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = floor_1e10(acc[i]);
          if (band_ok && f0 + i < F) {
            vmaxb = max(vmaxb, __float_as_uint(v));
            vminb = min(vminb, __float_as_uint(v));
            store_out(orow + i, logmel_of(v));
          }
        }
      }
      // the region's smallest mel value (its smallest output is that value's)
      vminb = row_min16(vminb);
      if (c == 0) tile_min[(gs * NB + cb) * 4 + g] = __uint_as_float(vminb);
      acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      ++cb;
      orow += 16 * F;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // the mel stage's batch pipeline: operands three batches ahead (see above)
#define LM_MEL_STEP(S, S1, S3)                \
  {                                           \
    eR[S1::value] = entry(i + 5);             \
    load(S3{}, i + 3);                        \
    compute(S{});                             \
    if (++i >= NBT) break;                    \
  }
#define LM_MEL_STAGE()                                                          \
  {                                                                             \
    eR[0] = entry(0);                                                           \
    eR[1] = entry(1);                                                           \
    eR[2] = entry(2);                                                           \
    eR[3] = entry(3);                                                           \
    /* loads past the last batch repeat it (every wait count stays static) */  \
    load(I0{}, 0);                                                              \
    load(I1{}, 1);                                                              \
    load(I2{}, 2);                                                              \
    eR[0] = entry(4);                                                           \
    /* step of batch i in slot S: the entry of batch i + 5 (slot S + 1), the */ \
    /* operands of batch i + 3 (slot S + 3), then the products of batch i    */ \
    for (int i = 0; i < NBT;) {                                                 \
      LM_MEL_STEP(I0, I1, I3)                                                   \
      LM_MEL_STEP(I1, I2, I0)                                                   \
      LM_MEL_STEP(I2, I3, I1)                                                   \
      LM_MEL_STEP(I3, I0, I2)                                                   \
    }                                                                           \
  }
    if constexpr (RES) {
      res_pass = 1;
      LM_MEL_STAGE()
      res_fl = res_sync(vmaxb, t.b);
      res_ok = s_ok != 0;
      res_done = true;
      // only a wave holding a value below its clip's floor runs the mel sums
      // again from its power rows (still in its LDS region) and overwrites
      // them floored; a barrier that ran out of polls makes every wave
      // overwrite its values with NaN
      if (!res_ok || __any(res_min < res_fl)) {
        res_pass = 2;
        cb = 0;
        acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        orow = orow0;
        LM_MEL_STAGE()
      }
    } else {
      LM_MEL_STAGE()
      vmaxb = row_max16(vmaxb);
      if (c == 0) a.tile_max[4 * gs + g] = __uint_as_float(vmaxb);
    }
#undef LM_MEL_STAGE
#undef LM_MEL_STEP
  }
  // a wave without a sub-tile still takes part in the workgroup's barriers
  if constexpr (RES) {
    if (!res_done) (void)res_sync(0u, -1);
  }
}

}  // namespace

// The n_fft = 400 path needs an even hop (runs of samples keep a parity
// known at compile time), a 16-frame span that fits the wave's region and a
// blocked filter table that fits its LDS share.
bool pcm400_supported(const lm_plan *p, bool in_i16) {
  (void)in_i16;   // both input types stage the same two fp16 planes
  if (p->n_fft != 400 || (p->hop & 1) || p->mfma400h.empty() || p->n_mels > 256) return false;
  if (p->melblk_w.size() > (size_t)kMelWLds) return false;
  const int span = (kSub - 1) * p->hop + 400;
  const int ndw = span / 2;
  const int lds_dw = p->hop == 160 ? ndw + 4 * (ndw / 80) : ndw;   // skewed layout at hop 160
  return lds_dw <= kLoff && kLoff + lds_dw <= kRegion;
}

// The 25-point stage runs on the matrix cores when that form is asked for,
// the blocked weights fit next to its operand table and the window keeps
// every first-stage value in fp16 range.
bool pcm400_matrix25(const lm_plan *p) {
  return p->fft_variant == LM_FFT_SPLIT_MFMA && p->mfma400t_fits && !p->mfma400t.empty() &&
         p->melblk_w.size() <= (size_t)kMelWLds2 && p->melblk_meta.size() / 4 <= (size_t)(kMelWLds2 / (16 * kMelBatch));
}

std::string pcm400_summary(const lm_plan *p) {
  char buf[400];
  const bool m25 = pcm400_matrix25(p);
  std::snprintf(buf, sizeof buf,
                "pcm400_kernel: first stage on v_mfma_f32_16x16x32_f16 (two-part fp16 operands, fp32 "
                "accumulate), 25-point DFTs %s, %d-frame sub-tiles per wave, %d waves per "
                "workgroup, one workgroup per compute unit; mel on 4x4x1 fp32 matrix blocks: %zu batches "
                "of %d steps, %zu of %d blocked weights",
                m25 ? "on v_mfma_f32_16x16x32_f16 (two-part fp16 operands, three products)" : "in registers",
                kSub, kWaves, p->melblk_meta.size() / 4, kMelBatch, p->melblk_w.size(), m25 ? kMelWLds2 : kMelWLds);
  return buf;
}

StatLayout pcm400_stat_layout(const lm_plan *p) {
  StatLayout st;
  st.frames_per_tile = kSub;
  st.sub_per_tile = 1;
  st.blk_per_sub = 4 * ((p->n_mels + 15) / 16);
  st.band_h = 4;
  st.max_per_tile = 4;   // one per quad group of lanes
  return st;
}

bool pcm400_single_pass(const lm_plan *p, bool in_i16, int64_t n_sub) {
  return p->single_pass && p->coop_launch && p->output == LM_OUTPUT_LOGMEL &&
         (p->fft_variant == LM_FFT_AUTO || p->fft_variant == LM_FFT_SPLIT_MFMA) &&
         pcm400_supported(p, in_i16) &&
         p->n_cu > 0 && n_sub <= (int64_t)p->n_cu * kWaves;
}

hipError_t launch_pcm400(const lm_plan *p, const PcmArgs &pa, hipStream_t s, const LaunchTiming *tm) {
  Args k;
  k.pcm = pa.pcm;
  k.T = pa.n_samples;
  k.F = pa.n_frames;
  k.S = pa.tiles_per_clip;
  k.n_sub = pa.n_clips * pa.tiles_per_clip;
  // every CU takes a share, even when there are fewer sub-tiles than waves
  // (fewer waves per SIMD then finish each sub-tile sooner)
  const int64_t n_wg = k.n_sub < p->n_cu ? k.n_sub : p->n_cu;
  k.per_wg = (int)((k.n_sub + n_wg - 1) / n_wg);
  k.hop = p->hop;
  k.pad = (p->center ? 200 : 0) + (int)p->sig_pad;
  k.sig_pad = (int)p->sig_pad;
  k.pad_mode = p->pad_mode;
  k.power = p->power;
  // every power value is 4 |X|^2 times the fp16 matrix's 2^12 on the
  // planes' sum squared: int16 planes hold x / 64 with x carrying 2^15, so
  // 2^12 2^15 / 64 = 2^21 per |X|; float planes hold x 2^e, so 2^12 2^e,
  // whose 2^e the kernel takes back per sub-tile (the normalisation's factor
  // on |X|^2 joins them)
  // The matrix-core 25-point stage takes the values times 2^-10 and its
  // matrix carries 2^8: 2^-2 per |X|, 2^-4 on every power value.
  const bool m25 = !pa.sync && pcm400_matrix25(p);
  const double in_scale2 = (pa.in_i16 ? 1.0 / 4398046511104.0 : 1.0 / 16777216.0) * power_scale2(p) *
                           (m25 ? 16.0 : 1.0);   // 2^-42, 2^-24 (times 2^4)
  if (p->power == 2.0f) {
    k.mel_scale = (float)(0.25 * in_scale2);
    k.pre_scale = 1.0f;
  } else {
    k.mel_scale = 1.0f;
    k.pre_scale = (float)(0.25 * in_scale2);
  }
  k.mel_out = p->output == LM_OUTPUT_MEL;
  k.n_mels = p->n_mels;
  k.n_melblk = p->dt.n_melblk;
  k.melw_n = (int)p->melblk_w.size();
  k.mel_batches = (int)(p->melblk_meta.size() / 4);
  static_assert(kMelBatMax <= 128, "end flags fit two 64-bit masks");
  k.end_mask[0] = k.end_mask[1] = 0;
  for (int bt = 0; bt < k.mel_batches; ++bt)
    if (p->melblk_meta[4 * (size_t)bt] >> 16) k.end_mask[bt >> 6] |= (uint64_t)1 << (bt & 63);
  k.tile_max = pa.tile_max;
  k.epoch = pa.epoch;
  k.parity = pa.parity;
  k.sync = pa.sync;
  k.a2 = reinterpret_cast<const v4f *>(p->dt.mfma400t);
  const dim3 grid((unsigned)n_wg), block(kThreads);
  const bool f16 = p->out_dtype == LM_F16;
  const v4f *am = reinterpret_cast<const v4f *>(p->dt.mfma400h);
  const int32_t *bm = p->dt.melblk_meta;
  const float *bw = p->dt.melblk_w;
  float *tmin = pa.tile_min;
  const bool sk = p->hop == 160;
#define LM_P400(IN, OUT, SK)                                                                       \
  do {                                                                                             \
    if (pa.sync) {                                                                                 \
      OUT *op = (OUT *)pa.out;                                                                     \
      void *args[] = {&k, (void *)&am, (void *)&bm, (void *)&bw, (void *)&op, (void *)&tmin};    \
      if (tm) (void)hipEventRecord(tm->beg, s);                                                    \
      const hipError_t e = hipLaunchCooperativeKernel(                                             \
          reinterpret_cast<const void *>(&pcm400_kernel<IN, OUT, SK, true, false>), grid, block, args, 0, s); \
      if (e != hipSuccess) return e;                                                               \
      if (tm) (void)hipEventRecord(tm->end, s);                                                    \
    } else if (m25) {                                                                              \
      LM_LAUNCH(tm, (pcm400_kernel<IN, OUT, SK, false, true>), grid, block, 0, s, k, am, bm, bw, (OUT *)pa.out, tmin); \
    } else {                                                                                       \
      LM_LAUNCH(tm, (pcm400_kernel<IN, OUT, SK, false, false>), grid, block, 0, s, k, am, bm, bw, (OUT *)pa.out, tmin); \
    }                                                                                              \
  } while (0)
  if (!pa.in_i16 && !f16) {
    if (sk) LM_P400(float, float, true);
    else LM_P400(float, float, false);
  } else if (!pa.in_i16 && f16) {
    if (sk) LM_P400(float, __half, true);
    else LM_P400(float, __half, false);
  } else if (pa.in_i16 && !f16) {
    if (sk) LM_P400(int16_t, float, true);
    else LM_P400(int16_t, float, false);
  } else {
    if (sk) LM_P400(int16_t, __half, true);
    else LM_P400(int16_t, __half, false);
  }
#undef LM_P400
  return hipGetLastError();
}

}  // namespace lm
