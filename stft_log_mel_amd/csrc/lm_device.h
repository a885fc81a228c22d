// Device helpers shared by the kernels: complex arithmetic, small DFT
// modules, the log10 used by every kernel, padding by index arithmetic,
// wave/block reductions.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "lm.h"

namespace lm {

// ---------------------------------------------------------------------------
// log10 and the output map
// ---------------------------------------------------------------------------

// log10(2) / 4
constexpr float kLog10_2_Q = 0.0752574989159952988f;

// max(v, 1e-10f) on the bit patterns, one integer max: the signed-integer
// order of float bits agrees with the float order whenever one operand is
// positive (a negative v, or -0, compares below).  Unlike fmaxf it needs no
// canonicalising of v, and it keeps a NaN (out of contract anyway).
constexpr int kBits1e10 = 0x2edbe6ff;   // 1e-10f
__device__ __forceinline__ float floor_1e10(float v) { return __int_as_float(max(__float_as_int(v), kBits1e10)); }

// The output value of a mel value v >= 1e-10 (after the floor):
// (log10 v + 4) / 4, as one fma on the hardware base-2 logarithm.  Every
// kernel writes exactly this value for every element, the region minima
// the kernels record are minima of the values v, and the clamp fix-up
// takes the clip's largest output as logmel_of(largest mel value) -- the
// same function of the same value -- and its floor as that minus 2, i.e.
// ((hi - 8) + 4) / 4.
__device__ __forceinline__ float logmel_of(float v) {
  return __builtin_fmaf(__builtin_amdgcn_logf(v), kLog10_2_Q, 1.0f);
}

// fp16 output is the fp32 value rounded to nearest even.  The empty asm
// keeps the compiler from fusing the conversion into the fma that produced
// v (a mixed-precision fma rounds the exact result once, which differs from
// rounding the fp32 value where that value is a tie in fp16).
__device__ __forceinline__ float fp32_value(float v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(__half *p, float v) { *p = __float2half_rn(fp32_value(v)); }
// Streaming stores for the main kernels: every output is written once and
// read again only by the fix-up's few flagged regions.
__device__ __forceinline__ void store_out_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_out_nt(__half *p, float v) {
  __builtin_nontemporal_store(__half_as_ushort(__float2half_rn(fp32_value(v))), reinterpret_cast<unsigned short *>(p));
}
__device__ __forceinline__ float load_out(const float *p) { return *p; }
__device__ __forceinline__ float load_out(const __half *p) { return __half2float(*p); }

// ---------------------------------------------------------------------------
// Complex arithmetic on float2 (x = re, y = im)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(__builtin_fmaf(a.x, b.x, -a.y * b.y), __builtin_fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
// a * (-i)
__device__ __forceinline__ float2 mul_mi(float2 a) { return make_float2(a.y, -a.x); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }

// ---------------------------------------------------------------------------
// Small forward DFT modules, in place: b[s] = sum_t a[t] exp(-2 pi i t s / R)
// ---------------------------------------------------------------------------

constexpr float kSqrtHalf = 0.70710678118654752440f;
constexpr float kCos1_16 = 0.92387953251128675613f;   // cos(pi/8)
constexpr float kSin1_16 = 0.38268343236508977173f;   // sin(pi/8)
// radix-5 (Winograd-style) constants: cos/sin of 2 pi/5 and 4 pi/5
constexpr float kC5_1 = 0.30901699437494742410f;
constexpr float kC5_2 = -0.80901699437494742410f;
constexpr float kS5_1 = 0.95105651629515357212f;
constexpr float kS5_2 = 0.58778525229247312917f;

__device__ __forceinline__ void dft2(float2 &a0, float2 &a1) {
  const float2 t = a0;
  a0 = cadd(t, a1);
  a1 = csub(t, a1);
}

__device__ __forceinline__ void dft4(float2 &a0, float2 &a1, float2 &a2, float2 &a3) {
  const float2 t0 = cadd(a0, a2), t1 = csub(a0, a2);
  const float2 t2 = cadd(a1, a3), t3 = mul_mi(csub(a1, a3));
  a0 = cadd(t0, t2);
  a2 = csub(t0, t2);
  a1 = cadd(t1, t3);
  a3 = csub(t1, t3);
}

// multiply by exp(-2 pi i/8) and exp(-6 pi i/8)
__device__ __forceinline__ float2 mul_w8_1(float2 a) {
  return make_float2((a.x + a.y) * kSqrtHalf, (a.y - a.x) * kSqrtHalf);
}
__device__ __forceinline__ float2 mul_w8_3(float2 a) {
  return make_float2((a.y - a.x) * kSqrtHalf, -(a.x + a.y) * kSqrtHalf);
}

__device__ __forceinline__ void dft8(float2 (&a)[8]) {
  // even / odd halves as 4-point transforms, then one radix-2 combine
  float2 e0 = a[0], e1 = a[2], e2 = a[4], e3 = a[6];
  float2 o0 = a[1], o1 = a[3], o2 = a[5], o3 = a[7];
  dft4(e0, e1, e2, e3);
  dft4(o0, o1, o2, o3);
  o1 = mul_w8_1(o1);
  o2 = mul_mi(o2);
  o3 = mul_w8_3(o3);
  a[0] = cadd(e0, o0);
  a[4] = csub(e0, o0);
  a[1] = cadd(e1, o1);
  a[5] = csub(e1, o1);
  a[2] = cadd(e2, o2);
  a[6] = csub(e2, o2);
  a[3] = cadd(e3, o3);
  a[7] = csub(e3, o3);
}

__device__ __forceinline__ void dft16(float2 (&a)[16]) {
  // 4 x 4: column transforms over t1 (stride 4), twiddle exp(-2 pi i t2 s1/16),
  // then row transforms over t2.
  float2 g[4][4];
#pragma unroll
  for (int t2 = 0; t2 < 4; ++t2) {
    g[t2][0] = a[t2];
    g[t2][1] = a[t2 + 4];
    g[t2][2] = a[t2 + 8];
    g[t2][3] = a[t2 + 12];
    dft4(g[t2][0], g[t2][1], g[t2][2], g[t2][3]);
  }
  // twiddles: W16^(t2*s1) for t2, s1 in 1..3
  const float2 w1 = make_float2(kCos1_16, -kSin1_16);   // W16^1
  const float2 w3 = make_float2(kSin1_16, -kCos1_16);   // W16^3
  const float2 w9 = make_float2(-kCos1_16, kSin1_16);   // W16^9 = -W16^1
  g[1][1] = cmul(g[1][1], w1);
  g[1][2] = mul_w8_1(g[1][2]);   // W16^2
  g[1][3] = cmul(g[1][3], w3);
  g[2][1] = mul_w8_1(g[2][1]);   // W16^2
  g[2][2] = mul_mi(g[2][2]);     // W16^4
  g[2][3] = mul_w8_3(g[2][3]);   // W16^6
  g[3][1] = cmul(g[3][1], w3);
  g[3][2] = mul_w8_3(g[3][2]);   // W16^6
  g[3][3] = cmul(g[3][3], w9);
#pragma unroll
  for (int s1 = 0; s1 < 4; ++s1) {
    float2 h0 = g[0][s1], h1 = g[1][s1], h2 = g[2][s1], h3 = g[3][s1];
    dft4(h0, h1, h2, h3);
    a[s1] = h0;
    a[s1 + 4] = h1;
    a[s1 + 8] = h2;
    a[s1 + 12] = h3;
  }
}

__device__ __forceinline__ void dft5(float2 (&a)[5]) {
  const float2 t1 = cadd(a[1], a[4]), t2 = cadd(a[2], a[3]);
  const float2 t3 = csub(a[1], a[4]), t4 = csub(a[2], a[3]);
  const float2 a0 = a[0];
  const float2 r1 = make_float2(__builtin_fmaf(kC5_2, t2.x, __builtin_fmaf(kC5_1, t1.x, a0.x)),
                                __builtin_fmaf(kC5_2, t2.y, __builtin_fmaf(kC5_1, t1.y, a0.y)));
  const float2 r2 = make_float2(__builtin_fmaf(kC5_1, t2.x, __builtin_fmaf(kC5_2, t1.x, a0.x)),
                                __builtin_fmaf(kC5_1, t2.y, __builtin_fmaf(kC5_2, t1.y, a0.y)));
  const float2 i1 = make_float2(__builtin_fmaf(kS5_2, t4.x, kS5_1 * t3.x),
                                __builtin_fmaf(kS5_2, t4.y, kS5_1 * t3.y));
  const float2 i2 = make_float2(__builtin_fmaf(-kS5_1, t4.x, kS5_2 * t3.x),
                                __builtin_fmaf(-kS5_1, t4.y, kS5_2 * t3.y));
  a[0] = make_float2(a0.x + t1.x + t2.x, a0.y + t1.y + t2.y);
  // b = r -/+ i * q:  -i q = (q.y, -q.x),  +i q = (-q.y, q.x)
  a[1] = make_float2(r1.x + i1.y, r1.y - i1.x);
  a[4] = make_float2(r1.x - i1.y, r1.y + i1.x);
  a[2] = make_float2(r2.x + i2.y, r2.y - i2.x);
  a[3] = make_float2(r2.x - i2.y, r2.y + i2.x);
}

template <int R>
__device__ __forceinline__ void dft(float2 (&a)[R]);
template <>
__device__ __forceinline__ void dft<2>(float2 (&a)[2]) { dft2(a[0], a[1]); }
template <>
__device__ __forceinline__ void dft<4>(float2 (&a)[4]) { dft4(a[0], a[1], a[2], a[3]); }
template <>
__device__ __forceinline__ void dft<5>(float2 (&a)[5]) { dft5(a); }
template <>
__device__ __forceinline__ void dft<8>(float2 (&a)[8]) { dft8(a); }
template <>
__device__ __forceinline__ void dft<16>(float2 (&a)[16]) { dft16(a); }

// ---------------------------------------------------------------------------
// Padding by index arithmetic (flashmel page, "How it works")
// ---------------------------------------------------------------------------

// Source index, in a clip of T samples, of position j of the signal that is
// read as P zeros, the clip, P zeros (torchaudio's pad; j counts from the
// clip's first sample, so those zeros are at -P..-1 and T..T+P-1), with the
// center padding of `mode` applied beyond that signal; -1 for a zero.  The
// center padding is at most n_fft/2 < T + 2P samples (reflect) or <= T + 2P
// (circular), which the entry points check, so one reflection or wrap
// suffices.
__device__ __forceinline__ int64_t signal_source(int64_t j, int64_t T, int64_t P, int mode) {
  if (j >= 0 && j < T) return j;
  const int64_t Tp = T + 2 * P;
  int64_t q = j + P;   // position in the zero-padded signal
  if (q < 0 || q >= Tp) {
    if (mode == LM_PAD_CONSTANT) return -1;
    if (mode == LM_PAD_REFLECT) q = q < 0 ? -q : 2 * (Tp - 1) - q;
    else if (mode == LM_PAD_REPLICATE) q = q < 0 ? 0 : Tp - 1;
    else q = q < 0 ? q + Tp : q - Tp;
  }
  q -= P;
  return (q >= 0 && q < T) ? q : -1;
}

// ---------------------------------------------------------------------------
// Reductions (wave64)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

// unsigned min over the 16 lanes of a DPP row (rotations by 1, 2, 4, 8);
// on the bit patterns of positive floats it is the float min
template <int N>
__device__ __forceinline__ uint32_t ror_min(uint32_t v) {
  const uint32_t r = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xf, 0xf, false);
  return min(v, r);
}
__device__ __forceinline__ uint32_t row_min16(uint32_t v) {
  v = ror_min<1>(v);
  v = ror_min<2>(v);
  v = ror_min<4>(v);
  return ror_min<8>(v);
}
// unsigned max over the 16 lanes of a DPP row; on the bit patterns of
// positive floats it is the float max
template <int N>
__device__ __forceinline__ uint32_t ror_max(uint32_t v) {
  const uint32_t r = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xf, 0xf, false);
  return max(v, r);
}
__device__ __forceinline__ uint32_t row_max16(uint32_t v) {
  v = ror_max<1>(v);
  v = ror_max<2>(v);
  v = ror_max<4>(v);
  return ror_max<8>(v);
}

// unsigned max / min over the whole wave: the DPP row reduction, then the
// four rows' results by readlane (uniform)
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = row_max16(v);
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = row_min16(v);
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Block-wide max of vmax and min of vmin, for non-negative values (mel
// values after the 1e-10 floor, +inf for none), reduced on their bit
// patterns; the result is valid in thread 0.  `red` must hold
// 2 * (blockDim.x / 64) floats of LDS.
template <int THREADS>
__device__ __forceinline__ void block_maxmin(float &vmax, float &vmin, float *red) {
  constexpr int NW = THREADS / 64;
  vmax = __uint_as_float(wave_umax(__float_as_uint(vmax)));
  vmin = __uint_as_float(wave_umin(__float_as_uint(vmin)));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    red[w] = vmax;
    red[NW + w] = vmin;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      vmax = fmaxf(vmax, red[i]);
      vmin = fminf(vmin, red[NW + i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Packed filterbank staging
// ---------------------------------------------------------------------------

// Row m of a packed filterbank covers bins [start[m], start[m] + width[m])
// with weights w[off[m] + j]; rows are stored back to back, so the weight
// count is off[NM-1] + width[NM-1] and `w` holds w_len >= that many floats.
// All loads are independent (the first min(cap, w_len) weights are copied
// whatever the count); one barrier.  Weights are read from LDS when the
// returned count is <= cap, else from global memory.  NM <= 256.
template <int THREADS>
__device__ __forceinline__ int stage_filters(int NM, const int32_t *__restrict__ start,
                                             const int32_t *__restrict__ width,
                                             const int32_t *__restrict__ off, const float *__restrict__ w,
                                             int w_len, int32_t *s_start, int32_t *s_width, int32_t *s_off,
                                             float *s_w, int cap) {
  const int tid = threadIdx.x;
  for (int m = tid; m < NM; m += THREADS) {
    s_start[m] = start[m];
    s_width[m] = width[m];
    s_off[m] = off[m];
  }
  const int n = min(cap, w_len);
  for (int i = tid; i < n; i += THREADS) s_w[i] = w[i];
  __syncthreads();
  return s_off[NM - 1] + s_width[NM - 1];
}

}  // namespace lm
