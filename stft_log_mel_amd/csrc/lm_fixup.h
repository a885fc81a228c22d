// Per-clip floor (KBench task page "audio-mel-spectrogram-fused", section
// "spec_md": the floor is per clip, at the clip's largest log value minus
// 8), applied after the main kernels have written (L + 4) / 4 everywhere.
//
// The main kernels write o = logmel_of(v) for every mel value v (after the
// 1e-10 floor) and record the largest v per tile and the smallest v per
// region of a tile (a frame range times a band range).  The clip's largest
// output is logmel_of(hi_v) for its largest mel value hi_v -- the same
// function of the same value, so that element's output equals it exactly --
// and its floor in output units is that minus 2, i.e. ((hi - 8) + 4) / 4.
// Since the cast to the output type is monotone, max(cast(o), cast(floor))
// equals cast(max(o, floor)); so only regions that may hold an o below the
// floor are read, and only values below it are rewritten.  A region with
// smallest mel value m holds no o below logmel_of(m) - kGateSlack: the
// hardware log2 is within a few ulp (an ulp is at most 2^-16 for results up
// to 128 in size), so outputs of ordered inputs are out of order by at most
// a few 1e-6 after the scale by log10(2) / 4; the slack is far above that.
//
// fixup_group is one unit of that work, run by a whole workgroup of the
// fix-up kernel (a second launch after the main kernel; its kernel boundary
// makes every workgroup's statistics and outputs visible to the fix-up).
#pragma once

#include "lm_device.h"
#include "lm_internal.h"

namespace lm {

constexpr int kFixEntries = 512;   // regions one group scans
constexpr float kGateSlack = 2.5e-4f;   // see above: regions within it of the floor are read
constexpr int kFixUnroll = 8;      // values per thread with loads in flight together

// Group units of a fix-up: (clip, group) pairs, entries_per_group regions
// each -- at most kFixEntries, and fewer when regions are large, so that a
// group never holds more than kFixValues values (a batch whose regions are
// all flagged then spreads its rewrite over many workgroups).
constexpr int kFixValues = 65536;
inline void prepare_fixup(FixupArgs &a) {
  const int n_ent = a.tiles_per_clip * a.st.min_per_tile();
  const int reg = (a.st.frames_per_tile / a.st.sub_per_tile) * a.st.band_h;
  // n / d == umulhi(n, ceil(2^32 / d)) for every n < 2^16 and 2 <= d <= 2^16
  // (d = 1 is taken apart where they are used): a group's flattened values
  // number at most kFixValues = 2^16
  const unsigned inner = (unsigned)(a.mel_major ? a.st.frames_per_tile / a.st.sub_per_tile : a.st.band_h);
  a.inner_magic = inner > 1 ? (unsigned)((0x100000000ull + inner - 1) / inner) : 0u;
  a.reg_magic = reg > 1 ? (unsigned)((0x100000000ull + (unsigned)reg - 1) / (unsigned)reg) : 0u;
  int per = kFixValues / (reg > 0 ? reg : 1);
  per = per < 1 ? 1 : (per > kFixEntries ? kFixEntries : per);
  a.entries_per_group = per;
  a.groups_per_clip = (n_ent + per - 1) / per;
  a.empty_units = a.n_empty > 0 ? (int)((a.n_frames + kFixValues - 1) / kFixValues) : 0;
}

// The clip's floor in output units: logmel_of(largest mel value) - 2;
// every thread of the workgroup must call it.
constexpr int kFixMaxUnroll = 8;   // maxima per thread with their loads in flight together
template <int THREADS>
__device__ float clip_floor(const FixupArgs &a, int64_t b, float *s_red) {
  const int n_max = a.tiles_per_clip * a.st.max_per_tile;
  const float *cmax = a.tile_max + b * (int64_t)n_max;
  float hi = 0.0f;
  for (int e0 = threadIdx.x; e0 < n_max; e0 += kFixMaxUnroll * THREADS) {
    float v[kFixMaxUnroll];
#pragma unroll
    for (int u = 0; u < kFixMaxUnroll; ++u) v[u] = e0 + u * THREADS < n_max ? cmax[e0 + u * THREADS] : 0.0f;
#pragma unroll
    for (int u = 0; u < kFixMaxUnroll; ++u) hi = fmaxf(hi, v[u]);
  }
  hi = __uint_as_float(wave_umax(__float_as_uint(hi)));   // maxima are >= 0
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = hi;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < THREADS / 64; ++i) hi = fmaxf(hi, s_red[i]);
  return logmel_of(fmaxf(hi, 1e-10f)) - 2.0f;
}

// Unit (clip b, empty band row e, segment r): the kFixValues frames from r
// kFixValues on of band empty_bands[e], which the main kernel left
// unwritten.  Their mel value is 1e-10 (no weight, so the sum is 0 before
// the floor), so the result is max(logmel_of(1e-10), floor), written
// without reading.  Mel-major output only.
// The segment is written with 16-byte stores between a scalar head (up to
// the first 16-byte boundary) and a scalar tail; every element of it gets
// the same value.
template <typename OUT, int THREADS>
__device__ void fixup_empty_row(const FixupArgs &a, int64_t b, int e, int r, float *s_red) {
  const float fl = clip_floor<THREADS>(a, b, s_red);
  const float v = fmaxf(logmel_of(1e-10f), fl);
  const int64_t F = a.n_frames;
  OUT *row = reinterpret_cast<OUT *>(a.out) + (b * a.n_mels + a.empty_bands[e]) * F;
  const int64_t f0 = (int64_t)r * kFixValues, f1 = min(F, f0 + kFixValues);
  OUT *const p = row + f0;
  const int n = (int)(f1 - f0);   // <= kFixValues
  constexpr int VE = 16 / (int)sizeof(OUT);   // elements per 16 bytes
  const int mis = (int)((reinterpret_cast<uintptr_t>(p) & 15) / sizeof(OUT));   // elements past a boundary
  const int head = min(n, (VE - mis) % VE);
  const int nv = (n - head) / VE;
  const int tid = threadIdx.x;
  if (tid < head) store_out(p + tid, v);
  // the value's bit pattern in the output type, four 32-bit words
  uint32_t w;
  if constexpr (sizeof(OUT) == 2) {
    const uint32_t hb = __half_as_ushort(__float2half_rn(fp32_value(v)));
    w = hb | (hb << 16);
  } else {
    w = __float_as_uint(v);
  }
  const uint4 q = make_uint4(w, w, w, w);
  uint4 *const pv = reinterpret_cast<uint4 *>(p + head);   // 16-byte aligned
  for (int i = tid; i < nv; i += THREADS) pv[i] = q;
  const int t0 = head + nv * VE;
  if (t0 + tid < n) store_out(p + t0 + tid, v);   // fewer than VE <= THREADS elements
}

// Unit (clip b, group gi): reduce the clip's maxima to its floor (every
// group of the clip does this itself, so no cross-workgroup atomics or
// resets are needed), list the regions of the group whose smallest mel
// value maps below the floor plus the slack (as their first frame and first band), then rewrite
// their values below the floor with all threads.  LDS: s_f0[kFixEntries],
// s_m0[kFixEntries], s_n[1], s_red[THREADS / 64].  Every thread of the
// workgroup must call it; it ends with a barrier.
template <typename OUT, int THREADS>
__device__ void fixup_group(const FixupArgs &a, int64_t b, int gi, int *s_f0, int *s_m0, int *s_n, float *s_red) {
  const int tid = threadIdx.x;
  const StatLayout st = a.st;
  const int ept = st.min_per_tile();
  const int n_ent = a.tiles_per_clip * ept;
  const float *cmin = a.tile_min + b * (int64_t)n_ent;
  const int sub_frames = st.frames_per_tile / st.sub_per_tile;
  if (tid == 0) *s_n = 0;
  // the group's region minima are loaded together with the maxima (one
  // round trip): kFixEntries / THREADS of them per thread
  constexpr int MPT = (kFixEntries + THREADS - 1) / THREADS;
  const int e0 = gi * a.entries_per_group, e1 = min(n_ent, e0 + a.entries_per_group);
  float mn[MPT];
#pragma unroll
  for (int u = 0; u < MPT; ++u) {
    const int e = e0 + tid + u * THREADS;
    mn[u] = e < e1 ? cmin[e] : __builtin_huge_valf();
  }
  const float fl = clip_floor<THREADS>(a, b, s_red);
#pragma unroll
  for (int u = 0; u < MPT; ++u)
    if (logmel_of(mn[u]) < fl + kGateSlack) {   // +inf (an empty region) never is
      const int e = e0 + tid + u * THREADS;
      const int t = e / ept, rem = e - t * ept;
      const int sub = rem / st.blk_per_sub, blk = rem - sub * st.blk_per_sub;
      const int k = atomicAdd(s_n, 1);   // LDS atomic: the order of the list is irrelevant
      s_f0[k] = t * st.frames_per_tile + sub * sub_frames;
      s_m0[k] = blk * st.band_h;
    }
  __syncthreads();
  const int n_flag = *s_n;

  float fo = fl;
  if (sizeof(OUT) == 2) fo = __half2float(__float2half_rn(fp32_value(fo)));
  // rewrite: value k of the flattened list is value el of region i; el
  // splits into a run index o and the position in the run (contiguous in
  // the output), both with precomputed multiplies (no division per value)
  OUT *out = reinterpret_cast<OUT *>(a.out);
  const int NM = a.n_mels;
  const int64_t F = a.n_frames;
  const int inner = a.mel_major ? sub_frames : st.band_h;   // values of one run
  const int reg = sub_frames * st.band_h;                    // values of a full region
  const int total = n_flag * reg;
  for (int k0 = tid; k0 < total; k0 += THREADS * kFixUnroll) {
    OUT *p[kFixUnroll];
    float v[kFixUnroll];
#pragma unroll
    for (int u = 0; u < kFixUnroll; ++u) {
      const int k = k0 + u * THREADS;
      p[u] = nullptr;
      if (k < total) {
        const int i = reg > 1 ? (int)__umulhi((unsigned)k, a.reg_magic) : k;   // k / reg
        const int el = k - i * reg;
        const int o = inner > 1 ? (int)__umulhi((unsigned)el, a.inner_magic) : el;   // el / inner
        const int in = el - o * inner;
        const int64_t f = (int64_t)s_f0[i] + (a.mel_major ? in : o);
        const int m = s_m0[i] + (a.mel_major ? o : in);
        if (f < F && m < NM) {
          p[u] = out + (a.mel_major ? (b * NM + m) * F + f : (b * F + f) * NM + m);
          v[u] = load_out(p[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kFixUnroll; ++u)
      if (p[u] && v[u] < fo) store_out(p[u], fo);
  }
  __syncthreads();
}

}  // namespace lm
