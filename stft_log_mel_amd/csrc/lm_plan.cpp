// Host side of a plan: argument validation and the tables a launch reads
// (window, FFT twiddles, packed mel filterbank).  Everything here runs on
// the host in float64 and rounds once to float32; no HIP call is made.
#include <cmath>
#include <cstdio>
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>

#include "lm_internal.h"

namespace lm {

static thread_local std::string g_last_error;

int fail(int status, const std::string &msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(hipError_t err, const char *what) {
  char buf[256];
  std::snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(err));
  g_last_error = buf;
  return err == hipErrorOutOfMemory ? LM_ERR_OOM : LM_ERR_HIP;
}

int Csr::max_width() const {
  int m = 0;
  for (int v : width) m = v > m ? v : m;
  return m;
}

static bool is_supported_nfft(int n) {
  if (n == 400) return true;
  if (n < 64 || n > 16384) return false;
  return (n & (n - 1)) == 0;
}

// Periodic Hann of win_length samples, 0.5 - 0.5 cos(2 pi i / win_length)
// (flashmel page, "Usage": the window is always the periodic Hann), placed
// at offset (n_fft - win_length) / 2 of the frame with zeros around it.
double window_at(const lm_plan *p, int n) {
  const int W = p->win_length, i = n - (p->n_fft - W) / 2;
  if (i < 0 || i >= W) return 0.0;
  if (W == 1) return 1.0;   // a one-point window is [1] (torch.hann_window's convention)
  return 0.5 - 0.5 * std::cos(2.0 * M_PI * (double)i / (double)W);
}

// Factor on |X|^2 from the normalisation: 1, 1 / sum_n w[n]^2 (window) or
// 1 / win_length (frame length).
double power_scale2(const lm_plan *p) {
  if (p->normalized == LM_NORMALIZED_WINDOW) {
    double s = 0.0;
    for (int n = 0; n < p->n_fft; ++n) s += window_at(p, n) * window_at(p, n);
    return 1.0 / s;
  }
  if (p->normalized == LM_NORMALIZED_FRAME_LENGTH) return 1.0 / (double)p->win_length;
  return 1.0;
}

void build_window(lm_plan *p) {
  const int N = p->n_fft;
  p->window.resize(N);
  for (int n = 0; n < N; ++n) p->window[n] = (float)window_at(p, n);
}

// exp(-2 pi i j / M) for the M-point complex FFT, and exp(-2 pi i k / N)
// for k = 0..M/2 to split its result into the N-point real transform.
void build_twiddles(lm_plan *p) {
  const int N = p->n_fft, M = N / 2;
  p->twiddle.resize(2 * (size_t)M);
  for (int j = 0; j < M; ++j) {
    const double a = 2.0 * M_PI * (double)j / (double)M;
    p->twiddle[2 * j] = (float)std::cos(a);
    p->twiddle[2 * j + 1] = (float)-std::sin(a);
  }
  p->untangle.resize(2 * (size_t)(M / 2 + 1));
  for (int k = 0; k <= M / 2; ++k) {
    const double a = 2.0 * M_PI * (double)k / (double)N;
    p->untangle[2 * k] = (float)std::cos(a);
    p->untangle[2 * k + 1] = (float)-std::sin(a);
  }
  // two-level table for the one-frame kernels (n_fft >= 8192):
  // exp(-2 pi i j / N) = hi[j / 128] * lo[j % 128]
  p->twid2.clear();
  if (N >= 8192) {
    const int nhi = N / 128;
    p->twid2.resize(2 * (size_t)(nhi + 128));
    for (int i = 0; i < nhi + 128; ++i) {
      const long j = i < nhi ? 128L * i : (long)(i - nhi);
      const double a = 2.0 * M_PI * (double)j / (double)N;
      p->twid2[2 * i] = (float)std::cos(a);
      p->twid2[2 * i + 1] = (float)-std::sin(a);
    }
  }
}

// Operand tables of the n_fft = 400 kernel's matrix-core stage (the
// 16 x 25 split of a 400-point DFT; matrices described below).
void build_mfma400(lm_plan *p) {
  // Matrix M_n1 (16 x 16) maps the samples y[n1 + 25 n2], n2 < 16, of 16
  // frames to row m: group g = m / 4 holds classes g + 1 (rows 4g, 4g+1,
  // real/imag) and 7 - g (rows 4g+2, 4g+3) for g < 3; group 3 holds class 4
  // (rows 12, 13) and the sums over even / odd n2 (rows 14, 15).  Class rows
  // are scaled by 2, so that every power value comes out as 4 |X|^2 like
  // the even/odd split's |2 S|^2.  Class k row: w[n] (cos, -sin)(2 pi k n / 400), n = n1 +
  // 25 n2 (angles reduced exactly in integers).
  static const int kA[4] = {1, 2, 3, 4}, kB[3] = {7, 6, 5};
  std::vector<double> win(400);
  for (int n = 0; n < 400; ++n) win[n] = window_at(p, n);
  auto entry = [&](int n1, int m, int n2) {
    const int n = n1 + 25 * n2;
    const int g = m / 4, sub = m % 4;
    if (g == 3 && sub >= 2) return ((n2 & 1) == sub - 2) ? win[n] : 0.0;
    const int k = sub < 2 ? kA[g] : kB[g];
    const double th = 2.0 * M_PI * (double)(((long)k * n) % 400) / 400.0;
    return 2.0 * win[n] * ((sub & 1) == 0 ? std::cos(th) : -std::sin(th));
  };
  // Operands of v_mfma_f32_16x16x32_f16, two products per n1: the samples
  // enter as two fp16 planes whose sum is x / 64 (int16: h = (x - (x mod
  // 64)) / 64 and l = x mod 64, both exact) or x 2^e (float: nearest fp16 and
  // nearest fp16 of the rest), and the matrix, scaled by 2^12, as the
  // sum of two fp16 parts (hi = nearest fp16, lo = nearest fp16 of the
  // rest), so that hi + lo carries about 22 bits.  Lane (m, g) holds
  // k-slots e < 8 standing for n2 = 4 (e / 2) + e % 2 + 2 (g % 2); lanes
  // of groups 0 and 3 supply h, those of groups 1 and 2 supply l / 64, so
  // both halves of every n2 are present once.  Entry [n1][part][g % 2][m]
  // holds the 8 values of slots e as fp16 bits.
  p->mfma400h.assign((size_t)25 * 2 * 2 * 16 * 8, 0);
  for (int n1 = 0; n1 < 25; ++n1)
    for (int h = 0; h < 2; ++h)
      for (int m = 0; m < 16; ++m)
        for (int e = 0; e < 8; ++e) {
          const int n2 = 4 * (e / 2) + e % 2 + 2 * h;
          const double v = 4096.0 * entry(n1, m, n2);
          const _Float16 hi = (_Float16)v;
          const _Float16 lo = (_Float16)(v - (double)hi);
          uint16_t bh, bl;
          std::memcpy(&bh, &hi, 2);
          std::memcpy(&bl, &lo, 2);
          p->mfma400h[((((size_t)n1 * 2 + 0) * 2 + h) * 16 + m) * 8 + e] = bh;
          p->mfma400h[((((size_t)n1 * 2 + 1) * 2 + h) * 16 + m) * 8 + e] = bl;
        }

  // Second stage: the 25-point DFT over n1, Z[k] = sum_n W25^(n k) z[n], as
  // a real 64 x 50 matrix (scaled by 2^8) on v_mfma_f32_16x16x32_f16.
  // Input index i = 2 n + (0: real, 1: imaginary part of z[n]).  Output rows
  // come in quads q = row / 4 < 13: Re Z[q], Im Z[q], Re Z[25 - q], Im
  // Z[25 - q] (q = 0 repeats Z[0]), so a lane holds the pair (q, 25 - q)
  // that a conjugate-mirror class or the 50-point real split needs; rows of
  // quads 13..15 are zero.  Both operands carry about 22 bits as fp16 hi +
  // lo parts, and the product keeps hi.hi, hi.lo and lo.hi: the K slots of
  // the five 32-wide steps pair, per 8-slot chunk of lane group gq,
  //   step 0: A hi, inputs 8 gq..          with B hi of the same inputs
  //   step 1: A hi, inputs 8 (4 + gq) (gq < 2) or 8 (gq - 2) (gq >= 2) with B hi / B lo
  //   step 2: A hi, inputs 8 (2 + gq)      with B lo
  //   step 3: A lo, inputs 8 gq            with B hi
  //   step 4: A lo, inputs 8 (4 + gq) (gq < 2); gq = 2: inputs 48, 49 as
  //           (hi.hi, hi.lo, lo.hi) and two zero slots; gq = 3: zero
  // (the kernel reads the matching B chunk).  Entry [mt][step][lane] holds
  // lane (row 16 mt + lane % 16, group lane / 16)'s 8 slots as fp16 bits.
  constexpr double kS2Scale = 256.0;
  // The second stage takes the first stage's values times 2^-10 as fp16:
  // with samples of magnitude at most 512 (both input forms) and the matrix
  // scaled by 2^12, every value stays below fp16's largest finite value when
  // each row's absolute sum over n2 keeps 2^12 * 512 * sum * 2^-10 under
  // 65504 (the periodic Hann gives sum <= 16 on a class row: 32768).
  double row_abs = 0.0;
  for (int n1 = 0; n1 < 25; ++n1)
    for (int m = 0; m < 16; ++m) {
      double sum = 0.0;
      for (int n2 = 0; n2 < 16; ++n2) sum += std::fabs(entry(n1, m, n2));
      row_abs = std::max(row_abs, sum);
    }
  p->mfma400t_fits = 4096.0 * 512.0 * row_abs / 1024.0 <= 60000.0;
  auto dft_coef = [](int row, int in) -> double {
    const int q = row / 4, r = row % 4;
    if (q > 12) return 0.0;
    const int k = r < 2 ? q : (25 - q) % 25;
    const int n = in / 2;
    const double th = 2.0 * M_PI * (double)((n * k) % 25) / 25.0;
    const double c = std::cos(th), s = std::sin(th);
    if ((r & 1) == 0) return (in & 1) == 0 ? c : s;   // Re Z[k] = sum cos re + sin im
    return (in & 1) == 0 ? -s : c;                     // Im Z[k] = sum -sin re + cos im
  };
  p->mfma400t.assign((size_t)4 * 5 * 64 * 8, 0);
  for (int mt = 0; mt < 4; ++mt)
    for (int t = 0; t < 5; ++t)
      for (int lane = 0; lane < 64; ++lane)
        for (int e = 0; e < 8; ++e) {
          const int row = 16 * mt + lane % 16, gq = lane / 16;
          int part = 0, in = -1;   // part 0: hi, 1: lo; in < 0: zero slot
          switch (t) {
            case 0: in = 8 * gq + e; break;
            case 1: in = 8 * (gq < 2 ? 4 + gq : gq - 2) + e; break;
            case 2: in = 8 * (2 + gq) + e; break;
            case 3: part = 1; in = 8 * gq + e; break;
            default:
              if (gq < 2) {
                part = 1;
                in = 8 * (4 + gq) + e;
              } else if (gq == 2 && e < 6) {
                part = e < 4 ? 0 : 1;
                in = 48 + e % 2;
              }
          }
          if (in < 0) continue;
          const double v = kS2Scale * dft_coef(row, in);
          const _Float16 hi = (_Float16)v;
          const _Float16 lo = (_Float16)(v - (double)hi);
          uint16_t b;
          std::memcpy(&b, part == 0 ? &hi : &lo, 2);
          p->mfma400t[(((size_t)mt * 5 + t) * 64 + lane) * 8 + e] = b;
        }
}

// Filterbank tables for the n_fft = 400 kernel's mel sum on 4x4x1 matrix
// blocks.  Bands go in blocks of 16 = 4 quads of 4; a step s of block jb
// multiplies, for every quad Q = 4 jb + q at once, the weights of its 4
// bands at bin qs[Q] + s by the power of 16 frames at that bin.  Block jb
// takes nst steps (the widest of its quads' bin spans, padded to whole
// batches of kMelBatch steps, at least one batch); qs[Q] is the quad's
// first non-zero bin, moved down so that qs[Q] + nst stays inside the
// kernel's power row.  The batches of all blocks form one sequence.  Tables:
// per batch, for each quad q of its block, the bin of its first step, with
// bit 16 set on a block's last batch; weights per batch as [q][band in
// quad][step], 16 kMelBatch floats, zero outside a band's support.
void build_mel_blocks(lm_plan *p) {
  p->melblk_meta.clear();
  p->melblk_w.clear();
  if (p->n_fft != 400) return;
  const Csr &c = p->csr;
  const int NM = c.n_rows, NB = (NM + 15) / 16;
  for (int jb = 0; jb < NB; ++jb) {
    int lo[4], span[4], nst = 0;
    for (int q = 0; q < 4; ++q) {
      int klo = 1 << 30, khi = 0;
      for (int m = 16 * jb + 4 * q; m < NM && m < 16 * jb + 4 * q + 4; ++m)
        if (c.width[m] > 0) {
          klo = std::min(klo, c.start[m]);
          khi = std::max(khi, c.start[m] + c.width[m]);
        }
      lo[q] = khi > klo ? klo : 0;
      span[q] = khi > klo ? khi - klo : 0;
      nst = std::max(nst, span[q]);
    }
    nst = std::max(kMelBatch, (nst + kMelBatch - 1) / kMelBatch * kMelBatch);
    int qs[4];
    for (int q = 0; q < 4; ++q) qs[q] = std::min(lo[q], kPcm400Row - nst);
    for (int s0 = 0; s0 < nst; s0 += kMelBatch) {
      for (int q = 0; q < 4; ++q) p->melblk_meta.push_back((qs[q] + s0) | (s0 + kMelBatch == nst ? 1 << 16 : 0));
      for (int q = 0; q < 4; ++q)
        for (int t = 0; t < 4; ++t)
          for (int u = 0; u < kMelBatch; ++u) {
            const int m = 16 * jb + 4 * q + t, k = qs[q] + s0 + u;
            float v = 0.0f;
            if (m < NM && k >= c.start[m] && k < c.start[m] + c.width[m]) v = c.w[c.off[m] + k - c.start[m]];
            p->melblk_w.push_back(v);
          }
    }
  }
}

// Lane table of the one-frame kernels' mel stage (n_fft >= 8192, `threads`
// lanes): every band gets a group of L lanes (a power of two, at most 64,
// aligned to L within its wave) that stride over its bins and add their
// partial sums with xor shuffles.  L starts at 1 and doubles for the band
// with the most bins per lane while lanes remain, so that the widest bands
// (hundreds of bins) get many lanes and the narrow ones few.  Entry of lane
// t: band | (position in group << 8) | (log2 L << 16), or -1 (idle).
void build_mel_lanes(lm_plan *p, int threads) {
  p->mel_lanes.clear();
  if (p->n_fft < 8192) return;
  const Csr &c = p->csr;
  const int NM = c.n_rows;
  std::vector<int> L(NM, 1);
  int used = NM;
  for (;;) {
    int best = -1, best_cost = 1;
    for (int m = 0; m < NM; ++m) {
      const int cost = (c.width[m] + L[m] - 1) / L[m];
      if (L[m] < 64 && used + L[m] <= threads && cost > best_cost) {
        best = m;
        best_cost = cost;
      }
    }
    if (best < 0) break;
    used += L[best];
    L[best] *= 2;
  }
  // place groups largest first: every offset is then a multiple of the group
  // size, so no group straddles a 64-lane wave
  std::vector<int> order(NM);
  for (int m = 0; m < NM; ++m) order[m] = m;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return L[x] > L[y]; });
  p->mel_lanes.assign(threads, -1);
  int off = 0;
  for (int m : order) {
    int lg = 0;
    while ((1 << lg) < L[m]) ++lg;
    for (int h = 0; h < L[m]; ++h) p->mel_lanes[off + h] = m | (h << 8) | (lg << 16);
    off += L[m];
  }
}

Csr pack_dense(const float *dense, int n_rows, int n_bins) {
  Csr c;
  c.n_rows = n_rows;
  c.n_bins = n_bins;
  c.start.assign(n_rows, 0);
  c.width.assign(n_rows, 0);
  c.off.assign(n_rows, 0);
  int off = 0;
  for (int m = 0; m < n_rows; ++m) {
    const float *row = dense + (size_t)m * n_bins;
    int first = -1, last = -1;
    for (int k = 0; k < n_bins; ++k)
      if (row[k] != 0.0f) {
        if (first < 0) first = k;
        last = k;
      }
    c.off[m] = off;
    if (first >= 0) {
      c.start[m] = first;
      c.width[m] = last - first + 1;
      for (int k = first; k <= last; ++k) c.w.push_back(row[k]);
      off += last - first + 1;
    }
  }
  return c;
}

// Mel scales.  Slaney: 3f/200 below 1 kHz, then 27 mels per factor 6.4.
static double hz_to_mel(double f, int scale) {
  if (scale == LM_MEL_HTK) return 2595.0 * std::log10(1.0 + f / 700.0);
  const double f_sp = 200.0 / 3.0, brk = 1000.0, step = std::log(6.4) / 27.0;
  return f < brk ? f / f_sp : brk / f_sp + std::log(f / brk) / step;
}

static double mel_to_hz(double m, int scale) {
  if (scale == LM_MEL_HTK) return 700.0 * (std::pow(10.0, m / 2595.0) - 1.0);
  const double f_sp = 200.0 / 3.0, brk = 1000.0, step = std::log(6.4) / 27.0;
  const double brk_mel = brk / f_sp;
  return m < brk_mel ? f_sp * m : brk * std::exp(step * (m - brk_mel));
}

}  // namespace lm

using namespace lm;

extern "C" {

const char *lm_last_error(void) { return g_last_error.c_str(); }

const char *lm_status_string(int s) {
  switch (s) {
    case LM_OK: return "ok";
    case LM_ERR_INVALID_ARG: return "invalid argument";
    case LM_ERR_UNSUPPORTED: return "unsupported configuration";
    case LM_ERR_NO_FILTERS: return "plan has no filterbank";
    case LM_ERR_HIP: return "HIP runtime error";
    case LM_ERR_OOM: return "out of memory";
    default: return "unknown status";
  }
}

int lm_plan_create(lm_plan **plan, int n_fft, int hop, int n_mels, int center, int pad_mode,
                   float power, int out_dtype) {
  g_last_error.clear();
  if (!plan) return fail(LM_ERR_INVALID_ARG, "plan out-pointer is NULL");
  if (!is_supported_nfft(n_fft))
    return fail(LM_ERR_UNSUPPORTED, "n_fft must be 400 or a power of two in [64, 16384]");
  if (hop < 1) return fail(LM_ERR_INVALID_ARG, "hop must be >= 1");
  if (n_mels < 1 || n_mels > 256) return fail(LM_ERR_INVALID_ARG, "n_mels must be in [1, 256]");
  if (center != 0 && center != 1) return fail(LM_ERR_INVALID_ARG, "center must be 0 or 1");
  if (pad_mode < LM_PAD_CONSTANT || pad_mode > LM_PAD_CIRCULAR)
    return fail(LM_ERR_INVALID_ARG, "unknown pad_mode");
  if (!(power > 0.0f) || !std::isfinite(power))
    return fail(LM_ERR_INVALID_ARG, "power must be finite and > 0");
  if (out_dtype != LM_F32 && out_dtype != LM_F16)
    return fail(LM_ERR_INVALID_ARG, "out_dtype must be LM_F32 or LM_F16");
  lm_plan *p = new (std::nothrow) lm_plan();
  if (!p) return fail(LM_ERR_OOM, "host allocation failed");
  p->n_fft = n_fft;
  p->hop = hop;
  p->n_mels = n_mels;
  p->center = center;
  p->pad_mode = pad_mode;
  p->power = power;
  p->out_dtype = out_dtype;
  p->n_bins = n_fft / 2 + 1;
  p->win_length = n_fft;
  build_window(p);
  build_twiddles(p);
  if (n_fft == 400) build_mfma400(p);
  *plan = p;
  return LM_OK;
}

int lm_plan_set_output(lm_plan *p, int output, int normalized) {
  g_last_error.clear();
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (output != LM_OUTPUT_LOGMEL && output != LM_OUTPUT_MEL) return fail(LM_ERR_INVALID_ARG, "unknown output");
  if (normalized < LM_NORMALIZED_NONE || normalized > LM_NORMALIZED_FRAME_LENGTH)
    return fail(LM_ERR_INVALID_ARG, "unknown normalized mode");
  p->output = output;
  p->normalized = normalized;
  return LM_OK;
}

int lm_plan_set_window(lm_plan *p, int win_length) {
  g_last_error.clear();
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (win_length < 1 || win_length > p->n_fft) return fail(LM_ERR_INVALID_ARG, "need 1 <= win_length <= n_fft");
  if (win_length == p->win_length) return LM_OK;
  p->win_length = win_length;
  build_window(p);
  if (p->n_fft == 400) build_mfma400(p);
  p->tables_dirty = true;
  return LM_OK;
}

int lm_plan_set_pad(lm_plan *p, int64_t pad) {
  g_last_error.clear();
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (pad < 0 || pad > ((int64_t)1 << 30)) return fail(LM_ERR_INVALID_ARG, "need 0 <= pad <= 2^30");
  p->sig_pad = pad;
  return LM_OK;
}

int lm_plan_set_mel(lm_plan *p, double sr, double f_min, double f_max, int scale, int norm) {
  g_last_error.clear();
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (!(sr > 0.0) || !std::isfinite(sr)) return fail(LM_ERR_INVALID_ARG, "sample_rate must be > 0");
  if (!(f_min >= 0.0) || !(f_max > f_min) || !(f_max <= sr / 2.0))
    return fail(LM_ERR_INVALID_ARG, "need 0 <= f_min < f_max <= sample_rate / 2");
  if (scale != LM_MEL_SLANEY && scale != LM_MEL_HTK) return fail(LM_ERR_INVALID_ARG, "mel_scale");
  if (norm != LM_NORM_SLANEY && norm != LM_NORM_NONE) return fail(LM_ERR_INVALID_ARG, "norm");
  const int NM = p->n_mels, K = p->n_bins;
  std::vector<double> fpts(NM + 2);
  const double m_lo = hz_to_mel(f_min, scale), m_hi = hz_to_mel(f_max, scale);
  for (int i = 0; i < NM + 2; ++i) {
    const double m = (i == NM + 1) ? m_hi : m_lo + (m_hi - m_lo) * (double)i / (double)(NM + 1);
    fpts[i] = mel_to_hz(m, scale);
  }
  std::vector<float> dense((size_t)NM * K, 0.0f);
  for (int m = 0; m < NM; ++m) {
    const double lo = fpts[m], mid = fpts[m + 1], hi = fpts[m + 2];
    const double g = (norm == LM_NORM_SLANEY) ? 2.0 / (hi - lo) : 1.0;
    for (int k = 0; k < K; ++k) {
      const double fk = (double)k * sr / (double)p->n_fft;
      const double rise = (fk - lo) / (mid - lo), fall = (hi - fk) / (hi - mid);
      const double w = std::fmax(0.0, std::fmin(rise, fall));
      dense[(size_t)m * K + k] = (float)(w * g);
    }
  }
  p->csr = pack_dense(dense.data(), NM, K);
  build_mel_blocks(p);
  build_mel_lanes(p, big_threads(p->n_fft));
  p->have_filters = true;
  p->tables_dirty = true;
  return LM_OK;
}

int lm_plan_set_filters(lm_plan *p, const float *host_dense, int n_mels, int n_bins) {
  g_last_error.clear();
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (!host_dense) return fail(LM_ERR_INVALID_ARG, "filters pointer is NULL");
  if (n_mels != p->n_mels || n_bins != p->n_bins)
    return fail(LM_ERR_INVALID_ARG, "filters must be (n_mels, n_fft/2 + 1)");
  for (size_t i = 0; i < (size_t)n_mels * n_bins; ++i)
    if (!std::isfinite(host_dense[i])) return fail(LM_ERR_INVALID_ARG, "filters hold a non-finite value");
  p->csr = pack_dense(host_dense, n_mels, n_bins);
  build_mel_blocks(p);
  build_mel_lanes(p, big_threads(p->n_fft));
  p->have_filters = true;
  p->tables_dirty = true;
  return LM_OK;
}

int lm_plan_get_filters(const lm_plan *p, float *out, int n_mels, int n_bins) {
  g_last_error.clear();
  if (!p || !out) return fail(LM_ERR_INVALID_ARG, "NULL argument");
  if (!p->have_filters) return fail(LM_ERR_NO_FILTERS, "plan has no filterbank");
  if (n_mels != p->n_mels || n_bins != p->n_bins)
    return fail(LM_ERR_INVALID_ARG, "shape must be (n_mels, n_fft/2 + 1)");
  std::memset(out, 0, sizeof(float) * (size_t)n_mels * n_bins);
  for (int m = 0; m < n_mels; ++m)
    for (int j = 0; j < p->csr.width[m]; ++j)
      out[(size_t)m * n_bins + p->csr.start[m] + j] = p->csr.w[p->csr.off[m] + j];
  return LM_OK;
}

int64_t lm_plan_num_frames(const lm_plan *p, int64_t n_samples) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (n_samples < 0) return fail(LM_ERR_INVALID_ARG, "n_samples < 0");
  const int64_t t_pad = n_samples + 2 * p->sig_pad + (p->center ? 2 * (int64_t)(p->n_fft / 2) : 0);
  if (t_pad < p->n_fft) return fail(LM_ERR_INVALID_ARG, "signal shorter than one frame");
  return 1 + (t_pad - p->n_fft) / p->hop;
}

}  // extern "C"
