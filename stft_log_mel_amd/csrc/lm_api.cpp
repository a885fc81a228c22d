// C-ABI entry points: per-call validation, device tables and workspace,
// and the launch sequence (main kernel, then the per-clip clamp fix-up) on
// the caller's stream.
#include <algorithm>
#include <cstring>

#include "lm_internal.h"

namespace lm {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int ensure_device(lm_plan *p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (p->device < 0) {
    int n_cu = 0;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    p->device = dev;
    p->n_cu = n_cu > 0 ? n_cu : 1;
  } else if (p->device != dev) {
    return fail(LM_ERR_INVALID_ARG, "plan is bound to another device");
  }
  return LM_OK;
}

int upload_tables(lm_plan *p) {
  if (!p->tables_dirty && p->dt.base) return LM_OK;
  const int N = p->n_fft, M = N / 2, NM = p->n_mels;
  const int nnz = (int)p->csr.w.size();
  size_t o_win = 0;
  size_t o_tw = align256(o_win + sizeof(float) * N);
  size_t o_ut = align256(o_tw + sizeof(float) * 2 * M);
  size_t o_st = align256(o_ut + sizeof(float) * 2 * (M / 2 + 1));
  size_t o_wd = align256(o_st + sizeof(int32_t) * NM);
  size_t o_of = align256(o_wd + sizeof(int32_t) * NM);
  size_t o_w = align256(o_of + sizeof(int32_t) * NM);
  size_t o_mf = align256(o_w + sizeof(float) * (nnz > 0 ? nnz : 1));
  size_t o_mh = o_mf;
  size_t o_bm = align256(o_mh + sizeof(uint16_t) * p->mfma400h.size());
  size_t o_bw = align256(o_bm + sizeof(int32_t) * p->melblk_meta.size());
  size_t o_t2 = align256(o_bw + sizeof(float) * p->melblk_w.size());
  std::vector<int32_t> empty;
  if (p->have_filters)
    for (int m = 0; m < NM; ++m)
      if (p->csr.width[m] == 0) empty.push_back(m);
  size_t o_eb = align256(o_t2 + sizeof(float) * p->twid2.size());
  size_t total = align256(o_eb + sizeof(int32_t) * empty.size() + 16);
  std::vector<unsigned char> host(total, 0);
  std::memcpy(host.data() + o_win, p->window.data(), sizeof(float) * N);
  std::memcpy(host.data() + o_tw, p->twiddle.data(), sizeof(float) * 2 * M);
  std::memcpy(host.data() + o_ut, p->untangle.data(), sizeof(float) * 2 * (M / 2 + 1));
  if (p->have_filters) {
    std::memcpy(host.data() + o_st, p->csr.start.data(), sizeof(int32_t) * NM);
    std::memcpy(host.data() + o_wd, p->csr.width.data(), sizeof(int32_t) * NM);
    std::memcpy(host.data() + o_of, p->csr.off.data(), sizeof(int32_t) * NM);
    if (nnz) std::memcpy(host.data() + o_w, p->csr.w.data(), sizeof(float) * nnz);
  }
  if (!p->mfma400h.empty())
    std::memcpy(host.data() + o_mh, p->mfma400h.data(), sizeof(uint16_t) * p->mfma400h.size());
  if (p->have_filters) {
    std::memcpy(host.data() + o_bm, p->melblk_meta.data(), sizeof(int32_t) * p->melblk_meta.size());
    std::memcpy(host.data() + o_bw, p->melblk_w.data(), sizeof(float) * p->melblk_w.size());
  }
  if (!p->twid2.empty()) std::memcpy(host.data() + o_t2, p->twid2.data(), sizeof(float) * p->twid2.size());
  if (!empty.empty()) std::memcpy(host.data() + o_eb, empty.data(), sizeof(int32_t) * empty.size());
  if (p->dt.base) {
    hipError_t e = hipFree(p->dt.base);
    p->dt.base = nullptr;
    if (e != hipSuccess) return hip_fail(e, "hipFree(tables)");
  }
  void *d = nullptr;
  hipError_t e = hipMalloc(&d, total);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(tables)");
  e = hipMemcpy(d, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(d);
    return hip_fail(e, "hipMemcpy(tables)");
  }
  unsigned char *c = static_cast<unsigned char *>(d);
  p->dt.base = d;
  p->dt.bytes = total;
  p->dt.window = reinterpret_cast<const float *>(c + o_win);
  p->dt.twiddle = reinterpret_cast<const float2 *>(c + o_tw);
  p->dt.untangle = reinterpret_cast<const float2 *>(c + o_ut);
  p->dt.tw2 = p->twid2.empty() ? nullptr : reinterpret_cast<const float2 *>(c + o_t2);
  p->dt.csr_start = reinterpret_cast<const int32_t *>(c + o_st);
  p->dt.csr_width = reinterpret_cast<const int32_t *>(c + o_wd);
  p->dt.csr_off = reinterpret_cast<const int32_t *>(c + o_of);
  p->dt.csr_w = reinterpret_cast<const float *>(c + o_w);
  p->dt.nnz = nnz;
  p->dt.mfma400h = p->mfma400h.empty() ? nullptr : reinterpret_cast<const uint16_t *>(c + o_mh);
  p->dt.melblk_meta = reinterpret_cast<const int32_t *>(c + o_bm);
  p->dt.melblk_w = reinterpret_cast<const float *>(c + o_bw);
  p->dt.n_melblk = p->have_filters ? (p->n_mels + 15) / 16 : 0;
  p->dt.empty_bands = reinterpret_cast<const int32_t *>(c + o_eb);
  p->dt.n_empty = (int)empty.size();
  p->tables_dirty = false;
  return LM_OK;
}

// Statistics workspace (minima, then maxima), grown on demand.  Every call
// overwrites all of the entries it reads, so nothing needs clearing.
int ensure_workspace(lm_plan *p, int64_t n_floats) {
  if ((size_t)n_floats <= p->stats_cap) return LM_OK;
  if (p->d_stats) {
    hipError_t e = hipFree(p->d_stats);
    p->d_stats = nullptr;
    p->stats_cap = 0;
    if (e != hipSuccess) return hip_fail(e, "hipFree(workspace)");
  }
  hipError_t e = hipMalloc(reinterpret_cast<void **>(&p->d_stats), sizeof(float) * n_floats);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
  p->stats_cap = n_floats;
  return LM_OK;
}

// Launch through `fn(tm)`; when profiling, tm carries two new events that
// the dispatch stamps at the kernel's start and end.
template <typename Fn>
static int timed_launch(lm_plan *p, hipStream_t s, int kind, const char *what, Fn fn) {
  (void)s;
  if (!p->profiling) {
    hipError_t e = fn(nullptr);
    return e == hipSuccess ? LM_OK : hip_fail(e, what);
  }
  LaunchTiming tm{};
  hipError_t e = hipEventCreate(&tm.beg);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  e = hipEventCreate(&tm.end);
  if (e != hipSuccess) {
    (void)hipEventDestroy(tm.beg);
    return hip_fail(e, "hipEventCreate");
  }
  e = fn(&tm);
  if (e != hipSuccess) {
    (void)hipEventDestroy(tm.beg);
    (void)hipEventDestroy(tm.end);
    return hip_fail(e, what);
  }
  p->prof.push_back(ProfileRec{tm.beg, tm.end, kind});
  return LM_OK;
}

}  // namespace lm

using namespace lm;

extern "C" {

int lm_from_pcm(lm_plan *p, const void *pcm, int in_dtype, int64_t n_clips, int64_t n_samples, void *out,
                void *stream) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (!p->have_filters) return fail(LM_ERR_NO_FILTERS, "call lm_plan_set_mel or lm_plan_set_filters first");
  if (in_dtype != LM_F32 && in_dtype != LM_I16) return fail(LM_ERR_INVALID_ARG, "in_dtype must be LM_F32 or LM_I16");
  if (n_clips < 0) return fail(LM_ERR_INVALID_ARG, "n_clips < 0");
  if (n_samples < 1) return fail(LM_ERR_INVALID_ARG, "n_samples < 1");
  const int64_t half = p->n_fft / 2;
  // the center padding applies to the signal with its zero padding (length t_sig)
  const int64_t t_sig = n_samples + 2 * p->sig_pad;
  if (!p->center && t_sig < p->n_fft) return fail(LM_ERR_INVALID_ARG, "center=0 needs n_samples + 2 pad >= n_fft");
  if (p->center && p->pad_mode == LM_PAD_REFLECT && t_sig <= half)
    return fail(LM_ERR_INVALID_ARG, "reflect padding needs n_samples + 2 pad > n_fft/2");
  if (p->center && p->pad_mode == LM_PAD_CIRCULAR && t_sig < half)
    return fail(LM_ERR_INVALID_ARG, "circular padding needs n_samples + 2 pad >= n_fft/2");
  if (n_clips == 0) return LM_OK;
  if (!pcm || !out) return fail(LM_ERR_INVALID_ARG, "pcm and out must be device pointers");
  const size_t in_align = in_dtype == LM_I16 ? 2 : 4, out_align = p->out_dtype == LM_F16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(pcm) % in_align) || (reinterpret_cast<uintptr_t>(out) % out_align))
    return fail(LM_ERR_INVALID_ARG, "misaligned pcm or out pointer");
  const int64_t F = lm_plan_num_frames(p, n_samples);
  if (F < 1) return (int)F;
  int rc = ensure_device(p);
  if (rc == LM_OK) rc = upload_tables(p);
  if (rc != LM_OK) return rc;
  const StatLayout st = pcm_stat_layout(p, in_dtype == LM_I16);
  const int64_t tiles = (F + st.frames_per_tile - 1) / st.frames_per_tile;
  if (tiles > INT32_MAX || n_clips * tiles > INT32_MAX) return fail(LM_ERR_UNSUPPORTED, "input too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n_min = n_clips * tiles * st.min_per_tile(), n_max = n_clips * tiles * st.max_per_tile;
  rc = ensure_workspace(p, n_min + n_max);
  if (rc != LM_OK) return rc;
  float *tmin = p->d_stats, *tmax = p->d_stats + n_min;

  PcmArgs a{pcm, in_dtype == LM_I16, n_clips, n_samples, F, (int)tiles, out, tmin, tmax};
  rc = timed_launch(p, s, 0, "launch(pcm kernel)", [&](const LaunchTiming *tm) { return launch_pcm(p, a, s, tm); });
  if (rc != LM_OK) return rc;
  if (p->output == LM_OUTPUT_MEL) return LM_OK;   // no per-clip tail
  FixupArgs fx{out, p->out_dtype == LM_F16, tmin, tmax, n_clips, F, p->n_mels, (int)tiles, st, 1};
  if (pcm_skips_empty_bands(p, in_dtype == LM_I16)) {
    fx.empty_bands = p->dt.empty_bands;
    fx.n_empty = p->dt.n_empty;
  }
  return timed_launch(p, s, 1, "launch(clamp fix-up)", [&](const LaunchTiming *tm) { return launch_fixup(fx, s, tm); });
}

int lm_from_stft(lm_plan *p, const void *stft, const float *mel_filters, int64_t n_clips, int64_t n_frames,
                 int64_t n_bins, int n_mels, void *out, void *stream) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (n_clips < 0 || n_frames < 0) return fail(LM_ERR_INVALID_ARG, "negative size");
  if (n_bins < 1 || n_bins > 8193) return fail(LM_ERR_INVALID_ARG, "n_bins must be in [1, 8193]");
  if (n_mels < 1 || n_mels > 256) return fail(LM_ERR_INVALID_ARG, "n_mels must be in [1, 256]");
  if (!mel_filters) {
    if (!p->have_filters) return fail(LM_ERR_NO_FILTERS, "no mel_filters given and the plan has none");
    if (n_bins != p->n_bins || n_mels != p->n_mels)
      return fail(LM_ERR_INVALID_ARG, "n_bins / n_mels do not match the plan's filterbank");
  } else if (reinterpret_cast<uintptr_t>(mel_filters) % 4) {
    return fail(LM_ERR_INVALID_ARG, "misaligned mel_filters pointer");
  }
  if (n_clips == 0 || n_frames == 0) return LM_OK;
  if (!stft || !out) return fail(LM_ERR_INVALID_ARG, "stft and out must be device pointers");
  const size_t out_align = p->out_dtype == LM_F16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(stft) % 8) || (reinterpret_cast<uintptr_t>(out) % out_align))
    return fail(LM_ERR_INVALID_ARG, "misaligned stft or out pointer");
  const int tf = stft_frames_per_tile((int)n_bins, n_mels);
  const int64_t tiles = (n_frames + tf - 1) / tf;
  if (tiles > INT32_MAX || n_clips * tiles > INT32_MAX) return fail(LM_ERR_UNSUPPORTED, "input too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int rc = ensure_device(p);
  if (rc == LM_OK && !mel_filters) rc = upload_tables(p);
  if (rc == LM_OK) rc = ensure_workspace(p, 2 * n_clips * tiles);
  if (rc != LM_OK) return rc;
  float *tmin = p->d_stats, *tmax = p->d_stats + n_clips * tiles;

  StftArgs a{reinterpret_cast<const float2 *>(stft), n_clips, n_frames, (int)n_bins, n_mels, tf, (int)tiles,
             nullptr, nullptr, nullptr, nullptr, 0, out, p->out_dtype == LM_F16, tmin, tmax, p->n_cu,
             p->output == LM_OUTPUT_MEL};
  if (mel_filters) {
    const size_t need = sizeof(int32_t) * 2 * n_mels;
    if (need > p->pack_cap) {
      if (p->d_pack) {
        hipError_t e = hipFree(p->d_pack);
        p->d_pack = nullptr;
        p->pack_cap = 0;
        if (e != hipSuccess) return hip_fail(e, "hipFree(pack)");
      }
      hipError_t e = hipMalloc(&p->d_pack, need);
      if (e != hipSuccess) return hip_fail(e, "hipMalloc(pack)");
      p->pack_cap = need;
    }
    int32_t *sw = reinterpret_cast<int32_t *>(p->d_pack);
    rc = timed_launch(p, s, 2, "launch(filter rows)",
                      [&](const LaunchTiming *tm) { return launch_pack(mel_filters, n_mels, (int)n_bins, sw, s, tm); });
    if (rc != LM_OK) return rc;
    a.f_start = sw;
    a.f_width = sw + n_mels;
    a.f_w = mel_filters;
    a.f_stride = (int)n_bins;
  } else {
    a.f_start = p->dt.csr_start;
    a.f_width = p->dt.csr_width;
    a.f_off = p->dt.csr_off;
    a.f_w = p->dt.csr_w;
  }
  rc = timed_launch(p, s, 0, "launch(stft kernel)", [&](const LaunchTiming *tm) { return launch_stft(a, s, tm); });
  if (rc != LM_OK) return rc;
  if (p->output == LM_OUTPUT_MEL) return LM_OK;   // no per-clip tail
  StatLayout st;
  st.frames_per_tile = tf;
  st.band_h = n_mels;
  FixupArgs fx{out, p->out_dtype == LM_F16, tmin, tmax, n_clips, n_frames, n_mels, (int)tiles, st, 0};
  return timed_launch(p, s, 1, "launch(clamp fix-up)", [&](const LaunchTiming *tm) { return launch_fixup(fx, s, tm); });
}

int lm_plan_profile(lm_plan *p, int enable) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  p->profiling = enable != 0;
  return LM_OK;
}

int lm_plan_profile_read(lm_plan *p, double *ms, int64_t *counts) {
  if (!p || !ms || !counts) return fail(LM_ERR_INVALID_ARG, "NULL argument");
  for (int i = 0; i < 3; ++i) {
    ms[i] = 0.0;
    counts[i] = 0;
  }
  int rc = LM_OK;
  for (auto &r : p->prof) {
    float t = 0.0f;
    hipError_t e = hipEventSynchronize(r.end);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.beg, r.end);
    if (e != hipSuccess && rc == LM_OK) rc = hip_fail(e, "profile events");
    if (r.kind >= 0 && r.kind < 3) {
      ms[r.kind] += t;
      counts[r.kind] += 1;
    }
    (void)hipEventDestroy(r.beg);
    (void)hipEventDestroy(r.end);
  }
  p->prof.clear();
  return rc;
}

void lm_plan_destroy(lm_plan *p) {
  if (!p) return;
  for (auto &r : p->prof) {
    (void)hipEventDestroy(r.beg);
    (void)hipEventDestroy(r.end);
  }
  if (p->dt.base) (void)hipFree(p->dt.base);
  if (p->d_stats) (void)hipFree(p->d_stats);
  if (p->d_pack) (void)hipFree(p->d_pack);
  delete p;
}

}  // extern "C"
