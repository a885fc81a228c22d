// C-ABI entry points: per-call validation, device tables and workspace,
// and the launch sequence (main kernel, then the per-clip clamp fix-up) on
// the caller's stream.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>

#include "lm_internal.h"

namespace lm {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device bytes the plan holds: tables, statistics, filter pack, single-pass slots.
size_t plan_device_bytes(const lm_plan *p) {
  return p->dt.bytes + p->stats_cap * sizeof(float) + p->pack_cap + p->sync_cap;
}

// Bytes a buffer of `cap` bytes may grow to under the plan's limit, given
// that it needs `need`: the doubled size if that fits, else `need`, else 0
// (the limit is exceeded).
static size_t limited_size(const lm_plan *p, size_t cap, size_t need) {
  const size_t want = std::max(need, 2 * cap);
  if (p->mem_limit == 0) return want;
  const size_t others = plan_device_bytes(p) - cap;
  if (others + want <= p->mem_limit) return want;
  if (others + need <= p->mem_limit) return need;
  return 0;
}

static int over_limit(const lm_plan *p, size_t need, const char *what) {
  char buf[192];
  std::snprintf(buf, sizeof buf, "%s: %zu more bytes would pass the plan's device-memory limit of %zu (%zu held)",
                what, need, p->mem_limit, plan_device_bytes(p));
  return fail(LM_ERR_OOM, buf);
}

int ensure_device(lm_plan *p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (p->device < 0) {
    int n_cu = 0;
    e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    int coop = 0;
    e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    p->device = dev;
    p->n_cu = n_cu > 0 ? n_cu : 1;
    p->coop_launch = coop != 0;
  } else if (p->device != dev) {
    return fail(LM_ERR_INVALID_ARG, "plan is bound to another device");
  }
  return LM_OK;
}

// A pinned staging buffer of at least `bytes` whose previous copy (if any)
// has finished, reusing the plan's own when possible.
static int acquire_staging(lm_plan *p, size_t bytes, Staging **out) {
  for (auto &st : p->staging)
    if (st.bytes >= bytes && hipEventQuery(st.done) == hipSuccess) {
      *out = &st;
      return LM_OK;
    }
  Staging st;
  hipError_t e = hipHostMalloc(&st.host, bytes, hipHostMallocDefault);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(table staging)");
  st.bytes = bytes;
  e = hipEventCreateWithFlags(&st.done, hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)hipHostFree(st.host);
    return hip_fail(e, "hipEventCreate(table staging)");
  }
  p->staging.push_back(st);
  *out = &p->staging.back();
  return LM_OK;
}

// Device tables of the plan, refreshed after its host tables change.  The
// image is assembled in pinned host memory and copied asynchronously into a
// new stream-ordered allocation; the previous copy is released in stream
// order behind the work already enqueued (every call on the plan is ordered
// after the one before, see begin_call), so no call waits for the device.
int upload_tables(lm_plan *p, hipStream_t s) {
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
  size_t o_mt = align256(o_mh + sizeof(uint16_t) * p->mfma400h.size());
  size_t o_bm = align256(o_mt + sizeof(uint16_t) * p->mfma400t.size());
  size_t o_bw = align256(o_bm + sizeof(int32_t) * p->melblk_meta.size());
  size_t o_t2 = align256(o_bw + sizeof(float) * p->melblk_w.size());
  std::vector<int32_t> empty;
  if (p->have_filters)
    for (int m = 0; m < NM; ++m)
      if (p->csr.width[m] == 0) empty.push_back(m);
  size_t o_eb = align256(o_t2 + sizeof(float) * p->twid2.size());
  size_t o_ml = align256(o_eb + sizeof(int32_t) * empty.size());
  size_t total = align256(o_ml + sizeof(int32_t) * p->mel_lanes.size() + 16);
  if (p->mem_limit && plan_device_bytes(p) - p->dt.bytes + total > p->mem_limit)
    return over_limit(p, total > p->dt.bytes ? total - p->dt.bytes : 0, "device tables");
  Staging *stg = nullptr;
  int rc = acquire_staging(p, total, &stg);
  if (rc != LM_OK) return rc;
  unsigned char *host = static_cast<unsigned char *>(stg->host);
  std::memset(host, 0, total);
  std::memcpy(host + o_win, p->window.data(), sizeof(float) * N);
  std::memcpy(host + o_tw, p->twiddle.data(), sizeof(float) * 2 * M);
  std::memcpy(host + o_ut, p->untangle.data(), sizeof(float) * 2 * (M / 2 + 1));
  if (p->have_filters) {
    std::memcpy(host + o_st, p->csr.start.data(), sizeof(int32_t) * NM);
    std::memcpy(host + o_wd, p->csr.width.data(), sizeof(int32_t) * NM);
    std::memcpy(host + o_of, p->csr.off.data(), sizeof(int32_t) * NM);
    if (nnz) std::memcpy(host + o_w, p->csr.w.data(), sizeof(float) * nnz);
  }
  if (!p->mfma400h.empty())
    std::memcpy(host + o_mh, p->mfma400h.data(), sizeof(uint16_t) * p->mfma400h.size());
  if (!p->mfma400t.empty())
    std::memcpy(host + o_mt, p->mfma400t.data(), sizeof(uint16_t) * p->mfma400t.size());
  if (p->have_filters) {
    std::memcpy(host + o_bm, p->melblk_meta.data(), sizeof(int32_t) * p->melblk_meta.size());
    std::memcpy(host + o_bw, p->melblk_w.data(), sizeof(float) * p->melblk_w.size());
  }
  if (!p->twid2.empty()) std::memcpy(host + o_t2, p->twid2.data(), sizeof(float) * p->twid2.size());
  if (!empty.empty()) std::memcpy(host + o_eb, empty.data(), sizeof(int32_t) * empty.size());
  if (!p->mel_lanes.empty()) std::memcpy(host + o_ml, p->mel_lanes.data(), sizeof(int32_t) * p->mel_lanes.size());
  void *d = nullptr;
  hipError_t e = hipMallocAsync(&d, total, s);
  if (e != hipSuccess) return hip_fail(e, "hipMallocAsync(tables)");
  e = hipMemcpyAsync(d, host, total, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(stg->done, s);
  if (e != hipSuccess) {
    (void)hipFreeAsync(d, s);
    return hip_fail(e, "hipMemcpyAsync(tables)");
  }
  if (p->dt.base) (void)hipFreeAsync(p->dt.base, s);
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
  p->dt.mfma400t = p->mfma400t.empty() ? nullptr : reinterpret_cast<const uint16_t *>(c + o_mt);
  p->dt.melblk_meta = reinterpret_cast<const int32_t *>(c + o_bm);
  p->dt.melblk_w = reinterpret_cast<const float *>(c + o_bw);
  p->dt.n_melblk = p->have_filters ? (p->n_mels + 15) / 16 : 0;
  p->dt.empty_bands = reinterpret_cast<const int32_t *>(c + o_eb);
  p->dt.n_empty = (int)empty.size();
  p->dt.mel_lanes = p->mel_lanes.empty() ? nullptr : reinterpret_cast<const int32_t *>(c + o_ml);
  p->tables_dirty = false;
  return LM_OK;
}

// Grow a stream-ordered device buffer to at least `need` bytes (doubling
// while the plan's memory limit allows), releasing the old one in stream
// order behind the work already enqueued.
static int grow(lm_plan *p, void **buf, size_t *cap, size_t need, hipStream_t s, const char *what) {
  if (need <= *cap) return LM_OK;
  const size_t bytes = limited_size(p, *cap, need);
  if (bytes == 0) return over_limit(p, need - *cap, what);
  void *d = nullptr;
  hipError_t e = hipMallocAsync(&d, bytes, s);
  if (e != hipSuccess) return hip_fail(e, what);
  if (*buf) (void)hipFreeAsync(*buf, s);
  *buf = d;
  *cap = bytes;
  return LM_OK;
}

// Statistics workspace (minima, then maxima).  Every call overwrites all of
// the entries it reads, so nothing needs clearing.
int ensure_workspace(lm_plan *p, int64_t n_floats, hipStream_t s) {
  void *buf = p->d_stats;
  size_t cap = p->stats_cap * sizeof(float);
  const int rc = grow(p, &buf, &cap, sizeof(float) * (size_t)n_floats, s, "hipMallocAsync(workspace)");
  p->d_stats = static_cast<float *>(buf);
  p->stats_cap = cap / sizeof(float);
  return rc;
}

// Single-pass slots of the plan (2 + n_clips words), zeroed when grown
// (which restarts the barrier parity).
static int ensure_sync(lm_plan *p, int64_t slots, hipStream_t s) {
  const size_t need = sizeof(uint64_t) * (size_t)slots;
  if (need <= p->sync_cap) return LM_OK;
  p->sync_calls = 0;
  void *buf = p->d_sync;
  size_t cap = p->sync_cap;
  int rc = grow(p, &buf, &cap, need, s, "hipMallocAsync(single-pass slots)");
  p->d_sync = static_cast<uint64_t *>(buf);
  p->sync_cap = cap;
  if (rc != LM_OK) return rc;
  const hipError_t e = launch_zero_u64(p->d_sync, cap / sizeof(uint64_t), s);
  return e == hipSuccess ? LM_OK : hip_fail(e, "launch(zero slots)");
}

uint32_t next_epoch() {
  static std::atomic<uint32_t> g_epoch{0};
  uint32_t e = ++g_epoch;
  while (e == 0) e = ++g_epoch;   // 0 marks a slot never used
  return e;
}

int begin_call(lm_plan *p, hipStream_t s) {
  int rc = ensure_device(p);
  if (rc != LM_OK) return rc;
  if (!p->done_event) {
    hipError_t e = hipEventCreateWithFlags(&p->done_event, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  if (p->has_last && p->last_stream != static_cast<void *>(s)) {
    hipError_t e = hipEventRecord(p->done_event, reinterpret_cast<hipStream_t>(p->last_stream));
    if (e == hipSuccess) e = hipStreamWaitEvent(s, p->done_event, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  return LM_OK;
}

int end_call(lm_plan *p, hipStream_t s, int rc) {
  p->last_stream = static_cast<void *>(s);
  p->has_last = true;
  return rc;
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

static int run_pcm_launches(lm_plan *p, const void *pcm, bool in_i16, int64_t n_clips, int64_t n_samples,
                            int64_t F, int tiles, const StatLayout &st, void *out, float *ws, uint64_t *sync,
                            int parity, hipStream_t s);

// Host-side checks of an lm_from_pcm call (no HIP call); fills the call's
// geometry.  n_clips == 0 passes and needs no launch.
int validate_pcm(const lm_plan *p, const void *pcm, int in_dtype, int64_t n_clips, int64_t n_samples,
                 const void *out, PcmCall *c) {
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
  c->F = F;
  c->st = pcm_stat_layout(p, in_dtype == LM_I16);
  const int64_t tiles = (F + c->st.frames_per_tile - 1) / c->st.frames_per_tile;
  if (tiles > INT32_MAX || n_clips * tiles > INT32_MAX) return fail(LM_ERR_UNSUPPORTED, "input too large");
  c->tiles = (int)tiles;
  c->ws_floats = n_clips * tiles * (c->st.min_per_tile() + c->st.max_per_tile);
  return LM_OK;
}

// The PCM launch sequence (main kernel, then the clamp fix-up) with the
// statistics workspace at `ws` (n_clips * tiles * (minima + maxima) floats).
// With allow_profile false no timing events are created (no allocation).
int run_pcm(lm_plan *p, const void *pcm, bool in_i16, int64_t n_clips, int64_t n_samples, int64_t F, int tiles,
            const StatLayout &st, void *out, float *ws, uint64_t *sync, int parity, hipStream_t s,
            bool allow_profile) {
  const bool prof = p->profiling;
  if (!allow_profile) p->profiling = false;
  const int rc = run_pcm_launches(p, pcm, in_i16, n_clips, n_samples, F, tiles, st, out, ws, sync, parity, s);
  p->profiling = prof;
  return rc;
}

static int run_pcm_launches(lm_plan *p, const void *pcm, bool in_i16, int64_t n_clips, int64_t n_samples,
                            int64_t F, int tiles, const StatLayout &st, void *out, float *ws, uint64_t *sync,
                            int parity, hipStream_t s) {
  float *tmin = ws, *tmax = ws ? ws + n_clips * tiles * st.min_per_tile() : nullptr;
  PcmArgs a{pcm, in_i16, n_clips, n_samples, F, tiles, out, tmin, tmax};
  if (sync) {   // one pass: the kernel floors each clip itself
    a.sync = sync;
    a.epoch = next_epoch();
    a.parity = parity;
    return timed_launch(p, s, 0, "launch(pcm kernel, single pass)",
                        [&](const LaunchTiming *tm) { return launch_pcm(p, a, s, tm); });
  }
  int rc = timed_launch(p, s, 0, "launch(pcm kernel)", [&](const LaunchTiming *tm) { return launch_pcm(p, a, s, tm); });
  if (rc != LM_OK) return rc;
  if (p->output == LM_OUTPUT_MEL) return LM_OK;   // no per-clip tail
  FixupArgs fx{out, p->out_dtype == LM_F16, tmin, tmax, n_clips, F, p->n_mels, tiles, st, 1};
  if (pcm_skips_empty_bands(p, in_i16)) {
    fx.empty_bands = p->dt.empty_bands;
    fx.n_empty = p->dt.n_empty;
  }
  return timed_launch(p, s, 1, "launch(clamp fix-up)", [&](const LaunchTiming *tm) { return launch_fixup(fx, s, tm); });
}

// The STFT launch sequence: row spans of a device filterbank (if given),
// main kernel, clamp fix-up.  Uses the plan's workspace and pack buffer.
static int run_stft(lm_plan *p, const void *stft, const float *mel_filters, int64_t n_clips, int64_t n_frames,
                    int n_bins, int n_mels, int tf, int tiles, void *out, hipStream_t s) {
  float *tmin = p->d_stats, *tmax = p->d_stats + n_clips * tiles;
  StftArgs a{reinterpret_cast<const float2 *>(stft), n_clips, n_frames, n_bins, n_mels, tf, tiles,
             nullptr, nullptr, nullptr, nullptr, 0, out, p->out_dtype == LM_F16, tmin, tmax, p->n_cu,
             p->output == LM_OUTPUT_MEL};
  int rc = LM_OK;
  if (mel_filters) {
    int32_t *sw = reinterpret_cast<int32_t *>(p->d_pack);
    rc = timed_launch(p, s, 2, "launch(filter rows)",
                      [&](const LaunchTiming *tm) { return launch_pack(mel_filters, n_mels, n_bins, sw, s, tm); });
    if (rc != LM_OK) return rc;
    a.f_start = sw;
    a.f_width = sw + n_mels;
    a.f_w = mel_filters;
    a.f_stride = n_bins;
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
  FixupArgs fx{out, p->out_dtype == LM_F16, tmin, tmax, n_clips, n_frames, n_mels, tiles, st, 0};
  return timed_launch(p, s, 1, "launch(clamp fix-up)", [&](const LaunchTiming *tm) { return launch_fixup(fx, s, tm); });
}

}  // namespace lm

using namespace lm;

extern "C" {

int lm_from_pcm(lm_plan *p, const void *pcm, int in_dtype, int64_t n_clips, int64_t n_samples, void *out,
                void *stream) {
  PcmCall c;
  int rc = validate_pcm(p, pcm, in_dtype, n_clips, n_samples, out, &c);
  if (rc != LM_OK || n_clips == 0) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  rc = begin_call(p, s);
  if (rc != LM_OK) return rc;
  rc = upload_tables(p, s);
  const bool one_pass = pcm400_single_pass(p, in_dtype == LM_I16, n_clips * c.tiles);
  if (rc == LM_OK) rc = one_pass ? ensure_sync(p, 2 + n_clips, s) : ensure_workspace(p, c.ws_floats, s);
  if (rc == LM_OK)
    rc = run_pcm(p, pcm, in_dtype == LM_I16, n_clips, n_samples, c.F, c.tiles, c.st, out, one_pass ? nullptr : p->d_stats,
                 one_pass ? p->d_sync : nullptr, one_pass ? (int)(p->sync_calls++ & 1) : 0, s, true);
  return end_call(p, s, rc);
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
  const int tf0 = stft_frames_per_tile((int)n_bins, n_mels, 0, 0);
  if ((n_frames + tf0 - 1) / tf0 > INT32_MAX || n_clips * ((n_frames + tf0 - 1) / tf0) > INT32_MAX)
    return fail(LM_ERR_UNSUPPORTED, "input too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int rc = begin_call(p, s);
  if (rc != LM_OK) return rc;
  // the tile size of a small call depends on the device's CU count (bound now)
  const int tf = stft_frames_per_tile((int)n_bins, n_mels, n_clips * n_frames, p->n_cu);
  const int64_t tiles = (n_frames + tf - 1) / tf;
  if (tiles > INT32_MAX || n_clips * tiles > INT32_MAX) return end_call(p, s, fail(LM_ERR_UNSUPPORTED, "input too large"));
  if (!mel_filters) rc = upload_tables(p, s);
  if (rc == LM_OK) rc = ensure_workspace(p, 2 * n_clips * tiles, s);
  if (mel_filters && rc == LM_OK) rc = grow(p, &p->d_pack, &p->pack_cap, sizeof(int32_t) * 2 * n_mels, s, "hipMallocAsync(pack)");
  if (rc == LM_OK) rc = run_stft(p, stft, mel_filters, n_clips, n_frames, (int)n_bins, n_mels, tf, (int)tiles, out, s);
  return end_call(p, s, rc);
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
  if (p->d_sync) (void)hipFree(p->d_sync);
  for (auto &st : p->staging) {
    (void)hipEventSynchronize(st.done);
    (void)hipEventDestroy(st.done);
    (void)hipHostFree(st.host);
  }
  if (p->done_event) (void)hipEventDestroy(p->done_event);
  delete p;
}

int lm_plan_set_single_pass(lm_plan *p, int enable) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (enable != 0 && enable != 1) return fail(LM_ERR_INVALID_ARG, "enable must be 0 or 1");
  p->single_pass = enable;
  return LM_OK;
}

int lm_plan_set_fft_variant(lm_plan *p, int variant) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is NULL");
  if (variant < LM_FFT_AUTO || variant > LM_FFT_SPLIT_MFMA) return fail(LM_ERR_INVALID_ARG, "unknown FFT variant");
  p->fft_variant = variant;
  return LM_OK;
}

int lm_plan_set_memory_limit(lm_plan *p, int64_t bytes) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is null");
  if (bytes < 0) return fail(LM_ERR_INVALID_ARG, "memory limit must be >= 0 (0: none)");
  p->mem_limit = (size_t)bytes;
  return LM_OK;
}

int64_t lm_plan_memory_bytes(const lm_plan *p) { return p ? (int64_t)plan_device_bytes(p) : -1; }

int64_t lm_plan_describe(const lm_plan *p, char *buf, int64_t cap) {
  if (!p) return fail(LM_ERR_INVALID_ARG, "plan is null");
  if (cap < 0 || (cap > 0 && !buf)) return fail(LM_ERR_INVALID_ARG, "buffer is null or cap < 0");
  static const char *pads[] = {"constant", "reflect", "replicate", "circular"};
  static const char *outs[] = {"log-mel", "mel"};
  char line[512];
  std::string t;
  std::snprintf(line, sizeof line,
                "plan: n_fft %d, hop %d, n_mels %d, center %d, pad mode %s, power %g, out %s, window %d, "
                "signal pad %lld, output %s, normalized %d\n",
                p->n_fft, p->hop, p->n_mels, p->center,
                p->pad_mode >= 0 && p->pad_mode < 4 ? pads[p->pad_mode] : "?", (double)p->power,
                p->out_dtype == LM_F16 ? "f16" : "f32", p->win_length, (long long)p->sig_pad,
                p->output >= 0 && p->output < 2 ? outs[p->output] : "?", p->normalized);
  t += line;
  if (p->have_filters) {
    int empty = 0;
    for (int w : p->csr.width) empty += w == 0;
    std::snprintf(line, sizeof line, "filters: %d bands over %d bins, %zu weights, widest band %d bins, %d empty\n",
                  p->csr.n_rows, p->csr.n_bins, p->csr.w.size(), p->csr.max_width(), empty);
  } else {
    std::snprintf(line, sizeof line, "filters: not set (lm_from_pcm needs lm_plan_set_mel or _set_filters)\n");
  }
  t += line;
  if (p->have_filters) {
    const std::string k16 = pcm_kernel_summary(p, true), k32 = pcm_kernel_summary(p, false);
    t += "lm_from_pcm: " + k16 + "\n";
    if (k32 != k16) t += "lm_from_pcm (float input): " + k32 + "\n";
    t += "  then clamp_fixup_kernel (per-clip floor; reads only regions whose smallest value may lie below it)\n";
  }
  t += "lm_from_stft: filter_rows_kernel (row spans of the caller's filterbank), stft_logmel_kernel, "
       "clamp_fixup_kernel\n";
  std::snprintf(line, sizeof line, "options: fft variant %s, single pass %s\n",
                p->fft_variant == LM_FFT_FOLDED   ? "folded"
                : p->fft_variant == LM_FFT_PAIRED ? "paired"
                : p->fft_variant == LM_FFT_SPLIT_MFMA ? "split_mfma"
                                                      : "auto",
                p->single_pass ? (p->device < 0 ? "requested" : p->coop_launch ? "requested (cooperative launch)"
                                                                             : "requested (not available here)")
                               : "off");
  t += line;
  if (p->device < 0)
    std::snprintf(line, sizeof line, "device: not bound yet (bound at the first lm_from_* call)\n");
  else
    std::snprintf(line, sizeof line, "device: %d, %d compute units\n", p->device, p->n_cu);
  t += line;
  char lim[32] = "none";
  if (p->mem_limit) std::snprintf(lim, sizeof lim, "%zu bytes", p->mem_limit);
  std::snprintf(line, sizeof line, "device memory: %zu bytes held (tables %zu, statistics %zu, filter pack %zu, "
                "single-pass slots %zu), limit %s\n",
                plan_device_bytes(p), p->dt.bytes, p->stats_cap * sizeof(float), p->pack_cap, p->sync_cap, lim);
  t += line;
  if (cap > 0) {
    const size_t n = std::min(t.size(), (size_t)(cap - 1));
    std::memcpy(buf, t.data(), n);
    buf[n] = 0;
  }
  return (int64_t)t.size();
}

}  // extern "C"
