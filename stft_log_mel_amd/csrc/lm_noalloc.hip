// lm_from_pcm_noalloc: lm_from_pcm for callers that cannot allocate device
// memory during the call (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The kernels are the same; the
// statistics workspace they fill (per-region output minima and per-tile mel
// maxima, read back by the clamp fix-up) lives in a fixed file-scope device
// array instead of plan-owned memory.
#include <atomic>
#include <mutex>

#include "lm_internal.h"

namespace lm {

namespace {

// 2^21 floats = 8 MiB: a 30 s clip at n_fft 400 / 128 mels needs 188
// sub-tiles x (32 minima + 4 maxima) = 6768 floats, so about 300 such clips
// per call.  Each GPU the library runs on holds one copy until the process
// ends.
constexpr size_t kScratchFloats = (size_t)1 << 21;
__device__ __align__(256) float scratch[kScratchFloats];
// The last 64 KiB hold the single-pass slots (8192 64-bit words: two grid
// barrier counters, which the device's calls use in turn, each zeroing the
// other, and clip maxima tagged by call; the array starts zeroed); the
// statistics use the rest.
constexpr size_t kSyncWords = 8192;
constexpr size_t kStatFloats = kScratchFloats - 2 * kSyncWords;

// The array's device address on each device, from hipGetSymbolAddress with
// that device current (the array's name is only a host-side stand-in).
constexpr int kMaxDevices = 64;
float *g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
// single-pass calls made on each device's array (the barrier counter parity)
std::atomic<uint32_t> g_sync_calls[kMaxDevices];

int scratch_on(int dev, float **out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(LM_ERR_UNSUPPORTED, "device index beyond the supported range");
  std::call_once(g_scratch_once[dev], [dev] {
    void *ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = static_cast<float *>(ptr);
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  if (!g_scratch[dev]) return fail(LM_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
  *out = g_scratch[dev];
  return LM_OK;
}

}  // namespace

}  // namespace lm

using namespace lm;

extern "C" int lm_from_pcm_noalloc(lm_plan *p, const void *pcm, int in_dtype, int64_t n_clips, int64_t n_samples,
                                   void *out, void *stream) {
  PcmCall c;
  int rc = validate_pcm(p, pcm, in_dtype, n_clips, n_samples, out, &c);
  if (rc != LM_OK || n_clips == 0) return rc;
  if ((size_t)c.ws_floats > kStatFloats)
    return fail(LM_ERR_UNSUPPORTED, "call too large for the fixed workspace of lm_from_pcm_noalloc (" +
                                        std::to_string(c.ws_floats) + " floats needed, " +
                                        std::to_string(kStatFloats) + " available): split the batch");
  // the plan's device tables and its call-order event must already exist:
  // creating either would allocate
  if (p->device < 0 || p->tables_dirty || !p->dt.base || !p->done_event)
    return fail(LM_ERR_INVALID_ARG, "the plan's tables are not on the device: make one lm_from_pcm call with it "
                                    "(after its last filterbank or window change) before lm_from_pcm_noalloc");
  rc = ensure_device(p);
  if (rc != LM_OK) return rc;
  float *ws = nullptr;
  rc = scratch_on(p->device, &ws);
  if (rc != LM_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  rc = begin_call(p, s);
  if (rc != LM_OK) return rc;
  const bool one_pass = pcm400_single_pass(p, in_dtype == LM_I16, n_clips * c.tiles);
  uint64_t *sync = reinterpret_cast<uint64_t *>(ws + kStatFloats);
  if (one_pass && 2 + n_clips > (int64_t)kSyncWords) return end_call(p, s, fail(LM_ERR_UNSUPPORTED, "too many clips"));
  const int parity = one_pass ? (int)(g_sync_calls[p->device]++ & 1) : 0;
  rc = run_pcm(p, pcm, in_dtype == LM_I16, n_clips, n_samples, c.F, c.tiles, c.st, out, one_pass ? nullptr : ws,
               one_pass ? sync : nullptr, parity, s, false);
  return end_call(p, s, rc);
}
