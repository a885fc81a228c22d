// Internal declarations shared by the host plan, the entry points and the
// kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "lm.h"

namespace lm {

// Optional timing of one kernel launch: events stamped by the dispatch
// itself at the kernel's start and end (hipExtLaunchKernelGGL), so a
// profiled duration excludes the launch gap before the kernel.
struct LaunchTiming {
  hipEvent_t beg, end;
};
#define LM_LAUNCH(tm, K, grid, block, shmem, s, ...)                                           \
  do {                                                                                         \
    if (tm) hipExtLaunchKernelGGL(K, grid, block, shmem, s, (tm)->beg, (tm)->end, 0u, __VA_ARGS__); \
    else hipLaunchKernelGGL(K, grid, block, shmem, s, __VA_ARGS__);                            \
  } while (0)

// Power row stride (floats) of the n_fft = 400 kernel: bins 0..200 plus
// zeroed padding that chunked mel reads may touch; odd, so that the rows
// of 16 frames read or written by one instruction fall on distinct LDS
// banks (even strides were measured to serialise LDS accesses).
constexpr int kPcm400Row = 213;
// Chunks of 4 bins the n_fft = 400 mel loop takes per step; every band
// block's chunk count is a multiple of it.
constexpr int kMelBatch = 4;
// Accelerator complex dies (XCDs) of the chip, each with its own L2;
// consecutive workgroup ids are handed to them in turn.
constexpr int kXcds = 8;
// Threads of the one-frame kernel's workgroup (n_fft 8192 and 16384; also
// the number of entries of its mel lane table).
constexpr int big_threads(int n_fft) { return n_fft == 8192 ? 512 : 1024; }

// Set the thread-local error text and return `status`.
int fail(int status, const std::string &msg);
int hip_fail(hipError_t err, const char *what);

// Packed triangular filterbank: row m covers bins [start[m], start[m] +
// width[m]) with weights w[off[m] + j].  Rows are contiguous in w.
struct Csr {
  std::vector<int32_t> start, width, off;
  std::vector<float> w;
  int n_rows = 0, n_bins = 0;
  int max_width() const;
};

// Device copy of the tables one PCM launch reads.  One allocation:
//   [window n_fft f32][fft twiddles M f32x2][untangle twiddles M/2+1 f32x2]
//   [csr start n_mels i32][csr width n_mels i32][csr off n_mels i32][csr w nnz f32]
//   [n_fft = 400 matrix-core operands][blocked filterbank][two-level twiddles]
struct DeviceTables {
  void *base = nullptr;
  size_t bytes = 0;
  const float *window = nullptr;
  const float2 *twiddle = nullptr;    // exp(-2 pi i j / M), j < M
  const float2 *untangle = nullptr;   // exp(-2 pi i k / n_fft), k <= M/2
  const float2 *tw2 = nullptr;        // n_fft >= 8192: two-level exp(-2 pi i j / n_fft) table
  const int32_t *csr_start = nullptr, *csr_width = nullptr, *csr_off = nullptr;
  const float *csr_w = nullptr;
  int nnz = 0;
  const uint16_t *mfma400h = nullptr;
  const uint16_t *mfma400t = nullptr;   // n_fft = 400: second-stage (25-point DFT) operands
  const int32_t *melblk_meta = nullptr;
  const float *melblk_w = nullptr;
  int n_melblk = 0;
  const int32_t *empty_bands = nullptr;   // bands with no non-zero weight, ascending
  int n_empty = 0;
  const int32_t *mel_lanes = nullptr;     // n_fft >= 8192: big_threads(n_fft) entries (build_mel_lanes)
};

struct ProfileRec {
  hipEvent_t beg, end;
  int kind;
};

// Pinned host buffer a table upload copies from; `done` is recorded after
// the copy, so the buffer is reused only once that copy has finished.
struct Staging {
  void *host = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
};

}  // namespace lm

struct lm_plan {
  int n_fft = 0, hop = 0, n_mels = 0, center = 0, pad_mode = 0, out_dtype = 0;
  float power = 2.0f;
  int n_bins = 0;  // n_fft / 2 + 1
  int win_length = 0;                   // periodic Hann length, centred in the frame (default n_fft)
  int64_t sig_pad = 0;                  // zeros read before and after each PCM clip (torchaudio's pad)
  int output = LM_OUTPUT_LOGMEL;        // LM_OUTPUT_*
  int normalized = LM_NORMALIZED_NONE;  // LM_NORMALIZED_*

  bool have_filters = false;
  lm::Csr csr;
  std::vector<float> window;      // n_fft
  std::vector<float> twiddle;     // 2 * M
  std::vector<float> untangle;    // 2 * (M/2 + 1)
  std::vector<float> twid2;       // n_fft >= 8192: 2 * (n_fft / 128 + 128), see build_twiddles
  std::vector<uint16_t> mfma400h;  // n_fft = 400 only: first-stage matrix as fp16 hi/lo parts (25 x 2 x 2 x 16 x 8)
  std::vector<uint16_t> mfma400t;  // n_fft = 400 only: 25-point DFT as fp16 hi/lo operands (4 x 5 x 64 x 8)
  bool mfma400t_fits = false;      // the window keeps every first-stage value in the second stage's fp16 range
  std::vector<int32_t> melblk_meta;  // per batch of mel steps: first bin of each quad, last-batch flag
  std::vector<float> melblk_w;       // blocked filter weights in matrix-core lane order
  std::vector<int32_t> mel_lanes;    // n_fft >= 8192: mel lane table of the one-frame kernel (build_mel_lanes)

  int device = -1;                // bound at first launch
  int n_cu = 0;                   // compute units of that device
  bool tables_dirty = true;
  lm::DeviceTables dt;

  // workspace: per-region smallest and per-tile largest mel value
  float *d_stats = nullptr;       // [minima][maxima], laid out per call
  size_t stats_cap = 0;           // floats
  // per-call packed copy of a device filterbank (STFT path)
  void *d_pack = nullptr;
  size_t pack_cap = 0;
  // pinned host buffers of the table uploads
  std::vector<lm::Staging> staging;
  // a call on a stream other than the last call's records this event on the
  // last call's stream and waits for it
  hipEvent_t done_event = nullptr;
  void *last_stream = nullptr;
  bool has_last = false;

  size_t mem_limit = 0;            // lm_plan_set_memory_limit (0: none)
  int fft_variant = LM_FFT_AUTO;   // lm_plan_set_fft_variant (n_fft = 400 only)
  int single_pass = 0;             // lm_plan_set_single_pass
  bool coop_launch = false;        // the device supports cooperative launches
  // single-pass slots: [0], [1] grid barrier counters (calls alternate
  // between them), [2 + b] clip b's maximum as (epoch << 32) | value;
  // zeroed when allocated
  uint64_t *d_sync = nullptr;
  size_t sync_cap = 0;             // bytes
  uint32_t sync_calls = 0;         // single-pass calls made on d_sync (barrier parity)

  bool profiling = false;
  std::vector<lm::ProfileRec> prof;
};

namespace lm {

// Workspace helpers (lm_api.cpp).  Allocation, upload and release are
// stream-ordered on `s`, the stream of the call that needs them.
int ensure_device(lm_plan *p);
int ensure_workspace(lm_plan *p, int64_t n_floats, hipStream_t s);
int upload_tables(lm_plan *p, hipStream_t s);
// Device bytes the plan holds (tables and workspace).
size_t plan_device_bytes(const lm_plan *p);
// Start and end of an lm_from_* call's GPU work on stream s: order it after
// the plan's previous call (an event, only when the stream changes), then
// note the stream.
int begin_call(lm_plan *p, hipStream_t s);
int end_call(lm_plan *p, hipStream_t s, int rc);

// Host table builders (lm_plan.cpp)
double window_at(const lm_plan *p, int n);   // the frame window at n (float64)
double power_scale2(const lm_plan *p);       // factor on |X|^2 from the plan's normalisation
void build_window(lm_plan *p);
void build_twiddles(lm_plan *p);
void build_mfma400(lm_plan *p);
void build_mel_blocks(lm_plan *p);
void build_mel_lanes(lm_plan *p, int threads);
Csr pack_dense(const float *dense, int n_rows, int n_bins);

// Kernel launchers.  Each returns hipSuccess or the launch error.
// Geometry of a main kernel's statistics for the clamp fix-up.  A tile is
// frames_per_tile consecutive frames of one clip.  Per tile there are
// sub_per_tile x blk_per_sub minimum entries: entry (sub, blk) holds the
// smallest mel value (after the 1e-10 floor, as float32) over frames [sub * frames_per_tile / sub_per_tile, +frames_per_tile /
// sub_per_tile) of the tile and bands [blk * band_h, (blk + 1) * band_h)
// (both clipped to the output), or +inf if that region is empty; and max_per_tile maximum entries whose largest value is the
// tile's largest mel value (after the 1e-10 floor).  Entries are stored
// clip-major, tile-major.
struct StatLayout {
  int frames_per_tile = 1, sub_per_tile = 1, blk_per_sub = 1, band_h = 1, max_per_tile = 1;
  __host__ __device__ int min_per_tile() const { return sub_per_tile * blk_per_sub; }
};

// Geometry of one lm_from_pcm call, from validate_pcm.
struct PcmCall {
  int64_t F = 0;
  int tiles = 0;
  StatLayout st;
  int64_t ws_floats = 0;   // statistics workspace the call needs
};
// Host-side checks of an lm_from_pcm call (no HIP call), filling c; LM_OK
// with nothing to do for n_clips == 0.
int validate_pcm(const lm_plan *p, const void *pcm, int in_dtype, int64_t n_clips, int64_t n_samples,
                 const void *out, PcmCall *c);
// The PCM launch sequence (main kernel, clamp fix-up) with its statistics
// workspace at ws; allow_profile false creates no timing events.
// A non-null sync (2 + n_clips single-pass slots) runs the call as one pass
// of the main kernel (pcm400_single_pass must hold) with barrier counter
// `parity`; ws is then unused.
int run_pcm(lm_plan *p, const void *pcm, bool in_i16, int64_t n_clips, int64_t n_samples, int64_t F, int tiles,
            const StatLayout &st, void *out, float *ws, uint64_t *sync, int parity, hipStream_t s,
            bool allow_profile);

struct PcmArgs {
  const void *pcm;
  bool in_i16;
  int64_t n_clips, n_samples, n_frames;
  int tiles_per_clip;
  void *out;
  float *tile_min;
  float *tile_max;
  // single pass (no fix-up launch): 2 + n_clips slots (two barrier
  // counters, then the clip maxima), this call's epoch and barrier parity;
  // nullptr for two passes
  uint64_t *sync = nullptr;
  uint32_t epoch = 0;
  int parity = 0;
};
// Statistics geometry of the PCM kernel launch_pcm picks for this plan and
// input type (the n_fft = 400 matrix-core kernel when it applies, else the
// generic one).
StatLayout pcm_stat_layout(const lm_plan *p, bool in_i16);
hipError_t launch_pcm(const lm_plan *p, const PcmArgs &a, hipStream_t s, const LaunchTiming *tm);
// True when launch_pcm leaves the plan's empty bands unwritten (the generic
// kernel, log-mel output, at least one empty band): the fix-up writes them.
bool pcm_skips_empty_bands(const lm_plan *p, bool in_i16);
// One line on the PCM kernel launch_pcm picks for this plan (lm_plan_describe).
std::string pcm_kernel_summary(const lm_plan *p, bool in_i16);
std::string pcm400_summary(const lm_plan *p);
bool pcm400_supported(const lm_plan *p, bool in_i16);
// True when a call of n_sub 16-frame sub-tiles runs as one pass of the
// n_fft = 400 kernel (every wave holds at most one sub-tile and keeps its
// outputs until the clip's maximum is known; cooperative launch).
bool pcm400_single_pass(const lm_plan *p, bool in_i16, int64_t n_sub);
// Next tag of a single-pass call (process-wide, never 0).
uint32_t next_epoch();
StatLayout pcm400_stat_layout(const lm_plan *p);
hipError_t launch_pcm400(const lm_plan *p, const PcmArgs &a, hipStream_t s, const LaunchTiming *tm);

struct StftArgs {
  const float2 *stft;
  int64_t n_clips, n_frames;
  int n_bins, n_mels;
  int frames_per_tile, tiles_per_clip;
  // band m covers bins [f_start[m], f_start[m] + f_width[m]); its weights are
  // at f_w + m * f_stride + f_start[m] (f_stride > 0: rows of a dense
  // matrix) or at f_w + f_off[m] (f_stride == 0: rows packed back to back)
  const int32_t *f_start, *f_width, *f_off;
  const float *f_w;
  int f_stride;
  void *out;
  int out_f16;
  float *tile_min;
  float *tile_max;
  int n_cu;
  int mel_out;   // 1: mel values without the log tail
};
int stft_frames_per_tile(int n_bins, int n_mels, int64_t total_frames, int n_cu);
hipError_t launch_stft(const StftArgs &a, hipStream_t s, const LaunchTiming *tm);

// First non-zero bin and width of every row of a device dense (n_mels,
// n_bins) filterbank into start_width[0, n_mels) and [n_mels, 2 n_mels).
hipError_t launch_pack(const float *dense, int n_mels, int n_bins, int32_t *start_width, hipStream_t s,
                       const LaunchTiming *tm);

struct FixupArgs {
  void *out;
  int out_f16;
  const float *tile_min;
  const float *tile_max;
  int64_t n_clips, n_frames;
  int n_mels;
  int tiles_per_clip;
  StatLayout st;
  int mel_major;  // 1: (B, NM, F); 0: (B, F, NM)
  // mel-major only: bands the main kernel left unwritten (no non-zero
  // weight, so their log value is log10(1e-10) in every frame); the fix-up
  // writes their floored value without reading them
  const int32_t *empty_bands = nullptr;
  int n_empty = 0;
  int entries_per_group = 0, groups_per_clip = 0;   // set by launch_fixup
  int empty_units = 0;                              // set by launch_fixup: units per empty band row
  unsigned inner_magic = 0, reg_magic = 0;          // set by launch_fixup: divide by a run / a region length
};
hipError_t launch_fixup(FixupArgs a, hipStream_t s, const LaunchTiming *tm);
// Zero n 64-bit words (a fill kernel, not a memset node, so that a captured
// graph replays it correctly).
hipError_t launch_zero_u64(uint64_t *p, size_t n, hipStream_t s);

}  // namespace lm
