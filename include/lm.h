/*
 * lm.h -- C ABI of the MI355X log-mel front end.
 *
 * The library turns raw PCM (float32 or int16) or a given complex64 STFT
 * into the normalised log-mel spectrogram used by speech encoders:
 *
 *   frames (center padding by index arithmetic) -> periodic Hann window
 *   -> one-sided real FFT -> |X|^power -> triangular mel projection
 *   -> log10(max(mel, 1e-10)) -> max(., clip max - 8) -> (. + 4) / 4
 *
 * Definitions follow two pages:
 *  - KBench task page "audio-mel-spectrogram-fused": the STFT -> log-mel
 *    chain (section "spec_md"), its tensor contract ("contract_md") and its
 *    float32-everywhere precision rule ("precision_md").
 *  - flashmel project page (PyPI): the PCM front half and its arguments
 *    (sections "Usage" and "How it works").
 *
 * Conventions for every entry point
 *  - Return value: LM_OK (0) or a negative lm_status code.  No call aborts
 *    the process.  lm_last_error() gives a thread-local message for the
 *    most recent failure on the calling thread.
 *  - Device pointers are plain HIP device addresses on the device that is
 *    current when the call is made (normally torch tensors' data_ptr()).
 *    The caller owns them.  Inputs are only read; outputs must not alias
 *    inputs.  Arrays are dense and row-major (C order).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    The lm_from_* calls only enqueue work on it and never wait for the
 *    device: the plan's tables go up with an asynchronous copy from
 *    plan-owned pinned host memory, and device tables and workspace are
 *    allocated, grown (by doubling) and retired in stream order
 *    (hipMallocAsync / hipFreeAsync on the call's stream).
 *  - A plan binds to the device current at its first lm_from_* call and
 *    must only be used on that device.  It may be used from several
 *    streams: a call on a stream other than the previous call's records an
 *    event on the previous call's stream and makes its own stream wait for
 *    it, so the GPU work of one plan always runs in call order and its
 *    shared workspace is never used by two calls at once (calls on one
 *    stream add no event).  A stream a plan was last used on must therefore
 *    stay valid until the plan's next call on another stream or its
 *    destruction.  Host calls on one plan must not run concurrently on
 *    several threads.  Do not change or destroy a plan while work that uses
 *    it is in flight.
 */
#ifndef LM_H
#define LM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lm_plan lm_plan;   /* opaque, owned by the library */

/* Status codes. */
enum {
  LM_OK = 0,
  LM_ERR_INVALID_ARG = -1,  /* a value outside what the call accepts     */
  LM_ERR_UNSUPPORTED = -2,  /* valid in principle, not built (e.g. size) */
  LM_ERR_NO_FILTERS = -3,   /* the plan has no filterbank yet            */
  LM_ERR_HIP = -4,          /* a HIP runtime call or launch failed       */
  LM_ERR_OOM = -5           /* device or host allocation failed          */
};

/* Padding modes for center=1 (flashmel page, "How it works": all four
 * modes are index arithmetic on the unpadded signal).
 *  CONSTANT  zeros outside the signal
 *  REFLECT   mirror about the edge sample, edge not repeated
 *  REPLICATE repeat the edge sample
 *  CIRCULAR  wrap around                                             */
enum { LM_PAD_CONSTANT = 0, LM_PAD_REFLECT = 1, LM_PAD_REPLICATE = 2, LM_PAD_CIRCULAR = 3 };

/* Element types.  LM_I16 is raw PCM scaled by 1/32768 (flashmel page,
 * "Usage").  Outputs are LM_F32 or LM_F16 (cast at the final store).  */
enum { LM_F32 = 0, LM_F16 = 1, LM_I16 = 2 };

/* Mel scale and filter normalisation for lm_plan_set_mel. */
enum { LM_MEL_SLANEY = 0, LM_MEL_HTK = 1 };
enum { LM_NORM_SLANEY = 0, LM_NORM_NONE = 1 };

/*
 * lm_plan_create -- validate the transform's shape and build a plan.
 *
 *  n_fft     FFT size: 400, or a power of two in [64, 16384] (flashmel
 *            page, "Usage", constraints).
 *  hop       frame step in samples, >= 1.
 *  n_mels    number of mel bands, 1..256.
 *  center    1: pad n_fft/2 samples on both sides with `pad_mode`;
 *            0: no padding (frames start at sample 0).
 *  pad_mode  one of LM_PAD_*.
 *  power     exponent p of |X|^p, finite and > 0 (2 = power spectrum).
 *  out_dtype LM_F32 or LM_F16.
 *
 * Host-only: makes no HIP call.  *plan receives a new plan on LM_OK and is
 * left untouched otherwise.  The plan has no filterbank until
 * lm_plan_set_mel or lm_plan_set_filters succeeds.
 */
int lm_plan_create(lm_plan **plan, int n_fft, int hop, int n_mels, int center, int pad_mode,
                   float power, int out_dtype);

/*
 * lm_plan_set_mel -- build the plan's triangular mel filterbank.
 *
 * n_mels + 2 corner frequencies evenly spaced in mel between f_min and
 * f_max (Slaney: linear below 1 kHz, logarithmic above; HTK:
 * 2595 log10(1 + f/700)); bin k sits at k * sample_rate / n_fft; row m is
 * the triangle on corners m, m+1, m+2; LM_NORM_SLANEY scales each row to
 * unit area (2 / (f[m+2] - f[m])).  Computed in float64 on the host and
 * rounded once to float32.  Requires 0 <= f_min < f_max <= sample_rate/2.
 * Host-only; the device copy is refreshed at the next lm_from_* call.
 */
int lm_plan_set_mel(lm_plan *plan, double sample_rate, double f_min, double f_max, int mel_scale,
                    int norm);

/*
 * lm_plan_set_filters -- use a caller-supplied dense filterbank.
 *
 * host_dense: host array (n_mels, n_bins) float32, row-major, with
 * n_mels == the plan's n_mels and n_bins == n_fft/2 + 1.  Copied; each row
 * is packed to its [first, last] non-zero range (interior zeros kept, so
 * the sparse sum is exact for any input).  Host-only.
 */
int lm_plan_set_filters(lm_plan *plan, const float *host_dense, int n_mels, int n_bins);

/*
 * lm_plan_get_filters -- copy the plan's filterbank (as used, float32) into
 * host_dense (n_mels, n_bins), zero outside each row's packed range.
 */
int lm_plan_get_filters(const lm_plan *plan, float *host_dense, int n_mels, int n_bins);

/* Output of a plan (lm_plan_set_output). */
enum { LM_OUTPUT_LOGMEL = 0, LM_OUTPUT_MEL = 1 };
/* Spectrum normalisation of the PCM path (lm_plan_set_output). */
enum { LM_NORMALIZED_NONE = 0, LM_NORMALIZED_WINDOW = 1, LM_NORMALIZED_FRAME_LENGTH = 2 };

/*
 * lm_plan_set_output -- what the lm_from_* calls write (flashmel page,
 * "Usage": a torchaudio-compatible MelSpectrogram, whose output is the mel
 * power itself; KBench page, "spec_md": the log / clamp / rescale tail).
 *
 *  output      LM_OUTPUT_LOGMEL (the default): the normalised log-mel,
 *              (max(L, hi_b - 8) + 4) / 4 with L = log10(max(mel, 1e-10)).
 *              LM_OUTPUT_MEL: the mel values themselves, sum_k W[m,k] |X_k|^p,
 *              with no floor, log, clamp or rescale (torchaudio's
 *              MelSpectrogram); an LM_F16 plan rounds them to fp16, so
 *              values beyond 65504 become infinite.
 *  normalized  LM_NORMALIZED_NONE (the default); LM_NORMALIZED_WINDOW:
 *              X divided by sqrt(sum_n w[n]^2) before |X|^p (torchaudio's
 *              normalized=True / "window"); LM_NORMALIZED_FRAME_LENGTH: X
 *              divided by sqrt(win_length) ("frame_length").  Applies to
 *              lm_from_pcm only (lm_from_stft takes a finished spectrum).
 * Host-only.  LM_ERR_INVALID_ARG for an unknown value.
 */
int lm_plan_set_output(lm_plan *plan, int output, int normalized);

/*
 * lm_plan_set_window -- window length of the PCM path (flashmel page,
 * "Usage": torchaudio's win_length).  The periodic Hann window of
 * win_length samples, 0.5 - 0.5 cos(2 pi n / win_length), is placed in the
 * n_fft-point frame starting at (n_fft - win_length) / 2 (integer
 * division) with zeros around it, as torch.stft pads a shorter window
 * (win_length 1 gives the window [1], torch's convention).
 * 1 <= win_length <= n_fft; the default is n_fft.  Host-only.
 */
int lm_plan_set_window(lm_plan *plan, int win_length);

/*
 * lm_plan_set_pad -- two-sided zero padding of the PCM signal (flashmel
 * page, "Usage": torchaudio's pad argument; "How it works": every padding
 * applied by index arithmetic).  Each clip of n_samples is read as `pad`
 * zeros, the clip, `pad` zeros (n_samples + 2 pad samples), and the center
 * padding of the plan (center=1, pad_mode) then applies to that longer
 * signal: reflect and circular see the zeros like any other sample.
 * Nothing padded is stored.  0 <= pad <= 2^30; the default is 0.  A pad
 * that is not a multiple of 16 bytes of samples (8 int16 or 4 float32
 * samples) keeps results identical but takes the slower per-sample load
 * path.  Host-only.  LM_ERR_INVALID_ARG out of range.
 */
int lm_plan_set_pad(lm_plan *plan, int64_t pad);

/*
 * lm_plan_num_frames -- frames produced for a clip of n_samples:
 * 1 + floor((n_samples + 2*sig_pad + 2*pad - n_fft) / hop), with sig_pad
 * the plan's signal padding (lm_plan_set_pad) and pad = n_fft/2 if center
 * else 0.  Returns a negative lm_status if no frame fits.
 */
int64_t lm_plan_num_frames(const lm_plan *plan, int64_t n_samples);

/*
 * lm_from_pcm -- PCM clips -> log-mel (flashmel page, "Usage": input
 * (..., time) -> output (..., n_mels, n_frames); then the log / per-clip
 * clamp / rescale tail of the KBench page's "spec_md").
 *
 *  pcm       device array (n_clips, n_samples) of LM_F32 or LM_I16, 4- or
 *            2-byte aligned.
 *  in_dtype  LM_F32 or LM_I16.
 *  out       device array (n_clips, n_mels, F) of the plan's out_dtype,
 *            F = lm_plan_num_frames(plan, n_samples).  Mel-major: each
 *            band's F frames are contiguous.
 *  Each clip is floored at its own maximum: out = (max(L, hi_b - 8) + 4)/4
 *  with L = log10(max(mel, 1e-10)) and hi_b the clip's largest L (or the
 *  mel values themselves under LM_OUTPUT_MEL, see lm_plan_set_output).
 *
 * With t = n_samples + 2 sig_pad (lm_plan_set_pad), needs t > n_fft/2 for
 * reflect, t >= n_fft/2 for circular and t >= n_fft for center=0.
 * n_clips == 0 is a no-op.  Returns
 * LM_ERR_NO_FILTERS before any filterbank is set.
 */
int lm_from_pcm(lm_plan *plan, const void *pcm, int in_dtype, int64_t n_clips, int64_t n_samples,
                void *out, void *stream);

/*
 * lm_from_stft -- complex STFT -> log-mel (KBench page, "reference_src",
 * "spec_md" and "contract_md").
 *
 *  stft        device array (n_clips, n_frames, n_bins) complex64, real and
 *              imaginary parts interleaved, 8-byte aligned.
 *  mel_filters device array (n_mels, n_bins) float32, row-major; or NULL
 *              to use the plan's own filterbank (then n_bins must be
 *              n_fft/2 + 1 and n_mels the plan's n_mels).  A device
 *              filterbank is packed on the device on every call (rows to
 *              their [first, last] non-zero range; exact for any input).
 *  out         device array (n_clips, n_frames, n_mels) of the plan's
 *              out_dtype.  Frame-major, as the contract fixes.
 *  power = re^2 + im^2 always (the plan's `power`, window, normalisation,
 *  framing and padding do not apply to this path); the plan's output mode
 *  does (LM_OUTPUT_MEL writes the mel values without the log tail).  1 <= n_bins <= 8193, 1 <= n_mels <= 256.
 *  n_clips == 0 or n_frames == 0 is a no-op.
 */
int lm_from_stft(lm_plan *plan, const void *stft, const float *mel_filters, int64_t n_clips,
                 int64_t n_frames, int64_t n_bins, int n_mels, void *out, void *stream);

/*
 * lm_plan_profile -- per-kernel timing for measurement.
 *
 * enable != 0 makes later lm_from_* calls bracket each kernel they launch
 * with HIP events on the same stream; enable == 0 stops it.
 * lm_plan_profile_read waits for the recorded events, writes the summed
 * milliseconds and launch counts of the main kernel (index 0: the
 * PCM or STFT kernel), the clamp fix-up kernel (1) and the filter-packing
 * kernel (2) into ms[3] / counts[3], and clears the record.
 */
int lm_plan_profile(lm_plan *plan, int enable);
int lm_plan_profile_read(lm_plan *plan, double *ms, int64_t *counts);

/*
 * lm_from_pcm_noalloc -- lm_from_pcm for callers that cannot allocate
 * device memory during a call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, kernels and
 * results as lm_from_pcm; no device or host memory is allocated or freed.
 *
 *  - The workspace is a fixed 8 MiB device array, one per GPU, held until
 *    the process ends: 2^21 - 16384 floats of statistics (per-region output
 *    minima and per-tile mel maxima that the clamp fix-up reads) and 8192
 *    64-bit slots of the single pass (see lm_plan_set_single_pass).  A call
 *    needing more returns LM_ERR_UNSUPPORTED before any launch (a 30 s clip
 *    at n_fft 400 / 128 mels needs 6768 floats: about 300 such clips per
 *    call).  Every statistic a call reads is written by that call, and the
 *    slots carry a per-call tag, so nothing needs clearing between calls.
 *  - Every call on one GPU shares that array: calls that overlap in time on
 *    one GPU (other streams, other plans, other threads) race on it.
 *    Calls on one stream, or otherwise ordered, are safe.
 *  - The plan's device tables must already exist: make one lm_from_pcm call
 *    with the plan after its last set_mel / set_filters / set_window;
 *    otherwise LM_ERR_INVALID_ARG.  Profiling (lm_plan_profile) is ignored.
 */
int lm_from_pcm_noalloc(lm_plan *plan, const void *pcm, int in_dtype, int64_t n_clips, int64_t n_samples,
                        void *out, void *stream);

/*
 * lm_plan_set_single_pass -- use (enable = 1) or not (0, the default) the
 * single-pass form of the per-clip floor (KBench page, "perf_md": the
 * clip-resident alternative to a second pass over the output).
 *
 * Where it applies, lm_from_pcm runs one cooperative launch instead of the
 * main kernel plus the clamp fix-up: each wave stores its log-mel values,
 * publishes its largest mel value on its clip's slot, and all workgroups
 * meet at a grid barrier (every wait bounded; a wait that runs out writes
 * NaN); a wave holding a value below its clip's floor then recomputes its
 * mel sums from the power rows still in its LDS and overwrites them
 * floored.  It applies at n_fft = 400 (the matrix-core kernel) with log-mel
 * output and at most one 16-frame sub-tile per resident wave (8 per
 * compute unit): the launch-bound batches.  Results are bit-identical to
 * the two-pass form.  It is off by default because it is slower on MI355X:
 * the cooperative launch alone costs more than the fix-up launch it saves.
 * Host-only.  LM_ERR_INVALID_ARG unless enable is 0 or 1.
 */
int lm_plan_set_single_pass(lm_plan *plan, int enable);

/* FFT variants of the n_fft = 400 PCM path (lm_plan_set_fft_variant). */
enum { LM_FFT_AUTO = 0, LM_FFT_FOLDED = 1, LM_FFT_PAIRED = 2, LM_FFT_SPLIT_MFMA = 3 };

/*
 * lm_plan_set_fft_variant -- which transform the n_fft = 400 PCM path runs,
 * for measurement and comparison only (flashmel page, "Performance": the
 * normal, folded and paired real-input transforms it compared).
 *
 *  LM_FFT_AUTO    (the default) the 16 x 25 split with its 16-point stage on
 *                 the matrix cores and its 25-point DFTs in registers
 *                 wherever it applies (even hop), else the folded form.
 *  LM_FFT_SPLIT_MFMA  the 16 x 25 split with the 25-point stage on the
 *                 matrix cores as well (two-part fp16 operands, three
 *                 products), where the blocked filterbank leaves room for
 *                 that stage's operands (up to 1920 blocked weights: 128
 *                 Slaney bands over 0-8 kHz take 1280); else as AUTO.
 *  LM_FFT_FOLDED  each frame as a 200-point complex sequence (radix 8, 5, 5),
 *                 then split into the real spectrum.
 *  LM_FFT_PAIRED  two frames as one 400-point complex sequence, separated by
 *                 conjugate symmetry.
 * Results agree within the same tolerance on every variant.  Other n_fft
 * ignore the setting.  Host-only.  LM_ERR_INVALID_ARG for an unknown value.
 */
int lm_plan_set_fft_variant(lm_plan *plan, int variant);

/*
 * lm_plan_set_memory_limit -- cap on the device memory the plan holds (its
 * tables, statistics workspace, filter pack and single-pass slots), for
 * callers that budget memory on a shared GPU.  0 (the default) is no
 * limit.  A call that would need more returns LM_ERR_OOM before it
 * allocates or launches anything, leaving the output untouched and the plan
 * usable; a buffer grows to the size the call needs rather than by doubling
 * when doubling would pass the cap.  A cap below what the plan already holds
 * frees nothing.  Host-only.  LM_ERR_INVALID_ARG if bytes < 0.
 */
int lm_plan_set_memory_limit(lm_plan *plan, int64_t bytes);

/* Device bytes the plan holds now (-1 for a NULL plan).  Host-only. */
int64_t lm_plan_memory_bytes(const lm_plan *plan);

/*
 * lm_plan_describe -- the plan's choices as text, for logs: its shape and
 * options, the filterbank it holds, the kernels lm_from_pcm and lm_from_stft
 * launch for it (n_fft = 400 matrix-core kernel, generic tile kernel or
 * one-frame kernel, with their tile sizes), the device it is bound to and
 * the device memory it holds.  Writes at most cap - 1 bytes and a NUL to
 * buf (nothing if cap is 0) and returns the full length, so a call with
 * cap = 0 sizes the buffer.  Host-only.  LM_ERR_INVALID_ARG (negative) for
 * a NULL plan, or a NULL buf with cap > 0.
 */
int64_t lm_plan_describe(const lm_plan *plan, char *buf, int64_t cap);

/* lm_plan_destroy -- free the plan and its device memory (NULL is a no-op). */
void lm_plan_destroy(lm_plan *plan);

/* Static text for a status code. */
const char *lm_status_string(int status);

/* Thread-local text describing the last failure on this thread ("" if none). */
const char *lm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LM_H */
