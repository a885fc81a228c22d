"""fp64 CPU oracle for the log-mel front end.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or
calls this module; only the test suite, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code, table or constant generator with
the HIP library.

Every function is the plain definition of its step, in float64, with no
blocking or fusion beyond what the definition states.  Sources:

* KBench task page "audio-mel-spectrogram-fused" (sections "reference_src"
  and "spec_md"): power spectrum, mel projection, log10 after a 1e-10 floor,
  a floor at the clip's maximum minus 8, and the (x + 4) / 4 rescale.
* flashmel project page (PyPI), sections "Usage" and "How it works": the
  PCM front half -- int16 scaled by 1/32768, (..., time) -> (..., n_mels,
  n_frames), padding (center and the four pad modes) applied to the signal,
  the periodic Hann window, the one-sided real-to-complex transform,
  |X|^power and a triangular mel filterbank.

Readings where the pages leave a step open (each also listed in the design
notes): the PCM path ends in the same log/clamp/rescale tail as the STFT
path; the mel filterbank is the Slaney scale with Slaney area normalisation
unless another scale/norm is asked for; f_min = 0 and f_max = sr/2 by
default; every frame 1 + floor((T_pad - n_fft) / hop) is kept; reflect
padding does not repeat the edge sample; each leading index is one clip and
its maximum runs over all of its (mel, frame) values.

Parity status: every function here is pinned by tests against closed forms,
library routines on special cases, invariants and a pure-Python brute force;
the Slaney-norm choice and the synthetic-signal recipe are readings, not
pins (they change inputs, not correctness).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode_pcm",
    "zero_pad_signal",
    "pad_signal",
    "num_frames",
    "frame_signal",
    "hann_periodic",
    "rdft_direct",
    "power_spectrum",
    "hz_to_mel",
    "mel_to_hz",
    "mel_filterbank",
    "log_mel_tail",
    "frame_window",
    "normalization_factor",
    "pcm_power_frames",
    "mel_from_pcm",
    "from_pcm",
    "mel_from_stft",
    "from_stft",
]

FLOOR = 1e-10        # pre-log floor (task page, "spec_md" and "precision_md")
DYN_RANGE = 8.0      # floor at the clip maximum minus 8 decades (80 dB)

PAD_MODES = ("constant", "reflect", "replicate", "circular")


# ----------------------------------------------------------------------------
# PCM front half (flashmel page, "Usage" and "How it works")
# ----------------------------------------------------------------------------

def decode_pcm(x: np.ndarray) -> np.ndarray:
    """Samples as float64: float input as is, int16 raw PCM times 1/32768."""
    x = np.asarray(x)
    if x.dtype == np.int16:
        return x.astype(np.float64) / 32768.0
    return x.astype(np.float64)


def zero_pad_signal(x: np.ndarray, pad: int) -> np.ndarray:
    """The signal padding ahead of the transform (flashmel page, "Usage":
    torchaudio's ``pad``): ``pad`` zeros before and after the last axis.
    The center padding of ``pad_signal`` then applies to the longer signal."""
    if pad < 0:
        raise ValueError("pad must be >= 0")
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape[:-1] + (x.shape[-1] + 2 * pad,), dtype=np.float64)
    out[..., pad:pad + x.shape[-1]] = x
    return out


def pad_signal(x: np.ndarray, n_fft: int, center: bool, pad_mode: str) -> np.ndarray:
    """Pad the last axis by n_fft // 2 on both sides when ``center``.

    constant: zeros; reflect: mirror about the edge sample without repeating
    it; replicate: repeat the edge sample; circular: wrap around.
    """
    if pad_mode not in PAD_MODES:
        raise ValueError(f"pad_mode {pad_mode!r}")
    x = np.asarray(x, dtype=np.float64)
    if not center:
        return x.copy()
    p = n_fft // 2
    T = x.shape[-1]
    j = np.arange(-p, T + p)
    if pad_mode == "constant":
        out = np.zeros(x.shape[:-1] + (T + 2 * p,), dtype=np.float64)
        out[..., p:p + T] = x
        return out
    if pad_mode == "reflect":
        if T <= p:
            raise ValueError("reflect padding needs more samples than n_fft // 2")
        idx = np.where(j < 0, -j, np.where(j >= T, 2 * (T - 1) - j, j))
    elif pad_mode == "replicate":
        idx = np.clip(j, 0, T - 1)
    else:  # circular
        if T < p:
            raise ValueError("circular padding needs at least n_fft // 2 samples")
        idx = np.mod(j, T)
    return x[..., idx]


def num_frames(T: int, n_fft: int, hop: int, center: bool, pad: int = 0) -> int:
    """Frame count: 1 + floor((T_padded - n_fft) / hop); no frame is dropped.
    T_padded = T + 2 pad (signal padding) + 2 (n_fft // 2) if center."""
    t_pad = T + 2 * pad + (2 * (n_fft // 2) if center else 0)
    if t_pad < n_fft:
        raise ValueError("signal shorter than one frame")
    return 1 + (t_pad - n_fft) // hop


def frame_signal(xp: np.ndarray, n_fft: int, hop: int) -> np.ndarray:
    """(..., T_pad) -> (..., F, n_fft); frame f is xp[f*hop : f*hop + n_fft]."""
    F = 1 + (xp.shape[-1] - n_fft) // hop
    starts = np.arange(F) * hop
    idx = starts[:, None] + np.arange(n_fft)[None, :]
    return xp[..., idx]


def hann_periodic(N: int) -> np.ndarray:
    """Periodic Hann window: 0.5 - 0.5 cos(2 pi n / N), n = 0..N-1."""
    n = np.arange(N, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * n / N)


def frame_window(n_fft: int, win_length: int | None = None) -> np.ndarray:
    """The n_fft-point frame window: the periodic Hann of win_length samples
    (default n_fft) with (n_fft - win_length) // 2 zeros before it and the
    rest after it (flashmel page, "Usage": torchaudio's win_length, whose
    shorter window torch.stft centres in the frame; a one-point window is
    [1], torch's convention)."""
    W = n_fft if win_length is None else int(win_length)
    if not 1 <= W <= n_fft:
        raise ValueError("need 1 <= win_length <= n_fft")
    w = np.zeros(n_fft, dtype=np.float64)
    left = (n_fft - W) // 2
    # a one-point window is [1], as torch.hann_window gives it (the formula
    # would give [0] and an all-zero spectrum)
    w[left:left + W] = hann_periodic(W) if W > 1 else 1.0
    return w


def normalization_factor(window: np.ndarray, normalized, win_length: int) -> float:
    """Factor applied to the complex spectrum before |X|^power (flashmel
    page, "Usage": torchaudio's ``normalized``): 1 for none,
    1 / sqrt(sum w^2) for True / "window", 1 / sqrt(win_length) for
    "frame_length"."""
    if normalized in (None, False, "none"):
        return 1.0
    if normalized in (True, "window"):
        return 1.0 / math.sqrt(float(np.sum(window * window)))
    if normalized == "frame_length":
        return 1.0 / math.sqrt(float(win_length))
    raise ValueError(normalized)


def rdft_direct(y: np.ndarray, chunk: int | None = None) -> np.ndarray:
    """One-sided DFT by its definition: X[k] = sum_n y[n] exp(-2 pi i k n / N).

    k = 0..N/2.  The angle uses the exact integer residue (k n) mod N before
    scaling, so no large-argument cos/sin is taken.  Evaluated as float64
    matrix products over chunks of bins (a library matmul is one step; the
    sum itself is the plain O(N^2) definition).  The default chunk keeps each
    temporary near 16 MB.
    """
    y = np.asarray(y, dtype=np.float64)
    N = y.shape[-1]
    if chunk is None:
        chunk = max(1, (1 << 21) // N)
    K = N // 2 + 1
    lead = y.shape[:-1]
    y2 = y.reshape(-1, N)
    out = np.empty((y2.shape[0], K), dtype=np.complex128)
    n = np.arange(N, dtype=np.int64)
    for k0 in range(0, K, chunk):
        k = np.arange(k0, min(K, k0 + chunk), dtype=np.int64)
        theta = (2.0 * np.pi / N) * ((n[:, None] * k[None, :]) % N).astype(np.float64)
        re = y2 @ np.cos(theta)
        im = -(y2 @ np.sin(theta))
        out[:, k0:k0 + k.size] = re + 1j * im
    return out.reshape(lead + (K,))


def power_spectrum(X: np.ndarray, power: float = 2.0) -> np.ndarray:
    """|X|^power; power 2 is re^2 + im^2 (the power spectrum, not magnitude)."""
    p2 = X.real * X.real + X.imag * X.imag
    if power == 2.0:
        return p2
    return p2 ** (power / 2.0)


# ----------------------------------------------------------------------------
# Mel filterbank (flashmel page, "Usage": torchaudio-style n_mels, f_min,
# f_max, norm and mel_scale arguments)
# ----------------------------------------------------------------------------

_SLANEY_F_SP = 200.0 / 3.0          # Hz per mel on the linear part
_SLANEY_BREAK_HZ = 1000.0
_SLANEY_BREAK_MEL = _SLANEY_BREAK_HZ / _SLANEY_F_SP   # = 15
_SLANEY_LOGSTEP = math.log(6.4) / 27.0


def hz_to_mel(f, scale: str = "slaney"):
    """Hz -> mel.  Slaney: linear 3f/200 below 1 kHz, logarithmic above
    (27 mels per factor 6.4).  HTK: 2595 log10(1 + f/700)."""
    f = np.asarray(f, dtype=np.float64)
    if scale == "htk":
        return 2595.0 * np.log10(1.0 + f / 700.0)
    if scale != "slaney":
        raise ValueError(scale)
    lin = f / _SLANEY_F_SP
    with np.errstate(divide="ignore", invalid="ignore"):
        log = _SLANEY_BREAK_MEL + np.log(np.maximum(f, 1e-300) / _SLANEY_BREAK_HZ) / _SLANEY_LOGSTEP
    return np.where(f >= _SLANEY_BREAK_HZ, log, lin)


def mel_to_hz(m, scale: str = "slaney"):
    """Inverse of ``hz_to_mel``."""
    m = np.asarray(m, dtype=np.float64)
    if scale == "htk":
        return 700.0 * (10.0 ** (m / 2595.0) - 1.0)
    if scale != "slaney":
        raise ValueError(scale)
    lin = _SLANEY_F_SP * m
    log = _SLANEY_BREAK_HZ * np.exp(_SLANEY_LOGSTEP * (m - _SLANEY_BREAK_MEL))
    return np.where(m >= _SLANEY_BREAK_MEL, log, lin)


def mel_filterbank(sample_rate: float, n_fft: int, n_mels: int, f_min: float = 0.0,
                   f_max: float | None = None, scale: str = "slaney",
                   norm: str | None = "slaney") -> np.ndarray:
    """(n_mels, n_fft//2 + 1) triangular filterbank in float64.

    Corner frequencies: n_mels + 2 points evenly spaced in mel between
    mel(f_min) and mel(f_max), mapped back to Hz.  Bin k sits at k*sr/n_fft.
    Row m is max(0, min(rising, falling)) of the triangle on corners m, m+1,
    m+2; the Slaney norm scales row m by 2 / (f[m+2] - f[m]) (unit area).
    """
    if f_max is None:
        f_max = sample_rate / 2.0
    n_bins = n_fft // 2 + 1
    fk = np.arange(n_bins, dtype=np.float64) * (sample_rate / n_fft)
    m_pts = np.linspace(hz_to_mel(f_min, scale), hz_to_mel(f_max, scale), n_mels + 2)
    f_pts = mel_to_hz(m_pts, scale)
    W = np.zeros((n_mels, n_bins), dtype=np.float64)
    for m in range(n_mels):
        lo, mid, hi = f_pts[m], f_pts[m + 1], f_pts[m + 2]
        rise = (fk - lo) / (mid - lo)
        fall = (hi - fk) / (hi - mid)
        W[m] = np.maximum(0.0, np.minimum(rise, fall))
        if norm == "slaney":
            W[m] *= 2.0 / (hi - lo)
        elif norm not in (None, "none"):
            raise ValueError(norm)
    return W


# ----------------------------------------------------------------------------
# Log / clamp / rescale tail (task page, "spec_md")
# ----------------------------------------------------------------------------

def log_mel_tail(mel: np.ndarray) -> np.ndarray:
    """Per clip (leading axis): log10(max(mel, 1e-10)), then the floor at the
    clip's maximum log value minus 8, then (x + 4) / 4.  The maximum runs
    over every (frame, band) value of that clip -- not per frame, not per
    batch -- and the 1e-10 floor comes before the log."""
    mel = np.asarray(mel, dtype=np.float64)
    L = np.log10(np.maximum(mel, FLOOR))
    axes = tuple(range(1, L.ndim))
    hi = L.max(axis=axes, keepdims=True)
    return (np.maximum(L, hi - DYN_RANGE) + 4.0) / 4.0


# ----------------------------------------------------------------------------
# Whole paths
# ----------------------------------------------------------------------------

def pcm_power_frames(x_clip: np.ndarray, n_fft: int, hop: int, center: bool = True,
                     pad_mode: str = "reflect", power: float = 2.0, win_length: int | None = None,
                     normalized=None, pad: int = 0) -> np.ndarray:
    """One clip (T,) -> (F, n_fft//2 + 1) |c X|^power of the windowed frames,
    c the normalisation factor (1 unless ``normalized``); the clip is first
    given ``pad`` zeros on both sides, then the center padding."""
    xp = pad_signal(zero_pad_signal(decode_pcm(x_clip), pad), n_fft, center, pad_mode)
    w = frame_window(n_fft, win_length)
    frames = frame_signal(xp, n_fft, hop) * w[None, :]
    c = normalization_factor(w, normalized, n_fft if win_length is None else win_length)
    return power_spectrum(c * rdft_direct(frames), power)


def mel_from_pcm(x: np.ndarray, n_fft: int, hop: int, filters: np.ndarray, center: bool = True,
                 pad_mode: str = "reflect", power: float = 2.0, win_length: int | None = None,
                 normalized=None, pad: int = 0) -> np.ndarray:
    """PCM (B, T) float32 or int16 -> (B, n_mels, F) mel values in float64:
    sum_k W[m, k] |c X_k|^power, the output of a torchaudio-style
    MelSpectrogram (flashmel page, "Usage").

    ``filters`` is the (n_mels, n_fft//2 + 1) filterbank (float64 or the
    float32 weights actually used); the mel sum is dense over all bins.
    """
    x = np.asarray(x)
    if x.ndim == 1:
        x = x[None, :]
    W = np.asarray(filters, dtype=np.float64)
    outs = []
    for b in range(x.shape[0]):
        P = pcm_power_frames(x[b], n_fft, hop, center, pad_mode, power, win_length, normalized, pad)
        mel = P @ W.T                       # (F, n_mels)
        outs.append(mel.T[None])            # (1, n_mels, F)
    return np.concatenate(outs, axis=0)


def from_pcm(x: np.ndarray, n_fft: int, hop: int, filters: np.ndarray, center: bool = True,
             pad_mode: str = "reflect", power: float = 2.0, win_length: int | None = None,
             normalized=None, pad: int = 0) -> np.ndarray:
    """PCM (B, T) float32 or int16 -> (B, n_mels, F) log-mel in float64: the
    mel values of ``mel_from_pcm`` through the per-clip log tail."""
    return log_mel_tail(mel_from_pcm(x, n_fft, hop, filters, center, pad_mode, power, win_length, normalized, pad))


def mel_from_stft(stft: np.ndarray, mel_filters: np.ndarray) -> np.ndarray:
    """Complex STFT (B, F, NF) -> (B, F, NM) mel values in float64:
    (re^2 + im^2) @ W^T (task page, "reference_src", before the log)."""
    s = np.asarray(stft)
    if s.ndim == 2:
        s = s[None]
    W = np.asarray(mel_filters, dtype=np.float64)
    out = np.empty(s.shape[:2] + (W.shape[0],), dtype=np.float64)
    for b in range(s.shape[0]):
        re = s[b].real.astype(np.float64)
        im = s[b].imag.astype(np.float64)
        mag = re * re + im * im
        out[b] = (mag @ W.T)
    return out


def from_stft(stft: np.ndarray, mel_filters: np.ndarray) -> np.ndarray:
    """Complex STFT (B, F, NF) -> (B, F, NM) log-mel in float64."""
    return log_mel_tail(mel_from_stft(stft, mel_filters))
