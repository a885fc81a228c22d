"""Seeded synthetic inputs for the log-mel front end.

This module only draws inputs.  It holds none of the transform's arithmetic
(no window, no DFT, no mel scale, no log): both the fp64 oracle and the HIP
path read the arrays it returns, bit for bit.

Workloads
---------
``WORKLOADS`` names the five shapes the library is measured and checked on:

* ``stft_b1``   complex STFT, 1 clip x 3000 frames x 201 bins, 80 linear
  triangles, fp32 out.
* ``pcm_f32_b8`` 8 clips x 480000 float32 samples (30 s at 16 kHz),
  n_fft 400, hop 160, 80 Slaney mels over 0-8 kHz, fp32 out.
* ``pcm_i16_b64`` 64 clips x 480000 int16 samples, n_fft 400, hop 160,
  128 Slaney mels over 0-8 kHz, fp32 out.  (The headline workload.)
* ``stft_b256`` complex STFT, 256 clips x 3000 x 201, 128 linear triangles.
* ``pcm_f32_nfft16384`` 16 clips x 441000 float32 samples (10 s at 44.1 kHz),
  n_fft 16384, hop 4096, 256 Slaney mels over 0-22.05 kHz, fp16 out.

and adds the n_fft sweep ``sweep_nfft{64..16384}``: 32 clips x 160000
standard-normal float32 samples, hop n_fft / 4, 128 Slaney mels, fp32 out.

Generators
----------
``stft_speechlike`` draws the STFT workload the KBench
``audio-mel-spectrogram-fused`` task page describes in words: a speech-like
spectrum, strong at low frequencies and with about 60 dB of level change
across frames.  Each bin is a circular complex Gaussian whose amplitude is a
spectral tilt (falling by a factor e every NF/3 bins) times a per-frame
level 0.05 + u^2, u uniform on [0, 1).

``lintri_filters`` is that page's "NM overlapping triangles spread over the
NF bins": NM+2 equally spaced points from bin 0 to bin NF-1, triangle m
peaking (at 1) on point m+1 and reaching 0 on its two neighbours.

``speech_pcm`` and ``music_pcm`` make the PCM workloads (the pages describe
only their character; the exact recipe is this module's reading of it and
is recorded by ``recipe()``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "stft_speechlike",
    "lintri_filters",
    "speech_pcm",
    "music_pcm",
    "make_inputs",
    "recipe",
]


# ----------------------------------------------------------------------------
# STFT-path inputs
# ----------------------------------------------------------------------------

def stft_speechlike(B: int, F: int, NF: int, seed: int) -> np.ndarray:
    """(B, F, NF) complex64 speech-like STFT.

    Bin k of frame f in clip b is ``level[b, f] * tilt[k] * z`` with z a
    complex normal whose real and imaginary parts are independent N(0, 1),
    ``tilt[k] = exp(-3 k / NF)`` and ``level = 0.05 + u^2``, u ~ U[0, 1).
    Levels span 0.05 .. 1.05 (about 26 dB of frame power) and the tilt
    another 26 dB across the bins, the page's "about 60 dB" in round terms.
    Draw order: all levels, then the (re, im) pairs of one clip after
    another, in float32.
    """
    rng = np.random.default_rng(seed)
    u = rng.random((B, F), dtype=np.float32)
    level = np.float32(0.05) + u * u
    tilt = np.exp(np.float32(-3.0 / NF) * np.arange(NF, dtype=np.float32)).astype(np.float32)
    out = np.empty((B, F, NF), dtype=np.complex64)
    pairs = out.view(np.float32).reshape(B, F, NF, 2)
    for b in range(B):
        amp = level[b][:, None] * tilt[None, :]
        pairs[b] = rng.standard_normal((F, NF, 2), dtype=np.float32) * amp[:, :, None]
    return out


def lintri_filters(NF: int, NM: int) -> np.ndarray:
    """(NM, NF) float32 triangles over bin indices.

    With spacing d = (NF - 1) / (NM + 1), triangle m is the hat
    max(0, 1 - |k - (m + 1) d| / d): 1 at bin (m + 1) d, 0 from (m + 2) d on
    and up to m d.  NF = 1 leaves no room for a triangle: all zero.
    """
    if NF < 1 or NM < 1:
        raise ValueError("lintri_filters needs NF >= 1 and NM >= 1")
    if NF == 1:
        return np.zeros((NM, 1), dtype=np.float32)
    d = (NF - 1) / (NM + 1)
    k = np.arange(NF, dtype=np.float64)
    peak = d * np.arange(1, NM + 1, dtype=np.float64)
    hat = 1.0 - np.abs(k[None, :] - peak[:, None]) / d
    return np.ascontiguousarray(np.maximum(hat, 0.0).astype(np.float32))


# ----------------------------------------------------------------------------
# PCM-path inputs
# ----------------------------------------------------------------------------

def speech_pcm(B: int, T: int, sr: float, seed: int, as_int16: bool = False) -> np.ndarray:
    """(B, T) speech-like PCM: float32, or int16 raw PCM.

    Per clip: one fundamental f0 ~ U(80, 300) Hz; harmonics h = 1..10 with
    amplitude 1/h and phase ~ U(0, 2pi); a 4 Hz syllable envelope
    0.5 * (1 - cos(2pi * 4 t + psi)), psi ~ U(0, 2pi); white Gaussian noise
    whose RMS is 30 dB below the RMS of the enveloped tone; the clip is then
    scaled so its peak magnitude is 0.5 (about -6 dBFS).  int16 output is
    round-half-even of x * 32768, clipped to the int16 range.
    Draw order: f0 (B), phases (B, 10), psi (B), noise (B, T).
    """
    rng = np.random.default_rng(seed)
    f0 = rng.uniform(80.0, 300.0, size=B)
    phases = rng.uniform(0.0, 2.0 * np.pi, size=(B, 10))
    psi = rng.uniform(0.0, 2.0 * np.pi, size=B)
    t = np.arange(T, dtype=np.float64) / sr
    out = np.empty((B, T), dtype=np.int16 if as_int16 else np.float32)
    noise_gain = 10.0 ** (-30.0 / 20.0)
    for b in range(B):
        tone = np.zeros(T, dtype=np.float64)
        for h in range(1, 11):
            tone += np.sin(2.0 * np.pi * h * f0[b] * t + phases[b, h - 1]) / h
        env = 0.5 * (1.0 - np.cos(2.0 * np.pi * 4.0 * t + psi[b]))
        sig = tone * env
        rms = math.sqrt(float(np.mean(sig * sig)))
        noise = rng.standard_normal(T)
        x = sig + noise * (noise_gain * rms)
        x *= 0.5 / float(np.max(np.abs(x)))
        if as_int16:
            q = np.rint(x * 32768.0)  # numpy rint rounds half to even
            out[b] = np.clip(q, -32768, 32767).astype(np.int16)
        else:
            out[b] = x.astype(np.float32)
    return out


def music_pcm(B: int, T: int, sr: float, seed: int) -> np.ndarray:
    """(B, T) float32: three random sinusoids plus pink noise at -20 dB.

    Frequencies ~ U(50, 15000) Hz, phases ~ U(0, 2pi), amplitude 0.25 each.
    Pink noise: white Gaussian noise whose spectrum is scaled by 1/sqrt(f)
    (DC removed), rescaled to an RMS one tenth of the sinusoid mix's RMS.
    No peak normalisation.  Draw order: freqs (B, 3), phases (B, 3),
    white noise (B, T).
    """
    rng = np.random.default_rng(seed)
    freqs = rng.uniform(50.0, 15000.0, size=(B, 3))
    phases = rng.uniform(0.0, 2.0 * np.pi, size=(B, 3))
    t = np.arange(T, dtype=np.float64) / sr
    out = np.empty((B, T), dtype=np.float32)
    fbin = np.fft.rfftfreq(T, d=1.0 / sr)
    shape = np.zeros_like(fbin)
    shape[1:] = 1.0 / np.sqrt(fbin[1:])
    for b in range(B):
        tones = np.zeros(T, dtype=np.float64)
        for i in range(3):
            tones += 0.25 * np.sin(2.0 * np.pi * freqs[b, i] * t + phases[b, i])
        white = rng.standard_normal(T)
        pink = np.fft.irfft(np.fft.rfft(white) * shape, n=T)
        pink *= 0.1 * math.sqrt(float(np.mean(tones * tones))) / math.sqrt(float(np.mean(pink * pink)))
        out[b] = (tones + pink).astype(np.float32)
    return out


# ----------------------------------------------------------------------------
# Workload registry
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    entry: str                      # "stft" or "pcm"
    seed: int
    B: int
    # STFT path
    F: int = 0
    NF: int = 0
    NM: int = 0
    # PCM path
    T: int = 0
    sample_rate: float = 0.0
    n_fft: int = 0
    hop: int = 0
    n_mels: int = 0
    f_min: float = 0.0
    f_max: float = 0.0
    in_dtype: str = "f32"           # "f32" | "i16"
    out_dtype: str = "f32"          # "f32" | "f16"
    center: bool = True
    pad_mode: str = "reflect"
    power: float = 2.0
    signal: str = ""                # "speech" | "music"
    extra: dict = field(default_factory=dict)

    @property
    def n_frames(self) -> int:
        if self.entry == "stft":
            return self.F
        pad = self.n_fft // 2 if self.center else 0
        return 1 + (self.T + 2 * pad - self.n_fft) // self.hop

    @property
    def out_shape(self) -> tuple:
        if self.entry == "stft":
            return (self.B, self.F, self.NM)
        return (self.B, self.n_mels, self.n_frames)

    def essential_bytes(self) -> int:
        """One read of the source plus one write of the result."""
        out_elt = 2 if self.out_dtype == "f16" else 4
        n_out = int(np.prod(self.out_shape))
        if self.entry == "stft":
            return self.B * self.F * self.NF * 8 + n_out * out_elt
        in_elt = 2 if self.in_dtype == "i16" else 4
        return self.B * self.T * in_elt + n_out * out_elt


WORKLOADS = {
    "stft_b1": Workload("stft_b1", "stft", seed=1, B=1, F=3000, NF=201, NM=80),
    "pcm_f32_b8": Workload("pcm_f32_b8", "pcm", seed=2, B=8, T=480000, sample_rate=16000.0,
                           n_fft=400, hop=160, n_mels=80, f_min=0.0, f_max=8000.0,
                           in_dtype="f32", out_dtype="f32", signal="speech"),
    "pcm_i16_b64": Workload("pcm_i16_b64", "pcm", seed=3, B=64, T=480000, sample_rate=16000.0,
                            n_fft=400, hop=160, n_mels=128, f_min=0.0, f_max=8000.0,
                            in_dtype="i16", out_dtype="f32", signal="speech"),
    "stft_b256": Workload("stft_b256", "stft", seed=4, B=256, F=3000, NF=201, NM=128),
    "pcm_f32_nfft16384": Workload("pcm_f32_nfft16384", "pcm", seed=5, B=16, T=441000,
                                  sample_rate=44100.0, n_fft=16384, hop=4096, n_mels=256,
                                  f_min=0.0, f_max=22050.0, in_dtype="f32", out_dtype="f16",
                                  signal="music"),
}


# The flashmel page's n_fft sweep ("Performance": n_fft 64..16384, hop =
# n_fft / 4, 128 mels, B = 32 clips of T = 160000 samples, randn input);
# the sample rate is not stated there: 16 kHz, mels over 0..8 kHz.
SWEEP_SIZES = (64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384)
for _n in SWEEP_SIZES:
    WORKLOADS[f"sweep_nfft{_n}"] = Workload(
        f"sweep_nfft{_n}", "pcm", seed=100 + _n.bit_length(), B=32, T=160000, sample_rate=16000.0,
        n_fft=_n, hop=_n // 4, n_mels=128, f_min=0.0, f_max=8000.0, in_dtype="f32", out_dtype="f32",
        signal="noise")


def noise_pcm(B: int, T: int, seed: int) -> np.ndarray:
    """(B, T) float32 standard normal samples (the sweep's randn input)."""
    return np.random.default_rng(seed).standard_normal((B, T)).astype(np.float32)


def make_inputs(w: Workload, B: int | None = None, T: int | None = None, F: int | None = None):
    """Inputs for workload ``w`` (optionally with fewer clips / samples / frames).

    STFT workloads return ``(stft complex64 (B,F,NF), filters float32 (NM,NF))``;
    PCM workloads return ``pcm`` (float32 or int16, (B, T)).
    """
    B = w.B if B is None else B
    if w.entry == "stft":
        F = w.F if F is None else F
        return stft_speechlike(B, F, w.NF, w.seed), lintri_filters(w.NF, w.NM)
    T = w.T if T is None else T
    if w.signal == "speech":
        return speech_pcm(B, T, w.sample_rate, w.seed, as_int16=(w.in_dtype == "i16"))
    if w.signal == "noise":
        return noise_pcm(B, T, w.seed)
    return music_pcm(B, T, w.sample_rate, w.seed)


def recipe() -> dict:
    """The generator readings, for recording next to results."""
    return {
        "stft": "level=0.05+u^2 per frame, tilt=exp(-3k/NF), bin=level*tilt*(N(0,1)+iN(0,1)), "
                "numpy PCG64(seed): levels, then (re, im) pairs clip by clip",
        "lintri": "hat max(0, 1-|k-(m+1)d|/d), d=(NF-1)/(NM+1), fp64 then fp32",
        "speech": "f0~U(80,300), h=1..10 amp 1/h phase U(0,2pi), env 0.5(1-cos(2pi*4t+psi)), "
                  "noise RMS -30 dB re tone RMS, peak 0.5; i16=rint(x*32768) clipped",
        "music": "3 sines U(50,15000) Hz amp 0.25 random phase + pink(1/sqrt f) at 0.1x RMS",
        "noise": "standard normal float32, numpy PCG64(seed) (the n_fft sweep)",
        "seeds": {k: v.seed for k, v in WORKLOADS.items()},
    }
