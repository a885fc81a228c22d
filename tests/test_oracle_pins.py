"""Pins of the fp64 oracle against things other than itself.

Each test ties one oracle step to a closed form, a library routine on a
special case, an invariant the pages fix, or a hand-derived fixture.  The
mutation tests at the end plant plausible mistakes in the oracle (on the
CPU) and check that at least one pin catches each.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tests.golden_io import load_stft_worked

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ----------------------------------------------------------------------------
# DFT
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N", [8, 16, 64, 400, 1024, 4096])
def test_rdft_matches_library_fft(N):
    """The direct DFT equals numpy's FFT (a library routine) to fp64 rounding."""
    rng = np.random.default_rng(N)
    y = rng.standard_normal((5, N))
    X = oracle.rdft_direct(y)
    ref = np.fft.rfft(y, axis=-1)
    assert X.shape == ref.shape == (5, N // 2 + 1)
    err = np.max(np.abs(X - ref)) / np.max(np.abs(ref))
    assert err < 1e-12, err


def test_rdft_16384_matches_library_fft():
    rng = np.random.default_rng(16384)
    y = rng.standard_normal((2, 16384))
    X = oracle.rdft_direct(y)
    ref = np.fft.rfft(y, axis=-1)
    assert np.max(np.abs(X - ref)) / np.max(np.abs(ref)) < 1e-11


@pytest.mark.parametrize("N", [16, 400, 2048])
def test_parseval(N):
    """|X0|^2 + |X_{N/2}|^2 + 2 sum_{0<k<N/2} |Xk|^2 = N sum y^2 (even N)."""
    rng = np.random.default_rng(7 + N)
    y = rng.standard_normal((4, N))
    P = oracle.power_spectrum(oracle.rdft_direct(y))
    lhs = P[:, 0] + P[:, -1] + 2.0 * P[:, 1:-1].sum(axis=1)
    rhs = N * (y * y).sum(axis=1)
    assert np.max(np.abs(lhs - rhs) / rhs) < 1e-12


def test_power_general_exponent():
    X = np.array([3 + 4j, 0 + 0j, -1 + 0j])
    assert np.allclose(oracle.power_spectrum(X, 2.0), [25.0, 0.0, 1.0], rtol=0, atol=1e-15)
    assert np.allclose(oracle.power_spectrum(X, 1.0), [5.0, 0.0, 1.0], rtol=0, atol=1e-15)
    assert np.allclose(oracle.power_spectrum(X, 3.0), [125.0, 0.0, 1.0], rtol=1e-14)


# ----------------------------------------------------------------------------
# Window, framing, padding
# ----------------------------------------------------------------------------

def test_hann_is_periodic():
    w = oracle.hann_periodic(400)
    assert w[0] == 0.0
    assert abs(w[200] - 1.0) < 1e-15            # peak at N/2 (periodic, denominator N)
    assert abs(w[100] - 0.5) < 1e-15
    assert np.allclose(w[1:], w[1:][::-1], atol=1e-15)   # symmetric about N/2
    tw = torch.hann_window(400, periodic=True, dtype=torch.float64).numpy()
    assert np.max(np.abs(w - tw)) < 1e-15


def test_bin_centred_tone_closed_form():
    """A bin-centred tone A cos(2 pi k0 n / N + phi) through the periodic Hann:
    |X[k0]|^2 = (A N / 4)^2, |X[k0 +- 1]|^2 = (A N / 8)^2, every other bin 0
    (the window's DFT has exactly three non-zero coefficients)."""
    N, hop, A, k0, phi = 400, 160, 0.5, 25, 0.3
    T = 16000
    n = np.arange(T)
    x = (A * np.cos(2 * np.pi * k0 * n / N + phi)).astype(np.float64)
    P = oracle.pcm_power_frames(x, N, hop, center=True, pad_mode="reflect")
    inner = P[3:-3]                      # frames whose span avoids the padded edges
    assert np.allclose(inner[:, k0], (A * N / 4) ** 2, rtol=1e-11)
    assert np.allclose(inner[:, k0 - 1], (A * N / 8) ** 2, rtol=1e-11)
    assert np.allclose(inner[:, k0 + 1], (A * N / 8) ** 2, rtol=1e-11)
    rest = np.delete(inner, [k0 - 1, k0, k0 + 1], axis=1)
    assert np.max(rest) < 1e-18 * (A * N) ** 2 * 1e6
    assert (A * N / 4) ** 2 == 2500.0 and (A * N / 8) ** 2 == 625.0


def test_impulse_gives_flat_power():
    """delta at frame offset n0: |X[k]|^2 = w[n0]^2 for every k."""
    N, hop = 64, 16
    x = np.zeros(640)
    x[300] = 1.0
    P = oracle.pcm_power_frames(x, N, hop, center=True, pad_mode="constant")
    w = oracle.hann_periodic(N)
    pad = N // 2
    for f in range(P.shape[0]):
        n0 = 300 + pad - f * hop
        if 0 <= n0 < N:
            assert np.allclose(P[f], w[n0] ** 2, rtol=1e-12, atol=1e-15)
        else:
            assert np.max(P[f]) == 0.0


@pytest.mark.parametrize("pad_mode", ["reflect", "replicate", "circular"])
def test_dc_closed_form_every_frame(pad_mode):
    """Constant c: P[0] = (c N/2)^2, P[1] = (c N/4)^2, all else 0, on every
    frame including the padded edges (any mode that repeats the signal)."""
    N, hop, c = 400, 160, 0.25
    x = np.full(4000, c)
    P = oracle.pcm_power_frames(x, N, hop, center=True, pad_mode=pad_mode)
    assert np.allclose(P[:, 0], (c * N / 2) ** 2, rtol=1e-12)
    assert np.allclose(P[:, 1], (c * N / 4) ** 2, rtol=1e-12)
    assert np.max(P[:, 2:]) < 1e-20 * (c * N) ** 2 * 1e8


@pytest.mark.parametrize("pad_mode", ["reflect", "constant", "replicate", "circular"])
@pytest.mark.parametrize("n_fft,hop,T", [(400, 160, 4321), (64, 16, 1000), (1024, 256, 5000),
                                        (16, 5, 37)])
def test_framing_padding_window_match_torch_stft(pad_mode, n_fft, hop, T):
    """torch.stft (CPU, fp64, periodic Hann, center=True) is an independent
    library routine for framing + padding + window + one-sided DFT."""
    rng = np.random.default_rng(T)
    x = rng.standard_normal(T)
    P = oracle.pcm_power_frames(x, n_fft, hop, center=True, pad_mode=pad_mode)
    S = torch.stft(torch.from_numpy(x), n_fft, hop_length=hop,
                   window=torch.hann_window(n_fft, periodic=True, dtype=torch.float64),
                   center=True, pad_mode=pad_mode if pad_mode != "replicate" else "replicate",
                   return_complex=True)
    ref = (S.abs() ** 2).numpy().T          # (F, K)
    assert P.shape == ref.shape
    assert np.max(np.abs(P - ref)) / np.max(ref) < 1e-12


def test_center_false_matches_torch_stft():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(3000)
    P = oracle.pcm_power_frames(x, 256, 100, center=False)
    S = torch.stft(torch.from_numpy(x), 256, hop_length=100,
                   window=torch.hann_window(256, periodic=True, dtype=torch.float64),
                   center=False, return_complex=True)
    ref = (S.abs() ** 2).numpy().T
    assert P.shape == ref.shape
    assert np.max(np.abs(P - ref)) / np.max(ref) < 1e-12


def test_frame_counts():
    assert oracle.num_frames(480000, 400, 160, True) == 3001
    assert oracle.num_frames(441000, 16384, 4096, True) == 108
    assert oracle.num_frames(400, 400, 160, False) == 1
    assert oracle.num_frames(559, 400, 160, False) == 1
    assert oracle.num_frames(560, 400, 160, False) == 2


def test_int16_decode_is_exact_scaling():
    x = np.array([-32768, -1, 0, 1, 32767], dtype=np.int16)
    d = oracle.decode_pcm(x)
    assert list(d) == [-1.0, -1.0 / 32768, 0.0, 1.0 / 32768, 32767.0 / 32768]


# ----------------------------------------------------------------------------
# Filterbank
# ----------------------------------------------------------------------------

def test_slaney_scale_closed_forms():
    m = oracle.hz_to_mel
    assert abs(m(1000.0) - 15.0) < 1e-12                      # break point
    assert abs(m(6400.0) - 42.0) < 1e-12                      # 27 mels per factor 6.4
    assert abs(m(200.0 / 3.0) - 1.0) < 1e-12                  # linear part, 200/3 Hz per mel
    assert abs(m(500.0) - 7.5) < 1e-12
    for f in [0.0, 123.0, 999.0, 1000.0, 1001.0, 8000.0, 22050.0]:
        assert abs(oracle.mel_to_hz(m(f)) - f) < 1e-9
    assert abs(m(700.0, "htk") - 2595.0 * math.log10(2.0)) < 1e-12


@pytest.mark.parametrize("sr,n_fft,n_mels,fmax", [(16000, 400, 80, 8000), (16000, 400, 128, 8000),
                                                  (44100, 16384, 256, 22050), (16000, 512, 40, 7600)])
@pytest.mark.parametrize("scale", ["slaney", "htk"])
def test_filterbank_invariants(sr, n_fft, n_mels, fmax, scale):
    W = oracle.mel_filterbank(sr, n_fft, n_mels, 0.0, fmax, scale=scale, norm=None)
    Wn = oracle.mel_filterbank(sr, n_fft, n_mels, 0.0, fmax, scale=scale, norm="slaney")
    fk = np.arange(n_fft // 2 + 1) * sr / n_fft
    f_pts = oracle.mel_to_hz(np.linspace(oracle.hz_to_mel(0.0, scale), oracle.hz_to_mel(fmax, scale),
                                         n_mels + 2), scale)
    assert (W >= 0).all()
    assert W.max() <= 1.0 + 1e-12
    for m in range(n_mels):
        nz = np.nonzero(W[m])[0]
        if nz.size:
            assert nz[-1] - nz[0] + 1 == nz.size          # one contiguous run
            assert fk[nz[0]] > f_pts[m] - 1e-9 and fk[nz[-1]] < f_pts[m + 2] + 1e-9
        # Slaney norm = unit-area scaling of the same row
        assert np.allclose(Wn[m], W[m] * 2.0 / (f_pts[m + 2] - f_pts[m]), rtol=1e-13, atol=0)
    # partition of unity between the first and last peak
    inside = (fk >= f_pts[1]) & (fk <= f_pts[n_mels])
    assert np.allclose(W[:, inside].sum(axis=0), 1.0, atol=1e-12)


def test_filterbank_peak_at_centre_when_on_bin():
    """A corner that falls exactly on a bin gives weight 1 there (un-normalised)."""
    # sr = 2000, n_fft = 20 -> bins every 100 Hz; HTK scale chosen so corners
    # land anywhere; use a linear-in-Hz check via slaney below 1 kHz instead:
    # below 1 kHz the Slaney scale is linear, so corners are evenly spaced in Hz.
    W = oracle.mel_filterbank(2000.0, 20, 8, 0.0, 900.0, scale="slaney", norm=None)
    # corners at 0,100,...,900 Hz = bins 0..9; row m peaks at bin m+1 with weight 1
    for m in range(8):
        assert abs(W[m, m + 1] - 1.0) < 1e-12
        assert abs(W[m].sum() - 1.0) < 1e-12


# ----------------------------------------------------------------------------
# Log / clamp / rescale tail
# ----------------------------------------------------------------------------

def test_worked_example_fixture():
    stft, W, exp = load_stft_worked()
    out = oracle.from_stft(stft, W)
    assert np.max(np.abs(out - exp)) < 1e-12


def test_silence_is_minus_one_point_five():
    x = np.zeros((2, 4000), dtype=np.float32)
    W = oracle.mel_filterbank(16000, 400, 80, 0, 8000)
    out = oracle.from_pcm(x, 400, 160, W)
    assert np.all(out == -1.5)


def test_clamp_invariants_and_per_clip_independence():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 8000)).astype(np.float32)
    x[1] *= 1e-3
    x[2, 2000:6000] = 0.0                  # digital silence inside a loud clip
    W = oracle.mel_filterbank(16000, 400, 64, 0, 8000)
    out = oracle.from_pcm(x, 400, 160, W)
    for b in range(3):
        mel = None
        P = oracle.pcm_power_frames(x[b], 400, 160)
        mel = P @ W.T
        hi = np.log10(np.maximum(mel, 1e-10)).max()
        assert abs(out[b].max() - (hi + 4) / 4) < 1e-13
        assert out[b].min() >= (hi - 4) / 4 - 1e-13
        # clip b alone gives the same result (per-clip, not per-batch)
        solo = oracle.from_pcm(x[b:b + 1], 400, 160, W)[0]
        assert np.array_equal(solo, out[b])
    # the silent stretch is floored at hi - 8 in clip 2
    assert np.isclose(out[2].min(), out[2].max() - 2.0, atol=1e-13)


def test_gain_shift_by_half():
    """x10 amplitude = x100 power = +2 decades: every output moves by +0.5."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1, 6000))
    W = oracle.mel_filterbank(16000, 400, 80, 0, 8000)
    a = oracle.from_pcm(x, 400, 160, W)
    b = oracle.from_pcm(10.0 * x, 400, 160, W)
    assert np.max(np.abs((b - a) - 0.5)) < 1e-12


def test_clip_permutation_equivariance():
    rng = np.random.default_rng(13)
    s = (rng.standard_normal((4, 7, 33)) + 1j * rng.standard_normal((4, 7, 33))).astype(np.complex64)
    s[2] *= 1e-4
    W = rng.random((5, 33)).astype(np.float32)
    out = oracle.from_stft(s, W)
    perm = [2, 0, 3, 1]
    assert np.array_equal(oracle.from_stft(s[perm], W), out[perm])


# ----------------------------------------------------------------------------
# Brute force on tiny inputs: pure-Python scalar loops, no numpy, no FFT
# ----------------------------------------------------------------------------

def _brute_from_pcm(x, n_fft, hop, W, pad_mode):
    T = len(x)
    p = n_fft // 2

    def sample(j):
        if 0 <= j < T:
            return x[j]
        if pad_mode == "constant":
            return 0.0
        if pad_mode == "reflect":
            return x[-j] if j < 0 else x[2 * (T - 1) - j]
        if pad_mode == "replicate":
            return x[0] if j < 0 else x[T - 1]
        return x[j % T]

    F = 1 + (T + 2 * p - n_fft) // hop
    K = n_fft // 2 + 1
    mel = [[0.0] * F for _ in W]
    for f in range(F):
        seg = []
        for n in range(n_fft):
            w = 0.5 - 0.5 * math.cos(2 * math.pi * n / n_fft)
            seg.append(w * sample(f * hop + n - p))
        for k in range(K):
            re = sum(seg[n] * math.cos(2 * math.pi * k * n / n_fft) for n in range(n_fft))
            im = -sum(seg[n] * math.sin(2 * math.pi * k * n / n_fft) for n in range(n_fft))
            pw = re * re + im * im
            for m, row in enumerate(W):
                mel[m][f] += row[k] * pw
    logs = [[math.log10(max(v, 1e-10)) for v in row] for row in mel]
    hi = max(max(r) for r in logs)
    return [[(max(v, hi - 8.0) + 4.0) / 4.0 for v in r] for r in logs]


@pytest.mark.parametrize("n_fft,hop,T,pad_mode", [(8, 3, 23, "reflect"), (16, 5, 40, "constant"),
                                                 (16, 4, 17, "replicate"), (8, 2, 11, "circular")])
def test_brute_force_tiny_pcm(n_fft, hop, T, pad_mode):
    rng = np.random.default_rng(n_fft * 100 + T)
    x = rng.standard_normal(T)
    x[T // 3: T // 3 + 3] *= 1e-5
    K = n_fft // 2 + 1
    W = rng.random((3, K))
    W[:, 0] = 0.0
    got = oracle.from_pcm(x[None], n_fft, hop, W, center=True, pad_mode=pad_mode)[0]
    ref = np.array(_brute_from_pcm(list(x), n_fft, hop, W.tolist(), pad_mode))
    assert got.shape == ref.shape
    assert np.max(np.abs(got - ref)) < 1e-12


def test_brute_force_tiny_stft():
    rng = np.random.default_rng(99)
    B, F, NF, NM = 2, 4, 5, 3
    s = (rng.standard_normal((B, F, NF)) + 1j * rng.standard_normal((B, F, NF))).astype(np.complex64)
    s[1, 2] = 0
    W = rng.random((NM, NF)).astype(np.float32)
    got = oracle.from_stft(s, W)
    for b in range(B):
        logs = []
        for f in range(F):
            row = []
            for n in range(NM):
                acc = 0.0
                for k in range(NF):
                    z = complex(s[b, f, k])
                    acc += (z.real * z.real + z.imag * z.imag) * float(W[n, k])
                row.append(math.log10(max(acc, 1e-10)))
            logs.append(row)
        hi = max(max(r) for r in logs)
        for f in range(F):
            for n in range(NM):
                assert abs(got[b, f, n] - (max(logs[f][n], hi - 8) + 4) / 4) < 1e-12


# ----------------------------------------------------------------------------
# torchaudio-style surface: window length, normalisation, mel output
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n_fft,win_length,hop", [(400, 300, 160), (512, 257, 128), (64, 64, 16), (16, 1, 4)])
def test_short_window_matches_torch_stft(n_fft, win_length, hop):
    """A window shorter than the frame is centred as torch.stft centres it
    (an independent library routine, fp64, reflect padding)."""
    rng = np.random.default_rng(n_fft + win_length)
    x = rng.standard_normal((2, 9 * n_fft + 7))
    P = np.stack([oracle.pcm_power_frames(x[b], n_fft, hop, True, "reflect", 2.0, win_length) for b in range(2)])
    S = torch.stft(torch.from_numpy(x), n_fft, hop, win_length,
                   torch.hann_window(win_length, periodic=True, dtype=torch.float64),
                   center=True, pad_mode="reflect", return_complex=True)
    ref = (S.abs() ** 2).numpy().transpose(0, 2, 1)
    assert P.shape == ref.shape
    assert np.max(np.abs(P - ref)) / np.max(ref) < 1e-12


@pytest.mark.parametrize("pad_mode", ["reflect", "constant", "replicate", "circular"])
@pytest.mark.parametrize("n_fft,hop,T,pad", [(400, 160, 1234, 37), (64, 16, 100, 200), (16, 5, 9, 3),
                                            (256, 64, 1000, 0)])
def test_signal_pad_matches_torch_pad_then_stft(pad_mode, n_fft, hop, T, pad):
    """torchaudio's pad: torch.nn.functional.pad with zeros, then torch.stft
    with its own center padding of the longer signal (both independent
    library routines, fp64).  pad > T and a tiny clip are included, so the
    reflection runs over the zeros."""
    rng = np.random.default_rng(T + pad)
    x = rng.standard_normal(T)
    P = oracle.pcm_power_frames(x, n_fft, hop, True, pad_mode, pad=pad)
    xt = torch.nn.functional.pad(torch.from_numpy(x)[None], (pad, pad), mode="constant", value=0.0)[0]
    S = torch.stft(xt, n_fft, hop_length=hop, window=torch.hann_window(n_fft, periodic=True, dtype=torch.float64),
                   center=True, pad_mode=pad_mode, return_complex=True)
    ref = (S.abs() ** 2).numpy().T
    assert P.shape == ref.shape
    assert P.shape[0] == oracle.num_frames(T, n_fft, hop, True, pad)
    assert np.max(np.abs(P - ref)) / np.max(ref) < 1e-12


def test_signal_pad_frame_counts():
    # T + 2 pad + 2 (n_fft // 2) samples: 480000 + 2 * 100 + 400 -> 3002 frames at hop 160
    assert oracle.num_frames(480000, 400, 160, True, 100) == 3002
    assert oracle.num_frames(480000, 400, 160, True, 79) == 3001
    assert oracle.num_frames(300, 400, 160, False, 50) == 1
    with pytest.raises(ValueError):
        oracle.num_frames(298, 400, 160, False, 50)


@pytest.mark.parametrize("W", [3, 64, 300, 400])
def test_normalized_window_closed_form(W):
    """The periodic Hann has sum_n w[n]^2 = 3 W / 8 (W >= 3), so the
    window-normalised power is the plain power times 8 / (3 W); the
    frame-length normalisation divides it by W."""
    n_fft = 400
    rng = np.random.default_rng(W)
    x = rng.standard_normal(3000)
    plain = oracle.pcm_power_frames(x, n_fft, 160, True, "reflect", 2.0, W)
    win = oracle.pcm_power_frames(x, n_fft, 160, True, "reflect", 2.0, W, normalized="window")
    fl = oracle.pcm_power_frames(x, n_fft, 160, True, "reflect", 2.0, W, normalized="frame_length")
    assert np.max(np.abs(win - plain * 8.0 / (3.0 * W))) / np.max(np.abs(win)) < 1e-12
    assert np.max(np.abs(fl - plain / W)) / np.max(np.abs(fl)) < 1e-12
    # magnitude (power 1): the factor enters before the exponent
    m1 = oracle.pcm_power_frames(x, n_fft, 160, True, "reflect", 1.0, W, normalized="window")
    p1 = oracle.pcm_power_frames(x, n_fft, 160, True, "reflect", 1.0, W)
    assert np.max(np.abs(m1 - p1 * math.sqrt(8.0 / (3.0 * W)))) / np.max(m1) < 1e-12


def test_mel_output_bin_centred_tone_closed_form():
    """Mel values of a bin-centred tone on interior frames:
    W[m, k0] (A N / 4)^2 + (W[m, k0-1] + W[m, k0+1]) (A N / 8)^2."""
    N, hop, A, k0, sr = 400, 160, 0.5, 25, 16000.0
    n = np.arange(20 * N)
    x = A * np.cos(2 * np.pi * k0 * n / N + 0.3)
    W = oracle.mel_filterbank(sr, N, 40)
    mel = oracle.mel_from_pcm(x[None], N, hop, W)[0]            # (40, F)
    ref = W[:, k0] * (A * N / 4) ** 2 + (W[:, k0 - 1] + W[:, k0 + 1]) * (A * N / 8) ** 2
    interior = mel[:, 3:-3]
    assert np.max(np.abs(interior - ref[:, None])) <= 1e-9 * np.max(ref)


def test_log_tail_of_mel_output():
    """The log-mel is the per-clip tail of the mel values, for both paths."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 5000)).astype(np.float32)
    W = oracle.mel_filterbank(16000.0, 400, 64)
    mel = oracle.mel_from_pcm(x, 400, 160, W)
    assert np.array_equal(oracle.from_pcm(x, 400, 160, W), oracle.log_mel_tail(mel))
    s = (rng.standard_normal((2, 7, 33)) + 1j * rng.standard_normal((2, 7, 33))).astype(np.complex64)
    Wl = rng.random((5, 33)).astype(np.float32)
    assert np.array_equal(oracle.from_stft(s, Wl), oracle.log_mel_tail(oracle.mel_from_stft(s, Wl)))
