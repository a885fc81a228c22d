"""Planted mistakes in the oracle (CPU only): each must trip at least one pin.

This shows the pins in test_oracle_pins.py are discriminating: a dropped
term, a wrong index, a wrong denominator or a wrong clamp scope anywhere in
the oracle fails one of them.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.logmel as L
from tests import test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(L, name, fn)
    monkeypatch.setattr(oracle, name, fn)


_orig = {n: getattr(L, n) for n in L.__all__}


def _tail_per_batch(mel):
    Lg = np.log10(np.maximum(mel, 1e-10))
    return (np.maximum(Lg, Lg.max() - 8.0) + 4.0) / 4.0


def _tail_per_frame(mel):
    Lg = np.log10(np.maximum(mel, 1e-10))
    hi = Lg.max(axis=-1, keepdims=True)        # one frame of an STFT-path clip
    return (np.maximum(Lg, hi - 8.0) + 4.0) / 4.0


def _tail_no_floor(mel):
    with np.errstate(divide="ignore"):
        Lg = np.log10(mel)
    hi = Lg.max(axis=tuple(range(1, Lg.ndim)), keepdims=True)
    return (np.maximum(Lg, hi - 8.0) + 4.0) / 4.0


def _tail_wrong_range(mel):
    Lg = np.log10(np.maximum(mel, 1e-10))
    hi = Lg.max(axis=tuple(range(1, Lg.ndim)), keepdims=True)
    return (np.maximum(Lg, hi - 80.0) + 4.0) / 4.0


def _tail_wrong_rescale(mel):
    Lg = np.log10(np.maximum(mel, 1e-10))
    hi = Lg.max(axis=tuple(range(1, Lg.ndim)), keepdims=True)
    return (np.maximum(Lg, hi - 8.0) + 4.0) * 4.0


def _hann_symmetric(N):
    n = np.arange(N, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * n / (N - 1))


def _rdft_index_slip(y, chunk=1024):
    y = np.asarray(y, dtype=np.float64)
    N = y.shape[-1]
    K = N // 2 + 1
    n = np.arange(N)
    k = np.arange(K)
    theta = 2.0 * np.pi * ((n[:, None] * (k[None, :] + 1)) % N) / N
    return (y @ np.cos(theta)) - 1j * (y @ np.sin(theta))


def _rdft_dropped_last_sample(y, chunk=1024):
    y = np.array(y, dtype=np.float64)
    y[..., -1] = 0.0
    return _orig["rdft_direct"](y, chunk)


def _pad_reflect_repeats_edge(x, n_fft, center, pad_mode):
    if pad_mode != "reflect" or not center:
        return _orig["pad_signal"](x, n_fft, center, pad_mode)
    p = n_fft // 2
    return np.concatenate([x[..., :p][..., ::-1], x, x[..., -p:][..., ::-1]], axis=-1)


def _frames_drop_last(xp, n_fft, hop):
    return _orig["frame_signal"](xp, n_fft, hop)[..., :-1, :]


def _frames_hop_slip(xp, n_fft, hop):
    return _orig["frame_signal"](xp, n_fft, hop + 1)


def _num_frames_drop_last(T, n_fft, hop, center, pad=0):
    return _orig["num_frames"](T, n_fft, hop, center, pad) - 1


def _zero_pad_left_only(x, pad):
    x = np.asarray(x, dtype=np.float64)
    return np.concatenate([np.zeros(x.shape[:-1] + (2 * pad,)), x], axis=-1)


def _zero_pad_reflects(x, pad):
    x = np.asarray(x, dtype=np.float64)
    if pad == 0:
        return x.copy()
    return np.pad(x, [(0, 0)] * (x.ndim - 1) + [(pad, pad)], mode="reflect")


def _fb_wrong_rise(sample_rate, n_fft, n_mels, f_min=0.0, f_max=None, scale="slaney", norm="slaney"):
    if f_max is None:
        f_max = sample_rate / 2.0
    fk = np.arange(n_fft // 2 + 1) * (sample_rate / n_fft)
    f_pts = L.mel_to_hz(np.linspace(L.hz_to_mel(f_min, scale), L.hz_to_mel(f_max, scale), n_mels + 2), scale)
    W = np.zeros((n_mels, fk.size))
    for m in range(n_mels):
        lo, mid, hi = f_pts[m], f_pts[m + 1], f_pts[m + 2]
        W[m] = np.maximum(0.0, np.minimum((fk - lo) / (hi - lo), (hi - fk) / (hi - mid)))
        if norm == "slaney":
            W[m] *= 2.0 / (hi - lo)
    return W


def _fb_no_norm(sample_rate, n_fft, n_mels, f_min=0.0, f_max=None, scale="slaney", norm="slaney"):
    return _orig["mel_filterbank"](sample_rate, n_fft, n_mels, f_min, f_max, scale, None)


def _decode_wrong_scale(x):
    x = np.asarray(x)
    if x.dtype == np.int16:
        return x.astype(np.float64) / 32767.0
    return x.astype(np.float64)


def _mel_scale_wrong_break(f, scale="slaney"):
    f = np.asarray(f, dtype=np.float64)
    if scale == "htk":
        return _orig["hz_to_mel"](f, scale)
    return np.where(f >= 700.0, 15.0 + np.log(np.maximum(f, 1e-300) / 1000.0) / (np.log(6.4) / 27.0),
                    f / (200.0 / 3.0))


def _power_magnitude(X, power=2.0):
    return np.abs(X)


def _window_off_by_one(n_fft, win_length=None):
    W = n_fft if win_length is None else int(win_length)
    w = np.zeros(n_fft, dtype=np.float64)
    left = (n_fft - W + 1) // 2            # rounds the offset up instead of down
    w[left:left + W] = L.hann_periodic(W) if W > 1 else 1.0
    return w


def _normalized_by_sum(window, normalized, win_length):
    if normalized in (None, False, "none"):
        return 1.0
    if normalized in (True, "window"):
        return 1.0 / float(np.sum(window))     # sum of w, not sqrt of sum of w^2
    return 1.0 / float(win_length) ** 0.5


MUTATIONS = [
    ("log_mel_tail", _tail_per_batch, [pins.test_worked_example_fixture]),
    ("log_mel_tail", _tail_per_frame, [pins.test_worked_example_fixture]),
    ("log_mel_tail", _tail_no_floor, [pins.test_worked_example_fixture]),
    ("log_mel_tail", _tail_wrong_range, [pins.test_worked_example_fixture]),
    ("log_mel_tail", _tail_wrong_rescale, [pins.test_worked_example_fixture]),
    ("hann_periodic", _hann_symmetric, [pins.test_hann_is_periodic, pins.test_bin_centred_tone_closed_form]),
    ("rdft_direct", _rdft_index_slip, [lambda: pins.test_rdft_matches_library_fft(64)]),
    ("rdft_direct", _rdft_dropped_last_sample, [lambda: pins.test_parseval(16)]),
    ("pad_signal", _pad_reflect_repeats_edge,
     [lambda: pins.test_framing_padding_window_match_torch_stft("reflect", 64, 16, 1000)]),
    ("frame_signal", _frames_drop_last,
     [lambda: pins.test_framing_padding_window_match_torch_stft("reflect", 64, 16, 1000)]),
    ("frame_signal", _frames_hop_slip,
     [lambda: pins.test_framing_padding_window_match_torch_stft("constant", 64, 16, 1000)]),
    ("num_frames", _num_frames_drop_last, [pins.test_frame_counts]),
    ("zero_pad_signal", _zero_pad_left_only,
     [lambda: pins.test_signal_pad_matches_torch_pad_then_stft("reflect", 400, 160, 1234, 37)]),
    ("zero_pad_signal", _zero_pad_reflects,
     [lambda: pins.test_signal_pad_matches_torch_pad_then_stft("constant", 16, 5, 9, 3)]),
    ("mel_filterbank", _fb_wrong_rise,
     [lambda: pins.test_filterbank_invariants(16000, 400, 80, 8000, "slaney")]),
    ("mel_filterbank", _fb_no_norm,
     [lambda: pins.test_filterbank_invariants(16000, 400, 80, 8000, "slaney")]),
    ("decode_pcm", _decode_wrong_scale, [pins.test_int16_decode_is_exact_scaling]),
    ("hz_to_mel", _mel_scale_wrong_break, [pins.test_slaney_scale_closed_forms]),
    ("power_spectrum", _power_magnitude, [pins.test_power_general_exponent,
                                          lambda: pins.test_parseval(16)]),
    ("frame_window", _window_off_by_one, [lambda: pins.test_short_window_matches_torch_stft(512, 257, 128)]),
    ("normalization_factor", _normalized_by_sum, [lambda: pins.test_normalized_window_closed_form(300)]),
]


@pytest.mark.parametrize("name,mutant,checks", MUTATIONS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, mutant, checks):
    _patch(monkeypatch, name, mutant)
    caught = 0
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, f"planted mistake in {name} ({mutant.__name__}) passed every pin"
