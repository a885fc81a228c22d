"""Properties of the seeded input generators (CPU only).

The generators hold none of the transform's arithmetic; these checks pin
them to the workload descriptions they follow, so that a change in a
generator shows here rather than as a drift in the parity inputs.
"""
import numpy as np
import pytest

import lm_synth


@pytest.mark.parametrize("NF,NM", [(201, 80), (201, 128), (33, 1), (9, 7), (2, 3)])
def test_lintri_filters_are_hats_on_equal_spacing(NF, NM):
    W = lm_synth.lintri_filters(NF, NM).astype(np.float64)
    assert W.shape == (NM, NF) and W.dtype == np.float64
    d = (NF - 1) / (NM + 1)
    k = np.arange(NF)
    for m in range(NM):
        peak = (m + 1) * d
        row = W[m]
        assert row.min() >= 0.0 and row.max() <= 1.0
        # zero (up to the rounding of the foot itself) at and beyond the neighbouring points
        assert np.all(row[(k <= peak - d) | (k >= peak + d)] <= 1e-12)
        # linear on each side: equal steps between integer bins inside a flank
        up = k[(k > peak - d) & (k <= peak)]
        if len(up) >= 2:
            np.testing.assert_allclose(np.diff(row[up]), 1.0 / d, rtol=1e-6)
        down = k[(k >= peak) & (k < peak + d)]
        if len(down) >= 2:
            np.testing.assert_allclose(np.diff(row[down]), -1.0 / d, rtol=1e-6)
    # neighbouring hats sum to one between the first and the last peak
    inner = (k >= d) & (k <= NM * d)
    np.testing.assert_allclose(W.sum(axis=0)[inner], 1.0, atol=1e-6)


def test_lintri_filters_integer_peaks_reach_one():
    # NF - 1 = 2 (NM + 1): every peak falls on an even bin
    W = lm_synth.lintri_filters(2 * 9 + 1, 8)
    for m in range(8):
        assert W[m, 2 * (m + 1)] == 1.0
        assert W[m, 2 * (m + 1) + 1] == 0.5 and W[m, 2 * (m + 1) - 1] == 0.5


def test_lintri_filters_degenerate():
    assert not lm_synth.lintri_filters(1, 4).any()
    with pytest.raises(ValueError):
        lm_synth.lintri_filters(0, 4)


def test_stft_speechlike_is_seeded_and_scaled():
    B, F, NF = 3, 4000, 201
    s = lm_synth.stft_speechlike(B, F, NF, seed=9)
    assert s.shape == (B, F, NF) and s.dtype == np.complex64
    assert np.array_equal(s, lm_synth.stft_speechlike(B, F, NF, seed=9))
    assert not np.array_equal(s, lm_synth.stft_speechlike(B, F, NF, seed=10))
    p = np.abs(s.astype(np.complex128)) ** 2
    # tilt: E|X|^2 = 2 level^2 tilt^2, so the frame-averaged power falls by
    # e^-6 from bin 0 to bin NF (about 26 dB)
    col = p.mean(axis=(0, 1))
    slope = np.polyfit(np.arange(NF), np.log(col), 1)[0]
    assert abs(slope - (-6.0 / NF)) < 0.05 * 6.0 / NF
    # level: per-frame power / (2 sum tilt^2) estimates level^2 in [0.05^2, 1.05^2)
    tilt2 = np.exp(-6.0 * np.arange(NF) / NF)
    lev2 = p.sum(axis=2) / (2.0 * tilt2.sum())
    assert lev2.min() > 0.5 * 0.05 ** 2 and lev2.max() < 1.5 * 1.05 ** 2
    # E[level^2] = E[(0.05 + u^2)^2] = 0.0025 + 0.1/3 + 1/5
    assert abs(lev2.mean() / (0.0025 + 0.1 / 3 + 0.2) - 1.0) < 0.03
    # real and imaginary parts: independent, zero mean, equal power
    re, im = s.real.astype(np.float64), s.imag.astype(np.float64)
    assert abs(np.mean(re * im)) < 0.01 * np.mean(re * re)
    assert abs(np.mean(re * re) / np.mean(im * im) - 1.0) < 0.02
