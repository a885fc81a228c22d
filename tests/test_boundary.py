"""C-ABI boundary on the CPU: the library loads, exports what include/lm.h
declares, validates arguments before any HIP call, and builds host tables
(filterbank, frame counts) that agree with the oracle.  No compute call is
made here, so these run without a GPU."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import stft_log_mel_amd as lm
from stft_log_mel_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lm.h")

OK, INVALID, UNSUPPORTED, NO_FILTERS = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ["lm_plan_create", "lm_from_pcm", "lm_from_stft", "lm_plan_destroy"]:
        assert must in names
    assert set(names) == set(lm.SIGNATURES), "binding signatures and header disagree"


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lm.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def _create(n_fft=400, hop=160, n_mels=80, center=1, pad=1, power=2.0, out=0):
    h = ctypes.c_void_p()
    rc = _lib.lm_plan_create(ctypes.byref(h), n_fft, hop, n_mels, center, pad, power, out)
    return rc, h


@pytest.mark.parametrize("n_fft", [400, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384])
def test_create_accepts_supported_sizes(n_fft):
    rc, h = _create(n_fft=n_fft)
    assert rc == OK
    _lib.lm_plan_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(n_fft=300), UNSUPPORTED), (dict(n_fft=32), UNSUPPORTED), (dict(n_fft=32768), UNSUPPORTED),
    (dict(n_fft=0), UNSUPPORTED), (dict(n_fft=-400), UNSUPPORTED), (dict(n_fft=401), UNSUPPORTED),
    (dict(hop=0), INVALID), (dict(hop=-1), INVALID),
    (dict(n_mels=0), INVALID), (dict(n_mels=257), INVALID),
    (dict(center=2), INVALID), (dict(pad=4), INVALID), (dict(pad=-1), INVALID),
    (dict(power=0.0), INVALID), (dict(power=-2.0), INVALID), (dict(power=float("inf")), INVALID),
    (dict(power=float("nan")), INVALID), (dict(out=2), INVALID), (dict(out=7), INVALID),
])
def test_create_rejects(kw, code):
    rc, h = _create(**kw)
    assert rc == code
    assert h.value is None
    assert _lib.lm_last_error().decode() != ""


def test_create_null_out_pointer():
    assert _lib.lm_plan_create(None, 400, 160, 80, 1, 1, 2.0, 0) == INVALID


def test_status_strings_and_destroy_null():
    for code in [0, -1, -2, -3, -4, -5]:
        assert _lib.lm_status_string(code).decode()
    _lib.lm_plan_destroy(None)


@pytest.mark.parametrize("sr,n_fft,n_mels,fmin,fmax,scale,norm", [
    (16000, 400, 80, 0, 8000, "slaney", "slaney"),
    (16000, 400, 128, 0, 8000, "slaney", "slaney"),
    (44100, 16384, 256, 0, 22050, "slaney", "slaney"),
    (16000, 512, 40, 20, 7600, "htk", None),
    (22050, 1024, 128, 0, 11025, "slaney", None),
])
def test_plan_filterbank_matches_oracle(sr, n_fft, n_mels, fmin, fmax, scale, norm):
    p = lm.Plan(n_fft, n_fft // 4, n_mels).set_mel(sr, fmin, fmax, scale, norm)
    got = p.get_filters().astype(np.float64)
    ref = oracle.mel_filterbank(sr, n_fft, n_mels, fmin, fmax, scale=scale, norm=norm)
    # fp32 rounding of fp64 weights; a weight the oracle puts at exactly 0
    # (a corner on a bin) may round to a tiny value either way
    assert np.max(np.abs(got - ref)) <= 2e-7 * np.max(ref)
    assert np.array_equal(got > 1e-6 * ref.max(), ref > 1e-6 * ref.max())


def test_set_mel_rejects():
    p = lm.Plan(400, 160, 80)
    for args in [(16000, 0, 8001), (16000, -1, 8000), (16000, 4000, 4000), (0, 0, 1), (16000, 5000, 4000)]:
        with pytest.raises(ValueError):
            p.set_mel(*args)


def test_set_filters_round_trip_and_packing():
    rng = np.random.default_rng(1)
    W = np.zeros((6, 33), dtype=np.float32)
    W[0, 3:7] = rng.random(4) + 0.1
    W[1, 5] = 2.0
    W[2, 10:20] = rng.random(10) + 0.1
    W[2, 14] = 0.0               # interior zero is kept inside the packed range
    W[4, 0] = 1.0
    W[5, 30:33] = 3.0            # row 3 stays all zero
    p = lm.Plan(64, 16, 6).set_filters(W)
    assert np.array_equal(p.get_filters(), W)
    with pytest.raises(ValueError):
        p.set_filters(np.ones((5, 33), np.float32))
    with pytest.raises(ValueError):
        p.set_filters(np.ones((6, 32), np.float32))
    bad = W.copy()
    bad[0, 0] = np.nan
    with pytest.raises(ValueError):
        p.set_filters(bad)


@pytest.mark.parametrize("T,n_fft,hop,center", [(480000, 400, 160, True), (441000, 16384, 4096, True),
                                               (400, 400, 160, False), (1000, 400, 160, False),
                                               (1, 64, 16, True), (12345, 1024, 333, True)])
def test_num_frames_matches_oracle(T, n_fft, hop, center):
    p = lm.Plan(n_fft, hop, 8, center=center)
    assert p.num_frames(T) == oracle.num_frames(T, n_fft, hop, center)


def test_num_frames_rejects_short_signal():
    p = lm.Plan(400, 160, 8, center=False)
    with pytest.raises(ValueError):
        p.num_frames(399)


def _plan_with_mel(**kw):
    rc, h = _create(**kw)
    assert rc == OK
    assert _lib.lm_plan_set_mel(h, 16000.0, 0.0, 8000.0, 0, 0) == OK
    return h


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case returns before any launch


def test_from_pcm_validation_before_any_hip_call():
    rc, bare = _create()
    assert _lib.lm_from_pcm(bare, FAKE, 0, 1, 16000, FAKE, None) == NO_FILTERS
    _lib.lm_plan_destroy(bare)
    h = _plan_with_mel()
    assert _lib.lm_from_pcm(None, FAKE, 0, 1, 16000, FAKE, None) == INVALID
    assert _lib.lm_from_pcm(h, FAKE, 1, 1, 16000, FAKE, None) == INVALID        # f16 input
    assert _lib.lm_from_pcm(h, FAKE, 0, -1, 16000, FAKE, None) == INVALID
    assert _lib.lm_from_pcm(h, FAKE, 0, 1, 0, FAKE, None) == INVALID
    assert _lib.lm_from_pcm(h, FAKE, 0, 1, 200, FAKE, None) == INVALID          # reflect needs T > 200
    assert _lib.lm_from_pcm(h, FAKE, 0, 1, 201, None, None) == INVALID         # NULL out
    assert _lib.lm_from_pcm(h, None, 0, 1, 201, FAKE, None) == INVALID         # NULL pcm
    assert _lib.lm_from_pcm(h, ctypes.c_void_p(0x10002), 0, 1, 16000, FAKE, None) == INVALID  # f32 misaligned
    assert _lib.lm_from_pcm(h, ctypes.c_void_p(0x10001), 2, 1, 16000, FAKE, None) == INVALID  # i16 misaligned
    assert _lib.lm_from_pcm(h, FAKE, 0, 0, 16000, None, None) == OK            # empty batch is a no-op
    _lib.lm_plan_destroy(h)
    h = _plan_with_mel(center=0)
    assert _lib.lm_from_pcm(h, FAKE, 0, 1, 399, FAKE, None) == INVALID
    _lib.lm_plan_destroy(h)
    h = _plan_with_mel(pad=3)
    assert _lib.lm_from_pcm(h, FAKE, 0, 1, 199, FAKE, None) == INVALID         # circular needs T >= 200
    _lib.lm_plan_destroy(h)


def test_from_stft_validation_before_any_hip_call():
    rc, h = _create(n_mels=80)
    assert _lib.lm_from_stft(h, FAKE, None, 1, 10, 201, 80, FAKE, None) == NO_FILTERS
    assert _lib.lm_from_stft(h, FAKE, FAKE, 1, 10, 0, 80, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, FAKE, FAKE, 1, 10, 8194, 80, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, FAKE, FAKE, 1, 10, 201, 0, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, FAKE, FAKE, 1, 10, 201, 257, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, FAKE, FAKE, -1, 10, 201, 80, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, FAKE, ctypes.c_void_p(0x10002), 1, 10, 201, 80, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, ctypes.c_void_p(0x10004), FAKE, 1, 10, 201, 80, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, None, FAKE, 1, 10, 201, 80, FAKE, None) == INVALID
    assert _lib.lm_from_stft(h, FAKE, FAKE, 0, 10, 201, 80, None, None) == OK
    assert _lib.lm_from_stft(h, FAKE, FAKE, 3, 0, 201, 80, None, None) == OK
    assert _lib.lm_plan_set_mel(h, 16000.0, 0.0, 8000.0, 0, 0) == OK
    assert _lib.lm_from_stft(h, FAKE, None, 1, 10, 129, 80, FAKE, None) == INVALID   # plan filters mismatch
    _lib.lm_plan_destroy(h)


def test_python_wrapper_rejects_unbuilt_options():
    with pytest.raises(ValueError):
        lm.MelSpectrogram(normalized="l2")
    with pytest.raises(ValueError):
        lm.MelSpectrogram(output="db")
    with pytest.raises(ValueError):
        lm.MelSpectrogram(n_fft=400, win_length=401)
    with pytest.raises(ValueError):
        lm.MelSpectrogram(onesided=False)
    with pytest.raises(ValueError):
        lm.MelSpectrogram(n_fft=300)
    with pytest.raises(ValueError):
        lm.Plan(400, 160, 80, pad_mode="mirror")
    m = lm.MelSpectrogram(sample_rate=16000, n_fft=400, hop_length=160, n_mels=80)
    ref = oracle.mel_filterbank(16000, 400, 80, 0, 8000)
    assert np.max(np.abs(m.filters() - ref)) <= 2e-7 * ref.max()


def test_binding_has_no_cpu_fallback():
    """The package's Python code launches nothing itself: every compute entry
    goes through the C library (the binding holds no transform arithmetic)."""
    src = open(os.path.join(ROOT, "stft_log_mel_amd", "__init__.py")).read()
    for word in ["fft", "log10", "hann", "oracle", "einsum", "matmul"]:
        text = src.lower().replace("n_fft", "").replace("rfft", "").replace("fft_variant", "")
        assert word not in text, word


def test_single_pass_validation():
    rc, h = _create()
    assert rc == OK
    assert _lib.lm_plan_set_single_pass(h, 1) == OK
    assert _lib.lm_plan_set_single_pass(h, 0) == OK
    assert _lib.lm_plan_set_single_pass(h, 2) == INVALID
    assert _lib.lm_plan_set_single_pass(None, 1) == INVALID
    _lib.lm_plan_destroy(h)


def test_fft_variant_validation():
    rc, h = _create()
    assert rc == OK
    for v in (0, 1, 2, 3):
        assert _lib.lm_plan_set_fft_variant(h, v) == OK
    for v in (-1, 4):
        assert _lib.lm_plan_set_fft_variant(h, v) == INVALID
    assert _lib.lm_plan_set_fft_variant(None, 0) == INVALID
    _lib.lm_plan_destroy(h)
    with pytest.raises(ValueError):
        lm.Plan(400, 160, 80).set_fft_variant("dense")


def test_set_output_and_window_validation():
    rc, h = _create()
    assert rc == OK
    assert _lib.lm_plan_set_output(h, 1, 2) == OK
    assert _lib.lm_plan_set_output(h, 2, 0) == INVALID
    assert _lib.lm_plan_set_output(h, 0, 3) == INVALID
    assert _lib.lm_plan_set_output(h, -1, 0) == INVALID
    assert _lib.lm_plan_set_window(h, 1) == OK
    assert _lib.lm_plan_set_window(h, 400) == OK
    assert _lib.lm_plan_set_window(h, 0) == INVALID
    assert _lib.lm_plan_set_window(h, 401) == INVALID
    assert _lib.lm_plan_set_output(None, 0, 0) == INVALID
    assert _lib.lm_plan_set_window(None, 10) == INVALID
    _lib.lm_plan_destroy(h)
    m = lm.MelSpectrogram(sample_rate=16000, n_fft=512, win_length=400, normalized=True, output="mel")
    assert m.hop_length == 200            # torchaudio's default: win_length // 2


def test_set_pad_validation_and_frame_counts():
    rc, h = _create()
    assert rc == OK
    assert _lib.lm_plan_set_pad(h, -1) == INVALID
    assert _lib.lm_plan_set_pad(h, (1 << 30) + 1) == INVALID
    assert _lib.lm_plan_set_pad(None, 0) == INVALID
    assert _lib.lm_plan_set_pad(h, 1 << 30) == OK
    assert _lib.lm_plan_set_pad(h, 100) == OK
    assert _lib.lm_plan_num_frames(h, 480000) == oracle.num_frames(480000, 400, 160, True, 100) == 3002
    _lib.lm_plan_destroy(h)
    rc, h = _create(center=0)
    assert _lib.lm_plan_set_pad(h, 50) == OK
    assert _lib.lm_plan_num_frames(h, 300) == 1       # 300 + 2 * 50 = 400 samples: one frame
    assert _lib.lm_plan_num_frames(h, 299) < 0
    _lib.lm_plan_destroy(h)
    m = lm.MelSpectrogram(sample_rate=16000, n_fft=400, hop_length=160, pad=37)
    assert m.pad == 37 and m._plan_for(None).num_frames(16000) == oracle.num_frames(16000, 400, 160, True, 37)
    with pytest.raises(Exception):
        lm.MelSpectrogram(pad=-3)


@pytest.mark.parametrize("n_fft,hop,variant,expect", [
    (400, 160, "auto", ["pcm400_kernel", "16-frame sub-tiles", "20 batches of 4 steps"]),
    (400, 160, "folded", ["pcm_logmel_kernel<400>:", "16 frames per workgroup", "(8 x 5 x 5)"]),
    (400, 160, "paired", ["pcm_logmel_kernel<400> (paired)", "two frames per 400-point"]),
    (400, 161, "auto", ["pcm_logmel_kernel<400>:"]),           # odd hop: no matrix-core path
    (1024, 256, "auto", ["pcm_logmel_kernel<1024>: 8 frames per workgroup"]),
    (16384, 4096, "auto", ["pcm_big_kernel<16384>"]),
])
def test_describe_names_the_kernel(n_fft, hop, variant, expect):
    p = lm.Plan(n_fft, hop, 128).set_mel(16000.0).set_fft_variant(variant)
    text = p.describe()
    for e in expect:
        assert e in text, (e, text)
    assert "device: not bound yet" in text
    assert "0 bytes held" in text and "limit none" in text


def test_describe_without_filters_and_with_a_wide_caller_filterbank():
    p = lm.Plan(400, 160, 256)
    assert "filters: not set" in p.describe()
    assert "lm_from_pcm:" not in p.describe()
    # a dense caller filterbank does not fit the matrix-core kernel's blocked table
    p.set_filters(np.ones((256, 201), dtype=np.float32))
    text = p.describe()
    assert "256 bands over 201 bins, 51456 weights, widest band 201 bins, 0 empty" in text
    assert "pcm_logmel_kernel<400>:" in text and "pcm400_kernel" not in text


def test_describe_buffer_sizing_and_truncation():
    rc, h = _create()
    assert rc == OK
    assert _lib.lm_plan_set_mel(h, 16000.0, 0.0, 8000.0, 1, 1) == OK
    n = _lib.lm_plan_describe(h, None, 0)
    assert n > 200
    full = ctypes.create_string_buffer(n + 1)
    assert _lib.lm_plan_describe(h, full, n + 1) == n
    assert len(full.value) == n
    short = ctypes.create_string_buffer(b"\xff" * 16, 16)
    assert _lib.lm_plan_describe(h, short, 10) == n
    assert short.raw[:10] == full.value[:9] + b"\0" and short.raw[10:] == b"\xff" * 6
    assert _lib.lm_plan_describe(h, None, 5) == INVALID
    assert _lib.lm_plan_describe(h, full, -1) == INVALID
    assert _lib.lm_plan_describe(None, full, n + 1) == INVALID
    _lib.lm_plan_destroy(h)


def test_memory_limit_validation():
    rc, h = _create()
    assert rc == OK
    assert _lib.lm_plan_memory_bytes(h) == 0
    assert _lib.lm_plan_memory_bytes(None) == -1
    assert _lib.lm_plan_set_memory_limit(h, -1) == INVALID
    assert _lib.lm_plan_set_memory_limit(None, 1) == INVALID
    assert _lib.lm_plan_set_memory_limit(h, 4096) == OK
    _lib.lm_plan_destroy(h)
    p = lm.Plan(400, 160, 80).set_mel(16000.0).set_memory_limit(1 << 20)
    assert "limit 1048576 bytes" in p.describe()
    with pytest.raises(ValueError):
        p.set_memory_limit(-5)
