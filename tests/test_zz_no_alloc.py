"""lm_from_pcm_noalloc through the C ABI: the same results as lm_from_pcm
(and the fp64 oracle) on two calls in a row, the second with a smaller
input, its workspace being a fixed device array instead of plan memory."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import lm_synth
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

LM_F32, LM_I16 = 0, 2
LM_ERR_INVALID_ARG, LM_ERR_UNSUPPORTED = -1, -2


def say(*a):
    print("[case]", *a, flush=True)


def _call(lib, fn, plan, x, out):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    in_dt = LM_I16 if x.dtype == torch.int16 else LM_F32
    return getattr(lib, fn)(plan._h, ctypes.c_void_p(x.data_ptr()), in_dt, x.shape[0], x.shape[1],
                            ctypes.c_void_p(out.data_ptr()), stream)


@pytest.mark.parametrize("in_dtype,n_fft,hop,n_mels,single", [("i16", 400, 160, 128, False),
                                                              ("f32", 400, 160, 80, False),
                                                              ("f32", 400, 160, 80, True),
                                                              ("f32", 1024, 256, 128, False)])
def test_noalloc_matches_lm_from_pcm(in_dtype, n_fft, hop, n_mels, single):
    import stft_log_mel_amd as lm
    lib = lm._lib
    sr = 16000.0
    i16 = in_dtype == "i16"
    plan = lm.Plan(n_fft, hop, n_mels).set_mel(sr).set_single_pass(single)
    W = oracle.mel_filterbank(sr, n_fft, n_mels)
    # the plan's tables go to the device with one ordinary call
    warm = torch.from_numpy(lm_synth.speech_pcm(1, 8000, sr, seed=300, as_int16=i16)).cuda()
    plan.from_pcm(warm)
    for k, (B, T) in enumerate([(6, 96000), (3, 40001)]):      # second call smaller
        x = lm_synth.speech_pcm(B, T, sr, seed=301 + k, as_int16=i16)
        x[0, T // 4: T // 2] = 0                               # the floor binds on clip 0
        dx = torch.from_numpy(x).cuda()
        F = plan.num_frames(T)
        out_a = torch.full((B, n_mels, F), float("nan"), device="cuda")
        out_b = torch.full((B, n_mels, F), float("nan"), device="cuda")
        say("noalloc", in_dtype, n_fft, "call", k, (B, T))
        assert _call(lib, "lm_from_pcm", plan, dx, out_a) == 0
        assert _call(lib, "lm_from_pcm_noalloc", plan, dx, out_b) == 0, lib.lm_last_error().decode()
        torch.cuda.synchronize()
        a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.array_equal(a, b), f"max |diff| {np.nanmax(np.abs(a - b))}"
        ref = oracle.from_pcm(x, n_fft, hop, W)
        err = np.abs(b.astype(np.float64) - ref).max()
        assert err <= 1e-4, err


def test_noalloc_rejects_what_it_cannot_do():
    import stft_log_mel_amd as lm
    lib = lm._lib
    sr = 16000.0
    x = torch.zeros((2, 16000), dtype=torch.int16, device="cuda")
    out = torch.empty((2, 128, 101), device="cuda")
    fresh = lm.Plan(400, 160, 128).set_mel(sr)
    say("noalloc: plan without device tables")
    assert _call(lib, "lm_from_pcm_noalloc", fresh, x, out) == LM_ERR_INVALID_ARG
    fresh.from_pcm(x, out=out)
    fresh.set_mel(sr, 30.0, 7000.0)                           # tables out of date again
    assert _call(lib, "lm_from_pcm_noalloc", fresh, x, out) == LM_ERR_INVALID_ARG
    fresh.from_pcm(x, out=out)
    assert _call(lib, "lm_from_pcm_noalloc", fresh, x, out) == 0
    say("noalloc: a call beyond the fixed workspace")
    big_clips = 2000                                           # 2000 x 1 s: 101 frames -> 7 sub-tiles x 36 floats each
    xb = torch.zeros((big_clips, 16000), dtype=torch.int16, device="cuda")
    ob = torch.empty((big_clips, 128, 101), device="cuda")
    # needs 2000 * 7 * 36 = 504000 floats: fits; 10x the clips does not
    assert _call(lib, "lm_from_pcm_noalloc", fresh, xb, ob) == 0
    xh = torch.zeros((20000, 16000), dtype=torch.int16, device="cuda")
    oh = torch.empty((20000, 128, 101), device="cuda")         # full size, though the call is rejected on the host
    assert _call(lib, "lm_from_pcm_noalloc", fresh, xh, oh) == LM_ERR_UNSUPPORTED
    assert "fixed workspace" in lib.lm_last_error().decode()
    torch.cuda.synchronize()
