"""Stream behaviour of the C ABI on the GPU: the lm_from_* calls only
enqueue work (no host wait for the device, also on a plan's first call, on
the first call after its filters change and on a call that grows its
workspace), and one plan used from two streams runs its calls in order.
Every output is checked against the fp64 oracle; the output map's own
invariants (largest value, floor) are checked exactly."""
from __future__ import annotations

import time

import numpy as np
import pytest

import lm_synth
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL32 = 1e-4
BUSY_CYCLES = 200_000_000       # a spin kernel of ~0.1 s at the shader clock


def lm():
    import stft_log_mel_amd
    return stft_log_mel_amd


def say(*a):
    print("[case]", *a, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def check(got, ref, tol, what):
    got = got.detach().float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    assert err.max() <= tol, f"{what}: max |err| {err.max():.3e}"


def _busy_then(call):
    """Queue a spin kernel on the current stream, then make `call`; returns
    (result, whether the spin kernel was still running when the call
    returned, host seconds the call took)."""
    torch.cuda.synchronize()
    torch.cuda._sleep(BUSY_CYCLES)
    ev = torch.cuda.Event()
    ev.record()
    t0 = time.perf_counter()
    res = call()
    dt = time.perf_counter() - t0
    running = not ev.query()
    return res, running, dt


def test_calls_never_wait_for_the_device():
    sr = 16000.0
    x1 = lm_synth.speech_pcm(2, 16000, sr, seed=201, as_int16=True)
    x2 = lm_synth.speech_pcm(6, 32000, sr, seed=202, as_int16=True)      # a larger call: workspace grows
    d1, d2 = to_dev(x1), to_dev(x2)
    torch.cuda.synchronize()
    plan = lm().Plan(400, 160, 128).set_mel(sr)
    say("first call (table upload, workspace)")
    out1, running, dt = _busy_then(lambda: plan.from_pcm(d1))
    assert running, f"first call waited for the device ({dt:.3f} s)"
    torch.cuda.synchronize()
    check(out1, oracle.from_pcm(x1, 400, 160, oracle.mel_filterbank(sr, 400, 128)), TOL32, "first call")

    say("first call after the filterbank changed (table upload)")
    plan.set_mel(sr, 20.0, 7600.0)
    out2, running, dt = _busy_then(lambda: plan.from_pcm(d1))
    assert running, f"call after set_mel waited for the device ({dt:.3f} s)"
    torch.cuda.synchronize()
    check(out2, oracle.from_pcm(x1, 400, 160, oracle.mel_filterbank(sr, 400, 128, 20.0, 7600.0)), TOL32,
          "after set_mel")

    say("workspace-growing call")
    out3, running, dt = _busy_then(lambda: plan.from_pcm(d2))
    assert running, f"workspace-growing call waited for the device ({dt:.3f} s)"
    torch.cuda.synchronize()
    check(out3, oracle.from_pcm(x2, 400, 160, oracle.mel_filterbank(sr, 400, 128, 20.0, 7600.0)), TOL32,
          "workspace growth")

    say("STFT entry: first call, device filterbank (row spans, workspace)")
    s = lm_synth.stft_speechlike(3, 500, 201, seed=203)
    W = lm_synth.lintri_filters(201, 64)
    ds, dW = to_dev(s), to_dev(W)
    p2 = lm().Plan(400, 160, 64)
    torch.cuda.synchronize()
    out4, running, dt = _busy_then(lambda: p2.from_stft(ds, dW))
    assert running, f"first STFT call waited for the device ({dt:.3f} s)"
    torch.cuda.synchronize()
    check(out4, oracle.from_stft(s, W), TOL32, "stft first call")


def test_one_plan_on_two_streams():
    """The module-level STFT helper keeps one plan per device; calls from two
    streams with different filterbanks share its workspace and row-span
    buffer.  The second stream's call must wait for the first's work (here
    held back by a spin kernel), so both outputs match the oracle."""
    s_a = lm_synth.stft_speechlike(2, 700, 201, seed=211)
    s_b = lm_synth.stft_speechlike(3, 400, 201, seed=212)
    W_a = lm_synth.lintri_filters(201, 80)
    W_b = lm_synth.lintri_filters(201, 48)
    da, db, dWa, dWb = to_dev(s_a), to_dev(s_b), to_dev(W_a), to_dev(W_b)
    st1, st2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    say("shared plan on two streams")
    for rep in range(3):
        with torch.cuda.stream(st1):
            torch.cuda._sleep(BUSY_CYCLES // 4)
            oa = lm().log_mel_spectrogram(da, dWa)
        with torch.cuda.stream(st2):
            ob = lm().log_mel_spectrogram(db, dWb)
        torch.cuda.synchronize()
        check(oa, oracle.from_stft(s_a, W_a), TOL32, f"stream 1, rep {rep}")
        check(ob, oracle.from_stft(s_b, W_b), TOL32, f"stream 2, rep {rep}")
    # the same for a PCM plan shared by two streams, second call larger
    sr = 16000.0
    xa = lm_synth.speech_pcm(2, 20000, sr, seed=213)
    xb = lm_synth.speech_pcm(5, 30000, sr, seed=214)
    dxa, dxb = to_dev(xa), to_dev(xb)
    plan = lm().Plan(400, 160, 80).set_mel(sr)
    torch.cuda.synchronize()
    with torch.cuda.stream(st1):
        torch.cuda._sleep(BUSY_CYCLES // 4)
        pa = plan.from_pcm(dxa)
    with torch.cuda.stream(st2):
        pb = plan.from_pcm(dxb)
    torch.cuda.synchronize()
    W = oracle.mel_filterbank(sr, 400, 80)
    check(pa, oracle.from_pcm(xa, 400, 160, W), TOL32, "pcm stream 1")
    check(pb, oracle.from_pcm(xb, 400, 160, W), TOL32, "pcm stream 2")


@pytest.mark.parametrize("path", ["pcm400", "generic", "big", "stft"])
def test_output_map_invariants_exact(path):
    """Per clip, the largest output equals the map of the largest mel value
    and every value is at least that minus 2 (the floor hi - 8 in output
    units), with floored values exactly equal to it: checked bit for bit in
    float32 on clamp-engaged clips."""
    sr = 16000.0
    if path == "stft":
        s = lm_synth.stft_speechlike(3, 300, 201, seed=221)
        s[0, 100:200] = 0                        # silent frames: floor binds
        s[1] *= np.float32(1e-3)
        out = lm().log_mel_spectrogram(to_dev(s), to_dev(lm_synth.lintri_filters(201, 80)))
    else:
        n_fft = {"pcm400": 400, "generic": 1024, "big": 8192}[path]
        x = lm_synth.speech_pcm(3, 48000, sr, seed=222)
        x[0, 12000:30000] = 0.0
        x[1] *= 1e-3
        out = lm().Plan(n_fft, n_fft // 4 if n_fft != 400 else 160, 80).set_mel(sr).from_pcm(to_dev(x))
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    say("output map invariants", path)
    for b in range(o.shape[0]):
        mx = np.float32(o[b].max())
        fl = np.float32(mx - np.float32(2.0))
        assert o[b].min() >= fl, (b, o[b].min(), fl)
        if b == 0:
            assert (o[b] == fl).sum() > 0, "the floor should bind on clip 0"


# ---------------------------------------------------------------------------
# Single pass (KBench page, perf_md: the clip-resident alternative to a second
# pass over the output)
# ---------------------------------------------------------------------------

def _run(x, n_fft, hop, n_mels, sr, single, out_dtype="f32", **kw):
    p = lm().Plan(n_fft, hop, n_mels, out_dtype=out_dtype, **kw).set_mel(sr).set_single_pass(single)
    out = p.from_pcm(to_dev(x))
    torch.cuda.synchronize()
    return out, p


@pytest.mark.parametrize("B,T,n_mels,in_dtype,out_dtype,pad_mode", [
    (8, 480000, 80, "f32", "f32", "reflect"),       # the 8 x 30 s float batch: 1504 sub-tiles
    (10, 480000, 128, "i16", "f32", "reflect"),     # 1880 sub-tiles of 128 bands
    (3, 40001, 200, "f32", "f16", "constant"),      # 200 bands, ragged length, fp16 out
    (1, 401, 40, "i16", "f32", "replicate"),        # one sub-tile
    (700, 3000, 64, "f32", "f32", "reflect"),       # many clips of two sub-tiles each
])
def test_single_pass_equals_two_pass_and_oracle(B, T, n_mels, in_dtype, out_dtype, pad_mode):
    sr = 16000.0
    x = lm_synth.speech_pcm(B, T, sr, seed=230 + B, as_int16=(in_dtype == "i16"))
    if T > 20000:
        x[0, T // 3: T // 2] = 0                          # the floor binds on clip 0
    if B > 1:
        x[1] = (x[1] // 100) if in_dtype == "i16" else x[1] * np.float32(1e-3)   # a quiet clip
    say("single pass", B, T, n_mels, in_dtype, out_dtype, pad_mode)
    one, p1 = _run(x, 400, 160, n_mels, sr, True, out_dtype, pad_mode=pad_mode)
    two, _ = _run(x, 400, 160, n_mels, sr, False, out_dtype, pad_mode=pad_mode)
    a, b = one.cpu().numpy(), two.cpu().numpy()
    # identical also for fp16: both round the same fp32 values to nearest even,
    # and rounding is monotone, so the fix-up's comparison of stored fp16
    # values with the floor's rounding decides as the fp32 comparison would
    assert np.array_equal(a, b), f"single vs two pass: max |diff| {np.abs(a.astype(np.float64) - b).max()}"
    # the single pass really ran: one launch per call, no fix-up
    p1.profile(True)
    p1.from_pcm(to_dev(x))
    torch.cuda.synchronize()
    p1.profile(False)
    prof = p1.profile_read()
    assert prof["main"]["count"] == 1 and prof["fixup"]["count"] == 0, prof
    n_check = min(B, 3)
    ref = oracle.from_pcm(x[:n_check], 400, 160, oracle.mel_filterbank(sr, 400, n_mels), pad_mode=pad_mode)
    check(one[:n_check], ref, TOL32 if out_dtype == "f32" else 2e-3, "single pass vs oracle")


def test_single_pass_repeated_calls_and_silence():
    """Back-to-back single-pass calls (the barrier and clip slots carry a
    per-call tag and are never cleared): a loud batch, then a silent one,
    then the loud one again, then batch sizes that change the grid."""
    sr = 16000.0
    loud = lm_synth.speech_pcm(4, 48000, sr, seed=240)
    silent = np.zeros((4, 48000), dtype=np.float32)
    p = lm().Plan(400, 160, 80).set_mel(sr).set_single_pass(True)
    W = oracle.mel_filterbank(sr, 400, 80)
    ref_loud = oracle.from_pcm(loud, 400, 160, W)
    say("single pass repeated")
    for rep in range(3):
        o1 = p.from_pcm(to_dev(loud))
        o2 = p.from_pcm(to_dev(silent))
        o3 = p.from_pcm(to_dev(loud[:1]))
        torch.cuda.synchronize()
        check(o1, ref_loud, TOL32, f"loud rep {rep}")
        assert np.abs(o2.cpu().numpy() + 1.5).max() <= 1e-6, "silence is -1.5 everywhere"
        check(o3, ref_loud[:1], TOL32, f"one clip rep {rep}")
