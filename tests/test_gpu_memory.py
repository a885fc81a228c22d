"""The plan's device-memory cap on the GPU: a call that would pass it fails
with LM_ERR_OOM before anything is allocated or launched (the output keeps
its contents and the plan stays usable), a buffer grows to exactly what a
call needs when doubling would pass the cap, and results under a cap equal
the oracle's."""
from __future__ import annotations

import numpy as np
import pytest

import lm_synth
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL32 = 1e-4
LM_ERR_OOM = -5


def lm():
    import stft_log_mel_amd
    return stft_log_mel_amd


def say(*a):
    print("[case]", *a, flush=True)


def oracle_pcm(x, n_fft, hop, n_mels, sr):
    W = oracle.mel_filterbank(sr, n_fft, n_mels, 0.0, sr / 2)
    return oracle.from_pcm(x, n_fft, hop, W)


@pytest.mark.parametrize("n_fft,hop", [(400, 160), (1024, 256)])
def test_memory_cap_fails_cleanly_then_fits_exactly(n_fft, hop):
    say("memory cap", n_fft, hop)
    sr = 16000.0
    assert lm().LM_ERR_OOM == LM_ERR_OOM
    x = lm_synth.speech_pcm(3, 24000, sr, seed=301)
    xd = torch.from_numpy(x).to("cuda:0")
    p = lm().Plan(n_fft, hop, 64).set_mel(sr).set_memory_limit(4096)
    out = torch.full((3, 64, p.num_frames(24000)), 7.0, device="cuda:0")
    with pytest.raises(lm().LmError) as ei:
        p.from_pcm(xd, out=out)
    assert ei.value.status == LM_ERR_OOM
    assert "device-memory limit" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call must not write its output"
    assert p.memory_bytes() == 0

    # no cap: the call runs and the plan holds its tables and workspace
    p.set_memory_limit(0)
    p.from_pcm(xd, out=out)
    torch.cuda.synchronize()
    ref = oracle_pcm(x, n_fft, hop, 64, sr)
    assert np.abs(out.cpu().numpy().astype(np.float64) - ref).max() <= TOL32
    held = p.memory_bytes()
    assert held > 0

    # capped at what it holds: the same batch runs again, a larger one
    # (more statistics) is refused and leaves its output alone
    p.set_memory_limit(held)
    out2 = torch.full_like(out, 3.0)
    p.from_pcm(xd, out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    x6 = lm_synth.speech_pcm(6, 24000, sr, seed=302)
    out6 = torch.full((6, 64, p.num_frames(24000)), 5.0, device="cuda:0")
    with pytest.raises(lm().LmError) as ei:
        p.from_pcm(torch.from_numpy(x6).to("cuda:0"), out=out6)
    assert ei.value.status == LM_ERR_OOM
    torch.cuda.synchronize()
    assert bool((out6 == 5.0).all())
    assert p.memory_bytes() == held
    p.close()


def test_growth_under_a_cap_takes_exactly_what_the_call_needs():
    """Doubling would pass the cap, the exact need does not: the workspace
    grows to the need and the result is right."""
    say("memory cap exact growth")
    sr = 16000.0
    short = lm_synth.speech_pcm(1, 48000, sr, seed=311)
    longer = lm_synth.speech_pcm(1, 64000, sr, seed=312)   # 4/3 of the statistics: less than double
    # what a fresh plan holds after the longer clip alone: tables + its exact need
    q = lm().Plan(400, 160, 80).set_mel(sr)
    q.from_pcm(torch.from_numpy(longer).to("cuda:0"))
    torch.cuda.synchronize()
    exact = q.memory_bytes()
    q.close()
    p = lm().Plan(400, 160, 80).set_mel(sr)
    p.from_pcm(torch.from_numpy(short).to("cuda:0"))
    torch.cuda.synchronize()
    assert p.memory_bytes() < exact
    p.set_memory_limit(exact)
    out = p.from_pcm(torch.from_numpy(longer).to("cuda:0"))
    torch.cuda.synchronize()
    ref = oracle_pcm(longer, 400, 160, 80, sr)
    assert np.abs(out.cpu().numpy().astype(np.float64) - ref).max() <= TOL32
    assert p.memory_bytes() == exact
    assert f"{exact} bytes held" in p.describe() and f"limit {exact} bytes" in p.describe()
    p.close()
