"""MI355X log-mel front end: Python binding over liblm.so.

Argument marshalling only: every step of the transform runs in the HIP
library behind ``include/lm.h``.  torch provides device memory and the
current stream; importing this package fails if the library is not built.

* ``Plan`` mirrors the C ABI (``lm_plan_create``, ``lm_plan_set_mel``,
  ``lm_from_pcm``, ``lm_from_stft`` ...).
* ``MelSpectrogram`` is the torchaudio-style wrapper of the flashmel page
  (section "Usage"): ``(..., time)`` float32 / int16 CUDA input ->
  ``(..., n_mels, n_frames)`` log-mel.
* ``log_mel_spectrogram(stft, mel_filters)`` is the KBench page's signature
  (section "reference_src"): ``(B, F, NF)`` complex64 -> ``(B, F, NM)``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

# torch first: its HIP runtime is then the process's one, and liblm.so's
# dependency (same soname) binds to it instead of loading a second runtime.
import torch  # noqa: F401  (device memory and streams only)

__all__ = [
    "LmError",
    "Plan",
    "MelSpectrogram",
    "log_mel_spectrogram",
    "lib_path",
    "LM_OK",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblm.so")

LM_OK, LM_ERR_INVALID_ARG, LM_ERR_UNSUPPORTED, LM_ERR_NO_FILTERS, LM_ERR_HIP, LM_ERR_OOM = 0, -1, -2, -3, -4, -5
_PAD = {"constant": 0, "reflect": 1, "replicate": 2, "circular": 3}
_DT = {"f32": 0, "f16": 1, "i16": 2}
_SCALE = {"slaney": 0, "htk": 1}
_NORM = {"slaney": 0, None: 1, "none": 1}
_OUTPUT = {"logmel": 0, "mel": 1}
_NORMALIZED = {None: 0, False: 0, "none": 0, True: 1, "window": 1, "frame_length": 2}
_FFT_VARIANT = {"auto": 0, "folded": 1, "paired": 2, "split_mfma": 3}

# Exported symbols and their C signatures (include/lm.h).
_c_int, _c_i64, _c_p, _c_f, _c_d = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_double
SIGNATURES = {
    "lm_plan_create": (_c_int, [ctypes.POINTER(_c_p), _c_int, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int]),
    "lm_plan_set_mel": (_c_int, [_c_p, _c_d, _c_d, _c_d, _c_int, _c_int]),
    "lm_plan_set_filters": (_c_int, [_c_p, _c_p, _c_int, _c_int]),
    "lm_plan_get_filters": (_c_int, [_c_p, _c_p, _c_int, _c_int]),
    "lm_plan_set_output": (_c_int, [_c_p, _c_int, _c_int]),
    "lm_plan_set_window": (_c_int, [_c_p, _c_int]),
    "lm_plan_set_pad": (_c_int, [_c_p, _c_i64]),
    "lm_plan_num_frames": (_c_i64, [_c_p, _c_i64]),
    "lm_from_pcm": (_c_int, [_c_p, _c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p]),
    "lm_from_stft": (_c_int, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_p, _c_p]),
    "lm_from_pcm_noalloc": (_c_int, [_c_p, _c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p]),
    "lm_plan_set_fft_variant": (_c_int, [_c_p, _c_int]),
    "lm_plan_set_single_pass": (_c_int, [_c_p, _c_int]),
    "lm_plan_set_memory_limit": (_c_int, [_c_p, _c_i64]),
    "lm_plan_memory_bytes": (_c_i64, [_c_p]),
    "lm_plan_describe": (_c_i64, [_c_p, _c_p, _c_i64]),
    "lm_plan_profile": (_c_int, [_c_p, _c_int]),
    "lm_plan_profile_read": (_c_int, [_c_p, ctypes.POINTER(_c_d), ctypes.POINTER(_c_i64)]),
    "lm_plan_destroy": (None, [_c_p]),
    "lm_status_string": (ctypes.c_char_p, [_c_int]),
    "lm_last_error": (ctypes.c_char_p, []),
}


def lib_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python stft_log_mel_amd/build.py` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


class LmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} [{_lib.lm_status_string(status).decode()}]")
        self.status = status


def _check(rc: int):
    if rc == LM_OK:
        return
    msg = _lib.lm_last_error().decode()
    if rc in (LM_ERR_INVALID_ARG, LM_ERR_UNSUPPORTED, LM_ERR_NO_FILTERS):
        raise ValueError(f"{msg} [{_lib.lm_status_string(rc).decode()}]")
    raise LmError(rc, msg)


def _torch():
    import torch
    return torch


def _stream_handle(device):
    """torch's current stream on `device` as a HIP stream handle."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)   # a direct lookup, ~0.3 us
    if raw is not None:
        return ctypes.c_void_p(raw(device.index))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_device(device, fn):
    """Call fn() with `device` current (switching only if it is not)."""
    torch = _torch()
    if torch.cuda.current_device() == device.index:
        return fn()
    with torch.cuda.device(device):
        return fn()


class Plan:
    """One lm_plan: transform shape, filterbank, device tables and workspace."""

    def __init__(self, n_fft: int, hop: int, n_mels: int, center: bool = True, pad_mode: str = "reflect",
                 power: float = 2.0, out_dtype: str = "f32"):
        if pad_mode not in _PAD:
            raise ValueError(f"pad_mode must be one of {sorted(_PAD)}")
        if out_dtype not in ("f32", "f16"):
            raise ValueError("out_dtype must be 'f32' or 'f16'")
        h = ctypes.c_void_p()
        _check(_lib.lm_plan_create(ctypes.byref(h), int(n_fft), int(hop), int(n_mels), int(bool(center)),
                                   _PAD[pad_mode], float(power), _DT[out_dtype]))
        self._h = h
        self.n_fft, self.hop, self.n_mels = int(n_fft), int(hop), int(n_mels)
        self.center, self.pad_mode, self.power, self.out_dtype = bool(center), pad_mode, float(power), out_dtype
        self.n_bins = self.n_fft // 2 + 1
        self.output = "logmel"
        self.lock = threading.Lock()

    # -- host-side configuration ------------------------------------------
    def set_mel(self, sample_rate: float, f_min: float = 0.0, f_max: float | None = None,
                mel_scale: str = "slaney", norm: str | None = "slaney") -> "Plan":
        if f_max is None:
            f_max = sample_rate / 2.0
        if mel_scale not in _SCALE or norm not in _NORM:
            raise ValueError("mel_scale must be 'slaney'|'htk' and norm 'slaney'|None")
        _check(_lib.lm_plan_set_mel(self._h, float(sample_rate), float(f_min), float(f_max),
                                    _SCALE[mel_scale], _NORM[norm]))
        return self

    def set_filters(self, dense) -> "Plan":
        a = np.ascontiguousarray(np.asarray(dense, dtype=np.float32))
        if a.ndim != 2:
            raise ValueError("filters must be 2-D (n_mels, n_fft//2 + 1)")
        _check(_lib.lm_plan_set_filters(self._h, a.ctypes.data, a.shape[0], a.shape[1]))
        return self

    def set_output(self, output: str = "logmel", normalized=None) -> "Plan":
        """output: "logmel" (normalised log-mel) or "mel" (mel values, no log
        tail); normalized: None/False, True/"window" or "frame_length"."""
        if output not in _OUTPUT or normalized not in _NORMALIZED:
            raise ValueError("output must be 'logmel'|'mel'; normalized None|True|'window'|'frame_length'")
        _check(_lib.lm_plan_set_output(self._h, _OUTPUT[output], _NORMALIZED[normalized]))
        self.output = output
        return self

    def set_window(self, win_length: int) -> "Plan":
        """Window of win_length samples, centred in the n_fft-point frame."""
        _check(_lib.lm_plan_set_window(self._h, int(win_length)))
        return self

    def set_pad(self, pad: int) -> "Plan":
        """Read each clip with pad zeros before and after it (torchaudio's pad)."""
        _check(_lib.lm_plan_set_pad(self._h, int(pad)))
        return self

    def set_fft_variant(self, variant: str = "auto") -> "Plan":
        """n_fft = 400 transform, for comparisons: "auto" (the matrix-core
        16 x 25 split where it applies), "folded" (200-point complex per
        frame) or "paired" (two frames per 400-point complex transform)."""
        if variant not in _FFT_VARIANT:
            raise ValueError(f"variant must be one of {sorted(_FFT_VARIANT)}")
        _check(_lib.lm_plan_set_fft_variant(self._h, _FFT_VARIANT[variant]))
        return self

    def set_single_pass(self, enable: bool = True) -> "Plan":
        """Use the one-launch (cooperative, grid-barrier) form of the per-clip
        floor where it applies; plans start with it off (two launches)."""
        _check(_lib.lm_plan_set_single_pass(self._h, int(bool(enable))))
        return self

    def set_memory_limit(self, n_bytes: int) -> "Plan":
        """Cap the device memory the plan holds (0: no cap); a call that
        would need more raises LmError (LM_ERR_OOM) before launching."""
        _check(_lib.lm_plan_set_memory_limit(self._h, int(n_bytes)))
        return self

    def memory_bytes(self) -> int:
        """Device bytes the plan holds now (tables and workspace)."""
        return int(_lib.lm_plan_memory_bytes(self._h))

    def describe(self) -> str:
        """The plan's choices as text: shape, filterbank, kernels, device, memory."""
        n = int(_lib.lm_plan_describe(self._h, None, 0))
        if n < 0:
            _check(n)
        buf = ctypes.create_string_buffer(n + 1)
        _lib.lm_plan_describe(self._h, buf, n + 1)
        return buf.value.decode()

    def get_filters(self) -> np.ndarray:
        a = np.zeros((self.n_mels, self.n_bins), dtype=np.float32)
        _check(_lib.lm_plan_get_filters(self._h, a.ctypes.data, self.n_mels, self.n_bins))
        return a

    def num_frames(self, n_samples: int) -> int:
        r = _lib.lm_plan_num_frames(self._h, int(n_samples))
        if r < 0:
            _check(int(r))
        return int(r)

    # -- launches ------------------------------------------------------------
    def from_pcm(self, pcm, out=None):
        """(B, T) float32 / int16 CUDA tensor -> (B, n_mels, F)."""
        torch = _torch()
        if pcm.dim() != 2:
            raise ValueError("pcm must be (n_clips, n_samples)")
        if pcm.dtype == torch.float32:
            in_dt = _DT["f32"]
        elif pcm.dtype == torch.int16:
            in_dt = _DT["i16"]
        else:
            raise ValueError("pcm must be float32 or int16")
        if not pcm.is_cuda or not pcm.is_contiguous():
            raise ValueError("pcm must be a contiguous CUDA tensor")
        B, T = pcm.shape
        F = self.num_frames(T)
        odt = torch.float16 if self.out_dtype == "f16" else torch.float32
        if out is None:
            out = torch.empty((B, self.n_mels, F), dtype=odt, device=pcm.device)
        elif (tuple(out.shape) != (B, self.n_mels, F) or out.dtype != odt or not out.is_contiguous()
              or out.device != pcm.device):
            raise ValueError("out has the wrong shape, dtype, layout or device")
        def call():
            with self.lock:
                return _lib.lm_from_pcm(self._h, ctypes.c_void_p(pcm.data_ptr()), in_dt, B, T,
                                        ctypes.c_void_p(out.data_ptr()), _stream_handle(pcm.device))
        _check(_on_device(pcm.device, call))
        return out

    def from_stft(self, stft, mel_filters=None, out=None):
        """(B, F, NF) complex64 CUDA tensor -> (B, F, NM)."""
        torch = _torch()
        if stft.dim() != 3 or stft.dtype != torch.complex64:
            raise ValueError("stft must be (B, F, NF) complex64")
        if not stft.is_cuda or not stft.is_contiguous():
            raise ValueError("stft must be a contiguous CUDA tensor")
        B, F, NF = stft.shape
        if mel_filters is not None:
            if (mel_filters.dim() != 2 or mel_filters.dtype != torch.float32 or not mel_filters.is_contiguous()
                    or mel_filters.device != stft.device or mel_filters.shape[1] != NF):
                raise ValueError("mel_filters must be contiguous (NM, NF) float32 on the stft's device")
            NM = mel_filters.shape[0]
            fptr = ctypes.c_void_p(mel_filters.data_ptr())
        else:
            NM = self.n_mels
            fptr = ctypes.c_void_p()
        odt = torch.float16 if self.out_dtype == "f16" else torch.float32
        if out is None:
            out = torch.empty((B, F, NM), dtype=odt, device=stft.device)
        elif (tuple(out.shape) != (B, F, NM) or out.dtype != odt or not out.is_contiguous()
              or out.device != stft.device):
            raise ValueError("out has the wrong shape, dtype, layout or device")
        def call():
            with self.lock:
                return _lib.lm_from_stft(self._h, ctypes.c_void_p(stft.data_ptr()), fptr, B, F, NF, NM,
                                         ctypes.c_void_p(out.data_ptr()), _stream_handle(stft.device))
        _check(_on_device(stft.device, call))
        return out

    # -- measurement -----------------------------------------------------------
    def profile(self, enable: bool = True):
        _check(_lib.lm_plan_profile(self._h, int(bool(enable))))

    def profile_read(self) -> dict:
        ms = (ctypes.c_double * 3)()
        cnt = (ctypes.c_int64 * 3)()
        _check(_lib.lm_plan_profile_read(self._h, ms, cnt))
        names = ("main", "fixup", "pack")
        return {n: {"ms": ms[i], "count": cnt[i]} for i, n in enumerate(names)}

    def close(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            _lib.lm_plan_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MelSpectrogram:
    """torchaudio-style mel transform (flashmel page, "Usage").

    Accepts the torchaudio ``MelSpectrogram`` arguments (``onesided=False``
    excepted).  ``output="logmel"`` (the default) gives
    the normalised log-mel; ``output="mel"`` the mel values themselves, as
    torchaudio does.  Output: ``(..., n_mels, n_frames)`` in float32 or
    float16 per ``dtype``.  Inference only.
    """

    def __init__(self, sample_rate: float = 16000, n_fft: int = 400, win_length: int | None = None,
                 hop_length: int | None = None, f_min: float = 0.0, f_max: float | None = None, pad: int = 0,
                 n_mels: int = 128, power: float = 2.0, normalized=False, center: bool = True,
                 pad_mode: str = "reflect", onesided: bool = True, norm: str | None = "slaney",
                 mel_scale: str = "slaney", dtype=None, output: str = "logmel"):
        torch = _torch()
        if normalized not in _NORMALIZED or output not in _OUTPUT:
            raise ValueError("normalized must be False|True|'window'|'frame_length'; output 'logmel'|'mel'")
        if not onesided:
            raise ValueError("only onesided=True (the mel projection needs a one-sided spectrum)")
        dtype = torch.float32 if dtype is None else dtype
        if dtype not in (torch.float32, torch.float16):
            raise ValueError("dtype must be torch.float32 or torch.float16")
        self.sample_rate = float(sample_rate)
        self.n_fft = int(n_fft)
        self.win_length = int(win_length) if win_length is not None else self.n_fft
        self.hop_length = int(hop_length) if hop_length is not None else self.win_length // 2
        self.normalized, self.output = normalized, output
        self.f_min, self.f_max = float(f_min), (float(f_max) if f_max is not None else self.sample_rate / 2)
        self.n_mels, self.power, self.center, self.pad_mode = int(n_mels), float(power), bool(center), pad_mode
        self.pad = int(pad)
        self.norm, self.mel_scale, self.dtype = norm, mel_scale, dtype
        self._plans = {}
        # validate now (host-only calls)
        self._plan_for(None)

    def _plan_for(self, device_index):
        p = self._plans.get(device_index)
        if p is None:
            p = Plan(self.n_fft, self.hop_length, self.n_mels, self.center, self.pad_mode, self.power,
                     "f16" if self.dtype == _torch().float16 else "f32")
            p.set_mel(self.sample_rate, self.f_min, self.f_max, self.mel_scale, self.norm)
            p.set_window(self.win_length)
            p.set_pad(self.pad)
            p.set_output(self.output, self.normalized)
            self._plans[device_index] = p
        return p

    def filters(self) -> np.ndarray:
        return self._plan_for(None).get_filters()

    def __call__(self, x):
        torch = _torch()
        if x.requires_grad and torch.is_grad_enabled():
            raise RuntimeError("inference only: no backward is implemented")
        if not x.is_cuda:
            raise ValueError("input must be a CUDA tensor")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        plan = self._plan_for(x.device.index)
        out = plan.from_pcm(x2)
        return out.reshape(*lead, out.shape[-2], out.shape[-1])


_stft_plans = {}
_stft_lock = threading.Lock()


def log_mel_spectrogram(stft, mel_filters):
    """(B, F, NF) complex64 STFT + (NM, NF) float32 filters -> (B, F, NM) float32."""
    torch = _torch()
    if stft.dim() == 2:
        return log_mel_spectrogram(stft.unsqueeze(0), mel_filters)[0]
    dev = stft.device.index
    with _stft_lock:
        p = _stft_plans.get(dev)
        if p is None:
            p = Plan(400, 160, 1, True, "reflect", 2.0, "f32")
            _stft_plans[dev] = p
    return p.from_stft(stft.contiguous(), mel_filters.to(torch.float32).contiguous())
