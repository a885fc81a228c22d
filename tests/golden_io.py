"""Readers for the hand-derived fixtures under tests/golden/."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_stft_worked(name: str = "stft_tail_worked.txt"):
    """Returns (stft complex64 (B,F,NF), filters float32 (NM,NF), expected float64 (B,F,NM))."""
    filt_rows, stft_rows, exp_rows = [], [], []
    mode = None
    with open(os.path.join(GOLDEN, name)) as fh:
        for raw in fh:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "filters":
                mode = "filters"
                continue
            if tok[0] == "stft":
                mode = None
                stft_rows.append((int(tok[1]), int(tok[2]), [float(t) for t in tok[3:]]))
                continue
            if tok[0] == "expect":
                mode = None
                exp_rows.append((int(tok[1]), int(tok[2]), [float(t) for t in tok[3:]]))
                continue
            if mode == "filters":
                filt_rows.append([float(t) for t in tok])
    W = np.array(filt_rows, dtype=np.float32)
    NM, NF = W.shape
    B = 1 + max(r[0] for r in stft_rows)
    F = 1 + max(r[1] for r in stft_rows)
    stft = np.zeros((B, F, NF), dtype=np.complex64)
    for b, f, v in stft_rows:
        stft[b, f] = np.array(v[0::2]) + 1j * np.array(v[1::2])
    exp = np.full((B, F, NM), np.nan)
    for b, f, v in exp_rows:
        exp[b, f] = v
    assert not np.isnan(exp).any(), "fixture leaves an expected value unset"
    return stft, W, exp
