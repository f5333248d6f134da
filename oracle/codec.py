"""Plain CPU definition of the codec decoder's two convolution kinds (numpy,
float64 by default).

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this package.

Source: "qwen3-tts-hip OPTIMIZATION_LOG", codec entries: the decoder's time
goes to a dilated causal 1-D convolution and a transposed 1-D convolution;
the transposed one is rewritten by output phase p (stride s) as
out[t*s + p] = in[t] W[p] + in[t-1] W[p+s] + bias.  Layout is channel-major
([channels, frames], the NEON page's sequence layout).  Readings (listed in
the design notes): a transposed convolution has kernel 2s (the two taps the
phase formula names) and keeps the T*s outputs whose sources are
in[0..T-1] (the trailing s samples of the full output are dropped, a causal
trim); the causal convolution pads only on the left with zeros.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def conv1d_causal(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray],
                  dilation: int = 1) -> np.ndarray:
    """y[co, t] = b[co] + sum over ci, j of w[co, ci, j] x[ci, t - (K-1-j) d],
    with x = 0 before t = 0.  x [Cin, T], w [Cout, Cin, K] -> y [Cout, T]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    cin, T = x.shape
    cout, cin2, K = w.shape
    assert cin == cin2
    y = np.zeros((cout, T))
    for j in range(K):
        shift = (K - 1 - j) * dilation
        if shift >= T:
            continue
        xs = np.zeros_like(x)
        xs[:, shift:] = x[:, :T - shift]
        y += w[:, :, j] @ xs
    if b is not None:
        y += np.asarray(b, np.float64)[:, None]
    return y


def transconv1d(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray], stride: int) -> np.ndarray:
    """Transposed convolution by its definition: every input frame t scatters
    w[ci, :, k] x[ci, t] onto output t*s + k (k < K); bias added; the first
    T*s outputs kept.  x [Cin, T], w [Cin, Cout, K] (K = 2s) -> [Cout, T*s]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    cin, T = x.shape
    cin2, cout, K = w.shape
    assert cin == cin2
    full = np.zeros((cout, (T - 1) * stride + K))
    for t in range(T):
        full[:, t * stride:t * stride + K] += np.einsum("ick,i->ck", w, x[:, t])
    y = full[:, :T * stride]
    if b is not None:
        y = y + np.asarray(b, np.float64)[:, None]
    return y
