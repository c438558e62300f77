"""fp64 oracle of the KDA feature path and output gate.

TEST INFRASTRUCTURE ONLY: the tests and the bench's CPU-baseline leg are the
only callers; the HIP path never imports this module.

What it computes (plain numpy, fp64, loops over sequences only):
  * q, k: x -> ShortConv(k=4) -> Swish -> L2Norm;  v: x -> ShortConv -> Swish
    ("Kimi K3：架构、训练与推理系统研究" §3.2, the parameterisation diagram;
    devpress K3 walk-through §3.1, around Eq 2).  ShortConv is a causal
    depthwise convolution over time with 4 taps per channel; tap 3 multiplies
    the current token, tap 0 the token three steps back.  Before a sequence's
    first token the window holds the caller's carried state (the last three
    pre-convolution tokens, oldest first), or zeros; the pages keep that window
    as the ShortConv state ("Kimi K3：架构…" §3.4 table: the last few projected
    tokens, a window of length 4).
  * y = Sigmoid(g) * RMSNorm(o) per (token, head), with g the full-rank gate
    projection W_g x given as an input ("Kimi K3：架构…" §3.3; devpress §3.3,
    Eq 6).  RMSNorm over the head's dv channels: o / sqrt(mean(o^2) + eps) * w,
    w a per-channel weight shared by the heads.
The projections W_q, W_k, W_v, W_g, W_o themselves are not part of the op.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

TAPS = 4


def swish(u: np.ndarray) -> np.ndarray:
    """u * sigmoid(u)."""
    return u / (1.0 + np.exp(-u))


def sigmoid(u: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-u))


def l2norm(u: np.ndarray) -> np.ndarray:
    """Unit L2 norm over the last axis."""
    return u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True))


def short_conv(x: np.ndarray, w: np.ndarray, cu_seqlens, window: Optional[np.ndarray] = None
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Causal depthwise convolution of every packed sequence.

    x: [T, H, d]; w: [H, d, 4]; cu_seqlens: [N + 1]; window: [N, 3, H, d] (the
    three tokens before each sequence, oldest first) or None for zeros.
    Returns (y [T, H, d], window_out [N, 3, H, d]): window_out is the last
    three tokens of [window, sequence], the state for the next call."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    T, H, d = x.shape
    y = np.zeros((T, H, d))
    out = np.zeros((N, TAPS - 1, H, d))
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        prev = np.zeros((TAPS - 1, H, d)) if window is None else np.asarray(window[n], np.float64)
        seq = np.concatenate([prev, x[s:e]], axis=0)          # row i = token s - 3 + i
        for t in range(e - s):
            # taps 0..3 meet tokens t-3..t of the sequence, i.e. rows t..t+3
            y[s + t] = np.einsum("ihd,hdi->hd", seq[t:t + TAPS], w)
        out[n] = seq[-(TAPS - 1):]
    return y, out


def qkv_features(xq, xk, xv, wq, wk, wv, cu_seqlens, window=None):
    """The q/k/v feature path.  window: [N, 3, H, 2 dk + dv] (q, k, v channels
    of the carried pre-convolution tokens) or None.  Returns
    (q, k, v, window_out) in fp64."""
    dk, dv = xq.shape[-1], xv.shape[-1]
    part = lambda a, b: None if window is None else np.asarray(window, np.float64)[..., a:b]
    cq, oq = short_conv(xq, wq, cu_seqlens, part(0, dk))
    ck, ok = short_conv(xk, wk, cu_seqlens, part(dk, 2 * dk))
    cv, ov = short_conv(xv, wv, cu_seqlens, part(2 * dk, 2 * dk + dv))
    q = l2norm(swish(cq))
    k = l2norm(swish(ck))
    v = swish(cv)
    return q, k, v, np.concatenate([oq, ok, ov], axis=-1)


def rmsnorm(o: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """o / sqrt(mean(o^2) + eps) * w over the last axis."""
    o = np.asarray(o, np.float64)
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def output_gate(o: np.ndarray, g: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Sigmoid(g) * RMSNorm(o), o and g [T, H, dv], w [dv]."""
    return sigmoid(np.asarray(g, np.float64)) * rmsnorm(o, w, eps)
