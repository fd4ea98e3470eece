"""Float64 brute force for tiny shapes (TEST INFRASTRUCTURE ONLY).

Builds the explicit nL x nL attention mask directly from the pages' 1-based
index maps and evaluates masked softmax attention with NumPy matrix products.
It is deliberately written differently from ``hd_oracle.c`` (1-based positions,
a materialised mask, whole-matrix products) so the two can check each other.

Source: WeLM blog "Hidden Decoding at Scale", section "Stream-Factorized
Attention": i(t) = ceil(t/n), s(t) = (t-1) mod n + 1 for 1-based t, and
Figure 2: (a) full cross-stream layers use the standard causal mask, (b) local
cross-stream layers a causal sliding window, (c) intra-stream layers are causal
within a stream with streams invisible to one another.

Readings taken where the pages are silent: the diagonal is visible in every
mask; a window of W tokens keeps i(t_q) - i(t_k) < W for intra layers and
t_q - t_k < n*W expanded positions for cross layers; W = 0 means no window.
"""
import math

import numpy as np


def token_index(t, n):
    """i(t) = ceil(t / n) for 1-based expanded position t."""
    return -(-t // n)


def stream_index(t, n):
    """s(t) = (t - 1) mod n + 1 for 1-based expanded position t."""
    return (t - 1) % n + 1


def mask(n, L, mode, window=0):
    """Boolean [nL, nL] mask, entry [tq-1, tk-1] True when tq may attend tk."""
    t = np.arange(1, n * L + 1)
    tq, tk = t[:, None], t[None, :]
    if mode == 0:  # intra-stream, Figure 2(c)
        m = (stream_index(tq, n) == stream_index(tk, n)) & (token_index(tk, n) <= token_index(tq, n))
        if window:
            m &= token_index(tq, n) - token_index(tk, n) < window
    else:  # cross-stream, Figure 2(a) / (b)
        m = tk <= tq
        if window:
            m &= tq - tk < n * window
    return m


def attention(q, k, v, n, mode, window=0, scale=0.0):
    """q [B, nL, Hq, d], k/v [B, nL, Hkv, d] (any float dtype) -> float64 o, lse.

    lse has shape [B, Hq, nL] and holds log(sum(exp(scores))) over visible keys."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nL, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    if scale <= 0:
        scale = 1.0 / math.sqrt(d)
    m = mask(n, nL // n, mode, window)
    o = np.empty_like(q)
    lse = np.empty((B, Hq, nL))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h, :] @ k[b, :, h // g, :].T)
            s = np.where(m, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            o[b, :, h, :] = (p / den) @ v[b, :, h // g, :]
            lse[b, h, :] = (mx + np.log(den))[:, 0]
    return o, lse
