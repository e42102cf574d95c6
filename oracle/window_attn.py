"""fp64 CPU oracle of the softmax block's sliding-window + persistent-sink attention -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use this
module; the GPU library never loads it and the two share no code.

What it computes.  SANA-Streaming pages, Chinese summary, "Core method": the hybrid DiT places
5 softmax-attention blocks among its 15 GDN blocks, and each softmax block attends over a
sliding window plus persistent sink tokens, so its memory stays fixed (the window has a fixed
size) while chunk boundaries keep token-level correspondence; "Prerequisites": softmax
attention forms token interactions from dot products normalised by a softmax, and its KV cache
would otherwise grow with the sequence.  The pages give neither sizes nor masks; the readings
taken here are:

  - the sink is the first ``n_sink`` tokens the stream ever produced, kept for the stream's life;
  - the window is the newest ``n_window`` tokens produced after the sink (older ones are evicted);
  - every query of a chunk sees the sink, the window, and all tokens of its own chunk (no mask
    inside a chunk: the chunk's latent frames are denoised together);
  - logits are ``scale * q.k`` with ``scale = 1/sqrt(d)`` unless given;
  - after a committed call the chunk's tokens join the stream's history; an uncommitted call
    (a denoising step that will be replayed) leaves the history as it was.

The history is kept whole and the visible set is taken from the definition above on every call:
slow, and plainly checkable.
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q k^T) v for one head: q [n, d], k [m, d], v [m, dv] -> [n, dv] in fp64.

    The row maximum is subtracted before exponentiating (the softmax is unchanged by it)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    logits = scale * (q @ k.T)
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def visible_tokens(history: int, n_sink: int, n_window: int) -> list:
    """Indices (into the stream's history of ``history`` tokens) that a new chunk attends to:
    the first ``n_sink`` tokens, then the newest ``n_window`` of those that came after them."""
    sink = list(range(min(history, n_sink)))
    start = max(n_sink, history - n_window)
    return sink + list(range(start, history))


class SinkWindowAttention:
    """One softmax block's attention state for B streams x H heads (history kept in fp64)."""

    def __init__(self, n_sink: int, n_window: int, scale: float | None = None):
        if n_sink < 0 or n_window < 0:
            raise ValueError("negative cache size")
        self.n_sink = n_sink
        self.n_window = n_window
        self.scale = scale
        self.k_hist = None   # [B, N, H, d]
        self.v_hist = None

    @property
    def history(self) -> int:
        return 0 if self.k_hist is None else self.k_hist.shape[1]

    def chunk(self, q, k, v, commit: bool = True) -> np.ndarray:
        """Attention of a chunk of T tokens: k [B, T, H, d], v [B, T, H, dv] -> o [B, Tq, H, dv] for
        the queries q [B, Tq, H, d] (Tq = T for the whole chunk; fewer rows give those rows' outputs)."""
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        B, Tq, H, d = q.shape
        scale = self.scale if self.scale is not None else 1.0 / np.sqrt(d)
        idx = visible_tokens(self.history, self.n_sink, self.n_window)
        o = np.empty((B, Tq, H, v.shape[-1]), np.float64)
        for b in range(B):
            for h in range(H):
                if idx:
                    keys = np.concatenate([self.k_hist[b, idx, h], k[b, :, h]])
                    vals = np.concatenate([self.v_hist[b, idx, h], v[b, :, h]])
                else:
                    keys, vals = k[b, :, h], v[b, :, h]
                o[b, :, h] = attend(q[b, :, h], keys, vals, scale)
        if commit:
            if self.k_hist is None:
                self.k_hist, self.v_hist = k.copy(), v.copy()
            else:
                self.k_hist = np.concatenate([self.k_hist, k], axis=1)
                self.v_hist = np.concatenate([self.v_hist, v], axis=1)
        return o
