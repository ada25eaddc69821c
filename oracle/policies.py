"""A second schedule generator: condensed scales plus a window of local
scales, wider in cache-demanding layers (oracle).

Test infrastructure only.

What the pages fix (the AMS-KV paper's abstract, as listed on the
kv-cache-management page): attending to tokens of local (recent) scales
contributes most to generation quality; a small amount of memory kept for the
coarsest scales, the condensed scales, stabilises generation; layers differ
in how similar their keys and values are across the finer scales, and the
layers with weaker inter-scale similarity are cache-demanding.  The policy
prioritises condensed and local scales and gives the cache-demanding layers
more.

Readings taken where the abstract stops:
  * condensed scales are 0 .. n_condensed-1 and stay cached to the end;
  * "local" means the `window` scales just before the one being generated:
    scale t reads cached scales t-window .. t-1 besides the condensed ones,
    so segment s (s >= n_condensed) is read by scales s+1 .. s+window and
    leaves the cache at step min(s + window, K-1);
  * the cache-demanding layers are the n_demanding layers with the lowest
    inter-scale similarity score (a per-layer input; ties pick the lower
    layer index first) and use `window_demanding` instead of `window`;
  * the policy is the same for every head of a layer.
The result is expressed as expiry steps (``oracle.progressive``): expire[l,
h, s] is the step at whose end segment s leaves the cache.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .schedule import ScheduleError


def demanding_layers(similarity: Sequence[float], n_demanding: int) -> list:
    """Indices of the n_demanding layers with the lowest similarity score."""
    order = sorted(range(len(similarity)), key=lambda l: (float(similarity[l]), l))
    return sorted(order[:n_demanding])


def scale_window_schedule(L: int, H: int, scale_tokens: Sequence[int], n_condensed: int,
                          window: int, window_demanding: int,
                          similarity: Optional[Sequence[float]] = None,
                          n_demanding: int = 0) -> np.ndarray:
    """Expiry steps [L][H][K] (uint8) of the condensed + local policy."""
    K = len(scale_tokens)
    if L < 1 or H < 1 or K < 1:
        raise ScheduleError("einval", "L, H, K must be >= 1")
    if any(int(n) < 1 for n in scale_tokens):
        raise ScheduleError("einval", "every scale needs at least one token")
    if not (0 <= n_condensed <= K) or window < 0 or window_demanding < 0:
        raise ScheduleError("einval", "bad n_condensed or window")
    if not (0 <= n_demanding <= L) or (n_demanding > 0 and (similarity is None or len(similarity) != L)):
        raise ScheduleError("einval", "n_demanding needs one similarity score per layer")
    wide = set(demanding_layers(similarity, n_demanding)) if n_demanding > 0 else set()
    expire = np.zeros((L, H, K), dtype=np.uint8)
    for l in range(L):
        w = window_demanding if l in wide else window
        for s in range(K):
            expire[l, :, s] = K - 1 if s < n_condensed else min(s + w, K - 1)
    return expire
