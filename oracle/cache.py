"""Ragged per-head cache: layout, expected compacted contents, size accounting (oracle).

Test infrastructure only.

The cache holds, for every (layer l, head h, batch entry b), the kept
segments of the completed scales, in scale order, one row of D values per
token (HeatKV project page, Method step 5: pruning happens during inference
as scales complete; Pith page of arXiv 2605.14877, Figure 4 caption: G_k is
absent by the end of scale k, so a pruned segment is never stored).

Layout (the library's documented contract, rewritten here from its
definition):
  * cap[l][h] = sum of n_s over cacheable scales s <= K-2 with keep = 1;
  * heads are laid out one after another in row-major (l, h) order; head
    (l, h) owns B * cap[l][h] * D elements, as [B][cap][D];
  * after scale k the first len_before(l, h, k+1) rows of (l, h, b) hold the
    kept segments s <= k; rows beyond are untouched.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def capacity(keep: np.ndarray, scale_tokens: Sequence[int]) -> np.ndarray:
    """cap[l][h]: cache rows per batch entry for head (l, h)."""
    L, H, K = keep.shape
    cap = np.zeros((L, H), dtype=np.int64)
    for s in range(K - 1):
        cap += keep[:, :, s].astype(np.int64) * scale_tokens[s]
    return cap


def bases(cap: np.ndarray, batch: int, head_dim: int) -> np.ndarray:
    """Element offset of head (l, h)'s region, heads in row-major (l, h) order."""
    flat = cap.reshape(-1) * batch * head_dim
    starts = np.concatenate([[0], np.cumsum(flat)[:-1]]).astype(np.int64)
    return starts.reshape(cap.shape)


def len_before(keep: np.ndarray, scale_tokens: Sequence[int], t: int) -> np.ndarray:
    """Rows of (l, h) cached before scale t: sum of n_s over kept s < t, s <= K-2."""
    L, H, K = keep.shape
    out = np.zeros((L, H), dtype=np.int64)
    for s in range(min(t, K - 1)):
        out += keep[:, :, s].astype(np.int64) * scale_tokens[s]
    return out


def expected_rows(k_scales: Sequence[np.ndarray], keep_lh: Sequence[int], k: int,
                  b: int, h: int) -> np.ndarray:
    """Rows of (l, h, b) after scale k: the kept segments s <= min(k, K-2), in order.

    k_scales[s]: [B][n_s][H][D] stored values (any dtype; compared bit for bit).
    """
    K = len(keep_lh)
    parts = [k_scales[s][b, :, h, :] for s in range(min(k, K - 2) + 1) if keep_lh[s]]
    if not parts:
        return np.zeros((0, k_scales[0].shape[3]), dtype=k_scales[0].dtype)
    return np.concatenate(parts, axis=0)


def cache_bytes(keep: np.ndarray, scale_tokens: Sequence[int], batch: int,
                head_dim: int, elem_bytes: int) -> int:
    """Bytes of one of the two caches (K or V) for the whole batch."""
    return int(capacity(keep, scale_tokens).sum()) * batch * head_dim * elem_bytes


def full_cache_bytes(sequences: int, layers: int, hidden: int,
                     scale_tokens: Sequence[int], elem_bytes: int) -> int:
    """K + V bytes of an unpruned cache after the last cached scale.

    Every layer caches keys and values of width ``hidden`` (heads * head_dim)
    for the tokens of scales 0..K-2; the final scale is attended by its own
    queries and never cached.
    """
    cached_tokens = sum(scale_tokens[: len(scale_tokens) - 1])
    return sequences * 2 * layers * hidden * cached_tokens * elem_bytes
