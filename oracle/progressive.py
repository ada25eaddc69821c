"""Progressive head-scale pruning: growing pruning sets, per-layer cache
accounting and the cache contents they imply (oracle).

Test infrastructure only.

What the pages fix (Pith page of arXiv 2605.14877, Figure 4 caption, and
appendix A, Algorithm 2):
  * every source scale i has an ordering O_i of the heads, from least to most
    dependent on the tokens of scale i;
  * after scale k the pruning set G_k is the union, over the scales i <= k,
    of the prefix of length N_k of O_i, and G_k is to be gone from the cache
    once scale k is done;
  * the cache size is tracked layer by layer inside a scale
    (CacheSizeAfterLayer(k, l, G_k, G_{k-1}, ...)); the listing's body is not
    on the pages.

Readings taken where the pages stop:
  * Prunable scales and orderings are those of the static schedule
    (``oracle.schedule``): n_sink <= i <= K-2, O_i ascending by (importance,
    flat index).
  * N_k is chosen greedily and lazily: the smallest N >= N_{k-1} for which the
    cache fits the budget floor(beta * F); so N_k never decreases, G_k grows
    with k, and a segment of an earlier scale can be dropped from the middle
    of a head's cache when the prefix grows past it.  The static schedule is
    the special case where N_k is the final N from the first scale on.
  * Cache size after layer l of scale k (the accounting of Algorithm 2):
    layers 0..l have finished scale k, so each holds its segments s <= k not
    in G_k; layers l+1..L-1 still hold their segments s <= k-1 not in G_{k-1}.
    With per-layer accounting the budget must hold after every layer; with
    end-of-scale accounting only after the last layer (l = L-1).
  * The final scale K-1 is never cached, so nothing changes after scale K-2.
  * A pair's expiry step: expire[l, h, s] = the first k >= s with (l, h, s)
    in G_k, or K-1 when it is never pruned.  Segment s is read from the cache
    by the queries of scales t with s < t <= expire; expire == s means it is
    never stored.  At scale t the cache of (l, h) holds, in scale order, the
    segments s < t with expire >= t; at the end of scale k (after the drops
    and the append) it holds the segments s <= min(k, K-2) with expire > k.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

from .schedule import ScheduleError, full_cache_slots, head_order, importance


def expire_from_keep(keep: np.ndarray) -> np.ndarray:
    """The static keep-mask as expiry steps: kept -> K-1, pruned -> s."""
    L, H, K = keep.shape
    exp = np.zeros((L, H, K), dtype=np.uint8)
    for s in range(K):
        exp[:, :, s] = np.where((keep[:, :, s] != 0) & (s <= K - 2), K - 1, s)
    return exp


def visible(expire_lh: Sequence[int], t: int) -> List[int]:
    """0/1 per source s < t: is segment s in the cache while scale t is attended.
    Entries s >= t are 0 (the current scale is read from its own tensors)."""
    K = len(expire_lh)
    return [1 if (s < t and s <= K - 2 and int(expire_lh[s]) >= t) else 0 for s in range(K)]


def pruned_mask(orders: dict, L: int, H: int, K: int, k: int, n: int) -> np.ndarray:
    """G_k as a [L][H][K] boolean: the first n heads of O_i for every ordered
    (prunable) scale i <= k."""
    g = np.zeros((L, H, K), dtype=bool)
    for i, order in orders.items():
        if i <= k:
            for f in order[:n]:
                g[f // H, f % H, i] = True
    return g


def held_rows(g: np.ndarray, scale_tokens: Sequence[int], k: int, layer: int) -> int:
    """Token slots of one layer at the end of scale k under pruning set g."""
    L, H, K = g.shape
    total = 0
    for s in range(min(k, K - 2) + 1):
        total += int((~g[layer, :, s]).sum()) * int(scale_tokens[s])
    return total


def sizes_after_layers(k: int, g_k: np.ndarray, g_prev: np.ndarray,
                       scale_tokens: Sequence[int]) -> List[int]:
    """Token slots per sequence once layer l has finished scale k, for every l:
    layers 0..l at the end of scale k under g_k, layers l+1.. at the end of
    scale k-1 under g_prev (nothing before scale 0)."""
    L = g_k.shape[0]
    done = [held_rows(g_k, scale_tokens, k, l) for l in range(L)]
    pending = [held_rows(g_prev, scale_tokens, k - 1, l) if k > 0 else 0 for l in range(L)]
    return [sum(done[: l + 1]) + sum(pending[l + 1:]) for l in range(L)]


def cache_size_after_layer(k: int, layer: int, g_k: np.ndarray, g_prev: np.ndarray,
                           scale_tokens: Sequence[int]) -> int:
    """Token slots per sequence once layer ``layer`` has finished scale k."""
    return sizes_after_layers(k, g_k, g_prev, scale_tokens)[layer]


def progressive_schedule(scas: np.ndarray, scale_tokens: Sequence[int], budget_frac: float,
                         n_sink: int, per_layer: bool = True
                         ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """S-CAS table + budget -> (expire [L][H][K] u8, N [K] int, live [K][L] int64).

    live[k][l] is the cache size after layer l of scale k (Algorithm 2's
    accounting); live[K-1] repeats the end of scale K-2.
    """
    scas = np.asarray(scas)
    if scas.ndim != 4 or scas.shape[2] != scas.shape[3]:
        raise ScheduleError("einval", "scas must be [L][H][K][K]")
    L, H, K, _ = scas.shape
    if L < 1 or H < 1 or K < 1 or len(scale_tokens) != K:
        raise ScheduleError("einval", "bad L, H, K or scale_tokens length")
    if any(int(n) < 1 for n in scale_tokens):
        raise ScheduleError("einval", "every scale needs at least one token")
    if not (0 <= n_sink <= K - 1):
        raise ScheduleError("einval", "n_sink must be in [0, K-1]")
    if not (budget_frac > 0.0 and budget_frac <= 1.0):
        raise ScheduleError("einval", "budget_frac must be in (0, 1]")

    heads = L * H
    imp = importance(scas)
    orders = {i: head_order(imp[:, :, i]) for i in range(n_sink, K - 1)}
    bud = math.floor(budget_frac * full_cache_slots(L, H, scale_tokens))

    n_of = np.zeros(K, dtype=np.int64)
    live = np.zeros((K, L), dtype=np.int64)
    expire = np.full((L, H, K), K - 1, dtype=np.uint8)
    g_prev = np.zeros((L, H, K), dtype=bool)
    n = 0
    for k in range(K - 1):
        while True:
            g = pruned_mask(orders, L, H, K, k, n)
            sizes = sizes_after_layers(k, g, g_prev, scale_tokens)
            if (max(sizes) if per_layer else sizes[-1]) <= bud:
                break
            if n == heads:
                raise ScheduleError("ebudget", f"budget {bud} slots cannot hold scale {k}")
            n += 1
        n_of[k] = n
        live[k] = sizes
        newly = g & ~g_prev
        expire[newly] = k
        g_prev = g
    if K >= 2:
        n_of[K - 1] = n_of[K - 2]
        live[K - 1] = live[K - 2][L - 1]
    return expire, n_of, live


def retained_per_step(expire: np.ndarray, scale_tokens: Sequence[int]) -> np.ndarray:
    """R_k: token slots per sequence at the end of scale k (k = 0..K-1)."""
    L, H, K = expire.shape
    out = np.zeros(K, dtype=np.int64)
    for k in range(K):
        kk = min(k, K - 2)
        total = 0
        for s in range(kk + 1):
            total += int((expire[:, :, s].astype(np.int64) > kk).sum()) * int(scale_tokens[s])
        out[k] = total
    return out


def rows_at_end(expire_lh: Sequence[int], scale_tokens: Sequence[int], k: int) -> int:
    """Rows of one (l, h, b) cache at the end of scale k."""
    K = len(expire_lh)
    kk = min(k, K - 2)
    return sum(int(scale_tokens[s]) for s in range(kk + 1) if int(expire_lh[s]) > kk)


def capacity(expire: np.ndarray, scale_tokens: Sequence[int]) -> np.ndarray:
    """cap[l][h]: the most rows head (l, h) holds at the end of any scale."""
    L, H, K = expire.shape
    cap = np.zeros((L, H), dtype=np.int64)
    for l in range(L):
        for h in range(H):
            cap[l, h] = max([rows_at_end(expire[l, h], scale_tokens, k) for k in range(K)] + [0])
    return cap


def expected_rows(k_scales: Sequence[np.ndarray], expire_lh: Sequence[int], k: int,
                  b: int, h: int) -> np.ndarray:
    """Rows of (l, h, b) at the end of scale k: with kk = min(k, K-2), the
    segments s <= kk with expire > kk, in scale order (k_scales[s]: [B][n_s][H][D] stored values)."""
    K = len(expire_lh)
    kk = min(k, K - 2)
    parts = [k_scales[s][b, :, h, :] for s in range(kk + 1) if int(expire_lh[s]) > kk]
    if not parts:
        return np.zeros((0, k_scales[0].shape[3]), dtype=k_scales[0].dtype)
    return np.concatenate(parts, axis=0)
