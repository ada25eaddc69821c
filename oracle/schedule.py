"""Static head-scale keep-mask from an S-CAS table and a budget (oracle).

Test infrastructure only.  The algorithm, in the pages' terms:

  * S-CAS ranks head-scale pairs by how much future predictions depend on
    them (HeatKV project page, Method step 3; Abstract: it ranks how strongly
    each head depends on previously generated scales).
  * For every source scale i there is an ordering O_i of the heads, from
    least to most dependent on the tokens of scale i.  After scale k the
    pruning set G_k is the union over i <= k of the prefix of length N_k of
    O_i; G_k is to be gone from the cache once scale k is done (Pith page of
    arXiv 2605.14877, Figure 4 caption, the binary variant of Algorithm 1
    with greedy early pruning).
  * The budget decides how many low-ranked head-scale pairs are removed,
    while the early sink scales are always kept (HeatKV project page, Method
    step 4); the schedule is static and prompt-independent, and keeps the
    cache within budget while new scales are generated (Method step 5).

Readings taken where the pages leave a step open:
  * Importance of (l, h, s): the S-CAS mass that the later scales t > s put
    on s, i.e. sum over t = s+1 .. K-1 of scas[l, h, t, s], accumulated in
    float64 in ascending t from the float32 table values.
  * Prunable scales: n_sink <= s <= K-2.  The final scale K-1 is never
    cached (no later query reads it).  Scales below n_sink are sinks.
  * O_s sorts the flat head index f = l*H + h ascending by (importance, f):
    equal importance prunes the lower flat index first.
  * Greedy early pruning with a static mask: every pair that will ever be
    pruned is pruned when its own scale completes, so one prefix length N
    serves every scale (N_k = N).  N is the smallest value whose retained
    cache fits the budget.
  * Budget: a cap on retained token slots per sequence, floor(beta * F),
    where F = L * H * sum of n_s over s <= K-2; the cap holds after every
    scale.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


class ScheduleError(ValueError):
    """Raised for invalid arguments (code 'einval') or an infeasible budget ('ebudget')."""

    def __init__(self, code: str, msg: str):
        super().__init__(msg)
        self.code = code


def importance(scas: np.ndarray) -> np.ndarray:
    """I[l, h, s] = sum over t > s of scas[l, h, t, s], fp64, ascending t."""
    L, H, K, _ = scas.shape
    imp = np.zeros((L, H, K), dtype=np.float64)
    for s in range(K):
        for t in range(s + 1, K):
            imp[:, :, s] = imp[:, :, s] + scas[:, :, t, s].astype(np.float64)
    return imp


def head_order(imp_s: np.ndarray) -> list:
    """O_s: flat head indices from least to most important for one source scale."""
    flat = imp_s.reshape(-1)
    return sorted(range(flat.size), key=lambda f: (float(flat[f]), f))


def full_cache_slots(L: int, H: int, scale_tokens: Sequence[int]) -> int:
    """F: token slots per sequence when every cacheable scale (0..K-2) is kept."""
    return L * H * sum(scale_tokens[: len(scale_tokens) - 1])


def retained_per_step(keep: np.ndarray, scale_tokens: Sequence[int]) -> np.ndarray:
    """R_k: token slots per sequence held by the cache after scale k, k = 0..K-1."""
    L, H, K = keep.shape
    out = np.zeros(K, dtype=np.int64)
    for k in range(K):
        total = 0
        for s in range(min(k, K - 2) + 1):
            total += int(keep[:, :, s].astype(np.int64).sum()) * scale_tokens[s]
        out[k] = total
    return out


def build_schedule(scas: np.ndarray, scale_tokens: Sequence[int], budget_frac: float,
                   n_sink: int) -> Tuple[np.ndarray, np.ndarray, int]:
    """S-CAS table [L][H][K][K] + budget -> (keep [L][H][K] u8, R [K] int64, N).

    keep[l, h, s] = 1 when segment s of head (l, h) is cached after scale s
    completes; keep[., ., K-1] = 0.
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
    prunable = list(range(n_sink, K - 1))

    F = full_cache_slots(L, H, scale_tokens)
    bud = math.floor(budget_frac * F)
    s_sink = heads * sum(scale_tokens[:n_sink])
    t_p = sum(scale_tokens[s] for s in prunable)
    if bud < s_sink:
        raise ScheduleError("ebudget", f"budget {bud} slots is below the sink cost {s_sink}")
    keep_count = heads if t_p == 0 else min(heads, (bud - s_sink) // t_p)
    n_prune = heads - keep_count

    keep = np.zeros((L, H, K), dtype=np.uint8)
    keep[:, :, : K - 1] = 1
    for s in prunable:
        for f in head_order(imp[:, :, s])[:n_prune]:
            keep[f // H, f % H, s] = 0
    return keep, retained_per_step(keep, scale_tokens), n_prune
