"""Calibration over many batches and the stability of its rankings (oracle).

Test infrastructure only.

* A small offline calibration set yields one S-CAS table (HeatKV project
  page, Method steps 1-2).  Streaming reading: the table of the whole set is
  the mean over all calibration images of the per-image S-CAS, whatever the
  batches they arrive in.
* Rankings stay stable with a small calibration set (HeatKV project page,
  Results; Pith page of arXiv 2605.14877, Figure 6 caption).  The pages give
  no formula; two measures are taken:
    - per prunable source scale s, Spearman's rank correlation between the
      positions of the heads in the two orderings O_s;
    - the Jaccard index of the two pruned (layer, head, scale) sets at a
      budget.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from . import schedule as osch


def streamed_mean(batch_tables: Sequence[np.ndarray], batch_sizes: Sequence[int]) -> np.ndarray:
    """Mean over images of per-image S-CAS, from per-batch tables (each the
    mean over its batch) and the batch sizes."""
    total = sum(batch_sizes)
    acc = np.zeros(np.asarray(batch_tables[0]).shape, dtype=np.float64)
    for tab, b in zip(batch_tables, batch_sizes):
        acc += np.asarray(tab, dtype=np.float64) * b
    return acc / total


def positions(scas: np.ndarray, s: int) -> np.ndarray:
    """Position of each flat head index in the ordering O_s."""
    imp = osch.importance(np.asarray(scas))
    order = osch.head_order(imp[:, :, s])
    pos = np.zeros(len(order), dtype=np.int64)
    for i, f in enumerate(order):
        pos[f] = i
    return pos


def spearman_positions(pa: np.ndarray, pb: np.ndarray) -> float:
    """Spearman's rho of two permutations (no ties): 1 - 6 sum d^2 / (n (n^2 - 1))."""
    n = len(pa)
    d2 = float(((pa - pb) ** 2).sum())
    return 1.0 - 6.0 * d2 / (n * (n * n - 1.0))


def ranking_stability(scas_a: np.ndarray, scas_b: np.ndarray, scale_tokens: Sequence[int],
                      budget_frac: float, n_sink: int) -> Tuple[np.ndarray, float]:
    L, H, K, _ = np.asarray(scas_a).shape
    rho = np.full(K, math.nan)
    if L * H >= 2:
        for s in range(n_sink, K - 1):
            rho[s] = spearman_positions(positions(scas_a, s), positions(scas_b, s))
    ka = osch.build_schedule(scas_a, scale_tokens, budget_frac, n_sink)[0]
    kb = osch.build_schedule(scas_b, scale_tokens, budget_frac, n_sink)[0]
    ga = {(l, h, s) for l in range(L) for h in range(H) for s in range(K - 1) if not ka[l, h, s]}
    gb = {(l, h, s) for l in range(L) for h in range(H) for s in range(K - 1) if not kb[l, h, s]}
    union = ga | gb
    jac = 1.0 if not union else len(ga & gb) / len(union)
    return rho, jac
