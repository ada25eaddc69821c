"""Block-causal multi-scale attention over kept segments, and S-CAS (oracle).

Test infrastructure only.  Plain fp64 NumPy: explicit scores, explicit
max-subtracted softmax, explicit probability-weighted sum of values.

What is computed (next-scale generation):
  * A VAR model emits token maps of growing size, one scale at a time; every
    token of scale t is produced together, conditioned on every earlier scale
    (Pith page of arXiv 2605.14877, Figure 2 caption: images are generated in
    increasing scale size, which makes the cache grow; HeatKV project page,
    Abstract).  Tokens inside a scale are in raster order (Pith page,
    Figure 3 caption).
  * So a query of scale t reads the keys of every earlier scale and of its
    own scale (block-causal: no mask inside a scale).
  * Head-scale pruning removes whole (layer, head, source-scale) segments
    from the cache (HeatKV project page, Method steps 4-5: low-ranked
    head-scale pairs are removed, sink scales retained, pruning during
    inference).  A query of scale t in head (l, h) therefore reads the
    segments s < t with keep[l, h, s] = 1, in scale order, then its own
    scale t, which is always present while it is being generated.
  * S-CAS, the Scale-dependent Cumulative Attention Score, aggregates the
    attention probabilities per layer, head, source scale and future
    generation scale (HeatKV project page, Abstract and Method step 2).

Readings taken where the pages are silent:
  * S-CAS of (l, h, t, s): for every query of scale t, the probability mass
    it puts on the keys of source scale s; averaged over the n_t queries of
    scale t and then over the batch.  Sources run over s <= t, the own scale
    included, so every row sums to 1; a dropped source has mass exactly 0.
  * The softmax scale alpha is an explicit input.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def kept_sources(keep_lh: Sequence[int], t: int) -> List[int]:
    """Source scales a query of scale t reads, in cache order.

    The kept earlier scales s < t (keep_lh[s] != 0) ascending, then t itself.
    """
    return [s for s in range(t) if keep_lh[s]] + [t]


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                      alpha: float) -> Tuple[np.ndarray, np.ndarray]:
    """Plain softmax attention of query rows over one key list, in fp64.

    q [n_q, d], k [n_k, d], v [n_k, d_v]  ->  (out [n_q, d_v], P [n_q, n_k])
    S = alpha * q k^T; P = exp(S - rowmax) / rowsum; out = P v.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = alpha * (q @ k.T)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v, p


def gather_keys(ks: Sequence[np.ndarray], vs: Sequence[np.ndarray],
                keep_lh: Sequence[int], t: int, b: int, h: int):
    """Concatenate the K and V rows a query of scale t of (b, h) reads.

    ks[s], vs[s]: [B][n_s][H][D] fp64 for s = 0..t.  Returns (K_J, V_J,
    sources, lengths): the stacked key and value rows, and the source scale
    and row count of each segment in order.
    """
    src = kept_sources(keep_lh, t)
    kj = np.concatenate([ks[s][b, :, h, :] for s in src], axis=0)
    vj = np.concatenate([vs[s][b, :, h, :] for s in src], axis=0)
    lens = [ks[s].shape[1] for s in src]
    return kj, vj, src, lens


def segment_mass(p: np.ndarray, sources: Sequence[int], lengths: Sequence[int],
                 t: int) -> np.ndarray:
    """Per-unit S-CAS: mass [t+1] that the queries of p put on each source.

    p [n_q, n_k] are the attention probabilities of all n_q = n_t queries of
    scale t (columns in the order of ``sources``).  Entry s is the mean over
    queries of the probability summed over the columns of source s; sources
    that are not read stay 0.
    """
    mass = np.zeros(t + 1, dtype=np.float64)
    col = 0
    for s, n in zip(sources, lengths):
        mass[s] = p[:, col:col + n].sum(axis=1).mean()
        col += n
    return mass


def attend_step(qt: np.ndarray, ks: Sequence[np.ndarray], vs: Sequence[np.ndarray],
                keep_layer: np.ndarray, t: int, alpha: float,
                q_rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of every (b, h) of one layer at scale t.

    qt: [B][n_t][H][D] fp64; ks[s], vs[s]: [B][n_s][H][D] fp64 for s <= t;
    keep_layer: [H][K] (row of the keep-mask for this layer).
    ``q_rows`` optionally restricts the query rows computed (sampling); the
    returned mass is then over those rows only.

    Returns (out [B][n_rows][H][D], mass [B][H][t+1]).
    """
    B, n_t, H, D = qt.shape
    rows = np.arange(n_t) if q_rows is None else np.asarray(q_rows)
    out = np.zeros((B, len(rows), H, vs[t].shape[3]), dtype=np.float64)
    mass = np.zeros((B, H, t + 1), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kj, vj, src, lens = gather_keys(ks, vs, keep_layer[h], t, b, h)
            o, p = softmax_attention(qt[b, rows, h, :], kj, vj, alpha)
            out[b, :, h, :] = o
            mass[b, h] = segment_mass(p, src, lens, t)
    return out, mass


def attend_step_masked(qt: np.ndarray, ks: Sequence[np.ndarray], vs: Sequence[np.ndarray],
                       keep_layer: np.ndarray, t: int, alpha: float) -> np.ndarray:
    """The same attention written as one masked softmax over all scales 0..t.

    Every key of scales 0..t is scored; keys of a scale s < t with
    keep[h, s] = 0 get score -inf, so their probability is exactly 0.
    Used to check that dropping a pair equals masking it out.
    """
    B, n_t, H, D = qt.shape
    out = np.zeros((B, n_t, H, vs[t].shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kall = np.concatenate([ks[s][b, :, h, :] for s in range(t + 1)], axis=0)
            vall = np.concatenate([vs[s][b, :, h, :] for s in range(t + 1)], axis=0)
            scale_of = np.concatenate([np.full(ks[s].shape[1], s) for s in range(t + 1)])
            dropped = np.array([(s < t) and not keep_layer[h][s] for s in scale_of])
            sc = alpha * (qt[b, :, h, :] @ kall.T)
            sc[:, dropped] = -np.inf
            sc = sc - sc.max(axis=1, keepdims=True)
            e = np.exp(sc)
            out[b, :, h, :] = (e / e.sum(axis=1, keepdims=True)) @ vall
    return out


def scas_row(mass: np.ndarray) -> np.ndarray:
    """S-CAS row t for one layer: [H][t+1], the batch mean of per-unit mass."""
    return mass.mean(axis=0)
