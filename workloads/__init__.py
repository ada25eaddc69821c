"""Seeded synthetic inputs for the head-scale KV-pruning hot path.

This module only *makes data*: workload shapes, seeded normal draws, the
round-to-nearest-even cast of fp32 draws to bfloat16 bits, and the
synthetic stand-ins for calibration outputs (Dirichlet S-CAS tables, the
per-(head, source-scale) key offsets and the tiny case's random keep-mask).
It holds none of the method's arithmetic: no attention, no S-CAS, no
ranking, no cache layout.  Both the fp64 CPU oracle and the HIP path draw
their inputs from here, so the two sides see identical bits.

Every tensor of a workload is regenerable on its own from
``SeedSequence([seed, config_index, layer, step, tensor_id])``, so a checker
can rebuild any (layer, step) unit without drawing the rest.

Workloads stand in for the pages' Infinity-2B / Infinity-8B generations at 13
scales (HeatKV project page, Results: "Experiments evaluate Infinity-2B and
Infinity-8B at 20%, 10%, and 4%"); the model weights, prompts and image
datasets are not used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

# tensor ids inside the seed sequence
TID_Q, TID_K, TID_V, TID_SCAS, TID_KOFF, TID_MASK = 0, 1, 2, 3, 4, 5

SIDES_13 = (1, 2, 4, 6, 8, 12, 16, 20, 24, 32, 40, 48, 64)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, precision, schedule recipe."""

    index: int                 # position in the workload list (enters the seed)
    name: str
    layers: int
    heads: int
    head_dim: int
    batch: int
    sides: Tuple[int, ...]
    dtype: str                 # "bf16" or "f32"
    budget: float              # fraction of the full cache kept (1.0 = no pruning)
    n_sink: int                # leading scales that are never pruned
    softmax_scale: float       # alpha applied to q.k
    qk_std: float              # std of the Q and K draws (V is N(0,1))
    schedule: str              # "full", "dirichlet", "random_drop2"
    key_offset_std: float = 0.0  # std of the per-(head, source-scale) key mean offset
    calibration: bool = False  # run attend_with_scas on every (layer, step)
    note: str = ""

    @property
    def n_scales(self) -> int:
        return len(self.sides)

    @property
    def scale_tokens(self) -> Tuple[int, ...]:
        return tuple(s * s for s in self.sides)

    @property
    def total_tokens(self) -> int:
        return sum(self.scale_tokens)


def _w(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS = (
    _w(index=0, name="tiny-l1h2d16-f32", layers=1, heads=2, head_dim=16, batch=1,
       sides=(1, 2, 3, 4), dtype="f32", budget=0.5, n_sink=1, softmax_scale=0.25,
       qk_std=1.0, schedule="random_drop2", calibration=True,
       note="two random (head, source-scale) pairs dropped, scale 0 kept"),
    _w(index=1, name="infinity2b-layer-full-b1", layers=1, heads=16, head_dim=128,
       batch=1, sides=SIDES_13, dtype="bf16", budget=1.0, n_sink=2,
       softmax_scale=1.0, qk_std=128 ** -0.25, schedule="full",
       note="Infinity-2B-shaped single layer, full cache"),
    _w(index=2, name="infinity2b-l32-b8-budget10", layers=32, heads=16, head_dim=128,
       batch=8, sides=SIDES_13, dtype="bf16", budget=0.10, n_sink=2,
       softmax_scale=1.0, qk_std=128 ** -0.25, schedule="dirichlet",
       note="Dirichlet(0.5) S-CAS table ranked into a 10% static keep-mask"),
    _w(index=3, name="infinity2b-l32-b4-calibration", layers=32, heads=16,
       head_dim=128, batch=4, sides=SIDES_13, dtype="bf16", budget=1.0, n_sink=2,
       softmax_scale=1.0, qk_std=128 ** -0.25, schedule="full",
       key_offset_std=1.5, calibration=True,
       note="full cache, S-CAS emitted for every (layer, step)"),
    _w(index=4, name="infinity8b-l40h28-b16-budget4", layers=40, heads=28,
       head_dim=128, batch=16, sides=SIDES_13, dtype="bf16", budget=0.04,
       n_sink=2, softmax_scale=1.0, qk_std=128 ** -0.25, schedule="dirichlet",
       note="Infinity-8B-shaped, 4% static keep-mask"),
)

BY_NAME = {w.name: w for w in WORKLOADS}


def get(key) -> Workload:
    """Look a workload up by index (0..4), short id ("c0".."c4") or name."""
    if isinstance(key, int):
        return WORKLOADS[key]
    if isinstance(key, str) and len(key) == 2 and key[0] == "c" and key[1].isdigit():
        return WORKLOADS[int(key[1])]
    return BY_NAME[key]


def rng(seed: int, wl: Workload, layer: int, step: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, wl.index, layer, step, tensor_id])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bfloat16 bit patterns, round to nearest even.

    Inputs are finite normal draws, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def key_offsets(wl: Workload, seed: int = 0) -> Optional[np.ndarray]:
    """Per-(head, source-scale) key mean offsets mu[h][s] ~ N(0, std^2), fp32.

    Shared by every layer and batch entry; None when the workload has none.
    """
    if wl.key_offset_std == 0.0:
        return None
    g = rng(seed, wl, 0, 0, TID_KOFF)
    return (g.standard_normal((wl.heads, wl.n_scales)) * wl.key_offset_std).astype(np.float32)


@dataclass
class StepInputs:
    """Q_t, K_t, V_t of one (layer, step), each [B][n_t][H][D].

    For bf16 workloads the arrays are uint16 bit patterns; for f32 they are
    float32 values.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str = "bf16"
    extra: dict = field(default_factory=dict)


def step_inputs(wl: Workload, layer: int, step: int, seed: int = 0,
                batch: Optional[int] = None) -> StepInputs:
    """Draw Q, K, V of one (layer, step).

    Q, K ~ N(0,1) * qk_std, V ~ N(0,1).  Where the workload has key offsets,
    K = (Z + mu[h, step]) * qk_std.  ``batch`` (<= wl.batch) keeps only the
    leading batch entries of the same draw (batch is the leading axis, so they
    are the first values of the generator's stream and only those are drawn).
    """
    n = wl.scale_tokens[step]
    nb = wl.batch if batch is None else min(int(batch), wl.batch)
    shape = (nb, n, wl.heads, wl.head_dim)
    out = []
    mu = key_offsets(wl, seed)
    for tid in (TID_Q, TID_K, TID_V):
        z = rng(seed, wl, layer, step, tid).standard_normal(shape, dtype=np.float32)
        if tid == TID_K and mu is not None:
            z = z + mu[None, None, :, step, None]
        if tid in (TID_Q, TID_K):
            z = z * np.float32(wl.qk_std)
        if wl.dtype == "bf16":
            out.append(round_to_bf16_bits(z))
        else:
            out.append(np.ascontiguousarray(z, dtype=np.float32))
    return StepInputs(*out, dtype=wl.dtype)


def dirichlet_scas(wl: Workload, seed: int = 0, concentration: float = 0.5) -> np.ndarray:
    """Synthetic S-CAS table [L][H][K][K] fp32.

    Row (l, h, t) over sources s <= t is a Dirichlet(concentration) draw;
    entries with s > t are zero.  Stands in for a calibration run.
    """
    K = wl.n_scales
    g = rng(seed, wl, 0, 0, TID_SCAS)
    table = np.zeros((wl.layers, wl.heads, K, K), dtype=np.float64)
    for t in range(K):
        table[:, :, t, : t + 1] = g.dirichlet(np.full(t + 1, concentration),
                                               size=(wl.layers, wl.heads))
    return table.astype(np.float32)


def random_drop2_keep(wl: Workload, seed: int = 0) -> np.ndarray:
    """Keep-mask [L][H][K] u8 for the tiny workload.

    Scale 0 is kept, the final scale is never cached, and two distinct
    (head, source-scale) pairs drawn uniformly from the scales 1..K-2 that a
    later query reads are dropped.
    """
    K = wl.n_scales
    keep = np.zeros((wl.layers, wl.heads, K), dtype=np.uint8)
    keep[:, :, : K - 1] = 1
    g = rng(seed, wl, 0, 0, TID_MASK)
    for layer in range(wl.layers):
        pairs = [(h, s) for h in range(wl.heads) for s in range(1, K - 1)]
        pick = g.choice(len(pairs), size=2, replace=False)
        for p in pick:
            h, s = pairs[int(p)]
            keep[layer, h, s] = 0
    return keep


def full_keep(wl: Workload) -> np.ndarray:
    """Keep-mask with every cacheable scale (0..K-2) retained."""
    keep = np.zeros((wl.layers, wl.heads, wl.n_scales), dtype=np.uint8)
    keep[:, :, : wl.n_scales - 1] = 1
    return keep


def random_scas_table(L: int, H: int, K: int, seed: int,
                      concentration: float = 0.5) -> np.ndarray:
    """Dirichlet S-CAS table of arbitrary shape for randomized schedule tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99, L, H, K])))
    table = np.zeros((L, H, K, K), dtype=np.float64)
    for t in range(K):
        table[:, :, t, : t + 1] = g.dirichlet(np.full(t + 1, concentration), size=(L, H))
    return table.astype(np.float32)


def random_tokens(K: int, seed: int, max_side: int = 4) -> Tuple[int, ...]:
    """Random nondecreasing scale sides for randomized tests -> token counts."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 98, K])))
    sides = np.sort(g.integers(1, max_side + 1, size=K))
    return tuple(int(s) * int(s) for s in sides)
