"""Group-wise 4-bit storage of the ragged cache and attention over it (oracle).

Test infrastructure only.

What the pages fix (VAR-Q summary page, Key contributions and Method):
quantization groups are indexed by (block, channel), where a block is what
the generation loop emits at once (one scale in next-scale prediction) and a
channel is one of the head's D dimensions; a sub-block ratio r splits each
block further along the token axis; low-bit values are packed into
byte-aligned containers when written and unpacked for attention, so the
nominal bit width becomes a real memory saving.  The pages also say the
quantizer composes with eviction, without measuring it.

Readings taken where the pages stop:
  * Sub-blocks: r = 1/m with m a whole number; sub-block j of a segment of n
    tokens covers tokens [floor(j*n/m), floor((j+1)*n/m)) (possibly empty
    when m > n).
  * Quantizer: asymmetric uniform 4-bit per group, in float32 as stored:
    lo = min, hi = max of the group's values, step = (hi - lo) / 15 (each
    operation rounded to float32), code = round-half-even((x - lo) / step)
    clamped to [0, 15], code 0 when step = 0; an empty group stores
    (step, lo) = (0, 0).
  * Dequantized value: lo + code * step (evaluated here in float64).
  * Packing: two codes per byte, channel 2i in the low nibble and 2i+1 in
    the high nibble; a row of D channels takes D/2 bytes.
  * Composition with pruning: only the segments the static keep-mask keeps
    are stored, each quantized when its scale completes; attention reads the
    dequantized values of the stored segments and the full-precision keys and
    values of the scale being generated.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .attention import softmax_attention

LEVELS = 15  # 4-bit codes 0..15


def sub_block_bounds(n: int, m: int) -> List[Tuple[int, int]]:
    """Token ranges of the m sub-blocks of an n-token segment."""
    return [((j * n) // m, ((j + 1) * n) // m) for j in range(m)]


def quantize_group(x: np.ndarray) -> Tuple[np.ndarray, np.float32, np.float32]:
    """One group's float32 values -> (codes uint8, step, lo), float32 arithmetic."""
    x = np.asarray(x, dtype=np.float32)
    if x.size == 0:
        return np.zeros(0, dtype=np.uint8), np.float32(0.0), np.float32(0.0)
    lo = np.float32(x.min())
    hi = np.float32(x.max())
    step = np.float32(np.float32(hi - lo) / np.float32(LEVELS))
    if step == 0:
        return np.zeros(x.shape, dtype=np.uint8), step, lo
    q = np.rint(np.float32(x - lo) / step)
    return np.clip(q, 0, LEVELS).astype(np.uint8), step, lo


def quantize_segment(seg: np.ndarray, m: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """A segment's rows [n][D] (float32 values) -> (codes [n][D] uint8,
    step [m][D] float32, lo [m][D] float32)."""
    seg = np.asarray(seg, dtype=np.float32)
    n, D = seg.shape
    codes = np.zeros((n, D), dtype=np.uint8)
    step = np.zeros((m, D), dtype=np.float32)
    lo = np.zeros((m, D), dtype=np.float32)
    for j, (a, b) in enumerate(sub_block_bounds(n, m)):
        for c in range(D):
            codes[a:b, c], step[j, c], lo[j, c] = quantize_group(seg[a:b, c])
    return codes, step, lo


def dequantize_segment(codes: np.ndarray, step: np.ndarray, lo: np.ndarray, m: int) -> np.ndarray:
    """Inverse map in float64: row i of sub-block j -> lo[j] + code * step[j]."""
    n, D = codes.shape
    out = np.zeros((n, D), dtype=np.float64)
    for j, (a, b) in enumerate(sub_block_bounds(n, m)):
        out[a:b] = lo[j].astype(np.float64) + codes[a:b].astype(np.float64) * step[j].astype(np.float64)
    return out


def pack(codes: np.ndarray) -> np.ndarray:
    """codes [n][D] (0..15) -> bytes [n][D/2]: low nibble = even channel."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    """bytes [n][D/2] -> codes [n][D]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, half = packed.shape
    codes = np.zeros((n, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def stored_segments(x_scales: Sequence[np.ndarray], keep_lh: Sequence[int], k: int, b: int, h: int,
                    m: int) -> list:
    """The quantized segments of (l, h, b) after scale k, in scale order:
    [(s, packed [n_s][D/2], step [m][D], lo [m][D])] for kept s <= min(k, K-2).
    x_scales[s]: [B][n_s][H][D] float32 values of K (or V)."""
    K = len(keep_lh)
    out = []
    for s in range(min(k, K - 2) + 1):
        if keep_lh[s]:
            codes, step, lo = quantize_segment(x_scales[s][b, :, h, :], m)
            out.append((s, pack(codes), step, lo))
    return out


def dequantized_keys(k_scales: Sequence[np.ndarray], v_scales: Sequence[np.ndarray],
                     keep_lh: Sequence[int], t: int, b: int, h: int, m: int):
    """The keys and values a query of scale t of (b, h) reads: the dequantized
    kept segments s < t, then scale t's own rows (fp64).  Returns (K_J, V_J,
    sources, lengths) like ``attention.gather_keys``.
    k_scales/v_scales[s]: [B][n_s][H][D] float32 values."""
    kparts, vparts, src, lens = [], [], [], []
    for s in range(t):
        if s <= len(keep_lh) - 2 and keep_lh[s]:
            for xs, parts in ((k_scales, kparts), (v_scales, vparts)):
                codes, step, lo = quantize_segment(xs[s][b, :, h, :], m)
                parts.append(dequantize_segment(codes, step, lo, m))
            src.append(s)
            lens.append(k_scales[s].shape[1])
    kparts.append(np.asarray(k_scales[t][b, :, h, :], dtype=np.float64))
    vparts.append(np.asarray(v_scales[t][b, :, h, :], dtype=np.float64))
    src.append(t)
    lens.append(k_scales[t].shape[1])
    return np.concatenate(kparts, axis=0), np.concatenate(vparts, axis=0), src, lens


def attend_rows(q: np.ndarray, k_scales: Sequence[np.ndarray], v_scales: Sequence[np.ndarray],
                keep_lh: Sequence[int], t: int, b: int, h: int, m: int, alpha: float,
                rows=None) -> np.ndarray:
    """Attention of query rows of scale t of (b, h) over the dequantized kept
    segments s < t followed by scale t's own keys and values (fp64).
    q: [B][n_t][H][D]."""
    kj, vj, _, _ = dequantized_keys(k_scales, v_scales, keep_lh, t, b, h, m)
    qr = np.asarray(q[b, :, h, :], dtype=np.float64)
    if rows is not None:
        qr = qr[rows]
    out, _ = softmax_attention(qr, kj, vj, alpha)
    return out
