"""Helpers for the GPU parity tests: drive the library through a generation
and compare against the fp64 oracle.  Inputs come from ``workloads`` only."""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import workloads
from oracle import attention as oatt
from oracle import cache as ocache
from oracle.numerics import to_f64

import kv_cache_compression_attend_amd as hk

SENTINEL_BF16 = 0x7FA5  # a NaN pattern no input or copy can produce
SENTINEL_F32 = 0x7FA5A5A5


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(wl) -> torch.dtype:
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def to_device(x: np.ndarray, wl) -> torch.Tensor:
    if wl.dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(x).to("cuda")


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def poison(ctx: hk.Context) -> None:
    for c in (ctx.k_cache, ctx.v_cache):
        if c.dtype == torch.bfloat16:
            c.view(torch.int16).fill_(SENTINEL_BF16)
        else:
            c.view(torch.int32).fill_(SENTINEL_F32)


@dataclass
class Run:
    """Outputs of one generation over some layers."""
    wl: workloads.Workload
    keep: np.ndarray
    layers: List[int]
    ctx: hk.Context
    inputs: Dict[int, List[workloads.StepInputs]] = field(default_factory=dict)
    outs: Dict[tuple, np.ndarray] = field(default_factory=dict)   # (l, t) -> host bits
    scas: Optional[np.ndarray] = None


def generate(wl, keep: np.ndarray, layers: Sequence[int], seed: int = 0, scas: bool = False,
             multi_layer_append: bool = False, keep_inputs: bool = True, fused: bool = False) -> Run:
    """Run all K scales for ``layers`` through the library: attend then append,
    or (fused) the single attend_append call per layer and scale."""
    ctx = hk.Context(wl.layers, wl.heads, wl.head_dim, wl.batch, wl.scale_tokens, keep,
                     torch_dtype(wl))
    poison(ctx)
    table = torch.zeros((wl.layers, wl.heads, wl.n_scales, wl.n_scales), dtype=torch.float32,
                        device="cuda") if scas else None
    run = Run(wl, keep, list(layers), ctx)
    for l in layers:
        run.inputs[l] = []
    for t in range(wl.n_scales):
        ks, vs = [], []
        for l in layers:
            inp = workloads.step_inputs(wl, l, t, seed)
            if keep_inputs:
                run.inputs[l].append(inp)
            q, k, v = to_device(inp.q, wl), to_device(inp.k, wl), to_device(inp.v, wl)
            out = torch.empty_like(q)
            call = "attend_append" if fused else ("attend_with_scas" if scas else "attend")
            note(f"{wl.name} layer {l} step {t}: {call} q {tuple(q.shape)}")
            if fused:
                ctx.attend_append(l, t, q, k, v, out, wl.softmax_scale, table)
            elif scas:
                ctx.attend_with_scas(l, t, q, k, v, out, wl.softmax_scale, table)
            else:
                ctx.attend(l, t, q, k, v, out, wl.softmax_scale)
            run.outs[(l, t)] = to_host_bits(out)
            ks.append(k)
            vs.append(v)
            if t < wl.n_scales - 1 and not multi_layer_append and not fused:
                note(f"{wl.name} layer {l} step {t}: append_scale")
                ctx.append_scale(l, l + 1, t, k, v)
        if t < wl.n_scales - 1 and multi_layer_append and not fused:
            assert list(layers) == list(range(layers[0], layers[0] + len(layers)))
            note(f"{wl.name} layers {layers[0]}..{layers[-1]} step {t}: append_scale")
            ctx.append_scale(layers[0], layers[-1] + 1, t, torch.stack(ks), torch.stack(vs))
        torch.cuda.synchronize()
    if scas:
        run.scas = table.cpu().numpy()
    return run


def oracle_rows(run: Run, l: int, t: int, b: int, h: int, rows) -> tuple:
    """fp64 oracle output for query rows of (l, t, b, h), plus the mass if all rows."""
    wl = run.wl
    ins = run.inputs[l]
    kj, vj, src, lens = oatt.gather_keys([x.k for x in ins[: t + 1]], [x.v for x in ins[: t + 1]],
                                         run.keep[l, h], t, b, h)
    q = to_f64(ins[t].q[b, rows, h, :], wl.dtype)
    o, p = oatt.softmax_attention(q, to_f64(kj, wl.dtype), to_f64(vj, wl.dtype), wl.softmax_scale)
    return o, oatt.segment_mass(p, src, lens, t)


def gpu_rows(run: Run, l: int, t: int, b: int, h: int, rows) -> np.ndarray:
    return to_f64(run.outs[(l, t)][b, rows, h, :], run.wl.dtype)


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """All rows for small n; otherwise k random rows plus the ragged tail."""
    if n <= k:
        return np.arange(n)
    g = np.random.default_rng(seed)
    pick = set(g.choice(n, size=k, replace=False).tolist())
    pick.update(range(max(0, n - 3), n))
    pick.add(0)
    return np.array(sorted(pick))


def _layer_bits(cache: torch.Tensor, lo: int, hi: int) -> np.ndarray:
    """Host copy of elements [lo, hi) of a cache buffer (only that slice moves)."""
    return to_host_bits(cache[lo:hi])


def check_cache(run: Run, layers: Sequence[int], heads: Optional[Sequence[int]] = None,
                edge_only_elems: int = 1 << 30) -> None:
    """Cache regions of the given layers equal the oracle's expected rows bit for bit;
    regions of layers that were never appended still hold the sentinel (every
    element, or for caches above edge_only_elems elements the first and last
    64 Ki elements of each such layer)."""
    wl, keep = run.wl, run.keep
    cap = ocache.capacity(keep, wl.scale_tokens)
    base = ocache.bases(cap, wl.batch, wl.head_dim)
    heads = range(wl.heads) if heads is None else heads
    K = wl.n_scales

    def span(l):
        return int(base[l, 0]), int(base[l, -1]) + wl.batch * int(cap[l, -1]) * wl.head_dim

    for l in layers:
        lo, hi = span(l)
        for which, cache in (("k", run.ctx.k_cache), ("v", run.ctx.v_cache)):
            bits = _layer_bits(cache, lo, hi)
            for h in heads:
                c = int(cap[l, h])
                region = bits[base[l, h] - lo: base[l, h] - lo + wl.batch * c * wl.head_dim]
                region = region.reshape(wl.batch, c, wl.head_dim)
                for b in range(wl.batch):
                    want = ocache.expected_rows([getattr(x, which) for x in run.inputs[l]],
                                                keep[l, h], K - 1, b, h)
                    assert np.array_equal(region[b], want), (which, l, h, b)
    sentinel = SENTINEL_BF16 if wl.dtype == "bf16" else SENTINEL_F32
    udt = np.uint16 if wl.dtype == "bf16" else np.uint32
    edge = 1 << 16
    for l in range(wl.layers):
        if l in run.layers:
            continue
        lo, hi = span(l)
        if hi <= lo:
            continue
        parts = [(lo, hi)] if run.ctx.k_cache.numel() <= edge_only_elems else \
            [(lo, min(hi, lo + edge)), (max(lo, hi - edge), hi)]
        for cache in (run.ctx.k_cache, run.ctx.v_cache):
            for a, b in parts:
                seg = _layer_bits(cache, a, b)
                assert (seg.view(udt) == sentinel).all(), l
