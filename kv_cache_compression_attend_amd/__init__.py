"""MI355X (gfx950) hot path of head-scale KV-cache pruning for next-scale
visual autoregressive transformers: Python binding of ``libheatkv.so``.

The binding only marshals arguments: every step of the path (schedule,
attention, S-CAS, compaction) runs in the C/HIP library declared in
``include/heatkv.h``.  PyTorch provides device memory and streams.  There is
no CPU fallback: importing this package fails if the library is not built.

Typical use for one generation (all layers, all scales)::

    keep, retained, n_pruned = build_schedule(scas_table, tokens, 0.10, n_sink=2)
    ctx = Context(L, H, D, B, tokens, keep, torch.bfloat16)   # allocates the caches
    for t in range(K):
        for l in range(L):
            ctx.attend(l, t, q, k, v, out, softmax_scale)
        if t < K - 1:
            ctx.append_scale(0, L, t, k_all_layers, v_all_layers, layer_stride)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np
import torch  # first: the library binds to the HIP runtime torch has loaded

__all__ = ["HeatKVError", "build_schedule", "build_progressive_schedule", "build_scale_window_schedule",
           "cache_size_after_layer", "layout", "layout_expiry", "layout_pooled", "layout_int4", "scas_mean",
           "ranking_stability", "plan_attend_bf16", "attend_noalloc", "Context", "library_path", "DTYPES"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libheatkv.so")

HK_OK, HK_EINVAL, HK_EBUDGET, HK_EORDER, HK_EHIP, HK_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {HK_EINVAL: "EINVAL", HK_EBUDGET: "EBUDGET", HK_EORDER: "EORDER",
                HK_EHIP: "EHIP", HK_EUNSUPPORTED: "EUNSUPPORTED"}
HK_DTYPE_F32, HK_DTYPE_BF16 = 0, 1
HK_MAX_SCALES = 16
DTYPES = {torch.float32: HK_DTYPE_F32, torch.bfloat16: HK_DTYPE_BF16}


class HeatKVError(RuntimeError):
    """A non-OK status from the library; ``status`` is the HK_E* code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python kv_cache_compression_attend_amd/build.py` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, D, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float
    sig = {
        "hk_last_error": ([], ctypes.c_char_p),
        "hk_build_schedule": ([I, I, I, P, P, D, I, P, P, P], I),
        "hk_layout": ([I, I, I, P, P, I, I, P, P, P], I),
        "hk_create": ([P, I, I, I, I, I, P, P, I, P, P], I),
        "hk_destroy": ([P], I),
        "hk_reset": ([P], I),
        "hk_attend": ([P, I, I, P, P, P, P, F, P], I),
        "hk_attend_with_scas": ([P, I, I, P, P, P, P, F, P, P], I),
        "hk_append_scale": ([P, I, I, I, P, P, I64, P], I),
        "hk_retained_tokens": ([P, I, P], I),
        "hk_attend_plan": ([P, I, I, P, P], I),
        "hk_plan_attend_bf16": ([I, I, I, I, I, P, P], I),
        "hk_attend_append": ([P, I, I, P, P, P, P, F, P, P], I),
        "hk_attend_with_scas_sum": ([P, I, I, P, P, P, P, F, P, P], I),
        "hk_scas_mean": ([I, I, I, P, D, P], I),
        "hk_ranking_stability": ([I, I, I, P, P, P, D, I, P, P], I),
        "hk_build_progressive_schedule": ([I, I, I, P, P, D, I, I, P, P, P], I),
        "hk_cache_size_after_layer": ([I, I, I, P, P, I, I, P], I),
        "hk_layout_expiry": ([I, I, I, P, P, I, I, P, P, P], I),
        "hk_create_expiry": ([P, I, I, I, I, I, P, P, I, P, P], I),
        "hk_build_scale_window_schedule": ([I, I, I, P, I, I, I, P, I, P], I),
        "hk_layout_int4": ([I, I, I, P, P, I, I, I, P, P], I),
        "hk_create_int4": ([P, I, I, I, I, I, P, P, I, P, P], I),
        "hk_attend_noalloc": ([I, I, I, P, P, I, P, P, P, P, P, P, F, P, P], I),
        "hk_layout_pooled": ([I, I, I, P, P, I, I, P, P, P], I),
        "hk_create_pooled": ([P, I, I, I, I, I, P, P, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(rc: int) -> None:
    if rc != HK_OK:
        raise HeatKVError(rc, _lib.hk_last_error().decode(errors="replace"))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def build_schedule(scas: np.ndarray, scale_tokens: Sequence[int], budget_frac: float,
                   n_sink: int) -> Tuple[np.ndarray, np.ndarray, int]:
    """S-CAS table [L][H][K][K] (float32) + budget -> (keep u8 [L][H][K], retained int64 [K], N)."""
    scas = np.ascontiguousarray(scas, dtype=np.float32)
    if scas.ndim != 4 or scas.shape[2] != scas.shape[3]:
        raise HeatKVError(HK_EINVAL, "scas must be [L][H][K][K]")
    L, H, K, _ = scas.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    keep = np.zeros((L, H, K), dtype=np.uint8)
    ret = np.zeros(K, dtype=np.int64)
    npr = np.zeros(1, dtype=np.int32)
    _check(_lib.hk_build_schedule(L, H, K, _ptr(tok), _ptr(scas), float(budget_frac), int(n_sink),
                                  _ptr(keep), _ptr(ret), _ptr(npr)))
    return keep, ret, int(npr[0])


def plan_attend_bf16(batch: int, heads: int, n: int, max_keys: int,
                     allow_split: bool = True) -> Tuple[int, int]:
    """(query rows per workgroup, key-range splits) of a bf16 launch (host only)."""
    rows = np.zeros(1, dtype=np.int32)
    splits = np.zeros(1, dtype=np.int32)
    _check(_lib.hk_plan_attend_bf16(int(batch), int(heads), int(n), int(max_keys),
                                    int(bool(allow_split)), _ptr(rows), _ptr(splits)))
    return int(rows[0]), int(splits[0])


def layout(scale_tokens: Sequence[int], keep: np.ndarray, batch: int,
           head_dim: int) -> Tuple[int, np.ndarray, np.ndarray]:
    """(elements per cache buffer, cap [L][H], element offset [L][H])."""
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    L, H, K = keep.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    elems = np.zeros(1, dtype=np.int64)
    cap = np.zeros((L, H), dtype=np.int64)
    base = np.zeros((L, H), dtype=np.int64)
    _check(_lib.hk_layout(L, H, K, _ptr(tok), _ptr(keep), int(batch), int(head_dim), _ptr(elems),
                          _ptr(cap), _ptr(base)))
    return int(elems[0]), cap, base


def build_progressive_schedule(scas: np.ndarray, scale_tokens: Sequence[int], budget_frac: float,
                               n_sink: int, per_layer: bool = True
                               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """S-CAS table + budget -> (expire u8 [L][H][K], prefix lengths N_k int32 [K],
    cache size after each layer int64 [K][L])."""
    scas = np.ascontiguousarray(scas, dtype=np.float32)
    if scas.ndim != 4 or scas.shape[2] != scas.shape[3]:
        raise HeatKVError(HK_EINVAL, "scas must be [L][H][K][K]")
    L, H, K, _ = scas.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    expire = np.zeros((L, H, K), dtype=np.uint8)
    prefix = np.zeros(K, dtype=np.int32)
    live = np.zeros((K, L), dtype=np.int64)
    _check(_lib.hk_build_progressive_schedule(L, H, K, _ptr(tok), _ptr(scas), float(budget_frac),
                                              int(n_sink), int(bool(per_layer)), _ptr(expire),
                                              _ptr(prefix), _ptr(live)))
    return expire, prefix, live


def build_scale_window_schedule(layers: int, heads: int, scale_tokens: Sequence[int],
                                n_condensed: int, window: int, window_demanding: int,
                                similarity: Optional[Sequence[float]] = None,
                                n_demanding: int = 0) -> np.ndarray:
    """Condensed + local scale-window policy -> expire u8 [L][H][K]."""
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    K = int(tok.shape[0])
    sim = None
    if similarity is not None:
        sim = np.ascontiguousarray(similarity, dtype=np.float32)
        if sim.shape != (int(layers),):
            raise HeatKVError(HK_EINVAL, "similarity must have one score per layer")
    expire = np.zeros((int(layers), int(heads), K), dtype=np.uint8)
    _check(_lib.hk_build_scale_window_schedule(int(layers), int(heads), K, _ptr(tok),
                                               int(n_condensed), int(window),
                                               int(window_demanding),
                                               _ptr(sim) if sim is not None else None,
                                               int(n_demanding), _ptr(expire)))
    return expire


def cache_size_after_layer(scale_tokens: Sequence[int], expire: np.ndarray, step: int,
                           layer: int) -> int:
    """Token slots per sequence once ``layer`` has finished scale ``step``."""
    expire = np.ascontiguousarray(expire, dtype=np.uint8)
    L, H, K = expire.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    out = np.zeros(1, dtype=np.int64)
    _check(_lib.hk_cache_size_after_layer(L, H, K, _ptr(tok), _ptr(expire), int(step), int(layer),
                                          _ptr(out)))
    return int(out[0])


def layout_expiry(scale_tokens: Sequence[int], expire: np.ndarray, batch: int,
                  head_dim: int) -> Tuple[int, np.ndarray, np.ndarray]:
    """layout() for a schedule given as expiry steps."""
    expire = np.ascontiguousarray(expire, dtype=np.uint8)
    L, H, K = expire.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    elems = np.zeros(1, dtype=np.int64)
    cap = np.zeros((L, H), dtype=np.int64)
    base = np.zeros((L, H), dtype=np.int64)
    _check(_lib.hk_layout_expiry(L, H, K, _ptr(tok), _ptr(expire), int(batch), int(head_dim),
                                 _ptr(elems), _ptr(cap), _ptr(base)))
    return int(elems[0]), cap, base


def layout_pooled(scale_tokens: Sequence[int], expire: np.ndarray, batch: int, head_dim: int,
                  with_rows: bool = False):
    """(elements of each pool buffer, pool rows per batch entry[, segment rows]) of the
    pooled layout of an expiry-step schedule; segment rows [L][H][sum n_s, s <= K-2]
    (int32, -1 for segments never stored) when with_rows."""
    expire = np.ascontiguousarray(expire, dtype=np.uint8)
    L, H, K = expire.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    elems = np.zeros(1, dtype=np.int64)
    rows = np.zeros(1, dtype=np.int64)
    seg = np.zeros((L, H, int(tok[: K - 1].sum())), dtype=np.int32) if with_rows else None
    _check(_lib.hk_layout_pooled(L, H, K, _ptr(tok), _ptr(expire), int(batch), int(head_dim),
                                 _ptr(elems), _ptr(rows), _ptr(seg) if with_rows else None))
    if with_rows:
        return int(elems[0]), int(rows[0]), seg
    return int(elems[0]), int(rows[0])


def layout_int4(scale_tokens: Sequence[int], keep: np.ndarray, batch: int, head_dim: int,
                sub_blocks: int) -> Tuple[int, int]:
    """(bytes of each 4-bit store buffer, byte offset of its group parameters)."""
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    L, H, K = keep.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    nbytes = np.zeros(1, dtype=np.int64)
    poff = np.zeros(1, dtype=np.int64)
    _check(_lib.hk_layout_int4(L, H, K, _ptr(tok), _ptr(keep), int(batch), int(head_dim),
                               int(sub_blocks), _ptr(nbytes), _ptr(poff)))
    return int(nbytes[0]), int(poff[0])


def scas_mean(scas_sum: np.ndarray, images: float) -> np.ndarray:
    """S-CAS table [L][H][K][K] float32 from a streamed double sum and the image count."""
    scas_sum = np.ascontiguousarray(scas_sum, dtype=np.float64)
    if scas_sum.ndim != 4:
        raise HeatKVError(HK_EINVAL, "scas_sum must be [L][H][K][K]")
    L, H, K, _ = scas_sum.shape
    out = np.zeros(scas_sum.shape, dtype=np.float32)
    _check(_lib.hk_scas_mean(L, H, K, _ptr(scas_sum), float(images), _ptr(out)))
    return out


def ranking_stability(scas_a: np.ndarray, scas_b: np.ndarray, scale_tokens: Sequence[int],
                      budget_frac: float, n_sink: int) -> Tuple[np.ndarray, float]:
    """(Spearman rho per source scale [K] (NaN where not prunable), Jaccard of pruned sets)."""
    a = np.ascontiguousarray(scas_a, dtype=np.float32)
    b = np.ascontiguousarray(scas_b, dtype=np.float32)
    if a.shape != b.shape or a.ndim != 4:
        raise HeatKVError(HK_EINVAL, "tables must both be [L][H][K][K]")
    L, H, K, _ = a.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    rho = np.zeros(K, dtype=np.float64)
    jac = np.zeros(1, dtype=np.float64)
    _check(_lib.hk_ranking_stability(L, H, K, _ptr(tok), _ptr(a), _ptr(b), float(budget_frac),
                                     int(n_sink), _ptr(rho), _ptr(jac)))
    return rho, float(jac[0])


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


HK_NOALLOC_MAX_HEADS = 32
HK_NOALLOC_SCRATCH_BYTES = 4 << 20


def attend_noalloc(keep: np.ndarray, scale_tokens: Sequence[int], step: int,
                   k_cache: Optional[torch.Tensor], v_cache: Optional[torch.Tensor], q: torch.Tensor,
                   k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, softmax_scale: float,
                   scas_table: Optional[torch.Tensor] = None, stream=None) -> None:
    """hk_attend_noalloc: one layer's attention at scale ``step`` with no context
    and no allocation.  keep [H][K] (this layer's static keep-mask); k_cache /
    v_cache are views of that layer's cache (bf16, hk_layout order); q, k, v,
    out bf16 [B][n_step][H][128]; scas_table float32 [H][K][K] or None."""
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    if keep.ndim != 2:
        raise HeatKVError(HK_EINVAL, "keep must be [H][K]")
    H, K = keep.shape
    tok = np.ascontiguousarray(scale_tokens, dtype=np.int32)
    if tok.shape != (K,):
        raise HeatKVError(HK_EINVAL, "scale_tokens must have K entries")
    if not (0 <= step < K):
        raise HeatKVError(HK_EINVAL, f"step {step} out of range")
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise HeatKVError(HK_EINVAL, "q must be [B][n][H][128]")
    B = q.shape[0]
    want = (B, int(tok[step]), H, 128)
    for x, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        if (not isinstance(x, torch.Tensor) or tuple(x.shape) != want or x.dtype != torch.bfloat16
                or not x.is_cuda or not x.is_contiguous()):
            raise HeatKVError(HK_EINVAL, f"{nm} must be a contiguous bf16 device tensor {want}")
    ptrs = []
    for c in (k_cache, v_cache):
        if c is None:
            ptrs.append(None)
        else:
            if c.dtype != torch.bfloat16 or not c.is_cuda or not c.is_contiguous():
                raise HeatKVError(HK_EINVAL, "caches must be contiguous bf16 device tensors")
            ptrs.append(ctypes.c_void_p(c.data_ptr()))
    tab = None
    if scas_table is not None:
        if (tuple(scas_table.shape) != (H, K, K) or scas_table.dtype != torch.float32
                or not scas_table.is_cuda or not scas_table.is_contiguous()):
            raise HeatKVError(HK_EINVAL, f"scas_table must be a contiguous float32 {(H, K, K)} device tensor")
        tab = ctypes.c_void_p(scas_table.data_ptr())
    _check(_lib.hk_attend_noalloc(int(H), int(B), int(K), _ptr(tok), _ptr(keep), int(step), ptrs[0],
                                  ptrs[1], ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                  ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                  float(softmax_scale), tab, _stream(stream)))


class Context:
    """A library context for one model (L layers x H heads) and one batch shape.

    Allocates the two ragged caches (K and V) with PyTorch on the current
    device unless ``k_cache``/``v_cache`` are given, and keeps them alive for
    the context's lifetime.  The schedule is a static keep-mask ``keep``
    [L][H][K], or expiry steps ``expire`` [L][H][K] (pass ``keep=None``).
    With ``sub_blocks`` set (static keep-mask, bf16, head_dim 128) the cache
    is stored in 4 bits: ``k_cache``/``v_cache`` are then uint8 buffers of
    ``layout_int4`` bytes holding codes and group parameters.
    """

    def __init__(self, layers: int, heads: int, head_dim: int, batch: int,
                 scale_tokens: Sequence[int], keep: Optional[np.ndarray], dtype: torch.dtype,
                 k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                 device=None, expire: Optional[np.ndarray] = None,
                 sub_blocks: Optional[int] = None, pooled: bool = False):
        if dtype not in DTYPES:
            raise HeatKVError(HK_EUNSUPPORTED, f"dtype {dtype} not supported")
        self.sub_blocks = sub_blocks
        if sub_blocks is not None:
            self._init_int4(layers, heads, head_dim, batch, scale_tokens, keep, dtype, k_cache,
                            v_cache, device, int(sub_blocks))
            return
        self.L, self.H, self.D, self.B = int(layers), int(heads), int(head_dim), int(batch)
        self.tokens = tuple(int(x) for x in scale_tokens)
        self.K = len(self.tokens)
        self.dtype = dtype
        if (keep is None) == (expire is None):
            raise HeatKVError(HK_EINVAL, "give exactly one of keep and expire")
        sched = keep if expire is None else expire
        self.keep = np.ascontiguousarray(keep, dtype=np.uint8) if expire is None else None
        self.expire = np.ascontiguousarray(expire, dtype=np.uint8) if expire is not None else None
        if np.asarray(sched).shape != (self.L, self.H, self.K):
            raise HeatKVError(HK_EINVAL, "the schedule must be [L][H][K]")
        self.pooled = bool(pooled)
        self.pool_rows = None
        if self.pooled:
            if expire is None:
                raise HeatKVError(HK_EINVAL, "a pooled cache takes a schedule of expiry steps")
            self.cache_elems, self.pool_rows = layout_pooled(self.tokens, self.expire, self.B,
                                                             self.D)
            self.cap = np.full((self.L, self.H), self.pool_rows, dtype=np.int64)
            self.base = np.zeros((self.L, self.H), dtype=np.int64)
        elif expire is None:
            self.cache_elems, self.cap, self.base = layout(self.tokens, self.keep, self.B, self.D)
        else:
            self.cache_elems, self.cap, self.base = layout_expiry(self.tokens, self.expire, self.B,
                                                                  self.D)
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        n_alloc = max(self.cache_elems, 1)
        if k_cache is None:
            k_cache = torch.empty(n_alloc, dtype=dtype, device=dev)
        if v_cache is None:
            v_cache = torch.empty(n_alloc, dtype=dtype, device=dev)
        for c in (k_cache, v_cache):
            if c.dtype != dtype or not c.is_cuda or not c.is_contiguous() or c.numel() < self.cache_elems:
                raise HeatKVError(HK_EINVAL, "cache buffers must be contiguous device tensors "
                                             "of the context dtype with hk_layout() elements")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.device = k_cache.device
        tok = np.ascontiguousarray(self.tokens, dtype=np.int32)
        handle = ctypes.c_void_p()
        create = _lib.hk_create if expire is None else _lib.hk_create_expiry
        table = self.keep if expire is None else self.expire
        with torch.cuda.device(self.device):
            if self.pooled:
                _check(_lib.hk_create_pooled(ctypes.byref(handle), self.L, self.H, self.D, self.B,
                                             self.K, _ptr(tok), _ptr(table),
                                             ctypes.c_void_p(k_cache.data_ptr()),
                                             ctypes.c_void_p(v_cache.data_ptr())))
            else:
                _check(create(ctypes.byref(handle), self.L, self.H, self.D, self.B, self.K,
                              _ptr(tok), _ptr(table), DTYPES[dtype],
                              ctypes.c_void_p(k_cache.data_ptr()),
                              ctypes.c_void_p(v_cache.data_ptr())))
        self._h = handle

    def _init_int4(self, layers, heads, head_dim, batch, scale_tokens, keep, dtype, k_store,
                   v_store, device, m):
        if dtype != torch.bfloat16 or keep is None:
            raise HeatKVError(HK_EUNSUPPORTED, "4-bit storage takes bf16 tensors and a keep-mask")
        self.L, self.H, self.D, self.B = int(layers), int(heads), int(head_dim), int(batch)
        self.tokens = tuple(int(x) for x in scale_tokens)
        self.K = len(self.tokens)
        self.dtype = dtype
        self.expire = None
        self.keep = np.ascontiguousarray(keep, dtype=np.uint8)
        if self.keep.shape != (self.L, self.H, self.K):
            raise HeatKVError(HK_EINVAL, "keep must be [L][H][K]")
        self.store_bytes, self.param_offset = layout_int4(self.tokens, self.keep, self.B, self.D, m)
        _, self.cap, _ = layout(self.tokens, self.keep, self.B, self.D)
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        n_alloc = max(self.store_bytes, 16)
        if k_store is None:
            k_store = torch.empty(n_alloc, dtype=torch.uint8, device=dev)
        if v_store is None:
            v_store = torch.empty(n_alloc, dtype=torch.uint8, device=dev)
        for c in (k_store, v_store):
            if c.dtype != torch.uint8 or not c.is_cuda or not c.is_contiguous() or c.numel() < self.store_bytes:
                raise HeatKVError(HK_EINVAL, "4-bit stores must be contiguous uint8 device tensors "
                                             "of layout_int4() bytes")
        self.k_cache, self.v_cache = k_store, v_store
        self.device = k_store.device
        tok = np.ascontiguousarray(self.tokens, dtype=np.int32)
        handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check(_lib.hk_create_int4(ctypes.byref(handle), self.L, self.H, self.D, self.B, self.K,
                                       _ptr(tok), _ptr(self.keep), int(m),
                                       ctypes.c_void_p(k_store.data_ptr()),
                                       ctypes.c_void_p(v_store.data_ptr())))
        self._h = handle

    # -- argument checks (shapes the kernels and their grids assume) -------------------
    def _step_tensor(self, x: torch.Tensor, step: int, name: str) -> ctypes.c_void_p:
        want = (self.B, self.tokens[step], self.H, self.D)
        if not isinstance(x, torch.Tensor) or tuple(x.shape) != want:
            raise HeatKVError(HK_EINVAL, f"{name} must have shape {want}")
        if x.dtype != self.dtype or x.device != self.device or not x.is_contiguous():
            raise HeatKVError(HK_EINVAL, f"{name} must be a contiguous {self.dtype} tensor on {self.device}")
        return ctypes.c_void_p(x.data_ptr())

    def _handle(self):
        if self._h is None:
            raise HeatKVError(HK_EINVAL, "context is closed")
        return self._h

    # -- entry points -------------------------------------------------------------------
    def reset(self) -> None:
        _check(_lib.hk_reset(self._handle()))

    def attend(self, layer: int, step: int, q, k, v, out, softmax_scale: float,
               stream=None) -> None:
        if not (0 <= step < self.K):
            raise HeatKVError(HK_EINVAL, f"step {step} out of range")
        args = [self._step_tensor(t, step, nm) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
        _check(_lib.hk_attend(self._handle(), int(layer), int(step), *args, float(softmax_scale),
                              _stream(stream)))

    def attend_with_scas(self, layer: int, step: int, q, k, v, out, softmax_scale: float,
                         scas_table: torch.Tensor, stream=None) -> None:
        if not (0 <= step < self.K):
            raise HeatKVError(HK_EINVAL, f"step {step} out of range")
        args = [self._step_tensor(t, step, nm) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
        want = (self.L, self.H, self.K, self.K)
        if (tuple(scas_table.shape) != want or scas_table.dtype != torch.float32
                or scas_table.device != self.device or not scas_table.is_contiguous()):
            raise HeatKVError(HK_EINVAL, f"scas_table must be a contiguous float32 {want} device tensor")
        _check(_lib.hk_attend_with_scas(self._handle(), int(layer), int(step), *args,
                                        float(softmax_scale), ctypes.c_void_p(scas_table.data_ptr()),
                                        _stream(stream)))

    def attend_with_scas_sum(self, layer: int, step: int, q, k, v, out, softmax_scale: float,
                             scas_sum: torch.Tensor, stream=None) -> None:
        """attend_with_scas, adding the batch's per-image S-CAS sum into a float64 table."""
        if not (0 <= step < self.K):
            raise HeatKVError(HK_EINVAL, f"step {step} out of range")
        args = [self._step_tensor(t, step, nm) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
        want = (self.L, self.H, self.K, self.K)
        if (tuple(scas_sum.shape) != want or scas_sum.dtype != torch.float64
                or scas_sum.device != self.device or not scas_sum.is_contiguous()):
            raise HeatKVError(HK_EINVAL, f"scas_sum must be a contiguous float64 {want} device tensor")
        _check(_lib.hk_attend_with_scas_sum(self._handle(), int(layer), int(step), *args,
                                            float(softmax_scale), ctypes.c_void_p(scas_sum.data_ptr()),
                                            _stream(stream)))

    def attend_append(self, layer: int, step: int, q, k, v, out, softmax_scale: float,
                      scas_table: Optional[torch.Tensor] = None, stream=None) -> None:
        """attend (with S-CAS when a table is given), then append this scale of
        this layer; one launch for bf16."""
        if not (0 <= step < self.K):
            raise HeatKVError(HK_EINVAL, f"step {step} out of range")
        args = [self._step_tensor(t, step, nm) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
        table = None
        if scas_table is not None:
            want = (self.L, self.H, self.K, self.K)
            if (tuple(scas_table.shape) != want or scas_table.dtype != torch.float32
                    or scas_table.device != self.device or not scas_table.is_contiguous()):
                raise HeatKVError(HK_EINVAL, f"scas_table must be a contiguous float32 {want} device tensor")
            table = ctypes.c_void_p(scas_table.data_ptr())
        _check(_lib.hk_attend_append(self._handle(), int(layer), int(step), *args,
                                     float(softmax_scale), table, _stream(stream)))

    def append_scale(self, layer_begin: int, layer_end: int, step: int, k, v,
                     stream=None) -> None:
        """Compact scale ``step`` of layers [layer_begin, layer_end).

        With one layer, k and v are [B][n][H][D]; with several, they are
        [layers][B][n][H][D] (one contiguous tensor per layer range).
        """
        nl = int(layer_end) - int(layer_begin)
        if not (0 <= step < self.K):
            raise HeatKVError(HK_EINVAL, f"step {step} out of range")
        per = (self.B, self.tokens[step], self.H, self.D)
        stride = 0
        ptrs = []
        for t, nm in ((k, "k"), (v, "v")):
            shape = per if nl == 1 and t.dim() == 4 else (nl,) + per
            if tuple(t.shape) != shape or t.dtype != self.dtype or t.device != self.device \
                    or not t.is_contiguous():
                raise HeatKVError(HK_EINVAL, f"{nm} must be a contiguous {self.dtype} tensor of shape {shape}")
            ptrs.append(ctypes.c_void_p(t.data_ptr()))
            stride = int(np.prod(per))
        _check(_lib.hk_append_scale(self._handle(), int(layer_begin), int(layer_end), int(step),
                                    ptrs[0], ptrs[1], stride if nl > 1 else 0, _stream(stream)))

    def attend_plan(self, step: int, with_scas: bool = False) -> Tuple[int, int]:
        """(query rows per workgroup, key-range splits) of scale ``step``'s launch."""
        rows, splits = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.hk_attend_plan(self._handle(), int(step), int(bool(with_scas)),
                                   ctypes.byref(rows), ctypes.byref(splits)))
        return rows.value, splits.value

    def retained_tokens(self, step: int) -> int:
        out = ctypes.c_int64()
        _check(_lib.hk_retained_tokens(self._handle(), int(step), ctypes.byref(out)))
        return int(out.value)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            h, self._h = self._h, None
            _check(_lib.hk_destroy(h))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
