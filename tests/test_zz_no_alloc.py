"""hk_attend_noalloc, the attention entry point that allocates nothing, against
the context entry points on the same inputs and cache: two calls in a row,
the second on a smaller input, and its size limits."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from oracle import cache as ocache

import kv_cache_compression_attend_amd as hk
from _gpu import note, to_device

pytestmark = pytest.mark.gpu


def _prepare(wl, keep, step, seed=0):
    """A one-layer context driven through scales 0..step-1 (its cache then
    holds every kept segment before `step`), the inputs of `step`, and the
    context's own outputs for that step: attend_with_scas and attend."""
    ctx = hk.Context(1, wl.heads, 128, wl.batch, wl.scale_tokens, keep, torch.bfloat16)
    dev = []
    for t in range(step + 1):
        x = workloads.step_inputs(wl, 0, t, seed)
        dev.append(tuple(to_device(a, wl) for a in (x.q, x.k, x.v)))
    for t in range(step):
        q, k, v = dev[t]
        ctx.attend_append(0, t, q, k, v, torch.empty_like(q), wl.softmax_scale)
    q, k, v = dev[step]
    K = wl.n_scales
    ref_scas_out = torch.empty_like(q)
    ref_table = torch.zeros((1, wl.heads, K, K), dtype=torch.float32, device="cuda")
    ctx.attend_with_scas(0, step, q, k, v, ref_scas_out, wl.softmax_scale, ref_table)
    ref_out = torch.empty_like(q)
    ctx.attend(0, step, q, k, v, ref_out, wl.softmax_scale)
    torch.cuda.synchronize()
    return ctx, (q, k, v), ref_scas_out, ref_table[0], ref_out


def _noalloc(ctx, wl, keep, step, qkv, with_scas):
    q, k, v = qkv
    out = torch.full_like(q, float("nan"))
    K = wl.n_scales
    table = torch.full((wl.heads, K, K), float("nan"), dtype=torch.float32, device="cuda") \
        if with_scas else None
    hk.attend_noalloc(keep[0], wl.scale_tokens, step, ctx.k_cache, ctx.v_cache, q, k, v, out,
                      wl.softmax_scale, table)
    return out, table


def _check(wl, step, ref_scas_out, ref_table, ref_out, got_scas, got_table, got_plain):
    # With S-CAS: the same kernels in the same plan, so bit for bit.
    assert torch.equal(got_scas.view(torch.int16), ref_scas_out.view(torch.int16))
    assert torch.equal(got_table[:, step, : step + 1], ref_table[:, step, : step + 1])
    # Without: the context's launch may split the key range (a different
    # summation order); the bf16 bar of the parity tests applies.
    e = (got_plain.float() - ref_out.float()).abs()
    assert torch.isfinite(got_plain.float()).all()
    assert float(e.max()) <= 1e-2 and float(e.mean()) <= 1e-3, (float(e.max()), float(e.mean()))


def test_noalloc_matches_context_entry_points_two_calls():
    # call 1: the full-cache Infinity-2B-shaped layer at its final scale
    big = workloads.get("c1")
    keep_big = workloads.full_keep(big)
    step_big = big.n_scales - 1
    # call 2: a smaller, pruned layer (3 heads, batch 2) at a middle scale
    small = workloads.Workload(index=95, name="noalloc-small", layers=1, heads=3, head_dim=128,
                               batch=2, sides=(1, 2, 3, 4, 6, 8, 12), dtype="bf16", budget=1.0,
                               n_sink=1, softmax_scale=1.0, qk_std=128 ** -0.25, schedule="custom")
    keep_small = np.ones((1, 3, small.n_scales), dtype=np.uint8)
    keep_small[0, :, -1] = 0
    keep_small[0, 1, 2:4] = 0
    keep_small[0, 2, 1:] = 0
    step_small = 5
    note("noalloc: references from the context entry points")
    ctx_b, qkv_b, rs_b, rt_b, ro_b = _prepare(big, keep_big, step_big)
    ctx_s, qkv_s, rs_s, rt_s, ro_s = _prepare(small, keep_small, step_small)
    assert ocache.capacity(keep_small, small.scale_tokens)[0].tolist() == list(ctx_s.cap[0])
    note("noalloc: call 1 (16 heads, 4096 queries), then call 2 (3 heads, 64 queries)")
    got_b = _noalloc(ctx_b, big, keep_big, step_big, qkv_b, True)
    got_s = _noalloc(ctx_s, small, keep_small, step_small, qkv_s, True)
    plain_b = _noalloc(ctx_b, big, keep_big, step_big, qkv_b, False)[0]
    plain_s = _noalloc(ctx_s, small, keep_small, step_small, qkv_s, False)[0]
    torch.cuda.synchronize()
    _check(big, step_big, rs_b, rt_b, ro_b, got_b[0], got_b[1], plain_b)
    _check(small, step_small, rs_s, rt_s, ro_s, got_s[0], got_s[1], plain_s)
    # the small call again after the large one, then the large again: the
    # shared scratch keeps only the last call's contents and nothing leaks
    again_s = _noalloc(ctx_s, small, keep_small, step_small, qkv_s, True)
    torch.cuda.synchronize()
    _check(small, step_small, rs_s, rt_s, ro_s, again_s[0], again_s[1], plain_s)
    ctx_b.close()
    ctx_s.close()


def test_noalloc_limits():
    K = 13
    tok = np.array(workloads.get("c1").scale_tokens, dtype=np.int32)
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: the call is refused first
    # more heads than the entry point holds tables for
    keep = np.ones((33, K), dtype=np.uint8)
    rc = hk._lib.hk_attend_noalloc(33, 1, K, hk._ptr(tok), hk._ptr(keep), 12, fake, fake, fake,
                                   fake, fake, fake, 1.0, None, None)
    assert rc == hk.HK_EINVAL and b"at most 32 heads" in hk._lib.hk_last_error()
    # S-CAS partial sums beyond the scratch array: 128 x 32 x 16 query tiles
    keep = np.ones((32, K), dtype=np.uint8)
    rc = hk._lib.hk_attend_noalloc(32, 128, K, hk._ptr(tok), hk._ptr(keep), 12, fake, fake, fake,
                                   fake, fake, fake, 1.0, fake, None)
    assert rc == hk.HK_EINVAL and b"partial sums" in hk._lib.hk_last_error()
    # misaligned pointer
    rc = hk._lib.hk_attend_noalloc(16, 1, K, hk._ptr(tok), hk._ptr(keep[:16].copy()), 3,
                                   ctypes.c_void_p((1 << 20) + 2), fake, fake, fake, fake, fake,
                                   1.0, None, None)
    assert rc == hk.HK_EINVAL
