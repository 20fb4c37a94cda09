"""Shared test helpers: oracle evaluation of the workloads and the parity check.

The oracle side (fp64 NumPy) and the GPU side receive the same synthetic bytes; no
expected value comes from the GPU path."""

from __future__ import annotations

import math

import numpy as np

from oracle import LayerKVCache, attention_layer_step

# Parity bar: every element satisfies |gpu - ref| <= atol + rtol * |ref|.
TOL_BF16 = (2e-2, 2e-2)
TOL_F32 = (1e-4, 1e-4)
# The score operands Q' and K' of a bf16 layer are IEEE halves (11 significant bits): one
# rounding of an fp32 value is within 2^-11 relative, under this bar with room for the fp32
# arithmetic before it.
TOL_F16 = (2e-3, 2e-3)


def parity(gpu, ref, tol):
    """Return (ok, max_abs, max_rel, worst_index) for the elementwise bar."""
    atol, rtol = tol
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    ok = bool(np.all(err <= bound)) and bool(np.all(np.isfinite(gpu)))
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / np.maximum(np.abs(ref), atol)).max()) if err.size else 0.0
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape) if err.size else None
    return ok, max_abs, max_rel, worst


def assert_parity(gpu, ref, tol, what=""):
    ok, ma, mr, worst = parity(gpu, ref, tol)
    assert ok, f"{what}: max_abs={ma:.3e} max_rel={mr:.3e} worst={worst}"
    return ma, mr


def oracle_prefill(q, k, v, *, window, rope, wq=None, wk=None, norm_offset=1.0, eps=1e-6,
                   scale=None, rows=None, legacy_4k=False):
    """Oracle of a prefill from an empty cache for every sequence: q [B,T,Hq,d] etc.
    Returns [B, T or len(rows), Hq, d] float64."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    outs = []
    for b in range(B):
        cache = LayerKVCache(Hkv, d, window, legacy_4k)
        outs.append(attention_layer_step(
            q[b], k[b], v[b], cache, theta=rope.theta, yarn_factor=rope.yarn_factor,
            orig_ctx=rope.orig_ctx, beta_fast=rope.beta_fast, beta_slow=rope.beta_slow,
            q_norm_w=wq, k_norm_w=wk, norm_offset=norm_offset, eps=eps,
            scale=scale if scale is not None else 1.0 / math.sqrt(d), rows=rows))
    return np.stack(outs)


def oracle_decode_one(q, k, v, prior_k, prior_v, pos_offset, *, window, rope, wq, wk,
                      norm_offset=1.0, eps=1e-6, legacy_4k=False, post_rope=False):
    """Oracle of one decode step of one sequence: q [1,Hq,d], k/v [1,Hkv,d]; prior_k/v are
    the kept tokens (normalised pre-RoPE K, raw V) in token order. Returns [1, Hq, d]."""
    cache = LayerKVCache.with_prior(prior_k, prior_v, pos_offset, window, legacy_4k, post_rope)
    return attention_layer_step(
        q, k, v, cache, theta=rope.theta, yarn_factor=rope.yarn_factor, orig_ctx=rope.orig_ctx,
        beta_fast=rope.beta_fast, beta_slow=rope.beta_slow, q_norm_w=wq, k_norm_w=wk,
        norm_offset=norm_offset, eps=eps, scale=1.0 / math.sqrt(q.shape[-1]))


def kept_slots(pos_offset, window):
    """Cache slots of the tokens a layer keeps before appending token pos_offset, in
    token order (ring slot n mod W on local layers)."""
    kept = pos_offset if window == 0 else min(pos_offset, window - 1)
    toks = np.arange(pos_offset - kept, pos_offset)
    return toks if window == 0 else toks % window


def window_mean_closed_form(v, window):
    """Uniform attention over the visible keys: O[t] = mean of V over the window
    ending at t (prefix sums in fp64). v [T, Hkv, d] -> [T, Hkv, d]."""
    v = np.asarray(v, dtype=np.float64)
    T = v.shape[0]
    csum = np.concatenate([np.zeros((1,) + v.shape[1:]), np.cumsum(v, axis=0)])
    t = np.arange(T)
    lo = np.zeros(T, dtype=np.int64) if window == 0 else np.maximum(0, t - window + 1)
    return (csum[t + 1] - csum[lo]) / (t + 1 - lo)[:, None, None]


def untile_k_rot(kr):
    """bf16 K' operand [B, Hkv, Tp/64, d/8, 64, 8] (include/plamo_attn.h) -> [B, Hkv, Tp, d]."""
    B, H, nt, nc, kt, w = kr.shape
    return kr.transpose(0, 1, 2, 4, 3, 5).reshape(B, H, nt * kt, nc * w)


def untile_v_t(vt):
    """bf16 V^T operand [B, Hkv, Tp/64, 8, d, 8] (include/plamo_attn.h) -> [B, Hkv, d, Tp]."""
    B, H, nt, nc, d, w = vt.shape
    return vt.transpose(0, 1, 4, 2, 3, 5).reshape(B, H, d, nt * nc * w)


def oracle_chunks(q, k, v, chunks, *, window, rope, wq=None, wk=None, norm_offset=1.0, eps=1e-6,
                  rows_of=None, legacy_4k=False, post_rope=False, caches_out=None):
    """Oracle of a prefill in consecutive chunks (each chunk attends the cache the previous
    ones left, then updates it): q [B,n,Hq,d] etc., chunks = chunk lengths summing to n.
    rows_of(T) -> row indices kept per chunk (default all). Returns a list per chunk of
    [B, rows, Hq, d] float64."""
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    caches = [LayerKVCache(Hkv, d, window, legacy_4k, post_rope) for _ in range(B)]
    if caches_out is not None:
        caches_out.extend(caches)
    outs, p = [], 0
    for T in chunks:
        rows = None if rows_of is None else rows_of(T)
        outs.append(np.stack([attention_layer_step(
            q[b, p:p + T], k[b, p:p + T], v[b, p:p + T], caches[b], theta=rope.theta,
            yarn_factor=rope.yarn_factor, orig_ctx=rope.orig_ctx, beta_fast=rope.beta_fast,
            beta_slow=rope.beta_slow, q_norm_w=wq, k_norm_w=wk, norm_offset=norm_offset, eps=eps,
            scale=1.0 / math.sqrt(d), rows=rows) for b in range(B)]))
        p += T
    return outs
