"""CPU oracle (NumPy, float64) for PLaMo 3's hybrid sliding-window / global
grouped-query attention, for prefill and for KV-cached decode.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Each function writes out the plain definition that the pages give, in float64,
with no tiling, fusion or reordering beyond evaluating independent query rows in
slices to bound memory. Inputs are the exact values of the tensors the GPU
receives (bf16 or fp32, promoted to float64).

Sources (page title, section):
  [P3] 「PLaMo 3アーキテクチャ徹底解析」 (imoz.jp, 2026-10-26)
       §2.1 configuration; §2.3 decode read volume; §3.2 offset RMSNorm;
       §4.2 GQA head sharing; §4.3 per-head Q/K norm; §4.4 order of cache update
       and RoPE, renumbered positions, local cache trimming; §4.5 attention
       equation; §5.1 causal and window masks; §5.2 KV capacity; §6.1 split-half
       RoPE; §6.2 bases; §6.3 YaRN; §6.4 p-RoPE; §8 comparison table (the
       Gemma-4-shaped layer: gain-only Q/K norm, gainless V norm, dot-product factor 1,
       K stored after RoPE); §9.4 constant Q/K gains of that layer.
  [TR] 「Transformerと大規模言語モデル 技術解説」 (troy-technical.jp), §4 worked
       attention example (Fig. 3).

Pins: every function here is checked in tests/test_oracle.py against values the
pages print, closed forms, library routines or brute force. None is "parity
unpinned".
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# Offset RMSNorm  [P3 §3.2, §4.3]
# ----------------------------------------------------------------------------

def offset_rms_norm(x, w, c: float, eps: float = 1e-6) -> np.ndarray:
    """[P3 §3.2] N_w^(c)(x) = (c + w) * x / sqrt(mean_r x_r^2 + eps) over the last axis.

    The effective gain is the stored weight plus the constant offset c. For the
    per-head Q/K norm [P3 §4.3] the last axis is one head's 128 components and the
    same [d] gain serves every head."""
    x = np.asarray(x, dtype=F64)
    gain = c + np.asarray(w, dtype=F64)
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(mean_sq + eps))


# ----------------------------------------------------------------------------
# RoPE with optional YaRN  [P3 §6.1-§6.3]
# ----------------------------------------------------------------------------

def yarn_ramp_bounds(d: int, theta: float, orig_ctx: float, beta_fast: float,
                     beta_slow: float) -> tuple[float, float]:
    """[P3 §6.3] Pair-index bounds of the interpolation ramp, left unrounded.

    The pages write the leading factor as 64, which is d/2 for d = 128; the
    general form uses d/2."""
    half = d / 2.0
    j_low = half * math.log(orig_ctx / (2.0 * math.pi * beta_fast)) / math.log(theta)
    j_high = half * math.log(orig_ctx / (2.0 * math.pi * beta_slow)) / math.log(theta)
    return j_low, j_high


def rope_frequencies(d: int, theta: float, yarn_factor: float = 0.0,
                     orig_ctx: float = 4096.0, beta_fast: float = 32.0,
                     beta_slow: float = 1.0, partial: float = 1.0) -> tuple[np.ndarray, float]:
    """Angular frequency per rotation pair and the amplitude factor.

    [P3 §6.1] omega_j = theta^(-2j/d), j = 0 .. d/2-1.
    [P3 §6.3] With YaRN factor s > 1: alpha_j = clip((j - j_low)/(j_high - j_low), 0, 1),
    omega~_j = omega_j * ((1 - alpha_j) + alpha_j / s), and cos and sin are both
    scaled by 1 + 0.1 ln s. Without YaRN the amplitude is 1.
    [P3 §6.4] p-RoPE (partial < 1): only the floor(p * d/2) highest-frequency pairs
    turn, still with the exponent over the whole head dim d; the other pairs get
    frequency 0 (cos 1, sin 0: left as they are). Not combined with YaRN."""
    j = np.arange(d // 2, dtype=F64)
    if partial < 1.0:
        if yarn_factor is not None and yarn_factor > 1.0:
            raise ValueError("p-RoPE is not combined with YaRN")
        n_rot = int(math.floor(partial * (d // 2)))
        omega = np.where(j < n_rot, np.power(F64(theta), -2.0 * j / d), 0.0)
        return omega, 1.0
    omega = np.power(F64(theta), -2.0 * j / d)
    if yarn_factor is None or yarn_factor <= 1.0:
        return omega, 1.0
    j_low, j_high = yarn_ramp_bounds(d, theta, orig_ctx, beta_fast, beta_slow)
    alpha = np.clip((j - j_low) / (j_high - j_low), 0.0, 1.0)
    omega = omega * ((1.0 - alpha) + alpha / yarn_factor)
    amplitude = 1.0 + 0.1 * math.log(yarn_factor)
    return omega, amplitude


def apply_rope(x, positions, omega, amplitude: float) -> np.ndarray:
    """[P3 §6.1] Split-half rotation: components j and j + d/2 form pair j and turn by
    the angle p * omega_j, (a, b) -> (a cos - b sin, a sin + b cos); [P3 §6.3] the
    result is scaled by the amplitude.

    x: [T, H, d] (token-major, as the layer sees it); positions: [T]."""
    x = np.asarray(x, dtype=F64)
    half = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=F64)[:, None] * np.asarray(omega, dtype=F64)[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = amplitude * (a * cos - b * sin)
    out[..., half:] = amplitude * (a * sin + b * cos)
    return out


# ----------------------------------------------------------------------------
# Masks and attention  [P3 §4.2, §4.5, §5.1]
# ----------------------------------------------------------------------------

def allowed(q_pos, k_pos, window: int, legacy_4k: bool = False) -> np.ndarray:
    """[P3 §5.1] Query at position i may read key at position j iff j <= i, and on a
    local layer (window W > 0) also i - j < W, so W keys including itself.

    legacy_4k: the band of the implementation shipped with the 4K release (same section),
    which reads up to distance W, i.e. W + 1 keys including itself."""
    i = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.asarray(k_pos, dtype=np.int64)[None, :]
    ok = j <= i
    if window > 0:
        if legacy_4k:
            ok &= (i - j) <= window
        else:
            ok &= (i - j) < window
    return ok


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """[P3 §4.2, §4.5] Consecutive query heads share a KV head: g(h) = floor(h / (Hq/Hkv))."""
    return h // (Hq // Hkv)


def gqa_attention(q_rot, k_rot, v, q_pos, k_pos, window: int, scale: float,
                  rows_per_slice: int = 512, return_weights: bool = False, legacy_4k: bool = False):
    """[P3 §4.5] A = softmax_s(Q'K'^T * scale + M), O = A V, per query head, with
    M = 0 where allowed and -inf elsewhere; K/V head g(h) for query head h.

    q_rot [T, Hq, d]; k_rot, v [S, Hkv, d]; q_pos [T]; k_pos [S].
    Returns out [T, Hq, d] (and, on request, the weights [Hq, T, S])."""
    q_rot = np.asarray(q_rot, dtype=F64)
    k_rot = np.asarray(k_rot, dtype=F64)
    v = np.asarray(v, dtype=F64)
    T, Hq, d = q_rot.shape
    S, Hkv, _ = k_rot.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    out = np.zeros((T, Hq, d), dtype=F64)
    weights = np.zeros((Hq, T, S), dtype=F64) if return_weights else None
    for r0 in range(0, T, rows_per_slice):
        r1 = min(T, r0 + rows_per_slice)
        mask = allowed(q_pos[r0:r1], k_pos, window, legacy_4k)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            scores = (q_rot[r0:r1, h, :] @ k_rot[:, g, :].T) * scale
            scores = np.where(mask, scores, -np.inf)
            row_max = np.max(scores, axis=1, keepdims=True)
            e = np.exp(scores - row_max)
            a = e / np.sum(e, axis=1, keepdims=True)
            out[r0:r1, h, :] = a @ v[:, g, :]
            if return_weights:
                weights[h, r0:r1, :] = a
    if return_weights:
        return out, weights
    return out


# ----------------------------------------------------------------------------
# KV cache model and the layer step  [P3 §4.4]
# ----------------------------------------------------------------------------

class LayerKVCache:
    """[P3 §4.4] KV cache of one attention layer for one sequence.

    Stores normalised K before RoPE and raw V. A global layer (window 0) keeps
    every token. A local layer keeps, after each update, at most the last W - 1
    tokens; the update itself returns all previously kept tokens plus the new
    ones, and that is what attention reads. legacy_4k: the cache class of the 4K
    release's implementation (§5.1), which keeps the last W tokens, for its W + 1 band.

    post_rope: the other order the page contrasts with PLaMo's (§4.4, the Gemma-style
    layer): K is rotated at its absolute position before it is stored, queries are
    rotated at theirs, and the cache returns K ready for use."""

    def __init__(self, Hkv: int, d: int, window: int, legacy_4k: bool = False, post_rope: bool = False):
        self.window = int(window)
        self.legacy_4k = bool(legacy_4k)
        self.post_rope = bool(post_rope)
        self.k = np.zeros((0, Hkv, d), dtype=F64)
        self.v = np.zeros((0, Hkv, d), dtype=F64)
        self.seen = 0  # tokens appended so far (absolute position of the next token)

    @classmethod
    def with_prior(cls, k_prior, v_prior, seen: int, window: int, legacy_4k: bool = False,
                   post_rope: bool = False):
        """A cache that already holds ``k_prior``/``v_prior`` [n, Hkv, d] as its kept
        tokens (as stored: rotated when post_rope), after ``seen`` tokens in total."""
        k_prior = np.asarray(k_prior, dtype=F64)
        c = cls(k_prior.shape[1], k_prior.shape[2], window, legacy_4k, post_rope)
        keep = k_prior.shape[0]
        expect = seen if window == 0 else min(seen, window if legacy_4k else window - 1)
        if keep != expect:
            raise ValueError(f"a cache after {seen} tokens keeps {expect}, got {keep}")
        c.k = k_prior.copy()
        c.v = np.asarray(v_prior, dtype=F64).copy()
        c.seen = seen
        return c

    def update(self, k_new, v_new):
        k_all = np.concatenate([self.k, np.asarray(k_new, dtype=F64)], axis=0)
        v_all = np.concatenate([self.v, np.asarray(v_new, dtype=F64)], axis=0)
        self.seen += np.asarray(k_new).shape[0]
        n = k_all.shape[0]
        keep = n if self.window == 0 else min(n, self.window - 1)
        if self.legacy_4k and self.window > 0:
            keep = min(n, self.window)
        self.k = k_all[n - keep:]
        self.v = v_all[n - keep:]
        return k_all, v_all


def attention_layer_step(q, k, v, cache: LayerKVCache, *, theta: float,
                         yarn_factor: float = 0.0, orig_ctx: float = 4096.0,
                         beta_fast: float = 32.0, beta_slow: float = 1.0,
                         q_norm_w=None, k_norm_w=None, norm_offset: float = 1.0,
                         eps: float = 1e-6, scale: float | None = None,
                         rows=None, return_intermediates: bool = False,
                         partial: float = 1.0, v_norm: bool = False):
    """One attention layer for one sequence, in the order of [P3 §4.4]:
    per-head Q/K RMSNorm -> cache update -> RoPE on the current Q and on every K the
    cache returns -> masked GQA attention. (A post_rope cache instead rotates K at its
    absolute position before the update and Q at its absolute position.)

    The Gemma-4-shaped layer of [P3 §8] is this step with norm_offset 0 (the gain is the
    stored weight itself), scale 1, a post_rope cache, p-RoPE on its global layer
    (``partial``, [P3 §6.4]) and ``v_norm``: each new V head vector is divided by its
    RMS (RMSNorm without gain, same eps) before it enters the cache.

    q [T, Hq, d]; k, v [T, Hkv, d] (projected, before norm). Positions are the
    internal running numbers of [P3 §4.4]: the S keys returned by the cache get
    0 .. S-1 and the T queries get S-T .. S-1. ``rows`` optionally restricts the
    output to a subset of the T query rows (same values as the full evaluation).
    Returns out [T or len(rows), Hq, d]."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    T, Hq, d = q.shape
    if (q_norm_w is None) != (k_norm_w is None):
        raise ValueError("give both norm weights or neither")
    if q_norm_w is not None:
        q = offset_rms_norm(q, q_norm_w, norm_offset, eps)
        k = offset_rms_norm(k, k_norm_w, norm_offset, eps)
    if v_norm:
        v = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    omega, amp = rope_frequencies(d, theta, yarn_factor, orig_ctx, beta_fast, beta_slow, partial)
    if cache.post_rope:
        # rotate the new K at its absolute positions, then store; the cache returns the
        # rotated K of the kept tokens and the new ones; queries at absolute positions
        first = cache.seen
        k_all, v_all = cache.update(apply_rope(k, np.arange(first, first + T), omega, amp), v)
        S = k_all.shape[0]
        k_pos = np.arange(first + T - S, first + T)
        q_pos = np.arange(first, first + T)
    else:
        k_all, v_all = cache.update(k, v)
        S = k_all.shape[0]
        k_pos = np.arange(S)
        q_pos = np.arange(S - T, S)
    if rows is not None:
        rows = np.asarray(rows)
        q = q[rows]
        q_pos = q_pos[rows]
    q_rot = apply_rope(q, q_pos, omega, amp)
    k_rot = k_all if cache.post_rope else apply_rope(k_all, k_pos, omega, amp)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = gqa_attention(q_rot, k_rot, v_all, q_pos, k_pos, cache.window, scale,
                        legacy_4k=cache.legacy_4k)
    if return_intermediates:
        return out, dict(q_norm=q, k_all=k_all, v_all=v_all, q_rot=q_rot, k_rot=k_rot,
                         q_pos=q_pos, k_pos=k_pos)
    return out


# ----------------------------------------------------------------------------
# The attention sublayer around the hot path  [P3 §3.2, §4.1, §4.5]
# ----------------------------------------------------------------------------

def mixer_layer_step(x, cache: LayerKVCache, *, w_pre, w_qkv, w_o, w_post, Hq: int, Hkv: int,
                     theta: float, yarn_factor: float = 0.0, q_norm_w=None, k_norm_w=None,
                     pre_offset: float = 1.0, post_offset: float = 0.2, qk_offset: float = 1.0,
                     eps: float = 1e-6, rows=None):
    """One attention sublayer for one sequence: x [T, D] -> x + post(o_proj(attn(pre(x)))).

    [P3 §3.2] pre_mixer_norm (offset 1) and post_mixer_norm (offset 0.2) over the D hidden
    components; [P3 §4.1] one fused projection U W_qkv^T, W_qkv [(Hq + 2 Hkv) d, D], whose
    output is split along its last axis into Q [0, Hq d), K [Hq d, (Hq + Hkv) d) and
    V [(Hq + Hkv) d, (Hq + 2 Hkv) d), each reshaped to [T, H, d]; the attention layer step
    of [P3 §4.4]; [P3 §4.5] the heads concatenated to [T, Hq d] and projected by
    W_o [D, Hq d]. The normalised output is added to the residual stream x (reading: the
    post norm acts on the sublayer output before the residual add). ``rows`` restricts
    the returned rows (every token still enters the cache)."""
    x = np.asarray(x, dtype=F64)
    T, D = x.shape
    w_qkv = np.asarray(w_qkv, dtype=F64)
    d = w_qkv.shape[0] // (Hq + 2 * Hkv)
    u = offset_rms_norm(x, w_pre, pre_offset, eps)
    qkv = u @ w_qkv.T
    q = qkv[:, :Hq * d].reshape(T, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(T, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(T, Hkv, d)
    attn = attention_layer_step(q, k, v, cache, theta=theta, yarn_factor=yarn_factor,
                                q_norm_w=q_norm_w, k_norm_w=k_norm_w, norm_offset=qk_offset,
                                eps=eps, rows=rows)
    o = attn.reshape(attn.shape[0], Hq * d) @ np.asarray(w_o, dtype=F64).T
    xr = x if rows is None else x[np.asarray(rows)]
    return xr + offset_rms_norm(o, w_post, post_offset, eps)


# ----------------------------------------------------------------------------
# Read volume and capacity accounting  [P3 §2.3, §5.2]
# ----------------------------------------------------------------------------

def attended_keys_total(N: int, window: int, n_global: int, n_local: int) -> int:
    """[P3 §2.3] A = N_g * N + N_l * min(N, W): keys read per token over all layers."""
    return n_global * N + n_local * min(N, window)


def kv_bytes(B: int, Hkv: int, d: int, attended: int, elem_bytes: int = 2) -> int:
    """[P3 §2.3, §5.2] K and V of every attended key, once per sequence and KV head:
    2 * elem_bytes * B * Hkv * d * A bytes (4 B Hkv d A for bf16)."""
    return 2 * elem_bytes * B * Hkv * d * attended
