"""Pins for the CPU oracle: values the pages print, closed forms, library routines and
brute force. Each pin is a function of the oracle module, so that
``test_planted_mistakes_are_caught`` can run every pin against copies of the oracle
with one plausible mistake planted in each and check that some pin fails.

CPU only (no GPU marker)."""

from __future__ import annotations

import importlib.util
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as oracle_pkg
from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
ORACLE_SRC = os.path.abspath(O.__file__)


def golden(name):
    with open(os.path.join(GOLDEN, name), "r", encoding="utf-8") as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# pins (each takes the oracle module)
# ----------------------------------------------------------------------------

def pin_worked_example(o):
    """「Transformerと大規模言語モデル 技術解説」 §4, Fig. 3: weights and outputs as printed."""
    g = golden("worked_example_attention.json")
    Q = np.array(g["Q"], dtype=float)[:, None, :]
    K = np.array(g["K"], dtype=float)[:, None, :]
    V = np.array(g["V"], dtype=float)[:, None, :]
    pos = np.arange(3)
    out, w = o.gqa_attention(Q, K, V, pos, pos, 0, 1.0 / math.sqrt(g["d"]), return_weights=True)
    half_unit = 0.5 * 10 ** (-g["printed_decimals"]) + 1e-9
    for t, row in enumerate(g["printed_weights"]):
        for s, pw in enumerate(row):
            if pw is None:
                assert w[0, t, s] == 0.0
            else:
                assert abs(w[0, t, s] - pw) <= half_unit, (t, s, w[0, t, s], pw)
    for t, po in enumerate(g["printed_outputs"]):
        for r in range(2):
            assert abs(out[t, 0, r] - po[r]) <= half_unit, (t, r, out[t, 0, r], po[r])


def pin_fig4_masks(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §5.1 Fig. 4: global and W=4 local patterns."""
    g = golden("mask_fig4_w4.json")
    n = g["tokens"]
    pos = np.arange(n)
    for key, W in (("global", 0), ("local", g["window"])):
        want = np.array([[c == "1" for c in row] for row in g[key]])
        got = o.allowed(pos, pos, W)
        assert np.array_equal(got, want), (key, got.astype(int))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_sdpa_float64(o):
    """Library cross-check: torch scaled_dot_product_attention in float64 with an explicit
    boolean mask; GQA both by repeat_interleave of K/V heads and by enable_gqa."""
    for (T, Hq, Hkv, d, W, seed) in [(9, 4, 2, 8, 0, 1), (17, 6, 3, 16, 5, 2), (13, 8, 8, 4, 1, 3),
                                     (11, 4, 1, 8, 4, 4)]:
        q, k, v = _rand((T, Hq, d), seed), _rand((T, Hkv, d), seed + 10), _rand((T, Hkv, d), seed + 20)
        pos = np.arange(T)
        scale = 1.0 / math.sqrt(d)
        got = o.gqa_attention(q, k, v, pos, pos, W, scale)
        mask = torch.ones(T, T, dtype=torch.bool).tril()
        if W > 0:
            mask &= ~torch.ones(T, T, dtype=torch.bool).tril(-W)
        qt = torch.from_numpy(q).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None]
        vt = torch.from_numpy(v).permute(1, 0, 2)[None]
        G = Hq // Hkv
        ref1 = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.repeat_interleave(G, 1), vt.repeat_interleave(G, 1), attn_mask=mask, scale=scale)
        ref2 = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
        for ref in (ref1, ref2):
            ref = ref[0].permute(1, 0, 2).numpy()
            assert np.max(np.abs(got - ref)) < 1e-12


def _brute_layer(q, k, v, prior_k, prior_v, W, theta, yarn, wq, wk, c, eps, n_rot=None,
                 v_norm=False, scale=None):
    """Pure-Python scalar evaluation of one layer step: norm, cache, RoPE, attention.
    n_rot: only pairs j < n_rot turn (p-RoPE); v_norm: new V rows divided by their RMS;
    scale: factor on the dot product (default 1/sqrt(d))."""
    T, Hq, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    half = d // 2

    def norm(x, w):
        ms = sum(e * e for e in x) / len(x)
        r = 1.0 / math.sqrt(ms + eps)
        return [(c + w[i]) * x[i] * r for i in range(len(x))]

    if wq is not None:
        q = [[norm(q[t][h], wq) for h in range(Hq)] for t in range(T)]
        k = [[norm(k[t][h], wk) for h in range(Hkv)] for t in range(T)]
    if v_norm:
        v = [[norm(v[t][h], [1.0 - c] * d) for h in range(Hkv)] for t in range(T)]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    keys = [list(map(list, r)) for r in prior_k] + k
    vals = [list(map(list, r)) for r in prior_v] + v
    S = len(keys)
    omega = []
    amp = 1.0
    for j in range(half):
        w0 = theta ** (-2.0 * j / d) if n_rot is None or j < n_rot else 0.0
        if yarn:
            lo = half * math.log(4096 / (2 * math.pi * 32)) / math.log(theta)
            hi = half * math.log(4096 / (2 * math.pi * 1)) / math.log(theta)
            a = min(1.0, max(0.0, (j - lo) / (hi - lo)))
            w0 = w0 * ((1 - a) + a / yarn)
            amp = 1 + 0.1 * math.log(yarn)
        omega.append(w0)

    def rot(x, p):
        y = [0.0] * d
        for j in range(half):
            cs, sn = math.cos(p * omega[j]), math.sin(p * omega[j])
            y[j] = amp * (x[j] * cs - x[j + half] * sn)
            y[j + half] = amp * (x[j] * sn + x[j + half] * cs)
        return y

    G = Hq // Hkv
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(T)]
    for t in range(T):
        i = S - T + t
        for h in range(Hq):
            qr = rot(q[t][h], i)
            g = h // G
            sc = []
            for s in range(S):
                if s <= i and (W == 0 or i - s < W):
                    kr = rot(keys[s][g], s)
                    sc.append((s, sum(qr[r] * kr[r] for r in range(d)) * scale))
            m = max(x for _, x in sc)
            e = [(s, math.exp(x - m)) for s, x in sc]
            z = sum(x for _, x in e)
            for r in range(d):
                out[t][h][r] = sum(wt * vals[s][g][r] for s, wt in e) / z
    return np.array(out)


def pin_bruteforce_layer(o):
    """Brute force on tiny inputs: the whole layer step (norm, cache, RoPE, mask, GQA)
    against scalar loops, with and without a populated cache."""
    cases = [
        dict(T=5, Hq=4, Hkv=2, d=8, W=3, theta=1e4, yarn=0, prior=0, norm=True, seed=5),
        dict(T=4, Hq=4, Hkv=1, d=8, W=0, theta=1e6, yarn=256.0, prior=3, norm=True, seed=6),
        dict(T=1, Hq=2, Hkv=2, d=4, W=4, theta=1e4, yarn=0, prior=3, norm=False, seed=7),
        dict(T=6, Hq=2, Hkv=1, d=6, W=0, theta=100.0, yarn=64.0, prior=2, norm=True, seed=8),
    ]
    for cs in cases:
        T, Hq, Hkv, d, W = cs["T"], cs["Hq"], cs["Hkv"], cs["d"], cs["W"]
        s = cs["seed"]
        q, k, v = _rand((T, Hq, d), s), _rand((T, Hkv, d), s + 1), _rand((T, Hkv, d), s + 2)
        n_prior = cs["prior"]
        pk, pv = _rand((n_prior, Hkv, d), s + 3), _rand((n_prior, Hkv, d), s + 4)
        wq = _rand((d,), s + 5) * 0.3 if cs["norm"] else None
        wk = _rand((d,), s + 6) * 0.3 if cs["norm"] else None
        c = 0.7
        cache = o.LayerKVCache.with_prior(pk, pv, n_prior, W)
        got = o.attention_layer_step(q, k, v, cache, theta=cs["theta"], yarn_factor=cs["yarn"],
                                     q_norm_w=wq, k_norm_w=wk, norm_offset=c, eps=1e-6)
        want = _brute_layer(q.tolist(), k.tolist(), v.tolist(), pk.tolist(), pv.tolist(), W,
                            cs["theta"], cs["yarn"], None if wq is None else wq.tolist(),
                            None if wk is None else wk.tolist(), c, 1e-6)
        assert np.max(np.abs(got - want)) < 1e-11, cs


def pin_rows_sum_to_one(o):
    T, Hq, Hkv, d = 40, 4, 2, 16
    q, k, v = _rand((T, Hq, d), 11), _rand((T, Hkv, d), 12), _rand((T, Hkv, d), 13)
    pos = np.arange(T)
    for W in (0, 1, 7, 40, 64):
        _, w = o.gqa_attention(q * 3, k * 3, v, pos, pos, W, 0.25, return_weights=True)
        assert np.max(np.abs(w.sum(-1) - 1.0)) < 1e-12
        assert np.all(w[:, ~o.allowed(pos, pos, W)] == 0.0)


def pin_swa_equals_global_short(o):
    T, Hq, Hkv, d = 24, 4, 2, 16
    q, k, v = _rand((T, Hq, d), 21), _rand((T, Hkv, d), 22), _rand((T, Hkv, d), 23)
    for W in (T, T + 1, 2048):
        outs = []
        for win in (W, 0):
            cache = o.LayerKVCache(Hkv, d, win)
            outs.append(o.attention_layer_step(q, k, v, cache, theta=1e4))
        assert np.max(np.abs(outs[0] - outs[1])) == 0.0
    cache_l = o.LayerKVCache(Hkv, d, T - 1)
    cache_g = o.LayerKVCache(Hkv, d, 0)
    a = o.attention_layer_step(q, k, v, cache_l, theta=1e4)
    b = o.attention_layer_step(q, k, v, cache_g, theta=1e4)
    assert np.max(np.abs(a - b)) > 1e-6  # the window must bite once T > W


def pin_uniform_closed_form(o):
    """Zero queries give uniform weights over the visible keys, so each output is the mean
    of V over the window: a closed form computed from prefix sums."""
    T, Hq, Hkv, d = 50, 4, 2, 8
    q = np.zeros((T, Hq, d))
    k, v = _rand((T, Hkv, d), 31), _rand((T, Hkv, d), 32)
    csum = np.concatenate([np.zeros((1, Hkv, d)), np.cumsum(v, axis=0)])
    for W in (0, 1, 6, 50):
        cache = o.LayerKVCache(Hkv, d, W)
        # gain c + w = 0 zeroes Q after the norm even though k is normalised normally
        got = o.attention_layer_step(_rand((T, Hq, d), 33), k, v, cache, theta=1e4,
                                     q_norm_w=-np.ones(d), k_norm_w=np.zeros(d), norm_offset=1.0)
        got0 = o.gqa_attention(q, k, v, np.arange(T), np.arange(T), W, 0.3)
        for t in range(T):
            lo = 0 if W == 0 else max(0, t - W + 1)
            mean = (csum[t + 1] - csum[lo]) / (t + 1 - lo)
            for h in range(Hq):
                g = h // (Hq // Hkv)
                assert np.max(np.abs(got[t, h] - mean[g])) < 1e-12
                assert np.max(np.abs(got0[t, h] - mean[g])) < 1e-12


def pin_gqa_grouping(o):
    """Consecutive query heads share a KV head (g(h) = floor(h / (Hq/Hkv))), not h mod Hkv:
    V made distinct per KV head, uniform weights."""
    T, Hq, Hkv, d = 6, 8, 2, 4
    v = np.zeros((T, Hkv, d))
    for g in range(Hkv):
        v[:, g, :] = 10.0 * g + 1.0
    out = o.gqa_attention(np.zeros((T, Hq, d)), _rand((T, Hkv, d), 41), v, np.arange(T),
                          np.arange(T), 0, 1.0)
    for h in range(Hq):
        assert np.allclose(out[:, h, :], 10.0 * (h // 4) + 1.0, atol=1e-12, rtol=0)


def pin_rope_library(o):
    """Library cross-check of the split-half rotation and the YaRN frequencies: Transformers'
    rotate-half RoPE (Llama) and its YaRN inverse-frequency routine with unrounded bounds."""
    from transformers import PretrainedConfig
    from transformers.modeling_rope_utils import _compute_yarn_parameters
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

    d = 128
    for theta, factor in ((1e6, 256.0), (1e6, 64.0), (1e4, 1.0), (1e6, 1.0)):
        cfg = PretrainedConfig()
        cfg.head_dim = d
        cfg.hidden_size = 5120
        cfg.num_attention_heads = 64
        cfg.max_position_embeddings = 262144
        cfg.rope_parameters = dict(rope_type="yarn", rope_theta=theta, factor=factor,
                                   original_max_position_embeddings=4096, beta_fast=32.0,
                                   beta_slow=1.0, truncate=False)
        inv, att = _compute_yarn_parameters(cfg, device="cpu")
        omega, amp = o.rope_frequencies(d, theta, factor)
        # the library works in float32 and forms 1 - ramp, which cancels near the top of the
        # ramp (j = 30 sits 0.02 below j_high): about 1e-5 relative there, 3e-7 elsewhere
        assert np.max(np.abs(omega / inv.double().numpy() - 1.0)) < 3e-5, (theta, factor)
        assert abs(amp - float(att)) < 1e-12
        # the rotation itself, with the library's rotate-half form in float64
        T, H = 7, 3
        x = _rand((T, H, d), 51)
        pos = np.array([0, 1, 5, 100, 2047, 32767, 131071])
        got = o.apply_rope(x, pos, omega, amp)
        ang = torch.from_numpy(pos.astype(np.float64))[:, None] * torch.from_numpy(omega)[None]
        emb = torch.cat([ang, ang], -1)
        cos, sin = emb.cos() * amp, emb.sin() * amp
        xt = torch.from_numpy(x).permute(1, 0, 2)[None]  # [1, H, T, d]
        ref, _ = apply_rotary_pos_emb(xt, xt, cos[None], sin[None])
        assert np.max(np.abs(got - ref[0].permute(1, 0, 2).numpy())) < 1e-12


def pin_rope_complex(o):
    """RoPE as complex multiplication: (x_j + i x_{j+d/2}) * amp * exp(i p omega_j)."""
    d = 16
    x = _rand((5, 2, d), 61)
    pos = np.array([0, 3, 10, 999, 65536])
    omega, amp = o.rope_frequencies(d, 1e6, 64.0)
    got = o.apply_rope(x, pos, omega, amp)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * (amp * np.exp(1j * pos[:, None, None] * omega))
    assert np.max(np.abs(got[..., : d // 2] - z.real)) < 1e-12
    assert np.max(np.abs(got[..., d // 2:] - z.imag)) < 1e-12
    # position 0: identity times the amplitude; pair norms scale by the amplitude
    assert np.max(np.abs(o.apply_rope(x, np.zeros(5), omega, amp) - amp * x)) < 1e-15
    n0 = np.hypot(x[..., : d // 2], x[..., d // 2:])
    n1 = np.hypot(got[..., : d // 2], got[..., d // 2:])
    assert np.max(np.abs(n1 - amp * n0)) < 1e-12


def pin_rope_shift_invariance(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §4.4: shifting Q and K positions by the same amount
    leaves the rotated dot product unchanged, with fixed frequencies and with YaRN."""
    d = 128
    q, k = _rand((6, 1, d), 71), _rand((6, 1, d), 72)
    qp = np.array([5, 9, 100, 2047, 3000, 7])
    kp = np.array([0, 9, 50, 1, 2999, 7])
    for theta, yarn in ((1e4, 0.0), (1e6, 256.0), (1e6, 64.0)):
        omega, amp = o.rope_frequencies(d, theta, yarn)
        base = np.sum(o.apply_rope(q, qp, omega, amp) * o.apply_rope(k, kp, omega, amp), -1)
        for delta in (1, 2047, 131072):
            sh = np.sum(o.apply_rope(q, qp + delta, omega, amp) * o.apply_rope(k, kp + delta, omega, amp), -1)
            assert np.max(np.abs(sh - base)) < 1e-9 * max(1.0, np.max(np.abs(base)))


def pin_local_window_slice(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §4.4, §5.1, §6.1: on a local layer, a one-shot prefill's
    row r attends keys r - W + 1 .. r only, and RoPE scores depend on positions through their
    difference, so the layer run on those W tokens alone (positions 0 .. W - 1) gives the same
    row (the full-size GPU checks rely on this to run the oracle on windows)."""
    T, Hq, Hkv, d, W = 300, 4, 2, 32, 64
    q, k, v = _rand((T, Hq, d), 301), _rand((T, Hkv, d), 302), _rand((T, Hkv, d), 303)
    wq, wk = _rand((d,), 304) * 0.1, _rand((d,), 305) * 0.1
    kw = dict(theta=1e4, yarn_factor=0.0, q_norm_w=wq, k_norm_w=wk, norm_offset=1.0)
    rows = np.array([0, 10, 63, 64, 200, 299])
    full = o.attention_layer_step(q, k, v, o.LayerKVCache(Hkv, d, W), rows=rows, **kw)
    for i, r in enumerate(rows):
        s0 = max(0, r - W + 1)
        sl = slice(s0, r + 1)
        one = o.attention_layer_step(q[sl], k[sl], v[sl], o.LayerKVCache(Hkv, d, W), rows=np.array([r - s0]), **kw)
        assert np.max(np.abs(one[0] - full[i])) < 1e-12, r


def pin_yarn_printed(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §6.3: the printed ramp bounds and amplitude figures."""
    g = golden("yarn_printed.json")
    p = g["params"]
    lo, hi = o.yarn_ramp_bounds(p["d"], p["theta"], p["orig_ctx"], p["beta_fast"], p["beta_slow"])
    _, amp = o.rope_frequencies(p["d"], p["theta"], p["factor"], p["orig_ctx"], p["beta_fast"], p["beta_slow"])

    def near(x, printed):
        val, dec = printed
        return abs(x - val) <= 0.5 * 10 ** (-dec) + 1e-12

    pr = g["printed"]
    assert near(lo, pr["j_low"]), lo
    assert near(hi, pr["j_high"]), hi
    assert near(amp, pr["amplitude"]), amp
    assert near(amp * amp, pr["amplitude_squared"]), amp * amp
    assert near(amp * amp / math.sqrt(128), pr["amplitude_squared_over_sqrt128"])


def pin_yarn_figure7(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §6.3 Fig. 7: ratio 1 below the ramp, 1/s above it,
    linear in j between, with unrounded bounds."""
    d, theta, s = 128, 1e6, 256.0
    omega_y, _ = o.rope_frequencies(d, theta, s)
    omega_0, amp0 = o.rope_frequencies(d, theta, 0.0)
    assert amp0 == 1.0
    ratio = omega_y / omega_0
    lo, hi = o.yarn_ramp_bounds(d, theta, 4096.0, 32.0, 1.0)
    j = np.arange(d // 2)
    assert np.allclose(ratio[j <= lo], 1.0, rtol=1e-14, atol=0)
    assert np.allclose(ratio[j >= hi], 1.0 / s, rtol=1e-14, atol=0)
    mid = (j > lo) & (j < hi)
    assert mid.sum() == 17  # j = 14 .. 30 (j_high is about 30.02)
    slope = np.diff(ratio[mid])
    assert np.allclose(slope, slope[0], rtol=1e-12, atol=1e-15) and slope[0] < 0
    # unrounded: at j = 14 the ramp has barely started
    assert 0.0 < 1.0 - ratio[14] < 0.01


def pin_rmsnorm(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §3.2: zero weight gives gain c; offset folded into a
    standard RMSNorm gain (library rms_norm); the output-RMS and input-scaling identities
    of §9's norm discussion."""
    x = _rand((7, 3, 128), 81)
    w = _rand((128,), 82) * 0.05
    eps = 1e-6
    for c in (1.0, 0.2, 5 ** -1.5):
        y0 = o.offset_rms_norm(x, np.zeros(128), c, eps)
        ref0 = c * x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)
        assert np.max(np.abs(y0 - ref0)) < 1e-14
        y = o.offset_rms_norm(x, w, c, eps)
        lib = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(c + w), eps)
        assert np.max(np.abs(y - lib.numpy())) < 1e-13
        gam = c + w
        lhs = np.mean(y * y, -1)
        rhs = np.mean(gam * gam * x * x, -1) / (np.mean(x * x, -1) + eps)
        assert np.max(np.abs(lhs - rhs)) < 1e-13
        for a in (1e-3, 7.0):
            ya = o.offset_rms_norm(a * x, w, c, eps)
            alt = gam * x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps / a ** 2)
            assert np.max(np.abs(ya - alt)) < 1e-12


def pin_cache_trim(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §4.4: after each update a local cache keeps at most
    W-1 tokens (the most recent ones); a global cache keeps all."""
    Hkv, d = 2, 4
    for W in (0, 1, 2, 4, 9):
        cache = o.LayerKVCache(Hkv, d, W)
        n, prev_keep = 0, 0
        for T in (1, 3, 1, 6, 2, 1, 12, 1):
            k = np.arange(n, n + T, dtype=float)[:, None, None] * np.ones((T, Hkv, d))
            k_all, _ = cache.update(k, k)
            n += T
            assert k_all.shape[0] == prev_keep + T  # attention reads the kept tokens plus the new ones
            assert np.array_equal(k_all[:, 0, 0], np.arange(n - prev_keep - T, n, dtype=float))
            keep = n if W == 0 else min(n, W - 1)
            prev_keep = keep
            assert cache.k.shape[0] == keep
            assert np.array_equal(cache.k[:, 0, 0], np.arange(n - keep, n, dtype=float))
            assert cache.seen == n


def pin_decode_equivalence(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §10 method: one-shot prefill equals token-by-token
    decode and equals a 3/6/3 chunked prefill (small model shape: d=16, W=4, T=12)."""
    T, Hq, Hkv, d = 12, 4, 2, 16
    q, k, v = _rand((T, Hq, d), 91), _rand((T, Hkv, d), 92), _rand((T, Hkv, d), 93)
    wq, wk = _rand((d,), 94) * 0.1, _rand((d,), 95) * 0.1
    for W, theta, yarn in ((4, 1e4, 0.0), (0, 1e6, 256.0), (1, 1e4, 0.0), (20, 1e4, 0.0)):
        kw = dict(theta=theta, yarn_factor=yarn, q_norm_w=wq, k_norm_w=wk, norm_offset=1.0)
        full = o.attention_layer_step(q, k, v, o.LayerKVCache(Hkv, d, W), **kw)
        for chunks in ([1] * T, [3, 6, 3], [5, 7]):
            cache = o.LayerKVCache(Hkv, d, W)
            outs, t0 = [], 0
            for n in chunks:
                outs.append(o.attention_layer_step(q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n], cache, **kw))
                t0 += n
            assert np.max(np.abs(np.concatenate(outs) - full)) < 1e-12, (W, chunks)
        # row subset equals the same rows of the full evaluation
        rows = np.array([0, 5, 11])
        sub = o.attention_layer_step(q, k, v, o.LayerKVCache(Hkv, d, W), rows=rows, **kw)
        assert np.max(np.abs(sub - full[rows])) < 1e-13


def pin_kv_accounting(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §2.3 and §5.2 tables: KV reads per token and capacity."""
    g = golden("kv_accounting.json")
    MiB, GiB = 2 ** 20, 2 ** 30
    for r in g["reads_per_token_MiB"]:
        L = r["layers"]
        A = o.attended_keys_total(4096, 2048, L // 8, 7 * L // 8)
        assert o.kv_bytes(1, r["Hkv"], r["d"], A) == r["MiB"] * MiB, r
    for r in g["capacity_31B"]:
        A = o.attended_keys_total(r["N"], 2048, 8, 56)
        assert o.kv_bytes(1, 8, 128, A) == r["hybrid_MiB"] * MiB
        assert o.kv_bytes(1, 8, 128, o.attended_keys_total(r["N"], 2048, 64, 0)) == r["all_global_GiB"] * GiB
    ap = g["append_31B_KiB"]
    assert o.kv_bytes(1, 8, 128, 56) == ap["local"] * 1024
    assert o.kv_bytes(1, 8, 128, 8) == ap["global"] * 1024


def pin_legacy_4k_band(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §5.1: the 4K release's implementation builds its band
    with triu(diagonal=-W) (W + 1 keys including self) and its cache keeps the last W; the
    current release uses triu(diagonal=-(W-1)). Masks against NumPy's tril/triu, attention
    against float64 SDPA with that mask, and the cache trimming."""
    n = 11
    pos = np.arange(n)
    ones = np.ones((n, n), dtype=bool)
    for W in (1, 2, 4, 7):
        assert np.array_equal(o.allowed(pos, pos, W, legacy_4k=True), np.tril(ones) & np.triu(ones, -W))
        assert np.array_equal(o.allowed(pos, pos, W), np.tril(ones) & np.triu(ones, -(W - 1)))
    T, Hq, Hkv, d, W = 13, 4, 2, 8, 3
    q, k, v = _rand((T, Hq, d), 71), _rand((T, Hkv, d), 72), _rand((T, Hkv, d), 73)
    scale = 1.0 / math.sqrt(d)
    got = o.gqa_attention(q, k, v, np.arange(T), np.arange(T), W, scale, legacy_4k=True)
    mask = torch.from_numpy(np.tril(np.ones((T, T), dtype=bool)) & np.triu(np.ones((T, T), dtype=bool), -W))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(k).permute(1, 0, 2)[None],
        torch.from_numpy(v).permute(1, 0, 2)[None], attn_mask=mask, scale=scale, enable_gqa=True)
    assert np.max(np.abs(got - ref[0].permute(1, 0, 2).numpy())) < 1e-12
    cache = o.LayerKVCache(1, 1, W, legacy_4k=True)
    seen = 0
    for t in (2, 1, 5, 1, 1):
        x = np.arange(seen, seen + t, dtype=float)[:, None, None]
        cache.update(x, x)
        seen += t
        keep = min(seen, W)
        assert np.array_equal(cache.k[:, 0, 0], np.arange(seen - keep, seen, dtype=float))
    # prefill equals token-by-token decode under the legacy band as well
    full = o.attention_layer_step(q, k, v, o.LayerKVCache(Hkv, d, W, legacy_4k=True), theta=1e4)
    c2 = o.LayerKVCache(Hkv, d, W, legacy_4k=True)
    steps = np.concatenate([o.attention_layer_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], c2, theta=1e4)
                            for t in range(T)])
    assert np.max(np.abs(steps - full)) < 1e-12


def pin_post_rope_cache(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §4.4 contrasts PLaMo's order (cache pre-RoPE K, rotate
    every returned K at renumbered positions) with rotating K before the store at absolute
    positions. Rotations compose (the score depends on i - j only, and the YaRN amplitude
    multiplies both sides), so both orders give the same outputs, for prefill, chunks and
    decode, on local and global layers, also past positions where absolute and renumbered
    positions differ. The post-RoPE cache then holds K rotated at the absolute position."""
    T, Hq, Hkv, d = 14, 4, 2, 16
    q, k, v = _rand((T, Hq, d), 61), _rand((T, Hkv, d), 62), _rand((T, Hkv, d), 63)
    wq, wk = _rand((d,), 64) * 0.1, _rand((d,), 65) * 0.1
    for W, theta, yarn in ((4, 1e4, 0.0), (0, 1e6, 64.0), (6, 1e4, 0.0)):
        kw = dict(theta=theta, yarn_factor=yarn, q_norm_w=wq, k_norm_w=wk, norm_offset=1.0)
        for chunks in ([T], [5, 1, 1, 7], [1] * T):
            pre, post = o.LayerKVCache(Hkv, d, W), o.LayerKVCache(Hkv, d, W, post_rope=True)
            t0 = 0
            for n in chunks:
                a = o.attention_layer_step(q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n], pre, **kw)
                b = o.attention_layer_step(q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n], post, **kw)
                assert np.max(np.abs(a - b)) < 1e-10, (W, chunks)
                t0 += n
            # what the post-RoPE cache holds: the kept tokens' normalised K, rotated at their
            # absolute positions (the rotation of each pair written out with cos / sin)
            omega, amp = o.rope_frequencies(d, theta, yarn)
            keep = post.k.shape[0]
            kn = o.offset_rms_norm(k[T - keep:], wk, 1.0)
            ang = np.arange(T - keep, T)[:, None, None] * omega[None, None, :]
            x0, x1 = kn[..., :d // 2], kn[..., d // 2:]
            want = np.concatenate([amp * (x0 * np.cos(ang) - x1 * np.sin(ang)),
                                   amp * (x0 * np.sin(ang) + x1 * np.cos(ang))], axis=-1)
            assert np.max(np.abs(post.k - want)) < 1e-12


def pin_mixer_bruteforce(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §3.2, §4.1, §4.5: the attention sublayer against scalar
    loops (pre norm with offset 1, the fused projection split into Q | K | V along its output
    axis, the attention step, heads concatenated, the output projection, post norm with
    offset 0.2, residual add), with an empty and a populated cache."""
    for (T, D, Hq, Hkv, d, W, prior, seed) in ((4, 6, 2, 1, 4, 3, 0, 31), (3, 5, 4, 2, 4, 0, 2, 32)):
        x = _rand((T, D), seed)
        w_pre, w_post = _rand((D,), seed + 1) * 0.2, _rand((D,), seed + 2) * 0.2
        w_qkv = _rand(((Hq + 2 * Hkv) * d, D), seed + 3) * 0.5
        w_o = _rand((D, Hq * d), seed + 4) * 0.5
        wq, wk = _rand((d,), seed + 5) * 0.3, _rand((d,), seed + 6) * 0.3
        pk, pv = _rand((prior, Hkv, d), seed + 7), _rand((prior, Hkv, d), seed + 8)
        cache = o.LayerKVCache.with_prior(pk, pv, prior, W)
        got = o.mixer_layer_step(x, cache, w_pre=w_pre, w_qkv=w_qkv, w_o=w_o, w_post=w_post, Hq=Hq, Hkv=Hkv,
                                 theta=1e4, q_norm_w=wq, k_norm_w=wk)

        def norm(vec, w, c):
            r = 1.0 / math.sqrt(sum(e * e for e in vec) / len(vec) + 1e-6)
            return [(c + w[i]) * vec[i] * r for i in range(len(vec))]

        xs = x.tolist()
        us = [norm(xs[t], w_pre.tolist(), 1.0) for t in range(T)]

        def proj(row, first):  # output feature first + i of the fused projection
            return [sum(w_qkv[first + i][j] * us[row][j] for j in range(D)) for i in range(d)]

        q = [[proj(t, h * d) for h in range(Hq)] for t in range(T)]
        k = [[proj(t, (Hq + g) * d) for g in range(Hkv)] for t in range(T)]
        v = [[proj(t, (Hq + Hkv + g) * d) for g in range(Hkv)] for t in range(T)]
        att = _brute_layer(q, k, v, pk.tolist(), pv.tolist(), W, 1e4, 0, wq.tolist(), wk.tolist(), 1.0, 1e-6)
        for t in range(T):
            flat = [att[t][h][r] for h in range(Hq) for r in range(d)]
            ov = [sum(w_o[i][j] * flat[j] for j in range(Hq * d)) for i in range(D)]
            want = [xs[t][i] + e for i, e in enumerate(norm(ov, w_post.tolist(), 0.2))]
            assert np.max(np.abs(got[t] - np.array(want))) < 1e-11, (T, D, t)


def pin_mixer_torch(o):
    """Library cross-check of the projections and norms: torch float64 rms_norm (gain c + w)
    and linear, the fused weight cut with torch.split at Hq d and Hkv d."""
    T, D, Hq, Hkv, d = 7, 24, 4, 2, 8
    x = _rand((T, D), 41)
    w_pre, w_post = _rand((D,), 42) * 0.1, _rand((D,), 43) * 0.1
    w_qkv, w_o = _rand(((Hq + 2 * Hkv) * d, D), 44) * 0.3, _rand((D, Hq * d), 45) * 0.3
    got = o.mixer_layer_step(x, o.LayerKVCache(Hkv, d, 4), w_pre=w_pre, w_qkv=w_qkv, w_o=w_o, w_post=w_post,
                             Hq=Hq, Hkv=Hkv, theta=1e4)
    F = torch.nn.functional
    xt = torch.from_numpy(x)
    u = F.rms_norm(xt, (D,), torch.from_numpy(1.0 + w_pre), eps=1e-6)
    qf, kf, vf = torch.split(F.linear(u, torch.from_numpy(w_qkv)), [Hq * d, Hkv * d, Hkv * d], dim=-1)
    att = o.attention_layer_step(qf.reshape(T, Hq, d).numpy(), kf.reshape(T, Hkv, d).numpy(),
                                 vf.reshape(T, Hkv, d).numpy(), o.LayerKVCache(Hkv, d, 4), theta=1e4)
    oo = F.linear(torch.from_numpy(att.reshape(T, Hq * d)), torch.from_numpy(w_o))
    want = xt + F.rms_norm(oo, (D,), torch.from_numpy(0.2 + w_post), eps=1e-6)
    assert np.max(np.abs(got - want.numpy())) < 1e-12


def pin_p_rope_page(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §6.4: p-RoPE of the Gemma-4-shaped global layer (d = 512,
    p = 0.25, base 1e6): the printed frequency formula over the whole head dim for the 64
    high-frequency pairs and frequency 0 for the other 192; pairs (j, j + 256); exactly the
    printed components turn; it is not a 128-dim RoPE on the first 128 components."""
    g = golden("p_rope_printed.json")
    d, theta, p = g["d"], g["theta"], g["p"]
    omega, amp = o.rope_frequencies(d, theta, partial=p)
    assert amp == 1.0 and omega.shape == (g["pairs"],)
    n_rot = g["rotated_pairs"]
    for j in range(g["pairs"]):
        want = math.exp(-2.0 * j / d * math.log(theta)) if j < n_rot else 0.0
        assert abs(omega[j] - want) <= 1e-15 * max(1.0, want), (j, omega[j], want)
    x = _rand((4, 3, d), 301)
    pos = np.array([1, 7, 1000, 131071])
    got = o.apply_rope(x, pos, omega, amp)
    changed = np.any(got != x, axis=(0, 1))
    want_set = np.zeros(d, dtype=bool)
    for lo, hi in g["rotated_components"]:
        want_set[lo:hi + 1] = True
    assert np.array_equal(changed, want_set), np.nonzero(changed != want_set)
    # each turning pair (j, j + 256) is a complex product with exp(i p w_j)
    h = d // 2
    z = (x[..., :n_rot] + 1j * x[..., h:h + n_rot]) * np.exp(1j * pos[:, None, None] * omega[None, None, :n_rot])
    assert np.max(np.abs(got[..., :n_rot] - z.real)) < 1e-12
    assert np.max(np.abs(got[..., h:h + n_rot] - z.imag)) < 1e-12
    # the reading the page warns against: a 128-dim RoPE on components 0..127
    w128 = np.exp(-2.0 * np.arange(64) / 128 * math.log(theta))
    alt = x.copy()
    a, b = x[..., :64], x[..., 64:128]
    ang = pos[:, None, None] * w128[None, None, :]
    alt[..., :64] = a * np.cos(ang) - b * np.sin(ang)
    alt[..., 64:128] = a * np.sin(ang) + b * np.cos(ang)
    assert np.max(np.abs(alt - got)) > 0.1
    # scores still depend on the position difference only
    q1, k1 = _rand((3, 1, d), 302), _rand((3, 1, d), 303)
    qp, kp = np.array([5, 900, 3]), np.array([0, 899, 3])
    base = np.sum(o.apply_rope(q1, qp, omega, amp) * o.apply_rope(k1, kp, omega, amp), -1)
    for delta in (1, 4095, 262143):
        sh = np.sum(o.apply_rope(q1, qp + delta, omega, amp) * o.apply_rope(k1, kp + delta, omega, amp), -1)
        assert np.max(np.abs(sh - base)) < 1e-9 * max(1.0, np.max(np.abs(base)))


def _gemma_kw(partial, wq, wk):
    return dict(theta=1e6 if partial < 1.0 else 1e4, partial=partial, q_norm_w=wq, k_norm_w=wk,
                norm_offset=0.0, scale=1.0, v_norm=True)


def pin_gemma_layer_bruteforce(o):
    """「PLaMo 3アーキテクチャ徹底解析」 §6.4 and the §8 comparison table: the Gemma-4-shaped layer
    (gain = stored weight, offset 0; V divided by its RMS; dot-product factor 1; K stored
    after RoPE at absolute positions; p-RoPE on the global layer) evaluated in chunks on a
    post-RoPE cache, against scalar loops over the whole sequence at renumbered positions."""
    cases = [dict(T=7, Hq=4, Hkv=2, d=8, W=3, partial=1.0, chunks=[3, 1, 3], seed=311),
             dict(T=6, Hq=4, Hkv=1, d=16, W=0, partial=0.25, chunks=[2, 1, 1, 2], seed=312),
             dict(T=5, Hq=2, Hkv=2, d=12, W=0, partial=0.5, chunks=[5], seed=313)]
    for cs in cases:
        T, Hq, Hkv, d, W = cs["T"], cs["Hq"], cs["Hkv"], cs["d"], cs["W"]
        s = cs["seed"]
        q, k, v = _rand((T, Hq, d), s), _rand((T, Hkv, d), s + 1), 3.0 * _rand((T, Hkv, d), s + 2)
        wq, wk = 1.0 + 0.05 * _rand((d,), s + 3), 0.3 + 0.05 * _rand((d,), s + 4)
        kw = _gemma_kw(cs["partial"], wq, wk)
        cache = o.LayerKVCache(Hkv, d, W, post_rope=True)
        outs, t0 = [], 0
        for n in cs["chunks"]:
            outs.append(o.attention_layer_step(q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n], cache, **kw))
            t0 += n
        got = np.concatenate(outs)
        n_rot = int(cs["partial"] * (d // 2))
        want = _brute_layer(q.tolist(), k.tolist(), v.tolist(), [], [], W, kw["theta"], 0, wq.tolist(),
                            wk.tolist(), 0.0, 1e-6, n_rot=n_rot, v_norm=True, scale=1.0)
        assert np.max(np.abs(got - want)) < 1e-11, cs
        # the post-RoPE cache holds V divided by its RMS
        keep = cache.v.shape[0]
        rms = np.sqrt(np.mean(cache.v ** 2, axis=-1))
        assert np.max(np.abs(rms - 1.0)) < 1e-5 and keep == (T if W == 0 else min(T, W - 1))


def pin_gemma_torch(o):
    """The Gemma-4-shaped layers at their real head shapes (「PLaMo 3アーキテクチャ徹底解析」 §8
    table: local d = 256, Hq = 32, Hkv = 16, W = 1024; global d = 512, Hkv = 4, p-RoPE
    §6.4), a short sequence in two chunks, against torch float64: F.rms_norm for the Q/K
    norms (weight = stored gain) and the gainless V norm, the rotation as a complex product
    over pairs (j, j + d/2) with the frequencies written out, and scaled_dot_product_attention
    with an explicit mask, scale 1 and enable_gqa. Also: scaling V leaves the output unchanged
    (the V norm removes it, up to eps)."""
    import torch.nn.functional as F
    T = 40
    for d, Hq, Hkv, W, partial, theta, seed in ((256, 32, 16, 24, 1.0, 1e4, 321),
                                                 (512, 32, 4, 0, 0.25, 1e6, 322)):
        q, k, v = _rand((T, Hq, d), seed), _rand((T, Hkv, d), seed + 1), _rand((T, Hkv, d), seed + 2)
        wq = np.full(d, 1.02)
        wk = np.full(d, 0.125 if W else 0.0625)
        kw = _gemma_kw(partial, wq, wk)
        kw["theta"] = theta
        cache = o.LayerKVCache(Hkv, d, W, post_rope=True)
        got = np.concatenate([o.attention_layer_step(q[:29], k[:29], v[:29], cache, **kw),
                              o.attention_layer_step(q[29:], k[29:], v[29:], cache, **kw)])
        qt = F.rms_norm(torch.from_numpy(q), (d,), torch.from_numpy(wq), eps=1e-6)
        kt = F.rms_norm(torch.from_numpy(k), (d,), torch.from_numpy(wk), eps=1e-6)
        vt = F.rms_norm(torch.from_numpy(v), (d,), None, eps=1e-6)
        h = d // 2
        n_rot = int(partial * h)
        jj = np.arange(h)
        om = np.where(jj < n_rot, np.exp(-2.0 * jj / d * math.log(theta)), 0.0)
        rot = torch.from_numpy(np.exp(1j * np.arange(T)[:, None] * om[None, :]))[:, None, :]

        def turn(x):
            z = torch.complex(x[..., :h], x[..., h:]) * rot
            return torch.cat([z.real, z.imag], -1)

        mask = torch.ones(T, T, dtype=torch.bool).tril()
        if W:
            mask &= ~torch.ones(T, T, dtype=torch.bool).tril(-W)
        ref = F.scaled_dot_product_attention(turn(qt).permute(1, 0, 2)[None], turn(kt).permute(1, 0, 2)[None],
                                             vt.permute(1, 0, 2)[None], attn_mask=mask, scale=1.0,
                                             enable_gqa=True)[0].permute(1, 0, 2).numpy()
        assert np.max(np.abs(got - ref)) < 1e-11, (d, np.max(np.abs(got - ref)))
        scaled = o.attention_layer_step(q, k, 7.5 * v, o.LayerKVCache(Hkv, d, W, post_rope=True), **kw)
        assert np.max(np.abs(scaled - got)) < 1e-5


PINS = [pin_worked_example, pin_fig4_masks, pin_sdpa_float64, pin_bruteforce_layer,
        pin_rows_sum_to_one, pin_swa_equals_global_short, pin_uniform_closed_form,
        pin_gqa_grouping, pin_rope_library, pin_rope_complex, pin_rope_shift_invariance, pin_local_window_slice,
        pin_yarn_printed, pin_yarn_figure7, pin_rmsnorm, pin_cache_trim,
        pin_decode_equivalence, pin_kv_accounting, pin_legacy_4k_band, pin_post_rope_cache,
        pin_mixer_bruteforce, pin_mixer_torch, pin_p_rope_page, pin_gemma_layer_bruteforce,
        pin_gemma_torch]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(O)


def test_package_exports_match_module():
    for name in oracle_pkg.__all__ if hasattr(oracle_pkg, "__all__") else []:
        assert getattr(oracle_pkg, name) is getattr(O, name)
    assert oracle_pkg.gqa_attention is O.gqa_attention


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

MISTAKES = {
    "rope_rotation_sign": ("out[..., :half] = amplitude * (a * cos - b * sin)",
                           "out[..., :half] = amplitude * (a * cos + b * sin)"),
    "rope_adjacent_pairs": ("a = x[..., :half]\n    b = x[..., half:]",
                            "a = x[..., 0::2]\n    b = x[..., 1::2]"),
    "rope_amplitude_cos_only": ("out[..., half:] = amplitude * (a * sin + b * cos)",
                                "out[..., half:] = a * sin + amplitude * b * cos"),
    "rope_base_exponent": ("omega = np.power(F64(theta), -2.0 * j / d)",
                           "omega = np.power(F64(theta), -1.0 * j / d)"),
    "yarn_ramp_reversed": ("omega = omega * ((1.0 - alpha) + alpha / yarn_factor)",
                           "omega = omega * (alpha + (1.0 - alpha) / yarn_factor)"),
    "yarn_bounds_rounded": ("alpha = np.clip((j - j_low) / (j_high - j_low), 0.0, 1.0)",
                            "alpha = np.clip((j - round(j_low)) / (round(j_high) - round(j_low)), 0.0, 1.0)"),
    "yarn_amplitude_sqrt": ("amplitude = 1.0 + 0.1 * math.log(yarn_factor)",
                            "amplitude = math.sqrt(1.0 + 0.1 * math.log(yarn_factor))"),
    "window_off_by_one": ("ok &= (i - j) < window", "ok &= (i - j) <= window"),
    "mask_excludes_self": ("ok = j <= i", "ok = j < i"),
    "gqa_modulo_heads": ("return h // (Hq // Hkv)", "return h % Hkv"),
    "norm_gain_product": ("gain = c + np.asarray(w, dtype=F64)", "gain = c * (1.0 + np.asarray(w, dtype=F64))"),
    "norm_eps_outside_sqrt": ("return gain * (x / np.sqrt(mean_sq + eps))", "return gain * (x / (np.sqrt(mean_sq) + eps))"),
    "cache_keeps_W": ("keep = n if self.window == 0 else min(n, self.window - 1)",
                      "keep = n if self.window == 0 else min(n, self.window)"),
    "legacy_band_minus_one": ("ok &= (i - j) <= window", "ok &= (i - j) < window + 0"),
    "legacy_cache_keeps_W_minus_one": ("keep = min(n, self.window)\n", "keep = min(n, self.window - 1)\n"),
    "post_rope_renumbered_keys": ("k_all, v_all = cache.update(apply_rope(k, np.arange(first, first + T), omega, amp), v)",
                                  "k_all, v_all = cache.update(apply_rope(k, np.arange(T), omega, amp), v)"),
    "post_rope_rotates_twice": ("k_rot = k_all if cache.post_rope else apply_rope(k_all, k_pos, omega, amp)",
                                "k_rot = apply_rope(k_all, k_pos, omega, amp)"),
    "mixer_k_v_swapped": ("k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(T, Hkv, d)",
                          "k = qkv[:, (Hq + Hkv) * d:].reshape(T, Hkv, d)"),
    "mixer_post_offset_one": ("return xr + offset_rms_norm(o, w_post, post_offset, eps)",
                              "return xr + offset_rms_norm(o, w_post, pre_offset, eps)"),
    "mixer_no_residual": ("return xr + offset_rms_norm(o, w_post, post_offset, eps)",
                          "return offset_rms_norm(o, w_post, post_offset, eps)"),
    "mixer_projection_untransposed": ("qkv = u @ w_qkv.T", "qkv = u @ w_qkv.reshape(w_qkv.shape[1], -1)"),
    "p_rope_exponent_over_rotated_dims": ("np.power(F64(theta), -2.0 * j / d), 0.0)",
                                          "np.power(F64(theta), -2.0 * j / (2 * n_rot)), 0.0)"),
    "p_rope_low_frequency_pairs": ("omega = np.where(j < n_rot,", "omega = np.where(j >= d // 2 - n_rot,"),
    "p_rope_count_over_head_dim": ("n_rot = int(math.floor(partial * (d // 2)))",
                                   "n_rot = int(math.floor(partial * d))"),
    "v_norm_with_k_gain": ("v = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)",
                           "v = offset_rms_norm(v, k_norm_w, norm_offset, eps)"),
    "v_norm_sum_not_mean": ("v = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)",
                            "v = v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True) + eps)"),
    "query_positions_from_zero": ("q_pos = np.arange(S - T, S)", "q_pos = np.arange(T)"),
    "default_scale_inverse_d": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "weighted_sum_uses_keys": ("out[r0:r1, h, :] = a @ v[:, g, :]", "out[r0:r1, h, :] = a @ k_rot[:, g, :]"),
    "scores_unscaled": ("scores = (q_rot[r0:r1, h, :] @ k_rot[:, g, :].T) * scale",
                        "scores = (q_rot[r0:r1, h, :] @ k_rot[:, g, :].T)"),
    "kv_bytes_missing_v": ("return 2 * elem_bytes * B * Hkv * d * attended",
                           "return elem_bytes * B * Hkv * d * attended"),
    "attended_window_plus_one": ("return n_global * N + n_local * min(N, window)",
                                 "return n_global * N + n_local * min(N, window + 1)"),
}


def _mutated_oracle(name, old, new):
    src = open(ORACLE_SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mistake {name}: pattern must occur exactly once"
    src = src.replace(old, new)
    spec = importlib.util.spec_from_loader(f"oracle_mut_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, f"<oracle with {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistakes_are_caught(name):
    old, new = MISTAKES[name]
    mod = _mutated_oracle(name, old, new)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
