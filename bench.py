"""Benchmark of the PLaMo 3 hybrid attention hot path on one MI355X.

One JSON line on stdout. The headline step is one local-layer prefill at the PLaMo 3
shape (B=1, T=8192, Hq=64, Hkv=8, d=128, W=2048): plamo_kv_append (QK norm, cache
write, RoPE, prefill operands) + plamo_attn_prefill, inputs resident in HBM; the same step
with the queries normalised and rotated inside the attention kernel
(plamo_attn_prefill_fused_q) is reported in ``extra``. ``value``
is algorithmic prefill FLOP (4*d per attended (query, key) pair and query head) per
second of that step. Also reported: the global-layer prefill (T=32768, YaRN), batched
decode (B=64; ring W=2048 and global 32768) as KV-read GB/s, the same global decode with
each sequence at its own position (ragged), both prefills fed in chunks (2048 local, 8192
global) after cached tokens, the whole attention sublayer (projections and norms around the
path, D = 5120), the Gemma-4-shaped layers (d = 256 local, d = 512 global with p-RoPE: prefill
and B = 64 decode), the 8-layer period decode
at 131072 context, the roofline object of the prefill kernel, and the CPU oracle timed
on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (SWA W=2048 + global) & decode KV-read GB/s, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# timing helpers: torch events on the stream the library launches on
# ----------------------------------------------------------------------------

class Timer:
    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def span(self):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        self.pairs.append((a, b))
        return a, b

    def median_ms(self):
        """Median of the recorded spans (robust to a stray slow launch)."""
        self.torch.cuda.synchronize()
        v = sorted(a.elapsed_time(b) for a, b in self.pairs)
        n = len(v)
        return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


SETTLE_S = 0.25  # seconds of untimed load before each workload's warmup steps


def settle(torch, fn, seconds=SETTLE_S):
    """Run fn (one step of the workload about to be timed) until `seconds` of wall time have
    passed, untimed. The GPU's clocks are still rising during the first tens of milliseconds of
    load: measured on MI355X, the local prefill kernel timed 0.52 ms after 5 warmup steps and
    0.46 ms after 100 or 400. The warmup steps follow this phase."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        n += 4
    return n


def dev_bf16(torch, x):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def rope_params(swg, r):
    return swg.RopeParams(r.theta, r.yarn_factor, r.orig_ctx, r.beta_fast, r.beta_slow)


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

def bench_prefill(torch, swg, wl, steps, warmup, norm_offset, fuse_q=False):
    """One prefill step: plamo_kv_append + the attention. fuse_q: the append writes only the K/V
    side and plamo_attn_prefill_fused_q normalises and rotates Q inside the attention kernel
    (Q' never goes through HBM); otherwise the append writes Q' and plamo_attn_prefill reads it."""
    from sliding_window_global_amd import layer
    inp = wl.draw()
    q, k, v = dev_bf16(torch, inp["q"]), dev_bf16(torch, inp["k"]), dev_bf16(torch, inp["v"])
    wq, wk = dev_bf16(torch, inp["wq"]), dev_bf16(torch, inp["wk"])
    tab = swg.make_rope_table(wl.T + 64, rope_params(swg, wl.rope))
    cap = wl.window if wl.window else wl.T
    kc = torch.empty((wl.B, wl.Hkv, cap, wl.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    bufs = layer.PrefillBuffers(wl.B, wl.T, wl.Hq, wl.Hkv, wl.d, torch.bfloat16)

    def append():
        swg.plamo_kv_append(q if not fuse_q else None, k, v, bufs.q_rot if not fuse_q else None,
                            window=wl.window, pos_offset=0, rope_table=tab, q_norm_w=wq, k_norm_w=wk,
                            norm_offset=norm_offset, k_rot_out=bufs.k_rot, v_t_out=bufs.v_t, k_cache=kc,
                            v_cache=vc)

    def attention():
        if fuse_q:
            swg.plamo_attn_prefill_fused_q(q, bufs.k_rot, bufs.v_t, bufs.out, window=wl.window, rope_table=tab,
                                           q_norm_w=wq, norm_offset=norm_offset)
        else:
            swg.plamo_attn_prefill(bufs.q_rot, bufs.k_rot, bufs.v_t, bufs.out, window=wl.window)

    def step(t_step=None, t_attn=None):
        if t_step:
            t_step[0].record()
        append()
        if t_attn:
            t_attn[0].record()
        attention()
        if t_attn:
            t_attn[1].record()
        if t_step:
            t_step[1].record()

    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ts, ta = Timer(torch), Timer(torch)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(steps):
        step(ts.span(), ta.span())
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_attn = ta.median_ms()
    # whole-step figure: the K steps back to back (first step's start to last step's end) / K
    ms_step = ts.pairs[0][0].elapsed_time(ts.pairs[-1][1]) / steps
    flops = wl.flops()
    out = dict(workload=wl.name, flops=flops, ms_per_step=ms_step, ms_attn=ms_attn,
               ms_step_median=ts.median_ms(), step_tflops=flops / ms_step / 1e9, attn_tflops=flops / ms_attn / 1e9,
               wall_ms_per_step=wall / steps * 1e3)
    out.update(cold_cache(torch, append, attention, steps))
    return out


def cold_summary(r):
    """The cold-cache figures of a bench_prefill result, with their TFLOP/s."""
    return {"cold_ms_append": r["cold_ms_append"], "cold_ms_attn": r["cold_ms_attn"],
            "cold_ms_step": r["cold_ms_step"], "cold_attn_tflops": r["flops"] / r["cold_ms_attn"] / 1e9,
            "cold_step_tflops": r["flops"] / r["cold_ms_step"] / 1e9}


def cold_cache(torch, append, attention, steps):
    """The step with the caches cold: a 512 MiB buffer (twice the 256 MB last-level cache) is
    rewritten before the append and again before the attention, so that each kernel reads its
    inputs from HBM; medians over `steps` repetitions of each kernel's own HIP-event time."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    t_app, t_att = Timer(torch), Timer(torch)
    for _ in range(steps):
        for fn, timer in ((append, t_app), (attention, t_att)):
            flush.zero_()
            a, b = timer.span()
            a.record()
            fn()
            b.record()
    ms_app, ms_att = t_app.median_ms(), t_att.median_ms()
    del flush
    return dict(cold_ms_append=ms_app, cold_ms_attn=ms_att, cold_ms_step=ms_app + ms_att)


def bench_chunked_prefill(torch, swg, wl, chunk, steps, warmup):
    """The same prefill fed in chunks of ``chunk`` tokens: chunk c runs kv_append at
    pos_offset c*chunk (its operands start with the cached keys it attends) and
    attn_prefill. One step = every chunk; the FLOP count equals the one-shot prefill's."""
    from sliding_window_global_amd import layer
    inp = wl.draw()
    q, k, v = dev_bf16(torch, inp["q"]), dev_bf16(torch, inp["k"]), dev_bf16(torch, inp["v"])
    wq, wk = dev_bf16(torch, inp["wq"]), dev_bf16(torch, inp["wk"])
    tab = swg.make_rope_table(wl.T + 64, rope_params(swg, wl.rope))
    cap = wl.window if wl.window else wl.T
    kc = torch.empty((wl.B, wl.Hkv, cap, wl.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    starts = list(range(0, wl.T, chunk))
    parts, bufs = [], []
    for p in starts:
        n = min(chunk, wl.T - p)
        parts.append((q[:, p:p + n].contiguous(), k[:, p:p + n].contiguous(), v[:, p:p + n].contiguous()))
        bufs.append(layer.PrefillBuffers(wl.B, n, wl.Hq, wl.Hkv, wl.d, torch.bfloat16, window=wl.window,
                                         pos_offset=p))

    def step(t_step=None):
        if t_step:
            t_step[0].record()
        for p, (qc, kc_, vc_), bf in zip(starts, parts, bufs):
            swg.plamo_kv_append(qc, kc_, vc_, bf.q_rot, window=wl.window, pos_offset=p, rope_table=tab,
                                q_norm_w=wq, k_norm_w=wk, norm_offset=wl.norm_offset, k_rot_out=bf.k_rot,
                                v_t_out=bf.v_t, k_cache=kc, v_cache=vc)
            swg.plamo_attn_prefill(bf.q_rot, bf.k_rot, bf.v_t, bf.out, window=wl.window, pos_offset=p)
        if t_step:
            t_step[1].record()

    settle(torch, step)
    for _ in range(warmup):
        step()
    ts = Timer(torch)
    for _ in range(steps):
        step(ts.span())
    ms = ts.median_ms()
    flops = wl.flops()
    return dict(workload=f"{wl.name}_chunks{chunk}", n_chunks=len(starts), ms_per_step=ms,
                step_tflops=flops / ms / 1e9)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def bench_decode_batched(torch, swg, wl, layer_idx, steps, warmup, post_rope=False):
    """attn_decode alone (the split kernel + combine) over a cache at its real size (post_rope:
    a cache that holds K already rotated, read as stored)."""
    from sliding_window_global_amd import layer
    from synthetic.workloads import device_normal_bf16
    ly = wl.layers[layer_idx]
    p = wl.pos_offset
    cap = wl.cache_cap(ly)
    kc = device_normal_bf16((wl.B, wl.Hkv, cap, wl.d), wl.cache_seed(layer_idx), "cuda")
    vc = device_normal_bf16((wl.B, wl.Hkv, cap, wl.d), wl.cache_seed(layer_idx) + 1, "cuda")
    new = wl.draw_new_tokens(0, layer_idx)
    tab = swg.make_rope_table(p + wl.steps + 64, rope_params(swg, ly.rope))
    bufs = layer.DecodeBuffers(wl.B, wl.Hq, wl.Hkv, wl.d, ly.window, p)
    swg.plamo_kv_append(dev_bf16(torch, new["q"]), dev_bf16(torch, new["k"]), dev_bf16(torch, new["v"]),
                        bufs.q_rot, window=ly.window, pos_offset=p, rope_table=tab,
                        q_norm_w=dev_bf16(torch, new["wq"]), k_norm_w=dev_bf16(torch, new["wk"]),
                        norm_offset=wl.norm_offset, k_cache=kc, v_cache=vc, cache_post_rope=post_rope)

    def run():
        swg.plamo_attn_decode(bufs.q_rot, kc, vc, bufs.out, bufs.workspace, window=ly.window,
                              pos_offset=p, rope_table=tab, cache_post_rope=post_rope)

    settle(torch, run)
    for _ in range(warmup):
        run()
    t = Timer(torch)
    for _ in range(steps):
        a, b = t.span()
        a.record()
        run()
        b.record()
    ms = t.median_ms()
    nbytes = wl.kv_bytes(ly)
    del kc, vc
    torch.cuda.empty_cache()
    return dict(workload=f"{wl.name}_{'global' if ly.window == 0 else 'local'}{'_post_rope' if post_rope else ''}",
                kv_bytes=nbytes,
                keys=wl.keys_attended(ly), ms=ms, gbs=nbytes / ms / 1e6, frac_hbm=nbytes / ms / 1e6 / PEAK_HBM_GBS)


def bench_decode_ragged(torch, swg, wl, layer_idx, steps, warmup):
    """attn_decode of a ragged batch: the batched-decode shape with every sequence at its own
    position (uniform in [0, max], seeded), the cache at the largest one's size."""
    from sliding_window_global_amd import layer
    from synthetic.workloads import RAGGED_DECODE_SEED, device_normal_bf16, ragged_positions
    ly = wl.layers[layer_idx]
    pos = ragged_positions(wl.B, wl.pos_offset, RAGGED_DECODE_SEED)
    maxp = int(pos.max())
    cap = wl.cache_cap(ly)
    kc = device_normal_bf16((wl.B, wl.Hkv, cap, wl.d), wl.cache_seed(layer_idx), "cuda")
    vc = device_normal_bf16((wl.B, wl.Hkv, cap, wl.d), wl.cache_seed(layer_idx) + 1, "cuda")
    new = wl.draw_new_tokens(0, layer_idx)
    tab = swg.make_rope_table(maxp + 64, rope_params(swg, ly.rope))
    sp = torch.from_numpy(pos).cuda()
    bufs = layer.DecodeBuffers(wl.B, wl.Hq, wl.Hkv, wl.d, ly.window, maxp, ragged=True)
    swg.plamo_kv_append_ragged(dev_bf16(torch, new["q"]), dev_bf16(torch, new["k"]), dev_bf16(torch, new["v"]),
                               bufs.q_rot, window=ly.window, seq_pos_offsets=sp, max_pos_offset=maxp,
                               rope_table=tab, q_norm_w=dev_bf16(torch, new["wq"]),
                               k_norm_w=dev_bf16(torch, new["wk"]), norm_offset=wl.norm_offset,
                               k_cache=kc, v_cache=vc)

    def run():
        swg.plamo_attn_decode_ragged(bufs.q_rot, kc, vc, bufs.out, bufs.workspace, window=ly.window,
                                     seq_pos_offsets=sp, max_pos_offset=maxp, rope_table=tab)

    settle(torch, run)
    for _ in range(warmup):
        run()
    t = Timer(torch)
    for _ in range(steps):
        a, b = t.span()
        a.record()
        run()
        b.record()
    ms = t.median_ms()
    keys = [int(p) + 1 if ly.window == 0 else min(int(p), ly.window - 1) + 1 for p in pos]
    nbytes = 2 * 2 * wl.Hkv * wl.d * sum(keys)
    del kc, vc
    torch.cuda.empty_cache()
    return dict(workload=f"ragged_decode_B{wl.B}_{'global' if ly.window == 0 else 'local'}_max{maxp + 1}",
                kv_bytes=nbytes, mean_keys=sum(keys) / len(keys), ms=ms, gbs=nbytes / ms / 1e6,
                frac_hbm=nbytes / ms / 1e6 / PEAK_HBM_GBS)


# ----------------------------------------------------------------------------
# the Gemma-4-shaped second workload (head dims 256 / 512, p-RoPE, V norm, factor 1)
# ----------------------------------------------------------------------------

def gemma_table(swg, L, max_pos):
    return swg.make_rope_table(max_pos, swg.RopeParams(L.theta, partial=L.partial), d=L.d)


def gemma_kw(torch, L, wq, wk):
    return dict(q_norm_w=dev_bf16(torch, wq), k_norm_w=dev_bf16(torch, wk), norm_offset=L.norm_offset,
                norm_eps=L.eps, cache_post_rope=True, v_norm=True)


def bench_gemma_prefill(torch, swg, wl, steps, warmup):
    """kv_append (gain-only QK norm, V norm, p-RoPE or RoPE, post-RoPE cache, operands) +
    attn_prefill (factor 1) of one Gemma-shaped layer from an empty cache."""
    from sliding_window_global_amd import layer
    L = wl.layer
    inp = wl.draw()
    q, k = dev_bf16(torch, inp["q"]), dev_bf16(torch, inp["k"])
    v = k if L.kv_shared else dev_bf16(torch, inp["v"])
    tab = gemma_table(swg, L, wl.T + 64)
    cap = L.window if L.window else wl.T
    kc = torch.empty((wl.B, L.Hkv, cap, L.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    bufs = layer.PrefillBuffers(wl.B, wl.T, L.Hq, L.Hkv, L.d, torch.bfloat16)
    kw = gemma_kw(torch, L, inp["wq"], inp["wk"])

    def step(t_step=None, t_attn=None):
        t_step[0].record() if t_step else None
        swg.plamo_kv_append(q, k, v, bufs.q_rot, window=L.window, pos_offset=0, rope_table=tab,
                            k_rot_out=bufs.k_rot, v_t_out=bufs.v_t, k_cache=kc, v_cache=vc, **kw)
        t_attn[0].record() if t_attn else None
        swg.plamo_attn_prefill(bufs.q_rot, bufs.k_rot, bufs.v_t, bufs.out, window=L.window,
                               softmax_scale=L.scale)
        t_attn[1].record() if t_attn else None
        t_step[1].record() if t_step else None

    settle(torch, step)
    for _ in range(warmup):
        step()
    ts, ta = Timer(torch), Timer(torch)
    for _ in range(steps):
        step(ts.span(), ta.span())
    ms_step, ms_attn = ts.median_ms(), ta.median_ms()
    flops = wl.flops()
    return dict(workload=wl.name, flops=flops, ms_per_step=ms_step, ms_attn=ms_attn,
                step_tflops=flops / ms_step / 1e9, attn_tflops=flops / ms_attn / 1e9,
                frac_mfma=flops / ms_attn / 1e9 / PEAK_BF16_TFLOPS)


def bench_gemma_decode(torch, swg, wl, steps, warmup):
    """attn_decode of one Gemma-shaped layer (B = 64, post-RoPE cache read as stored) at its real
    cache size; KV-read GB/s over the attended keys."""
    from sliding_window_global_amd import layer
    from synthetic.workloads import device_normal_bf16
    L = wl.layer
    p = wl.pos_offset
    cap = wl.cache_cap()
    kc = device_normal_bf16((wl.B, L.Hkv, cap, L.d), wl.cache_seed(), "cuda")
    vc = device_normal_bf16((wl.B, L.Hkv, cap, L.d), wl.cache_seed() + 1, "cuda")
    new = wl.draw_new_tokens()
    tab = gemma_table(swg, L, p + 64)
    bufs = layer.DecodeBuffers(wl.B, L.Hq, L.Hkv, L.d, L.window, p)
    k1 = dev_bf16(torch, new["k"])
    v1 = k1 if L.kv_shared else dev_bf16(torch, new["v"])
    swg.plamo_kv_append(dev_bf16(torch, new["q"]), k1, v1, bufs.q_rot, window=L.window, pos_offset=p,
                        rope_table=tab, k_cache=kc, v_cache=vc, **gemma_kw(torch, L, new["wq"], new["wk"]))

    def run():
        swg.plamo_attn_decode(bufs.q_rot, kc, vc, bufs.out, bufs.workspace, window=L.window, pos_offset=p,
                              rope_table=None, softmax_scale=L.scale, cache_post_rope=True)

    settle(torch, run)
    for _ in range(warmup):
        run()
    t = Timer(torch)
    for _ in range(steps):
        a, b = t.span()
        a.record()
        run()
        b.record()
    ms = t.median_ms()
    nbytes = wl.kv_bytes()
    del kc, vc
    torch.cuda.empty_cache()
    return dict(workload=wl.name, kv_bytes=nbytes, keys=wl.keys_attended(), ms=ms, gbs=nbytes / ms / 1e6,
                frac_hbm=nbytes / ms / 1e6 / PEAK_HBM_GBS)


def bench_mixer(torch, swg, wl, steps, warmup):
    """The attention sublayer around the hot path (pre norm, QKV projection, append +
    attention, output projection, post norm + residual) on a local-layer prefill at
    D = 5120, random weights; times the whole sublayer and its three stages."""
    from sliding_window_global_amd import layer
    x, wdev = wl.draw_device("cuda")
    wts = layer.MixerWeights(Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, **wdev)
    kc = torch.empty((wl.B, wl.Hkv, wl.window, wl.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    tab = swg.make_rope_table(wl.T + 64, rope_params(swg, wl.rope))
    mb = layer.MixerBuffers(wl.B, wl.T, wl.D, wts)
    ab = layer.PrefillBuffers(wl.B, wl.T, wl.Hq, wl.Hkv, wl.d, torch.bfloat16, window=wl.window)

    def step(ev=None):
        if ev:
            ev[0].record()
        layer._mixer_in(x, wts, mb, None)
        if ev:
            ev[1].record()
        layer.prefill(mb.q, mb.k, mb.v, window=wl.window, rope_table=tab, q_norm_w=wts.wq, k_norm_w=wts.wk,
                      norm_offset=wts.qk_offset, k_cache=kc, v_cache=vc, bufs=ab)
        if ev:
            ev[2].record()
        layer._mixer_out(x, ab.out, wts, mb, None)
        if ev:
            ev[3].record()

    settle(torch, step)
    for _ in range(warmup):
        step()
    evs = []
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    part = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i in range(3)]
    total = sum(part)
    M = wl.B * wl.T
    qkv_flops = 2.0 * M * wl.D * (wl.Hq + 2 * wl.Hkv) * wl.d
    o_flops = 2.0 * M * wl.Hq * wl.d * wl.D
    flops = wl.gemm_flops() + wl.attention_flops()
    return dict(workload=wl.name, ms_per_step=total, ms_norm_qkv=part[0], ms_attention=part[1],
                ms_oproj_norm=part[2], step_tflops=flops / total / 1e9,
                qkv_proj_tflops=qkv_flops / part[0] / 1e9, o_proj_tflops=o_flops / part[2] / 1e9)


def bench_period(torch, swg, wl, n_steps, fused=False):
    """The 8-layer period (7 local W=2048 + 1 global), append + decode per layer per step,
    at 131072+k global context, batch 8. fused: each layer's step is one launch
    (plamo_decode_step) instead of the append, the decode and the merge of its key ranges."""
    from sliding_window_global_amd import layer
    from synthetic.workloads import device_normal_bf16
    caches, tabs, bufs, news = [], [], [], []
    for li, ly in enumerate(wl.layers):
        cap = wl.cache_cap(ly)
        caches.append((device_normal_bf16((wl.B, wl.Hkv, cap, wl.d), wl.cache_seed(li), "cuda"),
                       device_normal_bf16((wl.B, wl.Hkv, cap, wl.d), wl.cache_seed(li) + 1, "cuda")))
        tabs.append(swg.make_rope_table(wl.pos_offset + wl.steps + 64, rope_params(swg, ly.rope)))
        bufs.append(layer.DecodeBuffers(wl.B, wl.Hq, wl.Hkv, wl.d, ly.window, wl.pos_offset + wl.steps, fused=fused))
    for s in range(min(n_steps, 4)):  # a few distinct token sets, reused cyclically
        news.append([{k: (dev_bf16(torch, x) if x is not None else None) for k, x in wl.draw_new_tokens(s, li).items()}
                     for li in range(len(wl.layers))])
    def step0():  # step 0 again writes the same token into the same cache slot: no state change
        for li, ly in enumerate(wl.layers):
            nt = news[0][li]
            kc, vc = caches[li]
            layer.decode(nt["q"], nt["k"], nt["v"], kc, vc, window=ly.window, pos_offset=wl.pos_offset,
                         rope_table=tabs[li], q_norm_w=nt["wq"], k_norm_w=nt["wk"],
                         norm_offset=wl.norm_offset, bufs=bufs[li], fused=fused)

    settle(torch, step0)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    total_bytes = 0
    t0.record()
    for s in range(n_steps):
        p = wl.pos_offset + s
        for li, ly in enumerate(wl.layers):
            nt = news[s % len(news)][li]
            kc, vc = caches[li]
            layer.decode(nt["q"], nt["k"], nt["v"], kc, vc, window=ly.window, pos_offset=p,
                         rope_table=tabs[li], q_norm_w=nt["wq"], k_norm_w=nt["wk"],
                         norm_offset=wl.norm_offset, bufs=bufs[li], fused=fused)
            total_bytes += wl.kv_bytes(ly, s)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    del caches
    torch.cuda.empty_cache()
    return dict(workload=wl.name + ("_one_launch" if fused else ""), steps=n_steps, ms_total=ms, ms_per_step=ms / n_steps,
                kv_bytes_total=total_bytes, gbs=total_bytes / ms / 1e6,
                frac_hbm=total_bytes / ms / 1e6 / PEAK_HBM_GBS)


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the headline workload)
# ----------------------------------------------------------------------------

def cpu_baseline(wl, norm_offset, n_rows):
    import numpy as np

    from oracle import LayerKVCache, attention_layer_step
    cores = _cpu_cores()
    inp = wl.draw()
    rows = np.linspace(0, wl.T - 1, n_rows).astype(np.int64)
    t0 = time.perf_counter()
    cache = LayerKVCache(wl.Hkv, wl.d, wl.window)
    attention_layer_step(inp["q"][0], inp["k"][0], inp["v"][0], cache, theta=wl.rope.theta,
                         yarn_factor=wl.rope.yarn_factor, q_norm_w=inp["wq"], k_norm_w=inp["wk"],
                         norm_offset=norm_offset, scale=1.0 / math.sqrt(wl.d), rows=rows)
    sec = time.perf_counter() - t0
    pairs = int(np.sum(np.minimum(rows + 1, wl.window if wl.window else wl.T)))
    flops = 4.0 * wl.d * wl.Hq * pairs
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{wl.name}: {n_rows} of {wl.T} query rows x {wl.Hq} heads (full norm, cache, "
                      f"RoPE of all {wl.T} keys; fp64 NumPy), {sec:.1f} s"}


def _cpu_cores():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def cpu_baseline_global_rows(wl, block=256):
    """The oracle on the global prefill workload at a fixed row subset: the first, the last and
    two middle blocks of `block` query rows, all heads (norm of every row, RoPE of every key,
    attention of the subset). Reported as TFLOP/s of the subset's attended pairs; the full
    run's time is extrapolated at that rate."""
    import numpy as np

    from oracle import LayerKVCache, attention_layer_step
    inp = wl.draw()
    T = wl.T
    starts = [0, T // 2 - block, T // 2, T - block]
    rows = np.concatenate([np.arange(s0, s0 + block) for s0 in starts])
    t0 = time.perf_counter()
    attention_layer_step(inp["q"][0], inp["k"][0], inp["v"][0], LayerKVCache(wl.Hkv, wl.d, 0),
                         theta=wl.rope.theta, yarn_factor=wl.rope.yarn_factor, q_norm_w=inp["wq"],
                         k_norm_w=inp["wk"], norm_offset=wl.norm_offset, scale=wl.scale, rows=rows)
    sec = time.perf_counter() - t0
    flops = 4.0 * wl.d * wl.Hq * float(np.sum(rows + 1))
    rate = flops / sec
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": _cpu_cores(), "kind": "oracle",
            "sample": f"{wl.name}: rows {starts} + 0..{block - 1} ({len(rows)} of {T}) x {wl.Hq} heads, "
                      f"fp64 NumPy, {sec:.1f} s",
            "full_run_s_extrapolated": wl.flops() / rate}


def _prior_kv(n_keys, Hkv, d, gen_seed):
    """Kept K/V of one sequence of a decode workload, drawn on the host with the device caches'
    recipe (N(0, 1) rounded to bf16), as float32 [n_keys, Hkv, d]."""
    import torch

    from synthetic.workloads import device_normal_bf16
    pk = device_normal_bf16((n_keys, Hkv, d), gen_seed, "cpu").to(torch.float32).numpy()
    pv = device_normal_bf16((n_keys, Hkv, d), gen_seed + 1, "cpu").to(torch.float32).numpy()
    return pk, pv


def _oracle_decode_one(wl, layer_idx, step, b, pk, pv):
    """Seconds of the oracle's decode step of sequence b (cache holding its kept tokens, norm
    and RoPE of the new token, RoPE of every cached key, attention) at `step`; pk / pv hold at
    least the kept tokens (the newest last)."""
    from oracle import LayerKVCache, attention_layer_step
    ly = wl.layers[layer_idx]
    p = wl.pos_offset + step
    kept = wl.keys_attended(ly, step) - 1
    new = wl.draw_new_tokens(step, layer_idx)
    t0 = time.perf_counter()
    cache = LayerKVCache.with_prior(pk[pk.shape[0] - kept:], pv[pv.shape[0] - kept:], p, ly.window)
    attention_layer_step(new["q"][b], new["k"][b], new["v"][b], cache, theta=ly.rope.theta,
                         yarn_factor=ly.rope.yarn_factor, q_norm_w=new["wq"], k_norm_w=new["wk"],
                         norm_offset=wl.norm_offset, scale=wl.scale)
    return time.perf_counter() - t0


def cpu_baselines_extra():
    """The oracle on the other workloads: a fixed row subset of the global prefill, the whole
    batched decode (both layers) and the 8-layer period decode at steps 0, 63 and 127."""
    from synthetic.workloads import BATCHED_DECODE, GLOBAL_PREFILL, PERIOD_DECODE
    out = {}
    log("[bench] cpu oracle: global prefill row subset")
    out["cpu_baseline_prefill_global"] = cpu_baseline_global_rows(GLOBAL_PREFILL)
    log(f"[bench]   {out['cpu_baseline_prefill_global']}")
    cores = _cpu_cores()
    wl = BATCHED_DECODE
    for li, ly in enumerate(wl.layers):
        log(f"[bench] cpu oracle: batched decode layer {li}, all {wl.B} sequences")
        kept = wl.keys_attended(ly) - 1
        sec = 0.0
        for b in range(wl.B):
            pk, pv = _prior_kv(kept, wl.Hkv, wl.d, 7001 + 31 * b + li)
            sec += _oracle_decode_one(wl, li, 0, b, pk, pv)
        name = f"cpu_baseline_{wl.name}_{'global' if ly.window == 0 else 'local'}"
        out[name] = {"value": wl.kv_bytes(ly) / sec / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                     "sample": f"all {wl.B} sequences, {wl.keys_attended(ly)} keys each, fp64 NumPy, {sec:.1f} s"}
        log(f"[bench]   {out[name]}")
    wl = PERIOD_DECODE
    steps = (0, 63, 127)
    sec_step = {s_: 0.0 for s_ in steps}
    log(f"[bench] cpu oracle: period decode steps {steps}, {wl.B} sequences x 8 layers")
    for b in range(wl.B):
        for li, ly in enumerate(wl.layers):
            pk, pv = _prior_kv(wl.keys_attended(ly, steps[-1]) - 1, wl.Hkv, wl.d, 9001 + 31 * b + li)
            for s_ in steps:
                sec_step[s_] += _oracle_decode_one(wl, li, s_, b, pk, pv)
    total_sec = sum(sec_step.values())
    total_bytes = sum(wl.kv_bytes(ly, s_) for s_ in steps for ly in wl.layers)
    out["cpu_baseline_period_decode"] = {
        "value": total_bytes / total_sec / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"{wl.name}: steps 0, 63, 127 x 8 layers x {wl.B} sequences, fp64 NumPy, {total_sec:.1f} s",
        "s_per_step": {str(k): round(v, 3) for k, v in sec_step.items()}}
    log(f"[bench]   {out['cpu_baseline_period_decode']}")
    return out


# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="",
                    help="prefill_local|prefill_global|prefill_chunked|mixer|decode|period|gemma|copy_calibration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--period-steps", type=int, default=128)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)

    import torch

    import sliding_window_global_amd as swg
    from sliding_window_global_amd.profiling import read_traffic
    from synthetic.workloads import (BATCHED_DECODE, GEMMA_GLOBAL_DECODE, GEMMA_GLOBAL_PREFILL,
                                     GEMMA_LOCAL_DECODE, GEMMA_LOCAL_PREFILL, GLOBAL_PREFILL, LOCAL_PREFILL,
                                     MIXER_LOCAL_PREFILL, PERIOD_DECODE)

    torch.cuda.set_device(0)
    swg._lib.load()
    only = args.only
    extra = {}
    local = None
    if only in ("", "prefill_local"):
        log("[bench] local prefill T=8192 W=2048")
        local = bench_prefill(torch, swg, LOCAL_PREFILL, args.steps, args.warmup, LOCAL_PREFILL.norm_offset)
        log(f"[bench]   {local}")
        extra["prefill_local_cold_cache"] = cold_summary(local)
        log("[bench] local prefill, Q normalised and rotated inside the attention kernel")
        u = bench_prefill(torch, swg, LOCAL_PREFILL, args.steps, args.warmup, LOCAL_PREFILL.norm_offset,
                          fuse_q=True)
        log(f"[bench]   {u}")
        extra["prefill_local_fused_q"] = {k: u[k] for k in ("workload", "ms_per_step", "ms_attn", "step_tflops",
                                                             "attn_tflops")}
        extra["prefill_local_fused_q"].update(cold_summary(u))
    if only in ("", "prefill_global"):
        log("[bench] global prefill T=32768 YaRN")
        g = bench_prefill(torch, swg, GLOBAL_PREFILL, max(3, args.steps // 4), max(1, args.warmup // 2),
                          GLOBAL_PREFILL.norm_offset)
        log(f"[bench]   {g}")
        extra["prefill_global"] = {k: g[k] for k in ("workload", "ms_per_step", "ms_attn", "step_tflops", "attn_tflops")}
        extra["prefill_global"]["frac_mfma"] = g["attn_tflops"] / PEAK_BF16_TFLOPS
        extra["prefill_global"].update(cold_summary(g))
    if only in ("", "prefill_chunked"):
        for wl, chunk, n in ((LOCAL_PREFILL, 2048, args.steps), (GLOBAL_PREFILL, 8192, max(3, args.steps // 4))):
            log(f"[bench] chunked prefill {wl.name} chunk={chunk}")
            r = bench_chunked_prefill(torch, swg, wl, chunk, n, max(1, args.warmup // 2))
            log(f"[bench]   {r}")
            extra[r["workload"]] = r
    if only in ("", "mixer"):
        log("[bench] attention sublayer, local prefill T=8192 D=5120")
        r = bench_mixer(torch, swg, MIXER_LOCAL_PREFILL, args.steps, args.warmup)
        log(f"[bench]   {r}")
        extra[r["workload"]] = r
    if only in ("", "decode"):
        for li in (0, 1):
            log(f"[bench] batched decode layer {li}")
            r = bench_decode_batched(torch, swg, BATCHED_DECODE, li, args.steps, args.warmup)
            log(f"[bench]   {r}")
            extra[r["workload"]] = r
        log("[bench] batched decode, global layer, post-RoPE cache")
        r = bench_decode_batched(torch, swg, BATCHED_DECODE, 1, args.steps, args.warmup, post_rope=True)
        log(f"[bench]   {r}")
        extra[r["workload"]] = r
        log("[bench] ragged batched decode, global layer")
        r = bench_decode_ragged(torch, swg, BATCHED_DECODE, 1, args.steps, args.warmup)
        log(f"[bench]   {r}")
        extra[r["workload"]] = r
    if only in ("", "gemma"):
        for wl, n in ((GEMMA_LOCAL_PREFILL, args.steps), (GEMMA_GLOBAL_PREFILL, max(3, args.steps // 4))):
            log(f"[bench] Gemma-shaped prefill {wl.name}")
            r = bench_gemma_prefill(torch, swg, wl, n, max(1, args.warmup // 2))
            log(f"[bench]   {r}")
            extra[r["workload"]] = r
        for wl in (GEMMA_LOCAL_DECODE, GEMMA_GLOBAL_DECODE):
            log(f"[bench] Gemma-shaped decode {wl.name}")
            r = bench_gemma_decode(torch, swg, wl, args.steps, args.warmup)
            log(f"[bench]   {r}")
            extra[r["workload"]] = r
    if only in ("", "period"):
        log("[bench] 8-layer period decode")
        r = bench_period(torch, swg, PERIOD_DECODE, args.period_steps)
        log(f"[bench]   {r}")
        extra["period_decode"] = r
        log("[bench] 8-layer period decode, one launch per layer step")
        r = bench_period(torch, swg, PERIOD_DECODE, args.period_steps, fused=True)
        log(f"[bench]   {r}")
        extra["period_decode_one_launch"] = r

    if only == "copy_calibration":
        # a plain device-to-device copy of known size: the reference for HBM byte counters
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration"] = {"bytes_read": n, "bytes_written": n, "launches": args.steps}
    if local is None:
        print(json.dumps({"metric": METRIC, "partial": only, "extra": extra}))
        return
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu oracle baseline")
        cpu = cpu_baseline(LOCAL_PREFILL, LOCAL_PREFILL.norm_offset, args.cpu_rows)
        log(f"[bench]   {cpu}")
        extra.update(cpu_baselines_extra())
    line = {
        "metric": METRIC,
        "value": round(local["step_tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(local["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": LOCAL_PREFILL.name, "B": 1, "T": 8192, "Hq": 64, "Hkv": 8, "d": 128,
                   "window": 2048,
                   "step": "kv_append + attn_prefill",
                   "cache_state": "inputs resident in HBM; the 256 MB last-level cache is not flushed "
                                  "between steps, so the prefill finds much of the Q' the append has just "
                                  "written there (as in an append -> prefill pipeline); extra."
                                  "prefill_local_cold_cache has each kernel after a 512 MiB flush",
                   "timing": f"{SETTLE_S} s of untimed steps (clocks settle), then W warmup steps, then "
                             "ms_per_step = K whole steps / K; roofline from the median HIP-event duration "
                             "of the attention launch"},
        "roofline": {"bound": "mfma", "achieved": round(local["attn_tflops"], 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(local["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": read_traffic(os.path.join(ROOT, "profiles", "prefill_local_T8192_hbm_traffic.txt")),
                     "kernel": "prefill_bf16_kernel<true, false>", "flop_per_launch": LOCAL_PREFILL.flops()},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
