"""The five synthetic workloads of PLaMo 3's attention hot path, with their sizes.

Shapes follow the PLaMo 3 31B configuration (64 query heads, 8 KV heads, head
dimension 128, window 2048, local RoPE base 1e4, global base 1e6) as given in
「PLaMo 3アーキテクチャ徹底解析」 §2.1. Values are synthetic N(0, 1) draws; the
norm gains are the stored-weight part only, drawn N(0, 0.02), with the offset
passed separately.

Draw order within a workload's stream: q, k, v, q-norm weight, k-norm weight.
Large decode caches are drawn separately (``cache_seed``), on the device that
holds them, by ``synthetic.device_normal_bf16``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import BASE_SEED, Draw, bf16_round


@dataclass(frozen=True)
class Rope:
    theta: float
    yarn_factor: float = 0.0  # <= 1 disables YaRN
    orig_ctx: float = 4096.0
    beta_fast: float = 32.0
    beta_slow: float = 1.0


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    window: int  # 0 = global causal layer
    rope: Rope
    norm_offset: float | None  # None = no Q/K norm
    bf16: bool
    seed: int
    norm_std: float = 0.02
    eps: float = 1e-6

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def draw(self):
        """Return dict of float32 arrays (bf16-exact when ``bf16``):
        q [B,T,Hq,d], k [B,T,Hkv,d], v [B,T,Hkv,d], wq [d], wk [d] (None without norm)."""
        dr = Draw(self.seed, self.bf16)
        q = dr.normal((self.B, self.T, self.Hq, self.d))
        k = dr.normal((self.B, self.T, self.Hkv, self.d))
        v = dr.normal((self.B, self.T, self.Hkv, self.d))
        wq = wk = None
        if self.norm_offset is not None:
            wq = dr.normal((self.d,), self.norm_std)
            wk = dr.normal((self.d,), self.norm_std)
        return dict(q=q, k=k, v=v, wq=wq, wk=wk)

    def attended_pairs_per_head(self) -> int:
        """Number of unmasked (query, key) pairs of one head, prefill from an empty cache."""
        T, W = self.T, self.window
        if W <= 0 or W >= T:
            return T * (T + 1) // 2
        return W * (W + 1) // 2 + (T - W) * W

    def flops(self) -> float:
        """Algorithmic FLOP: 2·d for the score and 2·d for the weighted sum per pair and head."""
        return 4.0 * self.d * self.Hq * self.B * self.attended_pairs_per_head()


TINY_SWA_FP32 = PrefillWorkload(
    name="tiny_swa_prefill_fp32", B=1, T=512, Hq=8, Hkv=2, d=128, window=128,
    rope=Rope(theta=1e4), norm_offset=None, bf16=False, seed=BASE_SEED + 1)

LOCAL_PREFILL = PrefillWorkload(
    name="local_prefill_T8192_W2048", B=1, T=8192, Hq=64, Hkv=8, d=128, window=2048,
    rope=Rope(theta=1e4), norm_offset=0.2, bf16=True, seed=BASE_SEED + 2)

GLOBAL_PREFILL = PrefillWorkload(
    name="global_prefill_T32768_yarn64", B=1, T=32768, Hq=64, Hkv=8, d=128, window=0,
    rope=Rope(theta=1e6, yarn_factor=64.0), norm_offset=5.0 ** -1.5, bf16=True,
    seed=BASE_SEED + 3)


@dataclass(frozen=True)
class DecodeLayer:
    window: int  # 0 = global
    rope: Rope


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    pos_offset: int  # absolute position of the first decoded token
    layers: tuple
    steps: int
    seed: int
    norm_offset: float = 1.0
    norm_std: float = 0.02
    eps: float = 1e-6

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def keys_attended(self, layer: DecodeLayer, step: int = 0) -> int:
        p = self.pos_offset + step
        kept = p if layer.window == 0 else min(p, layer.window - 1)
        return kept + 1

    def cache_cap(self, layer: DecodeLayer) -> int:
        if layer.window == 0:
            return self.pos_offset + self.steps
        return layer.window

    def kv_bytes(self, layer: DecodeLayer, step: int = 0) -> int:
        """Algorithmic KV bytes read by one decode of one layer: K and V rows (bf16) of every
        attended key, once per sequence and KV head (shared by the query heads of a group)."""
        return 2 * 2 * self.B * self.Hkv * self.d * self.keys_attended(layer, step)

    def draw_new_tokens(self, step: int, layer_index: int):
        """q [B,1,Hq,d], k, v [B,1,Hkv,d] and norm weights for one (step, layer), bf16-exact."""
        dr = Draw(self.seed * 1000003 + step * 64 + layer_index, True)
        q = dr.normal((self.B, 1, self.Hq, self.d))
        k = dr.normal((self.B, 1, self.Hkv, self.d))
        v = dr.normal((self.B, 1, self.Hkv, self.d))
        wq = dr.normal((self.d,), self.norm_std)
        wk = dr.normal((self.d,), self.norm_std)
        return dict(q=q, k=k, v=v, wq=wq, wk=wk)

    def cache_seed(self, layer_index: int) -> int:
        return self.seed * 7919 + layer_index


LOCAL_ROPE = Rope(theta=1e4)
GLOBAL_ROPE = Rope(theta=1e6, yarn_factor=64.0)

BATCHED_DECODE = DecodeWorkload(
    name="batched_decode_B64", B=64, Hq=64, Hkv=8, d=128, pos_offset=32767,
    layers=(DecodeLayer(2048, LOCAL_ROPE), DecodeLayer(0, GLOBAL_ROPE)), steps=1,
    seed=BASE_SEED + 4)

PERIOD_DECODE = DecodeWorkload(
    name="period8_decode_B8_ctx131072", B=8, Hq=64, Hkv=8, d=128, pos_offset=131071,
    layers=tuple([DecodeLayer(2048, LOCAL_ROPE)] * 7 + [DecodeLayer(0, GLOBAL_ROPE)]),
    steps=128, seed=BASE_SEED + 5)


@dataclass(frozen=True)
class MixerWorkload:
    """The attention sublayer around the hot path at PLaMo 3 31B's widths (hidden D = 5120,
    「PLaMo 3アーキテクチャ徹底解析」 §2.1, §3.2, §4.1): random weights, projections scaled by
    1/sqrt(fan-in) so that Q/K/V and the output projection stay O(1); norm weights N(0, 0.02);
    residual input N(0, 1)."""
    name: str
    B: int
    T: int
    D: int
    Hq: int
    Hkv: int
    d: int
    window: int
    rope: Rope
    seed: int
    norm_std: float = 0.02

    def draw_device(self, device):
        """(x [B, T, D], dict of bf16 weights) drawn on the device (synthetic.device_normal_bf16)."""
        qkv_rows = (self.Hq + 2 * self.Hkv) * self.d
        x = device_normal_bf16((self.B, self.T, self.D), self.seed, device)
        w = dict(
            w_pre=(device_normal_bf16((self.D,), self.seed + 1, device).float() * self.norm_std).bfloat16(),
            w_qkv=(device_normal_bf16((qkv_rows, self.D), self.seed + 2, device).float()
                   / math.sqrt(self.D)).bfloat16(),
            w_o=(device_normal_bf16((self.D, self.Hq * self.d), self.seed + 3, device).float()
                 / math.sqrt(self.Hq * self.d)).bfloat16(),
            w_post=(device_normal_bf16((self.D,), self.seed + 4, device).float() * self.norm_std).bfloat16(),
            wq=(device_normal_bf16((self.d,), self.seed + 5, device).float() * self.norm_std).bfloat16(),
            wk=(device_normal_bf16((self.d,), self.seed + 6, device).float() * self.norm_std).bfloat16(),
        )
        return x, w

    def gemm_flops(self) -> float:
        """2 M N K for the fused QKV projection and the output projection."""
        M = self.B * self.T
        return 2.0 * M * self.D * (self.Hq + 2 * self.Hkv) * self.d + 2.0 * M * self.Hq * self.d * self.D

    def attention_flops(self) -> float:
        T, W = self.T, self.window
        pairs = T * (T + 1) // 2 if W <= 0 or W >= T else W * (W + 1) // 2 + (T - W) * W
        return 4.0 * self.d * self.Hq * self.B * pairs


MIXER_LOCAL_PREFILL = MixerWorkload(
    name="mixer_local_prefill_T8192_D5120", B=1, T=8192, D=5120, Hq=64, Hkv=8, d=128, window=2048,
    rope=Rope(theta=1e4), seed=BASE_SEED + 7)


def ragged_positions(B: int, max_pos: int, seed: int) -> np.ndarray:
    """Positions of the new token of each sequence of a ragged decode batch: independent
    uniform integers in [0, max_pos], the last one set to max_pos so that the batch's bound
    is reached (int64 [B])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    p = rng.integers(0, max_pos + 1, size=B, dtype=np.int64)
    p[-1] = max_pos
    return p


RAGGED_DECODE_SEED = BASE_SEED + 6  # positions of the ragged batched-decode case


def device_normal_bf16(shape, seed: int, device):
    """N(0, 1) draws rounded to bfloat16, generated by torch on ``device`` (used for
    decode caches of several GiB). The same (shape, seed, device type) gives the same
    values; the CPU side copies whatever it needs from the returned tensor."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


# ----------------------------------------------------------------------------
# The Gemma-4-shaped second workload (「PLaMo 3アーキテクチャ徹底解析」 §8 comparison table,
# §6.4 p-RoPE, §9.4 gains): local layers d = 256, Hq = 32, Hkv = 16, window 1024, RoPE base
# 1e4 on every pair; global layers d = 512, Hq = 32, Hkv = 4, p-RoPE (p = 0.25, base 1e6),
# V taken from the K projection. Q/K norm gain = the stored weight (offset 0): a level
# drawn in the ranges the page reports for the released weights (Q in [0.95, 1.05], K in
# [0.120, 0.132] local or [0.060, 0.065] global; constant within each vector there) plus
# independent per-component N(0, 0.02) noise, so that each component of the gain differs;
# V divided by its RMS; dot-product factor 1; K cached after RoPE.
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class GemmaLayer:
    kind: str          # "local" or "global"
    d: int
    Hq: int
    Hkv: int
    window: int        # 0 = global causal layer
    theta: float
    partial: float     # p-RoPE fraction of pairs that turn; 0 = all
    k_gain: tuple      # range of the constant K gain
    kv_shared: bool    # V is the K projection output
    q_gain: tuple = (0.95, 1.05)
    scale: float = 1.0
    norm_offset: float = 0.0
    eps: float = 1e-6

    gain_noise_std: float = 0.02

    def draw_gains(self, dr: Draw):
        """(wq, wk) [d] (the gain itself, offset 0): the level of each vector uniform in its
        range, plus per-component N(0, gain_noise_std) noise; stored as bf16."""
        gq = dr.uniform(*self.q_gain)
        gk = dr.uniform(*self.k_gain)
        nq = dr.normal((self.d,), self.gain_noise_std)
        nk = dr.normal((self.d,), self.gain_noise_std)
        return (bf16_round(np.float32(gq) + nq), bf16_round(np.float32(gk) + nk))

    def draw_tokens(self, dr: Draw, B: int, T: int):
        """q [B,T,Hq,d], k [B,T,Hkv,d], v (the same array as k when shared), bf16-exact."""
        q = dr.normal((B, T, self.Hq, self.d))
        k = dr.normal((B, T, self.Hkv, self.d))
        v = k if self.kv_shared else dr.normal((B, T, self.Hkv, self.d))
        return q, k, v


GEMMA_LOCAL_LAYER = GemmaLayer("local", 256, 32, 16, 1024, 1e4, 0.0, (0.120, 0.132), False)
GEMMA_GLOBAL_LAYER = GemmaLayer("global", 512, 32, 4, 0, 1e6, 0.25, (0.060, 0.065), True)


@dataclass(frozen=True)
class GemmaPrefill:
    name: str
    layer: GemmaLayer
    B: int
    T: int
    seed: int

    def draw(self):
        dr = Draw(self.seed, True)
        q, k, v = self.layer.draw_tokens(dr, self.B, self.T)
        wq, wk = self.layer.draw_gains(dr)
        return dict(q=q, k=k, v=v, wq=wq, wk=wk)

    def attended_pairs_per_head(self) -> int:
        T, W = self.T, self.layer.window
        if W <= 0 or W >= T:
            return T * (T + 1) // 2
        return W * (W + 1) // 2 + (T - W) * W

    def flops(self) -> float:
        return 4.0 * self.layer.d * self.layer.Hq * self.B * self.attended_pairs_per_head()


@dataclass(frozen=True)
class GemmaDecode:
    """Batched decode of one Gemma-shaped layer: B sequences whose new token sits at
    pos_offset; the cache holds the kept earlier tokens (K after RoPE, scaled to the layer's
    K gain; V of unit RMS), drawn on the device."""
    name: str
    layer: GemmaLayer
    B: int
    pos_offset: int
    seed: int

    def keys_attended(self) -> int:
        W = self.layer.window
        return (self.pos_offset if W == 0 else min(self.pos_offset, W - 1)) + 1

    def cache_cap(self) -> int:
        return self.layer.window if self.layer.window else self.pos_offset + 1

    def kv_bytes(self) -> int:
        return 2 * 2 * self.B * self.layer.Hkv * self.layer.d * self.keys_attended()

    def draw_new_tokens(self):
        dr = Draw(self.seed, True)
        q, k, v = self.layer.draw_tokens(dr, self.B, 1)
        wq, wk = self.layer.draw_gains(dr)
        return dict(q=q, k=k, v=v, wq=wq, wk=wk)

    def cache_seed(self) -> int:
        return self.seed * 7919


GEMMA_LOCAL_PREFILL = GemmaPrefill("gemma_local_prefill_T8192_d256_W1024", GEMMA_LOCAL_LAYER, 1, 8192,
                                   BASE_SEED + 8)
GEMMA_GLOBAL_PREFILL = GemmaPrefill("gemma_global_prefill_T32768_d512_p0.25", GEMMA_GLOBAL_LAYER, 1, 32768,
                                    BASE_SEED + 9)
GEMMA_LOCAL_DECODE = GemmaDecode("gemma_local_decode_B64_ring1024", GEMMA_LOCAL_LAYER, 64, 32767, BASE_SEED + 10)
GEMMA_GLOBAL_DECODE = GemmaDecode("gemma_global_decode_B64_ctx32768", GEMMA_GLOBAL_LAYER, 64, 32767,
                                  BASE_SEED + 11)
