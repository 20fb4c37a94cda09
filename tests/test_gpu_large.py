"""GPU parity at the largest buffers: local-layer prefills of 524288 tokens from an empty
cache (「PLaMo 3アーキテクチャ徹底解析」 §4.4, §4.5, §5.1; the §8 table's d = 256 layer too),
whose Q, Q' and O hold 2^32 elements each, so the offsets of rows past 262144 exceed 2^31
elements.

The inputs are one seeded block of W tokens repeated along the sequence (every token
still sits at its own position, so the rotations differ). Sampled rows are checked against
the fp64 oracle run on their window alone: a one-shot local prefill's row r attends keys
r - W + 1 .. r at positions r - j apart, and RoPE scores depend on positions only through
that difference (§6.1), so the oracle on the slice of those W tokens (positions 0 .. W - 1)
gives the same row up to rounding.

Bar: |gpu - oracle| <= 2e-2 + 2e-2 |oracle| elementwise (bf16, helpers.TOL_BF16)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import TOL_BF16, assert_parity, oracle_prefill
from synthetic import Draw
from oracle import LayerKVCache, attention_layer_step
from synthetic.workloads import GEMMA_LOCAL_LAYER, Rope

pytestmark = pytest.mark.gpu

swg = pytest.importorskip("sliding_window_global_amd")
from sliding_window_global_amd import layer  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    swg._lib.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_local_prefill_half_million_tokens():
    T, base_T, Hq, Hkv, d, W = 524288, 2048, 64, 8, 128, 2048
    rope = Rope(1e4)
    dr = Draw(9500, True)
    q0, k0, v0 = dr.normal((1, base_T, Hq, d)), dr.normal((1, base_T, Hkv, d)), dr.normal((1, base_T, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    reps = T // base_T
    q = dev(q0).repeat(1, reps, 1, 1)
    k = dev(k0).repeat(1, reps, 1, 1)
    v = dev(v0).repeat(1, reps, 1, 1)
    assert q.numel() == 2 ** 32
    tab = swg.make_rope_table(T + 64, swg.RopeParams(rope.theta))
    kw = dict(q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0, window=W, rope_table=tab)
    rows = np.array([0, 2047, 262143, 262144, 262145, 393221, T - 2, T - 1])
    got = {}
    for fuse_q in (False, True):
        print(f"\n[large] local prefill T={T} fuse_q={fuse_q}", flush=True)
        bufs = layer.prefill(q, k, v, fuse_q=fuse_q, **kw)
        torch.cuda.synchronize()
        got[fuse_q] = host(bufs.out[:, torch.from_numpy(rows).cuda()])
        del bufs
        torch.cuda.empty_cache()
    for i, r in enumerate(rows):
        s0 = max(0, r - W + 1)
        idx = np.arange(s0, r + 1) % base_T
        ref = oracle_prefill(q0[:, idx], k0[:, idx], v0[:, idx], window=W, rope=rope, wq=wq, wk=wk,
                             norm_offset=1.0, rows=np.array([r - s0]))
        for fuse_q, g in got.items():
            assert_parity(g[:, i:i + 1], ref, TOL_BF16, f"row {r} fuse_q={fuse_q}")


def test_gemma_local_prefill_half_million_tokens():
    """The d = 256 local layer (window 1024, gain-only norms, V norm, factor 1, K cached after
    RoPE) through the wide kernels at the same size."""
    L = GEMMA_LOCAL_LAYER
    T, W = 524288, L.window
    dr = Draw(9501, True)
    q0, k0, v0 = L.draw_tokens(dr, 1, W)
    wq, wk = L.draw_gains(dr)
    reps = T // W
    q = dev(q0).repeat(1, reps, 1, 1)
    k = dev(k0).repeat(1, reps, 1, 1)
    v = dev(v0).repeat(1, reps, 1, 1)
    assert q.numel() == 2 ** 32
    tab = swg.make_rope_table(T + 64, swg.RopeParams(L.theta, partial=L.partial), d=L.d)
    print(f"\n[large] gemma local prefill T={T} d={L.d}", flush=True)
    bufs = layer.prefill(q, k, v, window=W, rope_table=tab, q_norm_w=dev(wq), k_norm_w=dev(wk),
                         norm_offset=L.norm_offset, norm_eps=L.eps, softmax_scale=L.scale, cache_post_rope=True,
                         v_norm=True)
    torch.cuda.synchronize()
    rows = np.array([0, 1023, 262143, 262144, 262145, 393221, T - 2, T - 1])
    got = host(bufs.out[:, torch.from_numpy(rows).cuda()])
    del bufs
    torch.cuda.empty_cache()
    for i, r in enumerate(rows):
        s0 = max(0, r - W + 1)
        idx = np.arange(s0, r + 1) % W
        ref = attention_layer_step(q0[0, idx], k0[0, idx], v0[0, idx], LayerKVCache(L.Hkv, L.d, W, post_rope=True),
                                   theta=L.theta, partial=1.0, q_norm_w=wq, k_norm_w=wk, norm_offset=L.norm_offset,
                                   eps=L.eps, scale=L.scale, v_norm=True, rows=np.array([r - s0]))
        assert_parity(got[0, i:i + 1], ref, TOL_BF16, f"row {r}")


def test_decode_caches_beyond_2_32_elements():
    """Batched global decode at 131072 keys and B = 64 (「PLaMo 3アーキテクチャ徹底解析」 §4.4,
    §4.5; §2.3: the KV bytes a decode step reads): each cache holds 64 x 8 x 131072 x 128 ≈
    8.6e9 elements (17 GiB), so the later sequences start past 2^32 elements. Through
    plamo_attn_decode and through the one-launch step; the first and the last sequence
    against the oracle."""
    from helpers import oracle_decode_one
    from synthetic.workloads import device_normal_bf16

    B, Hq, Hkv, d, pos = 64, 64, 8, 128, 131071
    rope = Rope(1e6, 64.0)
    cap = pos + 1
    print(f"\n[large] decode B={B} keys={cap} cache elements={B * Hkv * cap * d}", flush=True)
    kc = device_normal_bf16((B, Hkv, cap, d), 9510, "cuda")
    vc = device_normal_bf16((B, Hkv, cap, d), 9511, "cuda")
    torch.cuda.empty_cache()
    assert kc.numel() > 2 ** 32
    check_b = [0, B - 1]
    dr = Draw(9512, True)
    q, k, v = dr.normal((B, 1, Hq, d)), dr.normal((B, 1, Hkv, d)), dr.normal((B, 1, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    refs = {}
    for b in check_b:
        pk = host(kc[b, :, :pos]).transpose(1, 0, 2)
        pv = host(vc[b, :, :pos]).transpose(1, 0, 2)
        refs[b] = oracle_decode_one(q[b], k[b], v[b], pk, pv, pos, window=0, rope=rope, wq=wq, wk=wk)
        del pk, pv
    tab = swg.make_rope_table(cap + 64, swg.RopeParams(rope.theta, rope.yarn_factor, rope.orig_ctx,
                                                       rope.beta_fast, rope.beta_slow))
    for fused in (False, True):
        # (both calls write the same new token into slot pos; the oracle's prior is slots < pos)
        bufs = layer.decode(dev(q), dev(k), dev(v), kc, vc, window=0, pos_offset=pos, rope_table=tab,
                            q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0, fused=fused)
        torch.cuda.synchronize()
        out = host(bufs.out)
        for b in check_b:
            assert_parity(out[b], refs[b], TOL_BF16, f"decode b={b} fused={fused}")
        del bufs
