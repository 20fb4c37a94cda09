"""GPU parity of the attention sublayer around the hot path (「PLaMo 3アーキテクチャ徹底解析」
§3.2, §4.1, §4.5): the projections (plamo_linear), the offset RMSNorm (plamo_rms_norm) and
the composed sublayer (pre norm, fused QKV projection, attention, output projection, post
norm, residual) against the fp64 oracle on the same bf16 inputs. Bar: |gpu - ref| <=
2e-2 + 2e-2 |ref| elementwise (bf16)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from helpers import TOL_BF16, assert_parity
from oracle import LayerKVCache, mixer_layer_step, offset_rms_norm
from synthetic.workloads import MIXER_LOCAL_PREFILL, MixerWorkload, Rope

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


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(1, 1024, 5120), (300, 1536, 256), (8192, 1024, 5120), (77, 5120, 8192),
                                   (8192, 8192, 5120), (8192, 5120, 8192), (200, 264, 128)])
def test_linear_matches_fp64_matmul(M, N, K):
    g = torch.Generator(device="cuda").manual_seed(M + N + K)
    x = torch.randn((M, K), generator=g, device="cuda").bfloat16()
    w = (torch.randn((N, K), generator=g, device="cuda") / math.sqrt(K)).bfloat16()
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    swg.plamo_linear(x, w, y)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, 64).astype(int))
    ref = host(x)[rows] @ host(w).T
    assert_parity(host(y)[rows], ref, TOL_BF16, f"linear {M}x{N}x{K}")


def _canaried(n, shape):
    """A view of the first n elements of a NaN-filled buffer 1024 elements longer, and the buffer."""
    buf = torch.full((n + 1024,), float("nan"), dtype=torch.bfloat16, device="cuda")
    return buf[:n].view(*shape), buf


@pytest.mark.parametrize("M,N,K", [(77, 264, 128), (300, 1536, 256), (1, 1024, 5120), (513, 520, 64),
                                   (8000, 5112, 64)])
def test_linear_writes_exactly_its_output(M, N, K):
    """Every output element is written and nothing past the output: y sits at the front of a
    NaN-filled buffer, whose tail must stay NaN, with ragged row and column tiles (the epilogue
    stages each wave's tile in LDS and writes 16-byte chunks of whole rows); every row checked.
    8000 x 5112 takes the 320-wide column tiles (512 blocks of 320 against 640 of 256)."""
    g = torch.Generator(device="cuda").manual_seed(7 * M + N)
    x = torch.randn((M, K), generator=g, device="cuda").bfloat16()
    w = (torch.randn((N, K), generator=g, device="cuda") / math.sqrt(K)).bfloat16()
    y, buf = _canaried(M * N, (M, N))
    swg.plamo_linear(x, w, y)
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf[M * N:]).all()), "write past the output"
    assert not bool(torch.isnan(y).any()), "output element left unwritten"
    assert_parity(host(y), host(x) @ host(w).T, TOL_BF16, f"linear {M}x{N}x{K}, all rows")


def test_qkv_projection_writes_exactly_its_outputs():
    """The Q | K | V split of the fused projection at a ragged shape: each part written whole,
    nothing past any of them, every row checked."""
    M, D, Hq, Hkv, d = 301, 256, 8, 2, 128
    g = torch.Generator(device="cuda").manual_seed(4711)
    u = torch.randn((M, D), generator=g, device="cuda").bfloat16()
    w = (torch.randn(((Hq + 2 * Hkv) * d, D), generator=g, device="cuda") / math.sqrt(D)).bfloat16()
    q, qb = _canaried(M * Hq * d, (M, Hq, d))
    k, kb = _canaried(M * Hkv * d, (M, Hkv, d))
    v, vb = _canaried(M * Hkv * d, (M, Hkv, d))
    swg.plamo_qkv_projection(u, w, q, k, v)
    torch.cuda.synchronize()
    for name, t, buf in (("Q", q, qb), ("K", k, kb), ("V", v, vb)):
        assert bool(torch.isnan(buf[t.numel():]).all()), f"write past the {name} part"
        assert not bool(torch.isnan(t).any()), f"{name} element left unwritten"
    full = host(u) @ host(w).T
    assert_parity(host(q).reshape(M, -1), full[:, :Hq * d], TOL_BF16, "Q part, all rows")
    assert_parity(host(k).reshape(M, -1), full[:, Hq * d:(Hq + Hkv) * d], TOL_BF16, "K part, all rows")
    assert_parity(host(v).reshape(M, -1), full[:, (Hq + Hkv) * d:], TOL_BF16, "V part, all rows")


@pytest.mark.parametrize("M,D,Hq,Hkv", [(8192, 5120, 64, 8), (301, 256, 8, 2), (3, 5120, 64, 8)])
def test_qkv_projection_matches_fp64(M, D, Hq, Hkv):
    """One GEMM against the fused weight, its output columns split into Q | K | V at Hq d and
    (Hq + Hkv) d (「PLaMo 3アーキテクチャ徹底解析」 §4.1)."""
    d = 128
    g = torch.Generator(device="cuda").manual_seed(M + D)
    u = torch.randn((M, D), generator=g, device="cuda").bfloat16()
    w = (torch.randn(((Hq + 2 * Hkv) * d, D), generator=g, device="cuda") / math.sqrt(D)).bfloat16()
    q = torch.empty((M, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((M, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    swg.plamo_qkv_projection(u, w, q, k, v)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, M - 1, 48).astype(int))
    full = host(u)[rows] @ host(w).T
    assert_parity(host(q).reshape(M, -1)[rows], full[:, :Hq * d], TOL_BF16, "Q part")
    assert_parity(host(k).reshape(M, -1)[rows], full[:, Hq * d:(Hq + Hkv) * d], TOL_BF16, "K part")
    assert_parity(host(v).reshape(M, -1)[rows], full[:, (Hq + Hkv) * d:], TOL_BF16, "V part")


@pytest.mark.parametrize("offset,residual", [(1.0, False), (0.2, True)])
def test_rms_norm_matches_oracle(offset, residual):
    g = torch.Generator(device="cuda").manual_seed(7)
    x = (torch.randn((333, 5120), generator=g, device="cuda") * 3).bfloat16()
    w = (torch.randn((5120,), generator=g, device="cuda") * 0.02).bfloat16()
    r = torch.randn((333, 5120), generator=g, device="cuda").bfloat16() if residual else None
    y = torch.empty_like(x)
    swg.plamo_rms_norm(x, w, y, offset=offset, residual=r)
    torch.cuda.synchronize()
    ref = offset_rms_norm(host(x), host(w), offset) + (host(r) if residual else 0.0)
    assert_parity(host(y), ref, TOL_BF16, "rms_norm")


def _weights_host(w):
    return {k: host(v) for k, v in w.items()}


@pytest.mark.parametrize("fuse_q", [True, False], ids=["fused_q", "unfused"])
@pytest.mark.parametrize("window", [128, 0], ids=["local128", "global"])
def test_mixer_small_matches_oracle(window, fuse_q):
    """Chunks [200, 100] then two decode steps of the sublayer at a small hidden width
    (D = 256, Hq = 8, Hkv = 2, d = 128), B = 2; the attention with Q normalised and rotated
    inside the prefill kernel (the sublayer's default at d = 128) and through the append."""
    wl = MixerWorkload(name="mixer_small", B=2, T=302, D=256, Hq=8, Hkv=2, d=128, window=window,
                       rope=Rope(1e4) if window else Rope(1e6, 64.0), seed=4321 + window)
    x, wdev = wl.draw_device("cuda")
    wts = layer.MixerWeights(Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, **wdev)
    cap = window if window else wl.T
    kc = torch.zeros((wl.B, wl.Hkv, cap, wl.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    tab = swg.make_rope_table(wl.T + 64, swg.RopeParams(wl.rope.theta, wl.rope.yarn_factor))
    got, p = [], 0
    for T in (200, 100):
        mb, _ = layer.mixer_prefill(x[:, p:p + T].contiguous(), wts, window=window, rope_table=tab,
                                    k_cache=kc, v_cache=vc, pos_offset=p, fuse_q=fuse_q)
        torch.cuda.synchronize()
        got.append(host(mb.out))
        p += T
    for _ in range(2):
        mb, _ = layer.mixer_decode(x[:, p:p + 1].contiguous(), wts, kc, vc, window=window, pos_offset=p,
                                   rope_table=tab)
        torch.cuda.synchronize()
        got.append(host(mb.out))
        p += 1
    wh, xh = _weights_host(wdev), host(x)
    for b in range(wl.B):
        cache = LayerKVCache(wl.Hkv, wl.d, window)
        p = 0
        for i, T in enumerate((200, 100, 1, 1)):
            ref = mixer_layer_step(xh[b, p:p + T], cache, w_pre=wh["w_pre"], w_qkv=wh["w_qkv"], w_o=wh["w_o"],
                                   w_post=wh["w_post"], Hq=wl.Hq, Hkv=wl.Hkv, theta=wl.rope.theta,
                                   yarn_factor=wl.rope.yarn_factor, q_norm_w=wh["wq"], k_norm_w=wh["wk"])
            assert_parity(got[i][b], ref, TOL_BF16, f"sequence {b} call {i}")
            p += T


def test_mixer_full_size_sampled_rows():
    """The sublayer at PLaMo 3 31B's widths (D = 5120, 64/8 heads) on the local-layer prefill
    (T = 8192, W = 2048), as the benchmark runs it. A local row depends only on the W tokens
    ending at it and renumbering does not change scores (§4.4), so the oracle evaluates each
    sampled row block on the slice of the W - 1 tokens before it plus the block."""
    wl = MIXER_LOCAL_PREFILL
    x, wdev = wl.draw_device("cuda")
    wts = layer.MixerWeights(Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, **wdev)
    kc = torch.empty((wl.B, wl.Hkv, wl.window, wl.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    tab = swg.make_rope_table(wl.T + 64, swg.RopeParams(wl.rope.theta, wl.rope.yarn_factor))
    mb, _ = layer.mixer_prefill(x, wts, window=wl.window, rope_table=tab, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    out = host(mb.out[0])
    wh, xh = _weights_host(wdev), host(x[0])
    for r0, r1 in ((0, 8), (2045, 2053), (8184, 8192)):
        s0 = max(0, r0 - wl.window + 1)
        ref = mixer_layer_step(xh[s0:r1], LayerKVCache(wl.Hkv, wl.d, wl.window), w_pre=wh["w_pre"],
                               w_qkv=wh["w_qkv"], w_o=wh["w_o"], w_post=wh["w_post"], Hq=wl.Hq, Hkv=wl.Hkv,
                               theta=wl.rope.theta, q_norm_w=wh["wq"], k_norm_w=wh["wk"],
                               rows=np.arange(r0 - s0, r1 - s0))
        assert_parity(out[r0:r1], ref, TOL_BF16, f"rows {r0}..{r1}")
