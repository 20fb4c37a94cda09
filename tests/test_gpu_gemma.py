"""GPU parity of the Gemma-4-shaped layers (head dims 256 and 512) against the fp64 oracle.

The layer is 「PLaMo 3アーキテクチャ徹底解析」 §8's comparison model: local d = 256, Hq = 32,
Hkv = 16, window 1024; global d = 512, Hkv = 4 with p-RoPE (§6.4) and V from the K
projection; gain-only Q/K norm, gainless V norm, dot-product factor 1, K cached after RoPE.
Bar: |gpu - oracle| <= 2e-2 + 2e-2 |oracle| elementwise (bf16, helpers.TOL_BF16). Small
cases compare every output row of a chunked prefill and of decode steps, and the cache
contents; the full-size workloads compare sampled rows / sequences the oracle computes."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import TOL_BF16, assert_parity
from oracle import LayerKVCache, attention_layer_step, rope_frequencies
from synthetic import Draw
from synthetic.workloads import (GEMMA_GLOBAL_DECODE, GEMMA_GLOBAL_LAYER, GEMMA_GLOBAL_PREFILL,
                                 GEMMA_LOCAL_DECODE, GEMMA_LOCAL_LAYER, GEMMA_LOCAL_PREFILL, GemmaLayer,
                                 device_normal_bf16)

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


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_partial(L: GemmaLayer) -> float:
    return L.partial if 0.0 < L.partial < 1.0 else 1.0


def table_for(L: GemmaLayer, max_pos: int):
    return swg.make_rope_table(max_pos, swg.RopeParams(L.theta, partial=L.partial), d=L.d)


def oracle_step(L: GemmaLayer, q, k, v, cache, wq, wk, rows=None):
    return attention_layer_step(q, k, v, cache, theta=L.theta, partial=oracle_partial(L), q_norm_w=wq,
                                k_norm_w=wk, norm_offset=L.norm_offset, eps=L.eps, scale=L.scale,
                                v_norm=True, rows=rows)


def gpu_kw(L: GemmaLayer, wq, wk):
    return dict(q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=L.norm_offset, norm_eps=L.eps,
                softmax_scale=L.scale, cache_post_rope=True, v_norm=True)


@pytest.mark.parametrize("L,Hq,Hkv,window", [(GEMMA_LOCAL_LAYER, 4, 2, 128), (GEMMA_GLOBAL_LAYER, 4, 1, 0)],
                         ids=["d256", "d512_p025"])
def test_wide_prefill_writes_exactly_its_output(L, Hq, Hkv, window):
    """The wide prefill's output sits at the front of a NaN-filled buffer 1024 elements longer:
    every element written (ragged last block: T = 300), nothing past it (each wave stages its
    16-row blocks in LDS and stores whole rows), every row of both sequences against the oracle."""
    import dataclasses
    L = dataclasses.replace(L, Hq=Hq, Hkv=Hkv, window=window)
    B, T, d = 2, 300, L.d
    dr = Draw(9090 + d, True)
    q, k, v = L.draw_tokens(dr, B, T)
    wq, wk = L.draw_gains(dr)
    cap = window if window else T
    kc = torch.full((B, Hkv, cap, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    bufs = layer.PrefillBuffers(B, T, Hq, Hkv, d, torch.bfloat16, "cuda", window, 0)
    n = B * T * Hq * d
    canary = torch.full((n + 1024,), float("nan"), dtype=torch.bfloat16, device="cuda")
    bufs.out = canary[:n].view(B, T, Hq, d)
    kd = dev(k)
    layer.prefill(dev(q), kd, kd if L.kv_shared else dev(v), window=window, rope_table=table_for(L, T + 64),
                  k_cache=kc, v_cache=vc, bufs=bufs, **gpu_kw(L, wq, wk))
    torch.cuda.synchronize()
    assert bool(torch.isnan(canary[n:]).all()), "write past the output"
    assert not bool(torch.isnan(bufs.out).any()), "output element left unwritten"
    for b in range(B):
        cache = LayerKVCache(Hkv, d, window, post_rope=True)
        ref = oracle_step(L, q[b], k[b], v[b], cache, wq, wk)
        assert_parity(host(bufs.out[b]), ref, TOL_BF16, f"d={d} sequence {b}")


@pytest.mark.parametrize("L", [GEMMA_LOCAL_LAYER, GEMMA_GLOBAL_LAYER], ids=["d256", "d512_p025"])
def test_wide_rope_table(L):
    """Coarse x fine product equals exp(i p w_j) from the oracle's frequencies; with p-RoPE the
    idle pairs (j >= 64 of 256) hold exactly (1, 0) at every position."""
    max_pos = 40000
    h = L.d // 2
    tab = host(table_for(L, max_pos)).reshape(-1, h, 2)
    omega, amp = rope_frequencies(L.d, L.theta, partial=oracle_partial(L))
    pos = np.array([0, 1, 63, 64, 65, 1023, 1024, 4095, 32767, 39999])
    f = tab[pos & 63]
    c = tab[64 + (pos >> 6)]
    zr = c[..., 0] * f[..., 0] - c[..., 1] * f[..., 1]
    zi = c[..., 0] * f[..., 1] + c[..., 1] * f[..., 0]
    ang = pos[:, None] * omega[None, :]
    assert np.max(np.abs(zr - amp * np.cos(ang))) < 2e-6
    assert np.max(np.abs(zi - amp * np.sin(ang))) < 2e-6
    n_rot = int(oracle_partial(L) * h)
    if n_rot < h:
        assert np.all(tab[:, n_rot:, 0] == 1.0) and np.all(tab[:, n_rot:, 1] == 0.0)


def _small_stream(L: GemmaLayer, Hq, Hkv, window, chunks, steps, seed):
    """Chunked prefill then decode steps of B = 2 sequences on one token stream; every output
    row and the final cache contents (K after RoPE, V of unit RMS) against the oracle. The
    caches start as NaN: a slot that holds no kept token must never be read."""
    import dataclasses
    L = dataclasses.replace(L, Hq=Hq, Hkv=Hkv, window=window)
    B, d = 2, L.d
    n = sum(chunks) + steps
    dr = Draw(seed, True)
    q, k, v = L.draw_tokens(dr, B, n)
    wq, wk = L.draw_gains(dr)
    cap = window if window else n
    kc = torch.full((B, Hkv, cap, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    tab = table_for(L, n + 64)
    kw = gpu_kw(L, wq, wk)

    def chunk(a, b):  # contiguous device copies; one tensor serves K and V when they are shared
        kd = dev(k[:, a:b])
        return dev(q[:, a:b]), kd, (kd if L.kv_shared else dev(v[:, a:b]))

    got, p = [], 0
    for T in chunks:
        bufs = layer.prefill(*chunk(p, p + T), window=window, rope_table=tab, k_cache=kc, v_cache=vc,
                             pos_offset=p, **kw)
        torch.cuda.synchronize()
        got.append(host(bufs.out))
        p += T
    for _ in range(steps):
        db = layer.decode(*chunk(p, p + 1), kc, vc, window=window, pos_offset=p, rope_table=tab, **kw)
        torch.cuda.synchronize()
        got.append(host(db.out))
        p += 1
    calls = list(chunks) + [1] * steps
    for b in range(B):
        cache = LayerKVCache(Hkv, d, window, post_rope=True)
        p = 0
        for i, T in enumerate(calls):
            ref = oracle_step(L, q[b, p:p + T], k[b, p:p + T], v[b, p:p + T], cache, wq, wk)
            assert_parity(got[i][b], ref, TOL_BF16, f"sequence {b}, call {i} (T={T})")
            p += T
        keep = cache.k.shape[0]
        slots = np.arange(n - keep, n) if not window else np.arange(n - keep, n) % window
        sl = torch.from_numpy(slots).cuda()
        assert_parity(host(kc[b][:, sl]).transpose(1, 0, 2), cache.k, TOL_BF16, f"cache K, sequence {b}")
        assert_parity(host(vc[b][:, sl]).transpose(1, 0, 2), cache.v, TOL_BF16, f"cache V, sequence {b}")


def test_gemma_local_small():
    """d = 256, window 100 (several tiles, masked at both ends), GQA 2, chunks 200 + 100, then
    3 decode steps (the ring wraps)."""
    _small_stream(GEMMA_LOCAL_LAYER, 4, 2, 100, [200, 100], 3, 7101)


def test_gemma_global_small():
    """d = 512 with p-RoPE, V from the K projection, GQA 8, chunks 150 + 107, then 3 decodes."""
    _small_stream(GEMMA_GLOBAL_LAYER, 8, 1, 0, [150, 107], 3, 7102)


def test_gemma_local_small_window_edges():
    """d = 256 with windows around the 32-key step and the 64-key tile: 31, 33, 65."""
    for w in (31, 33, 65):
        _small_stream(GEMMA_LOCAL_LAYER, 4, 2, w, [97, 70], 2, 7200 + w)


def test_gemma_local_group_sizes():
    """d = 256 with query-head groups of 3 (not a multiple of the heads a prefill block takes)
    and 4 (two blocks per KV head). These are the first seeds the test was written with; with
    dot-product factor 1 some rows' scores span ~19 log2 units, so two keys carry most of the
    weight and the rounding of the score operands shows most on this layer."""
    _small_stream(GEMMA_LOCAL_LAYER, 3, 1, 100, [130, 40], 2, 7103)
    _small_stream(GEMMA_LOCAL_LAYER, 8, 2, 64, [150, 60], 2, 7104)


def test_gemma_partly_filled_caches():
    """Rings that never fill (window 100 after 40 + 7 tokens and 3 decodes) and a global cache
    whose later slots are still unwritten: the NaN in those slots must not reach an output."""
    _small_stream(GEMMA_LOCAL_LAYER, 4, 2, 100, [40, 7], 3, 7301)
    _small_stream(GEMMA_GLOBAL_LAYER, 8, 1, 0, [30, 20], 2, 7302)


def test_gemma_wide_kernels_deterministic():
    """Repeated calls give bit-identical outputs: the d = 256 prefill at full size and the
    d = 512 split decode (fixed merge order, no atomics)."""
    wl = GEMMA_LOCAL_PREFILL
    L = wl.layer
    x = wl.draw()
    tab = table_for(L, wl.T + 64)
    qd, kd, vd = dev(x["q"]), dev(x["k"]), dev(x["v"])
    outs = [layer.prefill(qd, kd, vd, window=L.window, rope_table=tab, **gpu_kw(L, x["wq"], x["wk"])).out.clone()
            for _ in range(2)]
    assert torch.equal(outs[0], outs[1])
    G = GEMMA_GLOBAL_LAYER
    B, p = 4, 5000
    kc = device_normal_bf16((B, G.Hkv, p + 1, G.d), 7401, "cuda")
    vc = device_normal_bf16((B, G.Hkv, p + 1, G.d), 7402, "cuda")
    dr = Draw(7403, True)
    q, k, _ = G.draw_tokens(dr, B, 1)
    wq, wk = G.draw_gains(dr)
    tab = table_for(G, p + 64)
    outs = []
    for _ in range(2):
        kd = dev(k)
        outs.append(layer.decode(dev(q), kd, kd, kc, vc, window=0, pos_offset=p, rope_table=tab,
                                 **gpu_kw(G, wq, wk)).out.clone())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("wl", [GEMMA_LOCAL_PREFILL, GEMMA_GLOBAL_PREFILL], ids=["local_T8192", "global_T32768"])
def test_gemma_prefill_full_size(wl):
    """The full-size prefill workloads (one sequence from an empty cache) on sampled rows: the
    first tiles, around the window edge and tile edges, the middle and the last rows."""
    L = wl.layer
    x = wl.draw()
    T = wl.T
    tab = table_for(L, T + 64)
    qd, kd = dev(x["q"]), dev(x["k"])
    vd = kd if L.kv_shared else dev(x["v"])
    bufs = layer.prefill(qd, kd, vd, window=L.window, rope_table=tab, pos_offset=0, **gpu_kw(L, x["wq"], x["wk"]))
    torch.cuda.synchronize()
    rows = np.unique(np.array([0, 1, 31, 32, 63, 64, 65, 1022, 1023, 1024, 1025, 2047, 2048, T // 3, T // 2,
                               T - 65, T - 64, T - 2, T - 1]).clip(0, T - 1))
    got = host(bufs.out[0][torch.from_numpy(rows).cuda()])
    ref = oracle_step(L, x["q"][0], x["k"][0], x["v"][0], LayerKVCache(L.Hkv, L.d, L.window, post_rope=True),
                      x["wq"], x["wk"], rows=rows)
    assert_parity(got, ref, TOL_BF16, wl.name)


@pytest.mark.parametrize("wl", [GEMMA_LOCAL_DECODE, GEMMA_GLOBAL_DECODE], ids=["local_ring1024", "global_ctx32768"])
def test_gemma_decode_full_size(wl):
    """Batched decode at the full shapes (B = 64, new token at position 32767) from a populated
    post-RoPE cache (K drawn at the layer's K-gain scale, V of unit RMS scale), sampled
    sequences against the oracle with the kept tokens as its prior cache."""
    L = wl.layer
    B, d, W = wl.B, L.d, L.window
    p = wl.pos_offset
    cap = wl.cache_cap()
    g = 0.5 * (L.k_gain[0] + L.k_gain[1])
    kc = (device_normal_bf16((B, L.Hkv, cap, d), wl.cache_seed(), "cuda").float() * g).to(torch.bfloat16)
    vc = device_normal_bf16((B, L.Hkv, cap, d), wl.cache_seed() + 1, "cuda")
    x = wl.draw_new_tokens()
    tab = table_for(L, p + 64)
    qd, kd = dev(x["q"]), dev(x["k"])
    vd = kd if L.kv_shared else dev(x["v"])
    kept = p if W == 0 else min(p, W - 1)
    slots = np.arange(p - kept, p) if W == 0 else np.arange(p - kept, p) % W
    sl = torch.from_numpy(slots).cuda()
    samples = [0, 17, B - 1]
    prior = {b: (host(kc[b][:, sl]).transpose(1, 0, 2), host(vc[b][:, sl]).transpose(1, 0, 2)) for b in samples}
    db = layer.decode(qd, kd, vd, kc, vc, window=W, pos_offset=p, rope_table=tab, **gpu_kw(L, x["wq"], x["wk"]))
    torch.cuda.synchronize()
    out = host(db.out)
    for b in samples:
        cache = LayerKVCache.with_prior(prior[b][0], prior[b][1], p, W, post_rope=True)
        ref = oracle_step(L, x["q"][b], x["k"][b], x["v"][b], cache, x["wq"], x["wk"])
        assert_parity(out[b], ref, TOL_BF16, f"{wl.name}, sequence {b}")


@pytest.mark.parametrize("L,window", [(GEMMA_LOCAL_LAYER, 100), (GEMMA_GLOBAL_LAYER, 0)], ids=["d256_W100", "d512"])
def test_gemma_ragged_batch(L, window):
    """A ragged batch of the Gemma-shaped layers: each step gives every sequence its own
    position and token count (0 = it sits the step out), then one ragged decode step; input
    rows past a sequence's count are NaN (never read), output rows past it keep a sentinel
    (never written). Every sequence against the oracle run on its own stream in the same chunks."""
    import dataclasses
    Hq, Hkv = (4, 2) if window else (8, 1)
    L = dataclasses.replace(L, Hq=Hq, Hkv=Hkv, window=window)
    B, d = 3, L.d
    lens = np.array([[150, 37, 90], [70, 130, 0]], dtype=np.int64)
    n_tot = lens.sum(0) + 1
    dr = Draw(7300 + window, True)
    streams = [L.draw_tokens(dr, 1, int(n)) for n in n_tot]
    wq, wk = L.draw_gains(dr)
    cap = window if window else int(n_tot.sum())
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    tab = table_for(L, int(n_tot.sum()) + 64)
    kw = gpu_kw(L, wq, wk)
    pos = np.zeros(B, np.int64)
    got = [[] for _ in range(B)]
    sentinel = 123.0

    def slabs(L_, T):
        out = []
        for i in range(3):
            x = np.full((B, T) + streams[0][i].shape[2:], np.nan, np.float32)
            for b in range(B):
                x[b, :L_[b]] = streams[b][i][0, pos[b]:pos[b] + L_[b]]
            out.append(dev(x))
        if L.kv_shared:  # one tensor for K and V, as the layer's projection gives them
            out[2] = out[1]
        return out

    for Ls in lens:
        T = int(Ls.max())
        maxp = int(pos.max())
        bufs = layer.PrefillBuffers(B, T, Hq, Hkv, d, torch.bfloat16, "cuda", window, maxp)
        bufs.out.fill_(sentinel)
        layer.prefill_ragged(*slabs(Ls, T), window=window, rope_table=tab,
                             seq_pos_offsets=torch.tensor(pos, device="cuda"), max_pos_offset=maxp,
                             seq_lens=torch.tensor(Ls, dtype=torch.int32, device="cuda"), k_cache=kc, v_cache=vc,
                             bufs=bufs, **kw)
        torch.cuda.synchronize()
        out = host(bufs.out)
        for b in range(B):
            assert np.all(out[b, Ls[b]:] == sentinel), f"rows past sequence {b}'s count were written"
            if Ls[b]:
                got[b].append(out[b, :Ls[b]])
        pos += Ls
    one = np.ones(B, np.int64)
    db = layer.decode_ragged(*slabs(one, 1), kc, vc, window=window, seq_pos_offsets=torch.tensor(pos, device="cuda"),
                             max_pos_offset=int(pos.max()), rope_table=tab, **kw)
    torch.cuda.synchronize()
    out = host(db.out)
    for b in range(B):
        got[b].append(out[b])
    for b in range(B):
        chunks = [int(Ls[b]) for Ls in lens if Ls[b]] + [1]
        q, k, v = streams[b]
        cache = LayerKVCache(Hkv, d, window, post_rope=True)
        p = 0
        for i, T in enumerate(chunks):
            ref = oracle_step(L, q[0, p:p + T], k[0, p:p + T], v[0, p:p + T], cache, wq, wk)
            assert_parity(got[b][i], ref, TOL_BF16, f"sequence {b}, call {i} (T={T})")
            p += T
