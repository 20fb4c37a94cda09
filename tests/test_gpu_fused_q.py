"""GPU parity of the fused-Q prefill (plamo_attn_prefill_fused_q): the append writes only the
K/V side and the prefill kernel normalises and rotates the queries itself
(「PLaMo 3アーキテクチャ徹底解析」 §4.3, §4.4, §6.1), against the fp64 oracle.

Bar: |gpu - oracle| <= 2e-2 + 2e-2 |oracle| elementwise (bf16, helpers.TOL_BF16)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import TOL_BF16, assert_parity, oracle_chunks, oracle_prefill
from synthetic import Draw
from synthetic.workloads import GLOBAL_PREFILL, LOCAL_PREFILL, Rope

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


def table(rope: Rope, max_pos: int):
    return swg.make_rope_table(max_pos, swg.RopeParams(rope.theta, rope.yarn_factor, rope.orig_ctx,
                                                       rope.beta_fast, rope.beta_slow))


# Norm offsets: the pages' q/k value 1 on every layer, the YaRN layers included (there the
# amplitude squared, 2.0 - 2.4, sharpens the scores the most).
C_GLOBAL = 1.0


@pytest.mark.parametrize("window,chunks,rope,post_rope,c", [
    (2048, [2500, 300, 1], Rope(1e4), False, 1.0),
    (16, [40, 5, 70], Rope(1e4), False, 1.0),
    (0, [300, 200], Rope(1e6, 64.0), False, C_GLOBAL),
    (0, [130, 77], Rope(1e6, 256.0), True, C_GLOBAL),
    (0, [200, 100], Rope(1e6), False, 1.0),
    (100, [250, 31], Rope(1e4), True, 1.0),
    (64, [200, 90], Rope(1e4), False, None),
], ids=["W2048", "W16", "global_yarn64", "global_yarn256_post", "global_no_yarn", "W100_post", "W64_no_norm"])
def test_fused_q_chunks_match_oracle(window, chunks, rope, post_rope, c):
    """Chunked prefill of B = 2 sequences through the fused path (every chunk after the first
    attends cached keys), every output row against the oracle run on the same stream."""
    norm = c is not None
    B, Hq, Hkv, d = 2, 8, 2, 128
    n = sum(chunks)
    dr = Draw(9100 + window + n + post_rope, True)
    q, k, v = dr.normal((B, n, Hq, d)), dr.normal((B, n, Hkv, d)), dr.normal((B, n, Hkv, d))
    wq, wk = (dr.normal((d,), 0.02), dr.normal((d,), 0.02)) if norm else (None, None)
    cap = window if window else n
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    tab = table(rope, n + 64)
    kw = dict(q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=c) if norm else {}
    got, p = [], 0
    for T in chunks:
        bufs = layer.prefill(dev(q[:, p:p + T]), dev(k[:, p:p + T]), dev(v[:, p:p + T]), window=window,
                             rope_table=tab, k_cache=kc, v_cache=vc, pos_offset=p, cache_post_rope=post_rope,
                             fuse_q=True, **kw)
        torch.cuda.synchronize()
        got.append(host(bufs.out))
        p += T
    ref = oracle_chunks(q, k, v, chunks, window=window, rope=rope, wq=wq, wk=wk, norm_offset=c if norm else 1.0,
                        post_rope=post_rope)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert_parity(g, r, TOL_BF16, f"chunk {i} (T={chunks[i]})")


@pytest.mark.parametrize("wl", [LOCAL_PREFILL, GLOBAL_PREFILL], ids=["local8192", "global32768"])
def test_fused_q_full_size(wl):
    """The full-size prefill workloads through the fused path: sampled rows against the oracle,
    and every row against the unfused path (the same attention on Q' rounded once more)."""
    inp = wl.draw()
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    tab = table(wl.rope, wl.T + 64)
    kw = dict(q_norm_w=dev(inp["wq"]), k_norm_w=dev(inp["wk"]), norm_offset=wl.norm_offset, window=wl.window,
              rope_table=tab)
    fused = layer.prefill(q, k, v, fuse_q=True, **kw)
    plain = layer.prefill(q, k, v, **kw)
    torch.cuda.synchronize()
    rows = np.unique(np.array([0, 1, 63, 64, 127, 128, 2047, 2048, 2049, wl.T // 2, wl.T - 2, wl.T - 1]))
    ref = oracle_prefill(inp["q"], inp["k"], inp["v"], window=wl.window, rope=wl.rope, wq=inp["wq"],
                         wk=inp["wk"], norm_offset=wl.norm_offset, rows=rows)
    assert_parity(host(fused.out[:, rows]), ref, TOL_BF16, f"{wl.name} fused")
    a, b = fused.out.float(), plain.out.float()
    assert torch.all((a - b).abs() <= 2e-2 + 2e-2 * b.abs()).item()


def test_fused_q_ragged_matches_oracle():
    """A ragged batch through the fused path: per-sequence positions and counts; input rows past
    a sequence's count are NaN (never read), output rows past it keep a sentinel (never written)."""
    B, Hq, Hkv, d, window = 3, 8, 2, 128, 64
    steps = [[150, 37, 90], [70, 200, 0]]
    lens = np.array(steps, dtype=np.int64)
    n_tot = lens.sum(0)
    rope = Rope(1e4)
    dr = Draw(9300, True)
    streams = [(dr.normal((1, n, Hq, d)), dr.normal((1, n, Hkv, d)), dr.normal((1, n, Hkv, d))) for n in n_tot]
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    kc = torch.zeros((B, Hkv, window, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    tab = table(rope, int(n_tot.sum()) + 64)
    pos = np.zeros(B, np.int64)
    got = [[] for _ in range(B)]
    sentinel = 123.0

    def slab(i, L, T):
        x = np.full((B, T) + streams[0][i].shape[2:], np.nan, np.float32)
        for b in range(B):
            x[b, :L[b]] = streams[b][i][0, pos[b]:pos[b] + L[b]]
        return dev(x)

    for L in lens:
        T = int(L.max())
        maxp = int(pos.max())
        bufs = layer.PrefillBuffers(B, T, Hq, Hkv, d, torch.bfloat16, "cuda", window, maxp)
        bufs.out.fill_(sentinel)
        layer.prefill_ragged(slab(0, L, T), slab(1, L, T), slab(2, L, T), window=window, rope_table=tab,
                             seq_pos_offsets=torch.tensor(pos, device="cuda"), max_pos_offset=maxp,
                             seq_lens=torch.tensor(L, dtype=torch.int32, device="cuda"), k_cache=kc, v_cache=vc,
                             bufs=bufs, q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0, fuse_q=True)
        torch.cuda.synchronize()
        out = host(bufs.out)
        for b in range(B):
            assert np.all(out[b, L[b]:] == sentinel), f"rows past sequence {b}'s count were written"
            if L[b]:
                got[b].append(out[b, :L[b]])
        pos += L
    for b in range(B):
        chunks = [int(L[b]) for L in lens if L[b]]
        q, k, v = streams[b]
        ref = oracle_chunks(q, k, v, chunks, window=window, rope=rope, wq=wq, wk=wk)
        for i, (g, r) in enumerate(zip(got[b], ref)):
            assert_parity(g, r[0], TOL_BF16, f"sequence {b} chunk {i}")
