"""GPU test of plamo_attn_decode_noalloc, the decode entry point that allocates nothing (its
split-K partials live in the library's static per-GPU scratch): two calls in a row, the
second smaller, each against plamo_attn_decode with a caller workspace on the same inputs
(「PLaMo 3アーキテクチャ徹底解析」 §4.4, §4.5: one decode step over the cache)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import TOL_BF16, assert_parity
from synthetic import Draw
from synthetic.workloads import device_normal_bf16

pytestmark = pytest.mark.gpu

swg = pytest.importorskip("sliding_window_global_amd")
from sliding_window_global_amd import layer  # noqa: E402


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


def _case(B, Hq, Hkv, window, pos_offset, theta, yarn, seed):
    """Caches holding the kept tokens, the new token appended; returns what both decode calls need."""
    d = 128
    cap = window if window else pos_offset + 1
    kc = device_normal_bf16((B, Hkv, cap, d), seed, "cuda")
    vc = device_normal_bf16((B, Hkv, cap, d), seed + 1, "cuda")
    dr = Draw(seed + 2, True)
    q, k, v = dr.normal((B, 1, Hq, d)), dr.normal((B, 1, Hkv, d)), dr.normal((B, 1, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    tab = swg.make_rope_table(pos_offset + 64, swg.RopeParams(theta, yarn))
    bufs = layer.DecodeBuffers(B, Hq, Hkv, d, window, pos_offset)
    swg.plamo_kv_append(dev(q), dev(k), dev(v), bufs.q_rot, window=window, pos_offset=pos_offset, rope_table=tab,
                        q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0, k_cache=kc, v_cache=vc)
    need = swg.plamo_attn_decode_workspace_bytes(B, Hq, Hkv, window, pos_offset)
    assert 0 < need <= swg.PLAMO_DECODE_SCRATCH_BYTES  # the case exercises the scratch
    return dict(q_rot=bufs.q_rot, kc=kc, vc=vc, tab=tab, window=window, pos_offset=pos_offset, ws=bufs.workspace)


def _both(c):
    ref = torch.empty(c["q_rot"].shape, dtype=torch.bfloat16, device="cuda")
    got = torch.full_like(ref, float("nan"))
    swg.plamo_attn_decode(c["q_rot"], c["kc"], c["vc"], ref, c["ws"], window=c["window"],
                          pos_offset=c["pos_offset"], rope_table=c["tab"])
    swg.plamo_attn_decode_noalloc(c["q_rot"], c["kc"], c["vc"], got, window=c["window"],
                                  pos_offset=c["pos_offset"], rope_table=c["tab"])
    torch.cuda.synchronize()
    return got, ref


def test_decode_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = _case(2, 16, 2, 0, 8191, 1e6, 64.0, 8801)      # 32 key ranges per (sequence, KV head)
    small = _case(1, 8, 1, 2048, 3000, 1e4, 0.0, 8802)   # ring, 8 key ranges
    for c in (big, small):
        got, ref = _both(c)
        ref_h = ref.float().cpu().numpy().astype(np.float64)
        assert_parity(got.float().cpu().numpy(), ref_h, TOL_BF16, "noalloc vs workspace decode")
        assert torch.equal(got, ref), "same kernels and plan: the outputs are bit-identical"
