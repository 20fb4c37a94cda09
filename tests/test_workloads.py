"""The work counts behind every reported throughput, checked on the CPU against the oracle's
own mask and byte accounting (「PLaMo 3アーキテクチャ徹底解析」 §2.3, §5.1, §5.2), and the
seeded input recipes (same seed, same bytes)."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import allowed, attended_keys_total, kv_bytes
from synthetic import Draw, bf16_round
from synthetic.workloads import (BATCHED_DECODE, GEMMA_GLOBAL_DECODE, GEMMA_GLOBAL_PREFILL, GEMMA_LOCAL_DECODE,
                                 GEMMA_LOCAL_PREFILL, GLOBAL_PREFILL, LOCAL_PREFILL, PERIOD_DECODE, TINY_SWA_FP32,
                                 GemmaPrefill, PrefillWorkload, Rope, ragged_positions)


@pytest.mark.parametrize("T,W", [(1, 0), (7, 0), (9, 3), (9, 9), (9, 20), (40, 1), (130, 64)])
def test_attended_pairs_match_the_mask(T, W):
    """Pairs per head = the number of allowed (query, key) entries of the oracle's mask."""
    wl = PrefillWorkload("t", 1, T, 2, 1, 8, W, Rope(1e4), None, False, 0)
    pos = np.arange(T)
    assert wl.attended_pairs_per_head() == int(allowed(pos, pos, W).sum())
    assert wl.flops() == 4.0 * 8 * 2 * wl.attended_pairs_per_head()


def test_full_size_prefill_counts():
    # closed forms: local sum_t min(t + 1, W); global T (T + 1) / 2
    T, W = LOCAL_PREFILL.T, LOCAL_PREFILL.window
    assert LOCAL_PREFILL.attended_pairs_per_head() == sum(min(t + 1, W) for t in range(T)) == 14_681_088
    assert GLOBAL_PREFILL.attended_pairs_per_head() == 32768 * 32769 // 2 == 536_887_296
    assert TINY_SWA_FP32.attended_pairs_per_head() == 57_408
    assert LOCAL_PREFILL.flops() == pytest.approx(4.811e11, rel=1e-3)
    assert GLOBAL_PREFILL.flops() == pytest.approx(1.759e13, rel=1e-3)
    # the Gemma-shaped layers: the same counts with their head dims and heads
    g = GEMMA_LOCAL_PREFILL
    assert g.attended_pairs_per_head() == sum(min(t + 1, 1024) for t in range(g.T))
    assert g.flops() == 4.0 * 256 * 32 * g.attended_pairs_per_head()
    assert GEMMA_GLOBAL_PREFILL.flops() == 4.0 * 512 * 32 * 32768 * 32769 // 2


def test_decode_bytes_match_the_oracle_accounting():
    """KV bytes of one decode = the oracle's 2 * 2 B * B * Hkv * d * keys (pages §2.3)."""
    wl = BATCHED_DECODE
    for ly, keys in zip(wl.layers, (2048, 32768)):
        assert wl.keys_attended(ly) == keys
        assert wl.kv_bytes(ly) == kv_bytes(wl.B, wl.Hkv, wl.d, keys)
    assert wl.kv_bytes(wl.layers[0]) == 536_870_912 and wl.kv_bytes(wl.layers[1]) == 8_589_934_592
    # the period's first step (8 layers, B = 8) reads as much as one sequence's token through
    # the 64 layers at N = 131072: the pages' 4544 MiB row (8 global + 56 local layers)
    p = PERIOD_DECODE
    per_step = sum(p.kv_bytes(ly) for ly in p.layers)
    assert per_step == kv_bytes(p.B, p.Hkv, p.d, attended_keys_total(131072, 2048, 1, 7))
    assert per_step == kv_bytes(1, p.Hkv, p.d, attended_keys_total(131072, 2048, 8, 56)) == 4544 * 2 ** 20
    for g, keys in ((GEMMA_LOCAL_DECODE, 1024), (GEMMA_GLOBAL_DECODE, 32768)):
        assert g.keys_attended() == keys
        assert g.kv_bytes() == kv_bytes(g.B, g.layer.Hkv, g.layer.d, keys)


def test_inputs_are_seeded_and_bf16_exact():
    a, b = Draw(123, True), Draw(123, True)
    x, y = a.normal((3, 5)), b.normal((3, 5))
    assert np.array_equal(x, y) and np.array_equal(bf16_round(x), x)
    assert a.uniform(0.95, 1.05) == b.uniform(0.95, 1.05)
    small = GemmaPrefill("s", GEMMA_GLOBAL_PREFILL.layer, 1, 5, 7)
    d1, d2 = small.draw(), small.draw()
    assert all(np.array_equal(d1[k], d2[k]) for k in d1)
    assert d1["v"] is d1["k"]  # the global layer's V is its K projection
    # gains: a level in the layer's range plus per-component noise (bf16-exact, not constant)
    for w, (lo, hi) in ((d1["wq"], small.layer.q_gain), (d1["wk"], small.layer.k_gain)):
        assert np.array_equal(bf16_round(w), w) and len(np.unique(w)) > 1
        assert lo - 0.1 <= float(np.mean(w)) <= hi + 0.1


def test_ragged_positions():
    p = ragged_positions(64, 32767, 5)
    assert p.dtype == np.int64 and p.shape == (64,) and p.max() == 32767 and p.min() >= 0
    assert np.array_equal(p, ragged_positions(64, 32767, 5))
