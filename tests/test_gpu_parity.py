"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Bar (written here, applied elementwise): |gpu - oracle| <= atol + rtol*|oracle| with
atol = rtol = 2e-2 for bf16 and 1e-4 for fp32 (helpers.TOL_*). Inputs are the seeded
synthetic workloads; full-size workloads are checked on sampled rows the oracle
computes one by one, and everywhere through size-independent closed forms."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from helpers import (TOL_BF16, TOL_F16, TOL_F32, assert_parity, kept_slots, oracle_chunks, oracle_decode_one,
                     oracle_prefill, window_mean_closed_form, untile_k_rot, untile_v_t)
from oracle import LayerKVCache, apply_rope, attention_layer_step, offset_rms_norm, rope_frequencies
from synthetic import Draw
from synthetic.workloads import (BATCHED_DECODE, GLOBAL_PREFILL, LOCAL_PREFILL, PERIOD_DECODE,
                                 TINY_SWA_FP32, Rope, device_normal_bf16)

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


def dev(x, bf16=True):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


_TABLES = {}


def rope_table(rope: Rope, max_pos: int):
    key = (rope, max_pos)
    if key not in _TABLES:
        _TABLES[key] = swg.make_rope_table(max_pos, swg.RopeParams(rope.theta, rope.yarn_factor,
                                                                    rope.orig_ctx, rope.beta_fast,
                                                                    rope.beta_slow))
    return _TABLES[key]


# ----------------------------------------------------------------------------
# rope table and the fused append
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("rope", [Rope(1e4), Rope(1e6, 64.0), Rope(1e6, 256.0)], ids=["local", "yarn64", "yarn256"])
def test_rope_table_factors(rope):
    """Coarse x fine product equals amp * exp(i p w_j) from the oracle's frequencies."""
    max_pos = 131200
    tab = host(rope_table(rope, max_pos)).reshape(-1, 64, 2)
    omega, amp = rope_frequencies(128, rope.theta, rope.yarn_factor)
    pos = np.array([0, 1, 63, 64, 65, 2047, 2048, 4095, 32767, 65536 + 17, 131071, 131199])
    f = tab[pos & 63]
    c = tab[64 + (pos >> 6)]
    zr = c[..., 0] * f[..., 0] - c[..., 1] * f[..., 1]
    zi = c[..., 0] * f[..., 1] + c[..., 1] * f[..., 0]
    ang = pos[:, None] * omega[None, :]
    assert np.max(np.abs(zr - amp * np.cos(ang))) < 2e-6 * amp
    assert np.max(np.abs(zi - amp * np.sin(ang))) < 2e-6 * amp


@pytest.mark.parametrize("window,pos_offset,T", [(0, 0, 200), (2048, 0, 300), (2048, 2046, 1),
                                                 (2048, 2047, 1), (2048, 2048, 1), (0, 32767, 1),
                                                 (16, 5, 40), (16, 100, 3), (2048, 1000, 1200),
                                                 (0, 77, 130)])
def test_kv_append_intermediates(window, pos_offset, T):
    """Q' (normalised, rotated at kept + t), the cache contents (pre-RoPE K, raw V, ring slot
    n mod W, only the last W of a chunk) and the prefill operands K' and V^T of all kept + T
    keys: the kept cached keys rotated at 0 .. kept-1, then the chunk, then zero padding."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    dr = Draw(1234 + pos_offset + T, True)
    q, k, v = dr.normal((B, T, Hq, d)), dr.normal((B, T, Hkv, d)), dr.normal((B, T, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    rope = Rope(1e6, 64.0) if window == 0 else Rope(1e4)
    c = 1.0
    cap = window if window else pos_offset + T
    kept = pos_offset if window == 0 else min(pos_offset, window - 1)
    prior = kept_slots(pos_offset, window)  # slots of the kept tokens, in token order
    prior_k, prior_v = dr.normal((B, kept, Hkv, d)), dr.normal((B, kept, Hkv, d))
    kc = torch.full((B, Hkv, cap, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    if kept:
        idx = torch.from_numpy(prior).cuda()
        kc[:, :, idx] = dev(prior_k).transpose(1, 2)
        vc[:, :, idx] = dev(prior_v).transpose(1, 2)
    q_out = torch.empty((B, T, Hq, d), dtype=torch.float16, device="cuda")
    k_shape, v_shape = swg.prefill_operand_shapes(B, T, Hkv, d, torch.bfloat16, window, pos_offset)
    k_rot = torch.full(k_shape, float("nan"), dtype=torch.float16, device="cuda")
    v_t = torch.full(v_shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    swg.plamo_kv_append(dev(q), dev(k), dev(v), q_out, window=window, pos_offset=pos_offset,
                        rope_table=rope_table(rope, 40000), q_norm_w=dev(wq), k_norm_w=dev(wk),
                        norm_offset=c, k_rot_out=k_rot, v_t_out=v_t, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    omega, amp = rope_frequencies(d, rope.theta, rope.yarn_factor)
    pos = kept + np.arange(T)
    S = kept + T
    qn = offset_rms_norm(q, wq, c)
    kn = offset_rms_norm(k, wk, c)
    q_ref = np.stack([apply_rope(qn[b], pos, omega, amp) for b in range(B)])
    # the score operands are IEEE halves rounded once from fp32: within the half bar
    assert_parity(host(q_out), q_ref, TOL_F16, "q_out")
    k_ref = np.stack([apply_rope(kn[b], pos, omega, amp) for b in range(B)])
    kr = untile_k_rot(host(k_rot))
    assert_parity(kr[:, :, kept:S].transpose(0, 2, 1, 3), k_ref, TOL_F16, "k_rot (chunk)")
    if kept:
        kp_ref = np.stack([apply_rope(prior_k[b], np.arange(kept), omega, amp) for b in range(B)])
        assert_parity(kr[:, :, :kept].transpose(0, 2, 1, 3), kp_ref, TOL_F16, "k_rot (cached keys)")
    assert np.all(kr[:, :, S:] == 0)
    vt = untile_v_t(host(v_t))
    assert np.array_equal(vt[..., kept:S].transpose(0, 3, 1, 2), v)  # exact copies
    assert np.array_equal(vt[..., :kept].transpose(0, 3, 1, 2), prior_v)
    assert np.all(vt[..., S:] == 0)
    kch, vch = host(kc), host(vc)
    written = np.arange(T) if window == 0 else np.arange(max(0, T - window), T)
    for t in written:
        n = pos_offset + t
        slot = n if window == 0 else n % window
        assert_parity(kch[:, :, slot], kn[:, t], TOL_BF16, f"k_cache slot {slot}")
        assert np.array_equal(vch[:, :, slot], v[:, t])
    touched = {(pos_offset + t) if window == 0 else (pos_offset + t) % window for t in written}
    untouched = [s for s in range(cap) if s not in touched and s not in set(prior.tolist())]
    assert np.all(np.isnan(kch[:, :, untouched])) and np.all(np.isnan(vch[:, :, untouched]))


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

def _run_prefill(inp, window, rope, norm_offset, bf16):
    B, T, Hq, d = inp["q"].shape
    tab = rope_table(rope, max(T, 64))
    kw = {}
    if inp.get("wq") is not None:
        kw = dict(q_norm_w=dev(inp["wq"], bf16), k_norm_w=dev(inp["wk"], bf16), norm_offset=norm_offset)
    bufs = layer.prefill(dev(inp["q"], bf16), dev(inp["k"], bf16), dev(inp["v"], bf16), window=window,
                         rope_table=tab, **kw)
    torch.cuda.synchronize()
    return bufs


def test_prefill_tiny_fp32():
    """The tiny fp32 sliding-window workload (T=512, Hq=8, Hkv=2, W=128), full oracle, 1e-4."""
    wl = TINY_SWA_FP32
    inp = wl.draw()
    bufs = _run_prefill(inp, wl.window, wl.rope, None, bf16=False)
    ref = oracle_prefill(inp["q"], inp["k"], inp["v"], window=wl.window, rope=wl.rope)
    assert_parity(host(bufs.out), ref, TOL_F32, wl.name)


@pytest.mark.parametrize("B,T,Hq,Hkv,W", [
    (1, 1, 8, 2, 0), (1, 5, 8, 2, 3), (2, 64, 4, 4, 0), (1, 130, 16, 1, 7), (2, 300, 8, 2, 128),
    (1, 1000, 8, 1, 200), (1, 777, 4, 2, 4096), (1, 513, 8, 8, 1), (1, 640, 16, 2, 64),
    (3, 257, 2, 1, 129)])
def test_prefill_bf16_small(B, T, Hq, Hkv, W):
    """Several tiles, ragged tails, window 1 (self only), W > T, G = 1..16; full oracle."""
    d = 128
    dr = Draw(777 + 31 * T + W, True)
    inp = dict(q=dr.normal((B, T, Hq, d)), k=dr.normal((B, T, Hkv, d)), v=dr.normal((B, T, Hkv, d)),
               wq=dr.normal((d,), 0.02), wk=dr.normal((d,), 0.02))
    rope = Rope(1e4) if W else Rope(1e6, 256.0)
    bufs = _run_prefill(inp, W, rope, 1.0, bf16=True)
    ref = oracle_prefill(inp["q"], inp["k"], inp["v"], window=W, rope=rope, wq=inp["wq"], wk=inp["wk"],
                         norm_offset=1.0)
    assert_parity(host(bufs.out), ref, TOL_BF16, f"B{B} T{T} Hq{Hq} Hkv{Hkv} W{W}")


@pytest.mark.parametrize("fuse_q", [False, True], ids=["unfused", "fused_q"])
def test_prefill_writes_exactly_its_output(fuse_q):
    """The output sits at the front of a NaN-filled buffer 1024 elements longer: every element
    of it written (ragged last 128-row block: T = 300), nothing past it (the epilogue stages
    each wave's rows in LDS and stores whole rows), every row against the oracle."""
    B, T, Hq, Hkv, W, d = 2, 300, 8, 2, 128, 128
    dr = Draw(31337, True)
    inp = dict(q=dr.normal((B, T, Hq, d)), k=dr.normal((B, T, Hkv, d)), v=dr.normal((B, T, Hkv, d)),
               wq=dr.normal((d,), 0.02), wk=dr.normal((d,), 0.02))
    rope = Rope(1e4)
    bufs = layer.PrefillBuffers(B, T, Hq, Hkv, d, torch.bfloat16, "cuda", W, 0)
    n = B * T * Hq * d
    canary = torch.full((n + 1024,), float("nan"), dtype=torch.bfloat16, device="cuda")
    bufs.out = canary[:n].view(B, T, Hq, d)
    layer.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), window=W, rope_table=rope_table(rope, T + 64),
                  q_norm_w=dev(inp["wq"]), k_norm_w=dev(inp["wk"]), norm_offset=1.0, bufs=bufs, fuse_q=fuse_q)
    torch.cuda.synchronize()
    assert bool(torch.isnan(canary[n:]).all()), "write past the output"
    assert not bool(torch.isnan(bufs.out).any()), "output element left unwritten"
    ref = oracle_prefill(inp["q"], inp["k"], inp["v"], window=W, rope=rope, wq=inp["wq"], wk=inp["wk"],
                         norm_offset=1.0)
    assert_parity(host(bufs.out), ref, TOL_BF16, f"canaried output fuse_q={fuse_q}")


def _sample_rows(T, n_mid, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, 128, 2047, 2048, 2049, T // 2, T - 129, T - 128, T - 2, T - 1]
    rows = set(r for r in fixed if 0 <= r < T)
    rows.update(rng.integers(0, T, n_mid).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("norm_offset", [0.2, 1.0], ids=["c0.2", "c1"])
def test_prefill_local_full_size(norm_offset):
    """Local layer at its real shape (T=8192, Hq=64, Hkv=8, W=2048): sampled rows vs the
    oracle, with the workload's offset 0.2 and the pages' q/k-norm offset 1."""
    wl = LOCAL_PREFILL
    inp = wl.draw()
    bufs = _run_prefill(inp, wl.window, wl.rope, norm_offset, bf16=True)
    rows = _sample_rows(wl.T, 10, 5)
    ref = oracle_prefill(inp["q"], inp["k"], inp["v"], window=wl.window, rope=wl.rope, wq=inp["wq"],
                         wk=inp["wk"], norm_offset=norm_offset, rows=rows)
    assert_parity(host(bufs.out[:, rows]), ref, TOL_BF16, f"{wl.name} c={norm_offset}")


@pytest.mark.parametrize("window,T", [(2048, 8192), (0, 32768)], ids=["local8192", "global32768"])
def test_prefill_uniform_closed_form_full_size(window, T):
    """Every row at full size: gain c + w = 0 zeroes Q, so each output is the mean of V over
    the window (prefix sums). Exercises every tile, the window edge and the tile skipping."""
    wl = LOCAL_PREFILL if window else GLOBAL_PREFILL
    dr = Draw(4242 + T, True)
    B, Hq, Hkv, d = 1, 64, 8, 128
    q = dr.normal((B, T, Hq, d))
    k = dr.normal((B, T, Hkv, d))
    v = dr.normal((B, T, Hkv, d))
    c = 1.0
    inp = dict(q=q, k=k, v=v, wq=np.full(d, -c, np.float32), wk=dr.normal((d,), 0.02))
    bufs = _run_prefill(inp, window, wl.rope, c, bf16=True)
    out = host(bufs.out)[0]
    mean = window_mean_closed_form(v[0], window)  # [T, Hkv, d]
    ref = np.repeat(mean, Hq // Hkv, axis=1)
    assert_parity(out, ref, TOL_BF16, f"closed form W={window}")


@pytest.mark.parametrize("yarn", [64.0, 256.0])
def test_prefill_global_full_size(yarn):
    """Global layer at its real shape (T=32768, causal, YaRN, theta 1e6): sampled rows."""
    wl = GLOBAL_PREFILL
    inp = wl.draw()
    rope = Rope(1e6, yarn)
    bufs = _run_prefill(inp, 0, rope, wl.norm_offset, bf16=True)
    rows = _sample_rows(wl.T, 4, 9)
    ref = oracle_prefill(inp["q"], inp["k"], inp["v"], window=0, rope=rope, wq=inp["wq"], wk=inp["wk"],
                         norm_offset=wl.norm_offset, rows=rows)
    assert_parity(host(bufs.out[:, rows]), ref, TOL_BF16, f"global s={yarn}")


def test_prefill_global_full_size_pages_setting():
    """The global layer at its real shape with the settings of 「PLaMo 3アーキテクチャ徹底解析」
    (§3.2 table: q/k-norm offset 1; §6.3: YaRN s = 256 over L0 = 4096; §6.2: base 1e6), where the YaRN
    amplitude squared (2.42) makes the scores the sharpest: the first 64 rows (few keys, the
    largest weights), tile edges, the middle and the last rows, through both the unfused path
    (Q' from the append) and the fused-Q path (Q normalised and rotated in the kernel)."""
    wl = GLOBAL_PREFILL
    inp = wl.draw()
    rope, c = Rope(1e6, 256.0), 1.0
    T = wl.T
    rows = np.unique(np.concatenate([np.arange(64), _sample_rows(T, 6, 11)]))
    ref = oracle_prefill(inp["q"], inp["k"], inp["v"], window=0, rope=rope, wq=inp["wq"], wk=inp["wk"],
                         norm_offset=c, rows=rows)
    tab = rope_table(rope, T + 64)
    args = (dev(inp["q"]), dev(inp["k"]), dev(inp["v"]))
    kw = dict(window=0, rope_table=tab, q_norm_w=dev(inp["wq"]), k_norm_w=dev(inp["wk"]), norm_offset=c)
    sel = torch.from_numpy(rows).cuda()
    for fuse_q in (False, True):
        out = layer.prefill(*args, fuse_q=fuse_q, **kw).out
        torch.cuda.synchronize()
        assert_parity(host(out[:, sel]), ref, TOL_BF16, f"global T={T} c=1 s=256 fuse_q={fuse_q}")
        del out


@pytest.mark.parametrize("window,pos_offset,T,d", [(0, 0, 300, 128), (0, 100, 200, 128), (64, 500, 130, 128),
                                                   (2048, 0, 777, 128), (100, 40, 150, 256)])
def test_prefill_pack_caller_operands(window, pos_offset, T, d):
    """plamo_prefill_pack + plamo_attn_prefill on keys and queries the caller rotated itself
    (here: the oracle's normalised and rotated K' and Q' of every attended key and query,
    rounded to bf16 / fp16): step 4 alone against the oracle's attention on those operands,
    and the packed layouts against a host re-tiling."""
    from oracle import gqa_attention
    B, Hq, Hkv = 2, 8, 2
    kept = pos_offset if window == 0 else min(pos_offset, window - 1)
    S = kept + T
    dr = Draw(8800 + S + window + d, True)
    k_rot = dr.normal((B, S, Hkv, d))            # caller's K' (bf16-exact values)
    v = dr.normal((B, S, Hkv, d))
    q_rot = dr.normal((B, T, Hq, d)).astype(np.float16).astype(np.float32)  # caller's Q' (fp16)
    scale = 1.0 / math.sqrt(d)
    k_shape, v_shape = swg.prefill_operand_shapes(B, T, Hkv, d, torch.bfloat16, window, pos_offset)
    k_out = torch.full(k_shape, float("nan"), dtype=torch.float16, device="cuda")
    v_out = torch.full(v_shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    swg.plamo_prefill_pack(dev(k_rot), dev(v), k_out, v_out)
    out = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    swg.plamo_attn_prefill(torch.from_numpy(q_rot).to(torch.float16).cuda(), k_out, v_out, out, window=window,
                           pos_offset=pos_offset, softmax_scale=scale)
    torch.cuda.synchronize()
    Sp = k_shape[2] * 64
    kr = untile_k_rot(host(k_out))
    k_half = k_rot.astype(np.float16).astype(np.float64)  # bf16 -> half: exact except below 2^-14
    assert np.array_equal(kr[:, :, :S].transpose(0, 2, 1, 3), k_half) and np.all(kr[:, :, S:] == 0)
    vt = untile_v_t(host(v_out))
    assert np.array_equal(vt[..., :S].transpose(0, 3, 1, 2), v) and np.all(vt[..., S:] == 0) and vt.shape[-1] == Sp
    got = host(out)
    for b in range(B):
        ref = gqa_attention(q_rot[b], k_half[b], v[b], np.arange(kept, S), np.arange(S), window, scale)
        assert_parity(got[b], ref, TOL_BF16, f"pack + prefill b={b} W={window} p={pos_offset} T={T} d={d}")


def test_prefill_deterministic():
    wl = LOCAL_PREFILL
    inp = wl.draw()
    a = _run_prefill(inp, wl.window, wl.rope, 0.2, True).out.clone()
    b = _run_prefill(inp, wl.window, wl.rope, 0.2, True).out.clone()
    assert torch.equal(a, b)


def test_prefill_empty_is_noop():
    q = torch.empty((1, 0, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    tab = rope_table(Rope(1e4), 64)
    swg.plamo_kv_append(q, k, k, q.to(swg.score_dtype(q.dtype)), window=16, pos_offset=0, rope_table=tab)
    lib = swg._lib.load()
    assert lib.plamo_attn_prefill(1, None, None, None, None, 1, 0, 8, 2, 128, 16, 0, 0.1, None) == 0


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def _decode_case(B, Hq, Hkv, window, pos_offset, rope, seed, check_b, poison_future=True, post_rope=False,
                 fused=False):
    d = 128
    cap = window if window else pos_offset + 1
    kc = device_normal_bf16((B, Hkv, cap, d), seed, "cuda")
    vc = device_normal_bf16((B, Hkv, cap, d), seed + 1, "cuda")
    slots = kept_slots(pos_offset, window)
    if poison_future:  # slots that hold no kept token must never be read
        live = np.zeros(cap, dtype=bool)
        live[slots] = True
        dead = torch.from_numpy(np.nonzero(~live)[0]).cuda()
        kc[:, :, dead] = float("nan")
        vc[:, :, dead] = float("nan")
    prior_k = {b: host(kc[b][:, torch.from_numpy(slots).cuda()]).transpose(1, 0, 2) for b in check_b}
    prior_v = {b: host(vc[b][:, torch.from_numpy(slots).cuda()]).transpose(1, 0, 2) for b in check_b}
    dr = Draw(seed + 7, True)
    q, k, v = dr.normal((B, 1, Hq, d)), dr.normal((B, 1, Hkv, d)), dr.normal((B, 1, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    tab = rope_table(rope, max(pos_offset + 2, 64))
    bufs = layer.decode(dev(q), dev(k), dev(v), kc, vc, window=window, pos_offset=pos_offset,
                        rope_table=tab, q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0,
                        cache_post_rope=post_rope, fused=fused)
    torch.cuda.synchronize()
    out = host(bufs.out)
    if fused:  # the counters of the merge are back at zero
        tickets = swg.plamo_decode_step_workspace_bytes(B, Hq, Hkv, window, pos_offset) > 0
        assert not tickets or torch.all(bufs.step_workspace.view(torch.int32)[:B * Hkv] == 0)
    for b in check_b:
        ref = oracle_decode_one(q[b], k[b], v[b], prior_k[b], prior_v[b], pos_offset, window=window,
                                rope=rope, wq=wq, wk=wk, post_rope=post_rope)
        assert_parity(out[b], ref, TOL_BF16, f"decode b={b} W={window} p={pos_offset}")
    return bufs


@pytest.mark.parametrize("window,pos_offset", [(2048, 0), (2048, 1), (2048, 100), (2048, 2046),
                                               (2048, 2047), (2048, 2048), (2048, 32767),
                                               (2048, 32767 + 1000), (0, 0), (0, 63), (0, 64),
                                               (0, 5000), (16, 3), (16, 40), (1, 0), (1, 50),
                                               (2, 7), (2, 8)])
def test_decode_small_batch(window, pos_offset):
    """Ring fill-up and wrap, contiguous growth, tile edges; dead slots hold NaN."""
    rope = Rope(1e4) if window else Rope(1e6, 64.0)
    _decode_case(3, 16, 2, window, pos_offset, rope, 100 + pos_offset + window, check_b=[0, 1, 2])


@pytest.mark.parametrize("window,pos_offset,post_rope", [
    (2048, 0, False), (2048, 100, False), (2048, 2047, False), (2048, 32767 + 1000, False), (0, 0, False),
    (0, 63, False), (0, 64, False), (0, 5000, False), (16, 40, False), (1, 50, False), (2, 8, False),
    (2048, 5000, True), (0, 5000, True), (16, 40, True)])
def test_decode_step_one_launch(window, pos_offset, post_rope):
    """plamo_decode_step (the append's work for the new token, attention and the merge of the
    key ranges in one launch): ring fill-up and wrap, contiguous growth, tile edges, both
    cache orders; dead slots hold NaN, also the slot the new token takes."""
    rope = Rope(1e4) if window else Rope(1e6, 64.0)
    _decode_case(3, 16, 2, window, pos_offset, rope, 500 + pos_offset + window, check_b=[0, 1, 2],
                 post_rope=post_rope, fused=True)


@pytest.mark.parametrize("layer_idx", [0, 1], ids=["local_ring2048", "global32768"])
def test_decode_step_one_launch_full_size(layer_idx):
    """The one-launch step at the batched-decode shape (B = 64) and at the period's (B = 8,
    131071 kept global tokens: eight key ranges merged by ticket)."""
    wl = BATCHED_DECODE
    ly = wl.layers[layer_idx]
    _decode_case(wl.B, wl.Hq, wl.Hkv, ly.window, wl.pos_offset, ly.rope, wl.cache_seed(layer_idx),
                 check_b=[0, 31, 63], poison_future=False, fused=True)
    wl = PERIOD_DECODE
    li = 7 if layer_idx else 0
    ly = wl.layers[li]
    _decode_case(wl.B, wl.Hq, wl.Hkv, ly.window, wl.pos_offset, ly.rope, wl.cache_seed(li),
                 check_b=[0, 7], poison_future=False, fused=True)


@pytest.mark.parametrize("G", [1, 4, 16])
def test_decode_group_sizes(G):
    _decode_case(2, 2 * G, 2, 2048, 3000, Rope(1e4), 900 + G, check_b=[0, 1])


@pytest.mark.parametrize("layer_idx", [0, 1], ids=["local_ring2048", "global32768"])
def test_decode_batched_full_size(layer_idx):
    """Batched decode at its real shape: B=64, Hq=64, Hkv=8, local ring (2047 kept + 1) and
    global cache (32767 kept + 1); sampled sequences vs the oracle."""
    wl = BATCHED_DECODE
    ly = wl.layers[layer_idx]
    _decode_case(wl.B, wl.Hq, wl.Hkv, ly.window, wl.pos_offset, ly.rope, wl.cache_seed(layer_idx),
                 check_b=[0, 31, 63], poison_future=False)


@pytest.mark.parametrize("fused", [False, True], ids=["split", "one_launch"])
def test_decode_global_full_size_pages_setting(fused):
    """The global decode at its batched shape (B = 64, 32767 kept + 1 keys) with the settings of
    「PLaMo 3アーキテクチャ徹底解析」 (§3.2 table: q/k-norm offset 1; §6.3: YaRN s = 256 over
    L0 = 4096; §6.2: base 1e6), where the YaRN amplitude squared (2.42) makes the scores the
    sharpest: sampled sequences, through plamo_attn_decode and through the one-launch step."""
    wl = BATCHED_DECODE
    ly = wl.layers[1]
    _decode_case(wl.B, wl.Hq, wl.Hkv, ly.window, wl.pos_offset, Rope(1e6, 256.0), wl.cache_seed(1),
                 check_b=[0, 31, 63], poison_future=False, fused=fused)


@pytest.mark.parametrize("pos_offset", [0, 63, 64, 5000])
def test_decode_small_batch_yarn256(pos_offset):
    """Global decode at YaRN s = 256 and norm offset 1 on contiguous growth and tile edges
    (dead slots NaN), split path and one-launch step."""
    for fused in (False, True):
        _decode_case(3, 16, 2, 0, pos_offset, Rope(1e6, 256.0), 700 + pos_offset, check_b=[0, 1, 2], fused=fused)


def test_decode_batched_full_size_post_rope():
    """The global batched-decode shape with a post-RoPE cache (the prior cache read as already
    rotated K, the new token rotated at its absolute position): sampled sequences."""
    wl = BATCHED_DECODE
    ly = wl.layers[1]
    _decode_case(wl.B, wl.Hq, wl.Hkv, ly.window, wl.pos_offset, ly.rope, wl.cache_seed(1),
                 check_b=[0, 63], poison_future=False, post_rope=True)


@pytest.mark.parametrize("window,pos_offset", [(2048, 100), (2048, 5000), (0, 5000), (16, 40)])
def test_decode_small_batch_post_rope(window, pos_offset):
    """Post-RoPE cache decode on ring fill-up, wrap and contiguous caches; dead slots NaN."""
    rope = Rope(1e4) if window else Rope(1e6, 64.0)
    _decode_case(3, 16, 2, window, pos_offset, rope, 300 + pos_offset + window, check_b=[0, 1, 2], post_rope=True)


def test_decode_period_long_context_step():
    """One step of the 8-layer period at B=8 with 131071 kept global tokens: the global
    layer and one local layer, sampled sequences."""
    wl = PERIOD_DECODE
    for li in (0, 7):
        ly = wl.layers[li]
        _decode_case(wl.B, wl.Hq, wl.Hkv, ly.window, wl.pos_offset, ly.rope, wl.cache_seed(li),
                     check_b=[0, 7], poison_future=False)


@pytest.mark.parametrize("li,fused", [(0, False), (7, False), (0, True), (7, True)],
                         ids=["local_ring2048", "global131072", "local_ring2048_one_launch", "global131072_one_launch"])
def test_decode_period_128_steps(li, fused):
    """The 8-layer period's 128 consecutive decode steps (append + decode per step) on one
    local and the global layer at B = 8 from 131071 kept tokens; steps 0, 63 and 127 of two
    sequences against the oracle run on the same token stream (its cache takes every step's
    normalised K and V, attention is evaluated at the checked steps)."""
    wl = PERIOD_DECODE
    ly = wl.layers[li]
    B, Hq, Hkv, d, W = wl.B, wl.Hq, wl.Hkv, wl.d, ly.window
    p0, steps, c = wl.pos_offset, wl.steps, wl.norm_offset
    cap = wl.cache_cap(ly)
    kc = device_normal_bf16((B, Hkv, cap, d), wl.cache_seed(li), "cuda")
    vc = device_normal_bf16((B, Hkv, cap, d), wl.cache_seed(li) + 1, "cuda")
    check_b, check_k = [0, 5], (0, 63, 127)
    sl = torch.from_numpy(kept_slots(p0, W)).cuda()
    caches = {b: LayerKVCache.with_prior(host(kc[b][:, sl]).transpose(1, 0, 2), host(vc[b][:, sl]).transpose(1, 0, 2),
                                         p0, W) for b in check_b}
    tab = rope_table(ly.rope, p0 + steps + 64)
    omega_kw = dict(theta=ly.rope.theta, yarn_factor=ly.rope.yarn_factor, orig_ctx=ly.rope.orig_ctx,
                    beta_fast=ly.rope.beta_fast, beta_slow=ly.rope.beta_slow)
    # one set of buffers for all steps (the one-launch step's counters must stay consistent)
    bufs = layer.DecodeBuffers(B, Hq, Hkv, d, W, p0 + steps, fused=fused)
    for k in range(steps):
        x = wl.draw_new_tokens(k, li)
        db = layer.decode(dev(x["q"]), dev(x["k"]), dev(x["v"]), kc, vc, window=W, pos_offset=p0 + k, rope_table=tab,
                          q_norm_w=dev(x["wq"]), k_norm_w=dev(x["wk"]), norm_offset=c, fused=fused, bufs=bufs)
        if k in check_k:
            torch.cuda.synchronize()
            out = host(db.out)
        for b in check_b:
            if k in check_k:
                ref = attention_layer_step(x["q"][b], x["k"][b], x["v"][b], caches[b], q_norm_w=x["wq"],
                                           k_norm_w=x["wk"], norm_offset=c, scale=1.0 / math.sqrt(d), **omega_kw)
                assert_parity(out[b], ref, TOL_BF16, f"layer {li} step {k} sequence {b}")
            else:  # the oracle's cache takes the step's normalised K and raw V
                caches[b].update(offset_rms_norm(x["k"][b], x["wk"], c), x["v"][b])


@pytest.mark.parametrize("window", [0, 16, 2048])
def test_prefill_then_decode_matches_oracle(window):
    """Prefill T tokens into the cache, then decode k more one by one: each step equals the
    oracle run on the same token stream (「PLaMo 3アーキテクチャ徹底解析」 §10 method)."""
    B, Hq, Hkv, d, T, steps = 2, 8, 2, 128, 2100, 4
    rope = Rope(1e4) if window else Rope(1e6, 256.0)
    dr = Draw(555 + window, True)
    n = T + steps
    q, k, v = dr.normal((B, n, Hq, d)), dr.normal((B, n, Hkv, d)), dr.normal((B, n, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    cap = window if window else n
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    tab = rope_table(rope, n + 64)
    pre = layer.prefill(dev(q[:, :T]), dev(k[:, :T]), dev(v[:, :T]), window=window, rope_table=tab,
                        q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0, k_cache=kc, v_cache=vc)
    outs = [host(pre.out)]
    for s in range(steps):
        p = T + s
        bufs = layer.decode(dev(q[:, p:p + 1]), dev(k[:, p:p + 1]), dev(v[:, p:p + 1]), kc, vc,
                            window=window, pos_offset=p, rope_table=tab, q_norm_w=dev(wq),
                            k_norm_w=dev(wk), norm_offset=1.0)
        torch.cuda.synchronize()
        outs.append(host(bufs.out))
    got = np.concatenate(outs, axis=1)
    rows = np.concatenate([np.array([0, 1, T // 2, T - 1]), T + np.arange(steps)])
    ref = oracle_prefill(q, k, v, window=window, rope=rope, wq=wq, wk=wk, norm_offset=1.0, rows=rows)
    assert_parity(got[:, rows], ref, TOL_BF16, f"prefill+decode W={window}")


@pytest.mark.parametrize("window,pos_offset,rope", [(2048, 100000, Rope(1e4)), (0, 100000, Rope(1e6, 256.0))],
                         ids=["ring2048", "global_yarn256"])
def test_prefill_chunk_after_long_context(window, pos_offset, rope):
    """A 300-token chunk after 100000 tokens (「PLaMo 3アーキテクチャ徹底解析」 §4.4: the chunk
    attends the kept keys the cache returns, renumbered from 0, then appends itself): the
    cache holds the kept tokens drawn directly (normalised pre-RoPE K, raw V) at their slots
    (the ring wrapped many times; the global cache 100000 deep, at the pages' s = 256 and norm
    offset 1), every other slot NaN; sampled rows of both sequences against the oracle."""
    B, Hq, Hkv, d, T = 2, 8, 2, 128, 300
    cap = window if window else pos_offset + T
    kc = device_normal_bf16((B, Hkv, cap, d), 4100 + window, "cuda")
    vc = device_normal_bf16((B, Hkv, cap, d), 4101 + window, "cuda")
    slots = kept_slots(pos_offset, window)
    live = np.zeros(cap, dtype=bool)
    live[slots] = True
    dead = torch.from_numpy(np.nonzero(~live)[0]).cuda()
    kc[:, :, dead] = float("nan")
    vc[:, :, dead] = float("nan")
    sel = torch.from_numpy(slots).cuda()
    prior_k = [host(kc[b][:, sel]).transpose(1, 0, 2) for b in range(B)]
    prior_v = [host(vc[b][:, sel]).transpose(1, 0, 2) for b in range(B)]
    dr = Draw(4102 + window, True)
    q, k, v = dr.normal((B, T, Hq, d)), dr.normal((B, T, Hkv, d)), dr.normal((B, T, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    tab = rope_table(rope, pos_offset + T + 64)
    bufs = layer.prefill(dev(q), dev(k), dev(v), window=window, rope_table=tab, k_cache=kc, v_cache=vc,
                         pos_offset=pos_offset, q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0)
    torch.cuda.synchronize()
    out = host(bufs.out)
    rows = np.array([0, 1, 63, 64, 150, T - 2, T - 1])
    for b in range(B):
        cache = LayerKVCache.with_prior(prior_k[b], prior_v[b], pos_offset, window)
        ref = attention_layer_step(q[b], k[b], v[b], cache, theta=rope.theta, yarn_factor=rope.yarn_factor,
                                   orig_ctx=rope.orig_ctx, beta_fast=rope.beta_fast, beta_slow=rope.beta_slow,
                                   q_norm_w=wq, k_norm_w=wk, norm_offset=1.0, scale=1.0 / math.sqrt(d), rows=rows)
        assert_parity(out[b][rows], ref, TOL_BF16, f"chunk after {pos_offset} W={window} b={b}")


@pytest.mark.parametrize("window,chunks,bf16", [(0, [100, 37, 300], True), (16, [5, 20, 3, 40], True),
                                                (2048, [1500, 700, 900, 64], True),
                                                (128, [200, 1, 311], False)],
                         ids=["global", "ring16", "ring2048", "fp32_ring128"])
def test_chunked_prefill_matches_oracle(window, chunks, bf16):
    """A prefill in chunks (pos_offset > 0: each chunk attends the cached keys the previous
    chunks left, then appends itself) equals the oracle run on the same token stream
    chunk by chunk (「PLaMo 3アーキテクチャ徹底解析」 §4.4, §10)."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    n = sum(chunks)
    rope = Rope(1e4) if window else Rope(1e6, 64.0)
    dr = Draw(777 + window + n, bf16)
    q, k, v = dr.normal((B, n, Hq, d)), dr.normal((B, n, Hkv, d)), dr.normal((B, n, Hkv, d))
    wq, wk = (dr.normal((d,), 0.02), dr.normal((d,), 0.02)) if bf16 else (None, None)
    dt = torch.bfloat16 if bf16 else torch.float32
    cap = window if window else n
    kc = torch.zeros((B, Hkv, cap, d), dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    tab = rope_table(rope, n + 64)
    put = lambda x: dev(x, bf16)
    norm = dict(q_norm_w=put(wq), k_norm_w=put(wk), norm_offset=1.0) if bf16 else {}
    got, p = [], 0
    for T in chunks:
        bufs = layer.prefill(put(q[:, p:p + T]), put(k[:, p:p + T]), put(v[:, p:p + T]), window=window,
                             rope_table=tab, k_cache=kc, v_cache=vc, pos_offset=p, **norm)
        torch.cuda.synchronize()
        got.append(host(bufs.out))
        p += T
    rows_of = lambda T: np.unique(np.array([0, 1, T // 3, T // 2, T - 2, T - 1]).clip(0, T - 1))
    ref = oracle_chunks(q, k, v, chunks, window=window, rope=rope, wq=wq, wk=wk, rows_of=rows_of)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert_parity(g[:, rows_of(chunks[i])], r, TOL_BF16 if bf16 else TOL_F32,
                      f"chunk {i} (T={chunks[i]}) W={window}")


@pytest.mark.parametrize("window,steps,bf16", [
    (0, [[150, 37, 600], [70, 200, 0]], True),
    (16, [[40, 3, 17], [9, 30, 0]], True),
    (2048, [[2500, 100, 1300], [300, 500, 0]], True),
    (128, [[300, 5, 130], [64, 190, 0]], False),
], ids=["global", "ring16", "ring2048", "fp32_ring128"])
def test_ragged_batch_matches_oracle(window, steps, bf16):
    """A ragged batch (「PLaMo 3アーキテクチャ徹底解析」 §4.4 per sequence): each step gives every
    sequence its own position and token count (0 = it sits the step out); then (bf16) one
    ragged decode step. Every sequence equals the oracle run on its own token stream in the
    same chunks. Input rows past a sequence's count are NaN (they must not be read) and output
    rows past it keep a sentinel (they must not be written)."""
    B, Hq, Hkv, d = 3, 8, 2, 128
    lens = np.array(steps, dtype=np.int64)
    n_tot = lens.sum(0) + (1 if bf16 else 0)
    rope = Rope(1e4) if window else Rope(1e6, 64.0)
    dr = Draw(4242 + window, bf16)
    streams = [(dr.normal((1, n, Hq, d)), dr.normal((1, n, Hkv, d)), dr.normal((1, n, Hkv, d))) for n in n_tot]
    wq, wk = (dr.normal((d,), 0.02), dr.normal((d,), 0.02)) if bf16 else (None, None)
    dt = torch.bfloat16 if bf16 else torch.float32
    cap = window if window else int(n_tot.sum())  # global: >= the largest position + T of any step
    kc = torch.zeros((B, Hkv, cap, d), dtype=dt, device="cuda")
    vc = torch.zeros_like(kc)
    tab = rope_table(rope, int(n_tot.sum()) + 64)  # renumbered positions stay below kept + T
    put = lambda x: dev(x, bf16)
    norm = dict(q_norm_w=put(wq), k_norm_w=put(wk), norm_offset=1.0) if bf16 else {}
    pos = np.zeros(B, np.int64)
    got = [[] for _ in range(B)]
    sentinel = 123.0

    def slab(i, L, T):
        x = np.full((B, T) + streams[0][i].shape[2:], np.nan, np.float32)
        for b in range(B):
            x[b, :L[b]] = streams[b][i][0, pos[b]:pos[b] + L[b]]
        return put(x)

    for L in lens:
        T = int(L.max())
        maxp = int(pos.max())
        sp = torch.tensor(pos, dtype=torch.int64, device="cuda")
        sl = torch.tensor(L, dtype=torch.int32, device="cuda")
        bufs = layer.PrefillBuffers(B, T, Hq, Hkv, d, dt, "cuda", window, maxp)
        bufs.out.fill_(sentinel)
        layer.prefill_ragged(slab(0, L, T), slab(1, L, T), slab(2, L, T), window=window, rope_table=tab,
                             seq_pos_offsets=sp, max_pos_offset=maxp, seq_lens=sl, k_cache=kc, v_cache=vc,
                             bufs=bufs, **norm)
        torch.cuda.synchronize()
        out = host(bufs.out)
        for b in range(B):
            assert np.all(out[b, L[b]:] == sentinel), f"rows past sequence {b}'s count were written"
            if L[b]:
                got[b].append(out[b, :L[b]])
        pos += L
    if bf16:
        one = np.ones(B, np.int64)
        sp = torch.tensor(pos, dtype=torch.int64, device="cuda")
        db = layer.decode_ragged(slab(0, one, 1), slab(1, one, 1), slab(2, one, 1), kc, vc, window=window,
                                 seq_pos_offsets=sp, max_pos_offset=int(pos.max()), rope_table=tab, **norm)
        torch.cuda.synchronize()
        out = host(db.out)
        for b in range(B):
            got[b].append(out[b])
    for b in range(B):
        chunks = [int(L[b]) for L in lens if L[b]] + ([1] if bf16 else [])
        q, k, v = streams[b]
        ref = oracle_chunks(q, k, v, chunks, window=window, rope=rope, wq=wq, wk=wk)
        for i, (g, r) in enumerate(zip(got[b], ref)):
            assert_parity(g, r[0], TOL_BF16 if bf16 else TOL_F32, f"sequence {b} chunk {i} W={window}")


def test_decode_ragged_full_size():
    """Ragged batched decode at its real shape (B=64, Hq=64, Hkv=8, global cache sized for
    32768 keys, each sequence at its own seeded position): sampled sequences, including the
    shortest and the longest, vs the oracle."""
    from synthetic.workloads import RAGGED_DECODE_SEED, ragged_positions
    wl = BATCHED_DECODE
    li = 1
    ly = wl.layers[li]
    d = wl.d
    pos = ragged_positions(wl.B, wl.pos_offset, RAGGED_DECODE_SEED)
    maxp = int(pos.max())
    cap = wl.cache_cap(ly)
    kc = device_normal_bf16((wl.B, wl.Hkv, cap, d), wl.cache_seed(li), "cuda")
    vc = device_normal_bf16((wl.B, wl.Hkv, cap, d), wl.cache_seed(li) + 1, "cuda")
    check_b = sorted({0, 31, int(np.argmin(pos)), int(np.argmax(pos))})
    prior_k = {b: host(kc[b, :, :pos[b]]).transpose(1, 0, 2) for b in check_b}
    prior_v = {b: host(vc[b, :, :pos[b]]).transpose(1, 0, 2) for b in check_b}
    new = wl.draw_new_tokens(0, li)
    tab = rope_table(ly.rope, maxp + 64)
    sp = torch.from_numpy(pos).cuda()
    bufs = layer.decode_ragged(dev(new["q"]), dev(new["k"]), dev(new["v"]), kc, vc, window=0, seq_pos_offsets=sp,
                               max_pos_offset=maxp, rope_table=tab, q_norm_w=dev(new["wq"]),
                               k_norm_w=dev(new["wk"]), norm_offset=wl.norm_offset)
    torch.cuda.synchronize()
    out = host(bufs.out)
    for b in check_b:
        ref = oracle_decode_one(new["q"][b], new["k"][b], new["v"][b], prior_k[b], prior_v[b], int(pos[b]),
                                window=0, rope=ly.rope, wq=new["wq"], wk=new["wk"], norm_offset=wl.norm_offset)
        assert_parity(out[b], ref, TOL_BF16, f"ragged decode b={b} p={pos[b]}")


def _stream_case(window_arg, oracle_window, legacy_4k, rope, chunks, steps, seed, post_rope=False):
    """Prefill in chunks, then `steps` decode steps, on one token stream of B=2 sequences;
    each call's output rows (sampled) against the oracle run on the same stream. With a
    post-RoPE cache, also the cache contents against the oracle's."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    n = sum(chunks) + steps
    dr = Draw(seed, True)
    q, k, v = dr.normal((B, n, Hq, d)), dr.normal((B, n, Hkv, d)), dr.normal((B, n, Hkv, d))
    wq, wk = dr.normal((d,), 0.02), dr.normal((d,), 0.02)
    cap = window_arg if window_arg else n
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    tab = rope_table(rope, n + 64)
    norm = dict(q_norm_w=dev(wq), k_norm_w=dev(wk), norm_offset=1.0)
    got, p = [], 0
    for T in chunks:
        bufs = layer.prefill(dev(q[:, p:p + T]), dev(k[:, p:p + T]), dev(v[:, p:p + T]), window=window_arg,
                             rope_table=tab, k_cache=kc, v_cache=vc, pos_offset=p, cache_post_rope=post_rope,
                             **norm)
        torch.cuda.synchronize()
        got.append(host(bufs.out))
        p += T
    for _ in range(steps):
        db = layer.decode(dev(q[:, p:p + 1]), dev(k[:, p:p + 1]), dev(v[:, p:p + 1]), kc, vc, window=window_arg,
                          pos_offset=p, rope_table=tab, cache_post_rope=post_rope, **norm)
        torch.cuda.synchronize()
        got.append(host(db.out))
        p += 1
    all_chunks = list(chunks) + [1] * steps
    edges = [0, 1, 15, 16, 17, 2046, 2047, 2048, 2049, 2050]
    rows_of = lambda T: np.unique(np.array(edges + [T // 3, T // 2, T - 2, T - 1]).clip(0, T - 1))
    caches = []
    ref = oracle_chunks(q, k, v, all_chunks, window=oracle_window, rope=rope, wq=wq, wk=wk, rows_of=rows_of,
                        legacy_4k=legacy_4k, post_rope=post_rope, caches_out=caches)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert_parity(g[:, rows_of(all_chunks[i])], r, TOL_BF16, f"call {i} (T={all_chunks[i]})")
    if post_rope:  # the kept tokens, as stored: K rotated at absolute positions, in their slots
        for b in range(B):
            keep = caches[b].k.shape[0]
            slots = np.arange(n - keep, n) if not window_arg else np.arange(n - keep, n) % window_arg
            assert_parity(host(kc[b][:, torch.from_numpy(slots).cuda()]).transpose(1, 0, 2), caches[b].k, TOL_BF16,
                          f"post-RoPE cache K, sequence {b}")


@pytest.mark.parametrize("W,chunks", [(2048, [2500, 300]), (16, [40, 5])], ids=["W2048", "W16"])
def test_legacy_4k_window(W, chunks):
    """The 4K release's local layer (「PLaMo 3アーキテクチャ徹底解析」 §5.1: band to distance W,
    cache of the last W tokens) run as window W + 1: chunked prefill then decode, against the
    oracle's own reading of that band (legacy_4k) at window W."""
    _stream_case(swg.legacy_4k_window(W), W, True, Rope(1e4), chunks, 3, 5150 + W)


def test_global_without_yarn():
    """A global layer without YaRN (the 4K release, 「PLaMo 3アーキテクチャ徹底解析」 §6.3): table
    built with yarn_factor 0; chunked prefill then decode against the oracle."""
    _stream_case(0, 0, False, Rope(1e6), [300, 200], 3, 5199)


@pytest.mark.parametrize("window,chunks,rope", [(2048, [2500, 300], Rope(1e4)), (16, [40, 5], Rope(1e4)),
                                                (0, [300, 200], Rope(1e6, 64.0))],
                         ids=["W2048", "W16", "global_yarn64"])
def test_post_rope_cache(window, chunks, rope):
    """The post-RoPE cache order (「PLaMo 3アーキテクチャ徹底解析」 §4.4's other order: K rotated
    at its absolute position before the store): chunked prefill then decode against the
    oracle's post-RoPE layer, and the cache contents against the oracle's cache."""
    _stream_case(window, window, False, rope, chunks, 3, 6100 + window, post_rope=True)
