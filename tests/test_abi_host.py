"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point the header declares, and rejects bad arguments with the documented status
before launching anything. Only calls that fail validation are made here."""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from sliding_window_global_amd import _lib
from sliding_window_global_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "plamo_attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4
BF16, F32 = 1, 0
FAKE = ctypes.c_void_p(0x7F0000000000)      # never dereferenced: every call below fails validation
MISALIGNED = ctypes.c_void_p(0x7F0000000008)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        pytest.fail(f"{LIB_PATH} not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    return re.findall(r"PLAMO_API[^;(]*?\b(plamo_\w+)\s*\(", src)


def test_header_declares_the_abi():
    names = set(declared_functions())
    assert {"plamo_kv_append", "plamo_attn_prefill", "plamo_attn_decode"} <= names
    assert names == set(_lib.SIGNATURES), "binding signatures must mirror the header"


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR):
        assert lib.plamo_status_str(st)
    assert lib.plamo_status_str(12345) == b"unknown status"


def test_pure_host_helpers(lib):
    assert lib.plamo_prefill_padded_len(0) == 0
    assert lib.plamo_prefill_padded_len(1) == 128
    assert lib.plamo_prefill_padded_len(128) == 128
    assert lib.plamo_prefill_padded_len(8193) == 8320
    # rope table: 64 fine rows + ceil(max_pos / 64) coarse rows of 64 (cos, sin) fp32 pairs
    assert lib.plamo_rope_table_bytes(1, 128) == (64 + 1) * 512
    assert lib.plamo_rope_table_bytes(131200, 128) == (64 + 2050) * 512
    assert lib.plamo_rope_table_bytes(0, 128) == 0
    assert lib.plamo_rope_table_bytes(100, 64) == 0
    # wider heads: d/2 pairs per row
    assert lib.plamo_rope_table_bytes(1, 256) == (64 + 1) * 1024
    assert lib.plamo_rope_table_bytes(131072, 512) == (64 + 2048) * 2048


def test_decode_workspace_sizes(lib):
    # a workspace holds (acc[128], m, l) fp32 per (sequence, query head, split)
    n = lib.plamo_attn_decode_workspace_bytes(8, 64, 8, 128, 0, 131071)
    assert n > 0 and n % (130 * 4 * 8 * 64) == 0 and n // (130 * 4 * 8 * 64) > 1
    # 512 (sequence, KV head) pairs fill the GPU with one key range each: no split state
    assert lib.plamo_attn_decode_workspace_bytes(64, 64, 8, 128, 0, 32767) == 0
    assert lib.plamo_attn_decode_workspace_bytes(64, 64, 8, 96, 0, 10) == 0  # d != 128
    assert lib.plamo_attn_decode_workspace_bytes(0, 64, 8, 128, 0, 10) == 0
    # a ragged batch cuts its key ranges finer than the uniform plan of its longest sequence
    n = lib.plamo_attn_decode_ragged_workspace_bytes(64, 64, 8, 128, 0, 32767)
    assert n > 0 and n % (130 * 4 * 64 * 64) == 0 and n // (130 * 4 * 64 * 64) > 1
    # wide heads: (acc[d], m, l) per split
    n = lib.plamo_attn_decode_workspace_bytes(8, 32, 4, 512, 0, 131071)
    assert n > 0 and n % (514 * 4 * 8 * 32) == 0 and n // (514 * 4 * 8 * 32) > 1


@pytest.mark.parametrize("B,Hq,Hkv,d,window", [(8, 64, 8, 128, 0), (8, 64, 8, 128, 2048), (1, 8, 2, 128, 0),
                                                 (64, 64, 8, 128, 0), (3, 32, 4, 512, 0), (5, 32, 16, 256, 1024)])
def test_decode_workspace_sizes_never_shrink(lib, B, Hq, Hkv, d, window):
    """A workspace sized for a position serves every smaller one: the three size queries are
    non-decreasing in the position (the key-range count can fall when a range is rounded up to
    whole tiles; the workspace is sized by the count before that rounding)."""
    queries = [lib.plamo_attn_decode_workspace_bytes, lib.plamo_attn_decode_ragged_workspace_bytes]
    if d == 128:
        queries.append(lib.plamo_decode_step_workspace_bytes)
    positions = list(range(0, 9000)) + list(range(9000, 300000, 97))
    for f in queries:
        prev = 0
        for p in positions:
            n = f(B, Hq, Hkv, d, window, p)
            assert n >= prev, (f.__name__, p, prev, n)
            prev = n


def _append(lib, **over):
    a = dict(dtype=BF16, q=FAKE, k=FAKE, v=FAKE, wq=None, wk=None, c=1.0, eps=1e-6, v_norm=0, q_out=FAKE,
             k_rot=None, v_t=None, kc=None, vc=None, cap=0, B=1, T=4, Hq=8, Hkv=2, d=128, window=16,
             pos=0, table=FAKE, table_bytes=(64 + 1) * 512, order=0, stream=None)
    a.update(over)
    return lib.plamo_kv_append(a["dtype"], a["q"], a["k"], a["v"], a["wq"], a["wk"], a["c"], a["eps"],
                               a["v_norm"], a["q_out"], a["k_rot"], a["v_t"], a["kc"], a["vc"], a["cap"], a["B"], a["T"],
                               a["Hq"], a["Hkv"], a["d"], a["window"], a["pos"], a["table"],
                               a["table_bytes"], a["order"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), INVALID),
    (dict(d=96), UNSUPPORTED),
    (dict(d=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID),
    (dict(Hq=34, Hkv=2), UNSUPPORTED),
    (dict(window=-1), INVALID),
    (dict(pos=-5), INVALID),
    (dict(B=-1), INVALID),
    (dict(q=None), INVALID),
    (dict(q_out=None), INVALID),
    (dict(wq=FAKE), INVALID),                       # one norm weight without the other
    (dict(kc=FAKE), INVALID),                       # one cache without the other
    (dict(kc=FAKE, vc=FAKE, cap=8), INVALID),       # local ring smaller than the window
    (dict(kc=FAKE, vc=FAKE, cap=3, window=0), INVALID),  # global cap < pos + T
    (dict(q=MISALIGNED), INVALID),
    (dict(table=None), INVALID),
    (dict(table_bytes=100), INVALID),               # not whole rows
    (dict(pos=64, window=0, table_bytes=(64 + 1) * 512), WORKSPACE),  # table too short
    (dict(eps=-1.0), INVALID),
    (dict(pos=3, k_rot=FAKE), INVALID),             # operands after cached keys need the caches
    (dict(order=2), INVALID),                        # unknown cache order
    (dict(order=1, pos=62, window=16), WORKSPACE),   # post-RoPE: table covers absolute positions
    (dict(v_norm=2), INVALID),
    (dict(d=256, dtype=F32), UNSUPPORTED),           # wide heads are bf16 only
    (dict(d=512, table_bytes=(64 + 1) * 512 + 512), INVALID),  # d = 512 rows are 2 KiB
    (dict(d=512, pos=64, window=0, table_bytes=(64 + 1) * 2048), WORKSPACE),
])
def test_kv_append_validation(lib, over, status):
    assert _append(lib, **over) == status
    assert lib.plamo_last_error()


def test_kv_append_without_queries(lib):
    # q and q_out both NULL: the K/V side only (for the fused-Q prefill); one of them alone is an error
    assert _append(lib, q=None) == INVALID
    assert _append(lib, q_out=None) == INVALID
    assert _append(lib, q=None, q_out=None, k=None) == INVALID


def test_prefill_fused_q_validation(lib):
    def fused(**over):
        a = dict(dtype=BF16, q=FAKE, wq=FAKE, c=1.0, eps=1e-6, k=FAKE, v=FAKE, out=FAKE, B=1, T=100, Hq=8, Hkv=2,
                 d=128, window=0, pos=0, table=FAKE, table_bytes=(64 + 2) * 512, order=0, scale=0.0884)
        a.update(over)
        return lib.plamo_attn_prefill_fused_q(a["dtype"], a["q"], a["wq"], a["c"], a["eps"], a["k"], a["v"], a["out"],
                                              a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["window"], a["pos"],
                                              a["table"], a["table_bytes"], a["order"], a["scale"], None)
    assert fused(dtype=F32) == UNSUPPORTED
    assert fused(d=256) == UNSUPPORTED
    assert fused(table=None) == INVALID
    assert fused(table_bytes=100) == INVALID
    assert fused(T=200) == WORKSPACE                  # the table covers positions < 128 only
    assert fused(order=1, pos=40, window=16, T=100) == WORKSPACE  # post-RoPE: absolute positions 40 .. 139
    assert fused(order=3) == INVALID
    assert fused(wq=MISALIGNED) == INVALID
    assert fused(eps=-1.0) == INVALID
    assert fused(T=0, q=None) == OK


def test_kv_append_empty_is_ok(lib):
    assert _append(lib, T=0, q=None, k=None, v=None, q_out=None) == OK
    assert _append(lib, B=0, q=None, k=None, v=None, q_out=None) == OK


def _prefill(lib, **over):
    a = dict(dtype=BF16, q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=1, T=100, Hq=8, Hkv=2, d=128, window=0,
             pos=0, scale=0.0884, stream=None)
    a.update(over)
    return lib.plamo_attn_prefill(a["dtype"], a["q"], a["k"], a["v"], a["out"], a["B"], a["T"], a["Hq"],
                                  a["Hkv"], a["d"], a["window"], a["pos"], a["scale"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dtype=3), INVALID), (dict(d=64), UNSUPPORTED), (dict(Hq=9, Hkv=2), INVALID),
    (dict(out=None), INVALID), (dict(k=MISALIGNED), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID), (dict(T=-3), INVALID),
    (dict(T=(1 << 22) + 1), UNSUPPORTED),            # bf16 operands use 32-bit buffer offsets
    (dict(d=512, T=(1 << 20) + 1), UNSUPPORTED),     # the same bound, (kept + T) * d <= 2^29
    (dict(d=256, dtype=F32), UNSUPPORTED), (dict(d=384), UNSUPPORTED),
])
def test_prefill_validation(lib, over, status):
    assert _prefill(lib, **over) == status


def _decode(lib, **over):
    a = dict(dtype=BF16, q=FAKE, kc=FAKE, vc=FAKE, cap=2048, out=FAKE, ws=FAKE, ws_bytes=1 << 30, B=4, T=1,
             Hq=64, Hkv=8, d=128, window=2048, pos=5000, table=FAKE, table_bytes=(64 + 32) * 512,
             scale=0.0884, order=0, stream=None)
    a.update(over)
    return lib.plamo_attn_decode(a["dtype"], a["q"], a["kc"], a["vc"], a["cap"], a["out"], a["ws"],
                                 a["ws_bytes"], a["B"], a["T"], a["Hq"], a["Hkv"], a["d"], a["window"],
                                 a["pos"], a["table"], a["table_bytes"], a["scale"], a["order"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(dtype=F32), UNSUPPORTED), (dict(dtype=9), INVALID), (dict(T=2), UNSUPPORTED),
    (dict(T=-1), INVALID), (dict(Hq=64, Hkv=2), UNSUPPORTED), (dict(cap=100), INVALID),
    (dict(window=0, cap=4000), INVALID), (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
    (dict(table_bytes=(64 + 31) * 512), WORKSPACE), (dict(kc=None), INVALID),
    (dict(out=MISALIGNED), INVALID), (dict(scale=-1.0), INVALID), (dict(order=-1), INVALID),
    (dict(order=1, table=None, ws=None), WORKSPACE),  # post-RoPE needs no table; still a workspace
    (dict(d=256), UNSUPPORTED),                       # wide heads decode from a post-RoPE cache
    (dict(d=512, order=1, table=None, ws=None), WORKSPACE),
    (dict(d=512, order=1, ws_bytes=16), WORKSPACE),
])
def test_decode_validation(lib, over, status):
    assert _decode(lib, **over) == status


def test_rope_init_validation(lib):
    r = _lib.PlamoRope(1e6, 256.0, 4096.0, 32.0, 1.0)
    bad_beta = _lib.PlamoRope(1e6, 256.0, 4096.0, 1.0, 32.0)
    bad_theta = _lib.PlamoRope(0.5, 0.0, 4096.0, 32.0, 1.0)
    need = lib.plamo_rope_table_bytes(1000, 128)
    assert lib.plamo_rope_table_init(None, need, 1000, 128, ctypes.byref(r), None) == INVALID
    assert lib.plamo_rope_table_init(FAKE, need - 512, 1000, 128, ctypes.byref(r), None) == WORKSPACE
    assert lib.plamo_rope_table_init(FAKE, need, 1000, 64, ctypes.byref(r), None) == UNSUPPORTED
    assert lib.plamo_rope_table_init(FAKE, need, 1000, 128, ctypes.byref(bad_beta), None) == INVALID
    assert lib.plamo_rope_table_init(FAKE, need, 1000, 128, ctypes.byref(bad_theta), None) == INVALID
    assert lib.plamo_rope_table_init(FAKE, need, 0, 128, ctypes.byref(r), None) == INVALID
    # p-RoPE: not with YaRN, and a fraction must be >= 0
    p_yarn = _lib.PlamoRope(1e6, 256.0, 4096.0, 32.0, 1.0, 0.25)
    p_neg = _lib.PlamoRope(1e6, 0.0, 4096.0, 32.0, 1.0, -0.25)
    need512 = lib.plamo_rope_table_bytes(1000, 512)
    assert lib.plamo_rope_table_init(FAKE, need512, 1000, 512, ctypes.byref(p_yarn), None) == UNSUPPORTED
    assert lib.plamo_rope_table_init(FAKE, need512, 1000, 512, ctypes.byref(p_neg), None) == INVALID
    assert lib.plamo_rope_table_init(FAKE, need512 - 2048, 1000, 512, ctypes.byref(p_neg), None) == WORKSPACE


def test_tiled_operand_helpers_invert_documented_layout():
    """The test-side untiling of the bf16 prefill operands follows the element order stated in
    include/plamo_attn.h, written out index by index here."""
    from helpers import untile_k_rot, untile_v_t
    rng = np.random.default_rng(5)
    B, H, Tp, d = 2, 3, 128, 16
    k = rng.standard_normal((B, H, Tp, d))
    vt = rng.standard_normal((B, H, d, Tp))
    nt = Tp // 64
    k_tiled = np.empty((B, H, nt, d // 8, 64, 8))
    v_tiled = np.empty((B, H, nt, 8, d, 8))
    for t in range(Tp):
        for j in range(d):
            k_tiled[:, :, t // 64, j // 8, t % 64, j % 8] = k[:, :, t, j]
            v_tiled[:, :, t // 64, (t % 64) // 8, j, t % 8] = vt[:, :, j, t]
    assert np.array_equal(untile_k_rot(k_tiled), k)
    assert np.array_equal(untile_v_t(v_tiled), vt)


def test_ragged_entry_points_validate_their_arrays(lib):
    ALIGNED4 = ctypes.c_void_p(0x7F0000000004)
    base = dict(dtype=BF16, q=FAKE, k=FAKE, v=FAKE, wq=None, wk=None, c=1.0, eps=1e-6, q_out=FAKE, k_rot=None,
                v_t=None, kc=None, vc=None, cap=0, B=2, T=4, Hq=8, Hkv=2, d=128, window=16, table=FAKE,
                table_bytes=(64 + 1) * 512)

    def append(seq_pos, seq_len, max_pos=0, **over):
        a = dict(base, **over)
        return lib.plamo_kv_append_ragged(a["dtype"], a["q"], a["k"], a["v"], a["wq"], a["wk"], a["c"], a["eps"],
                                          0, a["q_out"], a["k_rot"], a["v_t"], a["kc"], a["vc"], a["cap"], a["B"],
                                          a["T"], a["Hq"], a["Hkv"], a["d"], a["window"], seq_pos, seq_len,
                                          max_pos, a["table"], a["table_bytes"], 0, None)
    assert append(None, None) == INVALID                  # positions are required
    assert append(ALIGNED4, None) == INVALID              # int64 array not 8-byte aligned
    assert append(FAKE, ctypes.c_void_p(0x7F0000000002)) == INVALID  # int32 array not 4-byte aligned
    assert append(FAKE, None, max_pos=-1) == INVALID
    assert append(FAKE, None, max_pos=3, k_rot=FAKE) == INVALID  # operands after cached keys need caches
    assert append(FAKE, None, max_pos=64, window=0) == WORKSPACE  # table must cover kept_max + T
    assert append(None, None, B=0) == OK and append(None, None, T=0) == OK

    def prefill(seq_pos, seq_len, max_pos=0, **over):
        a = dict(dtype=BF16, B=2, T=100, Hq=8, Hkv=2, window=0, scale=0.0884)
        a.update(over)
        return lib.plamo_attn_prefill_ragged(a["dtype"], FAKE, FAKE, FAKE, FAKE, a["B"], a["T"], a["Hq"], a["Hkv"],
                                             128, a["window"], seq_pos, seq_len, max_pos, a["scale"], None)
    assert prefill(None, FAKE) == INVALID
    assert prefill(FAKE, ctypes.c_void_p(0x7F0000000001)) == INVALID
    assert prefill(FAKE, None, scale=0.0) == INVALID

    def decode(seq_pos, max_pos=5000, **over):
        a = dict(B=4, window=2048, cap=2048, ws=FAKE, ws_bytes=1 << 30, table_bytes=(64 + 32) * 512)
        a.update(over)
        return lib.plamo_attn_decode_ragged(BF16, FAKE, FAKE, FAKE, a["cap"], FAKE, a["ws"], a["ws_bytes"], a["B"],
                                            64, 8, 128, a["window"], seq_pos, max_pos, FAKE, a["table_bytes"],
                                            0.0884, 0, None)
    assert decode(None) == INVALID
    assert decode(ALIGNED4) == INVALID
    assert decode(FAKE, window=0, cap=4000) == INVALID     # global cap must exceed max_pos_offset
    assert decode(FAKE, ws=None) == WORKSPACE
    assert decode(FAKE, table_bytes=(64 + 31) * 512) == WORKSPACE


def test_sublayer_entry_points_validate(lib):
    assert lib.plamo_linear(FAKE, FAKE, FAKE, -1, 8, 64, None) == INVALID
    assert lib.plamo_linear(FAKE, FAKE, FAKE, 4, 12, 64, None) == UNSUPPORTED   # N % 8
    assert lib.plamo_linear(FAKE, FAKE, FAKE, 4, 8, 96, None) == UNSUPPORTED    # K % 64
    assert lib.plamo_linear(None, FAKE, FAKE, 4, 8, 64, None) == INVALID
    assert lib.plamo_linear(MISALIGNED, FAKE, FAKE, 4, 8, 64, None) == INVALID
    assert lib.plamo_linear(FAKE, FAKE, FAKE, 0, 8, 64, None) == OK
    assert lib.plamo_qkv_projection(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 100, 8, 2, 128, None) == UNSUPPORTED  # D % 64
    assert lib.plamo_qkv_projection(FAKE, FAKE, None, FAKE, FAKE, 4, 256, 8, 2, 128, None) == INVALID
    assert lib.plamo_qkv_projection(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 256, 8, 2, 128, None) == OK
    norm = lambda **o: lib.plamo_rms_norm(o.get("dtype", BF16), o.get("x", FAKE), o.get("w", FAKE), 0.2, 1e-6,
                                         o.get("r", None), o.get("y", FAKE), o.get("rows", 4), o.get("n", 64), None)
    assert norm(dtype=5) == INVALID
    assert norm(n=12) == UNSUPPORTED          # bf16 rows fill 16-byte chunks
    assert norm(rows=-1) == INVALID
    assert norm(x=MISALIGNED) == INVALID
    assert norm(y=None) == INVALID
    assert norm(rows=0) == OK


def test_decode_noalloc_rejects_partials_beyond_its_scratch(lib):
    """plamo_attn_decode_noalloc checks the split-K partials against its fixed scratch before
    touching the GPU: d = 512, one KV head of 16 query heads and 65536 keys need 256 ranges of
    16 x 514 floats, above the 8 MiB."""
    assert lib.plamo_attn_decode_workspace_bytes(1, 16, 1, 512, 0, 65535) > 8 << 20
    big = lib.plamo_attn_decode_noalloc(BF16, FAKE, FAKE, FAKE, 65536, FAKE, 1, 1, 16, 1, 512, 0, 65535,
                                        None, 0, 1.0, 1, None)
    assert big == -3
    assert lib.plamo_attn_decode_noalloc(BF16, FAKE, FAKE, FAKE, 65536, FAKE, 0, 1, 16, 1, 512, 0, 65535,
                                         None, 0, 1.0, 1, None) == 0  # B = 0: nothing to do


def test_prefill_pack_checks(lib):
    """plamo_prefill_pack validates before launching: dtype, head dim, sizes, pointers."""
    assert lib.plamo_prefill_pack(7, FAKE, FAKE, FAKE, FAKE, 1, 10, 2, 128, None) == INVALID
    assert lib.plamo_prefill_pack(BF16, FAKE, FAKE, FAKE, FAKE, 1, 10, 2, 64, None) == -2
    assert lib.plamo_prefill_pack(F32, FAKE, FAKE, FAKE, FAKE, 1, 10, 2, 256, None) == -2
    assert lib.plamo_prefill_pack(BF16, FAKE, FAKE, FAKE, FAKE, -1, 10, 2, 128, None) == INVALID
    assert lib.plamo_prefill_pack(BF16, None, FAKE, FAKE, FAKE, 1, 10, 2, 128, None) == INVALID
    assert lib.plamo_prefill_pack(BF16, ctypes.c_void_p(0x7F0000000008), FAKE, FAKE, FAKE, 1, 10, 2, 128, None) == INVALID
    assert lib.plamo_prefill_pack(BF16, None, None, None, None, 1, 0, 2, 128, None) == 0  # nothing to pack
