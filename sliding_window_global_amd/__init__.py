"""PLaMo 3 hybrid sliding-window / global GQA attention on MI355X (gfx950).

Thin Python binding over the C ABI of ``libplamo_attn.so`` (include/plamo_attn.h).
Each function takes torch tensors that already live on the GPU, checks their dtype,
device, contiguity and shapes, reads the sizes off them, and forwards raw device
pointers plus the current HIP stream to the C entry point of the same name. Every
step of the computation runs in the library's HIP kernels; there is no CPU path.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import PlamoRope

PLAMO_F32 = 0
PLAMO_BF16 = 1
PLAMO_CACHE_PRE_ROPE = 0   # PLaMo 3's order: the cache holds K before RoPE
PLAMO_CACHE_POST_ROPE = 1  # the cache holds K rotated at absolute positions
HEAD_DIM = 128

__all__ = [
    "PlamoError", "RopeParams", "LOCAL_ROPE", "GLOBAL_ROPE",
    "plamo_rope_table_bytes", "plamo_rope_table_init", "make_rope_table",
    "plamo_prefill_padded_len", "legacy_4k_window", "plamo_kv_append", "plamo_attn_prefill",
    "plamo_attn_decode_workspace_bytes", "plamo_attn_decode", "plamo_kv_append_ragged",
    "plamo_attn_prefill_ragged", "plamo_attn_decode_ragged_workspace_bytes", "plamo_attn_decode_ragged",
    "plamo_linear", "plamo_qkv_projection", "plamo_rms_norm", "library_path",
    "plamo_attn_prefill_fused_q", "plamo_attn_prefill_fused_q_ragged",
]


class PlamoError(RuntimeError):
    def __init__(self, status: int, fn: str):
        lib = _lib.load()
        self.status = status
        detail = lib.plamo_last_error().decode()
        super().__init__(f"{fn}: {lib.plamo_status_str(status).decode()} ({status}): {detail}")


@dataclass(frozen=True)
class RopeParams:
    """RoPE of one layer type: base theta, YaRN factor (<= 1 = off), L0, beta_fast, beta_slow, and
    the p-RoPE fraction ``partial`` (0 < p < 1: only the floor(p d/2) highest-frequency pairs turn;
    0 = all)."""
    theta: float
    yarn_factor: float = 0.0
    orig_ctx: float = 4096.0
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    partial: float = 0.0

    def c_struct(self) -> PlamoRope:
        return PlamoRope(self.theta, self.yarn_factor, self.orig_ctx, self.beta_fast, self.beta_slow,
                         self.partial)


LOCAL_ROPE = RopeParams(theta=1e4)
GLOBAL_ROPE = RopeParams(theta=1e6, yarn_factor=256.0)


def library_path() -> str:
    return _lib.LIB_PATH


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise PlamoError(status, fn)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor | None, name: str, dtype=None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _order(post_rope: bool) -> int:
    return PLAMO_CACHE_POST_ROPE if post_rope else PLAMO_CACHE_PRE_ROPE


def _nbytes(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def score_dtype(dt: torch.dtype) -> torch.dtype:
    """Storage type of the score operands Q' (q_out / q_rot) and K' (k_rot) of a layer of
    dtype dt: IEEE half on bf16 layers (include/plamo_attn.h), fp32 on fp32 ones."""
    return torch.float16 if dt == torch.bfloat16 else dt


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return PLAMO_BF16
    if dt == torch.float32:
        return PLAMO_F32
    raise ValueError(f"unsupported dtype {dt}")


def plamo_rope_table_bytes(max_pos: int, d: int = HEAD_DIM) -> int:
    return int(_lib.load().plamo_rope_table_bytes(int(max_pos), int(d)))


def plamo_rope_table_init(table: torch.Tensor, max_pos: int, rope: RopeParams, d: int = HEAD_DIM,
                          stream=None) -> None:
    p = _dev(table, "table")
    nbytes = table.numel() * table.element_size()
    st = _lib.load().plamo_rope_table_init(p, nbytes, int(max_pos), int(d), rope.c_struct(), _stream(stream))
    _check(st, "plamo_rope_table_init")


def make_rope_table(max_pos: int, rope: RopeParams, device="cuda", stream=None, d: int = HEAD_DIM) -> torch.Tensor:
    """Allocate (torch) and fill a rope table covering positions [0, max_pos) for head dim d."""
    nbytes = plamo_rope_table_bytes(max_pos, d)
    if nbytes == 0:
        raise ValueError("bad max_pos or head dim")
    table = torch.empty(nbytes // 4, dtype=torch.float32, device=device)
    plamo_rope_table_init(table, max_pos, rope, d=d, stream=stream)
    return table


def plamo_prefill_padded_len(T: int) -> int:
    return int(_lib.load().plamo_prefill_padded_len(int(T)))


PREFILL_KEY_TILE = 64


def kept_tokens(window: int, pos_offset: int) -> int:
    """Cached tokens a chunk at pos_offset attends before its own (global: all of them; local:
    the last window-1)."""
    return int(pos_offset) if window == 0 else min(int(pos_offset), int(window) - 1)


def legacy_4k_window(window: int) -> int:
    """Window argument that gives the 4K release's local layer (「PLaMo 3アーキテクチャ徹底解析」
    §5.1): its band reaches distance W (W + 1 keys including self) and its cache keeps W
    tokens, which is this library's window W + 1 (ring capacity >= W + 1). Global: 0."""
    return int(window) + 1 if window > 0 else 0


def prefill_operand_shapes(B: int, T: int, Hkv: int, d: int, dtype, window: int = 0,
                           pos_offset: int = 0) -> tuple[tuple, tuple]:
    """Shapes of (k_rot, v_t) as plamo_kv_append writes them (include/plamo_attn.h), for the
    S = kept + T keys a chunk of T tokens at pos_offset attends.

    fp32: [B, Hkv, Sp, d] and [B, Hkv, d, Sp]. bf16: tiled by 64 keys,
    [B, Hkv, Sp/64, d/8, 64, 8] and [B, Hkv, Sp/64, 8, d, 8]. Sp = plamo_prefill_padded_len(S).
    """
    Sp = plamo_prefill_padded_len(kept_tokens(window, pos_offset) + T)
    if dtype == torch.bfloat16:
        nt = Sp // PREFILL_KEY_TILE
        return (B, Hkv, nt, d // 8, PREFILL_KEY_TILE, 8), (B, Hkv, nt, PREFILL_KEY_TILE // 8, d, 8)
    return (B, Hkv, Sp, d), (B, Hkv, d, Sp)


def plamo_kv_append(q, k, v, q_out, *, window: int, pos_offset: int, rope_table,
                    q_norm_w=None, k_norm_w=None, norm_offset: float = 1.0, norm_eps: float = 1e-6,
                    k_rot_out=None, v_t_out=None, k_cache=None, v_cache=None, cache_post_rope: bool = False,
                    v_norm: bool = False, stream=None) -> None:
    """q [B,T,Hq,d], k/v [B,T,Hkv,d] (k and v may be one tensor); outputs as documented in
    plamo_attn.h. v_norm: divide each V head vector by its RMS first."""
    dt = k.dtype
    B, T, Hkv, d = k.shape
    if q is None:  # K/V side only: the queries go to plamo_attn_prefill_fused_q
        if q_out is not None:
            raise ValueError("give q and q_out, or neither")
        Hq = 0
    else:
        Hq = q.shape[2]
        if tuple(q.shape) != (B, T, Hq, d) or tuple(q_out.shape) != (B, T, Hq, d):
            raise ValueError("q and q_out must be [B, T, Hq, d] matching k")
    if tuple(v.shape) != (B, T, Hkv, d):
        raise ValueError("v must be [B, T, Hkv, d] matching k")
    k_shape, v_shape = prefill_operand_shapes(B, T, Hkv, d, dt, window, pos_offset)
    if k_rot_out is not None and tuple(k_rot_out.shape) != k_shape:
        raise ValueError(f"k_rot_out must be {list(k_shape)}")
    if v_t_out is not None and tuple(v_t_out.shape) != v_shape:
        raise ValueError(f"v_t_out must be {list(v_shape)}")
    cap = 0
    if k_cache is not None:
        cap = k_cache.shape[2]
        if tuple(k_cache.shape) != (B, Hkv, cap, d) or v_cache is None or tuple(v_cache.shape) != tuple(k_cache.shape):
            raise ValueError("caches must both be [B, Hkv, cap, d]")
    st = _lib.load().plamo_kv_append(
        _dtype_code(dt), _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt),
        _dev(q_norm_w, "q_norm_w", dt), _dev(k_norm_w, "k_norm_w", dt), float(norm_offset), float(norm_eps),
        int(bool(v_norm)), _dev(q_out, "q_out", score_dtype(dt)), _dev(k_rot_out, "k_rot_out", score_dtype(dt)),
        _dev(v_t_out, "v_t_out", dt),
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt), int(cap), B, T, Hq or Hkv, Hkv, d,
        int(window), int(pos_offset), _dev(rope_table, "rope_table", torch.float32),
        rope_table.numel() * 4, _order(cache_post_rope), _stream(stream))
    _check(st, "plamo_kv_append")


def plamo_prefill_pack(k_rot_in, v_in, k_rot_out, v_t_out, *, stream=None) -> None:
    """Caller-held K' and V [B, S, Hkv, d] into the prefill operand layouts (shapes from
    prefill_operand_shapes with T = S, pos_offset = 0; K' output in score_dtype)."""
    dt = v_in.dtype
    B, S, Hkv, d = v_in.shape
    if tuple(k_rot_in.shape) != (B, S, Hkv, d):
        raise ValueError("k_rot_in and v_in must both be [B, S, Hkv, d]")
    k_shape, v_shape = prefill_operand_shapes(B, S, Hkv, d, dt)
    if tuple(k_rot_out.shape) != k_shape or tuple(v_t_out.shape) != v_shape:
        raise ValueError(f"k_rot_out must be {list(k_shape)} and v_t_out {list(v_shape)}")
    st = _lib.load().plamo_prefill_pack(
        _dtype_code(dt), _dev(k_rot_in, "k_rot_in", dt), _dev(v_in, "v_in", dt),
        _dev(k_rot_out, "k_rot_out", score_dtype(dt)), _dev(v_t_out, "v_t_out", dt), B, S, Hkv, d, _stream(stream))
    _check(st, "plamo_prefill_pack")


def plamo_attn_prefill(q_rot, k_rot, v_t, out, *, window: int, pos_offset: int = 0,
                       softmax_scale: float | None = None, stream=None) -> None:
    """q_rot [B,T,Hq,d], k_rot / v_t as prefill_operand_shapes -> out [B,T,Hq,d] (q_rot and
    k_rot in score_dtype of the layer's dtype, v_t and out in the layer's dtype)."""
    dt = v_t.dtype
    B, T, Hq, d = q_rot.shape
    Hkv = k_rot.shape[1]
    k_shape, v_shape = prefill_operand_shapes(B, T, Hkv, d, dt, window, pos_offset)
    if tuple(k_rot.shape) != k_shape or tuple(v_t.shape) != v_shape:
        raise ValueError(f"k_rot must be {list(k_shape)} and v_t {list(v_shape)}")
    if tuple(out.shape) != (B, T, Hq, d):
        raise ValueError("out must match q_rot")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().plamo_attn_prefill(
        _dtype_code(dt), _dev(q_rot, "q_rot", score_dtype(dt)), _dev(k_rot, "k_rot", score_dtype(dt)),
        _dev(v_t, "v_t", dt), _dev(out, "out", dt), B, T, Hq, Hkv, d, int(window), int(pos_offset), scale, _stream(stream))
    _check(st, "plamo_attn_prefill")


def plamo_attn_prefill_fused_q(q, k_rot, v_t, out, *, window: int, rope_table, pos_offset: int = 0,
                               q_norm_w=None, norm_offset: float = 1.0, norm_eps: float = 1e-6,
                               cache_post_rope: bool = False, softmax_scale: float | None = None,
                               stream=None) -> None:
    """plamo_attn_prefill on the projected queries q [B,T,Hq,d] (bf16, d = 128): the kernel
    normalises and rotates them itself; call plamo_kv_append with q = q_out = None first."""
    dt = q.dtype
    B, T, Hq, d = q.shape
    Hkv = k_rot.shape[1]
    k_shape, v_shape = prefill_operand_shapes(B, T, Hkv, d, dt, window, pos_offset)
    if tuple(k_rot.shape) != k_shape or tuple(v_t.shape) != v_shape:
        raise ValueError(f"k_rot must be {list(k_shape)} and v_t {list(v_shape)}")
    if tuple(out.shape) != (B, T, Hq, d):
        raise ValueError("out must match q")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().plamo_attn_prefill_fused_q(
        _dtype_code(dt), _dev(q, "q", dt), _dev(q_norm_w, "q_norm_w", dt), float(norm_offset), float(norm_eps),
        _dev(k_rot, "k_rot", score_dtype(dt)), _dev(v_t, "v_t", dt), _dev(out, "out", dt), B, T, Hq, Hkv, d,
        int(window),
        int(pos_offset), _dev(rope_table, "rope_table", torch.float32), _nbytes(rope_table),
        _order(cache_post_rope), scale, _stream(stream))
    _check(st, "plamo_attn_prefill_fused_q")


def plamo_attn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, window: int, pos_offset: int,
                                      d: int = HEAD_DIM) -> int:
    return int(_lib.load().plamo_attn_decode_workspace_bytes(B, Hq, Hkv, d, int(window), int(pos_offset)))


def plamo_attn_decode(q_rot, k_cache, v_cache, out, workspace, *, window: int, pos_offset: int,
                      rope_table, softmax_scale: float | None = None, cache_post_rope: bool = False,
                      stream=None) -> None:
    """q_rot [B,1,Hq,d] (fp16); caches [B,Hkv,cap,d] (bf16) -> out [B,1,Hq,d] (bf16)."""
    dt = out.dtype
    B, T, Hq, d = q_rot.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must both be [B, Hkv, cap, d]")
    if tuple(out.shape) != (B, T, Hq, d):
        raise ValueError("out must match q_rot")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.load().plamo_attn_decode(
        _dtype_code(dt), _dev(q_rot, "q_rot", score_dtype(dt)), _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt),
        int(cap), _dev(out, "out", dt), _dev(workspace, "workspace"), ws_bytes, B, T, Hq, Hkv, d,
        int(window), int(pos_offset), _dev(rope_table, "rope_table", torch.float32), _nbytes(rope_table),
        scale, _order(cache_post_rope), _stream(stream))
    _check(st, "plamo_attn_decode")


def plamo_decode_step_workspace_bytes(B: int, Hq: int, Hkv: int, window: int, pos_offset: int,
                                      d: int = HEAD_DIM) -> int:
    return int(_lib.load().plamo_decode_step_workspace_bytes(B, Hq, Hkv, d, int(window), int(pos_offset)))


def plamo_decode_step(q, k, v, k_cache, v_cache, out, workspace, *, window: int, pos_offset: int, rope_table,
                      q_norm_w=None, k_norm_w=None, norm_offset: float = 1.0, norm_eps: float = 1e-6,
                      softmax_scale: float | None = None, cache_post_rope: bool = False, stream=None) -> None:
    """One decode step of a layer in one launch (plamo_kv_append + plamo_attn_decode): q
    [B,1,Hq,d], k/v [B,1,Hkv,d] (bf16) -> out [B,1,Hq,d]; the new token goes into the caches.
    workspace: a zero-initialised tensor of plamo_decode_step_workspace_bytes (kept across calls)."""
    dt = q.dtype
    B, T, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if T != 1 or tuple(k.shape) != (B, 1, Hkv, d) or tuple(v.shape) != (B, 1, Hkv, d):
        raise ValueError("need q [B,1,Hq,d] and k, v [B,1,Hkv,d]")
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must both be [B, Hkv, cap, d]")
    if tuple(out.shape) != (B, 1, Hq, d):
        raise ValueError("out must match q")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().plamo_decode_step(
        _dtype_code(dt), _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt), _dev(q_norm_w, "q_norm_w", dt),
        _dev(k_norm_w, "k_norm_w", dt), float(norm_offset), float(norm_eps), _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), int(cap), _dev(out, "out", dt), _dev(workspace, "workspace"),
        _nbytes(workspace), B, Hq, Hkv, d, int(window), int(pos_offset), _dev(rope_table, "rope_table", torch.float32),
        _nbytes(rope_table), scale, _order(cache_post_rope), _stream(stream))
    _check(st, "plamo_decode_step")


PLAMO_DECODE_SCRATCH_BYTES = 8 << 20


def plamo_attn_decode_noalloc(q_rot, k_cache, v_cache, out, *, window: int, pos_offset: int, rope_table,
                              softmax_scale: float | None = None, cache_post_rope: bool = False,
                              stream=None) -> None:
    """plamo_attn_decode without a workspace: the split-K partials go to the library's own
    per-GPU scratch (PLAMO_DECODE_SCRATCH_BYTES); calls that overlap on one GPU race."""
    dt = out.dtype
    B, T, Hq, d = q_rot.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must both be [B, Hkv, cap, d]")
    if tuple(out.shape) != (B, T, Hq, d):
        raise ValueError("out must match q_rot")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = _lib.load().plamo_attn_decode_noalloc(
        _dtype_code(dt), _dev(q_rot, "q_rot", score_dtype(dt)), _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt), int(cap), _dev(out, "out", dt), B, T, Hq, Hkv, d, int(window),
        int(pos_offset), _dev(rope_table, "rope_table", torch.float32), _nbytes(rope_table), scale,
        _order(cache_post_rope), _stream(stream))
    _check(st, "plamo_attn_decode_noalloc")


# ----------------------------------------------------------------------------
# ragged batches: one position (and, for append / prefill, one token count) per sequence
# ----------------------------------------------------------------------------

def _ragged_arrays(B: int, seq_pos_offsets, seq_lens):
    if seq_pos_offsets is None or tuple(seq_pos_offsets.shape) != (B,):
        raise ValueError("seq_pos_offsets must be an int64 GPU tensor of shape [B]")
    if seq_lens is not None and tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be an int32 GPU tensor of shape [B]")
    return _dev(seq_pos_offsets, "seq_pos_offsets", torch.int64), _dev(seq_lens, "seq_lens", torch.int32)


def plamo_kv_append_ragged(q, k, v, q_out, *, window: int, seq_pos_offsets, max_pos_offset: int,
                           rope_table, seq_lens=None, q_norm_w=None, k_norm_w=None,
                           norm_offset: float = 1.0, norm_eps: float = 1e-6, k_rot_out=None, v_t_out=None,
                           k_cache=None, v_cache=None, cache_post_rope: bool = False, v_norm: bool = False,
                           stream=None) -> None:
    """plamo_kv_append with per-sequence positions seq_pos_offsets [B] (int64, GPU) bounded by
    max_pos_offset and token counts seq_lens [B] (int32, GPU; None = T each)."""
    dt = k.dtype
    B, T, Hkv, d = k.shape
    if q is None:  # K/V side only: the queries go to plamo_attn_prefill_fused_q_ragged
        if q_out is not None:
            raise ValueError("give q and q_out, or neither")
        Hq = 0
    else:
        Hq = q.shape[2]
        if tuple(q.shape) != (B, T, Hq, d) or tuple(q_out.shape) != (B, T, Hq, d):
            raise ValueError("q and q_out must be [B, T, Hq, d] matching k")
    if tuple(v.shape) != (B, T, Hkv, d):
        raise ValueError("v must be [B, T, Hkv, d] matching k")
    k_shape, v_shape = prefill_operand_shapes(B, T, Hkv, d, dt, window, max_pos_offset)
    if k_rot_out is not None and tuple(k_rot_out.shape) != k_shape:
        raise ValueError(f"k_rot_out must be {list(k_shape)}")
    if v_t_out is not None and tuple(v_t_out.shape) != v_shape:
        raise ValueError(f"v_t_out must be {list(v_shape)}")
    cap = 0
    if k_cache is not None:
        cap = k_cache.shape[2]
        if tuple(k_cache.shape) != (B, Hkv, cap, d) or v_cache is None or tuple(v_cache.shape) != tuple(k_cache.shape):
            raise ValueError("caches must both be [B, Hkv, cap, d]")
    pos_p, len_p = _ragged_arrays(B, seq_pos_offsets, seq_lens)
    st = _lib.load().plamo_kv_append_ragged(
        _dtype_code(dt), _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt),
        _dev(q_norm_w, "q_norm_w", dt), _dev(k_norm_w, "k_norm_w", dt), float(norm_offset), float(norm_eps),
        int(bool(v_norm)), _dev(q_out, "q_out", score_dtype(dt)), _dev(k_rot_out, "k_rot_out", score_dtype(dt)),
        _dev(v_t_out, "v_t_out", dt),
        _dev(k_cache, "k_cache", dt), _dev(v_cache, "v_cache", dt), int(cap), B, T, Hq or Hkv, Hkv, d,
        int(window), pos_p, len_p, int(max_pos_offset), _dev(rope_table, "rope_table", torch.float32),
        rope_table.numel() * 4, _order(cache_post_rope), _stream(stream))
    _check(st, "plamo_kv_append_ragged")


def plamo_attn_prefill_ragged(q_rot, k_rot, v_t, out, *, window: int, seq_pos_offsets, max_pos_offset: int,
                              seq_lens=None, softmax_scale: float | None = None, stream=None) -> None:
    """plamo_attn_prefill with per-sequence positions and token counts (as plamo_kv_append_ragged)."""
    dt = v_t.dtype
    B, T, Hq, d = q_rot.shape
    Hkv = k_rot.shape[1]
    k_shape, v_shape = prefill_operand_shapes(B, T, Hkv, d, dt, window, max_pos_offset)
    if tuple(k_rot.shape) != k_shape or tuple(v_t.shape) != v_shape:
        raise ValueError(f"k_rot must be {list(k_shape)} and v_t {list(v_shape)}")
    if tuple(out.shape) != (B, T, Hq, d):
        raise ValueError("out must match q_rot")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    pos_p, len_p = _ragged_arrays(B, seq_pos_offsets, seq_lens)
    st = _lib.load().plamo_attn_prefill_ragged(
        _dtype_code(dt), _dev(q_rot, "q_rot", score_dtype(dt)), _dev(k_rot, "k_rot", score_dtype(dt)),
        _dev(v_t, "v_t", dt), _dev(out, "out", dt), B, T, Hq, Hkv, d, int(window), pos_p, len_p, int(max_pos_offset), scale,
        _stream(stream))
    _check(st, "plamo_attn_prefill_ragged")


def plamo_attn_prefill_fused_q_ragged(q, k_rot, v_t, out, *, window: int, seq_pos_offsets, max_pos_offset: int,
                                      rope_table, seq_lens=None, q_norm_w=None, norm_offset: float = 1.0,
                                      norm_eps: float = 1e-6, cache_post_rope: bool = False,
                                      softmax_scale: float | None = None, stream=None) -> None:
    """plamo_attn_prefill_fused_q with per-sequence positions and token counts."""
    dt = q.dtype
    B, T, Hq, d = q.shape
    Hkv = k_rot.shape[1]
    k_shape, v_shape = prefill_operand_shapes(B, T, Hkv, d, dt, window, max_pos_offset)
    if tuple(k_rot.shape) != k_shape or tuple(v_t.shape) != v_shape:
        raise ValueError(f"k_rot must be {list(k_shape)} and v_t {list(v_shape)}")
    if tuple(out.shape) != (B, T, Hq, d):
        raise ValueError("out must match q")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    pos_p, len_p = _ragged_arrays(B, seq_pos_offsets, seq_lens)
    st = _lib.load().plamo_attn_prefill_fused_q_ragged(
        _dtype_code(dt), _dev(q, "q", dt), _dev(q_norm_w, "q_norm_w", dt), float(norm_offset), float(norm_eps),
        _dev(k_rot, "k_rot", score_dtype(dt)), _dev(v_t, "v_t", dt), _dev(out, "out", dt), B, T, Hq, Hkv, d,
        int(window),
        pos_p, len_p, int(max_pos_offset), _dev(rope_table, "rope_table", torch.float32), _nbytes(rope_table),
        _order(cache_post_rope), scale, _stream(stream))
    _check(st, "plamo_attn_prefill_fused_q_ragged")


def plamo_attn_decode_ragged_workspace_bytes(B: int, Hq: int, Hkv: int, window: int, max_pos_offset: int,
                                             d: int = HEAD_DIM) -> int:
    return int(_lib.load().plamo_attn_decode_ragged_workspace_bytes(B, Hq, Hkv, d, int(window),
                                                                    int(max_pos_offset)))


def plamo_attn_decode_ragged(q_rot, k_cache, v_cache, out, workspace, *, window: int, seq_pos_offsets,
                             max_pos_offset: int, rope_table, softmax_scale: float | None = None,
                             cache_post_rope: bool = False, stream=None) -> None:
    """plamo_attn_decode with one position per sequence; workspace sized by
    plamo_attn_decode_ragged_workspace_bytes."""
    dt = out.dtype
    B, T, Hq, d = q_rot.shape
    if T != 1:
        raise ValueError("decode takes one token per sequence")
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must both be [B, Hkv, cap, d]")
    if tuple(out.shape) != (B, T, Hq, d):
        raise ValueError("out must match q_rot")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    pos_p, _ = _ragged_arrays(B, seq_pos_offsets, None)
    st = _lib.load().plamo_attn_decode_ragged(
        _dtype_code(dt), _dev(q_rot, "q_rot", score_dtype(dt)), _dev(k_cache, "k_cache", dt),
        _dev(v_cache, "v_cache", dt),
        int(cap), _dev(out, "out", dt), _dev(workspace, "workspace"), ws_bytes, B, Hq, Hkv, d, int(window),
        pos_p, int(max_pos_offset), _dev(rope_table, "rope_table", torch.float32), _nbytes(rope_table),
        scale, _order(cache_post_rope), _stream(stream))
    _check(st, "plamo_attn_decode_ragged")


# ----------------------------------------------------------------------------
# the attention sublayer around the hot path: projections and norms
# ----------------------------------------------------------------------------

def plamo_linear(x, w, y, *, stream=None) -> None:
    """y[M, N] = x[M, K] w[N, K]^T (bf16); x may have leading batch axes."""
    K = x.shape[-1]
    M = x.numel() // K
    N = w.shape[0]
    if tuple(w.shape) != (N, K) or y.numel() != M * N or y.shape[-1] != N:
        raise ValueError("need x [..., K], w [N, K], y [..., N]")
    bf = torch.bfloat16
    st = _lib.load().plamo_linear(_dev(x, "x", bf), _dev(w, "w", bf), _dev(y, "y", bf), M, N, K, _stream(stream))
    _check(st, "plamo_linear")


def plamo_qkv_projection(u, w_qkv, q, k, v, *, stream=None) -> None:
    """[Q | K | V] = u w_qkv^T split into q [..., Hq, d], k, v [..., Hkv, d]; u [..., D]."""
    D = u.shape[-1]
    M = u.numel() // D
    Hq, d = q.shape[-2], q.shape[-1]
    Hkv = k.shape[-2]
    if tuple(w_qkv.shape) != ((Hq + 2 * Hkv) * d, D) or q.numel() != M * Hq * d or \
            k.numel() != M * Hkv * d or v.shape != k.shape:
        raise ValueError("need u [..., D], w_qkv [(Hq + 2 Hkv) d, D], q [..., Hq, d], k and v [..., Hkv, d]")
    bf = torch.bfloat16
    st = _lib.load().plamo_qkv_projection(_dev(u, "u", bf), _dev(w_qkv, "w_qkv", bf), _dev(q, "q", bf),
                                          _dev(k, "k", bf), _dev(v, "v", bf), M, D, Hq, Hkv, d, _stream(stream))
    _check(st, "plamo_qkv_projection")


def plamo_rms_norm(x, w, y, *, offset: float, eps: float = 1e-6, residual=None, stream=None) -> None:
    """y = residual + (offset + w) * x / rms(x) over the last axis."""
    n = x.shape[-1]
    rows = x.numel() // n
    if tuple(w.shape) != (n,) or y.shape != x.shape or (residual is not None and residual.shape != x.shape):
        raise ValueError("need x, y (and residual) of one shape and w [n]")
    dt = x.dtype
    st = _lib.load().plamo_rms_norm(_dtype_code(dt), _dev(x, "x", dt), _dev(w, "w", dt), float(offset), float(eps),
                                    _dev(residual, "residual", dt), _dev(y, "y", dt), rows, n, _stream(stream))
    _check(st, "plamo_rms_norm")
