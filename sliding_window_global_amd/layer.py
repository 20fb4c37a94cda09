"""One attention layer step on the GPU, composed from the C-ABI calls.

Allocation of outputs and scratch uses torch (device memory only); every step of the
computation is a kernel of the library: plamo_kv_append (norm, cache update, RoPE,
prefill operands) followed by plamo_attn_prefill or plamo_attn_decode.
"""

from __future__ import annotations

import math

import torch

from dataclasses import dataclass

from . import (plamo_attn_decode, plamo_attn_decode_ragged, plamo_attn_decode_ragged_workspace_bytes,
               plamo_decode_step, plamo_decode_step_workspace_bytes,
               plamo_attn_decode_workspace_bytes, plamo_attn_prefill, plamo_attn_prefill_fused_q,
               plamo_attn_prefill_fused_q_ragged, plamo_attn_prefill_ragged, plamo_kv_append,
               plamo_kv_append_ragged, plamo_linear, plamo_qkv_projection, plamo_rms_norm,
               prefill_operand_shapes, score_dtype)


class PrefillBuffers:
    """Operands of one prefill chunk: normalised/rotated Q, rotated K and transposed V of the
    kept + T keys it attends (Q' and K' in score_dtype: fp16 on a bf16 layer)."""

    def __init__(self, B, T, Hq, Hkv, d, dtype, device="cuda", window=0, pos_offset=0):
        k_shape, v_shape = prefill_operand_shapes(B, T, Hkv, d, dtype, window, pos_offset)
        self.q_rot = torch.empty((B, T, Hq, d), dtype=score_dtype(dtype), device=device)
        self.k_rot = torch.empty(k_shape, dtype=score_dtype(dtype), device=device)
        self.v_t = torch.empty(v_shape, dtype=dtype, device=device)
        self.out = torch.empty((B, T, Hq, d), dtype=dtype, device=device)


def prefill(q, k, v, *, window, rope_table, q_norm_w=None, k_norm_w=None, norm_offset=1.0,
            norm_eps=1e-6, k_cache=None, v_cache=None, bufs: PrefillBuffers | None = None,
            softmax_scale=None, stream=None, pos_offset=0, cache_post_rope=False, v_norm=False,
            fuse_q=False) -> PrefillBuffers:
    """Prefill of a chunk q [B,T,Hq,d], k/v [B,T,Hkv,d] on the GPU whose first token sits at
    absolute position pos_offset. With pos_offset > 0 the caches must hold the earlier tokens
    (they are read for the chunk's attention, then updated with the chunk). v_norm: V divided
    by its RMS per head vector (the Gemma-4-shaped layer). fuse_q (bf16, d = 128): the append
    handles K and V only and the prefill kernel normalises and rotates Q itself."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if bufs is None:
        bufs = PrefillBuffers(B, T, Hq, Hkv, d, q.dtype, q.device, window, pos_offset)
    if fuse_q:
        plamo_kv_append(None, k, v, None, window=window, pos_offset=pos_offset, rope_table=rope_table,
                        q_norm_w=q_norm_w, k_norm_w=k_norm_w, norm_offset=norm_offset, norm_eps=norm_eps,
                        k_rot_out=bufs.k_rot, v_t_out=bufs.v_t, k_cache=k_cache, v_cache=v_cache,
                        cache_post_rope=cache_post_rope, v_norm=v_norm, stream=stream)
        plamo_attn_prefill_fused_q(q, bufs.k_rot, bufs.v_t, bufs.out, window=window, rope_table=rope_table,
                                   pos_offset=pos_offset, q_norm_w=q_norm_w, norm_offset=norm_offset,
                                   norm_eps=norm_eps, cache_post_rope=cache_post_rope,
                                   softmax_scale=softmax_scale, stream=stream)
        return bufs
    plamo_kv_append(q, k, v, bufs.q_rot, window=window, pos_offset=pos_offset, rope_table=rope_table,
                    q_norm_w=q_norm_w, k_norm_w=k_norm_w, norm_offset=norm_offset, norm_eps=norm_eps,
                    k_rot_out=bufs.k_rot, v_t_out=bufs.v_t, k_cache=k_cache, v_cache=v_cache,
                    cache_post_rope=cache_post_rope, v_norm=v_norm, stream=stream)
    plamo_attn_prefill(bufs.q_rot, bufs.k_rot, bufs.v_t, bufs.out, window=window, pos_offset=pos_offset,
                       softmax_scale=softmax_scale, stream=stream)
    return bufs


class DecodeBuffers:
    """Q', output and split workspace of one decode step (ragged: sized for a ragged batch
    whose positions are at most pos_offset)."""

    def __init__(self, B, Hq, Hkv, d, window, pos_offset, dtype=torch.bfloat16, device="cuda", ragged=False,
                 fused=False):
        self.q_rot = torch.empty((B, 1, Hq, d), dtype=score_dtype(dtype), device=device)
        self.out = torch.empty((B, 1, Hq, d), dtype=dtype, device=device)
        size = plamo_attn_decode_ragged_workspace_bytes if ragged else plamo_attn_decode_workspace_bytes
        nbytes = size(B, Hq, Hkv, window, pos_offset, d)
        self.workspace = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=device)
        # the one-launch step's workspace: zeroed once (its counters stay zero between calls)
        self.step_workspace = None
        if fused:
            nb = plamo_decode_step_workspace_bytes(B, Hq, Hkv, window, pos_offset, d)
            self.step_workspace = torch.zeros(max(1, (nb + 3) // 4), dtype=torch.float32, device=device)


def decode(q, k, v, k_cache, v_cache, *, window, pos_offset, rope_table, q_norm_w=None,
           k_norm_w=None, norm_offset=1.0, norm_eps=1e-6, bufs: DecodeBuffers | None = None,
           softmax_scale=None, stream=None, cache_post_rope=False, v_norm=False, fused=False) -> DecodeBuffers:
    """One decode step at absolute position pos_offset: q [B,1,Hq,d], k/v [B,1,Hkv,d]. fused
    (d = 128, no v_norm): one launch, plamo_decode_step, instead of the append and the decode."""
    B, _, Hq, d = q.shape
    Hkv = k.shape[2]
    if bufs is None:
        bufs = DecodeBuffers(B, Hq, Hkv, d, window, pos_offset, q.dtype, q.device, fused=fused)
    if fused:
        if v_norm:
            raise ValueError("the one-launch step takes V as given")
        plamo_decode_step(q, k, v, k_cache, v_cache, bufs.out, bufs.step_workspace, window=window,
                          pos_offset=pos_offset, rope_table=rope_table, q_norm_w=q_norm_w, k_norm_w=k_norm_w,
                          norm_offset=norm_offset, norm_eps=norm_eps, softmax_scale=softmax_scale,
                          cache_post_rope=cache_post_rope, stream=stream)
        return bufs
    plamo_kv_append(q, k, v, bufs.q_rot, window=window, pos_offset=pos_offset, rope_table=rope_table,
                    q_norm_w=q_norm_w, k_norm_w=k_norm_w, norm_offset=norm_offset, norm_eps=norm_eps,
                    k_cache=k_cache, v_cache=v_cache, cache_post_rope=cache_post_rope, v_norm=v_norm,
                    stream=stream)
    plamo_attn_decode(bufs.q_rot, k_cache, v_cache, bufs.out, bufs.workspace, window=window,
                      pos_offset=pos_offset, rope_table=rope_table,
                      softmax_scale=1.0 / math.sqrt(d) if softmax_scale is None else softmax_scale,
                      cache_post_rope=cache_post_rope, stream=stream)
    return bufs


def prefill_ragged(q, k, v, *, window, rope_table, seq_pos_offsets, max_pos_offset, seq_lens=None,
                   q_norm_w=None, k_norm_w=None, norm_offset=1.0, norm_eps=1e-6, k_cache=None,
                   v_cache=None, bufs: PrefillBuffers | None = None, softmax_scale=None,
                   stream=None, cache_post_rope=False, v_norm=False, fuse_q=False) -> PrefillBuffers:
    """Prefill of a ragged batch: sequence b's seq_lens[b] new tokens (rows of its [T] slab)
    start at absolute position seq_pos_offsets[b] <= max_pos_offset."""
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if bufs is None:
        bufs = PrefillBuffers(B, T, Hq, Hkv, d, q.dtype, q.device, window, max_pos_offset)
    if fuse_q:
        plamo_kv_append_ragged(None, k, v, None, window=window, seq_pos_offsets=seq_pos_offsets,
                               max_pos_offset=max_pos_offset, seq_lens=seq_lens, rope_table=rope_table,
                               q_norm_w=q_norm_w, k_norm_w=k_norm_w, norm_offset=norm_offset, norm_eps=norm_eps,
                               k_rot_out=bufs.k_rot, v_t_out=bufs.v_t, k_cache=k_cache, v_cache=v_cache,
                               cache_post_rope=cache_post_rope, v_norm=v_norm, stream=stream)
        plamo_attn_prefill_fused_q_ragged(q, bufs.k_rot, bufs.v_t, bufs.out, window=window,
                                          seq_pos_offsets=seq_pos_offsets, max_pos_offset=max_pos_offset,
                                          rope_table=rope_table, seq_lens=seq_lens, q_norm_w=q_norm_w,
                                          norm_offset=norm_offset, norm_eps=norm_eps,
                                          cache_post_rope=cache_post_rope, softmax_scale=softmax_scale,
                                          stream=stream)
        return bufs
    plamo_kv_append_ragged(q, k, v, bufs.q_rot, window=window, seq_pos_offsets=seq_pos_offsets,
                           max_pos_offset=max_pos_offset, seq_lens=seq_lens, rope_table=rope_table,
                           q_norm_w=q_norm_w, k_norm_w=k_norm_w, norm_offset=norm_offset, norm_eps=norm_eps,
                           k_rot_out=bufs.k_rot, v_t_out=bufs.v_t, k_cache=k_cache, v_cache=v_cache,
                           cache_post_rope=cache_post_rope, v_norm=v_norm, stream=stream)
    plamo_attn_prefill_ragged(bufs.q_rot, bufs.k_rot, bufs.v_t, bufs.out, window=window,
                              seq_pos_offsets=seq_pos_offsets, max_pos_offset=max_pos_offset,
                              seq_lens=seq_lens, softmax_scale=softmax_scale, stream=stream)
    return bufs


def decode_ragged(q, k, v, k_cache, v_cache, *, window, seq_pos_offsets, max_pos_offset, rope_table,
                  q_norm_w=None, k_norm_w=None, norm_offset=1.0, norm_eps=1e-6,
                  bufs: DecodeBuffers | None = None, softmax_scale=None, stream=None,
                  cache_post_rope=False, v_norm=False) -> DecodeBuffers:
    """One decode step of a ragged batch: sequence b's new token sits at seq_pos_offsets[b]."""
    B, _, Hq, d = q.shape
    Hkv = k.shape[2]
    if bufs is None:
        bufs = DecodeBuffers(B, Hq, Hkv, d, window, max_pos_offset, q.dtype, q.device, ragged=True)
    plamo_kv_append_ragged(q, k, v, bufs.q_rot, window=window, seq_pos_offsets=seq_pos_offsets,
                           max_pos_offset=max_pos_offset, rope_table=rope_table, q_norm_w=q_norm_w,
                           k_norm_w=k_norm_w, norm_offset=norm_offset, norm_eps=norm_eps, k_cache=k_cache,
                           v_cache=v_cache, cache_post_rope=cache_post_rope, v_norm=v_norm, stream=stream)
    plamo_attn_decode_ragged(bufs.q_rot, k_cache, v_cache, bufs.out, bufs.workspace, window=window,
                             seq_pos_offsets=seq_pos_offsets, max_pos_offset=max_pos_offset,
                             rope_table=rope_table, softmax_scale=softmax_scale,
                             cache_post_rope=cache_post_rope, stream=stream)
    return bufs


# ----------------------------------------------------------------------------
# the attention sublayer: x -> x + post_norm(o_proj(attention(qkv_proj(pre_norm(x)))))
# ----------------------------------------------------------------------------

@dataclass
class MixerWeights:
    """Weights of one attention sublayer (bf16 GPU tensors): pre/post norm weights [D], the
    fused projection w_qkv [(Hq + 2 Hkv) d, D], the output projection w_o [D, Hq d] and the
    per-head Q/K norm weights [d]."""
    w_pre: torch.Tensor
    w_qkv: torch.Tensor
    w_o: torch.Tensor
    w_post: torch.Tensor
    wq: torch.Tensor
    wk: torch.Tensor
    Hq: int
    Hkv: int
    d: int = 128
    pre_offset: float = 1.0
    post_offset: float = 0.2
    qk_offset: float = 1.0



class MixerBuffers:
    def __init__(self, B, T, D, wts: MixerWeights, device="cuda"):
        bf = torch.bfloat16
        self.u = torch.empty((B, T, D), dtype=bf, device=device)
        self.q = torch.empty((B, T, wts.Hq, wts.d), dtype=bf, device=device)
        self.k = torch.empty((B, T, wts.Hkv, wts.d), dtype=bf, device=device)
        self.v = torch.empty((B, T, wts.Hkv, wts.d), dtype=bf, device=device)
        self.p = torch.empty((B, T, D), dtype=bf, device=device)
        self.out = torch.empty((B, T, D), dtype=bf, device=device)


def _mixer_in(x, wts, bufs, stream):
    plamo_rms_norm(x, wts.w_pre, bufs.u, offset=wts.pre_offset, stream=stream)
    plamo_qkv_projection(bufs.u, wts.w_qkv, bufs.q, bufs.k, bufs.v, stream=stream)


def _mixer_out(x, attn_out, wts, bufs, stream):
    plamo_linear(attn_out.view(*attn_out.shape[:2], -1), wts.w_o, bufs.p, stream=stream)  # heads concatenated
    plamo_rms_norm(bufs.p, wts.w_post, bufs.out, offset=wts.post_offset, residual=x, stream=stream)


def mixer_prefill(x, wts: MixerWeights, *, window, rope_table, k_cache=None, v_cache=None,
                  pos_offset=0, bufs: MixerBuffers | None = None, attn_bufs: PrefillBuffers | None = None,
                  stream=None, fuse_q: bool | None = None):
    """The attention sublayer over a chunk x [B, T, D] at pos_offset; returns (bufs, attn_bufs),
    the new residual stream in bufs.out. fuse_q (default: wherever the fused-Q prefill applies,
    bf16 at d = 128): the attention kernel normalises and rotates the projected queries itself,
    so Q' never goes through HBM."""
    B, T, D = x.shape
    bufs = bufs or MixerBuffers(B, T, D, wts, x.device)
    _mixer_in(x, wts, bufs, stream)
    if fuse_q is None:
        fuse_q = bufs.q.dtype == torch.bfloat16 and bufs.q.shape[-1] == 128
    attn_bufs = prefill(bufs.q, bufs.k, bufs.v, window=window, rope_table=rope_table, q_norm_w=wts.wq,
                        k_norm_w=wts.wk, norm_offset=wts.qk_offset, k_cache=k_cache, v_cache=v_cache,
                        bufs=attn_bufs, stream=stream, pos_offset=pos_offset, fuse_q=fuse_q)
    _mixer_out(x, attn_bufs.out, wts, bufs, stream)
    return bufs, attn_bufs


def mixer_decode(x, wts: MixerWeights, k_cache, v_cache, *, window, pos_offset, rope_table,
                 bufs: MixerBuffers | None = None, attn_bufs: DecodeBuffers | None = None, stream=None):
    """One decode step of the attention sublayer: x [B, 1, D]; returns (bufs, attn_bufs)."""
    B, _, D = x.shape
    bufs = bufs or MixerBuffers(B, 1, D, wts, x.device)
    _mixer_in(x, wts, bufs, stream)
    attn_bufs = decode(bufs.q, bufs.k, bufs.v, k_cache, v_cache, window=window, pos_offset=pos_offset,
                       rope_table=rope_table, q_norm_w=wts.wq, k_norm_w=wts.wk, norm_offset=wts.qk_offset,
                       bufs=attn_bufs, stream=stream)
    _mixer_out(x, attn_bufs.out, wts, bufs, stream)
    return bufs, attn_bufs
