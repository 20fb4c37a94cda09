// C-ABI entry points: argument validation, position bookkeeping and kernel dispatch.
// The declarations and their contracts live in include/plamo_attn.h.
#include "plamo_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "kernels.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* what) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", what);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return PLAMO_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kHeadDim = 128;
constexpr long long kFine = 64;
constexpr long long kPad = 128;

// Head dims with kernels: PLaMo 3's 128, and 256 / 512 (the Gemma-4-shaped layers, bf16).
bool known_head_dim(int d) { return d == 128 || d == 256 || d == 512; }

// Bytes of one rope-table row: d/2 (cos, sin) pairs.
size_t row_bytes(int d) { return static_cast<size_t>(d / 2) * 2 * sizeof(float); }

// Positions [0, covered) that a table of `bytes` bytes can rotate.
long long table_positions(size_t bytes, int d) {
  if (bytes % row_bytes(d)) return -1;
  const long long rows = static_cast<long long>(bytes / row_bytes(d));
  if (rows <= kFine) return 0;
  return (rows - kFine) * kFine;
}

// Checks shared by every attention entry point; returns PLAMO_OK or an error status.
int check_heads(int B, int T, int Hq, int Hkv, int d, int window, long long pos_offset) {
  if (B < 0 || T < 0) return fail(PLAMO_ERR_INVALID_ARG, "B and T must be >= 0");
  if (!known_head_dim(d))
    return fail(d > 0 ? PLAMO_ERR_UNSUPPORTED : PLAMO_ERR_INVALID_ARG, "head dim must be 128, 256 or 512");
  if (Hq < 1 || Hkv < 1) return fail(PLAMO_ERR_INVALID_ARG, "Hq and Hkv must be >= 1");
  if (Hq % Hkv) return fail(PLAMO_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (Hq / Hkv > 16) return fail(PLAMO_ERR_UNSUPPORTED, "Hq/Hkv must be <= 16");
  if (window < 0) return fail(PLAMO_ERR_INVALID_ARG, "window must be >= 0");
  if (pos_offset < 0) return fail(PLAMO_ERR_INVALID_ARG, "pos_offset must be >= 0");
  if (B > 65535 || Hkv > 65535) return fail(PLAMO_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  if (T > (1LL << 30)) return fail(PLAMO_ERR_UNSUPPORTED, "T must be <= 2^30");
  if (pos_offset > (1LL << 40)) return fail(PLAMO_ERR_UNSUPPORTED, "pos_offset must be <= 2^40");
  return PLAMO_OK;
}

long long kept_tokens(int window, long long pos_offset) {
  if (window == 0) return pos_offset;
  return pos_offset < window - 1 ? pos_offset : static_cast<long long>(window - 1);
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(PLAMO_ERR_HIP, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* plamo_status_str(int status) {
  switch (status) {
    case PLAMO_OK: return "ok";
    case PLAMO_ERR_INVALID_ARG: return "invalid argument";
    case PLAMO_ERR_UNSUPPORTED: return "unsupported";
    case PLAMO_ERR_WORKSPACE: return "rope table or workspace too small";
    case PLAMO_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* plamo_last_error(void) { return g_last_error; }

long long plamo_prefill_padded_len(long long S) {
  if (S <= 0 || S > (1LL << 40)) return 0;
  return (S + kPad - 1) / kPad * kPad;
}

size_t plamo_rope_table_bytes(long long max_pos, int d) {
  if (max_pos < 1 || !known_head_dim(d) || max_pos > (1LL << 40)) return 0;
  const long long coarse = (max_pos + kFine - 1) / kFine;
  return static_cast<size_t>(kFine + coarse) * row_bytes(d);
}

int plamo_rope_table_init(void* table, size_t table_bytes, long long max_pos, int d,
                          const plamo_rope* rope, void* stream) {
  if (!known_head_dim(d))
    return fail(d > 0 ? PLAMO_ERR_UNSUPPORTED : PLAMO_ERR_INVALID_ARG, "head dim must be 128, 256 or 512");
  if (max_pos < 1 || max_pos > (1LL << 40)) return fail(PLAMO_ERR_INVALID_ARG, "max_pos must be in [1, 2^40]");
  if (!table || !rope) return fail(PLAMO_ERR_INVALID_ARG, "table and rope must be non-NULL");
  if (!aligned16(table)) return fail(PLAMO_ERR_INVALID_ARG, "table must be 16-byte aligned");
  const size_t need = plamo_rope_table_bytes(max_pos, d);
  if (table_bytes < need) return fail(PLAMO_ERR_WORKSPACE, "table_bytes < plamo_rope_table_bytes(max_pos, d)");
  if (!(rope->theta > 1.0) || !std::isfinite(rope->theta)) return fail(PLAMO_ERR_INVALID_ARG, "theta must be > 1");
  double j_low = 0, j_high = 1, amp = 1.0, s = rope->yarn_factor;
  if (s > 1.0) {
    if (!std::isfinite(s) || !(rope->orig_ctx > 0) || !(rope->beta_slow > 0) ||
        !(rope->beta_fast > rope->beta_slow))
      return fail(PLAMO_ERR_INVALID_ARG, "YaRN needs orig_ctx > 0 and beta_fast > beta_slow > 0");
    // 「PLaMo 3アーキテクチャ徹底解析」 §6.3: unrounded ramp bounds, leading factor d/2
    const double half = d / 2.0, lt = std::log(rope->theta);
    j_low = half * std::log(rope->orig_ctx / (2.0 * M_PI * rope->beta_fast)) / lt;
    j_high = half * std::log(rope->orig_ctx / (2.0 * M_PI * rope->beta_slow)) / lt;
    amp = 1.0 + 0.1 * std::log(s);
  } else {
    s = 0.0;
  }
  // 「PLaMo 3アーキテクチャ徹底解析」 §6.4 (p-RoPE): floor(p d/2) pairs turn
  int n_rot = d / 2;
  const double p = rope->partial;
  if (!(p >= 0.0) || !std::isfinite(p)) return fail(PLAMO_ERR_INVALID_ARG, "partial must be >= 0");
  if (p > 0.0 && p < 1.0) {
    if (s > 1.0) return fail(PLAMO_ERR_UNSUPPORTED, "p-RoPE is not combined with YaRN");
    n_rot = static_cast<int>(std::floor(p * (d / 2)));
  }
  const long long coarse = (max_pos + kFine - 1) / kFine;
  return launched(plamo::launch_rope_table(static_cast<float2*>(table), coarse, d, rope->theta, s,
                                           j_low, j_high, amp, n_rot, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Per-sequence arrays of a ragged batch: device memory, 8- and 4-byte aligned.
int check_ragged(const long long* seq_pos, const int* seq_len) {
  if (!seq_pos) return fail(PLAMO_ERR_INVALID_ARG, "seq_pos_offsets must be non-NULL");
  if (reinterpret_cast<uintptr_t>(seq_pos) & 7u) return fail(PLAMO_ERR_INVALID_ARG, "seq_pos_offsets must be 8-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_len) & 3u) return fail(PLAMO_ERR_INVALID_ARG, "seq_lens must be 4-byte aligned");
  return PLAMO_OK;
}

// pos_offset is the batch's position (uniform) or the bound of every seq_pos entry (ragged).
int kv_append_impl(int dtype, const void* q, const void* k, const void* v, const void* q_norm_w,
                   const void* k_norm_w, float norm_offset, float norm_eps, int v_norm, void* q_out,
                   void* k_rot_out, void* v_t_out, void* k_cache, void* v_cache, long long cap,
                   int B, int T, int Hq, int Hkv, int d, int window, long long pos_offset,
                   const long long* seq_pos, const int* seq_len, const void* rope_table,
                   size_t rope_table_bytes, int cache_order, void* stream) {
  if (dtype != PLAMO_F32 && dtype != PLAMO_BF16) return fail(PLAMO_ERR_INVALID_ARG, "unknown dtype");
  if (cache_order != PLAMO_CACHE_PRE_ROPE && cache_order != PLAMO_CACHE_POST_ROPE)
    return fail(PLAMO_ERR_INVALID_ARG, "unknown cache_order");
  if (int st = check_heads(B, T, Hq, Hkv, d, window, pos_offset)) return st;
  if (d != kHeadDim && dtype != PLAMO_BF16) return fail(PLAMO_ERR_UNSUPPORTED, "head dims 256 and 512 are bf16 only");
  if (v_norm != 0 && v_norm != 1) return fail(PLAMO_ERR_INVALID_ARG, "v_norm must be 0 or 1");
  if (B == 0 || T == 0) return ok();
  if (!k || !v) return fail(PLAMO_ERR_INVALID_ARG, "k and v must be non-NULL");
  if ((q == nullptr) != (q_out == nullptr)) return fail(PLAMO_ERR_INVALID_ARG, "give q and q_out, or neither");
  if ((q_norm_w == nullptr) != (k_norm_w == nullptr))
    return fail(PLAMO_ERR_INVALID_ARG, "give both norm weights or neither");
  if ((k_cache == nullptr) != (v_cache == nullptr))
    return fail(PLAMO_ERR_INVALID_ARG, "give both caches or neither");
  const void* ptrs[] = {q, k, v, q_norm_w, k_norm_w, q_out, k_rot_out, v_t_out, k_cache, v_cache, rope_table};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (!(norm_eps >= 0.f) || !std::isfinite(norm_offset)) return fail(PLAMO_ERR_INVALID_ARG, "bad norm offset/eps");
  if (k_cache) {
    if (window > 0 && cap < window) return fail(PLAMO_ERR_INVALID_ARG, "local cache needs cap >= window");
    if (window == 0 && cap < pos_offset + T) return fail(PLAMO_ERR_INVALID_ARG, "global cache needs cap >= pos_offset + T");
  }
  const long long kept = kept_tokens(window, pos_offset);
  if (kept > 0 && (k_rot_out || v_t_out) && !k_cache)
    return fail(PLAMO_ERR_INVALID_ARG, "prefill operands after cached tokens need the caches");
  if (!rope_table) return fail(PLAMO_ERR_INVALID_ARG, "rope_table must be non-NULL");
  const long long covered = table_positions(rope_table_bytes, d);
  if (covered < 0) return fail(PLAMO_ERR_INVALID_ARG, "rope_table_bytes is not a whole number of rows");
  const bool post = cache_order == PLAMO_CACHE_POST_ROPE;
  if (!post && covered < kept + T) return fail(PLAMO_ERR_WORKSPACE, "rope table does not cover positions < kept + T");
  if (post && covered < pos_offset + T)
    return fail(PLAMO_ERR_WORKSPACE, "post-RoPE cache: rope table does not cover positions < pos_offset + T");

  plamo::AppendArgs a{};
  a.q = q; a.k = k; a.v = v; a.wq = q_norm_w; a.wk = k_norm_w;
  a.norm_offset = norm_offset; a.eps = norm_eps;
  a.q_out = q_out; a.k_rot_out = k_rot_out; a.v_t_out = v_t_out;
  a.k_cache = k_cache; a.v_cache = v_cache; a.cap = cap;
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.window = window;
  a.Tp = plamo_prefill_padded_len(kept + T);
  a.pos_offset = pos_offset; a.kept = kept;
  a.seq_pos = seq_pos; a.seq_len = seq_len;
  a.ops_kernel = (k_rot_out || v_t_out) && (kept > 0 || seq_pos || seq_len);
  a.post_rope = post;
  a.v_norm = v_norm != 0;
  a.d = d;
  a.rope = static_cast<const float2*>(rope_table);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(dtype == PLAMO_BF16 ? plamo::launch_kv_append_bf16(a, s) : plamo::launch_kv_append_f32(a, s));
}

// Steps 1 and 3 for Q done inside the prefill (plamo_attn_prefill_fused_q).
struct FusedQ {
  const void* q_norm_w;
  float norm_offset, norm_eps;
  const void* rope_table;
  size_t rope_table_bytes;
  int cache_order;
};

int attn_prefill_impl(int dtype, const void* q_rot, const void* k_rot, const void* v_t, void* out,
                      int B, int T, int Hq, int Hkv, int d, int window, long long pos_offset,
                      const long long* seq_pos, const int* seq_len, float softmax_scale, void* stream,
                      const FusedQ* fq = nullptr) {
  if (dtype != PLAMO_F32 && dtype != PLAMO_BF16) return fail(PLAMO_ERR_INVALID_ARG, "unknown dtype");
  if (int st = check_heads(B, T, Hq, Hkv, d, window, pos_offset)) return st;
  if (d != kHeadDim && dtype != PLAMO_BF16) return fail(PLAMO_ERR_UNSUPPORTED, "head dims 256 and 512 are bf16 only");
  if (B == 0 || T == 0) return ok();
  const long long kept = kept_tokens(window, pos_offset);
  if (kept + T > (1LL << 30)) return fail(PLAMO_ERR_UNSUPPORTED, "kept + T must be <= 2^30");
  // bf16 operand tiles are addressed with 32-bit buffer offsets within one (b, KV head)
  if (dtype == PLAMO_BF16 && (kept + T) * d > (1LL << 29))
    return fail(PLAMO_ERR_UNSUPPORTED, "bf16 prefill needs (kept + T) * d <= 2^29");
  if (!q_rot || !k_rot || !v_t || !out) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be non-NULL");
  const void* ptrs[] = {q_rot, k_rot, v_t, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return fail(PLAMO_ERR_INVALID_ARG, "softmax_scale must be > 0");
  if (fq) {
    if (dtype != PLAMO_BF16 || d != kHeadDim)
      return fail(PLAMO_ERR_UNSUPPORTED, "the fused-Q prefill is bf16 with d = 128");
    if (fq->cache_order != PLAMO_CACHE_PRE_ROPE && fq->cache_order != PLAMO_CACHE_POST_ROPE)
      return fail(PLAMO_ERR_INVALID_ARG, "unknown cache_order");
    if (!(fq->norm_eps >= 0.f) || !std::isfinite(fq->norm_offset))
      return fail(PLAMO_ERR_INVALID_ARG, "bad norm offset/eps");
    if (!fq->rope_table) return fail(PLAMO_ERR_INVALID_ARG, "rope_table must be non-NULL");
    if ((fq->q_norm_w && !aligned16(fq->q_norm_w)) || !aligned16(fq->rope_table))
      return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    const long long covered = table_positions(fq->rope_table_bytes, d);
    if (covered < 0) return fail(PLAMO_ERR_INVALID_ARG, "rope_table_bytes is not a whole number of rows");
    const bool post = fq->cache_order == PLAMO_CACHE_POST_ROPE;
    if (covered < (post ? pos_offset : kept) + T)
      return fail(PLAMO_ERR_WORKSPACE, "rope table does not cover the queries' positions");
  }
  const int rows_per_block = 128;  // every prefill kernel takes 128 query rows per block
  const long long blocks = (static_cast<long long>(T) + rows_per_block - 1) / rows_per_block * Hq * static_cast<long long>(B);
  if (blocks > 0x7fffffffLL) return fail(PLAMO_ERR_UNSUPPORTED, "grid too large");

  plamo::PrefillArgs a{};
  a.q_rot = q_rot; a.k_rot = k_rot; a.v_t = v_t; a.out = out;
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.window = window;
  a.Tp = plamo_prefill_padded_len(kept + T);
  a.kept = kept;
  a.pos_offset = pos_offset;
  a.seq_pos = seq_pos; a.seq_len = seq_len;
  a.scale = softmax_scale;
  a.d = d;
  if (fq) {
    a.fuse_q = true;
    a.post_rope = fq->cache_order == PLAMO_CACHE_POST_ROPE;
    a.wq = fq->q_norm_w;
    a.norm_offset = fq->norm_offset;
    a.eps = fq->norm_eps;
    a.rope = static_cast<const float2*>(fq->rope_table);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d != kHeadDim) return launched(plamo::launch_prefill_wide_bf16(a, s));
  return launched(dtype == PLAMO_BF16 ? plamo::launch_prefill_bf16(a, s) : plamo::launch_prefill_f32(a, s));
}

int attn_decode_impl(int dtype, const void* q_rot, const void* k_cache, const void* v_cache,
                     long long cap, void* out, void* workspace, size_t workspace_bytes, int B, int T,
                     int Hq, int Hkv, int d, int window, long long pos_offset, const long long* seq_pos,
                     const void* rope_table, size_t rope_table_bytes, float softmax_scale,
                     int cache_order, void* stream, bool own_scratch = false) {
  if (dtype != PLAMO_BF16) return fail(dtype == PLAMO_F32 ? PLAMO_ERR_UNSUPPORTED : PLAMO_ERR_INVALID_ARG,
                                       "decode reads a bf16 cache");
  if (T != 1) return fail(T < 0 ? PLAMO_ERR_INVALID_ARG : PLAMO_ERR_UNSUPPORTED, "decode takes T = 1");
  if (int st = check_heads(B, T, Hq, Hkv, d, window, pos_offset)) return st;
  if (cache_order != PLAMO_CACHE_PRE_ROPE && cache_order != PLAMO_CACHE_POST_ROPE)
    return fail(PLAMO_ERR_INVALID_ARG, "unknown cache_order");
  const bool post = cache_order == PLAMO_CACHE_POST_ROPE;
  if (d != kHeadDim && !post)
    return fail(PLAMO_ERR_UNSUPPORTED, "head dims 256 and 512 decode from a post-RoPE cache");
  if (B == 0) return ok();
  if (!q_rot || !k_cache || !v_cache || !out || (!rope_table && !post))
    return fail(PLAMO_ERR_INVALID_ARG, "q_rot, caches, out and rope_table must be non-NULL");
  const void* ptrs[] = {q_rot, k_cache, v_cache, out, workspace, rope_table};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (window > 0 && cap < window) return fail(PLAMO_ERR_INVALID_ARG, "local cache needs cap >= window");
  if (window == 0 && cap < pos_offset + 1) return fail(PLAMO_ERR_INVALID_ARG, "global cache needs cap >= pos_offset + 1");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return fail(PLAMO_ERR_INVALID_ARG, "softmax_scale must be > 0");
  const long long kept = kept_tokens(window, pos_offset);
  const long long S = kept + 1;
  if (!post) {  // a post-RoPE cache is read as stored: no table
    const long long covered = table_positions(rope_table_bytes, d);
    if (covered < 0) return fail(PLAMO_ERR_INVALID_ARG, "rope_table_bytes is not a whole number of rows");
    if (covered < S) return fail(PLAMO_ERR_WORKSPACE, "rope table does not cover positions < kept + 1");
  }
  const plamo::DecodePlan plan = plamo::plan_decode(B, Hkv, S, seq_pos != nullptr);
  const size_t need = plamo::decode_workspace_bytes(B, Hq, d, plan);
  if (own_scratch) {
    if (need > plamo::kDecodeScratchBytes)
      return fail(PLAMO_ERR_WORKSPACE, "split-K partials of this call exceed the 8 MiB scratch of "
                                       "plamo_attn_decode_noalloc; use plamo_attn_decode with a workspace");
  } else if (need > 0 && (!workspace || workspace_bytes < need)) {
    return fail(PLAMO_ERR_WORKSPACE, "workspace too small");
  }
  if (static_cast<long long>(B) * Hq > 0x7fffffffLL) return fail(PLAMO_ERR_UNSUPPORTED, "grid too large");
  if (own_scratch && need > 0) {
    float* ptr = nullptr;
    const hipError_t e = plamo::decode_scratch(&ptr);
    if (e != hipSuccess) return fail(PLAMO_ERR_HIP, "no device address for the decode scratch");
    workspace = ptr;
  }

  plamo::DecodeArgs a{};
  a.q_rot = q_rot; a.k_cache = k_cache; a.v_cache = v_cache; a.cap = cap; a.out = out;
  a.ws = static_cast<float*>(workspace);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.window = window;
  a.S = S; a.base = pos_offset - kept; a.plan = plan;
  a.pos_offset = pos_offset; a.seq_pos = seq_pos;
  a.post_rope = post;
  a.rope = static_cast<const float2*>(rope_table);
  a.scale = softmax_scale;
  a.d = d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(d != kHeadDim ? plamo::launch_decode_wide_bf16(a, s) : plamo::launch_decode_bf16(a, s));
}

}  // namespace

extern "C" {

int plamo_kv_append(int dtype, const void* q, const void* k, const void* v, const void* q_norm_w,
                    const void* k_norm_w, float norm_offset, float norm_eps, int v_norm, void* q_out,
                    void* k_rot_out, void* v_t_out, void* k_cache, void* v_cache, long long cap,
                    int B, int T, int Hq, int Hkv, int d, int window, long long pos_offset,
                    const void* rope_table, size_t rope_table_bytes, int cache_order, void* stream) {
  return kv_append_impl(dtype, q, k, v, q_norm_w, k_norm_w, norm_offset, norm_eps, v_norm, q_out, k_rot_out,
                        v_t_out, k_cache, v_cache, cap, B, T, Hq, Hkv, d, window, pos_offset, nullptr,
                        nullptr, rope_table, rope_table_bytes, cache_order, stream);
}

int plamo_kv_append_ragged(int dtype, const void* q, const void* k, const void* v, const void* q_norm_w,
                           const void* k_norm_w, float norm_offset, float norm_eps, int v_norm, void* q_out,
                           void* k_rot_out, void* v_t_out, void* k_cache, void* v_cache, long long cap,
                           int B, int T, int Hq, int Hkv, int d, int window,
                           const long long* seq_pos_offsets, const int* seq_lens,
                           long long max_pos_offset, const void* rope_table, size_t rope_table_bytes,
                           int cache_order, void* stream) {
  if (B > 0 && T > 0)
    if (int st = check_ragged(seq_pos_offsets, seq_lens)) return st;
  return kv_append_impl(dtype, q, k, v, q_norm_w, k_norm_w, norm_offset, norm_eps, v_norm, q_out, k_rot_out,
                        v_t_out, k_cache, v_cache, cap, B, T, Hq, Hkv, d, window, max_pos_offset,
                        seq_pos_offsets, seq_lens, rope_table, rope_table_bytes, cache_order, stream);
}

int plamo_attn_prefill(int dtype, const void* q_rot, const void* k_rot, const void* v_t, void* out,
                       int B, int T, int Hq, int Hkv, int d, int window, long long pos_offset,
                       float softmax_scale, void* stream) {
  return attn_prefill_impl(dtype, q_rot, k_rot, v_t, out, B, T, Hq, Hkv, d, window, pos_offset, nullptr,
                           nullptr, softmax_scale, stream);
}

int plamo_attn_prefill_ragged(int dtype, const void* q_rot, const void* k_rot, const void* v_t, void* out,
                              int B, int T, int Hq, int Hkv, int d, int window,
                              const long long* seq_pos_offsets, const int* seq_lens,
                              long long max_pos_offset, float softmax_scale, void* stream) {
  if (B > 0 && T > 0)
    if (int st = check_ragged(seq_pos_offsets, seq_lens)) return st;
  return attn_prefill_impl(dtype, q_rot, k_rot, v_t, out, B, T, Hq, Hkv, d, window, max_pos_offset,
                           seq_pos_offsets, seq_lens, softmax_scale, stream);
}

int plamo_attn_prefill_fused_q(int dtype, const void* q, const void* q_norm_w, float norm_offset,
                               float norm_eps, const void* k_rot, const void* v_t, void* out, int B, int T,
                               int Hq, int Hkv, int d, int window, long long pos_offset,
                               const void* rope_table, size_t rope_table_bytes, int cache_order,
                               float softmax_scale, void* stream) {
  const FusedQ fq{q_norm_w, norm_offset, norm_eps, rope_table, rope_table_bytes, cache_order};
  return attn_prefill_impl(dtype, q, k_rot, v_t, out, B, T, Hq, Hkv, d, window, pos_offset, nullptr, nullptr,
                           softmax_scale, stream, &fq);
}

int plamo_attn_prefill_fused_q_ragged(int dtype, const void* q, const void* q_norm_w, float norm_offset,
                                      float norm_eps, const void* k_rot, const void* v_t, void* out, int B,
                                      int T, int Hq, int Hkv, int d, int window,
                                      const long long* seq_pos_offsets, const int* seq_lens,
                                      long long max_pos_offset, const void* rope_table,
                                      size_t rope_table_bytes, int cache_order, float softmax_scale,
                                      void* stream) {
  if (B > 0 && T > 0)
    if (int st = check_ragged(seq_pos_offsets, seq_lens)) return st;
  const FusedQ fq{q_norm_w, norm_offset, norm_eps, rope_table, rope_table_bytes, cache_order};
  return attn_prefill_impl(dtype, q, k_rot, v_t, out, B, T, Hq, Hkv, d, window, max_pos_offset, seq_pos_offsets,
                           seq_lens, softmax_scale, stream, &fq);
}

size_t plamo_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int window, long long pos_offset) {
  if (check_heads(B, 1, Hq, Hkv, d, window, pos_offset) != PLAMO_OK) return 0;
  if (B == 0) return 0;
  const long long S = kept_tokens(window, pos_offset) + 1;
  return plamo::decode_workspace_bytes(B, Hq, d, plamo::plan_decode(B, Hkv, S, false));
}

size_t plamo_attn_decode_ragged_workspace_bytes(int B, int Hq, int Hkv, int d, int window,
                                                long long max_pos_offset) {
  if (check_heads(B, 1, Hq, Hkv, d, window, max_pos_offset) != PLAMO_OK) return 0;
  if (B == 0) return 0;
  const long long S = kept_tokens(window, max_pos_offset) + 1;
  return plamo::decode_workspace_bytes(B, Hq, d, plamo::plan_decode(B, Hkv, S, true));
}

int plamo_attn_decode(int dtype, const void* q_rot, const void* k_cache, const void* v_cache,
                      long long cap, void* out, void* workspace, size_t workspace_bytes, int B, int T,
                      int Hq, int Hkv, int d, int window, long long pos_offset,
                      const void* rope_table, size_t rope_table_bytes, float softmax_scale,
                      int cache_order, void* stream) {
  return attn_decode_impl(dtype, q_rot, k_cache, v_cache, cap, out, workspace, workspace_bytes, B, T, Hq,
                          Hkv, d, window, pos_offset, nullptr, rope_table, rope_table_bytes,
                          softmax_scale, cache_order, stream);
}

size_t plamo_decode_step_workspace_bytes(int B, int Hq, int Hkv, int d, int window, long long pos_offset) {
  if (B < 1 || Hq < 1 || Hkv < 1 || window < 0 || pos_offset < 0 || d != kHeadDim) return 0;
  const long long S = kept_tokens(window, pos_offset) + 1;
  return plamo::decode_step_workspace_bytes(B, Hq, Hkv, d, plamo::plan_decode(B, Hkv, S, false, plamo::kStepMinChunk));
}

int plamo_decode_step(int dtype, const void* q, const void* k, const void* v, const void* q_norm_w,
                      const void* k_norm_w, float norm_offset, float norm_eps, void* k_cache, void* v_cache,
                      long long cap, void* out, void* workspace, size_t workspace_bytes, int B, int Hq,
                      int Hkv, int d, int window, long long pos_offset, const void* rope_table,
                      size_t rope_table_bytes, float softmax_scale, int cache_order, void* stream) {
  if (dtype != PLAMO_BF16) return fail(dtype == PLAMO_F32 ? PLAMO_ERR_UNSUPPORTED : PLAMO_ERR_INVALID_ARG,
                                       "the decode step reads and writes a bf16 cache");
  if (int st = check_heads(B, 1, Hq, Hkv, d, window, pos_offset)) return st;
  if (d != kHeadDim) return fail(PLAMO_ERR_UNSUPPORTED, "the one-launch decode step is for d = 128");
  if (cache_order != PLAMO_CACHE_PRE_ROPE && cache_order != PLAMO_CACHE_POST_ROPE)
    return fail(PLAMO_ERR_INVALID_ARG, "unknown cache_order");
  if (B == 0) return ok();
  if (!q || !k || !v || !k_cache || !v_cache || !out || !rope_table)
    return fail(PLAMO_ERR_INVALID_ARG, "q, k, v, caches, out and rope_table must be non-NULL");
  if ((q_norm_w == nullptr) != (k_norm_w == nullptr))
    return fail(PLAMO_ERR_INVALID_ARG, "give both norm weights or neither");
  const void* ptrs[] = {q, k, v, q_norm_w, k_norm_w, k_cache, v_cache, out, workspace, rope_table};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (!(norm_eps >= 0.f) || !std::isfinite(norm_offset)) return fail(PLAMO_ERR_INVALID_ARG, "bad norm offset/eps");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return fail(PLAMO_ERR_INVALID_ARG, "softmax_scale must be > 0");
  if (window > 0 && cap < window) return fail(PLAMO_ERR_INVALID_ARG, "local cache needs cap >= window");
  if (window == 0 && cap < pos_offset + 1) return fail(PLAMO_ERR_INVALID_ARG, "global cache needs cap >= pos_offset + 1");
  const long long kept = kept_tokens(window, pos_offset);
  const long long S = kept + 1;
  const bool post = cache_order == PLAMO_CACHE_POST_ROPE;
  const long long covered = table_positions(rope_table_bytes, d);
  if (covered < 0) return fail(PLAMO_ERR_INVALID_ARG, "rope_table_bytes is not a whole number of rows");
  if (covered < (post ? pos_offset + 1 : S)) return fail(PLAMO_ERR_WORKSPACE, "rope table does not cover the positions");
  const plamo::DecodePlan plan = plamo::plan_decode(B, Hkv, S, false, plamo::kStepMinChunk);
  const size_t need = plamo::decode_step_workspace_bytes(B, Hq, Hkv, d, plan);
  if (need > 0 && (!workspace || workspace_bytes < need)) return fail(PLAMO_ERR_WORKSPACE, "workspace too small");
  if (static_cast<long long>(B) * Hq > 0x7fffffffLL) return fail(PLAMO_ERR_UNSUPPORTED, "grid too large");

  plamo::DecodeArgs a{};
  a.k_cache = k_cache; a.v_cache = v_cache; a.cap = cap; a.out = out;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.window = window;
  a.S = S; a.base = pos_offset - kept; a.plan = plan;
  a.pos_offset = pos_offset;
  a.post_rope = post;
  a.rope = static_cast<const float2*>(rope_table);
  a.scale = softmax_scale;
  a.d = d;
  a.fused = true;
  a.q_in = q; a.k_in = k; a.v_in = v; a.wq = q_norm_w; a.wk = k_norm_w;
  a.norm_offset = norm_offset; a.eps = norm_eps;
  if (need > 0) {
    a.tickets = static_cast<unsigned*>(workspace);
    a.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + plamo::decode_step_tickets_bytes(B, Hkv));
  }
  return launched(plamo::launch_decode_bf16(a, static_cast<hipStream_t>(stream)));
}

int plamo_prefill_pack(int dtype, const void* k_rot, const void* v, void* k_rot_out, void* v_t_out, int B,
                       long long S, int Hkv, int d, void* stream) {
  if (dtype != PLAMO_F32 && dtype != PLAMO_BF16) return fail(PLAMO_ERR_INVALID_ARG, "unknown dtype");
  if (B < 0 || S < 0 || Hkv < 1) return fail(PLAMO_ERR_INVALID_ARG, "need B >= 0, S >= 0, Hkv >= 1");
  if (!known_head_dim(d)) return fail(PLAMO_ERR_UNSUPPORTED, "head dim must be 128, 256 or 512");
  if (d != kHeadDim && dtype != PLAMO_BF16) return fail(PLAMO_ERR_UNSUPPORTED, "head dims 256 and 512 are bf16 only");
  if (S > (1LL << 40)) return fail(PLAMO_ERR_UNSUPPORTED, "S must be <= 2^40");
  if (B == 0 || S == 0) return ok();
  if (!k_rot || !v || !k_rot_out || !v_t_out) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be non-NULL");
  const void* ptrs[] = {k_rot, v, k_rot_out, v_t_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  const long long Tp = plamo_prefill_padded_len(S);
  if (Tp / 64 > 0x7fffffffLL || static_cast<long long>(B) * Hkv > 65535LL * 65535LL || B > 65535 || Hkv > 65535)
    return fail(PLAMO_ERR_UNSUPPORTED, "grid too large");
  plamo::PackArgs a{};
  a.k = k_rot; a.v = v; a.k_rot_out = k_rot_out; a.v_t_out = v_t_out;
  a.B = B; a.Hkv = Hkv; a.d = d; a.S = S; a.Tp = Tp;
  return launched(plamo::launch_prefill_pack(a, dtype == PLAMO_BF16, static_cast<hipStream_t>(stream)));
}

static_assert(plamo::kDecodeScratchBytes == PLAMO_DECODE_SCRATCH_BYTES, "scratch size as declared");

int plamo_attn_decode_noalloc(int dtype, const void* q_rot, const void* k_cache, const void* v_cache,
                              long long cap, void* out, int B, int T, int Hq, int Hkv, int d, int window,
                              long long pos_offset, const void* rope_table, size_t rope_table_bytes,
                              float softmax_scale, int cache_order, void* stream) {
  return attn_decode_impl(dtype, q_rot, k_cache, v_cache, cap, out, nullptr, 0, B, T, Hq, Hkv, d, window,
                          pos_offset, nullptr, rope_table, rope_table_bytes, softmax_scale, cache_order,
                          stream, true);
}

int plamo_attn_decode_ragged(int dtype, const void* q_rot, const void* k_cache, const void* v_cache,
                             long long cap, void* out, void* workspace, size_t workspace_bytes, int B,
                             int Hq, int Hkv, int d, int window, const long long* seq_pos_offsets,
                             long long max_pos_offset, const void* rope_table, size_t rope_table_bytes,
                             float softmax_scale, int cache_order, void* stream) {
  if (B > 0)
    if (int st = check_ragged(seq_pos_offsets, nullptr)) return st;
  return attn_decode_impl(dtype, q_rot, k_cache, v_cache, cap, out, workspace, workspace_bytes, B, 1, Hq,
                          Hkv, d, window, max_pos_offset, seq_pos_offsets, rope_table, rope_table_bytes,
                          softmax_scale, cache_order, stream);
}

/* ---- the sublayer around attention: projections and norms ---------------------- */

int plamo_linear(const void* x, const void* w, void* y, long long M, int N, int K, void* stream) {
  if (M < 0 || N < 1 || K < 1) return fail(PLAMO_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1");
  if (N % 8 || K % 64) return fail(PLAMO_ERR_UNSUPPORTED, "need N % 8 == 0 and K % 64 == 0");
  if (M > 65535LL * 256 || static_cast<long long>(K) * 256 * 2 > 0x7fffffffLL)
    return fail(PLAMO_ERR_UNSUPPORTED, "M or K too large");
  if (M == 0) return ok();
  if (!x || !w || !y) return fail(PLAMO_ERR_INVALID_ARG, "x, w and y must be non-NULL");
  const void* ptrs[] = {x, w, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  plamo::GemmArgs a;
  a.x = x; a.w = w; a.M = M; a.N = N; a.K = K;
  a.y[0] = a.y[1] = a.y[2] = y;
  a.part_end[0] = a.part_end[1] = a.part_end[2] = N;
  return launched(plamo::launch_gemm_bf16(a, static_cast<hipStream_t>(stream)));
}

int plamo_qkv_projection(const void* u, const void* w_qkv, void* q, void* k, void* v, long long M, int D,
                         int Hq, int Hkv, int d, void* stream) {
  if (M < 0 || D < 1 || Hq < 1 || Hkv < 1 || d < 1) return fail(PLAMO_ERR_INVALID_ARG, "bad sizes");
  if (D % 64 || d % 8) return fail(PLAMO_ERR_UNSUPPORTED, "need D % 64 == 0 and d % 8 == 0");
  const long long N = (static_cast<long long>(Hq) + 2LL * Hkv) * d;
  if (M > 65535LL * 256 || N > (1LL << 30) || static_cast<long long>(D) * 256 * 2 > 0x7fffffffLL)
    return fail(PLAMO_ERR_UNSUPPORTED, "sizes too large");
  if (M == 0) return ok();
  if (!u || !w_qkv || !q || !k || !v) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be non-NULL");
  const void* ptrs[] = {u, w_qkv, q, k, v};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  plamo::GemmArgs a;
  a.x = u; a.w = w_qkv; a.M = M; a.N = N; a.K = D;
  a.y[0] = q; a.y[1] = k; a.y[2] = v;
  a.part_end[0] = static_cast<long long>(Hq) * d;
  a.part_end[1] = (static_cast<long long>(Hq) + Hkv) * d;
  a.part_end[2] = N;
  return launched(plamo::launch_gemm_bf16(a, static_cast<hipStream_t>(stream)));
}

int plamo_rms_norm(int dtype, const void* x, const void* w, float offset, float eps, const void* residual,
                   void* y, long long rows, int n, void* stream) {
  if (dtype != PLAMO_F32 && dtype != PLAMO_BF16) return fail(PLAMO_ERR_INVALID_ARG, "unknown dtype");
  if (rows < 0 || n < 1) return fail(PLAMO_ERR_INVALID_ARG, "need rows >= 0 and n >= 1");
  if (n % (dtype == PLAMO_BF16 ? 8 : 4)) return fail(PLAMO_ERR_UNSUPPORTED, "n must fill 16-byte chunks");
  if (rows > (1LL << 33)) return fail(PLAMO_ERR_UNSUPPORTED, "too many rows");
  if (!(eps >= 0.f) || !std::isfinite(offset)) return fail(PLAMO_ERR_INVALID_ARG, "bad offset/eps");
  if (rows == 0) return ok();
  if (!x || !w || !y) return fail(PLAMO_ERR_INVALID_ARG, "x, w and y must be non-NULL");
  const void* ptrs[] = {x, w, y, residual};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(PLAMO_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  plamo::NormArgs a;
  a.x = x; a.w = w; a.residual = residual; a.y = y; a.rows = rows; a.n = n; a.offset = offset; a.eps = eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launched(dtype == PLAMO_BF16 ? plamo::launch_rms_norm_bf16(a, s) : plamo::launch_rms_norm_f32(a, s));
}

}  // extern "C"
