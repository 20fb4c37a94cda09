/*
 * plamo_attn.h -- C ABI of the MI355X (gfx950) implementation of PLaMo 3's hybrid
 * sliding-window / global grouped-query attention, prefill and KV-cached decode.
 *
 * Sources (page title, section):
 *   [P3] 「PLaMo 3アーキテクチャ徹底解析」 (imoz.jp, 2026-10-26)
 *
 * What one attention layer computes, in this order [P3 §4.4]:
 *   1. per-head RMSNorm of Q and K with gain (c + w) [P3 §3.2, §4.3]; V untouched;
 *   2. KV-cache update: the cache stores normalised K *before* RoPE and raw V
 *      [P3 §4.4]; a global layer keeps every token, a local layer keeps at most the
 *      last W-1 tokens after the update [P3 §4.4];
 *   3. split-half RoPE (pairs j, j+d/2) [P3 §6.1] on the current Q and on every K
 *      the cache returns, with YaRN frequencies and amplitude on global layers
 *      [P3 §6.3]; positions are renumbered: the S returned keys get 0..S-1 and the
 *      T queries S-T..S-1 [P3 §4.4];
 *   4. softmax(Q'K'^T * scale + M) V with the causal mask, plus i - j < W on local
 *      layers [P3 §4.5, §5.1]; query head h reads KV head h / (Hq/Hkv) [P3 §4.2].
 *
 * Conventions for every entry point
 *   - Pointers are device memory owned by the caller unless stated otherwise. The
 *     library never allocates or frees device memory; decode scratch comes in as
 *     a caller-provided workspace.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Nothing synchronises; buffers must stay alive until the stream has run it.
 *   - Arguments are checked before anything is launched; on failure the call
 *     returns a negative plamo_status and enqueues nothing. A launch error is
 *     reported as PLAMO_ERR_HIP. No C++ exception crosses this boundary.
 *   - dtype PLAMO_BF16: bf16 tensors, fp32 arithmetic inside, except the two score
 *     operands Q' (q_out / q_rot) and K' (k_rot_out / k_rot), which are IEEE half (fp16):
 *     each is rounded once from its fp32 normalised and rotated value, and the score
 *     product runs on fp16 MFMA (same rate as bf16, three more mantissa bits; V, P and the
 *     outputs stay bf16). Range: these operands are RMS-normalised, so with the norm they
 *     stay inside the half range for gains |c + w_r| <= 512 at any head dim and RoPE
 *     amplitude here; without the norm the inputs must satisfy |q|, |k| <= 8192 (not
 *     checked: a larger value would overflow to inf). PLAMO_F32: fp32 tensors and
 *     arithmetic (prefill path only).
 *   - Head dimension d is 128 (PLaMo 3's head_dim [P3 §2.1]), or 256 / 512 for the
 *     Gemma-4-shaped layers the page compares it with [P3 §8 table] (bf16 only; decode
 *     then needs a post-RoPE cache). Hq must be a multiple of Hkv and Hq/Hkv <= 16.
 *   - Positions are 64-bit; one pos_offset serves every sequence of the batch
 *     (the *_ragged calls take one position per sequence).
 *   - Entry points hold no mutable global state and may be called from several
 *     host threads on different streams (except plamo_attn_decode_noalloc, whose
 *     per-GPU scratch is shared by all its calls on that GPU).
 */
#ifndef PLAMO_ATTN_H
#define PLAMO_ATTN_H

#include <stddef.h>

#if defined(__GNUC__)
#define PLAMO_API __attribute__((visibility("default")))
#else
#define PLAMO_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PLAMO_OK = 0,
  PLAMO_ERR_INVALID_ARG = -1, /* shape, pointer, alignment or size mismatch */
  PLAMO_ERR_UNSUPPORTED = -2, /* valid per the method, not implemented here */
  PLAMO_ERR_WORKSPACE = -3,   /* rope table or workspace too small */
  PLAMO_ERR_HIP = -4          /* the HIP runtime reported an error at launch */
} plamo_status;

typedef enum { PLAMO_F32 = 0, PLAMO_BF16 = 1 } plamo_dtype;

/* What the K cache holds [P3 §4.4]. PRE_ROPE is PLaMo 3's order: normalised K before
 * RoPE, rotated at renumbered positions 0..S-1 every time the cache returns it.
 * POST_ROPE is the other order the page contrasts it with (the Gemma-style layer, for
 * engines whose caches hold rotated K): K rotated at its absolute position before it is
 * stored, queries rotated at their absolute positions, the cache read as stored. Both
 * give the same attention up to rounding; the rope table must then cover absolute
 * positions < pos_offset + T, and decode needs no table. A cache is written and read in
 * one order only. */
typedef enum { PLAMO_CACHE_PRE_ROPE = 0, PLAMO_CACHE_POST_ROPE = 1 } plamo_cache_order;

/* RoPE parameters of one layer type [P3 §2.1, §6.2, §6.3, §6.4].
 * PLaMo 3: local layers theta = 1e4, no YaRN; global layers theta = 1e6 with YaRN.
 * Gemma-4-shaped global layer: theta = 1e6, p-RoPE with partial = 0.25. */
typedef struct {
  double theta;       /* RoPE base */
  double yarn_factor; /* YaRN factor s; <= 1 disables YaRN (amplitude 1) */
  double orig_ctx;    /* YaRN original context L0 (4096) */
  double beta_fast;   /* 32 */
  double beta_slow;   /* 1 */
  double partial;     /* p-RoPE [P3 §6.4]: with 0 < p < 1 only the floor(p d/2)
                         highest-frequency pairs turn (exponent still over d), the others
                         keep frequency 0; 0 or >= 1 = every pair turns. Not with YaRN
                         (PLAMO_ERR_UNSUPPORTED). */
} plamo_rope;

/* ---------------------------------------------------------------------------
 * RoPE table [P3 §6.1, §6.3]
 *
 * Opaque device table of rotation factors for positions 0 .. max_pos-1 and the
 * d/2 pairs, built in fp64 and stored as fp32 (cos, sin) pairs, the YaRN
 * amplitude included. One table serves one layer type; a table built for
 * max_pos covers every position below it.
 * ------------------------------------------------------------------------- */

/* Bytes needed for a table covering positions [0, max_pos). 0 on bad arguments. */
PLAMO_API size_t plamo_rope_table_bytes(long long max_pos, int d);

/* Fill `table` (device, `table_bytes` >= plamo_rope_table_bytes(max_pos, d)). */
PLAMO_API int plamo_rope_table_init(void* table, size_t table_bytes, long long max_pos, int d,
                          const plamo_rope* rope, void* stream);

/* Padded key count used by the prefill operand layouts: S rounded up to 128, where a
 * chunk of T tokens after `kept` cached ones (below) attends S = kept + T keys. Returns 0
 * for S <= 0 and for S > 2^40 (beyond any position the rope table covers). */
PLAMO_API long long plamo_prefill_padded_len(long long S);

/* ---------------------------------------------------------------------------
 * plamo_kv_append -- steps 1-3 for T new tokens of B sequences [P3 §4.3, §4.4, §6]
 *
 * The new tokens have absolute positions pos_offset .. pos_offset+T-1. kept =
 * pos_offset (global, window = 0) or min(pos_offset, window-1) (local); their
 * renumbered positions are kept .. kept+T-1.
 *
 * q        [B, T, Hq,  d]  projected queries                     (dtype)
 * k, v     [B, T, Hkv, d]  projected keys and values             (dtype)
 * q_norm_w, k_norm_w [d]   stored norm weights w (gain c + w); both NULL = no norm
 * norm_offset, norm_eps    c (1 for q_norm/k_norm [P3 §3.2]; 0 where the gain is the
 *                          weight itself, the Gemma-4-shaped layer [P3 §8]) and eps (1e-6)
 * v_norm   1 = divide each new V head vector by its RMS (eps norm_eps, no gain) before it
 *          is cached or used (the Gemma-4-shaped layer [P3 §8 table]); 0 = V as given.
 *          k and v may be the same buffer (that layer's global K = V projection).
 * q_out    [B, T, Hq, d]   normalised and rotated Q (fp16 for PLAMO_BF16, fp32 for
 *                          PLAMO_F32). q and q_out both NULL: the queries are left to
 *                          plamo_attn_prefill_fused_q.
 * k_rot_out rotated K of the S = kept + T keys the chunk attends, Tp =
 *                          plamo_prefill_padded_len(S) rows per (b, KV head): rows
 *                          0..kept-1 the cached (pre-RoPE) keys read from k_cache before
 *                          this call updates it, rotated at renumbered positions
 *                          0..kept-1; rows kept..S-1 the new tokens (normalised and
 *                          rotated in fp32, rounded once); rows S..Tp-1 zero. NULL = not
 *                          written. (Prefill operand.) With kept > 0 the caches must be
 *                          given. Layout per (b, KV head):
 *                            PLAMO_F32: fp32 [Tp][d];
 *                            PLAMO_BF16: fp16, Tp/64 tiles of 64 tokens, tile = [d/8][64][8]
 *                                  (dim / 8, token in tile, dim % 8), 128 d bytes.
 * v_t_out  V of the same S keys (cached, then new) transposed, pad zeroed. NULL = not
 *                          written. (Prefill operand.) Layout
 *                          per (b, KV head):
 *                            fp32: [d][Tp] (token index fastest);
 *                            bf16: Tp/64 tiles, tile = [8][d][8]
 *                                  (token in tile / 8, dim, token % 8), 16 KiB.
 *                          Either operand occupies B*Hkv*Tp*d elements.
 * k_cache, v_cache [B, Hkv, cap, d]  normalised pre-RoPE K and raw V (dtype). NULL
 *                          (both) = no cache. Global: token n goes to slot n,
 *                          cap >= pos_offset + T. Local: slot n mod window (a ring of
 *                          `window` slots, cap >= window); only the last `window`
 *                          new tokens are written.
 * window   0 = global layer, W > 0 = local layer with W keys including self. The
 *          4K release's local layer (band up to distance W, cache of W tokens [P3
 *          §5.1]) is window = W + 1 here. A global layer without YaRN (also the 4K
 *          release [P3 §6.3]) is a rope table built with yarn_factor <= 1.
 * rope_table / rope_table_bytes  a table built for this layer type covering every
 *                          renumbered position < kept + T (POST_ROPE: absolute < pos_offset + T).
 * cache_order PLAMO_CACHE_PRE_ROPE or PLAMO_CACHE_POST_ROPE (above).
 * ------------------------------------------------------------------------- */
PLAMO_API int plamo_kv_append(int dtype, const void* q, const void* k, const void* v,
                    const void* q_norm_w, const void* k_norm_w, float norm_offset,
                    float norm_eps, int v_norm, void* q_out, void* k_rot_out, void* v_t_out,
                    void* k_cache, void* v_cache, long long cap, int B, int T, int Hq,
                    int Hkv, int d, int window, long long pos_offset,
                    const void* rope_table, size_t rope_table_bytes, int cache_order,
                    void* stream);

/* ---------------------------------------------------------------------------
 * plamo_prefill_pack -- caller-held keys and values into the prefill operand layouts
 * [P3 §4.1, §4.5]
 *
 * For callers that hold the attended keys already rotated (an engine's post-RoPE cache, or
 * their own norm and RoPE) and want plamo_attn_prefill without plamo_kv_append: writes the
 * k_rot and v_t operands that plamo_attn_prefill reads, exactly in the layouts documented
 * for plamo_kv_append's k_rot_out and v_t_out, for the S keys (S = kept + T of that call;
 * Tp = plamo_prefill_padded_len(S) rows each, rows S .. Tp-1 zero).
 * k_rot [B, S, Hkv, d]  rotated K' of the keys in renumbered (or absolute, post-RoPE) order
 * v     [B, S, Hkv, d]  V of the same keys
 * dtype PLAMO_BF16: inputs bf16 (d = 128, 256 or 512), K' written as fp16 (exact for values
 * in the half range, |x| <= 65504); PLAMO_F32: inputs fp32, d = 128. The query operand
 * q_rot for plamo_attn_prefill is [B, T, Hq, d] (fp16 for PLAMO_BF16), the caller's Q'.
 * ------------------------------------------------------------------------- */
PLAMO_API int plamo_prefill_pack(int dtype, const void* k_rot, const void* v, void* k_rot_out,
                       void* v_t_out, int B, long long S, int Hkv, int d, void* stream);

/* ---------------------------------------------------------------------------
 * plamo_attn_prefill -- step 4 for a prefill of T tokens [P3 §4.5, §5.1]
 *
 * q_rot [B, T, Hq, d] (fp16 for PLAMO_BF16); k_rot and v_t in the dtype's layout written by
 * plamo_kv_append with the same window and pos_offset (Tp =
 * plamo_prefill_padded_len(kept + T), kept as for plamo_kv_append); out
 * [B, T, Hq, d] (token major, i.e. [B, T, Hq*d] ready for the output projection
 * [P3 §4.5]). Query t (0..T-1) sits at renumbered position i = kept + t and
 * attends operand keys j <= i, and i - j < window when window > 0: a chunk after
 * pos_offset cached tokens sees the cached keys first, then its own causally.
 * softmax_scale is 1/sqrt(d) [P3 §4.5] (1 for the Gemma-4-shaped layers [P3 §8
 * table]); the YaRN amplitude is already in q_rot and k_rot. bf16: (kept + T) * d <=
 * 2^29 (PLAMO_ERR_UNSUPPORTED beyond).
 * ------------------------------------------------------------------------- */
PLAMO_API int plamo_attn_prefill(int dtype, const void* q_rot, const void* k_rot, const void* v_t,
                       void* out, int B, int T, int Hq, int Hkv, int d, int window,
                       long long pos_offset, float softmax_scale, void* stream);

/* ---------------------------------------------------------------------------
 * plamo_attn_prefill_fused_q -- plamo_attn_prefill that applies steps 1 and 3 to the
 * queries itself [P3 §4.3, §4.4, §6.1]
 *
 * q [B, T, Hq, d] are the projected queries as plamo_kv_append takes them; each query
 * row is normalised (gain norm_offset + q_norm_w, eps norm_eps; q_norm_w NULL = no norm)
 * and rotated with `rope_table` at the position plamo_kv_append would give it (renumbered
 * kept + t, or absolute pos_offset + t with cache_order PLAMO_CACHE_POST_ROPE), in fp32,
 * then scaled and rounded once to fp16 for the MFMA. Call plamo_kv_append with q = q_out = NULL
 * first (it then writes only the K/V side: cache, k_rot, v_t), so Q' never goes through
 * HBM. k_rot, v_t, out and the mask as for plamo_attn_prefill. bf16 and d = 128 only
 * (PLAMO_ERR_UNSUPPORTED otherwise); the table must cover the queries' positions
 * (PLAMO_ERR_WORKSPACE otherwise).
 * ------------------------------------------------------------------------- */
PLAMO_API int plamo_attn_prefill_fused_q(int dtype, const void* q, const void* q_norm_w,
                       float norm_offset, float norm_eps, const void* k_rot, const void* v_t,
                       void* out, int B, int T, int Hq, int Hkv, int d, int window,
                       long long pos_offset, const void* rope_table, size_t rope_table_bytes,
                       int cache_order, float softmax_scale, void* stream);

/* ---------------------------------------------------------------------------
 * plamo_attn_decode -- step 4 for one new token per sequence, read from the cache
 * [P3 §4.4, §4.5, §5.1]
 *
 * Call after plamo_kv_append(T = 1) at the same pos_offset p. The cache then holds
 * the S = kept + 1 attended tokens p-kept .. p (kept as in plamo_kv_append);
 * their renumbered positions 0 .. S-1 rotate the pre-RoPE K on the fly with
 * `rope_table`; q_rot carries position S-1.
 *
 * q_rot [B, 1, Hq, d] (fp16, as plamo_kv_append writes it); k_cache, v_cache [B, Hkv, cap,
 * d] (bf16); out [B, 1, Hq, d] (bf16). Cached K is rotated in fp32 and rounded to fp16 for
 * the score product.
 * workspace: device scratch of at least plamo_attn_decode_workspace_bytes(...)
 * bytes (split-K partial results); contents on entry do not matter. When that
 * size is 0 (one key range per sequence and KV head) workspace may be NULL. The
 * size never decreases as pos_offset grows (the same holds for the ragged and the
 * one-launch step sizes below), so a workspace sized for the largest position a
 * caller will pass serves every smaller one.
 * dtype must be PLAMO_BF16; T must be 1. cache_order as given to plamo_kv_append
 * (POST_ROPE: rope_table may be NULL and is not read).
 * ------------------------------------------------------------------------- */
PLAMO_API size_t plamo_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int window,
                                         long long pos_offset);

PLAMO_API int plamo_attn_decode(int dtype, const void* q_rot, const void* k_cache,
                      const void* v_cache, long long cap, void* out, void* workspace,
                      size_t workspace_bytes, int B, int T, int Hq, int Hkv, int d,
                      int window, long long pos_offset, const void* rope_table,
                      size_t rope_table_bytes, float softmax_scale, int cache_order,
                      void* stream);

/* ---------------------------------------------------------------------------
 * plamo_decode_step -- one decode step of a layer in one launch: steps 1-4 for one new
 * token per sequence [P3 §3.2, §4.3, §4.4, §4.5, §5.1, §6]
 *
 * The same result as plamo_kv_append(T = 1) followed by plamo_attn_decode at the same
 * pos_offset p, without the Q' buffer and the separate merge: q [B, 1, Hq, d], k, v
 * [B, 1, Hkv, d] are the projected new token (bf16); gains, offset, eps, caches, rope table,
 * window and cache_order as for plamo_kv_append (V as given: no v_norm); out [B, 1, Hq, d]
 * (bf16). The token's normalised K (rotated first with POST_ROPE) and V go into cache slot
 * p (global) or p mod window (local); attention reads the kept tokens and the new one.
 * d = 128 only (PLAMO_ERR_UNSUPPORTED otherwise); bf16; uniform batch.
 *
 * workspace: at least plamo_decode_step_workspace_bytes(...) bytes (NULL allowed when 0),
 * dedicated to this call. Its first bytes hold one 32-bit counter per (sequence, KV head)
 * that must be zero before the first call (allocate it zeroed once); every call leaves them
 * at zero again. The key ranges' partial states follow. Calls sharing a workspace must be
 * ordered (one stream).
 * ------------------------------------------------------------------------- */
PLAMO_API size_t plamo_decode_step_workspace_bytes(int B, int Hq, int Hkv, int d, int window,
                                                   long long pos_offset);

PLAMO_API int plamo_decode_step(int dtype, const void* q, const void* k, const void* v,
                      const void* q_norm_w, const void* k_norm_w, float norm_offset,
                      float norm_eps, void* k_cache, void* v_cache, long long cap, void* out,
                      void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int d,
                      int window, long long pos_offset, const void* rope_table,
                      size_t rope_table_bytes, float softmax_scale, int cache_order,
                      void* stream);

/* ---------------------------------------------------------------------------
 * plamo_attn_decode_noalloc -- plamo_attn_decode without a workspace argument
 *
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, checks, kernels and
 * results as plamo_attn_decode; the split-K partials go to the library's own scratch, a
 * static device array of PLAMO_DECODE_SCRATCH_BYTES on each GPU, held until the process
 * ends. Nothing is allocated or freed by the call. A call whose partials would need more
 * (plamo_attn_decode_workspace_bytes(...) > PLAMO_DECODE_SCRATCH_BYTES) returns
 * PLAMO_ERR_WORKSPACE and launches nothing. The scratch belongs to the GPU that is current
 * on the calling thread (its address is looked up once per device); `stream` must be a
 * stream of that GPU. Every call on a GPU shares its scratch: calls that overlap on one GPU
 * (different streams, or host threads without ordering) race; order them on one stream.
 * The scratch needs no clearing (each call writes every partial it reads).
 * ------------------------------------------------------------------------- */
#define PLAMO_DECODE_SCRATCH_BYTES (8u << 20)

PLAMO_API int plamo_attn_decode_noalloc(int dtype, const void* q_rot, const void* k_cache,
                      const void* v_cache, long long cap, void* out, int B, int T, int Hq,
                      int Hkv, int d, int window, long long pos_offset, const void* rope_table,
                      size_t rope_table_bytes, float softmax_scale, int cache_order,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Ragged batches: every sequence at its own position [P3 §4.4]
 *
 * The three calls below are plamo_kv_append, plamo_attn_prefill and
 * plamo_attn_decode for a batch whose sequences sit at different positions and
 * (append, prefill) carry different numbers of new tokens. Tensors keep the padded
 * batch layout of the uniform calls with T = the largest token count: sequence b
 * uses rows 0 .. seq_lens[b]-1 of its [T, ...] slab; its other rows of q_out and
 * out are left untouched and its other input rows are not read.
 *
 * seq_pos_offsets  device int64 [B]: absolute position of sequence b's first new
 *                  token. Required, 8-byte aligned.
 * seq_lens         device int32 [B]: new tokens of sequence b (0 .. T; 0 = the
 *                  sequence sits this call out). NULL = T for every sequence.
 *                  4-byte aligned.
 * max_pos_offset   host bound of every seq_pos_offsets entry. The library validates
 *                  cache capacity, rope table, operand sizes and workspace against
 *                  it, exactly as it validates pos_offset in the uniform calls: for
 *                  sequence b, kept_b = seq_pos_offsets[b] (global) or
 *                  min(seq_pos_offsets[b], window-1) (local), and all sizes
 *                  plamo_prefill_padded_len is that of the uniform call at
 *                  pos_offset = max_pos_offset.
 * The kernels read the arrays on the device and clamp each entry into
 * [0, max_pos_offset] and [0, T], so a wrong entry can only give its own sequence a
 * wrong result, never an access outside the buffers.
 * Operand rows of sequence b: 0 .. kept_b-1 cached keys, kept_b .. kept_b+n_b-1 its
 * new tokens, zero up to Tp. Decode needs plamo_kv_append_ragged(T = 1) before it and
 * a workspace of plamo_attn_decode_ragged_workspace_bytes(...) bytes (NULL allowed
 * when that is 0): its key ranges are planned for the longest sequence and cut finer
 * than the uniform call's, so that sequences of different lengths even out.
 * ------------------------------------------------------------------------- */
PLAMO_API size_t plamo_attn_decode_ragged_workspace_bytes(int B, int Hq, int Hkv, int d,
                                                int window, long long max_pos_offset);

PLAMO_API int plamo_kv_append_ragged(int dtype, const void* q, const void* k, const void* v,
                    const void* q_norm_w, const void* k_norm_w, float norm_offset,
                    float norm_eps, int v_norm, void* q_out, void* k_rot_out, void* v_t_out,
                    void* k_cache, void* v_cache, long long cap, int B, int T, int Hq,
                    int Hkv, int d, int window, const long long* seq_pos_offsets,
                    const int* seq_lens, long long max_pos_offset, const void* rope_table,
                    size_t rope_table_bytes, int cache_order, void* stream);

PLAMO_API int plamo_attn_prefill_ragged(int dtype, const void* q_rot, const void* k_rot,
                    const void* v_t, void* out, int B, int T, int Hq, int Hkv, int d,
                    int window, const long long* seq_pos_offsets, const int* seq_lens,
                    long long max_pos_offset, float softmax_scale, void* stream);

PLAMO_API int plamo_attn_prefill_fused_q_ragged(int dtype, const void* q, const void* q_norm_w,
                    float norm_offset, float norm_eps, const void* k_rot, const void* v_t,
                    void* out, int B, int T, int Hq, int Hkv, int d, int window,
                    const long long* seq_pos_offsets, const int* seq_lens, long long max_pos_offset,
                    const void* rope_table, size_t rope_table_bytes, int cache_order,
                    float softmax_scale, void* stream);

PLAMO_API int plamo_attn_decode_ragged(int dtype, const void* q_rot, const void* k_cache,
                    const void* v_cache, long long cap, void* out, void* workspace,
                    size_t workspace_bytes, int B, int Hq, int Hkv, int d, int window,
                    const long long* seq_pos_offsets, long long max_pos_offset,
                    const void* rope_table, size_t rope_table_bytes, float softmax_scale,
                    int cache_order, void* stream);

/* ---------------------------------------------------------------------------
 * The attention sublayer around the hot path [P3 §3.2, §4.1, §4.5]
 *
 * x_out = x + N^(0.2)_{w_post}( O W_o^T ),  O = attention(split(N^(1)_{w_pre}(x) W_qkv^T))
 * composed from plamo_rms_norm, plamo_linear and the attention calls above:
 *   U = plamo_rms_norm(x, w_pre, offset 1)                 [B*T, D]
 *   Q | K | V = plamo_qkv_projection(U, W_qkv)            one GEMM, output split [P3 §4.1]
 *   O = plamo_kv_append + plamo_attn_prefill / plamo_attn_decode    [B*T, Hq d]
 *   P = plamo_linear(O, W_o [D, Hq d])                     [B*T, D]
 *   x_out = plamo_rms_norm(P, w_post, offset 0.2, residual x)
 * ------------------------------------------------------------------------- */

/* y[M, N] = x[M, K] W[N, K]^T, bf16 row-major, fp32 accumulation (the sublayer's
 * projections [P3 §4.1, §4.5]). N % 8 == 0, K % 64 == 0 (PLAMO_ERR_UNSUPPORTED
 * otherwise); y must not overlap x or W. */
PLAMO_API int plamo_linear(const void* x, const void* w, void* y, long long M, int N, int K,
                    void* stream);

/* The fused QKV projection [P3 §4.1]: [Q | K | V] = U W_qkv^T with U [M, D] (M = B*T
 * tokens) and W_qkv [(Hq + 2 Hkv) d, D], the output columns cut at Hq d and (Hq + Hkv) d
 * and written to q [M, Hq d], k [M, Hkv d], v [M, Hkv d] (i.e. [B, T, H, d] each, the
 * layouts plamo_kv_append takes). bf16, fp32 accumulation; D % 64 == 0, d % 8 == 0. */
PLAMO_API int plamo_qkv_projection(const void* u, const void* w_qkv, void* q, void* k, void* v,
                    long long M, int D, int Hq, int Hkv, int d, void* stream);

/* y = residual + (offset + w) * x / sqrt(mean(x^2) + eps) per row of n [P3 §3.2];
 * residual NULL = no add. x, residual, y [rows, n], w [n], all of `dtype`, fp32 math;
 * y may alias x or residual. n a multiple of 8 (bf16) or 4 (fp32). */
PLAMO_API int plamo_rms_norm(int dtype, const void* x, const void* w, float offset, float eps,
                    const void* residual, void* y, long long rows, int n, void* stream);

/* Human-readable text for a status code (static storage). */
PLAMO_API const char* plamo_status_str(int status);

/* Detail of the last failed check on the calling thread (static thread-local). */
PLAMO_API const char* plamo_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PLAMO_ATTN_H */
