// Host-side launchers of the gfx950 kernels. Arguments have been validated by the
// C-ABI layer (abi.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#ifndef STEP_MIN_CHUNK
#define STEP_MIN_CHUNK 256
#endif

namespace plamo {

// n_rot: pairs j < n_rot turn; the others get frequency 0 (p-RoPE); n_rot = d/2 for all.
hipError_t launch_rope_table(float2* table, long long n_coarse, int d, double theta,
                             double yarn_factor, double j_low, double j_high,
                             double amplitude, int n_rot, hipStream_t stream);

struct AppendArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* wq;  // NULL = no norm
  const void* wk;
  float norm_offset;
  float eps;
  void* q_out;
  void* k_rot_out;  // may be NULL
  void* v_t_out;    // may be NULL
  void* k_cache;    // may be NULL (then v_cache is NULL too)
  void* v_cache;
  long long cap;
  int B, T, Hq, Hkv, window;
  long long Tp;          // padded key count of the prefill operands (kept + T keys)
  long long pos_offset;  // absolute position of the first new token (ragged: the largest)
  long long kept;        // cached tokens returned before the new ones (ragged: the largest)
  const long long* seq_pos;  // ragged batch: per-sequence pos_offset (device), else NULL
  const int* seq_len;        // ragged batch: per-sequence new-token count (device), else NULL
  bool ops_kernel;           // the operand kernel writes every operand row outside the chunk
  bool post_rope;            // the cache holds K rotated at absolute positions (else pre-RoPE)
  bool v_norm;               // divide each new V head vector by its RMS before use
  int d;                     // head dim: 128 (fp32 and bf16), 256 or 512 (bf16)
  const float2* rope;
  int q_split;               // (set by the launch) blocks sharing one token block's query heads
};
// Both launch, when prefill operands are requested after cached tokens or for a ragged
// batch, first the operand kernel (the kept keys from the cache, all of V^T and the
// padding) and then the append kernel (new tokens).
hipError_t launch_kv_append_bf16(const AppendArgs& a, hipStream_t stream);
hipError_t launch_kv_append_f32(const AppendArgs& a, hipStream_t stream);

// Caller-held K' and V [B, S, Hkv, d] into the prefill operand layouts (Tp rows each).
struct PackArgs {
  const void* k;
  const void* v;
  void* k_rot_out;
  void* v_t_out;
  int B, Hkv, d;
  long long S, Tp;
};
hipError_t launch_prefill_pack(const PackArgs& a, bool bf16, hipStream_t stream);

struct PrefillArgs {
  const void* q_rot;  // [B, T, Hq, d]
  const void* k_rot;  // [B, Hkv, Tp, d]
  const void* v_t;    // [B, Hkv, d, Tp]
  void* out;          // [B, T, Hq, d]
  int B, T, Hq, Hkv, window;
  long long Tp;    // padded key count of K', V^T
  long long kept;  // keys before the chunk: query t sits at renumbered position kept + t
  long long pos_offset;      // absolute position of the first new token (ragged: the largest)
  const long long* seq_pos;  // ragged batch: per-sequence pos_offset (device), else NULL
  const int* seq_len;        // ragged batch: per-sequence token count (device), else NULL
  float scale;
  int d;                     // head dim: 128, 256 or 512 (bf16)
  // Fused Q (bf16, d = 128): q_rot then holds the projected queries, normalised (when wq is
  // given: gain norm_offset + w, eps) and rotated here at the positions the append uses.
  bool fuse_q;
  bool post_rope;            // (fused Q) rotate at absolute positions
  const void* wq;
  float norm_offset, eps;
  const float2* rope;
};
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// Head dims 256 and 512 (bf16).
hipError_t launch_prefill_wide_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

struct DecodePlan {
  int n_split;         // key ranges per (sequence, KV head)
  long long chunk;     // keys per range, a multiple of the key tile
  int max_split;       // n_split <= max_split, and max_split never decreases as S grows: the
                       // workspace is sized by it, so a workspace sized for a position serves
                       // every smaller one
};
// min_chunk: keys per range, at least (a multiple of the 64-key tile)
DecodePlan plan_decode(int B, int Hkv, long long S, bool ragged, long long min_chunk = 256);
// the one-launch step's ranges (fewer, longer: each range's state goes through the merge)
constexpr long long kStepMinChunk = STEP_MIN_CHUNK;
size_t decode_workspace_bytes(int B, int Hq, int d, const DecodePlan& plan);
// Size of the library's own split-K scratch (plamo_attn_decode_noalloc), and its device
// address on the current GPU (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
hipError_t decode_scratch(float** ptr);

struct DecodeArgs {
  const void* q_rot;    // [B, 1, Hq, d]
  const void* k_cache;  // [B, Hkv, cap, d]
  const void* v_cache;
  long long cap;
  void* out;            // [B, 1, Hq, d]
  float* ws;            // [B, Hq, n_split, d + 2]
  int B, Hq, Hkv, window;
  long long S;          // attended keys (renumbered 0 .. S-1; ragged: the largest)
  long long base;       // absolute position of renumbered key 0 (uniform batch)
  long long pos_offset; // position of the new token (ragged: the largest)
  const long long* seq_pos;  // ragged batch: per-sequence position (device), else NULL
  bool post_rope;            // the cache holds K rotated at absolute positions: no rotation
  DecodePlan plan;
  const float2* rope;
  float scale;
  int d;                     // head dim: 128; 256 or 512 with a post-RoPE cache
  // One-launch step (d = 128, uniform batch): the decode kernel also does what the append
  // does for the new token (Q norm and rotation in every block; K norm, K and V into the
  // cache in the block holding the newest key) and merges the key ranges itself (the last
  // block of a (sequence, KV head) to finish, counted on `tickets`, which start and end at 0).
  bool fused;
  const void* q_in;          // [B, 1, Hq, d] projected (bf16)
  const void* k_in;          // [B, 1, Hkv, d]
  const void* v_in;
  const void* wq;            // NULL = no Q/K norm
  const void* wk;
  float norm_offset, eps;
  unsigned* tickets;         // [B * Hkv]
};
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// Workspace of the one-launch step: the tickets (a 256-byte multiple), then the partial
// states (0 bytes in all when no merge).
size_t decode_step_tickets_bytes(int B, int Hkv);
size_t decode_step_workspace_bytes(int B, int Hq, int Hkv, int d, const DecodePlan& plan);
// Head dims 256 and 512, post-RoPE cache.
hipError_t launch_decode_wide_bf16(const DecodeArgs& a, hipStream_t stream);

struct GemmArgs {
  const void* x;            // [M, K] bf16
  const void* w;            // [N, K] bf16
  void* y[3];               // output parts: columns [part_end[p-1], part_end[p]) go to y[p],
  long long part_end[3];    // a row-major [M, width_p] tensor; unused parts end at N
  long long M, N;
  int K;                    // a multiple of 64
};
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream);

struct NormArgs {
  const void* x;         // [rows, n]
  const void* w;         // [n] stored gain weights (gain = offset + w)
  const void* residual;  // [rows, n] or NULL
  void* y;               // [rows, n]; may alias residual
  long long rows;
  int n;                 // a multiple of 8 (bf16) or 4 (fp32)
  float offset, eps;
};
hipError_t launch_rms_norm_bf16(const NormArgs& a, hipStream_t stream);
hipError_t launch_rms_norm_f32(const NormArgs& a, hipStream_t stream);

}  // namespace plamo
