// Fused per-head Q/K RMSNorm + RoPE + KV-cache append, and the prefill operand copies.
//
// 「PLaMo 3アーキテクチャ徹底解析」:
//   §3.2/§4.3  per (token, head): y = (c + w) * x / sqrt(mean(x^2) + eps) over the 128
//              components, one [128] gain shared by all Q heads (k_norm by all KV heads);
//              V is not normalised.
//   §4.4       the cache receives normalised K before RoPE and raw V; RoPE then turns the
//              current Q and the K the cache returns, at renumbered positions.
//   §6.1/§6.3  split-half pairs (j, j + 64); rotation factors from the two-level table.
//
// One block = 64 tokens of one sequence and one KV head: its G = Hq/Hkv query heads,
// the K head and the V head. Lane j of a wave owns pair j of the row it works on, so the
// rotation is lane-local and the norm is one wave reduction. V is staged through LDS to
// write the transposed prefill operand with 128-byte rows.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int kTokBlock = 64;
constexpr int kThreads = 256;

template <typename E>
struct Io;

template <>
struct Io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float x) { *p = x; }
  static __device__ __forceinline__ float rnd(float x) { return x; }
};

template <>
struct Io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float x) { *p = f32_to_bf16(x); }
  static __device__ __forceinline__ float rnd(float x) { return bf16_to_f32(f32_to_bf16(x)); }
};

template <typename E>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kTokBlock;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const E* __restrict__ wq = static_cast<const E*>(a.wq);
  const E* __restrict__ wk = static_cast<const E*>(a.wk);
  E* __restrict__ q_out = static_cast<E*>(a.q_out);
  E* __restrict__ k_rot = static_cast<E*>(a.k_rot_out);
  E* __restrict__ v_t = static_cast<E*>(a.v_t_out);
  E* __restrict__ k_cache = static_cast<E*>(a.k_cache);
  E* __restrict__ v_cache = static_cast<E*>(a.v_cache);
  const bool norm = wq != nullptr;
  const float gq0 = norm ? a.norm_offset + Io<E>::ld(wq + lane) : 1.f;
  const float gq1 = norm ? a.norm_offset + Io<E>::ld(wq + lane + kHalf) : 1.f;
  const float gk0 = norm ? a.norm_offset + Io<E>::ld(wk + lane) : 1.f;
  const float gk1 = norm ? a.norm_offset + Io<E>::ld(wk + lane + kHalf) : 1.f;
  const int n_tok = min(kTokBlock, a.T - t0);  // may be <= 0 in the padding blocks

  // --- queries: norm, rotate at renumbered position kept + t ---------------------------
  for (int r = wave; r < n_tok * G; r += kThreads / 64) {
    const int t = t0 + r / G;
    const int hq = kvh * G + r % G;
    const long long row = ((static_cast<long long>(b) * a.T + t) * a.Hq + hq) * kHeadDim;
    float x0 = Io<E>::ld(q + row + lane);
    float x1 = Io<E>::ld(q + row + lane + kHalf);
    if (norm) {
      const float inv = rsqrtf(wave_sum(x0 * x0 + x1 * x1) * (1.f / kHeadDim) + a.eps);
      x0 *= inv * gq0;
      x1 *= inv * gq1;
    }
    const float2 z = rope_factor(a.rope, a.kept + t, lane);
    Io<E>::st(q_out + row + lane, x0 * z.x - x1 * z.y);
    Io<E>::st(q_out + row + lane + kHalf, x0 * z.y + x1 * z.x);
  }

  // --- keys: norm, round to the cache type, cache write, rotate -----------------------
  const int k_rows = k_rot ? kTokBlock : n_tok;  // padding rows only feed k_rot zeros
  for (int r = wave; r < k_rows; r += kThreads / 64) {
    const int t = t0 + r;
    if (t >= a.T) {
      if (t < a.Tp) {
        const long long orow = ((static_cast<long long>(b) * a.Hkv + kvh) * a.Tp + t) * kHeadDim;
        Io<E>::st(k_rot + orow + lane, 0.f);
        Io<E>::st(k_rot + orow + lane + kHalf, 0.f);
      }
      continue;
    }
    const long long row = ((static_cast<long long>(b) * a.T + t) * a.Hkv + kvh) * kHeadDim;
    float x0 = Io<E>::ld(k + row + lane);
    float x1 = Io<E>::ld(k + row + lane + kHalf);
    if (norm) {
      const float inv = rsqrtf(wave_sum(x0 * x0 + x1 * x1) * (1.f / kHeadDim) + a.eps);
      x0 = Io<E>::rnd(x0 * inv * gk0);
      x1 = Io<E>::rnd(x1 * inv * gk1);
    }
    if (k_cache) {
      const long long n = a.pos_offset + t;
      const bool write = a.window == 0 || t >= a.T - a.window;
      if (write) {
        const long long slot = a.window == 0 ? n : n % a.window;
        const long long crow = ((static_cast<long long>(b) * a.Hkv + kvh) * a.cap + slot) * kHeadDim;
        Io<E>::st(k_cache + crow + lane, x0);
        Io<E>::st(k_cache + crow + lane + kHalf, x1);
      }
    }
    if (k_rot) {
      const float2 z = rope_factor(a.rope, a.kept + t, lane);
      const long long orow = ((static_cast<long long>(b) * a.Hkv + kvh) * a.Tp + t) * kHeadDim;
      Io<E>::st(k_rot + orow + lane, x0 * z.x - x1 * z.y);
      Io<E>::st(k_rot + orow + lane + kHalf, x0 * z.y + x1 * z.x);
    }
  }

  // --- values: raw copy into the cache, transposed prefill operand --------------------
  if (v_cache) {
    for (int r = wave; r < n_tok; r += kThreads / 64) {
      const int t = t0 + r;
      if (!(a.window == 0 || t >= a.T - a.window)) continue;
      const long long n = a.pos_offset + t;
      const long long slot = a.window == 0 ? n : n % a.window;
      const long long row = ((static_cast<long long>(b) * a.T + t) * a.Hkv + kvh) * kHeadDim;
      const long long crow = ((static_cast<long long>(b) * a.Hkv + kvh) * a.cap + slot) * kHeadDim;
      v_cache[crow + lane] = v[row + lane];
      v_cache[crow + lane + kHalf] = v[row + lane + kHalf];
    }
  }
  if (v_t) {
    __shared__ E tile[kHeadDim][kTokBlock + 1];
    for (int i = threadIdx.x; i < kTokBlock * kHeadDim; i += kThreads) {
      const int r = i / kHeadDim;
      const int c = i % kHeadDim;
      const int t = t0 + r;
      E x = E(0);
      if (t < a.T) x = v[((static_cast<long long>(b) * a.T + t) * a.Hkv + kvh) * kHeadDim + c];
      tile[c][r] = x;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kTokBlock * kHeadDim; i += kThreads) {
      const int c = i / kTokBlock;
      const int r = i % kTokBlock;
      const long long t = t0 + r;
      if (t < a.Tp)
        v_t[((static_cast<long long>(b) * a.Hkv + kvh) * kHeadDim + c) * a.Tp + t] = tile[c][r];
    }
  }
}

template <typename E>
hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const long long tokens = (a.k_rot_out || a.v_t_out) ? a.Tp : a.T;
  const unsigned gx = static_cast<unsigned>((tokens + kTokBlock - 1) / kTokBlock);
  hipLaunchKernelGGL(kv_append_kernel<E>, dim3(gx, a.Hkv, a.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append_bf16(const AppendArgs& a, hipStream_t stream) {
  return launch_append<bf16_t>(a, stream);
}
hipError_t launch_kv_append_f32(const AppendArgs& a, hipStream_t stream) {
  return launch_append<float>(a, stream);
}

}  // namespace plamo
