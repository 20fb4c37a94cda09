// Shared device helpers for the gfx950 attention kernels: storage types, bf16
// conversion, the rope-table lookup and small wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plamo {

constexpr int kHeadDim = 128;      // PLaMo 3 head_dim (「PLaMo 3アーキテクチャ徹底解析」 §2.1)
constexpr int kHalf = kHeadDim / 2;
constexpr int kRopeFine = 64;      // positions per coarse rope-table row
constexpr int kPadT = 128;         // prefill operand padding of the token axis

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory
typedef uint16_t f16_t;   // raw IEEE half bits in memory (the Q' and K' score operands)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(bf16_t, b);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Pack two floats into one dword of two bf16 (lo in the low half), round to nearest
// even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

// Pack two floats into one dword of two IEEE halves (lo in the low half), round to nearest
// even: one v_cvt_pk_f16_f32. The score operands Q' and K' are stored and multiplied in
// this format: they are RMS-normalised (bounded by |gain| sqrt(d) times the RoPE amplitude),
// so the three extra mantissa bits over bf16 come at no range cost.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2v));
}

__device__ __forceinline__ float lo_f16(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2v, w).x);
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(f16x2v, w).y);
}

// acc + lo(w) + hi(w) for a dword of two bf16 (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  const bf16x2v one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w), one, acc, false);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// bf16 pair -> IEEE half pair (exact for |x| in [2^-14, 65504], the range of normalised K).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) { return pack_f16x2(lo_bf16(w), hi_bf16(w)); }

// Rotation factor amp * exp(i p w_j) from the two-level table: coarse row p >> 6 times
// fine row p & 63 (complex product, fp32). Layout: fine [64][d/2] float2 first, then
// coarse [n_coarse][d/2] float2.
// kH = d/2 pairs per table row.
template <int kH = kHalf>
__device__ __forceinline__ float2 rope_factor(const float2* __restrict__ table, long long p, int j) {
  const float2 f = table[(p & (kRopeFine - 1)) * kH + j];
  const float2 c = table[(kRopeFine + (p >> 6)) * kH + j];
  return make_float2(c.x * f.x - c.y * f.y, c.x * f.y + c.y * f.x);
}

// Positions of sequence b of a batch (「PLaMo 3アーキテクチャ徹底解析」 §4.4): its first new
// token sits at absolute position `pos`, the cache returns `kept` earlier tokens (all of
// them on a global layer, at most window - 1 on a local one) and the call carries `T` new
// tokens. A uniform batch passes no per-sequence arrays. A ragged batch passes seq_pos
// (and, for more than one new token, seq_len) in device memory; each value is clamped to
// the bounds the host validated (0 .. pos_max, 0 .. T_max), so a bad entry can give a
// wrong result for its own sequence but never an access outside the buffers.
struct SeqPos {
  long long pos;
  long long kept;
  int T;
};
__device__ __forceinline__ SeqPos seq_pos_of(const long long* seq_pos, const int* seq_len, long long pos_max,
                                             int T_max, int window, int b) {
  long long p = pos_max;
  if (seq_pos) {
    p = seq_pos[b];
    p = p < 0 ? 0 : (p > pos_max ? pos_max : p);
  }
  int t = T_max;
  if (seq_len) {
    t = seq_len[b];
    t = t < 0 ? 0 : (t > T_max ? T_max : t);
  }
  const long long kept = window == 0 ? p : (p < window - 1 ? p : static_cast<long long>(window - 1));
  return SeqPos{p, kept, t};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace plamo
