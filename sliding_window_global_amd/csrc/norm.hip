// Row RMSNorm with a gain offset, optionally added to a residual row.
//
// 「PLaMo 3アーキテクチャ徹底解析」 §3.2: N_w^(c)(x) = (c + w) * x / sqrt(mean(x^2) + eps) over
// the n components of a row; the attention sublayer applies it before the projections
// (pre_mixer_norm, c = 1) and to the sublayer output (post_mixer_norm, c = 0.2), which is
// then added to the residual stream.
//
// One wave per row: lanes hold 16-byte chunks (8 bf16 or 4 fp32), strided by 64 chunks,
// the sum of squares is a wave reduction, the second pass reads the row again (it is in
// L2) and writes (residual +) gain * x * 1/rms. fp32 arithmetic.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int kWavesPerBlock = 4;

template <typename E>
struct Vec16;
template <>
struct Vec16<bf16_t> {
  static constexpr int kN = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = lo_bf16(w[e]);
      x[2 * e + 1] = hi_bf16(w[e]);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* x) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
};
template <>
struct Vec16<float> {
  static constexpr int kN = 4;
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

template <typename E>
__global__ __launch_bounds__(64 * kWavesPerBlock) void rms_norm_kernel(NormArgs a) {
  using V = Vec16<E>;
  constexpr int kN = V::kN;
  const int lane = threadIdx.x & 63;
  const long long row = static_cast<long long>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= a.rows) return;  // wave-uniform; no barrier in this kernel
  const int chunks = a.n / kN;
  const E* x = static_cast<const E*>(a.x) + row * a.n;
  float ss = 0.f;
  for (int c = lane; c < chunks; c += 64) {
    float v[kN];
    V::load(x + c * kN, v);
#pragma unroll
    for (int e = 0; e < kN; ++e) ss += v[e] * v[e];
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / static_cast<float>(a.n) + a.eps);
  const E* w = static_cast<const E*>(a.w);
  const E* r = a.residual ? static_cast<const E*>(a.residual) + row * a.n : nullptr;
  E* y = static_cast<E*>(a.y) + row * a.n;
  for (int c = lane; c < chunks; c += 64) {
    float v[kN], g[kN], o[kN];
    V::load(x + c * kN, v);
    V::load(w + c * kN, g);
    if (r) {
      V::load(r + c * kN, o);
    } else {
#pragma unroll
      for (int e = 0; e < kN; ++e) o[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < kN; ++e) o[e] += (a.offset + g[e]) * (v[e] * inv);
    V::store(y + c * kN, o);
  }
}

}  // namespace

hipError_t launch_rms_norm_bf16(const NormArgs& a, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((a.rows + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(rms_norm_kernel<bf16_t>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, stream, a);
  return hipGetLastError();
}
hipError_t launch_rms_norm_f32(const NormArgs& a, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((a.rows + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(rms_norm_kernel<float>, dim3(blocks), dim3(64 * kWavesPerBlock), 0, stream, a);
  return hipGetLastError();
}

}  // namespace plamo
