// Two-level RoPE rotation table, built in fp64 on the device and stored as fp32.
//
// 「PLaMo 3アーキテクチャ徹底解析」 §6.1: split-half RoPE turns pair j (components j and
// j + d/2) by the angle p * w_j with w_j = theta^(-2j/d). §6.3 (global layers, YaRN):
// w_j is blended towards w_j / s over the unrounded ramp [j_low, j_high] and both cos
// and sin carry the amplitude 1 + 0.1 ln s.
//
// Layout (float2 = (cos, sin)):
//   fine   [64][d/2]      amp * exp(i * delta * w_j),   delta = 0 .. 63
//   coarse [n_coarse][d/2]      exp(i * 64c * w_j),     c = 0 .. n_coarse-1
// so that amp * exp(i p w_j) = coarse[p >> 6][j] * fine[p & 63][j]. Angles are formed
// in fp64 (an fp32 angle at p = 131072 would be off by ~0.01 rad).
//
// §6.4 (p-RoPE): only the n_rot highest-frequency pairs turn, with the exponent still over
// the whole head dim; the other pairs have frequency 0, so their entries are (1, 0).
#include "common.h"
#include "kernels.h"

namespace plamo {

__global__ void rope_table_kernel(float2* __restrict__ table, long long rows, int d,
                                  double theta, double yarn_factor, double j_low,
                                  double j_high, double amplitude, int n_rot) {
  const int half = d / 2;
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= rows * half) return;
  const long long row = idx / half;
  const int j = static_cast<int>(idx % half);
  double omega = j < n_rot ? pow(theta, -2.0 * j / d) : 0.0;
  if (yarn_factor > 1.0) {
    double alpha = (j - j_low) / (j_high - j_low);
    alpha = alpha < 0.0 ? 0.0 : (alpha > 1.0 ? 1.0 : alpha);
    omega *= (1.0 - alpha) + alpha / yarn_factor;
  }
  double pos, amp;
  if (row < kRopeFine) {
    pos = static_cast<double>(row);
    amp = amplitude;
  } else {
    pos = static_cast<double>(row - kRopeFine) * kRopeFine;
    amp = 1.0;
  }
  double s, c;
  sincos(pos * omega, &s, &c);
  table[idx] = make_float2(static_cast<float>(amp * c), static_cast<float>(amp * s));
}

hipError_t launch_rope_table(float2* table, long long n_coarse, int d, double theta,
                             double yarn_factor, double j_low, double j_high,
                             double amplitude, int n_rot, hipStream_t stream) {
  const long long rows = kRopeFine + n_coarse;
  const long long n = rows * (d / 2);
  const int block = 256;
  const long long grid = (n + block - 1) / block;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(grid)), dim3(block), 0,
                     stream, table, rows, d, theta, yarn_factor, j_low, j_high, amplitude, n_rot);
  return hipGetLastError();
}

}  // namespace plamo
