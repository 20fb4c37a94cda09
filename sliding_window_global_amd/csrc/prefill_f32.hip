// fp32 causal / sliding-window GQA prefill (the fp32 path of the tiny-config checks).
//
// Same definition as the bf16 kernel (「PLaMo 3アーキテクチャ徹底解析」 §4.5, §5.1), kept in
// fp32 end to end on the vector ALUs: a block owns 64 query rows of one head, two lanes
// per row (one per half of the 128 components), K and V tiles of 32 keys in LDS, and an
// online softmax per tile. Tiles outside every row's window are skipped.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int kRows = 64;
constexpr int kThreads = 2 * kRows;
constexpr int kKeys = 32;

__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(PrefillArgs a) {
  __shared__ float ks[kKeys][kHeadDim];
  __shared__ float vs[kKeys][kHeadDim];
  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int nqb = (a.T + kRows - 1) / kRows;
  const int qb = blockIdx.x % nqb;
  const int hq = (blockIdx.x / nqb) % a.Hq;
  const int b = blockIdx.x / (nqb * a.Hq);
  const int kvh = hq / (a.Hq / a.Hkv);
  const int i0 = qb * kRows;
  const int row = i0 + tid / 2;
  // this sequence's kept keys and token count (a.T is the row stride)
  const SeqPos sp = seq_pos_of(a.seq_pos, a.seq_len, a.pos_offset, a.T, a.window, b);
  if (i0 >= sp.T) return;  // block-uniform, before any barrier
  const bool valid = row < sp.T;

  const float* __restrict__ qp = static_cast<const float*>(a.q_rot) +
                                 (static_cast<long long>(b) * a.T + (valid ? row : 0)) * a.Hq * kHeadDim +
                                 static_cast<long long>(hq) * kHeadDim + half * kHalf;
  const float* __restrict__ kbase =
      static_cast<const float*>(a.k_rot) + (static_cast<long long>(b) * a.Hkv + kvh) * a.Tp * kHeadDim;
  const float* __restrict__ vbase =
      static_cast<const float*>(a.v_t) + (static_cast<long long>(b) * a.Hkv + kvh) * kHeadDim * a.Tp;

  float qv[kHalf], ov[kHalf];
#pragma unroll
  for (int r = 0; r < kHalf; ++r) {
    qv[r] = valid ? qp[r] : 0.f;
    ov[r] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale * 1.4426950408889634f;

  // query row t sits at renumbered position kept + t; keys 0 .. kept-1 came from the cache
  const int kept = static_cast<int>(sp.kept);
  const int pos = kept + row;
  const int last = kept + min(i0 + kRows, sp.T) - 1;
  const int lo = a.window > 0 ? max(0, kept + i0 - a.window + 1) : 0;
  for (int j0 = (lo / kKeys) * kKeys; j0 <= last; j0 += kKeys) {
    __syncthreads();
    for (int e = tid; e < kKeys * kHeadDim; e += kThreads) {
      const int key = e / kHeadDim, dim = e % kHeadDim;
      ks[key][dim] = kbase[static_cast<long long>(j0 + key) * kHeadDim + dim];
    }
    for (int e = tid; e < kKeys * kHeadDim; e += kThreads) {
      const int dim = e / kKeys, key = e % kKeys;
      vs[key][dim] = vbase[static_cast<long long>(dim) * a.Tp + j0 + key];
    }
    __syncthreads();
    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < kKeys; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < kHalf; ++r) part = fmaf(qv[r], ks[kk][half * kHalf + r], part);
      float dot = part + __shfl_xor(part, 1, 64);
      const int key = j0 + kk;
      const bool ok = key <= pos && (a.window == 0 || pos - key < a.window);
      s[kk] = ok ? dot * c : -INFINITY;
      mx = fmaxf(mx, s[kk]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int r = 0; r < kHalf; ++r) ov[r] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kKeys; ++kk) {
      const float p = exp2f(s[kk] - m_use);
      l_run += p;
#pragma unroll
      for (int r = 0; r < kHalf; ++r) ov[r] = fmaf(p, vs[kk][half * kHalf + r], ov[r]);
    }
    m_run = m_new;
  }
  if (valid) {
    float* dst = static_cast<float*>(a.out) + (static_cast<long long>(b) * a.T + row) * a.Hq * kHeadDim +
                 static_cast<long long>(hq) * kHeadDim + half * kHalf;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int r = 0; r < kHalf; ++r) dst[r] = ov[r] * inv;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  const long long nqb = (a.T + kRows - 1) / kRows;
  const long long blocks = nqb * a.Hq * a.B;
  hipLaunchKernelGGL(prefill_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace plamo
