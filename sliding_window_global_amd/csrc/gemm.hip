// Projection GEMM of the attention sublayer on gfx950 bf16 MFMA:
// y[M, N] = x[M, K] W[N, K]^T (both operands K-contiguous, fp32 accumulation, bf16 out).
// 「PLaMo 3アーキテクチャ徹底解析」 §4.1: the fused QKV projection (N = (Hq + 2 Hkv) d, cut into
// its Q | K | V row blocks), §4.5: the output projection (K = Hq d, N = hidden).
//
// block  = 128 rows of x (m) x 256 rows of W (n), 4 waves in a 2 x 2 grid, each wave
//          64 m x 128 n = 2 x 4 blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators).
//          W fragments are the MFMA A operand (32 n x 16 k), x fragments the B operand, so a
//          lane's accumulators hold one m and runs of 4 consecutive n: 8-byte stores.
// tiles  = 64 k per step: W tile 256 x 64, x tile 128 x 64 (32 + 16 KiB), double buffered,
//          copied global -> LDS by buffer loads with the LDS bit (a resource per operand
//          block bounds every read; rows past M or N read 0). LDS rows are 128 B; the
//          16-byte chunk c of row r sits at position c ^ ((r >> 1) & 7), so that the eight
//          lanes of a row read one contiguous 128 B of global memory and the 16 rows that a
//          quarter-wave's fragment read touches fall into distinct banks.
// Requirements (checked by the caller): K % 64 == 0, N % 8 == 0.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int BM = 128;  // rows of x per block
constexpr int BN = 256;  // rows of W per block
constexpr int BK = 64;   // k per step (8 chunks of 8)
constexpr int kThreads = 256;
constexpr unsigned kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters untouched

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) bf16_t as0[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t as1[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t bs0[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t bs1[BM * BK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const long long n0 = static_cast<long long>(blockIdx.x) * BN;
  const long long m0 = static_cast<long long>(blockIdx.y) * BM;
  const int K = a.K;
  const int nk = K / BK;

  // operand blocks: rows past N (M) lie outside the resource and read as 0
  const long long n_rows = min(static_cast<long long>(BN), a.N - n0);
  const long long m_rows = min(static_cast<long long>(BM), a.M - m0);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      make_rsrc(static_cast<const bf16_t*>(a.w) + n0 * K, static_cast<int>(n_rows * K * 2));
  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc(static_cast<const bf16_t*>(a.x) + m0 * K, static_cast<int>(m_rows * K * 2));

  // copy of one 64-k step: 1 KiB per direct load = 8 rows x 128 B; lane l fills position
  // l % 8 of row l / 8 with global chunk (l % 8) ^ swz(row)
  const int sub_row = lane >> 3, pos = lane & 7;
  auto issue = [&](__amdgpu_buffer_rsrc_t rsrc, int rows_per_wave, int step, bf16_t* buf)
      __attribute__((always_inline)) {
    const int k_off = step * BK * 2;  // bytes
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i * 8 >= rows_per_wave) break;
      const int row = wave * rows_per_wave + i * 8 + sub_row;
      const int voff = (row * K + ((pos ^ swz(row)) * 8)) * 2;
      lds_ptr_t dst = (lds_ptr_t)(buf + (wave * rows_per_wave + i * 8) * BK);  // generic -> LDS
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, k_off, 0, 0);
    }
  };
  auto issue_step = [&](int step, bf16_t* abuf, bf16_t* bbuf) __attribute__((always_inline)) {
    issue(w_rsrc, BN / 4, step, abuf);
    issue(x_rsrc, BM / 4, step, bbuf);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment of rows r0 .. r0+31 at k sub-step s: lane l reads row r0 + l % 32, chunk
  // 2s + l / 32
  const int fr_row = lane & 31, fr_half = lane >> 5;
  auto frag = [&](const bf16_t* buf, int r0, int s) __attribute__((always_inline)) {
    const int r = r0 + fr_row;
    const int c = 2 * s + fr_half;
    return *reinterpret_cast<const bf16x8*>(buf + (r * 8 + (c ^ swz(r))) * 8);
  };
  auto compute = [&](const bf16_t* abuf, const bf16_t* bbuf) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = frag(abuf, wn * 128 + i * 32, s);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = frag(bbuf, wm * 64 + j * 32, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  issue_step(0, as0, bs0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  for (int t = 0; t < nk; t += 2) {
    if (t + 1 < nk) issue_step(t + 1, as1, bs1);
    compute(as0, bs0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 < nk) {
      if (t + 2 < nk) issue_step(t + 2, as0, bs0);
      compute(as1, bs1);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }
  }

  // store: accumulator (i, j) register e holds m = m0 + wm*64 + j*32 + lane % 32 and
  // n = n0 + wn*128 + i*32 + (e/4)*8 + (lane/32)*4 + e%4
  bf16_t* y = static_cast<bf16_t*>(a.y);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long long m = m0 + wm * 64 + j * 32 + (lane & 31);
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const long long n = n0 + wn * 128 + i * 32 + q * 8 + (lane >> 5) * 4;
        if (n >= a.N) continue;
        u32x2 w;
        w[0] = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
        w[1] = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
        *reinterpret_cast<u32x2*>(y + m * a.N + n) = w;
      }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((a.N + BN - 1) / BN), static_cast<unsigned>((a.M + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace plamo
