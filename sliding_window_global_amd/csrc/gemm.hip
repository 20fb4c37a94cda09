// Projection GEMM of the attention sublayer on gfx950 bf16 MFMA:
// y[M, N] = x[M, K] W[N, K]^T (both operands K-contiguous, fp32 accumulation, bf16 out).
// 「PLaMo 3アーキテクチャ徹底解析」 §4.1: the fused QKV projection (N = (Hq + 2 Hkv) d), whose
// output columns are split into Q | K | V; the epilogue writes each part to its own tensor.
// §4.5: the output projection (K = Hq d, N = hidden).
//
// block  = 256 rows of x (m) x 256 rows of W (n), 8 waves in a 4 (m) x 2 (n) grid, each wave
//          64 m x 128 n = 2 x 4 blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators).
//          W fragments are the MFMA A operand (32 n x 16 k), x fragments the B operand, so a
//          lane's accumulators hold one m and runs of 4 consecutive n; the output goes out
//          through LDS as whole 256-byte row segments.
// tiles  = 64 k per step: W and x tiles 256 x 64 (32 KiB each), double buffered (128 KiB,
//          one block per CU), copied global -> LDS by buffer loads with the LDS bit (a
//          resource per operand block bounds every read; rows past M or N read 0). LDS rows
//          are 128 B; the 16-byte chunk c of row r sits at position c ^ ((r >> 1) & 7), so
//          that the eight lanes of a row read one contiguous 128 B of global memory and the
//          16 rows of a quarter-wave's fragment read fall into distinct banks. The next
//          sub-step's fragments are read while the current sub-step's MFMAs run.
// Measured on the sublayer shapes: ~1.0-1.1 PFLOP/s; the same kernel without the tile copies
// (timing only) runs ~1.5-1.8, a 4-stage copy ring and an XCD-grouped tile order changed
// nothing, so the LDS traffic of the copies plus the operand reads is what limits it.
// Requirements (checked by the caller): K % 64 == 0, every output part's width % 8 == 0.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int BM = 256;  // rows of x per block
constexpr int BN = 256;  // rows of W per block
constexpr int BK = 64;   // k per step (8 chunks of 8)
constexpr int kChunks = BK / 8;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
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
  const int wm = wave & 3, wn = wave >> 2;  // 4 (m) x 2 (n) waves
  const long long n0 = static_cast<long long>(blockIdx.x) * BN;
  const long long m0 = static_cast<long long>(blockIdx.y) * BM;
  const int K = a.K;
  const int nk = K / BK;
  const long long N = a.N;

  // operand blocks: rows past N (M) lie outside the resource and read as 0
  const long long n_rows = min(static_cast<long long>(BN), N - n0);
  const long long m_rows = min(static_cast<long long>(BM), a.M - m0);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      make_rsrc(static_cast<const bf16_t*>(a.w) + n0 * K, static_cast<int>(n_rows * K * 2));
  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc(static_cast<const bf16_t*>(a.x) + m0 * K, static_cast<int>(m_rows * K * 2));

  // copy of one 64-k step: 1 KiB per direct load = 8 rows x 128 B; lane l fills position
  // l % 8 of row l / 8 with global chunk (l % 8) ^ swz(row)
  constexpr int kRowsPerLoad = 64 / kChunks;  // rows one 1 KiB direct load covers
  const int sub_row = lane / kChunks, pos = lane % kChunks;
  auto issue = [&](__amdgpu_buffer_rsrc_t rsrc, int rows_per_wave, int step, bf16_t* buf)
      __attribute__((always_inline)) {
    const int k_off = step * BK * 2;  // bytes
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i * kRowsPerLoad >= rows_per_wave) break;
      const int row = wave * rows_per_wave + i * kRowsPerLoad + sub_row;
      const int voff = (row * K + ((pos ^ swz(row)) * 8)) * 2;
      lds_ptr_t dst = (lds_ptr_t)(buf + (wave * rows_per_wave + i * kRowsPerLoad) * BK);  // generic -> LDS
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, k_off, 0, 0);
    }
  };
  auto issue_step = [&](int step, bf16_t* abuf, bf16_t* bbuf) __attribute__((always_inline)) {
    issue(w_rsrc, BN / kWaves, step, abuf);
    issue(x_rsrc, BM / kWaves, step, bbuf);
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
    return *reinterpret_cast<const bf16x8*>(buf + (r * kChunks + (c ^ swz(r))) * 8);
  };
  auto compute = [&](const bf16_t* abuf, const bf16_t* bbuf) __attribute__((always_inline)) {
    bf16x8 af[2][4], bfr[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = frag(abuf, wn * 128 + i * 32, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) bfr[0][j] = frag(bbuf, wm * 64 + j * 32, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) {  // next sub-step's fragments go out before this one's MFMAs
#pragma unroll
        for (int i = 0; i < 4; ++i) af[(s + 1) & 1][i] = frag(abuf, wn * 128 + i * 32, s + 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[(s + 1) & 1][j] = frag(bbuf, wm * 64 + j * 32, s + 1);
      }
      // (without these the scheduler moves each read back next to its use, and every MFMA
      // group waits for its own fragments)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bfr[s & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
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

  // store through LDS: accumulator (i, j) register e holds m = wm*64 + j*32 + lane % 32 and
  // n = wn*128 + i*32 + (e/4)*8 + (lane/32)*4 + e%4 of the block tile. Stored as they are,
  // every store would write 16 B into each of 32 rows; instead each wave stages its 64 x 128
  // tile (16 KiB, one eighth of the operand buffers, which the last barrier freed), 16-byte
  // chunk c of row r at chunk c ^ (r mod 16), and writes 256-byte row segments, 16 bytes per
  // lane. Column n belongs to output part p (parts are multiples of 8 wide, so a 16-byte
  // chunk never straddles two parts).
  bf16_t* const stage = (wave < 2 ? as0 : wave < 4 ? as1 : wave < 6 ? bs0 : bs1) + (wave & 1) * (64 * 128);
  static_assert(BN * BK / 2 == 64 * 128 && BM * BK / 2 == 64 * 128, "a wave stages 64 x 128 in half a buffer");
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
        w[1] = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
        const int c = i * 4 + q;
        *reinterpret_cast<u32x2*>(stage + r * 128 + (c ^ (r & 15)) * 8 + (lane >> 5) * 4) = w;
      }
  }
  // the wave's own staging writes are done before its reads (no other wave touches them)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  const int c = lane & 15;
  const long long n = n0 + wn * 128 + c * 8;
  if (n < N) {
    const int p = n < a.part_end[0] ? 0 : (n < a.part_end[1] ? 1 : 2);
    const long long first = p == 0 ? 0 : a.part_end[p - 1];
    const long long width = a.part_end[p] - first;
    bf16_t* const dst = static_cast<bf16_t*>(a.y[p]) + (n - first);
#pragma unroll
    for (int k4 = 0; k4 < 16; ++k4) {
      const int r = k4 * 4 + (lane >> 4);  // row of the wave's tile, chunk c of it
      const long long m = m0 + wm * 64 + r;
      const u32x4 w = *reinterpret_cast<const u32x4*>(stage + r * 128 + (c ^ (r & 15)) * 8);
      if (m < a.M) *reinterpret_cast<u32x4*>(dst + m * width) = w;
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
