// Projection GEMM of the attention sublayer on gfx950 bf16 MFMA:
// y[M, N] = x[M, K] W[N, K]^T (both operands K-contiguous, fp32 accumulation, bf16 out).
// 「PLaMo 3アーキテクチャ徹底解析」 §4.1: the fused QKV projection (N = (Hq + 2 Hkv) d), whose
// output columns are split into Q | K | V; the epilogue writes each part to its own tensor.
// §4.5: the output projection (K = Hq d, N = hidden).
//
// block  = 256 rows of x (m) x BN rows of W (n), BN = 256 or 320, 8 waves in a 4 (m) x 2 (n)
//          grid, each wave 64 m x BN/2 n = 2 x BN/64 blocks of v_mfma_f32_32x32x16_bf16 (128 or
//          160 fp32 accumulators). W fragments are the MFMA A operand (32 n x 16 k), x fragments
//          the B operand, so a lane's accumulators hold one m and runs of 4 consecutive n; the
//          output goes out through LDS as whole row segments. The launch takes the column tile
//          with the fewer rounds of one block per CU, weighted by its width (a 5120-wide output:
//          16 tiles of 320 instead of 20 of 256, 2 rounds instead of 2.5 at M = 8192).
// tiles  = 64 k per step: W tiles BN x 64 (32 or 40 KiB) and x tiles 256 x 64 (32 KiB), double
//          buffered (128 or 144 KiB, one block per CU), copied global -> LDS by buffer loads with
//          the LDS bit (a resource per operand block bounds every read; rows past M or N read
//          0). LDS rows are 128 B; the 16-byte chunk c of row r sits at position c ^ ((r >> 1) &
//          7), so that the eight lanes of a row read one contiguous 128 B of global memory and
//          the 16 rows of a quarter-wave's fragment read fall into distinct banks. The next
//          sub-step's fragments are read while the current sub-step's MFMAs run.
// Measured on the sublayer shapes: ~1.2-1.26 PFLOP/s; the same kernel without the tile copies
// (timing only) ran ~1.5-1.8 before the output went through LDS, a 4-stage copy ring and an
// XCD-grouped tile order changed nothing, so the LDS traffic of the copies plus the operand
// reads is what limits it.
// Requirements (checked by the caller): K % 64 == 0, every output part's width % 8 == 0.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int BM = 256;  // rows of x per block
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

// BN: rows of W per block, 256 or 320; a wave covers 64 m x BN/2 n, NI = BN/64 MFMA blocks
// of 32 n (320 = 2 x 5 x 32: a 5120-wide output in 16 column tiles instead of 20)
template <int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NI = BN / 64;   // 32-wide n blocks per wave
  constexpr int WN = BN / 2;    // n per wave
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

  f32x16 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
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
    bf16x8 af[2][NI], bfr[2][2];
#pragma unroll
    for (int i = 0; i < NI; ++i) af[0][i] = frag(abuf, wn * WN + i * 32, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) bfr[0][j] = frag(bbuf, wm * 64 + j * 32, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) {  // next sub-step's fragments go out before this one's MFMAs
#pragma unroll
        for (int i = 0; i < NI; ++i) af[(s + 1) & 1][i] = frag(abuf, wn * WN + i * 32, s + 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[(s + 1) & 1][j] = frag(bbuf, wm * 64 + j * 32, s + 1);
      }
      // (without these the scheduler moves each read back next to its use, and every MFMA
      // group waits for its own fragments)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NI; ++i)
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
  // n = wn*WN + i*32 + (e/4)*8 + (lane/32)*4 + e%4 of the block tile. Stored as they are,
  // every store would write 16 B into each of 32 rows; instead each wave stages 32 rows x WN
  // at a time (8 KiB at BN = 256, 10 KiB at 320: a quarter of one W buffer, free after the
  // last barrier) and writes whole row segments of WN columns, 16 bytes per lane (at BN = 256
  // the 16-byte chunk c of row r sits at c ^ (r mod 16), which keeps the staging writes free
  // of bank conflicts). Column n belongs to output part p (parts are multiples of 8 wide, so
  // a 16-byte chunk never straddles two parts).
  constexpr int CW = WN / 8;            // 16-byte chunks per staged row
  constexpr int kRowsPerRead = 64 / CW;  // rows one 64-lane read covers (16 or 20 lanes each)
  static_assert(4 * 32 * WN == BN * BK, "four waves stage 32 rows x WN in one W buffer");
  auto phys = [](int r, int c) __attribute__((always_inline)) { return CW == 16 ? (c ^ (r & 15)) : c; };
  bf16_t* const stage = (wave < 4 ? as0 : as1) + (wave & 3) * (32 * WN);
  const int c = lane % CW;
  const int r_lane = lane / CW;  // row of the read within its group (lanes past the last group idle)
  const long long n = n0 + wn * WN + c * 8;
  const bool col_ok = r_lane < kRowsPerRead && n < N;
  int p = 0;
  long long first = 0, width = 0;
  if (col_ok) {
    p = n < a.part_end[0] ? 0 : (n < a.part_end[1] ? 1 : 2);
    first = p == 0 ? 0 : a.part_end[p - 1];
    width = a.part_end[p] - first;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = lane & 31;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
        w[1] = pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
        *reinterpret_cast<u32x2*>(stage + r * WN + phys(r, i * 4 + q) * 8 + (lane >> 5) * 4) = w;
      }
    // the wave's own staging writes are done before its reads (no other wave touches them)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    if (col_ok) {
      bf16_t* const dst = static_cast<bf16_t*>(a.y[p]) + (n - first);
#pragma unroll
      for (int k = 0; k < (32 + kRowsPerRead - 1) / kRowsPerRead; ++k) {
        const int rr = k * kRowsPerRead + r_lane;  // staged row, chunk c of it
        const long long m = m0 + wm * 64 + j * 32 + rr;
        if (rr < 32 && m < a.M)
          *reinterpret_cast<u32x4*>(dst + m * width) = *reinterpret_cast<const u32x4*>(stage + rr * WN + phys(rr, c) * 8);
      }
    }
    if (j == 0) {  // the reads are done before the next half's writes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t stream) {
  // Column tiles of 256 or 320: the one whose rounds of one block per CU times its width is
  // smaller (e.g. N = 5120, M = 8192: 640 blocks of 256 are 2.5 rounds, 512 blocks of 320 are 2;
  // a tie goes to 320, which reads fewer operand bytes per FLOP).
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const long long mb = (a.M + BM - 1) / BM;
  auto cost = [&](long long bn) { return ((a.N + bn - 1) / bn * mb + cus - 1) / cus * bn; };
  if (cost(320) <= cost(256)) {
    const dim3 grid(static_cast<unsigned>((a.N + 319) / 320), static_cast<unsigned>(mb));
    hipLaunchKernelGGL(gemm_bf16_kernel<320>, grid, dim3(kThreads), 0, stream, a);
  } else {
    const dim3 grid(static_cast<unsigned>((a.N + 255) / 256), static_cast<unsigned>(mb));
    hipLaunchKernelGGL(gemm_bf16_kernel<256>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace plamo
