// Flash-style causal / sliding-window GQA prefill on gfx950 bf16 MFMA.
//
// 「PLaMo 3アーキテクチャ徹底解析」 §4.5: A = softmax(Q'K'^T / sqrt(128) + M), O = A V per
// query head, KV head h / (Hq/Hkv) (§4.2); §5.1: the mask keeps j <= i and, on local
// layers, i - j < W. The score matrix is never stored (§4.5 notes a kernel need not hold
// it) and key tiles wholly outside every row's window are skipped, so a local layer
// costs O(T W) (§5.3).
//
// Work decomposition
//   block  = 128 query rows of one (sequence, query head); 4 waves x 32 rows.
//   tile   = 64 keys. K' and V^T tiles go straight from HBM into LDS
//            (global_load_lds_dwordx4, no register staging), double buffered, with
//            16-byte chunks XOR-swizzled so that the MFMA operand reads are free of
//            bank conflicts.
//   order  = key tiles from the diagonal downwards, so every row sees its own key in
//            the first tile it computes.
//   math   = S^T = K' Q'^T and O^T = V^T P^T with v_mfma_f32_32x32x16_bf16: the query
//            index is the MFMA column in both, so each lane owns one query row for the
//            online softmax and for the rescaling of its O^T accumulators. K' rows are
//            read in the order that makes each lane's eight consecutive S^T entries
//            eight consecutive keys, which is what the P^T operand of the next MFMA
//            needs; V^T is then read in natural key order.
//   pipeline = the K' tile runs one step ahead of V^T: while the softmax of tile k runs
//            on the vector ALUs, the matrix cores already compute S for tile k+1.
//   softmax = exp2 domain, lazy rescaling (the running max moves only when a row gains
//            more than 2^8), row sums taken from the same bf16-rounded P as P V.
//   launch = 1-D grid remapped so that the query heads sharing a KV head and
//            neighbouring query blocks land on the same XCD (shared K/V in its L2);
//            causal work is ordered longest-first.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int BM = 128;  // query rows per block
constexpr int BN = 64;   // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTileElems = BN * kHeadDim;  // K' tile and V^T tile alike: 16 KiB
constexpr float kRescaleLog2 = 8.f;        // lazy-rescale threshold (log2 units)
// s_waitcnt vmcnt(0) with expcnt / lgkmcnt left alone (gfx9 encoding)
constexpr unsigned kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Key (within a 32-key block) whose K' row feeds MFMA row m: swaps bits 2 and 3, so that
// the S^T entries (m = i*8 + half*4 + j) of one lane hold keys i/2*16 + half*8 + i%2*4 + j.
__device__ __forceinline__ int key_of_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS element offset of 16-byte chunk c of K' row r (16 chunks per row).
__device__ __forceinline__ int k_chunk(int r, int c) { return (r * 16 + (c ^ (r & 15))) * 8; }
// LDS element offset of 16-byte chunk c of V^T row d (8 chunks per row).
__device__ __forceinline__ int v_chunk(int d, int c) { return (d * 8 + (c ^ ((d >> 1) & 7))) * 8; }

// kLocal: sliding-window layer (window > 0); otherwise the global causal layer.
template <bool kLocal>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillArgs a) {
  // Four separate LDS objects (not one indexed array): with the loop unrolled by two,
  // every LDS read names a buffer that no in-flight direct load targets, so the
  // compiler need not wait for those loads before reading.
  __shared__ __attribute__((aligned(1024))) bf16_t ks0[kTileElems];
  __shared__ __attribute__((aligned(1024))) bf16_t ks1[kTileElems];
  __shared__ __attribute__((aligned(1024))) bf16_t vs0[kTileElems];
  __shared__ __attribute__((aligned(1024))) bf16_t vs1[kTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;   // MFMA column = query row within the wave
  const int hl = lane >> 5;  // lane half

  // ---- block -> (b, kv head, query block, query head in group), XCD-aware ----------
  const int G = a.Hq / a.Hkv;
  const int nqb = (a.T + BM - 1) / BM;
  const unsigned total = gridDim.x;
  unsigned logical = blockIdx.x;
  if ((total & 7u) == 0) logical = (blockIdx.x & 7u) * (total >> 3) + (blockIdx.x >> 3);
  const int g_in = logical % G;
  unsigned rest = logical / G;
  const int qb_order = rest % nqb;
  rest /= nqb;
  const int kvh = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int hq = kvh * G + g_in;
  // causal work grows with the query block: longest first (local work is flat)
  const int qb = kLocal ? qb_order : nqb - 1 - qb_order;
  const int i0 = qb * BM;

  const bf16_t* __restrict__ q = static_cast<const bf16_t*>(a.q_rot);
  const bf16_t* __restrict__ kbase =
      static_cast<const bf16_t*>(a.k_rot) + (static_cast<long long>(b) * a.Hkv + kvh) * a.Tp * kHeadDim;
  const bf16_t* __restrict__ vbase =
      static_cast<const bf16_t*>(a.v_t) + (static_cast<long long>(b) * a.Hkv + kvh) * kHeadDim * a.Tp;

  // ---- key tiles this block touches, processed from kt_hi down to kt_lo -------------
  const int last_row = min(i0 + BM, a.T) - 1;
  const int lo = kLocal ? max(0, i0 - a.window + 1) : 0;
  const int kt_hi = last_row / BN;
  const int n_tiles = kt_hi - lo / BN + 1;

  // Each wave moves 4 x 1 KiB of a tile: LDS chunk p = (wave*4 + i)*64 + lane receives
  // the global chunk that the swizzle assigns to p.
  // Per-lane 32-bit element offsets of the 4 chunks each lane moves per tile (a wave-
  // uniform base plus these offsets lets the loads use a scalar base address).
  int k_off[4], v_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = (wave * 4 + i) * 64 + lane;
    const int r = p >> 4, kc = (p & 15) ^ (r & 15);
    k_off[i] = r * kHeadDim + kc * 8;
    const int d = p >> 3, vc = (p & 7) ^ ((d >> 1) & 7);
    v_off[i] = d * static_cast<int>(a.Tp) + vc * 8;
  }
  auto issue_k = [&](int step, bf16_t* buf) {
    const bf16_t* src = kbase + static_cast<long long>(kt_hi - step) * BN * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(src + k_off[i], buf + (wave * 4 + i) * 512, 16, 0, 0);
  };
  auto issue_v = [&](int step, bf16_t* buf) {
    const bf16_t* src = vbase + (kt_hi - step) * BN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(src + v_off[i], buf + (wave * 4 + i) * 512, 16, 0, 0);
  };

  // ---- Q' fragment (MFMA B operand): lane holds dims s*16 + hl*8 .. +7 of its row ----
  const int r0 = i0 + wave * 32;
  const int qrow = r0 + n;
  bf16x8 qf[8];
  {
    const bool ok = qrow < a.T;
    const bf16_t* src = q + (static_cast<long long>(b) * a.T + (ok ? qrow : 0)) * a.Hq * kHeadDim +
                        static_cast<long long>(hq) * kHeadDim + hl * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 w = ok ? *reinterpret_cast<const u32x4*>(src + s * 16) : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // wave-uniform: does tile `step` hold any visible (row, key) pair for rows r0..r0+31?
  auto visible = [&](int step) {
    const int j0 = (kt_hi - step) * BN;
    return (j0 <= r0 + 31) && (!kLocal || j0 + BN - 1 > r0 - a.window);
  };
  // S^T of one tile from K' buffer `buf` (MFMA rows in key_of_row order)
  auto scores = [&](const bf16_t* kbuf, f32x16* sacc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 32 + key_of_row(n);
        const u32x4 w = *reinterpret_cast<const u32x4*>(kbuf + k_chunk(r, 2 * s + hl));
        sacc[kb] = mfma32(__builtin_bit_cast(bf16x8, w), qf[s], sacc[kb]);
      }
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = a.scale * 1.4426950408889634f;  // scores in the exp2 domain

  // ---- prologue: K'(0), V^T(0), K'(1) in LDS; S(0) -----------------------------------
  issue_k(0, ks0);
  issue_v(0, vs0);
  if (n_tiles > 1) issue_k(1, ks1);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  f32x16 s_a[2], s_b[2];  // S of the current and of the next tile, roles alternating
  if (visible(0)) scores(ks0, s_a);
  __syncthreads();  // step 0 refills ks0: every wave must be done reading K'(0)

  // One step; `k_next`, `v_cur` are read, `k_fill`, `v_fill` receive direct loads.
  auto run_step = [&](int step, const bf16_t* k_next, const bf16_t* v_cur, bf16_t* k_fill,
                      bf16_t* v_fill, f32x16* s_cur, f32x16* s_next) {
      // LDS holds K'(step+1) in ks[(step+1)&1] and V^T(step) in vs[step&1]; the buffers
      // refilled here were last read before the previous barrier.
      if (step + 2 < n_tiles) issue_k(step + 2, k_fill);
      if (step + 1 < n_tiles) issue_v(step + 1, v_fill);
      if (step + 1 < n_tiles && visible(step + 1)) scores(k_next, s_next);

      if (visible(step)) {
        const int j0 = (kt_hi - step) * BN;
        const bool need_mask = (j0 + BN - 1 > r0) || (kLocal && r0 + 31 - j0 >= a.window);
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = j0 + kb * 32 + (e >> 3) * 16 + hl * 8 + (e & 7);
              const bool ok = key <= qrow && (!kLocal || qrow - key < a.window);
              if (!ok) s_cur[kb][e] = -INFINITY;
            }
        }
        float mx = s_cur[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s_cur[kb][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // Lazy rescaling: the running reference max only moves (and O, l are only rescaled)
        // when some row of the wave gains more than 2^8 over it, so p stays <= 256.
        const float mx_c = mx * c;
        if (__builtin_amdgcn_ballot_w64(mx_c > m_run + kRescaleLog2) != 0) {  // wave-uniform
          const float m_new = fmaxf(m_run, mx_c);
          const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
          m_run = m_new;
        }
        // a row whose keys so far are all masked has m_run = -inf and only -inf scores here
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) s_cur[kb][e] = fast_exp2(fmaf(s_cur[kb][e], c, -m_use));

        // P^T as MFMA B operand: k-step u covers keys 16u..16u+15 = s_cur[u/2][(u%2)*8 ..+7].
        // The row sum adds the same bf16-rounded p that enter the P V product.
        bf16x8 pb[4];
        float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kb = u >> 1, e0 = (u & 1) * 8;
          u32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            w[i] = pack_bf16x2(s_cur[kb][e0 + 2 * i], s_cur[kb][e0 + 2 * i + 1]);
            psum[i] = add_bf16x2(w[i], psum[i]);
          }
          pb[u] = __builtin_bit_cast(bf16x8, w);
        }
        l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(v_cur + v_chunk(dt * 32 + n, 2 * u + hl));
            oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, w), pb[u], oacc[dt]);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
  };
  for (int step = 0; step < n_tiles; step += 2) {
    run_step(step, ks1, vs0, ks0, vs1, s_a, s_b);
    if (step + 1 < n_tiles) run_step(step + 1, ks0, vs1, ks1, vs0, s_b, s_a);
  }

  // ---- normalise and store: lane writes d = dt*32 + i*8 + hl*4 + 0..3 of its row ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qrow < a.T) {
    const float inv = 1.f / l_tot;
    bf16_t* dst = static_cast<bf16_t*>(a.out) +
                  (static_cast<long long>(b) * a.T + qrow) * a.Hq * kHeadDim +
                  static_cast<long long>(hq) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = dt * 32 + i * 8 + hl * 4;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[dt][i * 4 + 0] * inv, oacc[dt][i * 4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[dt][i * 4 + 2] * inv, oacc[dt][i * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(dst + d0) = w;
      }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const long long nqb = (a.T + BM - 1) / BM;
  const long long blocks = nqb * a.Hq * a.B;
  if (a.window > 0)
    hipLaunchKernelGGL(prefill_bf16_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace plamo
