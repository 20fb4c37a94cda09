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
//   tile   = 64 keys; K' and V^T tiles staged in LDS, double buffered, the next tile
//            prefetched into registers while the current one is consumed.
//   order  = key tiles from the diagonal downwards, so every row sees its own key in
//            the first tiles it computes.
//   math   = S^T = K' Q'^T and O^T = V^T P^T with v_mfma_f32_32x32x16_bf16: the query
//            index is the MFMA column in both, so each lane owns one query row for the
//            online softmax (row max needs one cross-half exchange) and for the
//            rescaling of its O^T accumulators.
//   launch = 1-D grid remapped so that the query heads sharing a KV head and
//            neighbouring query blocks land on the same XCD (shared K/V in its L2);
//            causal work is ordered longest-first.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int BM = 128;           // query rows per block
constexpr int BN = 64;            // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int KS = kHeadDim + 8;  // K tile row stride (elements): 272 B
constexpr int VS = BN + 8;        // V^T tile row stride (elements): 144 B
constexpr int kKTile = BN * KS;
constexpr int kVTile = kHeadDim * VS;
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 units)

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// K' tile: 64 rows x 256 B contiguous in [B, Hkv, Tp, d]; chunk c -> row c/16, col c%16.
// V^T tile: 128 rows (d) x 128 B (64 keys), row stride Tp.
__device__ __forceinline__ void load_tile(TileRegs& r, const bf16_t* __restrict__ kbase,
                                          const bf16_t* __restrict__ vbase, long long Tp,
                                          int j0, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 4, col = c & 15;
    r.k[i] = *reinterpret_cast<const u32x4*>(kbase + static_cast<long long>(j0 + row) * kHeadDim + col * 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int dr = c >> 3, k8 = c & 7;
    r.v[i] = *reinterpret_cast<const u32x4*>(vbase + static_cast<long long>(dr) * Tp + j0 + k8 * 8);
  }
}

// Within each 16-key group, key r = ii*8 + h*4 + j sits at LDS position h*8 + ii*4 + j, so
// that the 8 keys one lane feeds to an MFMA k-step are 16 contiguous bytes.
__device__ __forceinline__ void store_tile(const TileRegs& r, bf16_t* ks, bf16_t* vs, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 4, col = c & 15;
    *reinterpret_cast<u32x4*>(ks + row * KS + col * 8) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int dr = c >> 3, k8 = c & 7;
    const int g16 = k8 >> 1, ii = k8 & 1;
    bf16_t* row = vs + dr * VS + g16 * 16 + ii * 4;
    *reinterpret_cast<u32x2*>(row) = u32x2{r.v[i][0], r.v[i][1]};      // h = 0 keys
    *reinterpret_cast<u32x2*>(row + 8) = u32x2{r.v[i][2], r.v[i][3]};  // h = 1 keys
  }
}

// kLocal: sliding-window layer (window > 0); otherwise the global causal layer.
template <bool kLocal>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (kKTile + kVTile)];

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

  // ---- key tiles this block touches ------------------------------------------------
  const int last_row = min(i0 + BM, a.T) - 1;
  const int lo = kLocal ? max(0, i0 - a.window + 1) : 0;
  const int kt_lo = lo / BN;
  const int kt_hi = last_row / BN;

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

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = a.scale * 1.4426950408889634f;  // scores in the exp2 domain

  TileRegs regs;
  load_tile(regs, kbase, vbase, a.Tp, kt_hi * BN, tid);
  store_tile(regs, smem, smem + 2 * kKTile, tid);
  __syncthreads();

  for (int kt = kt_hi; kt >= kt_lo; --kt) {
    const int buf = (kt_hi - kt) & 1;
    bf16_t* ks = smem + buf * kKTile;
    bf16_t* vs = smem + 2 * kKTile + buf * kVTile;
    if (kt > kt_lo) load_tile(regs, kbase, vbase, a.Tp, (kt - 1) * BN, tid);

    const int j0 = kt * BN;
    // wave-uniform visibility of this tile for rows r0 .. r0+31
    const bool any = (j0 <= r0 + 31) && (!kLocal || j0 + BN - 1 > r0 - a.window);
    if (any) {
      const bool need_mask = (j0 + BN - 1 > r0) || (kLocal && r0 + 31 - j0 >= a.window);
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(ks + (kb * 32 + n) * KS + s * 16 + hl * 8);
          sacc[kb] = mfma32(__builtin_bit_cast(bf16x8, w), qf[s], sacc[kb]);
        }
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = j0 + kb * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
            const bool ok = key <= qrow && (!kLocal || qrow - key < a.window);
            if (!ok) sacc[kb][e] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
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
        for (int e = 0; e < 16; ++e) sacc[kb][e] = fast_exp2(fmaf(sacc[kb][e], c, -m_use));

      // P^T as MFMA B operand: k-step u covers keys 16u..16u+15 = sacc[u/2][(u%2)*8 ..+7].
      // The row sum adds the same bf16-rounded p that enter the P V product.
      bf16x8 pb[4];
      float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kb = u >> 1, e0 = (u & 1) * 8;
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w[i] = pack_bf16x2(sacc[kb][e0 + 2 * i], sacc[kb][e0 + 2 * i + 1]);
          psum[i] = add_bf16x2(w[i], psum[i]);
        }
        pb[u] = __builtin_bit_cast(bf16x8, w);
      }
      l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(vs + (dt * 32 + n) * VS + u * 16 + hl * 8);
          oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, w), pb[u], oacc[dt]);
        }
      }
    }

    if (kt > kt_lo) store_tile(regs, smem + (buf ^ 1) * kKTile, smem + 2 * kKTile + (buf ^ 1) * kVTile, tid);
    __syncthreads();
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
