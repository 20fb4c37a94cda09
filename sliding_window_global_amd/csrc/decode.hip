// Split-K GQA decode over the KV cache, K rotated on the fly.
//
// 「PLaMo 3アーキテクチャ徹底解析」 §4.4: the cache holds normalised K before RoPE; every
// forward rotates all returned K at renumbered positions 0..S-1 (the query sits at S-1).
// Local layers read a ring of W slots holding the last W-1 tokens plus the new one;
// global layers a contiguous cache. §4.5: softmax(Q'K'^T / sqrt(128)) V; §4.2: the
// Hq/Hkv query heads of a group share one K/V stream, so one block reads each K/V row
// once for the whole group (the read volume of §2.3: 4 B Hkv d A bytes).
//
// Decomposition: block = (split, KV head, sequence), 4 waves; a split is a contiguous
// range of renumbered keys, a multiple of 64. Per 64-key tile, K and V rows are loaded
// with 16-byte coalesced loads (prefetched one tile ahead), staged in LDS, and each wave
// takes 16 keys:
//   S^T[16 keys][16 heads] = K'[16][128] Q'^T  (v_mfma_f32_16x16x32_bf16; heads padded to 16)
//   O^T[128 d][16 heads]  += V^T[128][16] P^T   (v_mfma_f32_16x16x16_bf16)
// Each lane rotates its key's 16 pairs in registers: the fine rope factor of its key is
// fixed for the whole loop (tile starts are multiples of 64), the coarse row comes with
// the tile. The 4 waves' partial softmax states merge in LDS; a second kernel merges the
// splits in a fixed order (deterministic, no atomics).
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int KS = kHeadDim + 8;  // LDS row stride (elements): 272 B
constexpr int kMaxGroup = 16;
constexpr int kPartial = kHeadDim + 2;  // acc[128], m, l
constexpr int kMaxSplit = 256;         // key ranges per (sequence, KV head)
constexpr long long kMinChunk = 256;   // keys per range, at least

struct DecTile {
  u32x4 k[4];
  u32x4 v[4];
  float4 cr;  // 16 B of the coarse rope row (threads 0..31)
};

__device__ __forceinline__ long long slot_of(long long n, int window) {
  return window == 0 ? n : n % window;
}

__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t ks[2][kTile * KS];
  __shared__ __attribute__((aligned(16))) bf16_t vs[2][kTile * KS];
  __shared__ __attribute__((aligned(16))) float2 cs[2][kHalf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m16 = lane & 15;  // MFMA row/col index within 16
  const int g = lane >> 4;    // lane group 0..3
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;

  const long long s_begin = static_cast<long long>(split) * a.plan.chunk;
  const long long s_end = min(a.S, s_begin + a.plan.chunk);
  const bf16_t* __restrict__ kc =
      static_cast<const bf16_t*>(a.k_cache) + (static_cast<long long>(b) * a.Hkv + kvh) * a.cap * kHeadDim;
  const bf16_t* __restrict__ vc =
      static_cast<const bf16_t*>(a.v_cache) + (static_cast<long long>(b) * a.Hkv + kvh) * a.cap * kHeadDim;

  // ---- Q' fragment (B operand of S^T): head m16, dims of the lane's 16 pairs --------
  // slice 0: 16g+e, slice 1: 16g+8+e, slice 2: 64+16g+e, slice 3: 64+16g+8+e (e = 0..7)
  bf16x8 qf[4];
  {
    const bool ok = m16 < G;
    const bf16_t* src = static_cast<const bf16_t*>(a.q_rot) +
                        (static_cast<long long>(b) * a.Hq + kvh * G + (ok ? m16 : 0)) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = (s >> 1) * kHalf + g * 16 + (s & 1) * 8;
      u32x4 w = ok ? *reinterpret_cast<const u32x4*>(src + d0) : u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- fine rope factors of this lane's key (position & 63 is fixed) -----------------
  const int key_in_tile = wave * 16 + m16;
  float2 fine[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) fine[e] = a.rope[key_in_tile * kHalf + g * 16 + e];

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale * 1.4426950408889634f;

  auto load = [&](DecTile& r, long long tb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch >> 4, col = ch & 15;
      const long long s = tb + row;
      if (s < s_end) {
        const long long off = slot_of(a.base + s, a.window) * kHeadDim + col * 8;
        r.k[i] = *reinterpret_cast<const u32x4*>(kc + off);
        r.v[i] = *reinterpret_cast<const u32x4*>(vc + off);
      } else {
        r.k[i] = u32x4{0, 0, 0, 0};
        r.v[i] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < 32)
      r.cr = reinterpret_cast<const float4*>(a.rope + (kRopeFine + (tb >> 6)) * kHalf)[tid];
  };
  auto store = [&](const DecTile& r, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + kThreads * i;
      const int row = ch >> 4, col = ch & 15;
      *reinterpret_cast<u32x4*>(&ks[buf][row * KS + col * 8]) = r.k[i];
      *reinterpret_cast<u32x4*>(&vs[buf][row * KS + col * 8]) = r.v[i];
    }
    if (tid < 32) reinterpret_cast<float4*>(cs[buf])[tid] = r.cr;
  };

  // Software pipeline: two register sets alternate so that two tiles are in flight
  // while the LDS copy of the current one is consumed.
  auto compute = [&](int buf, long long tb) {
    const long long wave_key0 = tb + wave * 16;
    if (wave_key0 < s_end) {  // wave-uniform
      // K' rows: lane reads its key's 4 x 8 dims, rotates its 16 pairs, packs to bf16
      const bf16_t* krow = &ks[buf][key_in_tile * KS];
      u32x4 kw[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int d0 = (s >> 1) * kHalf + g * 16 + (s & 1) * 8;
        kw[s] = *reinterpret_cast<const u32x4*>(krow + d0);
      }
      bf16x8 kf[4];
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {  // hs: slices (hs, hs+2) hold pairs 16g + 8hs + e
        u32x4 lo_w, hi_w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float ra[2], rb[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = e2 * 2 + u;
            const float x0 = u ? hi_bf16(kw[hs][e2]) : lo_bf16(kw[hs][e2]);
            const float x1 = u ? hi_bf16(kw[hs + 2][e2]) : lo_bf16(kw[hs + 2][e2]);
            const float2 cr = cs[buf][g * 16 + hs * 8 + e];
            const float2 f = fine[hs * 8 + e];
            const float zx = cr.x * f.x - cr.y * f.y;
            const float zy = cr.x * f.y + cr.y * f.x;
            ra[u] = x0 * zx - x1 * zy;
            rb[u] = x0 * zy + x1 * zx;
          }
          lo_w[e2] = pack_bf16x2(ra[0], ra[1]);
          hi_w[e2] = pack_bf16x2(rb[0], rb[1]);
        }
        kf[hs] = __builtin_bit_cast(bf16x8, lo_w);
        kf[hs + 2] = __builtin_bit_cast(bf16x8, hi_w);
      }
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qf[s], sacc, 0, 0, 0);

      // S^T layout: lane holds head m16, keys wave_key0 + 4g + i
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long key = wave_key0 + 4 * g + i;
        if (key >= s_end) sacc[i] = -INFINITY;
        mx = fmaxf(mx, sacc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * c);  // finite: key wave_key0 is valid
      const float alpha = fast_exp2(m_run - m_new);
      float p[4];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(sacc[i] * c - m_new);
        psum += p[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const u32x2 pw = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      const s16x4 pb = __builtin_bit_cast(s16x4, pw);

      // V^T fragments: d = 16dt + m16, keys wave_key0 + 4g + i (row-major V in LDS)
      const bf16_t* vrow = &vs[buf][(wave * 16 + 4 * g) * KS + m16];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        oacc[dt] *= alpha;
        const uint32_t v01 = static_cast<uint32_t>(vrow[dt * 16]) |
                             (static_cast<uint32_t>(vrow[KS + dt * 16]) << 16);
        const uint32_t v23 = static_cast<uint32_t>(vrow[2 * KS + dt * 16]) |
                             (static_cast<uint32_t>(vrow[3 * KS + dt * 16]) << 16);
        const s16x4 va = __builtin_bit_cast(s16x4, u32x2{v01, v23});
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[dt], 0, 0, 0);
      }
    }
  };

  const int n_tiles = static_cast<int>((s_end - s_begin + kTile - 1) / kTile);
  DecTile ra, rb;
  load(ra, s_begin);
  if (n_tiles > 1) load(rb, s_begin + kTile);
  store(ra, 0);
  __syncthreads();
  for (int it = 0; it < n_tiles; it += 2) {
    const long long tb = s_begin + static_cast<long long>(it) * kTile;
    if (it + 2 < n_tiles) load(ra, tb + 2 * kTile);
    compute(0, tb);
    if (it + 1 < n_tiles) store(rb, 1);
    __syncthreads();
    if (it + 1 >= n_tiles) break;
    if (it + 3 < n_tiles) load(rb, tb + 3 * kTile);
    compute(1, tb + kTile);
    if (it + 2 < n_tiles) store(ra, 0);
    __syncthreads();
  }

  // ---- merge the 4 waves' states in LDS (reusing the K tile buffers) ----------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  float* red = reinterpret_cast<float*>(&ks[0][0]);  // [4][16][128] acc, then m, l
  float* red_m = red + 4 * kMaxGroup * kHeadDim;
  float* red_l = red_m + 4 * kMaxGroup;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      red[(wave * kMaxGroup + m16) * kHeadDim + dt * 16 + 4 * g + i] = oacc[dt][i];
  if (g == 0) {
    red_m[wave * kMaxGroup + m16] = m_run;
    red_l[wave * kMaxGroup + m16] = l_run;
  }
  __syncthreads();
  float* ws = a.ws;
  for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
    const int h = idx / kHeadDim, d = idx % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w * kMaxGroup + h]);
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = fast_exp2(red_m[w * kMaxGroup + h] - M);
      acc += sc * red[(w * kMaxGroup + h) * kHeadDim + d];
      l += sc * red_l[w * kMaxGroup + h];
    }
    float* dst = ws + ((static_cast<long long>(b) * a.Hq + kvh * G + h) * a.plan.n_split + split) * kPartial;
    dst[d] = acc;
    if (d == 0) {
      dst[kHeadDim] = M;
      dst[kHeadDim + 1] = l;
    }
  }
}

// One block per (sequence, query head): the split states are merged in a fixed order
// (deterministic); thread d owns output component d.
__global__ __launch_bounds__(kHeadDim) void decode_combine_kernel(const float* __restrict__ ws,
                                                                  bf16_t* __restrict__ out,
                                                                  int n_split) {
  __shared__ float wsc[kMaxSplit];
  __shared__ float red[2][kHeadDim / 64];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const float* p = ws + static_cast<long long>(bh) * n_split * kPartial;
  float M = -INFINITY;
  for (int i = tid; i < n_split; i += kHeadDim) M = fmaxf(M, p[i * kPartial + kHeadDim]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  if ((tid & 63) == 0) red[0][wv] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[0][1]);
  float L = 0.f;
  for (int i = tid; i < n_split; i += kHeadDim) {
    const float w = fast_exp2(p[i * kPartial + kHeadDim] - M);
    wsc[i] = w;
    L += w * p[i * kPartial + kHeadDim + 1];
  }
  L = wave_sum(L);
  if ((tid & 63) == 0) red[1][wv] = L;
  __syncthreads();
  L = red[1][0] + red[1][1];
  float acc = 0.f;
#pragma unroll 8
  for (int i = 0; i < n_split; ++i) acc += wsc[i] * p[i * kPartial + tid];
  out[static_cast<long long>(bh) * kHeadDim + tid] = f32_to_bf16(acc / L);
}

}  // namespace

DecodePlan plan_decode(int B, int Hkv, long long S) {
  // Aim for ~2048 blocks (8 per CU) with at least kMinChunk keys each and at most
  // kMaxSplit ranges per (sequence, KV head).
  const long long pairs = static_cast<long long>(B) * Hkv;
  const long long target_blocks = 2048;
  long long n = (target_blocks + pairs - 1) / pairs;
  const long long by_min_chunk = (S + kMinChunk - 1) / kMinChunk;
  if (n > by_min_chunk) n = by_min_chunk;
  if (n > kMaxSplit) n = kMaxSplit;
  if (n < 1) n = 1;
  long long chunk = (S + n - 1) / n;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  DecodePlan p;
  p.chunk = chunk;
  p.n_split = static_cast<int>((S + chunk - 1) / chunk);
  return p;
}

size_t decode_workspace_bytes(int B, int Hq, const DecodePlan& plan) {
  return static_cast<size_t>(B) * Hq * plan.n_split * kPartial * sizeof(float);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(decode_split_kernel, dim3(a.plan.n_split, a.Hkv, a.B), dim3(kThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(kHeadDim), 0, stream, a.ws,
                     static_cast<bf16_t*>(a.out), a.plan.n_split);
  return hipGetLastError();
}

}  // namespace plamo
