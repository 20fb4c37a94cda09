// Split-K GQA decode for wide heads (d = 256, 512) over a post-RoPE KV cache.
//
// 「PLaMo 3アーキテクチャ徹底解析」 §8 table: the Gemma-4-shaped layers (local d = 256,
// global d = 512) keep K in the cache after RoPE, so the cache rows are the attention
// operands as stored; §4.5: softmax(Q'K'^T * scale) V with the layer's factor as `scale`;
// §4.2: the Hq/Hkv query heads of a group share one K/V stream, so one block reads each
// K/V row once for the whole group.
//
// Decomposition (as for d = 128, with the rotation gone and the rows four times longer):
// block = (split, KV head, sequence), 4 waves; a split is a contiguous range of renumbered
// keys cut into 64-key tiles; wave w owns keys 16w .. 16w+15 of every tile and streams
// them without block barriers: K rows global -> registers in the MFMA operand layout
// (d/32 x 16 B per lane), V rows global -> LDS by direct loads (rows padded by 16 bytes, so
// the transposed operand reads are free of bank conflicts), two sub-tiles per wave in
// flight or in use.
//   S^T[16 keys][16 heads] = K'[16][d] Q'^T     (v_mfma_f32_16x16x32_f16: Q' arrives as IEEE
//                                               halves, the bf16 cache rows convert exactly;
//                                               heads padded to 16)
//   O^T[d][16 heads]      += V^T[d][16] P^T     (v_mfma_f32_16x16x16_bf16)
// The softmax reference moves lazily (only when a head's score exceeds it by 2^8). The 4
// waves' states merge in LDS; with one split the block writes the output, otherwise a
// second kernel merges the splits in a fixed order (deterministic, no atomics).
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 64;      // keys per tile = kWaves x kSub
constexpr int kSub = 16;       // keys per wave per tile
constexpr int kMaxGroup = 16;
constexpr float kRescaleLog2 = 8.f;

// Cache policy of the V row loads: non-temporal (every row is read once, in whole 16-byte
// chunks of consecutive rows; a plain streaming read measured ~7.0 TB/s with it, ~6.1-6.2
// TB/s without). K rows stay cached: each of their 128-byte lines is fetched by two loads,
// and non-temporal K loads made the decode slower (d = 512: 6.09 against 6.19 TB/s with
// both non-temporal; 6.88 with cached K and non-temporal V).
constexpr int kNonTemporal = 2;

constexpr unsigned wait_vmcnt(int n) { return 0x0F70u | (n & 15) | ((n >> 4) << 14); }

enum CacheMode { kContiguous = 0, kRing = 1, kSmallRing = 2 };

template <int D>
struct WideShape {
  static constexpr int kKC = D / 32;                      // 16-byte K chunks per lane per key
  static constexpr int kVRow = D + 8;                     // padded V row in LDS (elements)
  static constexpr int kRC = kVRow / 8;                   // 16-byte slots per padded row
  static constexpr int kVLoads = (kSub * kRC + 63) / 64;  // direct loads per V sub-tile
  static constexpr int kVSlot = kVLoads * 64 * 8;         // elements per V sub-tile slot
  static constexpr int kLoads = kKC + kVLoads;            // loads per issue
  static constexpr int kDT = D / 16;                      // 16-dim blocks of O^T
  // d = 512: Q' is read from LDS at each use (rows padded by 16 bytes), since Q' and two
  // K slots in registers would leave too few for the rest; d = 256 keeps it in registers.
  static constexpr bool kQLds = D == 512;
  static constexpr int kQRow = D + 8;
};

template <int kMode, int D>
__global__ __launch_bounds__(kThreads, D == 256 ? 2 : 1) void decode_wide_kernel(DecodeArgs a) {
  using W = WideShape<D>;
  __shared__ __attribute__((aligned(16))) bf16_t vs0[kWaves][W::kVSlot];
  __shared__ __attribute__((aligned(16))) bf16_t vs1[kWaves][W::kVSlot];
  __shared__ float red_m[kWaves * kMaxGroup], red_l[kWaves * kMaxGroup];
  __shared__ __attribute__((aligned(16))) f16_t q_s[W::kQLds ? kMaxGroup * W::kQRow : 8];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m16 = lane & 15;
  const int g = lane >> 4;
  const bool range_major = a.seq_pos != nullptr;  // (ragged: key range slowest, see the launcher)
  const int split = range_major ? blockIdx.z : blockIdx.x;
  const int kvh = range_major ? blockIdx.x : blockIdx.y;
  const int b = range_major ? blockIdx.y : blockIdx.z;
  const int G = a.Hq / a.Hkv;

  long long S = a.S, base = a.base;
  if (a.seq_pos) {
    const SeqPos sp = seq_pos_of(a.seq_pos, nullptr, a.pos_offset, 1, a.window, b);
    S = sp.kept + 1;
    base = sp.pos - sp.kept;
  }
  const long long s_begin = static_cast<long long>(split) * a.plan.chunk;
  if (s_begin >= S) return;  // block-uniform
  const long long s_end = min(S, s_begin + a.plan.chunk);
  const int n_tiles = static_cast<int>((s_end - s_begin + kTile - 1) / kTile);
  const bf16_t* __restrict__ kc =
      static_cast<const bf16_t*>(a.k_cache) + (static_cast<long long>(b) * a.Hkv + kvh) * a.cap * D;
  const bf16_t* __restrict__ vc =
      static_cast<const bf16_t*>(a.v_cache) + (static_cast<long long>(b) * a.Hkv + kvh) * a.cap * D;

  // ---- Q' fragment (B operand of S^T): head m16, dims 32 s + 8 g .. +7 ----------------
  const bool q_ok = m16 < G;
  u32x4 qw[W::kQLds ? 1 : W::kKC];
  f16x8 qf[W::kQLds ? 1 : W::kKC];
  if (W::kQLds) {  // the block's G heads into LDS, padding heads zero
    const f16_t* src = static_cast<const f16_t*>(a.q_rot) + (static_cast<long long>(b) * a.Hq + kvh * G) * D;
    for (int i = threadIdx.x; i < kMaxGroup * (D / 8); i += kThreads) {
      const int h = i / (D / 8), cc = i % (D / 8);
      const u32x4 w = h < G ? reinterpret_cast<const u32x4*>(src + h * D)[cc] : u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4*>(q_s + h * W::kQRow + cc * 8) = w;
    }
    __syncthreads();
  } else {
    const f16_t* src = static_cast<const f16_t*>(a.q_rot) +
                       (static_cast<long long>(b) * a.Hq + kvh * G + (q_ok ? m16 : 0)) * D + g * 8;
#pragma unroll
    for (int s = 0; s < (W::kQLds ? 1 : W::kKC); ++s) qw[s] = *reinterpret_cast<const u32x4*>(src + s * 32);
  }
  auto q_frag = [&](int s) __attribute__((always_inline)) {
    if (W::kQLds) return *reinterpret_cast<const f16x8*>(q_s + m16 * W::kQRow + s * 32 + g * 8);
    return qf[W::kQLds ? 0 : s];
  };

  // V direct load i, lane l fills padded slot p = 64 i + l: row p / kRC, chunk p % kRC (the
  // pad chunk and the slots past 16 rows copy a chunk of the last row, never read). Formed
  // at each issue: holding them would cost 2 kVLoads registers.
  // Tiles are issued in order; past the end the last tile is issued again (the same count
  // of loads stays in flight), and keys past s_end read the last key (their p is zero).
  const int key_in_tile = wave * kSub + m16;
  int t_issue = 0;
  long long tb_issue = s_begin;
  int s0 = kMode != kContiguous ? static_cast<int>((base + s_begin) % a.window) : 0;
  auto cache_row = [&](int j) __attribute__((always_inline)) {
    j = min(j, static_cast<int>(s_end - 1 - tb_issue));
    if (kMode == kContiguous) return base + tb_issue + j;
    int sl = s0 + j;
    if (kMode == kRing) sl -= sl >= a.window ? a.window : 0;
    else sl %= a.window;
    return static_cast<long long>(sl);
  };
  auto issue = [&](u32x4* kw, bf16_t* vslot) __attribute__((always_inline)) {
    {
      const bf16_t* row = kc + cache_row(key_in_tile) * D + g * 8;
#pragma unroll
      for (int s = 0; s < W::kKC; ++s) kw[s] = *reinterpret_cast<const u32x4*>(row + s * 32);
    }
#pragma unroll
    for (int i = 0; i < W::kVLoads; ++i) {
      const int p = 64 * i + lane;
      const int v_row = min(p / W::kRC, kSub - 1), v_col = min(p % W::kRC, D / 8 - 1);
      const bf16_t* src = vc + cache_row(wave * kSub + v_row) * D + v_col * 8;
      __builtin_amdgcn_global_load_lds(src, vslot + i * 512, 16, 0, kNonTemporal);
    }
    if (t_issue + 1 < n_tiles) {
      ++t_issue;
      tb_issue += kTile;
      if (kMode == kRing) {
        s0 += kTile;
        s0 -= s0 >= a.window ? a.window : 0;
      } else if (kMode == kSmallRing) {
        s0 = (s0 + kTile) % a.window;
      }
    }
  };

  f32x4 oacc[W::kDT];
#pragma unroll
  for (int dt = 0; dt < W::kDT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale * 1.4426950408889634f;

  auto compute = [&](int t, const u32x4* kw, const bf16_t* vslot) __attribute__((always_inline)) {
    const long long key0 = s_begin + static_cast<long long>(t) * kTile + wave * kSub;
    if (key0 >= s_end) return;  // wave-uniform
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < W::kKC; ++s) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = bf16x2_to_f16x2(kw[s][i]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, w), q_frag(s), sacc, 0, 0, 0);
    }
    // S^T layout: lane holds head m16, keys key0 + 4g + i
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sacc[i] *= c;
      if (key0 + 4 * g + i >= s_end) sacc[i] = -INFINITY;
      mx = fmaxf(mx, sacc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // finite: key key0 is valid
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0) {  // wave-uniform
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < W::kDT; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    u32x2 pw;
    pw[0] = pack_bf16x2(fast_exp2(sacc[0] - m_run), fast_exp2(sacc[1] - m_run));
    pw[1] = pack_bf16x2(fast_exp2(sacc[2] - m_run), fast_exp2(sacc[3] - m_run));
    l_run = add_bf16x2(pw[1], add_bf16x2(pw[0], l_run));  // the same bf16 p as P V
    const s16x4 pb = __builtin_bit_cast(s16x4, pw);
    // V^T fragments: d = 16 dt + m16, keys 4g + i of the sub-tile (padded rows in LDS)
    const bf16_t* vrow = vslot + (4 * g) * W::kVRow + m16;
#pragma unroll
    for (int dt = 0; dt < W::kDT; ++dt) {
      s16x4 va;
#pragma unroll
      for (int i = 0; i < 4; ++i) va[i] = static_cast<short>(vrow[i * W::kVRow + dt * 16]);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[dt], 0, 0, 0);
    }
  };

  // ---- two sub-tiles per wave: compute t while t+1 lands ------------------------------
  u32x4 k0[W::kKC], k1[W::kKC];
  bf16_t* const v0 = vs0[wave];
  bf16_t* const v1 = vs1[wave];
  issue(k0, v0);  // tile 0
  // Q' (loaded before the tile) is in once all but the tile's loads have landed
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(W::kLoads));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < (W::kQLds ? 0 : W::kKC); ++s) asm volatile("" : "+v"(qw[s]));
#pragma unroll
  for (int s = 0; s < (W::kQLds ? 0 : W::kKC); ++s) qf[s] = __builtin_bit_cast(f16x8, q_ok ? qw[s] : u32x4{0, 0, 0, 0});
  constexpr unsigned kOneBehind = wait_vmcnt(W::kLoads);
  int t = 0;
  for (; t + 2 <= n_tiles; t += 2) {
    issue(k1, v1);  // tile t + 1
    __builtin_amdgcn_s_waitcnt(kOneBehind);
    compute(t, k0, v0);
    issue(k0, v0);  // tile t + 2
    __builtin_amdgcn_s_waitcnt(kOneBehind);
    compute(t + 1, k1, v1);
  }
  if (t < n_tiles) {
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    compute(t, k0, v0);
  }
  // the repeated tile past the end may still be landing in LDS
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  __syncthreads();

  // ---- merge the 4 waves' states in LDS (reusing the V slots) -------------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // [16 heads][d] accumulators of waves 0, 1 in vs0 and of waves 2, 3 in vs1
  static_assert(sizeof(vs0) >= 2 * kMaxGroup * D * sizeof(float), "merge buffer");
  auto red_of = [&](int w) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(w < 2 ? &vs0[0][0] : &vs1[0][0]) + (w & 1) * kMaxGroup * D;
  };
  {
    float* mine = red_of(wave);
#pragma unroll
    for (int dt = 0; dt < W::kDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[m16 * D + dt * 16 + 4 * g + i] = oacc[dt][i];
  }
  if (g == 0) {
    red_m[wave * kMaxGroup + m16] = m_run;
    red_l[wave * kMaxGroup + m16] = l_run;
  }
  __syncthreads();
  const bool single = a.plan.n_split == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w * kMaxGroup + h]);
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(red_m[w * kMaxGroup + h] - M);  // 0 for a wave with no key
      acc += sc * red_of(w)[h * D + d];
      l += sc * red_l[w * kMaxGroup + h];
    }
    const long long bh = static_cast<long long>(b) * a.Hq + kvh * G + h;
    if (single) {
      static_cast<bf16_t*>(a.out)[bh * D + d] = f32_to_bf16(acc / l);
    } else {
      float* dst = a.ws + (bh * a.plan.n_split + split) * (D + 2);
      dst[d] = acc;
      if (d == 0) {
        dst[D] = M;
        dst[D + 1] = l;
      }
    }
  }
}

// One block per (sequence, query head), thread d owns output component d; the split
// states merge in a fixed order. A sequence of a ragged batch merges only its own ranges.
template <int D>
__global__ __launch_bounds__(D) void decode_wide_combine_kernel(DecodeArgs a) {
  constexpr int kMaxSplit = 256;
  __shared__ float ms[kMaxSplit], ls[kMaxSplit];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  int n_split = a.plan.n_split;
  if (a.seq_pos) {
    const SeqPos sp = seq_pos_of(a.seq_pos, nullptr, a.pos_offset, 1, a.window, bh / a.Hq);
    n_split = static_cast<int>((sp.kept + 1 + a.plan.chunk - 1) / a.plan.chunk);
  }
  const float* p = a.ws + static_cast<long long>(bh) * a.plan.n_split * (D + 2);
  for (int i = tid; i < n_split; i += D) {
    ms[i] = p[i * (D + 2) + D];
    ls[i] = p[i * (D + 2) + D + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < n_split; ++i) M = fmaxf(M, ms[i]);
  float L = 0.f, acc = 0.f;
  for (int i = 0; i < n_split; ++i) {
    const float w = fast_exp2(ms[i] - M);
    L += w * ls[i];
    acc += w * p[i * (D + 2) + tid];
  }
  static_cast<bf16_t*>(a.out)[static_cast<long long>(bh) * D + tid] = f32_to_bf16(acc / L);
}

template <int D>
hipError_t launch_wide(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid = a.seq_pos ? dim3(a.Hkv, a.B, a.plan.n_split) : dim3(a.plan.n_split, a.Hkv, a.B);
  if (a.window == 0)
    hipLaunchKernelGGL((decode_wide_kernel<kContiguous, D>), grid, dim3(kThreads), 0, stream, a);
  else if (a.window >= kTile)
    hipLaunchKernelGGL((decode_wide_kernel<kRing, D>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_wide_kernel<kSmallRing, D>), grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.plan.n_split == 1) return e;
  hipLaunchKernelGGL(decode_wide_combine_kernel<D>, dim3(a.B * a.Hq), dim3(D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_wide_bf16(const DecodeArgs& a, hipStream_t stream) {
  return a.d == 256 ? launch_wide<256>(a, stream) : launch_wide<512>(a, stream);
}

}  // namespace plamo
