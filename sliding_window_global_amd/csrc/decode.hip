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
// range of renumbered keys, a multiple of 64 long, cut into 64-key tiles. Wave w owns
// keys 16w .. 16w+15 of every tile and streams them on its own, without block barriers:
//   K rows   global -> registers, already in the MFMA operand layout (4 x 16 B per lane),
//   V rows   global -> LDS by direct loads, four rows per load; the 16-byte chunks of a row
//            are stored XOR-swizzled by the row index (each lane loads the chunk its LDS
//            slot should hold), so that the transposing operand reads below, 32 B of eight
//            rows at a time, are free of bank conflicts without padding,
//   rope     the tile's coarse factor row global -> LDS by one direct load,
// three sub-tiles per wave in flight or in use (a ring unrolled by three).
//   S^T[16 keys][16 heads] = K'[16][128] Q'^T  (v_mfma_f32_16x16x32_f16: Q' arrives as IEEE
//                                              halves, K' is rotated in fp32 and rounded to
//                                              half; heads padded to 16)
//   O^T[128 d][16 heads]  += V^T[128][16] P^T   (v_mfma_f32_16x16x16_bf16)
// Each lane rotates its key's 16 pairs in registers: the fine rope factor of its key is
// fixed for the whole loop (tile starts are multiples of 64), the coarse row comes with
// the tile. The softmax reference max moves lazily (only when a head's score exceeds it
// by 2^8). The 4 waves' partial states merge in LDS; with one split the block writes the
// output, otherwise a second kernel merges the splits in a fixed order (deterministic,
// no atomics).
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace plamo {

// Split-K partial results of plamo_attn_decode_noalloc, for callers that cannot allocate:
// one array per GPU, held until the process ends. Every call on a GPU reuses that GPU's
// array (calls that overlap on one GPU race). Host code never passes the array's name to a
// kernel: it passes the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = static_cast<float*>(p);
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 64;                  // keys per tile = kWaves x kSub
constexpr int kSub = 16;                   // keys per wave per tile
constexpr int kMaxGroup = 16;
constexpr int kPartial = kHeadDim + 2;     // acc[128], m, l
constexpr int kMaxSplit = 256;             // key ranges per (sequence, KV head)
constexpr int kVLoads = kSub * kHeadDim / 8 / 64;  // direct loads per V sub-tile (16 B a lane): 4
constexpr int kVSlot = kSub * kHeadDim;    // elements of one V sub-tile in LDS
// 16-byte chunk c of V row r of a sub-tile sits at chunk c ^ v_swizzle(r) of that row
__device__ __forceinline__ int v_swizzle(int r) { return 2 * (r & 7); }
constexpr float kRescaleLog2 = 8.f;        // lazy-rescale threshold (log2 units)
// loads per tile issue: K rows, V rows and (when K is rotated here) the coarse rope row
template <bool kRotate>
constexpr int kLoadsPerIssue = 4 + kVLoads + (kRotate ? 1 : 0);

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Cache policy of the V row loads: non-temporal (every row is read once, whole rows per
// load). Measured on a plain 4 GiB streaming read: ~7.0 TB/s with it, ~6.1-6.2 TB/s without,
// whatever the grid. The K row loads stay cached: each 128-byte line of a K row is fetched
// by two loads (64 B of 16 rows each), and non-temporal K loads fetched some lines twice
// from HBM (period local layer 80 MB per launch against 74 MB cached, 67 MB of rows).
constexpr int kNonTemporal = 2;

// s_waitcnt vmcnt(n), expcnt / lgkmcnt left alone (gfx9 encoding: vmcnt bits 3:0, 15:14)
constexpr unsigned wait_vmcnt(int n) { return 0x0F70u | (n & 15) | ((n >> 4) << 14); }

// Cache addressing: contiguous (global layer), ring of W >= 64 slots (at most one wrap per
// 64-key tile), ring of W < 64 slots.
enum CacheMode { kContiguous = 0, kRing = 1, kSmallRing = 2 };

// kRotate: the cache holds K before RoPE (rotated here at renumbered positions); otherwise
// it holds K already rotated at absolute positions and is used as stored.
// kFused: the one-launch step (see DecodeArgs::fused): Q' is formed here from the projected
// query, the block holding the newest key first writes that token's K and V into the cache,
// and the key ranges of a (sequence, KV head) are merged by whichever of its blocks ends last.
template <int kMode, bool kRotate, bool kFused>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(DecodeArgs a) {
  constexpr int kLoads = kLoadsPerIssue<kRotate>;
  // three ring slots, separate LDS objects so that reads of one slot never wait for the
  // direct loads in flight into the others
  __shared__ __attribute__((aligned(16))) bf16_t vs0[kWaves][kVSlot];
  __shared__ __attribute__((aligned(16))) bf16_t vs1[kWaves][kVSlot];
  __shared__ __attribute__((aligned(16))) bf16_t vs2[kWaves][kVSlot];
  __shared__ __attribute__((aligned(16))) float2 cs0[kWaves][2 * kHalf];
  __shared__ __attribute__((aligned(16))) float2 cs1[kWaves][2 * kHalf];
  __shared__ __attribute__((aligned(16))) float2 cs2[kWaves][2 * kHalf];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m16 = lane & 15;  // MFMA row/col index within 16
  const int g = lane >> 4;    // lane group 0..3
  // a ragged batch and the one-launch step launch their key ranges range-major (see the launcher)
  const bool range_major = kFused || a.seq_pos != nullptr;
  const int split = range_major ? blockIdx.z : blockIdx.x;
  const int kvh = range_major ? blockIdx.x : blockIdx.y;
  const int b = range_major ? blockIdx.y : blockIdx.z;
  const int G = a.Hq / a.Hkv;

  // keys of this sequence: all of them on a uniform batch, its own count on a ragged one
  long long S = a.S, base = a.base;
  if (a.seq_pos) {
    const SeqPos sp = seq_pos_of(a.seq_pos, nullptr, a.pos_offset, 1, a.window, b);
    S = sp.kept + 1;
    base = sp.pos - sp.kept;
  }
  const long long s_begin = static_cast<long long>(split) * a.plan.chunk;
  if (s_begin >= S) return;  // (ragged) a shorter sequence has fewer ranges; block-uniform
  const long long s_end = min(S, s_begin + a.plan.chunk);
  const int n_tiles = static_cast<int>((s_end - s_begin + kTile - 1) / kTile);
  const bf16_t* __restrict__ kc =
      static_cast<const bf16_t*>(a.k_cache) + (static_cast<long long>(b) * a.Hkv + kvh) * a.cap * kHeadDim;
  const bf16_t* __restrict__ vc =
      static_cast<const bf16_t*>(a.v_cache) + (static_cast<long long>(b) * a.Hkv + kvh) * a.cap * kHeadDim;

  // ---- one-launch step: the new token's K and V into the cache -----------------------
  // 「PLaMo 3アーキテクチャ徹底解析」 §3.2 / §4.3: k is normalised (gain c + w, eps) over its
  // 128 components; §4.4: the cache stores it before RoPE (post-RoPE order: rotated at its
  // absolute position first) and V as given, token p in slot p (global) or p mod W (local).
  // Only the block whose range ends with the newest key (renumbered S - 1) reads that key,
  // and in it only the wave that owns that key's place in its tile: that wave writes the row
  // (two components per lane) and waits for the stores before it issues any load. (It is
  // also the only wave that uses the row as the filler of keys past the range end: a wave
  // before it has a full tile, a wave after it has no key there and skips the tile.)
  __shared__ float2 zq[kHalf];  // (one-launch step) rotation factors of the query position
  if (kFused && s_end == S) {  // block-uniform
    if (wave == static_cast<int>(((S - 1 - s_begin) & (kTile - 1)) / kSub)) {
      const long long p = a.pos_offset;
      const long long slot = a.window == 0 ? p : p % a.window;
      const long long row = (static_cast<long long>(b) * a.Hkv + kvh) * a.cap + slot;
      const uint32_t* ksrc = static_cast<const uint32_t*>(a.k_in) + (static_cast<long long>(b) * a.Hkv + kvh) * kHalf;
      const uint32_t* vsrc = static_cast<const uint32_t*>(a.v_in) + (static_cast<long long>(b) * a.Hkv + kvh) * kHalf;
      const uint32_t kw2 = ksrc[lane], vw2 = vsrc[lane];
      float x0 = lo_bf16(kw2), x1 = hi_bf16(kw2);  // components 2 lane, 2 lane + 1
      if (a.wk) {
        const float inv = rsqrtf(wave_sum(x0 * x0 + x1 * x1) * (1.f / kHeadDim) + a.eps);
        const uint32_t gw = static_cast<const uint32_t*>(a.wk)[lane];
        x0 *= inv * (a.norm_offset + lo_bf16(gw));
        x1 *= inv * (a.norm_offset + hi_bf16(gw));
      }
      if (!kRotate) {  // post-RoPE cache: pair j = 2 (lane & 31) + u of components (j, j + 64)
        const float y0 = __shfl_xor(x0, 32, 64), y1 = __shfl_xor(x1, 32, 64);
        const float2 z0 = rope_factor(a.rope, p, 2 * (lane & 31)), z1 = rope_factor(a.rope, p, 2 * (lane & 31) + 1);
        if (lane < 32) {
          x0 = x0 * z0.x - y0 * z0.y;
          x1 = x1 * z1.x - y1 * z1.y;
        } else {
          x0 = y0 * z0.y + x0 * z0.x;
          x1 = y1 * z1.y + x1 * z1.x;
        }
      }
      reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(const_cast<void*>(a.k_cache)) + row * kHeadDim)[lane] = pack_bf16x2(x0, x1);
      reinterpret_cast<uint32_t*>(static_cast<bf16_t*>(const_cast<void*>(a.v_cache)) + row * kHeadDim)[lane] = vw2;
      __builtin_amdgcn_s_waitcnt(0);  // (gfx9: the stores count in vmcnt)
    }
  }

  // ---- Q' fragment (B operand of S^T): head m16, dims of the lane's 16 pairs --------
  // slice s: dims 32s + 8g + e (e = 0..7); slices s and s + 2 hold the rotation pairs
  // j = 32s + 8g + e and j + 64. Each slice of a key row is 64 contiguous bytes.
  // (loaded here, zeroed for the padding heads once the loads have landed, below; in the
  // one-launch step the projected query and its gains are loaded here and Q' is formed below)
  const bool q_ok = m16 < G;
  u32x4 qw[4];
  u32x4 gq[kFused ? 4 : 1];
  float2 zf = {0.f, 0.f}, zc = {0.f, 0.f};  // (one-launch step, wave 0) fine / coarse factor of pair `lane`
  f16x8 qf[4];
#pragma unroll
  for (int s = 0; s < (kFused ? 4 : 1); ++s) gq[s] = u32x4{0, 0, 0, 0};
  {
    if (kFused) {
      const bf16_t* src = static_cast<const bf16_t*>(a.q_in) +
                          (static_cast<long long>(b) * a.Hq + kvh * G + (q_ok ? m16 : 0)) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 4; ++s) qw[s] = *reinterpret_cast<const u32x4*>(src + s * 32 + g * 8);
      if (a.wq) {
#pragma unroll
        for (int s = 0; s < 4; ++s) gq[s] = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(a.wq) + s * 32 + g * 8);
      }
      if (wave == 0) {  // table rows of the query position (the product is formed below)
        const long long rp = a.post_rope ? a.pos_offset : S - 1;
        zf = a.rope[(rp & (kRopeFine - 1)) * kHalf + lane];
        zc = a.rope[(kRopeFine + (rp >> 6)) * kHalf + lane];
      }
    } else {
      const f16_t* src = static_cast<const f16_t*>(a.q_rot) +
                         (static_cast<long long>(b) * a.Hq + kvh * G + (q_ok ? m16 : 0)) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 4; ++s) qw[s] = *reinterpret_cast<const u32x4*>(src + s * 32 + g * 8);
    }
  }

  // ---- fine rope factors of this lane's key (its position & 63 is fixed) -------------
  const int key_in_tile = wave * kSub + m16;
  float2 fine[16];
#pragma unroll
  for (int e = 0; e < 16; ++e)
    fine[e] = kRotate ? a.rope[key_in_tile * kHalf + (e >> 3) * 32 + g * 8 + (e & 7)] : float2{0.f, 0.f};

  // ---- per-lane pieces of the loads ---------------------------------------------------
  // V direct load i, lane l fills chunk slot l & 15 of row 4 i + l / 16: it loads the
  // row's chunk (l & 15) ^ v_swizzle(row).
  int v_row[kVLoads], v_col[kVLoads];
#pragma unroll
  for (int i = 0; i < kVLoads; ++i) {
    v_row[i] = 4 * i + (lane >> 4);
    v_col[i] = (lane & 15) ^ v_swizzle(v_row[i]);
  }
  // Issue the loads of this wave's keys of the next tile into a K register set, a V slot
  // and a coarse-row slot. Tiles are issued in order 0, 1, 2, ...; past the end the last
  // tile is issued again (the same count of loads stays in flight at every step), and keys
  // past s_end read the last key (their p is zero). The cache slot of renumbered key
  // tb + j is s0 + j with s0 = (base + tb) mod W kept per tile (one wrap at most when
  // W >= 64), or base + tb + j on global layers.
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
  auto issue = [&](u32x4* kw, bf16_t* vslot, float2* cslot) __attribute__((always_inline)) {
    {
      const bf16_t* row = kc + cache_row(key_in_tile) * kHeadDim;
#pragma unroll
      for (int s = 0; s < 4; ++s) kw[s] = *reinterpret_cast<const u32x4*>(row + s * 32 + g * 8);
    }
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      // (the address goes through a named pointer: passing the lambda call straight into
      // the builtin drops this kernel's host-side launch stub)
      const bf16_t* src = vc + cache_row(wave * kSub + v_row[i]) * kHeadDim + v_col[i] * 8;
      __builtin_amdgcn_global_load_lds(src, vslot + i * 512, 16, 0, kNonTemporal);
    }
    if (kRotate) {  // coarse row of the tile (64 pairs, 512 B), copied twice over the 64 lanes
      const float2* crow = a.rope + (kRopeFine + (tb_issue >> 6)) * kHalf + (lane & 31) * 2;
      __builtin_amdgcn_global_load_lds(crow, cslot, 16, 0, 0);
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

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;  // reference max (log2 units) and row sum of head m16
  const float c = a.scale * 1.4426950408889634f;

  auto compute = [&](int t, const u32x4* kw, const bf16_t* vslot, const float2* cslot)
      __attribute__((always_inline)) {
    const long long key0 = s_begin + static_cast<long long>(t) * kTile + wave * kSub;
    if (key0 >= s_end) return;  // wave-uniform: no key of this wave in the tile
    // K': rotate the lane's 16 pairs, pack to half in the A-operand layout (a post-RoPE
    // cache row is already that operand, converted bf16 -> half exactly)
    f16x8 kf[4];
#pragma unroll
    for (int s = 0; s < 4 && !kRotate; ++s) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = bf16x2_to_f16x2(kw[s][i]);
      kf[s] = __builtin_bit_cast(f16x8, w);
    }
#pragma unroll
    for (int hs = 0; hs < 2 && kRotate; ++hs) {  // hs: slices (hs, hs+2) hold pairs 32hs + 8g + e
      u32x4 lo_w, hi_w;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float ra[2], rb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = e2 * 2 + u;
          const float x0 = u ? hi_bf16(kw[hs][e2]) : lo_bf16(kw[hs][e2]);
          const float x1 = u ? hi_bf16(kw[hs + 2][e2]) : lo_bf16(kw[hs + 2][e2]);
          const float2 cr = cslot[hs * 32 + g * 8 + e];
          const float2 f = fine[hs * 8 + e];
          const float zx = cr.x * f.x - cr.y * f.y;
          const float zy = cr.x * f.y + cr.y * f.x;
          ra[u] = x0 * zx - x1 * zy;
          rb[u] = x0 * zy + x1 * zx;
        }
        lo_w[e2] = pack_f16x2(ra[0], ra[1]);
        hi_w[e2] = pack_f16x2(rb[0], rb[1]);
      }
      kf[hs] = __builtin_bit_cast(f16x8, lo_w);
      kf[hs + 2] = __builtin_bit_cast(f16x8, hi_w);
    }
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s], qf[s], sacc, 0, 0, 0);

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
    // Lazy rescaling: the reference only moves when a head gains more than 2^8 over it.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0) {  // wave-uniform
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    u32x2 pw;
    pw[0] = pack_bf16x2(fast_exp2(sacc[0] - m_run), fast_exp2(sacc[1] - m_run));
    pw[1] = pack_bf16x2(fast_exp2(sacc[2] - m_run), fast_exp2(sacc[3] - m_run));
    l_run = add_bf16x2(pw[1], add_bf16x2(pw[0], l_run));  // the same bf16 p as P V
    const s16x4 pb = __builtin_bit_cast(s16x4, pw);

    // V^T fragments: d = 16dt + m16, keys 4g + i of the sub-tile, one transposing LDS read
    // each: lane 4r + q of lane group g addresses key 4g + r, dims 16dt + 4q .. +3 (half
    // q & 1 of chunk 2dt + q / 2, stored at chunk (2dt + q / 2) ^ v_swizzle(4g + r)), and the
    // read hands lane m16 of the group dim 16dt + m16 of the four keys (key 4g + i in i).
    const int vr = 4 * g + (m16 >> 2);
    const bf16_t* vrow = vslot + vr * kHeadDim + (m16 & 3) * 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const s16x4 va = __builtin_bit_cast(s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                     (lds_v4i16_t*)(vrow + 8 * ((2 * dt) ^ v_swizzle(vr)))));
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[dt], 0, 0, 0);
    }
  };

  // ---- three sub-tiles per wave: compute t while t+1, t+2 land ------------------------
  u32x4 k0[4], k1[4], k2[4];
  bf16_t* const v0 = vs0[wave];
  bf16_t* const v1 = vs1[wave];
  bf16_t* const v2 = vs2[wave];
  float2* const c0 = cs0[wave];
  float2* const c1 = cs1[wave];
  float2* const c2 = cs2[wave];
  issue(k0, v0, c0);  // tile 0
  issue(k1, v1, c1);  // tile 1
  // Q' and the fine factors (loaded before the tiles) are in once all but the tiles' loads
  // have landed; settle that here, once: a first use inside the loop would otherwise wait
  // for every load in flight.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * kLoads));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(qw[s]));
#pragma unroll
  for (int e = 0; e < 16 && kRotate; ++e) asm volatile("" : "+v"(fine[e].x), "+v"(fine[e].y));
  if constexpr (kFused) {
    // §3.2 / §4.3: q (c + w) / sqrt(mean(q^2) + eps) over the head's 128 components (the
    // lane holds 32, the other lane groups of head m16 the rest); §6.1: pair j = 32s + 8g + e
    // (slices s and s + 2) turns by the factor of the query position; rounded once to half.
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(gq[s]));
    asm volatile("" : "+v"(zf.x), "+v"(zf.y), "+v"(zc.x), "+v"(zc.y));
    if (wave == 0)  // rotation factor of the query position for pair `lane` (rope_factor's product)
      zq[lane] = make_float2(zc.x * zf.x - zc.y * zf.y, zc.x * zf.y + zc.y * zf.x);
    __syncthreads();  // zq written
    float x[4][8];
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[s][2 * i] = lo_bf16(qw[s][i]);
        x[s][2 * i + 1] = hi_bf16(qw[s][i]);
        ss += x[s][2 * i] * x[s][2 * i] + x[s][2 * i + 1] * x[s][2 * i + 1];
      }
    if (a.wq) {
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      const float inv = rsqrtf(ss * (1.f / kHeadDim) + a.eps);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[s][2 * i] *= inv * (a.norm_offset + lo_bf16(gq[s][i]));
          x[s][2 * i + 1] *= inv * (a.norm_offset + hi_bf16(gq[s][i]));
        }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 z = zq[32 * s + 8 * g + e];
        const float x0 = x[s][e], x1 = x[s + 2][e];
        x[s][e] = x0 * z.x - x1 * z.y;
        x[s + 2][e] = x0 * z.y + x1 * z.x;
      }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) qw[s][i] = pack_f16x2(x[s][2 * i], x[s][2 * i + 1]);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = __builtin_bit_cast(f16x8, q_ok ? qw[s] : u32x4{0, 0, 0, 0});
  // Before computing tile t, an explicit wait leaves the loads of the tiles issued after it
  // in flight (the compiler's own waits cannot follow the ring across loop iterations).
  constexpr unsigned kTwoBehind = wait_vmcnt(2 * kLoads);
  constexpr unsigned kOneBehind = wait_vmcnt(kLoads);
  int t = 0;
  for (; t + 3 <= n_tiles; t += 3) {
    issue(k2, v2, c2);  // tile t + 2
    __builtin_amdgcn_s_waitcnt(kTwoBehind);
    compute(t, k0, v0, c0);
    issue(k0, v0, c0);  // tile t + 3
    __builtin_amdgcn_s_waitcnt(kTwoBehind);
    compute(t + 1, k1, v1, c1);
    issue(k1, v1, c1);  // tile t + 4
    __builtin_amdgcn_s_waitcnt(kTwoBehind);
    compute(t + 2, k2, v2, c2);
  }
  if (t < n_tiles) {
    __builtin_amdgcn_s_waitcnt(kOneBehind);
    compute(t, k0, v0, c0);
  }
  if (t + 1 < n_tiles) {
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    compute(t + 1, k1, v1, c1);
  }
  // the repeated tiles past the end may still be landing in LDS
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  // ---- merge the 4 waves' states in LDS (reusing the V slots) -------------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // [16 heads][128] accumulators of waves 0, 1 in vs0 and of waves 2, 3 in vs1; m, l in cs0, cs1
  static_assert(sizeof(vs0) >= 2 * kMaxGroup * kHeadDim * sizeof(float), "merge buffer");
  auto red_of = [&](int w) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(w < 2 ? &vs0[0][0] : &vs1[0][0]) + (w & 1) * kMaxGroup * kHeadDim;
  };
  float* red_m = reinterpret_cast<float*>(&cs0[0][0]);
  float* red_l = reinterpret_cast<float*>(&cs1[0][0]);
  {
    float* mine = red_of(wave);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[m16 * kHeadDim + dt * 16 + 4 * g + i] = oacc[dt][i];
  }
  if (g == 0) {
    red_m[wave * kMaxGroup + m16] = m_run;
    red_l[wave * kMaxGroup + m16] = l_run;
  }
  __syncthreads();
  const bool single = a.plan.n_split == 1;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
    const int h = idx / kHeadDim, d = idx % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w * kMaxGroup + h]);
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(red_m[w * kMaxGroup + h] - M);  // 0 for a wave with no key
      acc += sc * red_of(w)[h * kHeadDim + d];
      l += sc * red_l[w * kMaxGroup + h];
    }
    const long long bh = static_cast<long long>(b) * a.Hq + kvh * G + h;
    if (single) {
      static_cast<bf16_t*>(a.out)[bh * kHeadDim + d] = f32_to_bf16(acc / l);
    } else {
      float* dst = a.ws + (bh * a.plan.n_split + split) * kPartial;
      if (kFused) {  // written through to the device-coherent level (read by another block)
        __hip_atomic_store(dst + d, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          __hip_atomic_store(dst + kHeadDim, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(dst + kHeadDim + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        dst[d] = acc;
        if (d == 0) {
          dst[kHeadDim] = M;
          dst[kHeadDim + 1] = l;
        }
      }
    }
  }
  if constexpr (kFused) {
    // One-launch step: the last block of this (sequence, KV head) to get here merges the
    // ranges' states in range order (deterministic) and writes the output. The ticket
    // wraps back to 0 on the last arrival (atomicInc with limit n_split - 1).
    // The states go out as device-coherent (write-through) stores and are read back as
    // device-coherent loads, so no cache-wide writeback or invalidation is needed: each thread
    // waits until its stores are acknowledged, the barrier then covers the whole block, and
    // only after that does the block take its ticket; the block that takes the last ticket
    // issues its loads after the ticket has returned.
    if (single) return;  // block-uniform
    __shared__ int is_last;
    __builtin_amdgcn_s_waitcnt(0);  // (gfx9: stores count in vmcnt)
    __syncthreads();
    if (threadIdx.x == 0)
      is_last = atomicInc(a.tickets + (static_cast<long long>(b) * a.Hkv + kvh),
                          static_cast<unsigned>(a.plan.n_split - 1)) == static_cast<unsigned>(a.plan.n_split - 1);
    __syncthreads();
    if (!is_last) return;  // block-uniform
    const int n_split = a.plan.n_split;
    // this (sequence, KV head)'s states: [G heads][n_split][acc[128], m, l], read with
    // device-coherent (sc1) buffer loads, all of them independent of each other
    const float* base_p = a.ws + (static_cast<long long>(b) * a.Hq + kvh * G) * n_split * kPartial;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(base_p), 0, G * n_split * kPartial * static_cast<int>(sizeof(float)), 0x00020000);
    constexpr int kCoherent = 16;  // sc1
    auto ld = [&](int off) { return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off * 4, 0, kCoherent)); };
    // m and l of every (head, range) into LDS (the V slots are free now)
    float* sm = reinterpret_cast<float*>(&vs0[0][0]);
    float* sl = reinterpret_cast<float*>(&vs1[0][0]);
    static_assert(sizeof(vs0) >= kMaxGroup * kMaxSplit * sizeof(float), "merge buffer");
    for (int t = threadIdx.x; t < G * n_split; t += kThreads) {
      sm[t] = ld(t * kPartial + kHeadDim);
      sl[t] = ld(t * kPartial + kHeadDim + 1);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
      const int h = idx / kHeadDim, d = idx % kHeadDim;
      const long long bh = static_cast<long long>(b) * a.Hq + kvh * G + h;
      float M = -INFINITY;
      for (int i = 0; i < n_split; ++i) M = fmaxf(M, sm[h * n_split + i]);
      float acc = 0.f, l = 0.f;
#pragma unroll 8
      for (int i = 0; i < n_split; ++i) {
        const float w = fast_exp2(sm[h * n_split + i] - M);
        acc += w * ld((h * n_split + i) * kPartial + d);
        l += w * sl[h * n_split + i];
      }
      static_cast<bf16_t*>(a.out)[bh * kHeadDim + d] = f32_to_bf16(acc / l);
    }
  }
}

// One block per (sequence, query head): the split states are merged in a fixed order
// (deterministic); thread d owns output component d. All loads (every split's m, l and
// this thread's accumulators, up to kRegSplits of them in registers) go out together.
// A sequence of a ragged batch merges only the ranges its keys reach.
constexpr int kRegSplits = 32;
__global__ __launch_bounds__(kHeadDim) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float ms[kMaxSplit], ls[kMaxSplit];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  int n_split = a.plan.n_split;
  if (a.seq_pos) {
    const SeqPos sp = seq_pos_of(a.seq_pos, nullptr, a.pos_offset, 1, a.window, bh / a.Hq);
    n_split = static_cast<int>((sp.kept + 1 + a.plan.chunk - 1) / a.plan.chunk);
  }
  const float* p = a.ws + static_cast<long long>(bh) * a.plan.n_split * kPartial;
  bf16_t* __restrict__ out = static_cast<bf16_t*>(a.out);
  float av[kRegSplits];
#pragma unroll
  for (int i = 0; i < kRegSplits; ++i) av[i] = i < n_split ? p[i * kPartial + tid] : 0.f;
  for (int i = tid; i < n_split; i += kHeadDim) {
    ms[i] = p[i * kPartial + kHeadDim];
    ls[i] = p[i * kPartial + kHeadDim + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < n_split; ++i) M = fmaxf(M, ms[i]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int i = 0; i < kRegSplits; ++i) {
    if (i < n_split) {
      const float w = fast_exp2(ms[i] - M);
      L += w * ls[i];
      acc += w * av[i];
    }
  }
  for (int i = kRegSplits; i < n_split; ++i) {
    const float w = fast_exp2(ms[i] - M);
    L += w * ls[i];
    acc += w * p[i * kPartial + tid];
  }
  out[static_cast<long long>(bh) * kHeadDim + tid] = f32_to_bf16(acc / L);
}

}  // namespace

namespace {
template <bool kFused>
void launch_split(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  if (!a.post_rope) {
    if (a.window == 0)
      hipLaunchKernelGGL((decode_split_kernel<kContiguous, true, kFused>), grid, dim3(kThreads), 0, stream, a);
    else if (a.window >= kTile)
      hipLaunchKernelGGL((decode_split_kernel<kRing, true, kFused>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<kSmallRing, true, kFused>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (a.window == 0)
      hipLaunchKernelGGL((decode_split_kernel<kContiguous, false, kFused>), grid, dim3(kThreads), 0, stream, a);
    else if (a.window >= kTile)
      hipLaunchKernelGGL((decode_split_kernel<kRing, false, kFused>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<kSmallRing, false, kFused>), grid, dim3(kThreads), 0, stream, a);
  }
}
}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  // Blocks are dispatched in index order. A ragged batch puts the key range slowest: the
  // first ranges of every (sequence, KV head) start together, later ranges (only the longer
  // sequences have them) fill the slots as they free up, and the empty ranges of short
  // sequences come last. The one-launch step does the same, so that with B Hkv a multiple of
  // 8 the ranges of one (sequence, KV head) go to one XCD (blocks are dealt to the 8 XCDs
  // round robin) and its merge reads states from that XCD's L2.
  if (a.fused) {
    launch_split<true>(a, dim3(a.Hkv, a.B, a.plan.n_split), stream);
    return hipGetLastError();
  }
  const dim3 grid = a.seq_pos ? dim3(a.Hkv, a.B, a.plan.n_split) : dim3(a.plan.n_split, a.Hkv, a.B);
  launch_split<false>(a, grid, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.plan.n_split == 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(kHeadDim), 0, stream, a);
  return hipGetLastError();
}

}  // namespace plamo
