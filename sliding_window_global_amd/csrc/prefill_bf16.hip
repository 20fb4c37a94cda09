// Flash-style causal / sliding-window GQA prefill on gfx950 bf16 MFMA.
//
// 「PLaMo 3アーキテクチャ徹底解析」 §4.5: A = softmax(Q'K'^T / sqrt(128) + M), O = A V per
// query head, KV head h / (Hq/Hkv) (§4.2); §5.1: the mask keeps j <= i and, on local
// layers, i - j < W. The score matrix is never stored (§4.5 notes a kernel need not hold
// it) and key tiles wholly outside every row's window are skipped, so a local layer
// costs O(T W) (§5.3).
//
// Work decomposition
//   block  = 128 query rows of one (sequence, query head); 4 waves x 32 rows. Query row t
//            sits at renumbered position kept + t: a chunk after `kept` cached keys
//            (§4.4) attends keys 0 .. kept+t, all of them in the K' / V^T operands.
//   tile   = 64 keys. K' and V^T arrive tiled in HBM in exactly the LDS order, so each
//            tile is one contiguous copy straight into LDS (buffer_load_dwordx4 ... lds, no
//            register staging), double buffered. The LDS order is chunk-major: the
//            operand reads of one MFMA are 64 consecutive 16-byte slots (no bank
//            conflicts) and the reads of different chunks differ by constant offsets.
//   order  = key tiles from the diagonal downwards. A row with no visible key in the
//            first tiles keeps a -inf reference until its first visible key.
//   math   = S^T = K' Q'^T on v_mfma_f32_32x32x16_f16 (Q' and K' are IEEE halves) and
//            O^T = V^T P^T on v_mfma_f32_32x32x16_bf16 (V and P bf16): the query
//            index is the MFMA column in both, so each lane owns one query row for the
//            online softmax and for the rescaling of its O^T accumulators. K' rows are
//            read in the order that makes each lane's eight consecutive S^T entries
//            eight consecutive keys, which is what the P^T operand of the next MFMA
//            needs; V^T is then read in natural key order.
//   pipeline = one basic block per step: the QK MFMAs of tile t+1 interleaved with the
//            exp2 / pack / row-sum work of tile t, then the P V MFMAs of tile t
//            interleaved with the row maxima of tile t+1.
//   softmax = exp2 domain; Q' is pre-scaled by scale * log2(e) and the S accumulator
//            starts at -m, so the numerator is a bare exp2; lazy rescaling (the
//            reference moves only when a row gains more than 2^8); row sums taken from
//            the same bf16-rounded P as P V.
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3: 32-bit data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// the score product: Q' and K' are IEEE halves (same MFMA rate as bf16, three more bits)
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Key (within a 32-key block) whose K' row feeds MFMA row m: swaps bits 2 and 3, so that
// the S^T entries (m = i*8 + half*4 + j) of one lane hold keys i/2*16 + half*8 + i%2*4 + j.
__device__ __forceinline__ int key_of_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS element offset of 16-byte chunk c of K' row r (16 chunks per row): chunk-major, so
// the operand reads of one MFMA cover consecutive 16-byte slots and the reads of the
// different chunks differ by compile-time offsets.
__device__ __forceinline__ int k_chunk(int r, int c) { return (c * BN + r) * 8; }
// LDS element offset of 16-byte chunk c of V^T row d (8 chunks per row), chunk-major.
__device__ __forceinline__ int v_chunk(int d, int c) { return (c * kHeadDim + d) * 8; }

// kLocal: sliding-window layer (window > 0); otherwise the global causal layer.
// kFuseQ: q_rot holds the projected queries; the block normalises and rotates its rows
// itself (steps 1 and 3 of §4.4 for Q), so that the append need not write Q' to HBM.
template <bool kLocal, bool kFuseQ>
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
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
  // Query row t sits at renumbered position kept + t; keys 0 .. kept-1 came from the cache.
  // (a.T is the row stride; the sequence's own token count n_rows may be smaller.)
  const SeqPos sp = seq_pos_of(a.seq_pos, a.seq_len, a.pos_offset, a.T, a.window, b);
  const int kept = static_cast<int>(sp.kept);
  const int n_rows = sp.T;
  if (i0 >= n_rows) return;  // block-uniform, before any barrier
  const int last_row = min(i0 + BM, n_rows) - 1;
  const int lo = kLocal ? max(0, kept + i0 - a.window + 1) : 0;
  const int kt_hi = (kept + last_row) / BN;
  const int n_tiles = kt_hi - lo / BN + 1;

  // K' and V^T arrive tiled by 64 keys, each tile 16 KiB in exactly the LDS order below, so
  // a tile is one contiguous copy: direct load g = wave*4 + i moves bytes 1024g .. +1023
  // (lane l: 16 bytes at 1024g + 16l). The copies are buffer loads with the LDS bit over a
  // resource spanning this (sequence, KV head)'s operand (out-of-range reads return 0):
  // the tile offset goes in the scalar offset, the lane's in the vector one. (The global-
  // segment form of the same copy makes the compiler wait for every outstanding LDS read
  // before each MFMA operand use while a copy is in flight; with the buffer form its waits
  // leave the three younger operand reads in flight.)
  const uint32_t lane_off = static_cast<uint32_t>(lane) * 16 + static_cast<uint32_t>(wave) * 4096;
  const int op_bytes = static_cast<int>(a.Tp * kHeadDim * sizeof(bf16_t));
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(kbase, op_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(vbase, op_bytes);
  auto issue = [&](__amdgpu_buffer_rsrc_t rsrc, int step, bf16_t* buf) __attribute__((always_inline)) {
    const int tile_off = (kt_hi - step) * kTileElems * static_cast<int>(sizeof(bf16_t));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds_ptr_t dst = (lds_ptr_t)(buf + (wave * 4 + i) * 512);  // generic -> LDS address space
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, lane_off + i * 1024, tile_off, 0, 0);
    }
  };
  auto issue_k = [&](int step, bf16_t* buf) __attribute__((always_inline)) { issue(k_rsrc, step, buf); };
  auto issue_v = [&](int step, bf16_t* buf) __attribute__((always_inline)) { issue(v_rsrc, step, buf); };

  // ---- Q' fragment (MFMA B operand): lane holds dims s*16 + hl*8 .. +7 of its row ----
  // Pre-multiplied by scale * log2(e), so that S comes out of the MFMA in exp2 units, and
  // rounded to IEEE half (Q' arrives as halves from the append, or is formed here in fp32).
  const float c = a.scale * 1.4426950408889634f;
  const int r0 = i0 + wave * 32;
  const int qrow = r0 + n;
  const int p0 = kept + r0;  // position of the wave's first row
  f16x8 qf[8];
  {
    const bool ok = qrow < n_rows;
    const bf16_t* src = q + (static_cast<long long>(b) * a.T + (ok ? qrow : 0)) * a.Hq * kHeadDim +
                        static_cast<long long>(hq) * kHeadDim + hl * 8;
    // The rows' Q (or Q') go out first, since they gate the first MFMA; K'(0), K'(1) and
    // V^T(0) are copied while they arrive (and, fused, while Q' is formed).
    // (src is row 0 for rows past n_rows: the loads are unconditional and the values are
    // zeroed afterwards; a load under a branch made the compiler wait for every load in
    // flight, the tile copies included, in the middle of these)
    u32x4 qraw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qraw[s] = *reinterpret_cast<const u32x4*>(src + s * 16);
    __builtin_amdgcn_sched_barrier(0);
    issue_k(0, ks0);
    if (n_tiles > 1) issue_k(1, ks1);
    issue_v(0, vs0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) qraw[s][i] = ok ? qraw[s][i] : 0u;
    if (!kFuseQ) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 w = qraw[s];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = pack_f16x2(lo_f16(w[i]) * c, hi_f16(w[i]) * c);
        qf[s] = __builtin_bit_cast(f16x8, w);
      }
    } else {
      // §3.2 / §4.3: x (c' + w) / sqrt(mean(x^2) + eps) over the row's 128 dims (the other 64
      // sit in lane n ^ 32); §6.1: pair j (dims j, j + 64) turns by the angle of position
      // kept + qrow (post-RoPE cache: pos + qrow), factor amp exp(i p w_j) from the table. The
      // lane's pairs are j = s*16 + hl*8 + e, s < 4, partners in slice s + 4: all lane-local.
      float x[8][8];
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 w = qraw[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[s][2 * i] = lo_bf16(w[i]);
          x[s][2 * i + 1] = hi_bf16(w[i]);
          ss += x[s][2 * i] * x[s][2 * i] + x[s][2 * i + 1] * x[s][2 * i + 1];
        }
      }
      if (a.wq) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        const float inv = rsqrtf((__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * (1.f / kHeadDim) + a.eps);
        const bf16_t* wq = static_cast<const bf16_t*>(a.wq) + hl * 8;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const u32x4 gw = *reinterpret_cast<const u32x4*>(wq + s * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[s][2 * i] *= inv * (a.norm_offset + lo_bf16(gw[i]));
            x[s][2 * i + 1] *= inv * (a.norm_offset + hi_bf16(gw[i]));
          }
        }
      }
      const long long pos = (a.post_rope ? sp.pos : sp.kept) + (ok ? qrow : 0);
      const float2* fine = a.rope + (pos & (kRopeFine - 1)) * kHalf + hl * 8;
      const float2* coarse = a.rope + (kRopeFine + (pos >> 6)) * kHalf + hl * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 f = fine[s * 16 + e], cz = coarse[s * 16 + e];
          const float zx = cz.x * f.x - cz.y * f.y, zy = cz.x * f.y + cz.y * f.x;
          const float x0 = x[s][e], x1 = x[s + 4][e];
          x[s][e] = x0 * zx - x1 * zy;
          x[s + 4][e] = x0 * zy + x1 * zx;
        }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_f16x2(x[s][2 * i] * c, x[s][2 * i + 1] * c);
        qf[s] = __builtin_bit_cast(f16x8, w);
      }
    }
  }

  // wave-uniform: does tile `step` hold a masked pair for some row of the wave? (A tile that
  // lies wholly outside the wave's rows' windows is computed fully masked: the four waves
  // of a block move through the tiles in step, so skipping it would not end the step
  // sooner.)
  auto needs_mask = [&](int step) __attribute__((always_inline)) {
    const int j0 = (kt_hi - step) * BN;
    return (j0 + BN - 1 > p0) || (kLocal && p0 + 31 - j0 >= a.window);
  };

  // MFMA operand i of one step: i < 16 is K' chunk (s = i/2, key block i%2) of the next
  // tile's S^T = K' Q'^T; i >= 16 is V^T chunk (k-step (i-16)/4, d block (i-16)%4) of
  // this tile's O^T += V^T P^T.
  auto frag = [&](int i, const bf16_t* kbuf, const bf16_t* vbuf) __attribute__((always_inline)) {
    if (i < 16)
      return *reinterpret_cast<const u32x4*>(kbuf + k_chunk((i & 1) * 32 + key_of_row(n), i + hl - (i & 1)));
    const int j = i - 16;
    return *reinterpret_cast<const u32x4*>(vbuf + v_chunk((j & 3) * 32 + n, 2 * (j >> 2) + hl));
  };

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  // Running reference max of the lane's row in exp2 units (-inf until its first tile);
  // S^T of a tile is produced already shifted by it (the MFMA accumulator starts at
  // -m_run), so the softmax numerator is a bare exp2.
  float m_run = -INFINITY;
  float l_run = 0.f;
  // -reference in all 16 accumulator slots: the start value of every S^T accumulator
  // (rewritten only when the reference moves)
  f32x16 neg_m;
#pragma unroll
  for (int e = 0; e < 16; ++e) neg_m[e] = 0.f;
  constexpr int kDepth = 4;  // MFMA operands read ahead from LDS

  using T1 = std::integral_constant<bool, true>;
  using T0 = std::integral_constant<bool, false>;
  // One pipeline step: S^T(step+1) = K'(step+1) Q'^T (if kQK) on the matrix cores while
  // the vector ALUs turn S^T(step) into P^T (if kPV); then O^T += V^T(step) P^T (if kPV)
  // while the row maxima of S^T(step+1) are taken. `s_cur` holds S^T(step) shifted and
  // masked; `s_next` receives S^T(step+1).
  auto step_body = [&](auto QK, auto PV, int step, const bf16_t* kbuf, const bf16_t* vbuf,
                       f32x16* s_cur, f32x16* s_next) __attribute__((always_inline)) {
    constexpr bool kQK = decltype(QK)::value, kPV = decltype(PV)::value;
    constexpr int i_first = kQK ? 0 : 16, i_last = kPV ? 32 : 16;
    const float m_base = m_run == -INFINITY ? 0.f : m_run;

    u32x4 fr[kDepth];
#pragma unroll
    for (int i = i_first; i < i_first + kDepth; ++i) fr[i % kDepth] = frag(i, kbuf, vbuf);

    // part A: 16 QK MFMAs; P^T words: pair j = keys 2j, 2j+1 of the lane's 32 (flat index
    // f = kb*16 + e), word j of the B operand for k-step j/4
    u32x4 pw[4];
    float* sc = reinterpret_cast<float*>(s_cur);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (kQK) {
        const int kb = i & 1, s = i >> 1;
        s_next[kb] = mfma32_f16(__builtin_bit_cast(f16x8, fr[i % kDepth]), qf[s], s == 0 ? neg_m : s_next[kb]);
        if (i + kDepth < i_last) fr[i % kDepth] = frag(i + kDepth, kbuf, vbuf);
      }
      if (kPV) {
        sc[2 * i] = fast_exp2(sc[2 * i]);
        sc[2 * i + 1] = fast_exp2(sc[2 * i + 1]);
        if (i >= 1) pw[(i - 1) >> 2][(i - 1) & 3] = pack_bf16x2(sc[2 * i - 2], sc[2 * i - 1]);
        // row sum: one dot product per P word, chained straight into l (one link per
        // MFMA slot, so the chain's latency stays hidden; no partial sums to clear or add)
        if (i >= 2) l_run = add_bf16x2(pw[(i - 2) >> 2][(i - 2) & 3], l_run);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kPV) {
      pw[3][3] = pack_bf16x2(sc[30], sc[31]);
      l_run = add_bf16x2(pw[3][3], add_bf16x2(pw[3][2], l_run));
      // keep the P^T words computed here, under the QK MFMAs, rather than sunk past the
      // mask branch below
#pragma unroll
      for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(pw[u]));
      asm volatile("" : "+v"(l_run));
    }

    // (kQK: a next tile exists; the last step is run without the QK half)
    if (kQK && needs_mask(step + 1)) {
      // key k of the tile is visible to the row at position kept + qrow iff
      // 0 <= kept + qrow - j0 - k (< window on local layers): one unsigned compare
      const int dq = kept + qrow - (kt_hi - step - 1) * BN - hl * 8;
      const unsigned lim = kLocal ? static_cast<unsigned>(a.window) : 0x80000000u;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ko = kb * 32 + (e >> 3) * 16 + (e & 7);
          if (!(static_cast<unsigned>(dq - ko) < lim)) s_next[kb][e] = -INFINITY;
        }
    }

    // part B: 16 PV MFMAs; row max of S^T(step+1) over the second half
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int i = 16; i < 32; ++i) {
      if (kPV) {
        const int j = i - 16;
        oacc[j & 3] = mfma32(__builtin_bit_cast(bf16x8, fr[i % kDepth]),
                             __builtin_bit_cast(bf16x8, pw[j >> 2]), oacc[j & 3]);
        if (i + kDepth < 32) fr[i % kDepth] = frag(i + kDepth, kbuf, vbuf);
      }
      if (kQK && (!kPV || i >= 24)) {
        const int f = kPV ? (i - 24) * 4 : (i - 16) * 2;
        const int cnt = kPV ? 4 : 2;
#pragma unroll
        for (int u = 0; u < cnt; u += 2) {
          const float x = s_next[(f + u) >> 4][(f + u) & 15], y = s_next[(f + u + 1) >> 4][(f + u + 1) & 15];
          // max(max(m, x), y): one v_max3 per two scores
          if (((f + u) >> 1) & 1) mx1 = fmaxf(fmaxf(mx1, x), y);
          else mx0 = fmaxf(fmaxf(mx0, x), y);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if (kQK) {
      float mx = fmaxf(mx0, mx1);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      // Lazy rescaling: the reference max only moves (and O, l are only rescaled) when some
      // row of the wave gains more than 2^8 over it, or on a row's first tile.
      const bool first = m_run == -INFINITY;
      if (__builtin_amdgcn_ballot_w64(mx > kRescaleLog2 || first) != 0) {  // wave-uniform
        // first tile: the reference becomes the row max (a row with no visible key yet
        // keeps -inf); later: it moves up by the gain, if any
        const float bump = first ? (mx == -INFINITY ? 0.f : mx) : fmaxf(mx, 0.f);
        const float alpha = first ? 0.f : fast_exp2(-bump);
        // (while no row of the wave has seen a key, O and l are still zero: nothing to scale)
        if (__builtin_amdgcn_ballot_w64(!first) != 0) {  // wave-uniform
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) s_next[kb][e] -= bump;
        m_run = (first && mx == -INFINITY) ? -INFINITY : m_base + bump;
        const float nb = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
        for (int e = 0; e < 16; ++e) neg_m[e] = nb;
      }
    }
  };
  // `k_fill`, `v_fill` receive K'(step+2) and V^T(step+1); `kbuf` holds K'(step+1) and
  // `vbuf` V^T(step). The buffers refilled here were last read before the previous barrier.
  // QK: whether a next tile exists (the last step only multiplies P V).
  auto run_step = [&](auto QK, int step, const bf16_t* kbuf, const bf16_t* vbuf, bf16_t* k_fill, bf16_t* v_fill,
                      f32x16* s_cur, f32x16* s_next) __attribute__((always_inline)) {
    if (step + 2 < n_tiles) issue_k(step + 2, k_fill);
    if (step + 1 < n_tiles) issue_v(step + 1, v_fill);
    step_body(QK, T1{}, step, kbuf, vbuf, s_cur, s_next);
    if (decltype(QK)::value) {  // (after the last step nothing is read from LDS again)
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }
  };

  // ---- K'(0), K'(1), V^T(0) in LDS; S^T(0); then steps 0 .. n_tiles-1 ----
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  f32x16 s_a[2], s_b[2];  // S^T of the current and of the next tile, roles alternating
  step_body(T1{}, T0{}, -1, ks0, vs1, s_b, s_a);
  __syncthreads();  // every wave is done with K'(0) before step 0 refills its buffer
  int step = 0;
  for (; step + 2 < n_tiles; step += 2) {
    run_step(T1{}, step, ks1, vs0, ks0, vs1, s_a, s_b);
    run_step(T1{}, step + 1, ks0, vs1, ks1, vs0, s_b, s_a);
  }
  if (step + 1 < n_tiles) {
    run_step(T1{}, step, ks1, vs0, ks0, vs1, s_a, s_b);
    run_step(T0{}, step + 1, ks0, vs1, ks1, vs0, s_b, s_a);
  } else {
    run_step(T0{}, step, ks1, vs0, ks0, vs1, s_a, s_b);
  }

  // ---- normalise, then store whole rows through LDS ----------------------------------
  // The lane holds d = dt*32 + i*8 + hl*4 + 0..3 of its row: stored as they are, every store
  // would write 16 B into each of 32 rows. Instead each wave stages its 32 rows (8 KiB, in
  // a K' buffer: the last step reads none) with the 16-byte chunk c of row n at chunk
  // c ^ (n mod 16), which keeps both the staging writes and the row reads free of bank
  // conflicts, and then writes four whole 256-byte rows per store.
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  const float inv = 1.f / l_tot;  // (rows past n_rows: never stored)
  bf16_t* const stage = (wave < 2 ? ks0 : ks1) + (wave & 1) * 32 * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = dt * 4 + i;
      u32x2 w;
      w[0] = pack_bf16x2(oacc[dt][i * 4 + 0] * inv, oacc[dt][i * 4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[dt][i * 4 + 2] * inv, oacc[dt][i * 4 + 3] * inv);
      *reinterpret_cast<u32x2*>(stage + n * kHeadDim + (chunk ^ (n & 15)) * 8 + hl * 4) = w;
    }
  // the wave's own staging writes are done before its reads (no other wave touches them)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  bf16_t* const out_base = static_cast<bf16_t*>(a.out) + static_cast<long long>(hq) * kHeadDim;
  const int c16 = lane & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = j * 4 + (lane >> 4);  // row of the wave, chunk c16 of it
    const u32x4 w = *reinterpret_cast<const u32x4*>(stage + r * kHeadDim + (c16 ^ (r & 15)) * 8);
    if (r0 + r < n_rows)  // (not read again by this kernel: streamed past the caches)
      __builtin_nontemporal_store(
          w, reinterpret_cast<u32x4*>(out_base + (static_cast<long long>(b) * a.T + r0 + r) * a.Hq * kHeadDim +
                                      c16 * 8));
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  const long long nqb = (a.T + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(nqb * a.Hq * a.B));
  if (a.window > 0) {
    if (a.fuse_q)
      hipLaunchKernelGGL((prefill_bf16_kernel<true, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<true, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (a.fuse_q)
      hipLaunchKernelGGL((prefill_bf16_kernel<false, true>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<false, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace plamo
