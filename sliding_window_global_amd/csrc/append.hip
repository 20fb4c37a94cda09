// Fused per-head Q/K RMSNorm + RoPE + KV-cache append, and the prefill operand copies.
//
// 「PLaMo 3アーキテクチャ徹底解析」:
//   §3.2/§4.3  per (token, head): y = (c + w) * x / sqrt(mean(x^2) + eps) over the 128
//              components, one [128] gain shared by all Q heads (k_norm by all KV heads);
//              V is not normalised.
//   §4.4       the cache receives normalised K before RoPE and raw V; RoPE then turns the
//              current Q and the K the cache returns, at renumbered positions.
//   §6.1/§6.3  split-half pairs (j, j + 64); rotation factors from the two-level table.
//
// Head dims 256 and 512 (the Gemma-4-shaped layers of the same page's §8 table) run the
// same code: gain-only norms are offset 0, p-RoPE (§6.4) is a table whose idle pairs
// hold (1, 0), and the optional V norm divides each V head vector by its RMS before it
// is cached or used.
//
// One block = 64 tokens of one sequence and one KV head: its G = Hq/Hkv query heads,
// the K head and the V head. The block forms the rotation factors of its positions in
// LDS, 32 KiB at a time: all 64 positions at d = 128, 32 or 16 of them at d = 256 or 512.
// A row (one token of one head) is handled by a group of
// lanes, each holding one 16-byte chunk of the first half and the matching chunk of the
// second half, so every rotation pair is lane-local and the norm is a reduction over the
// group. bf16 V is read once, into registers: a lane holds one dim chunk of 8 keys, which
// it writes to the cache as it is and to the transposed prefill operand after an 8 x 8
// transpose in registers; fp32 V is staged through LDS for the transpose.
//
// bf16 prefill operands are tiled by 64 keys, each tile 64 d elements in the order the
// prefill kernels copy straight into LDS: K' tile = [d/8 dim chunks][64 keys][8 dims], V^T
// tile = [8 key chunks][d dims][8 keys]. fp32 operands are plain [Tp][d] and [d][Tp].
// On a bf16 layer the score operands Q' and K' are written as IEEE halves, each rounded once
// from the fp32 normalised and rotated value (a new key is rotated before the cache rounds
// it); the cache and V^T stay bf16.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int kTokBlock = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// One LDS area per block, used first for the rotation factors of kRopeTok positions at a
// time ([kRopeTok][d/2] float2, 32 KiB: all 64 positions at d = 128, 32 or 16 of them at
// d = 256 or 512) and afterwards, behind a barrier, for the fp32 V^T staging tile ([d dims]
// [64 + 4 tokens]). bf16 blocks need no staging tile, so every head dim takes 32 KiB and
// five blocks fit on a CU.
template <typename E>
constexpr int kTileStride = kTokBlock + 16 / static_cast<int>(sizeof(E));  // tokens, 16-byte rows
template <int D>
constexpr int kRopeTok = kTokBlock * kHeadDim / D;
template <int D>
constexpr bool kStageRope = D == kHeadDim;  // the operand kernel stages its factors at d = 128 only
template <typename E, int D>
constexpr int kSmemBytes = sizeof(E) == 2 || kRopeTok<D> * (D / 2) * 8 > D * kTileStride<E> * static_cast<int>(sizeof(E))
                               ? kRopeTok<D> * (D / 2) * 8
                               : D * kTileStride<E> * static_cast<int>(sizeof(E));

template <typename E>
struct Io;

template <>
struct Io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void unpack(const u32x4& w, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
  }
  static __device__ __forceinline__ u32x4 pack(const float* x) {
    return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  }
  // score operands (Q', K') keep the storage type
  static __device__ __forceinline__ u32x4 pack_op(const float* x) { return pack(x); }
};

template <>
struct Io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void unpack(const u32x4& w, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = lo_bf16(w[e]);
      x[2 * e + 1] = hi_bf16(w[e]);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float* x) {
    return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
  }
  // score operands (Q', K') of a bf16 layer are IEEE halves: one rounding of the fp32
  // normalised and rotated value, with three more mantissa bits than bf16
  static __device__ __forceinline__ u32x4 pack_op(const float* x) {
    return u32x4{pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(x[4], x[5]),
                 pack_f16x2(x[6], x[7])};
  }
};

// A 16-byte chunk of one V row times s (the inverse RMS of the row, V norm), rounded back
// to the storage type.
template <typename E>
__device__ __forceinline__ u32x4 scaled_chunk(u32x4 w, float s) {
  float x[16 / sizeof(E)];
  Io<E>::unpack(w, x);
#pragma unroll
  for (int e = 0; e < static_cast<int>(16 / sizeof(E)); ++e) x[e] *= s;
  return Io<E>::pack(x);
}

// V norm: v_inv[r] = 1 / sqrt(mean(V_r^2) + eps) for rows r < n <= 64 of `src` (row r at
// src + r * stride): wave w takes rows w, w + 4, ..., each lane reading its D/64 consecutive
// elements of a row at once; all of a wave's loads are issued before the first reduction.
template <typename E, int D>
__device__ __forceinline__ void v_row_inv_rms(const E* __restrict__ src, long long stride, int n, float eps,
                                              float* v_inv, int wave, int lane) {
  constexpr int kPer = D / 64;
  constexpr int kRows = kTokBlock / kWaves;
  E x[kRows][kPer];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int r = wave + k * kWaves;
    if (r < n) __builtin_memcpy(x[k], src + r * stride + lane * kPer, sizeof(x[k]));
  }
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int r = wave + k * kWaves;
    if (r >= n) break;  // wave-uniform
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const float f = Io<E>::ld(&x[k][e]);
      s += f * f;
    }
    s = wave_sum(s);
    if (lane == 0) v_inv[r] = rsqrtf(s * (1.f / D) + eps);
  }
}

// bf16 V of one 8-key chunk of a 64-key operand tile, in registers: the lane's dims
// 8 cidx .. 8 cidx + 7 of keys r = 0 .. 7, w[r] as 4 packed pairs. src(r) is key r's row
// (nullptr: a zero row); with the V norm, rows for which scaled(r) holds are divided by
// their RMS (rows that were normalised before they were cached are not). The row sums of
// squares are reduced over the d/8 lanes that hold the other dim chunks of the same keys,
// adjacent lanes of one wave that all take this call together.
template <int D, typename Src, typename Scaled>
__device__ __forceinline__ void v_key_chunk(Src src, Scaled scaled, bool v_norm, float eps, int cidx, u32x4 (&w)[8]) {
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const bf16_t* p = src(r);
    w[r] = p ? reinterpret_cast<const u32x4*>(p)[cidx] : u32x4{0, 0, 0, 0};
  }
  if (!v_norm) return;
  float s[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    s[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s[r] += lo_bf16(w[r][e]) * lo_bf16(w[r][e]) + hi_bf16(w[r][e]) * hi_bf16(w[r][e]);
  }
#pragma unroll
  for (int m = 1; m < kChunks; m <<= 1)
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] += __shfl_xor(s[r], m, 64);
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (scaled(r)) w[r] = scaled_chunk<bf16_t>(w[r], rsqrtf(s[r] * (1.f / D) + eps));
}

// 8 x 8 bf16 transpose: o[e] = dim e of keys 0 .. 7, key 2q in the low half of word q (the
// V^T tile's 8-key runs).
__device__ __forceinline__ void transpose8x8_bf16(const u32x4 (&w)[8], u32x4 (&o)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x = w[2 * q][e >> 1], y = w[2 * q + 1][e >> 1];
      o[e][q] = (e & 1) ? (x >> 16) | (y & 0xFFFF0000u) : (x & 0xFFFFu) | (y << 16);
    }
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a) {
  constexpr int kH = D / 2;                     // rotation pairs
  constexpr int kVec = 16 / sizeof(E);          // elements per 16-byte chunk
  constexpr int kLanesPerRow = kH / kVec;       // d = 128: 8 (bf16) or 16 (fp32)
  constexpr int kRowsPerPass = 64 / kLanesPerRow;
  constexpr int kUnroll = 2;  // rows in flight per lane (4 measured slower at every head dim: fewer resident waves)
  constexpr bool kTiled = sizeof(E) == 2;      // bf16 prefill operands are tiled
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes<E, D>];
  __shared__ float v_inv[kTokBlock];
  float2 (*zs)[kH] = reinterpret_cast<float2 (*)[kH]>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane % kLanesPerRow;  // chunk index within a half row: pairs c*kVec ..
  const int slot = lane / kLanesPerRow;
  const int t0 = blockIdx.x * kTokBlock;
  const int b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  // A short chunk's few token blocks are spread wider: n_qs blocks share one (token block,
  // KV head), block qs normalising and rotating query heads qs Gs .. qs Gs + Gs - 1; the first
  // of them also handles K, V and the operand padding.
  const int n_qs = a.q_split > 1 ? a.q_split : 1;
  const int kvh = blockIdx.y / n_qs;
  const int qs = blockIdx.y % n_qs;
  const int Gs = G / n_qs;
  const bool kv_part = qs == 0;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const E* __restrict__ wq = static_cast<const E*>(a.wq);
  const E* __restrict__ wk = static_cast<const E*>(a.wk);
  E* __restrict__ q_out = static_cast<E*>(a.q_out);
  E* __restrict__ k_rot = static_cast<E*>(a.k_rot_out);
  E* __restrict__ v_t = static_cast<E*>(a.v_t_out);
  E* __restrict__ k_cache = static_cast<E*>(a.k_cache);
  E* __restrict__ v_cache = static_cast<E*>(a.v_cache);
  const bool norm = wq != nullptr;
  // this sequence's first position, kept keys and token count (a.T is the row stride)
  const SeqPos sp = seq_pos_of(a.seq_pos, a.seq_len, a.pos_offset, a.T, a.window, b);
  const int n_tok = min(kTokBlock, sp.T - t0);  // may be <= 0 in the padding blocks
  if (n_tok <= 0 && (a.ops_kernel || !(k_rot || v_t) || !kv_part)) return;  // block-uniform

  // rotation factors of the block's renumbered positions kept + t (post-RoPE cache:
  // absolute positions pos + t), kRopeTok tokens from token ts on
  const long long p_first = a.post_rope ? sp.pos : sp.kept;
  // (two adjacent pairs per step: 16-byte table reads and LDS writes; the product of each
  // pair is the one rope_factor forms)
  auto stage = [&](int ts) {
    for (int i = threadIdx.x; i < kRopeTok<D> * (kH / 2); i += kThreads) {
      const int r = i / (kH / 2), j = 2 * (i % (kH / 2));
      if (ts + r >= n_tok) continue;
      const long long p = p_first + t0 + ts + r;
      const float4 f = *reinterpret_cast<const float4*>(a.rope + (p & (kRopeFine - 1)) * kH + j);
      const float4 cz = *reinterpret_cast<const float4*>(a.rope + (kRopeFine + (p >> 6)) * kH + j);
      *reinterpret_cast<float4*>(&zs[r][j]) = make_float4(cz.x * f.x - cz.y * f.y, cz.x * f.y + cz.y * f.x,
                                                          cz.z * f.z - cz.w * f.w, cz.z * f.w + cz.w * f.z);
    }
  };
  stage(0);
  if (!kTiled && a.v_norm && n_tok > 0)
    v_row_inv_rms<E, D>(v + ((static_cast<long long>(b) * a.T + t0) * a.Hkv + kvh) * D,
                        static_cast<long long>(a.Hkv) * D, n_tok, a.eps, v_inv, wave, lane);
  float gq[2 * kVec], gk[2 * kVec];  // gains c + w of this lane's dims (both halves)
#pragma unroll
  for (int e = 0; e < 2 * kVec; ++e) gq[e] = gk[e] = 1.f;
  if (norm) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Io<E>::unpack(*reinterpret_cast<const u32x4*>(wq + h * kH + c * kVec), gq + h * kVec);
      Io<E>::unpack(*reinterpret_cast<const u32x4*>(wk + h * kH + c * kVec), gk + h * kVec);
    }
#pragma unroll
    for (int e = 0; e < 2 * kVec; ++e) {
      gq[e] += a.norm_offset;
      gk[e] += a.norm_offset;
    }
  }
  __syncthreads();

  // One pass normalises and rotates kRowsPerPass rows per wave (kUnroll passes in flight).
  // is_k: row r is token t0 + ts + r of the K head; else row r is (token ts + r / Gs, head
  // qs Gs + r % Gs of the group), ts the first token whose factors are staged. Row passes start at wave `first`,
  // so that with few rows (a decode step) the Q rows, the K rows and the V copy below run
  // on different waves at the same time.
  auto rows = [&](const E* __restrict__ src, int n_rows, bool is_k, int first, int ts) {
    const float* g = is_k ? gk : gq;
    const int w = (wave + kWaves - first) % kWaves;
    for (int base = w * kRowsPerPass * kUnroll; base < n_rows; base += kWaves * kRowsPerPass * kUnroll) {
      float x[kUnroll][2 * kVec];
      float ss[kUnroll];
      long long off[kUnroll];
      int tt[kUnroll], zr[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int r = min(base + u * kRowsPerPass + slot, n_rows - 1);
        zr[u] = is_k ? r : r / Gs;
        tt[u] = ts + zr[u];
        const int head = is_k ? kvh : kvh * G + qs * Gs + r % Gs;
        const int H = is_k ? a.Hkv : a.Hq;
        off[u] = ((static_cast<long long>(b) * a.T + t0 + tt[u]) * H + head) * D + c * kVec;
        // (the projected rows are read once: non-temporal loads, ~3 us less per local prefill append)
        const u32x4 w0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off[u]));
        const u32x4 w1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off[u] + kH));
        Io<E>::unpack(w0, x[u]);
        Io<E>::unpack(w1, x[u] + kVec);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 2 * kVec; ++e) s += x[u][e] * x[u][e];
        ss[u] = s;
      }
      if (norm) {
#pragma unroll
        for (int m = 1; m < kLanesPerRow; m <<= 1)
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) ss[u] += __shfl_xor(ss[u], m, 64);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int r = base + u * kRowsPerPass + slot;
        if (r >= n_rows) continue;
        const int t = t0 + tt[u];
        if (norm) {
          const float inv = rsqrtf(ss[u] * (1.f / D) + a.eps);
#pragma unroll
          for (int e = 0; e < 2 * kVec; ++e) x[u][e] *= inv * g[e];
        }
        const bool to_cache = is_k && k_cache && (a.window == 0 || t >= sp.T - a.window);
        E* cdst = nullptr;
        if (to_cache) {
          const long long n = sp.pos + t;
          const long long s = a.window == 0 ? n : n % a.window;
          cdst = k_cache + ((static_cast<long long>(b) * a.Hkv + kvh) * a.cap + s) * D + c * kVec;
        }
        if (is_k && !a.post_rope) {  // the cache stores K before RoPE (rounded to the cache type)
          if (to_cache) {
            *reinterpret_cast<u32x4*>(cdst) = Io<E>::pack(x[u]);
            *reinterpret_cast<u32x4*>(cdst + kH) = Io<E>::pack(x[u] + kVec);
          }
          if (!k_rot) continue;
        }
        float y[2 * kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          const float2 z = zs[zr[u]][c * kVec + e];
          const float x0 = x[u][e], x1 = x[u][kVec + e];
          y[e] = x0 * z.x - x1 * z.y;
          y[kVec + e] = x0 * z.y + x1 * z.x;
        }
        if (is_k && a.post_rope) {  // the cache stores K rotated at its absolute position
          if (to_cache) {
            *reinterpret_cast<u32x4*>(cdst) = Io<E>::pack(y);
            *reinterpret_cast<u32x4*>(cdst + kH) = Io<E>::pack(y + kVec);
          }
          if (!k_rot) continue;
        }
        // the operand row of new token t follows the kept cached keys
        const long long R = sp.kept + t;
        if (kTiled && is_k) {  // chunks c and c + d/16 of key R within its tile
          E* dst = k_rot + ((static_cast<long long>(b) * a.Hkv + kvh) * a.Tp + (R & ~63LL)) * D +
                   (c * kTokBlock + (R & 63)) * kVec;
          *reinterpret_cast<u32x4*>(dst) = Io<E>::pack_op(y);
          *reinterpret_cast<u32x4*>(dst + kLanesPerRow * kTokBlock * kVec) = Io<E>::pack_op(y + kVec);
        } else {
          E* dst = is_k ? k_rot + ((static_cast<long long>(b) * a.Hkv + kvh) * a.Tp + R) * D + c * kVec
                        : q_out + off[u];
          *reinterpret_cast<u32x4*>(dst) = Io<E>::pack_op(y);
          *reinterpret_cast<u32x4*>(dst + kH) = Io<E>::pack_op(y + kVec);
        }
      }
    }
  };
  for (int ts = 0; ts < n_tok; ts += kRopeTok<D>) {  // one pass at d = 128
    if (ts > 0) {
      __syncthreads();  // every wave is done with the previous factors
      stage(ts);
      __syncthreads();
    }
    const int nt = min(kRopeTok<D>, n_tok - ts);
    if (q_out) rows(q, nt * Gs, false, 0, ts);  // (no Q: the prefill normalises and rotates it)
    if (kv_part) rows(k, nt, true, 1, ts);
  }

  if (kv_part && k_rot && !a.ops_kernel) {  // zero the padding rows T .. Tp-1 of this block
    for (int i = threadIdx.x; i < kTokBlock * (D / kVec); i += kThreads) {
      if (kTiled) {  // i = chunk * 64 + key in tile
        const long long t = t0 + i % kTokBlock;
        if (t >= sp.T && t < a.Tp)
          reinterpret_cast<u32x4*>(k_rot + ((static_cast<long long>(b) * a.Hkv + kvh) * a.Tp + t0) * D)[i] =
              u32x4{0, 0, 0, 0};
      } else {
        const long long t = t0 + i / (D / kVec);
        if (t >= sp.T && t < a.Tp)
          reinterpret_cast<u32x4*>(k_rot + ((static_cast<long long>(b) * a.Hkv + kvh) * a.Tp + t) * D)
              [i % (D / kVec)] = u32x4{0, 0, 0, 0};
      }
    }
  }

  // --- values: copy into the cache (16-byte chunks), transposed prefill operand --------
  // (V norm: every chunk scaled by its row's inverse RMS, rounded once)
  constexpr int kChunks = D / kVec;  // 16-byte chunks per row
  if constexpr (kTiled) {
    const bool vt_here = kv_part && v_t && !a.ops_kernel && t0 < a.Tp;  // Tp: a multiple of 128, so whole tiles
    if ((kv_part && v_cache) || vt_here) {
      // lane task i = key chunk kc (8 tokens) x dim chunk cidx; from wave 2, as above
      for (int i = (threadIdx.x + kThreads - 128) % kThreads; i < 8 * kChunks; i += kThreads) {
        const int kc = i / kChunks, cidx = i % kChunks;
        const int tk = t0 + kc * 8;
        if (tk >= sp.T && !vt_here) continue;  // uniform over the lanes of one key chunk
        u32x4 w[8];
        v_key_chunk<D>(
            [&](int r) -> const bf16_t* {
              return tk + r < sp.T ? v + ((static_cast<long long>(b) * a.T + tk + r) * a.Hkv + kvh) * D : nullptr;
            },
            [](int) { return true; }, a.v_norm, a.eps, cidx, w);
        if (v_cache) {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int t = tk + r;
            if (t >= sp.T || !(a.window == 0 || t >= sp.T - a.window)) continue;
            const long long n = sp.pos + t;
            const long long s = a.window == 0 ? n : n % a.window;
            reinterpret_cast<u32x4*>(v_cache + ((static_cast<long long>(b) * a.Hkv + kvh) * a.cap + s) * D)[cidx] = w[r];
          }
        }
        if (vt_here) {  // tile [8 key chunks][d dims][8 keys]: dims 8 cidx .. +7 of key chunk kc
          u32x4 o[8];
          transpose8x8_bf16(w, o);
          u32x4* dst = reinterpret_cast<u32x4*>(v_t + ((static_cast<long long>(b) * a.Hkv + kvh) * a.Tp + t0) * D) +
                       kc * D + cidx * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = o[e];
        }
      }
    }
  } else {
    if (v_cache) {
      for (int i = (threadIdx.x + kThreads - 128) % kThreads; i < n_tok * kChunks; i += kThreads) {  // from wave 2
        const int t = t0 + i / kChunks;
        if (!(a.window == 0 || t >= sp.T - a.window)) continue;
        const long long n = sp.pos + t;
        const long long s = a.window == 0 ? n : n % a.window;
        const int cidx = i % kChunks;
        const long long row = ((static_cast<long long>(b) * a.T + t) * a.Hkv + kvh) * D;
        const long long crow = ((static_cast<long long>(b) * a.Hkv + kvh) * a.cap + s) * D;
        u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + row) + cidx);
        if (a.v_norm) w = scaled_chunk<E>(w, v_inv[t - t0]);
        reinterpret_cast<u32x4*>(v_cache + crow)[cidx] = w;
      }
    }
    if (v_t && !a.ops_kernel) {  // (otherwise the operand kernel writes all of V^T)
      constexpr int kTS = kTileStride<E>;
      E* tile = reinterpret_cast<E*>(smem);
      __syncthreads();  // every wave is done with the rotation factors
      for (int i = threadIdx.x; i < kTokBlock * kChunks; i += kThreads) {
        const int r = i / kChunks, cidx = i % kChunks;
        const int t = t0 + r;
        E x[kVec];
        if (t < sp.T) {
          u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + ((static_cast<long long>(b) * a.T + t) * a.Hkv + kvh) * D) + cidx);
          if (a.v_norm) w = scaled_chunk<E>(w, v_inv[r]);
          __builtin_memcpy(x, &w, 16);
        } else {
#pragma unroll
          for (int e = 0; e < kVec; ++e) x[e] = E(0);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) tile[(cidx * kVec + e) * kTS + r] = x[e];
      }
      __syncthreads();
      constexpr int kTokChunks = kTokBlock / kVec;
      for (int i = threadIdx.x; i < D * kTokChunks; i += kThreads) {
        const int cc = i / kTokChunks, tc = i % kTokChunks;
        const long long t = t0 + tc * kVec;
        if (t < a.Tp) {  // Tp is a multiple of 128, so a chunk is wholly inside or outside
          const u32x4 w = *reinterpret_cast<const u32x4*>(&tile[cc * kTS + tc * kVec]);
          *reinterpret_cast<u32x4*>(v_t + ((static_cast<long long>(b) * a.Hkv + kvh) * D + cc) * a.Tp + t) = w;
        }
      }
    }
  }
}

// Prefill operands of a chunk that follows kept > 0 cached keys, or of a ragged batch
// (「PLaMo 3アーキテクチャ徹底解析」 §4.4: the attention reads every key the cache returns).
// One block = one 64-key operand tile of one (sequence, KV head): K' rows of the kept keys
// (pre-RoPE K from the cache, rotated at their renumbered positions 0 .. kept-1), V^T of
// all kept + T keys (cached V, then the chunk's own V), zeros past kept + T, with kept and
// T those of the block's sequence. Runs before the append kernel, which may overwrite
// ring slots these keys still occupy and writes the chunk's own K' rows.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void prefill_operands_kernel(AppendArgs a) {
  constexpr int kH = D / 2;
  constexpr int kVec = 16 / sizeof(E);
  constexpr int kLanesPerRow = kH / kVec;
  constexpr int kRowsPerPass = 64 / kLanesPerRow;
  constexpr bool kTiled = sizeof(E) == 2;
  constexpr int kChunks = D / kVec;
  constexpr int kTS = kTileStride<E>;  // LDS row stride (tokens) of the V^T staging tile
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes<E, D>];
  __shared__ float v_inv[kTokBlock];
  float2 (*zs)[kH] = reinterpret_cast<float2 (*)[kH]>(smem);
  E* tile = reinterpret_cast<E*>(smem);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane % kLanesPerRow;
  const int slot = lane / kLanesPerRow;
  const long long R0 = static_cast<long long>(blockIdx.x) * kTokBlock;  // first operand row
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const SeqPos sp = seq_pos_of(a.seq_pos, a.seq_len, a.pos_offset, a.T, a.window, b);
  const long long kept = sp.kept;
  const long long S = kept + sp.T;
  const long long base = sp.pos - kept;  // absolute position of renumbered key 0
  const long long bh = static_cast<long long>(b) * a.Hkv + kvh;
  const E* __restrict__ kc = static_cast<const E*>(a.k_cache) + bh * a.cap * D;
  const E* __restrict__ vc = static_cast<const E*>(a.v_cache) + bh * a.cap * D;
  const E* __restrict__ v = static_cast<const E*>(a.v);
  E* __restrict__ k_rot = static_cast<E*>(a.k_rot_out);
  E* __restrict__ v_t = static_cast<E*>(a.v_t_out);
  auto cache_row = [&](long long R) {
    const long long n = base + R;
    return (a.window == 0 ? n : n % a.window) * D;
  };

  if (k_rot) {
    if (kStageRope<D>) {  // (two adjacent pairs per step, as in the append kernel)
      for (int i = threadIdx.x; i < kTokBlock * (kH / 2); i += kThreads) {
        const int r = i / (kH / 2), j = 2 * (i % (kH / 2));
        if (R0 + r >= kept || a.post_rope) continue;
        const long long p = R0 + r;
        const float4 f = *reinterpret_cast<const float4*>(a.rope + (p & (kRopeFine - 1)) * kH + j);
        const float4 cz = *reinterpret_cast<const float4*>(a.rope + (kRopeFine + (p >> 6)) * kH + j);
        *reinterpret_cast<float4*>(&zs[r][j]) = make_float4(cz.x * f.x - cz.y * f.y, cz.x * f.y + cz.y * f.x,
                                                            cz.z * f.z - cz.w * f.w, cz.z * f.w + cz.w * f.z);
      }
      __syncthreads();
    }
    for (int r = wave * kRowsPerPass + slot; r < kTokBlock; r += kWaves * kRowsPerPass) {
      const long long R = R0 + r;
      if (R >= kept && R < S) continue;  // the chunk's own keys: the append kernel
      float y[2 * kVec];
      if (R < kept) {
        float x[2 * kVec];
        const E* src = kc + cache_row(R) + c * kVec;
        Io<E>::unpack(*reinterpret_cast<const u32x4*>(src), x);
        Io<E>::unpack(*reinterpret_cast<const u32x4*>(src + kH), x + kVec);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
          if (a.post_rope) {  // already rotated (at its absolute position) in the cache
            y[e] = x[e];
            y[kVec + e] = x[kVec + e];
          } else {
            const float2 z = kStageRope<D> ? zs[r][c * kVec + e] : rope_factor<kH>(a.rope, R, c * kVec + e);
            y[e] = x[e] * z.x - x[kVec + e] * z.y;
            y[kVec + e] = x[e] * z.y + x[kVec + e] * z.x;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 2 * kVec; ++e) y[e] = 0.f;
      }
      if (kTiled) {
        E* dst = k_rot + (bh * a.Tp + R0) * D + (c * kTokBlock + r) * kVec;
        *reinterpret_cast<u32x4*>(dst) = Io<E>::pack_op(y);
        *reinterpret_cast<u32x4*>(dst + kLanesPerRow * kTokBlock * kVec) = Io<E>::pack_op(y + kVec);
      } else {
        E* dst = k_rot + (bh * a.Tp + R) * D + c * kVec;
        *reinterpret_cast<u32x4*>(dst) = Io<E>::pack_op(y);
        *reinterpret_cast<u32x4*>(dst + kH) = Io<E>::pack_op(y + kVec);
      }
    }
  }

  if constexpr (kTiled) {
    if (v_t) {
      // V norm: the chunk's own rows (R in [kept, S)) come raw from v; cached rows were
      // normalised when they were appended
      for (int i = threadIdx.x; i < 8 * kChunks; i += kThreads) {
        const int kc = i / kChunks, cidx = i % kChunks;
        const long long Rk = R0 + kc * 8;
        u32x4 w[8];
        v_key_chunk<D>(
            [&](int r) -> const bf16_t* {
              const long long R = Rk + r;
              if (R < kept) return reinterpret_cast<const bf16_t*>(vc + cache_row(R));
              if (R < S) return reinterpret_cast<const bf16_t*>(v + ((static_cast<long long>(b) * a.T + (R - kept)) * a.Hkv + kvh) * D);
              return nullptr;
            },
            [&](int r) { return Rk + r >= kept; }, a.v_norm, a.eps, cidx, w);
        u32x4 o[8];
        transpose8x8_bf16(w, o);
        u32x4* dst = reinterpret_cast<u32x4*>(v_t + (bh * a.Tp + R0) * D) + kc * D + cidx * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = o[e];
      }
    }
  } else {
    if (v_t) {
      // V norm: the chunk's own rows (R in [kept, S)) come raw from v; cached rows were
      // normalised when they were appended
      const long long r_new = kept > R0 ? kept - R0 : 0;  // first tile row holding a new token
      const long long r_end = S - R0 < kTokBlock ? S - R0 : kTokBlock;
      if (a.v_norm && r_end > r_new)
        v_row_inv_rms<E, D>(v + ((static_cast<long long>(b) * a.T + (R0 + r_new - kept)) * a.Hkv + kvh) * D,
                            static_cast<long long>(a.Hkv) * D, static_cast<int>(r_end - r_new), a.eps,
                            v_inv + r_new, wave, lane);
      __syncthreads();  // every wave is done with the rotation factors; v_inv is complete
      for (int i = threadIdx.x; i < kTokBlock * kChunks; i += kThreads) {
        const int r = i / kChunks, cidx = i % kChunks;
        const long long R = R0 + r;
        E x[kVec];
        if (R < S) {
          const E* src = R < kept ? vc + cache_row(R)
                                  : v + ((static_cast<long long>(b) * a.T + (R - kept)) * a.Hkv + kvh) * D;
          u32x4 w = reinterpret_cast<const u32x4*>(src)[cidx];
          if (a.v_norm && R >= kept) w = scaled_chunk<E>(w, v_inv[r]);
          __builtin_memcpy(x, &w, 16);
        } else {
#pragma unroll
          for (int e = 0; e < kVec; ++e) x[e] = E(0);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) tile[(cidx * kVec + e) * kTS + r] = x[e];
      }
      __syncthreads();
      constexpr int kTokChunks = kTokBlock / kVec;
      for (int i = threadIdx.x; i < D * kTokChunks; i += kThreads) {
        const int cc = i / kTokChunks, tc = i % kTokChunks;
        const u32x4 w = *reinterpret_cast<const u32x4*>(&tile[cc * kTS + tc * kVec]);
        *reinterpret_cast<u32x4*>(v_t + (bh * D + cc) * a.Tp + R0 + tc * kVec) = w;
      }
    }
  }
}

// Caller-held rotated keys K' and values V [B, S, Hkv, D] into the prefill operand layouts
// (the ones the append kernels write). One block = one 64-key tile of one (sequence, KV
// head); rows S .. Tp-1 are zero. bf16: K' tile [D/8][64][8] as IEEE halves (exact for
// bf16 inputs in the half range), V^T tile [8][D][8]; fp32: [Tp][D] and [D][Tp].
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void prefill_pack_kernel(PackArgs a) {
  constexpr int kVec = 16 / sizeof(E);
  constexpr int kChunks = D / kVec;  // 16-byte chunks per row
  const long long R0 = static_cast<long long>(blockIdx.x) * kTokBlock;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const long long bh = static_cast<long long>(b) * a.Hkv + kvh;
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  E* __restrict__ k_out = static_cast<E*>(a.k_rot_out);
  E* __restrict__ v_out = static_cast<E*>(a.v_t_out);
  auto row_of = [&](const E* base, long long R) { return base + ((static_cast<long long>(b) * a.S + R) * a.Hkv + kvh) * D; };
  for (int i = threadIdx.x; i < kTokBlock * kChunks; i += kThreads) {
    const int r = i / kChunks, c = i % kChunks;
    const long long R = R0 + r;
    u32x4 w = R < a.S ? reinterpret_cast<const u32x4*>(row_of(k, R))[c] : u32x4{0, 0, 0, 0};
    if constexpr (sizeof(E) == 2) {
      w = u32x4{bf16x2_to_f16x2(w[0]), bf16x2_to_f16x2(w[1]), bf16x2_to_f16x2(w[2]), bf16x2_to_f16x2(w[3])};
      *reinterpret_cast<u32x4*>(k_out + (bh * a.Tp + R0) * D + (c * kTokBlock + r) * kVec) = w;
    } else {
      *reinterpret_cast<u32x4*>(k_out + (bh * a.Tp + R) * D + c * kVec) = w;
    }
  }
  if constexpr (sizeof(E) == 2) {
    for (int i = threadIdx.x; i < 8 * kChunks; i += kThreads) {  // key chunk kc x dim chunk cidx
      const int kc = i / kChunks, cidx = i % kChunks;
      u32x4 w[8], o[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const long long R = R0 + kc * 8 + r;
        w[r] = R < a.S ? reinterpret_cast<const u32x4*>(row_of(v, R))[cidx] : u32x4{0, 0, 0, 0};
      }
      transpose8x8_bf16(w, o);
      u32x4* dst = reinterpret_cast<u32x4*>(v_out + (bh * a.Tp + R0) * D) + kc * D + cidx * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = o[e];
    }
  } else {
    for (int i = threadIdx.x; i < kTokBlock * D; i += kThreads) {  // dim dd, key r (keys fastest)
      const int dd = i / kTokBlock, r = i % kTokBlock;
      const long long R = R0 + r;
      v_out[(bh * D + dd) * a.Tp + R] = R < a.S ? row_of(v, R)[dd] : E(0);
    }
  }
}

template <typename E, int D>
hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_pack_kernel<E, D>), dim3(static_cast<unsigned>(a.Tp / kTokBlock), a.Hkv, a.B),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const bool operands = a.k_rot_out || a.v_t_out;
  if (operands && a.ops_kernel) {
    const unsigned tiles = static_cast<unsigned>(a.Tp / kTokBlock);
    hipLaunchKernelGGL((prefill_operands_kernel<E, D>), dim3(tiles, a.Hkv, a.B), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // without the operand kernel the append kernel also covers the padding tokens T .. Tp-1
  const long long tokens = (operands && !a.ops_kernel) ? a.Tp : a.T;
  const unsigned gx = static_cast<unsigned>((tokens + kTokBlock - 1) / kTokBlock);
  // a bf16 chunk of a few token blocks: split the query heads over up to 2^k blocks until
  // about 1024 blocks are in flight (single-token steps keep one block per KV head)
  AppendArgs b = a;
  b.q_split = 1;
  if (sizeof(E) == 2 && a.q_out && a.T >= kTokBlock) {
    const long long blocks = static_cast<long long>(gx) * a.Hkv * a.B;
    const int G = a.Hq / a.Hkv;
    while (blocks * b.q_split < 1024 && G % (2 * b.q_split) == 0) b.q_split *= 2;
  }
  hipLaunchKernelGGL((kv_append_kernel<E, D>), dim3(gx, a.Hkv * b.q_split, a.B), dim3(kThreads), 0, stream, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append_bf16(const AppendArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 256: return launch_append<bf16_t, 256>(a, stream);
    case 512: return launch_append<bf16_t, 512>(a, stream);
    default: return launch_append<bf16_t, kHeadDim>(a, stream);
  }
}
hipError_t launch_kv_append_f32(const AppendArgs& a, hipStream_t stream) {
  return launch_append<float, kHeadDim>(a, stream);
}

hipError_t launch_prefill_pack(const PackArgs& a, bool bf16, hipStream_t stream) {
  if (!bf16) return launch_pack<float, kHeadDim>(a, stream);
  switch (a.d) {
    case 256: return launch_pack<bf16_t, 256>(a, stream);
    case 512: return launch_pack<bf16_t, 512>(a, stream);
    default: return launch_pack<bf16_t, kHeadDim>(a, stream);
  }
}

}  // namespace plamo
