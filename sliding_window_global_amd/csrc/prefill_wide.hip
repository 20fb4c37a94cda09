// Flash-style causal / sliding-window GQA prefill for wide heads (d = 256, 512) on gfx950
// bf16 MFMA.
//
// 「PLaMo 3アーキテクチャ徹底解析」 §4.5: A = softmax(Q'K'^T * scale + M), O = A V per query
// head, KV head h / (Hq/Hkv) (§4.2); §5.1: the mask keeps j <= i and, on local layers,
// i - j < W. The wide heads are those of the Gemma-4-shaped layers of the page's §8 table
// (local d = 256, global d = 512, dot-product factor 1 passed as `scale`). Key tiles wholly
// outside every row's window are skipped, so a local layer costs O(T W) (§5.3).
//
// Why not the d = 128 kernel widened: its wave holds 32 query rows, i.e. Q' and O^T of
// 32 x d each in registers, which at d = 512 is 384 of the 512 registers a lane can have.
// Here a wave holds NB blocks of 16 rows and uses the 16x16x32 MFMAs: f16 for the scores
// (Q' and K' are IEEE halves), bf16 for P V.
//
// Work decomposition
//   block  = waves x 16 NB query rows of one sequence, for kHeads query heads of one KV
//            group: at d = 256 8 waves, two query heads x 4 waves x 32 rows sharing every
//            K'/V^T copy (128-row blocks waste fewer masked pairs at the window edge than
//            256-row ones; the two heads halve the copies per row); at d = 512 8 waves x 16
//            rows of one head (the 128 KiB of buffers allow one block). Either way two waves
//            per SIMD, each within 256 registers (with one wave per SIMD the LDS reads and the
//            step barrier are not hidden). Query row t sits at renumbered position kept + t and
//            attends operand keys 0 .. kept + t.
//   step   = 32 keys, one half of a 64-key operand tile (K' tile [d/8][64][8], V^T tile
//            [8][d][8], both written by the append kernel). Each half is one set of
//            1 KiB direct copies into LDS (buffer loads with the LDS bit: the K' half is
//            512-byte runs of each dim chunk, the V^T half is contiguous), double
//            buffered over four LDS objects, one barrier per step, steps from the
//            diagonal downwards.
//   math   = S^T[32 keys][16 rows] = K' Q'^T as two 16-key blocks, then
//            O^T[d][16 rows] += V^T[d][32 keys] P^T. The query index is the MFMA column,
//            so each lane owns one row (of each of its NB blocks) and the 16 lanes of a
//            row group share it: row maxima and sums reduce over lanes l, l^16, l^32, l^48.
//            K' rows are read in the order that gives each lane eight consecutive keys
//            across the two S^T blocks, exactly the P^T operand of the P V MFMA (the copy
//            into LDS already places them in that order, so each fragment read is
//            contiguous); V^T is read in natural key order. Each K' fragment feeds NB MFMAs.
//            Fragments come from LDS through a 3-deep register ring, so a read has three
//            MFMA groups to land before its own.
//   softmax = exp2 domain (Q' pre-scaled by scale * log2 e, rounded to half); lazy rescaling: the
//            reference of a row moves only when a score exceeds it by 2^8; row sums from
//            the same bf16-rounded P as P V.
//   launch = 1-D grid remapped so that the query heads sharing a KV head and neighbouring
//            query blocks land on the same XCD; causal work is ordered longest-first.
#include "common.h"
#include "kernels.h"

namespace plamo {

namespace {

constexpr int kBN = 32;                // keys per step
constexpr int kRing = 3;               // LDS operand fragments in flight per wave (2 and 4 measured no better)
constexpr float kRescaleLog2 = 8.f;    // lazy-rescale threshold (log2 units)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left alone (gfx9 encoding: bits 3:0 and 15:14)
constexpr unsigned wait_vmcnt(int n) { return 0x0F70u | (n & 15) | ((n >> 4) << 14); }

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3: 32-bit data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// the score product: Q' and K' are IEEE halves (same MFMA rate as bf16, three more bits)
__device__ __forceinline__ f32x4 mfma16_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Barrier without the memory fence of __syncthreads (which would also wait for the copies
// of the next step still in flight); each wave has waited for its own copies before.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Key (within a 32-key step) whose K' row feeds row m of S^T block kb. The accumulator
// rows of lane group g are 4g .. 4g+3, so group g then holds keys 8g + 4kb + 0..3 of block
// kb: keys 8g .. 8g+7 over both blocks, in the order of the P^T operand.
__device__ __forceinline__ int key_of(int m, int kb) { return ((m >> 2) << 3) | (kb << 2) | (m & 3); }

// D: head dim; NB: 16-row blocks per wave; kWaves: waves per block; kOcc: blocks per CU the
// register budget is cut for; kHeads: query heads of one KV group per block (its waves split
// into kHeads row groups of the same query rows, sharing every K'/V^T copy).
template <int D, int NB, int kWaves, int kOcc, bool kLocal, int kHeads>
__global__ __launch_bounds__(kWaves * 64, kOcc) void prefill_wide_kernel(PrefillArgs a) {
  constexpr int kRowsW = 16 * NB;         // query rows per wave
  constexpr int kWavesH = kWaves / kHeads;  // waves per query head
  constexpr int BM = kWavesH * kRowsW;    // query rows per block
  constexpr int kKS = D / 32;             // k-steps of S^T over the head dim
  constexpr int kDT = D / 16;             // 16-dim blocks of O^T
  constexpr int kSub = kBN * D;           // bf16 elements of a K' or V^T half tile
  constexpr int kLoads = kSub * 2 / 1024 / kWaves;  // 1 KiB copies per wave per half tile
  constexpr int kTileBytes = 64 * D * 2;  // one 64-key operand tile
  __shared__ __attribute__((aligned(1024))) bf16_t ks0[kSub];
  __shared__ __attribute__((aligned(1024))) bf16_t ks1[kSub];
  __shared__ __attribute__((aligned(1024))) bf16_t vs0[kSub];
  __shared__ __attribute__((aligned(1024))) bf16_t vs1[kSub];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // MFMA column = query row within a 16-row block
  const int g = lane >> 4;  // lane group

  // ---- block -> (b, kv head, query block, query heads in group), XCD-aware ---------
  const int G = a.Hq / a.Hkv;
  const int GH = G / kHeads;  // blocks per (query block, KV head)
  const int nqb = (a.T + BM - 1) / BM;
  const unsigned total = gridDim.x;
  unsigned logical = blockIdx.x;
  if ((total & 7u) == 0) logical = (blockIdx.x & 7u) * (total >> 3) + (blockIdx.x >> 3);
  const int g_in = logical % GH;
  unsigned rest = logical / GH;
  const int qb_order = rest % nqb;
  rest /= nqb;
  const int kvh = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int hq = kvh * G + g_in * kHeads + wave / kWavesH;  // the wave's query head
  const int qb = kLocal ? qb_order : nqb - 1 - qb_order;
  const int i0 = qb * BM;

  const SeqPos sp = seq_pos_of(a.seq_pos, a.seq_len, a.pos_offset, a.T, a.window, b);
  const int kept = static_cast<int>(sp.kept);
  const int n_rows = sp.T;
  if (i0 >= n_rows) return;  // block-uniform, before any barrier
  const int last_row = min(i0 + BM, n_rows) - 1;
  const int lo = kLocal ? max(0, kept + i0 - a.window + 1) : 0;
  const int kt_hi = (kept + last_row) / kBN;
  const int n_steps = kt_hi - lo / kBN + 1;

  const long long bh = static_cast<long long>(b) * a.Hkv + kvh;
  const int op_bytes = static_cast<int>(a.Tp * D * 2);
  const __amdgpu_buffer_rsrc_t k_rsrc = make_rsrc(static_cast<const bf16_t*>(a.k_rot) + bh * a.Tp * D, op_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = make_rsrc(static_cast<const bf16_t*>(a.v_t) + bh * a.Tp * D, op_bytes);
  // Copy i (0 .. kWaves kLoads - 1) of a half tile fills LDS bytes 1024 i .. +1023. K': dim chunks
  // 2i and 2i+1, 32 keys each, from 512-byte runs 1 KiB apart in the 64-key tile, slot
  // 16 kb + m of a run taking key key_of(m, kb) (each lane fetches the key its LDS slot
  // holds), so that the 16 keys one S^T fragment read needs are 256 contiguous bytes; V^T:
  // the half's bytes in order. The half (0 or 1) goes in the scalar offset with the tile.
  const uint32_t k_off = static_cast<uint32_t>((2 * wave * kLoads + (lane >> 5)) * 1024 +
                                               key_of(lane & 15, (lane >> 4) & 1) * 16);
  const uint32_t v_off = static_cast<uint32_t>(wave * kLoads * 1024 + lane * 16);
  auto issue = [&](int step, bf16_t* kbuf, bf16_t* vbuf) __attribute__((always_inline)) {
    const int key32 = kt_hi - step;
    const int t_off = (key32 >> 1) * kTileBytes;
    const int h = key32 & 1;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (lds_ptr_t)(kbuf + (wave * kLoads + i) * 512), 16,
                                               k_off + i * 2048, t_off + h * 512, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rsrc, (lds_ptr_t)(vbuf + (wave * kLoads + i) * 512), 16,
                                               v_off + i * 1024, t_off + h * (kSub * 2), 0, 0);
    }
  };

  // ---- Q' fragments (B operand of S^T): block nb, row n, dims 32 s + 8 g .. +7 -------
  const float c = a.scale * 1.4426950408889634f;
  const int r0 = i0 + (wave % kWavesH) * kRowsW;  // first row of the wave
  const int p0 = kept + r0;           // its position
  f16x8 qf[NB][kKS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int row = r0 + nb * 16 + n;
    const bool ok = row < n_rows;
    const f16_t* src = static_cast<const f16_t*>(a.q_rot) +
                       ((static_cast<long long>(b) * a.T + (ok ? row : 0)) * a.Hq + hq) * D + g * 8;
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      u32x4 w = ok ? *reinterpret_cast<const u32x4*>(src + s * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_f16x2(lo_f16(w[i]) * c, hi_f16(w[i]) * c);
      qf[nb][s] = __builtin_bit_cast(f16x8, w);
    }
  }

  f32x4 oacc[NB][kDT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) oacc[nb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
  }

  // wave-uniform: does the step hold a masked pair for some row of the wave?
  auto needs_mask = [&](int key0) __attribute__((always_inline)) {
    return (key0 + kBN - 1 > p0) || (kLocal && p0 + kRowsW - 1 - key0 >= a.window);
  };

  auto compute = [&](int step, const bf16_t* kbuf, const bf16_t* vbuf) __attribute__((always_inline)) {
    const int key0 = (kt_hi - step) * kBN;
    f32x4 sacc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sacc[nb][0] = sacc[nb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K' in LDS: [d/8 chunks][32 slots][8], slot 16 kb + n holding key key_of(n, kb); fragment
    // i = 2s + kb (k-step s) reads chunk 4s + g. V^T in LDS: [4 key chunks][d][8]; dim block dt
    // reads chunk g, dim 16 dt + n. Both go through a ring of kRing registers: fragment i + kRing
    // is read as soon as fragment i has been issued to the MFMAs, so each LDS read has kRing
    // MFMA groups to land (read one at a time, the wave stalled on every read).
    auto kread = [&](int i) __attribute__((always_inline)) {
      return *reinterpret_cast<const f16x8*>(kbuf + ((4 * (i >> 1) + g) * kBN + (i & 1) * 16 + n) * 8);
    };
    auto vread = [&](int dt) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(vbuf + (g * D + dt * 16 + n) * 8);
    };
    f16x8 kr[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) kr[i] = kread(i);
#pragma unroll
    for (int i = 0; i < 2 * kKS; ++i) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[nb][i & 1] = mfma16_f16(kr[i % kRing], qf[nb][i >> 1], sacc[nb][i & 1]);
      if (i + kRing < 2 * kKS) kr[i % kRing] = kread(i + kRing);
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 vr[kRing];  // the first V^T fragments land during the softmax below
#pragma unroll
    for (int i = 0; i < kRing; ++i) vr[i] = vread(i);

    // P^T: lane (n, g) of block nb holds keys key0 + 8g + j, j = 4 kb + e
    const bool mask = needs_mask(key0);
    bf16x8 pf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float x[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[kb * 4 + e] = sacc[nb][kb][e];
      if (mask) {
        const int dq = p0 + nb * 16 + n - key0 - 8 * g;  // row position minus the lane's first key
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (!(j <= dq && (!kLocal || dq - j < a.window))) x[j] = -INFINITY;
      }
      float mx = x[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (__builtin_amdgcn_ballot_w64(mx > m_run[nb] + kRescaleLog2) != 0) {  // wave-uniform
        const float m_new = fmaxf(m_run[nb], mx);
        // a row with no visible key so far keeps -inf (and its zero state)
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run[nb] - m_new);
        l_run[nb] *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) oacc[nb][dt] *= alpha;
        m_run[nb] = m_new;
      }
      const float m_use = m_run[nb] == -INFINITY ? 0.f : m_run[nb];
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[i] = pack_bf16x2(fast_exp2(x[2 * i] - m_use), fast_exp2(x[2 * i + 1] - m_use));
        l_run[nb] = add_bf16x2(w[i], l_run[nb]);
      }
      pf[nb] = __builtin_bit_cast(bf16x8, w);
    }

#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[nb][dt] = mfma16(vr[dt % kRing], pf[nb], oacc[nb][dt]);
      if (dt + kRing < kDT) vr[dt % kRing] = vread(dt + kRing);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One step, one barrier: each wave waits for its own copies of this step, and the barrier
  // then says both that every copy of the step has landed and that every wave is done
  // reading the other buffers (the previous step), which are refilled with the next half
  // tile while this one is computed.
  auto run_step = [&](int step, const bf16_t* kbuf, const bf16_t* vbuf, bf16_t* k_next, bf16_t* v_next)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    block_barrier();
    if (step + 1 < n_steps) issue(step + 1, k_next, v_next);
    compute(step, kbuf, vbuf);
  };

  issue(0, ks0, vs0);
  for (int step = 0; step < n_steps; step += 2) {
    run_step(step, ks0, vs0, ks1, vs1);
    if (step + 1 < n_steps) run_step(step + 1, ks1, vs1, ks0, vs0);
  }

  // ---- normalise, then store whole rows through LDS ----------------------------------
  // The lane holds dims 16 dt + 4 g .. +3 of its row: stored as they are, every store would
  // write 32 B into each of 16 rows. Instead each wave stages one 16-row block at a time in
  // its share of the four operand buffers (with 8 waves one eighth of them: 16 whole rows at
  // d = 256 and at d = 512), 16-byte chunk c of row n at chunk c ^ n (conflict-free writes and
  // row reads), and writes whole rows with 16-byte stores.
  block_barrier();  // every wave is past its last operand read
  constexpr int kPerBuf = kWaves / 4;  // waves sharing one operand buffer
  static_assert(kWaves % 4 == 0 && 16 * D <= kSub / kPerBuf, "a wave stages 16 whole rows in its share");
  const int bi = wave / kPerBuf;
  bf16_t* const stage = (bi == 0 ? ks0 : bi == 1 ? ks1 : bi == 2 ? vs0 : vs1) + (wave % kPerBuf) * (kSub / kPerBuf);
  constexpr int kRowChunks = D / 8;             // 16-byte chunks per row
  constexpr int kRowsPerRead = 64 / kRowChunks;  // rows one 64-lane read covers
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = l_run[nb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.f / l;  // (rows past n_rows: never stored)
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[nb][dt][0] * inv, oacc[nb][dt][1] * inv);
      w[1] = pack_bf16x2(oacc[nb][dt][2] * inv, oacc[nb][dt][3] * inv);
      const int c = 2 * dt + (g >> 1);
      *reinterpret_cast<u32x2*>(stage + n * D + (c ^ n) * 8 + (g & 1) * 4) = w;
    }
    // the wave's own staging writes are done before its reads (no other wave touches them)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    bf16_t* const out_base = static_cast<bf16_t*>(a.out) + static_cast<long long>(hq) * D;
    const int c = lane % kRowChunks;
#pragma unroll
    for (int j = 0; j < 16 / kRowsPerRead; ++j) {
      const int r = j * kRowsPerRead + lane / kRowChunks;  // row of the block, chunk c of it
      const u32x4 w = *reinterpret_cast<const u32x4*>(stage + r * D + (c ^ r) * 8);
      const int row = r0 + nb * 16 + r;
      if (row < n_rows)  // (not read again by this kernel: streamed past the caches)
        __builtin_nontemporal_store(
            w, reinterpret_cast<u32x4*>(out_base + (static_cast<long long>(b) * a.T + row) * a.Hq * D + c * 8));
    }
    if (nb + 1 < NB) {  // the reads are done before the next block's writes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
    }
  }
}

template <int D, int NB, int kWaves, int kOcc, int kHeads>
hipError_t launch_wide(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (kHeads > 1) {  // a group size kHeads does not divide: one head per block
    if ((a.Hq / a.Hkv) % kHeads != 0) return launch_wide<D, NB, kWaves / kHeads, kOcc * kHeads, 1>(a, stream);
  }
  constexpr int BM = kWaves / kHeads * 16 * NB;
  const long long blocks = (a.T + BM - 1) / BM * static_cast<long long>(a.Hq / kHeads) * a.B;
  if (a.window > 0)
    hipLaunchKernelGGL((prefill_wide_kernel<D, NB, kWaves, kOcc, true, kHeads>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_wide_kernel<D, NB, kWaves, kOcc, false, kHeads>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

#ifndef WIDE_CFG256
#define WIDE_CFG256 2, 8, 1, 2
#endif
#ifndef WIDE_CFG512
#define WIDE_CFG512 1, 8, 1, 1
#endif
hipError_t launch_prefill_wide_bf16(const PrefillArgs& a, hipStream_t stream) {
  if (a.d == 256) return launch_wide<256, WIDE_CFG256>(a, stream);
  return launch_wide<512, WIDE_CFG512>(a, stream);
}

}  // namespace plamo
