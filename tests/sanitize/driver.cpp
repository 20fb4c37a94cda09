// Drives every C-ABI entry point of include/plamo_attn.h with directed and pseudo-random
// arguments on the host (the kernel launchers are stand-ins that check their invariants).
// Built with -fsanitize=address,undefined by tests/test_host_sanitizers.py: any
// out-of-bounds access, overflow or other undefined behaviour in the argument validation or
// the decode planning aborts the run, and so does a call that passes validation with
// arguments a kernel could not take.
#include "plamo_attn.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

extern int g_launches;

namespace {

uint64_t g_state = 0x2545F4914F6CDD1DULL;
uint64_t next() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1DULL;
}
template <typename T, size_t N>
T pick(const T (&v)[N]) { return v[next() % N]; }

const long long kInts[] = {-1, 0, 1, 2, 3, 7, 8, 16, 63, 64, 65, 127, 128, 129, 255, 256, 512, 2047, 2048,
                           4096, 32767, 65535, 65536, 1LL << 30, INT_MAX};
const long long kLongs[] = {-1, 0, 1, 5, 63, 64, 2046, 2047, 2048, 32767, 131071, 1LL << 40, (1LL << 40) + 1,
                            LLONG_MAX};
const size_t kSizes[] = {0, 1, 256, 4096, 1u << 20, size_t(1) << 40, SIZE_MAX};
const float kFloats[] = {0.f, 1.f, -1.f, 1e-6f, 0.125f, NAN, INFINITY};
void* const kPtrs[] = {nullptr, reinterpret_cast<void*>(0x7F0000000000ULL), reinterpret_cast<void*>(0x7F0000000008ULL)};

int I() { return static_cast<int>(pick(kInts) > INT_MAX ? INT_MAX : pick(kInts)); }
long long L() { return pick(kLongs); }
size_t Z() { return pick(kSizes); }
float F() { return pick(kFloats); }
void* P() { return pick(kPtrs); }
int D() { return static_cast<int>(next() % 3); }        // dtypes 0, 1 and an unknown one
int O() { return static_cast<int>(next() % 3) * 2 - 1 < 0 ? 0 : static_cast<int>(next() % 3); }
int Hd() { const int v[] = {64, 128, 256, 512, 0}; return pick(v); }

int g_bad = 0;
void check(int st, const char* what) {
  if (st != 0 && st != -1 && st != -2 && st != -3) {
    std::fprintf(stderr, "%s returned %d\n", what, st);
    ++g_bad;
  }
  if (st != 0 && std::strlen(plamo_last_error()) == 0) {
    std::fprintf(stderr, "%s failed with no message\n", what);
    ++g_bad;
  }
}

void* const A = kPtrs[1];  // aligned stand-in pointer (never dereferenced)

}  // namespace

int main() {
  // ---- directed: valid calls pass validation and launch --------------------------------
  const int before = g_launches;
  float table_stub[4];
  (void)table_stub;
  plamo_rope rope = {1e6, 64.0, 4096.0, 32.0, 1.0, 0.0};
  const size_t tb = plamo_rope_table_bytes(40000, 128);
  check(plamo_rope_table_init(A, tb, 40000, 128, &rope, nullptr), "rope_table_init");
  check(plamo_kv_append(1, A, A, A, A, A, 1.f, 1e-6f, 0, A, A, A, A, A, 2048, 2, 300, 8, 2, 128, 2048, 100,
                        A, tb, 0, nullptr), "kv_append");
  check(plamo_attn_prefill(1, A, A, A, A, 2, 300, 8, 2, 128, 2048, 100, 0.088f, nullptr), "attn_prefill");
  check(plamo_attn_decode(1, A, A, A, 40000, A, A, SIZE_MAX, 8, 1, 64, 8, 128, 0, 32767, A, tb, 0.088f, 0, nullptr),
        "attn_decode");
  check(plamo_attn_decode_noalloc(1, A, A, A, 40000, A, 8, 1, 64, 8, 128, 0, 32767, A, tb, 0.088f, 0, nullptr),
        "attn_decode_noalloc");
  check(plamo_decode_step(1, A, A, A, A, A, 1.f, 1e-6f, A, A, 40000, A, A, SIZE_MAX, 8, 64, 8, 128, 0, 32767, A, tb,
                          0.088f, 0, nullptr), "decode_step");
  check(plamo_prefill_pack(1, A, A, A, A, 2, 777, 2, 128, nullptr), "prefill_pack");
  if (g_launches - before != 7 || g_bad) {
    std::fprintf(stderr, "directed valid calls: %d launches, %d bad\n", g_launches - before, g_bad);
    return 1;
  }

  // ---- valid shapes pass, and each becomes a rejection when one argument is made wrong ----
  // (the sizes reported by the *_bytes queries are exactly what the calls require)
  for (int it = 0; it < 4000; ++it) {
    const int Bs[] = {1, 2, 3, 8, 64, 1000};
    const int Hks[] = {1, 2, 8};
    const int Gs[] = {1, 2, 4, 8};
    const int Ws[] = {0, 16, 100, 2048};
    const long long Ps[] = {0, 1, 15, 16, 99, 2047, 2048, 5000, 32767, 131071, 1LL << 22};
    const int Ts[] = {1, 2, 127, 128, 300};
    const int B = pick(Bs), Hkv = pick(Hks), Hq = Hkv * pick(Gs), window = pick(Ws), T = pick(Ts);
    const long long pos = pick(Ps);
    const int d = 128, order = static_cast<int>(next() % 2);
    const long long kept = window ? (pos < window - 1 ? pos : window - 1) : pos;
    const long long cap = window ? window : pos + T;
    // pre-RoPE reads cover renumbered positions < kept + T, post-RoPE absolute ones < pos + T
    const size_t tb = plamo_rope_table_bytes(order ? pos + T : kept + T, d);
    void* const M = static_cast<char*>(A) + 8;  // 8-byte aligned only
    auto want = [&](int got, int expect, const char* what) {
      if (got != expect) {
        std::fprintf(stderr, "%s: status %d, expected %d (B=%d Hq=%d Hkv=%d W=%d T=%d pos=%lld order=%d): %s\n",
                     what, got, expect, B, Hq, Hkv, window, T, pos, order, plamo_last_error());
        ++g_bad;
      }
    };

    // append + prefill of a chunk of T tokens
    want(plamo_kv_append(1, A, A, A, A, A, 1.f, 1e-6f, 0, A, A, A, A, A, cap, B, T, Hq, Hkv, d, window, pos, A, tb,
                         order, nullptr), 0, "kv_append");
    want(plamo_kv_append(1, A, A, A, A, A, 1.f, 1e-6f, 0, A, A, A, A, A, cap - 1, B, T, Hq, Hkv, d, window, pos, A,
                         tb, order, nullptr), -1, "kv_append cap - 1");
    want(plamo_kv_append(1, A, A, A, A, nullptr, 1.f, 1e-6f, 0, A, A, A, A, A, cap, B, T, Hq, Hkv, d, window, pos,
                         A, tb, order, nullptr), -1, "kv_append one norm weight");
    want(plamo_kv_append(1, A, A, A, A, A, 1.f, 1e-6f, 0, A, M, A, A, A, cap, B, T, Hq, Hkv, d, window, pos, A, tb,
                         order, nullptr), -1, "kv_append misaligned");
    // the bf16 prefill's documented limit on the attended keys
    const int big = (kept + T) * d > (1LL << 29) ? -2 : 0;
    want(plamo_attn_prefill(1, A, A, A, A, B, T, Hq, Hkv, d, window, pos, 0.088f, nullptr), big, "attn_prefill");
    want(plamo_attn_prefill(1, A, A, A, A, B, T, Hq + (Hkv > 1 ? 1 : 0), Hkv, d, window, pos, 0.088f, nullptr),
         Hkv > 1 ? -1 : big, "attn_prefill Hq % Hkv");
    want(plamo_attn_prefill_fused_q(1, A, A, 1.f, 1e-6f, A, A, A, B, T, Hq, Hkv, d, window, pos, A, tb, order,
                                    0.088f, nullptr), big, "fused_q");
    want(plamo_attn_prefill_fused_q(1, A, A, 1.f, 1e-6f, A, A, A, B, T, Hq, Hkv, d, window, pos, A, 0, order,
                                    0.088f, nullptr), big ? big : -3, "fused_q no table");
    want(plamo_prefill_pack(1, A, A, A, A, B, kept + T, Hkv, d, nullptr), 0, "prefill_pack");

    // decode of one token (the workspace sizes queried are the sizes required)
    const long long cd = window ? window : pos + 1;
    const size_t tbd = plamo_rope_table_bytes(order ? pos + 1 : kept + 1, d);
    const size_t ws = plamo_attn_decode_workspace_bytes(B, Hq, Hkv, d, window, pos);
    want(plamo_attn_decode(1, A, A, A, cd, A, ws ? A : nullptr, ws, B, 1, Hq, Hkv, d, window, pos, A, tbd, 0.088f,
                           order, nullptr), 0, "attn_decode");
    if (ws)
      want(plamo_attn_decode(1, A, A, A, cd, A, A, ws - 1, B, 1, Hq, Hkv, d, window, pos, A, tbd, 0.088f, order,
                             nullptr), -3, "attn_decode workspace - 1");
    want(plamo_attn_decode(1, A, A, A, cd - 1, A, A, ws, B, 1, Hq, Hkv, d, window, pos, A, tbd, 0.088f, order,
                           nullptr), -1, "attn_decode cap - 1");
    // a workspace sized for a later position serves this one
    const size_t ws_later = plamo_attn_decode_workspace_bytes(B, Hq, Hkv, d, window, pos + 1 + static_cast<long long>(next() % 5000));
    if (ws_later < ws) {
      std::fprintf(stderr, "decode workspace shrinks with the position (pos %lld)\n", pos);
      ++g_bad;
    }
    want(plamo_attn_decode(1, A, A, A, window ? cd : cd + 5000, A, ws_later ? A : nullptr, ws_later, B, 1, Hq, Hkv, d,
                           window, pos, A, tbd, 0.088f, order, nullptr), 0, "attn_decode, later workspace");
    want(plamo_attn_decode_noalloc(1, A, A, A, cd, A, B, 1, Hq, Hkv, d, window, pos, A, tbd, 0.088f, order, nullptr),
         ws > PLAMO_DECODE_SCRATCH_BYTES ? -3 : 0, "attn_decode_noalloc");
    const size_t wss = plamo_decode_step_workspace_bytes(B, Hq, Hkv, d, window, pos);
    const size_t tbs = plamo_rope_table_bytes(order ? pos + 1 : kept + 1, d);
    want(plamo_decode_step(1, A, A, A, A, A, 1.f, 1e-6f, A, A, cd, A, wss ? A : nullptr, wss, B, Hq, Hkv, d, window,
                           pos, A, tbs, 0.088f, order, nullptr), 0, "decode_step");
    if (wss)
      want(plamo_decode_step(1, A, A, A, A, A, 1.f, 1e-6f, A, A, cd, A, A, wss - 1, B, Hq, Hkv, d, window, pos, A,
                             tbs, 0.088f, order, nullptr), -3, "decode_step workspace - 1");
    want(plamo_decode_step(1, A, A, A, A, A, 1.f, 1e-6f, A, A, cd, A, A, wss, B, Hq, Hkv, d, window, pos, A, tbs,
                           -1.f, order, nullptr), -1, "decode_step negative scale");
    const size_t wsr = plamo_attn_decode_ragged_workspace_bytes(B, Hq, Hkv, d, window, pos);
    want(plamo_attn_decode_ragged(1, A, A, A, cd, A, wsr ? A : nullptr, wsr, B, Hq, Hkv, d, window,
                                  static_cast<const long long*>(A), pos, A, tbd, 0.088f, order, nullptr),
         0, "attn_decode_ragged");
    if (g_bad) return 1;
  }

  // ---- pseudo-random arguments, every entry point --------------------------------------
  for (int it = 0; it < 20000; ++it) {
    plamo_rope r = {static_cast<double>(F()) * 1e6, static_cast<double>(F()) * 64, 4096.0, 32.0, 1.0,
                    static_cast<double>(F())};
    const int d = Hd();
    const long long mp = L();
    (void)plamo_rope_table_bytes(mp, d);
    (void)plamo_prefill_padded_len(L());
    switch (next() % 14) {
      case 0: check(plamo_rope_table_init(P(), Z(), mp, d, (next() & 1) ? &r : nullptr, nullptr), "rope_table_init"); break;
      case 1: check(plamo_kv_append(D(), P(), P(), P(), P(), P(), F(), F(), I() & 1, P(), P(), P(), P(), P(), L(), I(),
                                    I(), I(), I(), d, I(), L(), P(), Z(), O(), nullptr), "kv_append"); break;
      case 2: check(plamo_kv_append_ragged(D(), P(), P(), P(), P(), P(), F(), F(), I() & 1, P(), P(), P(), P(), P(),
                                           L(), I(), I(), I(), I(), d, I(), static_cast<const long long*>(P()),
                                           static_cast<const int*>(P()), L(), P(), Z(), O(), nullptr),
                    "kv_append_ragged"); break;
      case 3: check(plamo_attn_prefill(D(), P(), P(), P(), P(), I(), I(), I(), I(), d, I(), L(), F(), nullptr),
                    "attn_prefill"); break;
      case 4: check(plamo_attn_prefill_ragged(D(), P(), P(), P(), P(), I(), I(), I(), I(), d, I(),
                                              static_cast<const long long*>(P()), static_cast<const int*>(P()), L(),
                                              F(), nullptr), "attn_prefill_ragged"); break;
      case 5: check(plamo_attn_prefill_fused_q(D(), P(), P(), F(), F(), P(), P(), P(), I(), I(), I(), I(), d, I(), L(),
                                               P(), Z(), O(), F(), nullptr), "fused_q"); break;
      case 6: check(plamo_attn_prefill_fused_q_ragged(D(), P(), P(), F(), F(), P(), P(), P(), I(), I(), I(), I(), d,
                                                      I(), static_cast<const long long*>(P()),
                                                      static_cast<const int*>(P()), L(), P(), Z(), O(), F(), nullptr),
                    "fused_q_ragged"); break;
      case 7: (void)plamo_attn_decode_workspace_bytes(I(), I(), I(), d, I(), L());
              check(plamo_attn_decode(D(), P(), P(), P(), L(), P(), P(), Z(), I(), I(), I(), I(), d, I(), L(), P(), Z(),
                                      F(), O(), nullptr), "attn_decode"); break;
      case 8: check(plamo_attn_decode_noalloc(D(), P(), P(), P(), L(), P(), I(), I(), I(), I(), d, I(), L(), P(), Z(),
                                              F(), O(), nullptr), "attn_decode_noalloc"); break;
      case 9: (void)plamo_attn_decode_ragged_workspace_bytes(I(), I(), I(), d, I(), L());
              check(plamo_attn_decode_ragged(D(), P(), P(), P(), L(), P(), P(), Z(), I(), I(), I(), d, I(),
                                             static_cast<const long long*>(P()), L(), P(), Z(), F(), O(), nullptr),
                    "attn_decode_ragged"); break;
      case 10: (void)plamo_decode_step_workspace_bytes(I(), I(), I(), d, I(), L());
               check(plamo_decode_step(D(), P(), P(), P(), P(), P(), F(), F(), P(), P(), L(), P(), P(), Z(), I(), I(),
                                       I(), d, I(), L(), P(), Z(), F(), O(), nullptr), "decode_step"); break;
      case 11: check(plamo_prefill_pack(D(), P(), P(), P(), P(), I(), L(), I(), d, nullptr), "prefill_pack"); break;
      case 12: check(plamo_linear(P(), P(), P(), L(), I(), I(), nullptr), "linear");
               check(plamo_qkv_projection(P(), P(), P(), P(), P(), L(), I(), I(), I(), d, nullptr), "qkv_projection");
               break;
      default: check(plamo_rms_norm(D(), P(), P(), F(), F(), P(), P(), L(), I(), nullptr), "rms_norm");
               (void)plamo_status_str(static_cast<int>(next() % 11) - 5); break;
    }
    if (g_bad) return 1;
  }
  std::printf("host sanitizer drive ok: %d launches passed validation\n", g_launches);
  return 0;
}
