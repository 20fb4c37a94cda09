// Host-only stand-ins for the kernel launchers and the HIP calls the C ABI makes, so that
// the argument validation and the decode planning (abi.cpp, plan.cpp) can be built with
// AddressSanitizer and UndefinedBehaviorSanitizer and driven on a machine without a GPU.
// Each launcher checks the invariants its kernel relies on and counts the launch.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "kernels.h"

int g_launches = 0;

#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "launcher invariant failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
      std::abort();                                                      \
    }                                                                    \
  } while (0)

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace plamo {

namespace {
float* scratch_stand_in() {  // never dereferenced
  static float fake[16];
  return fake;
}
}  // namespace

hipError_t launch_rope_table(float2* table, long long n_coarse, int d, double, double, double j_low,
                             double j_high, double, int n_rot, hipStream_t) {
  EXPECT(table && n_coarse >= 1 && (d == 128 || d == 256 || d == 512));
  EXPECT(n_rot >= 0 && n_rot <= d / 2);
  (void)j_low;
  (void)j_high;
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_kv_append_bf16(const AppendArgs& a, hipStream_t) {
  EXPECT(a.B >= 1 && a.T >= 1 && a.Hkv >= 1 && a.Hq % a.Hkv == 0 && a.Tp % 128 == 0);
  EXPECT(a.kept >= 0 && a.kept <= a.pos_offset && a.rope);
  if (a.k_rot_out || a.v_t_out) EXPECT(a.Tp >= a.kept + a.T);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_kv_append_f32(const AppendArgs& a, hipStream_t s) { return launch_kv_append_bf16(a, s); }

hipError_t launch_prefill_pack(const PackArgs& a, bool, hipStream_t) {
  EXPECT(a.B >= 1 && a.S >= 1 && a.Tp >= a.S && a.Tp % 128 == 0);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t) {
  EXPECT(a.B >= 1 && a.T >= 1 && a.Hq % a.Hkv == 0 && a.Tp % 128 == 0 && a.Tp >= a.kept + a.T);
  EXPECT(a.scale > 0.f);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefill_wide_bf16(const PrefillArgs& a, hipStream_t s) { return launch_prefill_bf16(a, s); }
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) { return launch_prefill_bf16(a, s); }

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t) {
  EXPECT(a.B >= 1 && a.Hq % a.Hkv == 0 && a.S >= 1 && a.plan.n_split >= 1 && a.plan.chunk % 64 == 0);
  EXPECT(static_cast<long long>(a.plan.n_split) * a.plan.chunk >= a.S);
  EXPECT(static_cast<long long>(a.plan.n_split - 1) * a.plan.chunk < a.S);
  EXPECT(a.plan.n_split == 1 || a.ws);
  if (a.fused && a.plan.n_split > 1) EXPECT(a.tickets);
  if (a.ws && a.ws == scratch_stand_in())  // the no-allocation decode: partials fit the scratch
    EXPECT(decode_workspace_bytes(a.B, a.Hq, a.d, a.plan) <= kDecodeScratchBytes);
  EXPECT(a.window == 0 || a.S <= a.window);
  EXPECT(a.base >= 0 && a.base + a.S == a.pos_offset + 1);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode_wide_bf16(const DecodeArgs& a, hipStream_t s) { return launch_decode_bf16(a, s); }

hipError_t decode_scratch(float** ptr) {
  *ptr = scratch_stand_in();
  return hipSuccess;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t) {
  EXPECT(a.M >= 1 && a.N >= 8 && a.K >= 64 && a.K % 64 == 0);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_rms_norm_bf16(const NormArgs& a, hipStream_t) {
  EXPECT(a.rows >= 1 && a.n >= 4);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_rms_norm_f32(const NormArgs& a, hipStream_t s) { return launch_rms_norm_bf16(a, s); }

}  // namespace plamo
