// Stand-ins for the device launchers, linked into the sanitized host build
// in their place.  The host checks only drive calls that must be refused (or
// must fail on allocation) before any device work, so reaching one of these
// is itself a failure: each one reports the launcher's name and aborts.
#include <cstdio>
#include <cstdlib>

#include "qi21_internal.h"

namespace {
[[noreturn]] void reached(const char* name) {
  std::fprintf(stderr, "host check reached the device launcher %s\n", name);
  std::abort();
}
}  // namespace

namespace qi21 {

hipError_t launch_gemm(int, const GemmArgs&, int, hipStream_t) { reached("launch_gemm"); }
hipError_t launch_flash(const FlashArgs&, hipStream_t) { reached("launch_flash"); }
hipError_t launch_flash(const FlashArgs*, int, hipStream_t) { reached("launch_flash (segments)"); }
hipError_t launch_rowop(int, int, int, float*, const float*, f16*, const float*, int, int, float, float, hipStream_t,
                        int, size_t, uint8_t*, int) {
  reached("launch_rowop");
}
hipError_t launch_txtnorm(int, int, const float*, const float*, float, f16*, hipStream_t) { reached("launch_txtnorm"); }
hipError_t launch_qkrope(int, int, f16*, int, const float*, const float*, const float*, const float*, float, f16*, int,
                         hipStream_t) {
  reached("launch_qkrope");
}
hipError_t launch_embed(int, int, const float*, const float*, float*, hipStream_t) { reached("launch_embed"); }
hipError_t launch_final(int, int, const float*, const float*, const float*, float, float*, int*, hipStream_t) {
  reached("launch_final");
}
hipError_t launch_commit(int, const float*, float*, const int*, hipStream_t) { reached("launch_commit"); }
hipError_t launch_mods(int, const float*, float*, hipStream_t) { reached("launch_mods"); }
hipError_t launch_plane(int, const void*, int, int, f16*, int, int, int, hipStream_t, int, int) {
  reached("launch_plane");
}
hipError_t launch_plane4(int, int, f16*, int, uint8_t*, hipStream_t) { reached("launch_plane4"); }
hipError_t launch_plane8(int, int, f16*, int, uint8_t*, hipStream_t) { reached("launch_plane8"); }
hipError_t launch_time_mods(int, float, const float*, const float*, const float*, const float*, float*, float*, float*,
                            hipStream_t) {
  reached("launch_time_mods");
}
hipError_t launch_axpy(int, float, const float*, float*, hipStream_t) { reached("launch_axpy"); }
hipError_t launch_to_f32(int, const void*, size_t, float*, hipStream_t) { reached("launch_to_f32"); }
hipError_t launch_fill32(void*, uint32_t, size_t, hipStream_t) { reached("launch_fill32"); }
hipError_t launch_scale(int, const float*, float, float*, hipStream_t) { reached("launch_scale"); }
hipError_t launch_rope_pack(int, const float*, const float*, float*, hipStream_t) { reached("launch_rope_pack"); }

}  // namespace qi21
