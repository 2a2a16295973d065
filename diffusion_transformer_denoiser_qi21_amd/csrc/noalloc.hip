// qi21_txt_in_noalloc: the text front with its intermediates in a scratch
// array that the library holds for the life of the process, for callers
// that may not allocate device memory during the call (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in device memory as a file-scope __device__ symbol, one
// copy per GPU the library runs on.  Its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) on the entry
// point's first call there and kept; host code never hands the symbol's
// name itself to a kernel, only that address.  Nothing in it has to start
// at zero: the normalised rows and the GELU hidden are written in full
// before they are read.  Every call on one GPU shares that GPU's array, so
// calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qi21.h"
#include "status.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)32 << 20;
constexpr int MAX_DEVICES = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

namespace {

std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// The current device's copy of the array (nullptr and the last error set on
// failure).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    (void)hipGetLastError();
    qi21::set_error_text("txt_in_noalloc: no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      qi21::set_error_text("txt_in_noalloc: hipGetSymbolAddress of the scratch array failed");
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t qi21_txt_in_noalloc_bytes(void) { return SCRATCH_BYTES; }

int qi21_txt_in_noalloc(qi21_model* m, int n, const float* feats, float* out, void* stream) {
  void* p = scratch_ptr();
  if (!p) return QI21_EDEVICE;
  return qi21::txt_in_scratch(m, n, feats, out, p, SCRATCH_BYTES, stream);
}

}  // extern "C"
