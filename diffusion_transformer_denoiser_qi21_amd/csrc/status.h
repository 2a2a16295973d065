// The calling thread's last-error text, shared by the host sources of the C
// ABI (qi21_last_error returns it; every entry point clears it on entry and
// sets it when it returns an error status).
#ifndef QI21_STATUS_H
#define QI21_STATUS_H

#include <stddef.h>

struct qi21_model;

namespace qi21 {
void set_error_text(const char* msg);  // "" clears

// qi21_txt_in with its two intermediates carved from the caller's scratch
// (bytes long, 256-byte aligned): EINVAL, before any device work, when n
// rows do not fit.  Allocates nothing.
int txt_in_scratch(qi21_model* m, int n, const float* feats, float* out, void* scratch, size_t bytes, void* stream);
}  // namespace qi21

#endif
