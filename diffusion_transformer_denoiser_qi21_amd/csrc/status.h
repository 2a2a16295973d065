// The calling thread's last-error text, shared by the host sources of the C
// ABI (qi21_last_error returns it; every entry point clears it on entry and
// sets it when it returns an error status).
#ifndef QI21_STATUS_H
#define QI21_STATUS_H

namespace qi21 {
void set_error_text(const char* msg);  // "" clears
}  // namespace qi21

#endif
