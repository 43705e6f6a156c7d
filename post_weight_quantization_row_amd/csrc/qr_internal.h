// qr_internal.h -- helpers shared by the translation units of libqrow.so
// (not part of the C-ABI; hidden from the exported symbol table).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#define QR_HIDDEN __attribute__((visibility("hidden")))

// Clears this thread's error message (every entry point starts with it).
QR_HIDDEN void qr_clear_error();
// Records a printf-style message for qr_last_error() and returns `code`.
QR_HIDDEN int qr_fail(int code, const char* fmt, ...);
// QR_OK, or QR_EDEVICE with the HIP error string after a launch.
QR_HIDDEN int qr_check_launch(const char* what);

inline bool qr_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The weight-row types (everything but the Q8_K_128 activation format).
inline bool qr_is_weight_type(int t) { return (t >= 0 && t <= 4) || t == 6 || t == 9 || t == 10; }
