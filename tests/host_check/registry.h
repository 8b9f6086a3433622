// Test-only registry of host buffers that stand in for device buffers in the
// host-only sanitizer build of the C-ABI layer (tests/host_check): every
// recorded kernel launch checks that each byte range its kernel would touch
// lies inside one registered buffer.
#pragma once

#include <stddef.h>
#include <stdint.h>

// A zero-filled, 256-byte aligned buffer of `bytes` bytes, registered.
void* hc_alloc(size_t bytes);
// Frees every registered buffer.
void hc_free_all();
// Aborts the program (with `what` in the message) unless [p, p + bytes) lies
// inside one registered buffer; bytes == 0 passes.
void hc_need(const void* p, size_t bytes, const char* what);
// Aborts with `what` when cond is false (a kernel precondition).
void hc_expect(bool cond, const char* what);
// Launches recorded since the last reset, and the reset.
int hc_launches();
void hc_reset_launches();
void hc_count_launch();
