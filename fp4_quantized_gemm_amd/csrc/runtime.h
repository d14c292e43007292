// Host-side plumbing shared by the C-ABI entry points: status codes,
// per-thread error messages, argument checks and small fill kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "nvfp4rac.h"

namespace nvfp4 {

// Record a message for nvfp4_last_error() and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message; return NVFP4_OK.
int ok();
// Turn a pending launch error into NVFP4_ERR_HIP (with the kernel's name).
int check_launch(const char* what);

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Device fills (a kernel rather than hipMemsetAsync, so the calls can be
// recorded into a HIP graph safely).
void fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
void fill_u64(uint64_t* p, int64_t n, uint64_t v, hipStream_t s);

// Number of compute units of the current device (cached per device).
int num_cus();

}  // namespace nvfp4

#define NV_REQUIRE(cond, status, ...)                                  \
  do {                                                                 \
    if (!(cond)) return ::nvfp4::fail((status), __VA_ARGS__);          \
  } while (0)
