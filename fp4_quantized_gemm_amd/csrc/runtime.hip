// C-ABI utilities: version, status strings, per-thread error text, fills.
#include "runtime.h"

#include <cstdarg>
#include <cstdio>
#include <mutex>

namespace nvfp4 {

static thread_local char g_msg[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_msg[0] = '\0';
  return NVFP4_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_fill_u64(uint64_t* p, int64_t n, uint64_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

void fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return;
  int64_t b = (n + 255) / 256;
  k_fill_u32<<<(unsigned)(b < 1024 ? b : 1024), 256, 0, s>>>(p, n, v);
}

void fill_u64(uint64_t* p, int64_t n, uint64_t v, hipStream_t s) {
  if (n <= 0) return;
  int64_t b = (n + 255) / 256;
  k_fill_u64<<<(unsigned)(b < 1024 ? b : 1024), 256, 0, s>>>(p, n, v);
}

int num_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace nvfp4

extern "C" {

int nvfp4_version(void) { return 100; }

const char* nvfp4_status_str(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP";
    default: return "NVFP4_ERR_UNKNOWN";
  }
}

const char* nvfp4_last_error(void) { return nvfp4::g_msg; }

}  // extern "C"
