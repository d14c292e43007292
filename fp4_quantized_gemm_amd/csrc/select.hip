// High-residual channel selection for Residual Activation Compensation
// (QUADS, gist.science technical summary §2.2 B: a binary mask picks the
// channels of largest residual magnitude; their residual is added back).
//
//   1. k_select_topk (one workgroup): bitonic sort of (score desc, index asc)
//      over all K channels in LDS; flag the first k; compact the flags in
//      index order, which writes S ascending.
//   2. k_gather_residual: R_S[m][j] = bf16(fma(-(q*s), g, x[m][S[j]])), the
//      same rounding as the residual behind the scores.
#include "device.h"
#include "runtime.h"

namespace nvfp4 {

constexpr int kSelectMaxK = 4096;
constexpr int kSelectThreads = 1024;

__device__ __forceinline__ bool key_before(uint64_t sa, uint32_t ia, uint64_t sb, uint32_t ib) {
  return sa > sb || (sa == sb && ia < ib);
}

__global__ void __launch_bounds__(kSelectThreads)
k_select_topk(const uint64_t* __restrict__ score, int K, int Kpad, int k, int32_t* __restrict__ S) {
  __shared__ uint64_t key[kSelectMaxK];
  __shared__ uint16_t idx[kSelectMaxK];
  __shared__ uint8_t flag[kSelectMaxK];
  __shared__ int wsum[kSelectThreads / 64];
  const int tid = threadIdx.x;
  for (int i = tid; i < Kpad; i += kSelectThreads) {
    key[i] = i < K ? score[i] : 0ull;
    idx[i] = (uint16_t)(i < K ? i : 0xFFFF);
    flag[i] = 0;
  }
  __syncthreads();
  for (int size = 2; size <= Kpad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < Kpad; i += kSelectThreads) {
        int j = i ^ stride;
        if (j > i) {
          uint64_t si = key[i], sj = key[j];
          uint32_t ii = idx[i], ij = idx[j];
          bool want_i_first = (i & size) == 0;
          bool swap = want_i_first ? key_before(sj, ij, si, ii) : key_before(si, ii, sj, ij);
          if (swap) {
            key[i] = sj; key[j] = si;
            idx[i] = (uint16_t)ij; idx[j] = (uint16_t)ii;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < k; i += kSelectThreads) flag[idx[i]] = 1;
  __syncthreads();
  // ordered compaction: each thread owns a contiguous run of channels
  const int per = (Kpad + kSelectThreads - 1) / kSelectThreads;
  const int lo = tid * per;
  int cnt = 0;
  for (int i = lo; i < lo + per && i < K; ++i) cnt += flag[i];
  // exclusive scan of cnt over the workgroup
  int incl = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += v;
  }
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
  int pos = base + incl - cnt;
  for (int i = lo; i < lo + per && i < K; ++i)
    if (flag[i]) S[pos++] = i;
}

__global__ void __launch_bounds__(256)
k_gather_residual(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ codes,
                  const uint8_t* __restrict__ scales, const float* __restrict__ g_x,
                  const int32_t* __restrict__ S, int64_t M, int64_t K, int k,
                  uint16_t* __restrict__ R) {
  const float g = *g_x;
  const int64_t total = M * (int64_t)k;
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t m = e / k;
    const int j = S[e - m * k];
    const uint32_t byte = codes[m * (K / 2) + (j >> 1)];
    const uint32_t code = (byte >> (4 * (j & 1))) & 0xFu;
    const float q = e2m1_unpack2<0>(code).x;
    const float s = e4m3_decode(scales[m * (K / 16) + (j >> 4)]);
    const float xv = bf16_bits_to_f32(x[m * ldx + j]);
    R[e] = (uint16_t)f32_to_bf16_rne(__builtin_fmaf(-(q * s), g, xv));
  }
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t select_residual_channels_workspace_size(int64_t M, int64_t K, int64_t k) {
  (void)M;
  (void)K;
  (void)k;
  return 0;
}

int select_residual_channels(const void* x_used, int64_t ldx, const uint8_t* codes,
                             const uint8_t* scales, const float* g_x, const uint64_t* score,
                             int64_t M, int64_t K, int64_t k, int32_t* S, void* R_S, void* ws,
                             size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  NV_REQUIRE(M >= 0 && K >= 32 && K % 32 == 0 && K <= kSelectMaxK && k >= 0 && k <= K,
             NVFP4_ERR_SHAPE,
             "select_residual_channels: need 0 <= k <= K <= %d, K %% 32 == 0 (K=%lld k=%lld)",
             kSelectMaxK, (long long)K, (long long)k);
  if (k == 0) return ok();
  NV_REQUIRE(score && S && g_x && (M == 0 || (x_used && codes && scales && R_S)), NVFP4_ERR_NULL,
             "select_residual_channels: missing pointer");
  NV_REQUIRE(ldx >= K, NVFP4_ERR_SHAPE, "select_residual_channels: ldx < K");
  NV_REQUIRE(aligned(score, 8) && aligned(S, 4) && aligned(R_S, 2) && aligned(x_used, 2),
             NVFP4_ERR_ALIGN, "select_residual_channels: misaligned pointer");
  hipStream_t s = as_stream(stream);
  int Kpad = 1;
  while (Kpad < K) Kpad <<= 1;
  k_select_topk<<<1, kSelectThreads, 0, s>>>(score, (int)K, Kpad, (int)k, S);
  if (M > 0) {
    int64_t total = M * k;
    int64_t blocks = (total + 255) / 256;
    int64_t cap = 16LL * num_cus();
    k_gather_residual<<<(unsigned)(blocks < cap ? blocks : cap), 256, 0, s>>>(
        static_cast<const uint16_t*>(x_used), ldx, codes, scales, g_x, S, M, K, (int)k,
        static_cast<uint16_t*>(R_S));
  }
  return check_launch("select_residual_channels");
}

}  // extern "C"
