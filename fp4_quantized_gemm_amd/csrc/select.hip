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

// One compare-exchange decision: element e with partner value (ps, pi) in a
// bitonic stage of block `size`; returns true if e should take the partner.
__device__ __forceinline__ bool take_partner(int e, int partner, int size, uint64_t s, uint32_t i,
                                             uint64_t ps, uint32_t pi) {
  const bool first = ((e & size) == 0) == (e < partner);  // e should hold the earlier key
  return first ? key_before(ps, pi, s, i) : key_before(s, i, ps, pi);
}

// Bitonic sort of up to 4096 (score desc, index asc) keys by one workgroup.
// Thread t holds elements 4t .. 4t+3 in registers.  Strides 1 and 2 stay in
// the thread, strides 4 .. 128 cross lanes of one wave (shuffles), larger
// strides go through LDS with a barrier.  The first k sorted keys are flagged
// and compacted in index order, which writes S ascending.
__global__ void __launch_bounds__(kSelectThreads)
k_select_topk(const uint64_t* __restrict__ score, int K, int Kpad, int k, int32_t* __restrict__ S) {
  __shared__ uint64_t xs[kSelectMaxK];
  __shared__ uint16_t xi[kSelectMaxK];
  __shared__ uint8_t flag[kSelectMaxK];
  __shared__ int wsum[kSelectThreads / 64];
  const int tid = threadIdx.x;
  uint64_t ks[4];
  uint32_t ki[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * tid + q;
    ks[q] = e < K ? score[e] : 0ull;
    ki[q] = e < K ? (uint32_t)e : 0xFFFFu;
  }
  for (int i = tid; i < kSelectMaxK; i += kSelectThreads) flag[i] = 0;
  const int nt = Kpad / 4;                          // active threads
  for (int size = 2; size <= Kpad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 256) {
        __syncthreads();
        if (tid < nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) { xs[4 * tid + q] = ks[q]; xi[4 * tid + q] = (uint16_t)ki[q]; }
        __syncthreads();
        if (tid < nt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int e = 4 * tid + q, pe = e ^ stride;
            const uint64_t ps = xs[pe];
            const uint32_t pi = xi[pe];
            if (take_partner(e, pe, size, ks[q], ki[q], ps, pi)) { ks[q] = ps; ki[q] = pi; }
          }
      } else if (stride >= 4) {
        const int lanes = stride >> 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = __shfl_xor((uint32_t)ks[q], lanes);
          const uint32_t hi = __shfl_xor((uint32_t)(ks[q] >> 32), lanes);
          const uint32_t pi = __shfl_xor(ki[q], lanes);
          const uint64_t ps = ((uint64_t)hi << 32) | lo;
          const int e = 4 * tid + q, pe = e ^ stride;
          if (tid < nt && take_partner(e, pe, size, ks[q], ki[q], ps, pi)) { ks[q] = ps; ki[q] = pi; }
        }
      } else {
        // stride 2 or 1: both elements of each pair are in this thread
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int pq = q ^ stride;
          if (pq < q) continue;
          const int e = 4 * tid + q, pe = 4 * tid + pq;
          if (take_partner(e, pe, size, ks[q], ki[q], ks[pq], ki[pq])) {
            const uint64_t ts = ks[q]; const uint32_t ti = ki[q];
            ks[q] = ks[pq]; ki[q] = ki[pq];
            ks[pq] = ts; ki[pq] = ti;
          }
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (4 * tid + q < k) flag[ki[q]] = 1;
  __syncthreads();
  // ordered compaction: each thread owns a contiguous run of channels
  const int per = (Kpad + kSelectThreads - 1) / kSelectThreads;
  const int lo = tid * per;
  int cnt = 0;
  for (int i = lo; i < lo + per && i < K; ++i) cnt += flag[i];
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

// R[m][j] = bf16(fma(-(q*s), g, x[m][S[j]])): a block owns 64 rows; each
// thread walks channels j = tid, tid + 256, ... of each row.
constexpr int kGatherRows = 64;

__global__ void __launch_bounds__(256)
k_gather_residual(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ codes,
                  const uint8_t* __restrict__ scales, const float* __restrict__ g_x,
                  const int32_t* __restrict__ S, int64_t M, int64_t K, int k,
                  uint16_t* __restrict__ R) {
  const float g = *g_x;
  const int64_t m0 = (int64_t)blockIdx.x * kGatherRows;
  for (int j = threadIdx.x; j < k; j += 256) {
    const int c = S[j];
    const int64_t cb = c >> 1, cs = c >> 4;
    const int sh = 4 * (c & 1);
    for (int64_t m = m0; m < m0 + kGatherRows && m < M; ++m) {
      const uint32_t code = (codes[m * (K / 2) + cb] >> sh) & 0xFu;
      const float q = e2m1_unpack2<0>(code).x;
      const float s = e4m3_decode(scales[m * (K / 16) + cs]);
      const float xv = bf16_bits_to_f32(x[m * ldx + c]);
      R[m * k + j] = (uint16_t)f32_to_bf16_rne(__builtin_fmaf(-(q * s), g, xv));
    }
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
  int Kpad = 4;
  while (Kpad < K) Kpad <<= 1;
  k_select_topk<<<1, kSelectThreads, 0, s>>>(score, (int)K, Kpad, (int)k, S);
  if (M > 0) {
    const int64_t blocks = (M + kGatherRows - 1) / kGatherRows;
    k_gather_residual<<<(unsigned)blocks, 256, 0, s>>>(
        static_cast<const uint16_t*>(x_used), ldx, codes, scales, g_x, S, M, K, (int)k,
        static_cast<uint16_t*>(R_S));
  }
  return check_launch("select_residual_channels");
}

}  // extern "C"
