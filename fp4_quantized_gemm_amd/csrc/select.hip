// High-residual channel selection for Residual Activation Compensation
// (QUADS, gist.science technical summary §2.2 B: a binary mask picks the
// channels of largest residual magnitude; their residual is added back).
//
//   1. k_select_topk (one workgroup): bitonic sort of (score desc, index asc)
//      over all K channels in LDS; flag the first k; compact the flags in
//      index order, which writes S ascending.
//   2. k_gather_residual: R_S[m][j] = bf16(fma(-(q*s), g, x[m][S[j]])), the
//      same rounding as the residual behind the scores.
//
// Per-expert variant (each expert ranks the channels by the residual of its
// own rows): k_expert_scores sums the same fixed-point statistic per expert
// over its permuted rows, k_select_topk runs once per expert, and
// k_gather_residual_rows gathers R per permuted row from its expert's S.
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
  // one score vector per workgroup (several for the per-expert selection)
  score += (int64_t)blockIdx.x * K;
  S += (int64_t)blockIdx.x * k;
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

// Largest e with offsets[e] <= p (offsets non-decreasing, offsets[0] = 0).
__device__ __forceinline__ int expert_of(const int32_t* __restrict__ offsets, int E, int64_t p) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

constexpr int kExpertRows = 64;      // permuted rows per workgroup

// score[e][j] += floor(|r[t][j]| * 2^(31 - E_A)) over the permuted rows p of
// expert e (t = a_rows[p]).  Thread b owns channels 16 b .. 16 b + 15 (K <=
// 4096); a workgroup walks 64 consecutive permuted rows, which belong to one
// expert or a few, and adds its integer sums per expert with 64-bit atomics
// (any order gives the same bits).  The residual is the quantizer's: r =
// bf16(fma(-(q * s), g, x)).  A, whose binary exponent scales the terms, is
// the bf16 value nearest g * 2688 (g = fp32(A / 2688) is within 2^-23 of
// A / 2688 and A is a bf16 value, so the rounding recovers it exactly).
__global__ void __launch_bounds__(256)
k_expert_scores(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ codes,
                const uint8_t* __restrict__ scales, const float* __restrict__ g_x,
                const int32_t* __restrict__ a_rows, const int32_t* __restrict__ offsets, int E,
                int64_t M_src, int64_t M_total, int64_t K, uint64_t* __restrict__ score) {
  const float g = *g_x;
  if (!(g > 0.0f)) return;                     // A == 0: every score is 0
  const float A = bf16_bits_to_f32(f32_to_bf16_rne(g * kScaleDen));
  const int ea = frexp_exponent(A);
  const int b = threadIdx.x;
  const bool active = b < K / 16;
  const int64_t p_lo = (int64_t)blockIdx.x * kExpertRows;
  const int64_t p_hi = p_lo + kExpertRows < M_total ? p_lo + kExpertRows : M_total;
  int e = expert_of(offsets, E, p_lo);
  uint64_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0;
  auto flush = [&](int ex) {
    if (!active) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (acc[i]) atomicAdd(reinterpret_cast<unsigned long long*>(score + (int64_t)ex * K + 16 * b + i),
                            (unsigned long long)acc[i]);
      acc[i] = 0;
    }
  };
  for (int64_t p = p_lo; p < p_hi; ++p) {
    while (e + 1 < E && offsets[e + 1] <= p) {   // uniform over the workgroup
      flush(e);
      ++e;
    }
    if (!active) continue;
    int64_t t = a_rows ? (int64_t)a_rows[p] : p;
    t = t < 0 ? 0 : (t >= M_src ? M_src - 1 : t);
    const uint16_t* xr = x + t * ldx + 16 * b;
    const uint4 v0 = *reinterpret_cast<const uint4*>(xr);
    const uint4 v1 = *reinterpret_cast<const uint4*>(xr + 8);
    const uint2 cw = *reinterpret_cast<const uint2*>(codes + t * (K / 2) + 8 * b);
    const float sv = e4m3_decode(scales[t * (K / 16) + b]);
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x2 q = e2m1_unpack2<0>(((i < 4 ? cw.x : cw.y) >> (8 * (i & 3))) & 0xFFu);
      const float r0 = __builtin_fmaf(-(q.x * sv), g, bf16_bits_to_f32(w[i] & 0xFFFFu));
      const float r1 = __builtin_fmaf(-(q.y * sv), g, bf16_bits_to_f32(w[i] >> 16));
      const float b0 = bf16_bits_to_f32(f32_to_bf16_rne(r0));
      const float b1 = bf16_bits_to_f32(f32_to_bf16_rne(r1));
      acc[2 * i] += (uint64_t)(uint32_t)__builtin_ldexpf(__builtin_fabsf(b0), 31 - ea);
      acc[2 * i + 1] += (uint64_t)(uint32_t)__builtin_ldexpf(__builtin_fabsf(b1), 31 - ea);
    }
  }
  flush(e);
}

// R[p][j] = bf16(fma(-(q*s), g, x[t][S_e[j]])) for permuted row p of expert
// e, t = a_rows[p]: 64 permuted rows per workgroup, channels j over threads.
__global__ void __launch_bounds__(256)
k_gather_residual_rows(const uint16_t* __restrict__ x, int64_t ldx,
                       const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       const float* __restrict__ g_x, const int32_t* __restrict__ a_rows,
                       const int32_t* __restrict__ offsets, int E, int64_t M_src, int64_t M_total,
                       int64_t K, int k, const int32_t* __restrict__ S, uint16_t* __restrict__ R) {
  const float g = *g_x;
  const int64_t p_lo = (int64_t)blockIdx.x * kExpertRows;
  const int64_t p_hi = p_lo + kExpertRows < M_total ? p_lo + kExpertRows : M_total;
  int e = expert_of(offsets, E, p_lo);
  for (int64_t p = p_lo; p < p_hi; ++p) {
    while (e + 1 < E && offsets[e + 1] <= p) ++e;
    int64_t t = a_rows ? (int64_t)a_rows[p] : p;
    t = t < 0 ? 0 : (t >= M_src ? M_src - 1 : t);
    for (int j = threadIdx.x; j < k; j += 256) {
      int c = S[(int64_t)e * k + j];
      c = c < 0 ? 0 : (c >= K ? (int)K - 1 : c);
      const uint32_t code = (codes[t * (K / 2) + (c >> 1)] >> (4 * (c & 1))) & 0xFu;
      const float q = e2m1_unpack2<0>(code).x;
      const float sv = e4m3_decode(scales[t * (K / 16) + (c >> 4)]);
      const float xv = bf16_bits_to_f32(x[t * ldx + c]);
      R[p * k + j] = (uint16_t)f32_to_bf16_rne(__builtin_fmaf(-(q * sv), g, xv));
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

size_t select_residual_channels_per_expert_workspace_size(int64_t E, int64_t K) {
  if (E < 1 || K < 1) return 256;
  return round_up((size_t)E * (size_t)K * sizeof(uint64_t), 256);
}

int select_residual_channels_per_expert(const void* x_used, int64_t ldx, const uint8_t* codes,
                                        const uint8_t* scales, const float* g_x,
                                        const int32_t* a_rows, const int32_t* expert_offsets,
                                        int64_t E, int64_t M_src, int64_t M_total, int64_t K,
                                        int64_t k, int32_t* S, void* R, void* ws, size_t ws_bytes,
                                        void* stream) {
  NV_REQUIRE(E >= 1 && E <= 1024 && M_src >= 0 && M_total >= 0 && K >= 32 && K % 32 == 0 &&
                 K <= kSelectMaxK && k >= 0 && k <= K,
             NVFP4_ERR_SHAPE,
             "select_residual_channels_per_expert: need 1 <= E <= 1024, 0 <= k <= K <= %d, "
             "K %% 32 == 0 (E=%lld K=%lld k=%lld)",
             kSelectMaxK, (long long)E, (long long)K, (long long)k);
  if (k == 0) return ok();
  NV_REQUIRE(a_rows != nullptr || M_src >= M_total, NVFP4_ERR_SHAPE,
             "select_residual_channels_per_expert: without a_rows, M_src must be >= M_total");
  NV_REQUIRE(M_total == 0 || M_src >= 1, NVFP4_ERR_SHAPE,
             "select_residual_channels_per_expert: M_src == 0");
  NV_REQUIRE(S && g_x && expert_offsets && ws &&
                 (M_total == 0 || (x_used && codes && scales && R)),
             NVFP4_ERR_NULL, "select_residual_channels_per_expert: missing pointer");
  NV_REQUIRE(ldx >= K && ldx % 8 == 0, NVFP4_ERR_SHAPE,
             "select_residual_channels_per_expert: need ldx >= K, ldx %% 8 == 0");
  NV_REQUIRE(aligned(x_used, 16) && aligned(codes, 8) && aligned(S, 4) && aligned(R, 2) &&
                 aligned(ws, 8),
             NVFP4_ERR_ALIGN, "select_residual_channels_per_expert: misaligned pointer");
  NV_REQUIRE(ws_bytes >= select_residual_channels_per_expert_workspace_size(E, K),
             NVFP4_ERR_WORKSPACE, "select_residual_channels_per_expert: workspace too small");
  hipStream_t s = as_stream(stream);
  uint64_t* score = static_cast<uint64_t*>(ws);
  fill_u64(score, E * K, 0ull, s);
  const int64_t blocks = (M_total + kExpertRows - 1) / kExpertRows;
  if (M_total > 0)
    k_expert_scores<<<(unsigned)blocks, 256, 0, s>>>(
        static_cast<const uint16_t*>(x_used), ldx, codes, scales, g_x, a_rows, expert_offsets,
        (int)E, M_src, M_total, K, score);
  int Kpad = 4;
  while (Kpad < K) Kpad <<= 1;
  k_select_topk<<<(unsigned)E, kSelectThreads, 0, s>>>(score, (int)K, Kpad, (int)k, S);
  if (M_total > 0)
    k_gather_residual_rows<<<(unsigned)blocks, 256, 0, s>>>(
        static_cast<const uint16_t*>(x_used), ldx, codes, scales, g_x, a_rows, expert_offsets,
        (int)E, M_src, M_total, K, (int)k, S, static_cast<uint16_t*>(R));
  return check_launch("select_residual_channels_per_expert");
}

}  // extern "C"
