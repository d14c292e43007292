// High-residual channel selection for Residual Activation Compensation
// (QUADS, gist.science technical summary §2.2 B: a binary mask picks the
// channels of largest residual magnitude; their residual is added back).
//
//   1. k_select_topk (one workgroup): an MSB-first radix select of the k-th
//      largest score over all K channels, then the channels above it and the
//      lowest-index ties, compacted in index order, which writes S ascending.
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

constexpr int kSelectMaxK = 16384;
constexpr int kSelectThreads = 1024;

__device__ __forceinline__ uint64_t wave_or_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o), hi = __shfl_xor((uint32_t)(v >> 32), o);
    v |= ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// Exclusive prefix sum of one int per thread over the workgroup (in thread
// order); wsum holds kSelectThreads / 64 ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
  const int tid = threadIdx.x;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int w = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += w;
  }
  __syncthreads();
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
  return base + incl - v;
}

// Top-k of up to 1024 * CPT (score desc, index asc) keys by one workgroup
// (one score vector per workgroup: several for the per-expert selection).
// Thread t holds channels CPT t .. CPT t + CPT - 1.  An MSB-first radix select finds the
// k-th largest score T one byte at a time (a 256-bin LDS histogram of the
// remaining candidates, then one wave scans the bins from the top); the
// channels above T are taken, and of the channels equal to T the ones of
// lowest index, as many as k still needs.  The selected channels are then
// written in index order, so S is ascending.
template <int CPT>
__global__ void __launch_bounds__(kSelectThreads)
k_select_topk(const uint64_t* __restrict__ score, int K, int k, int32_t* __restrict__ S) {
  score += (int64_t)blockIdx.x * K;
  S += (int64_t)blockIdx.x * k;
  __shared__ uint32_t hist[2][256];                    // passes alternate buffers
  __shared__ uint64_t orw[kSelectThreads / 64];
  __shared__ int wsum[kSelectThreads / 64];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need, s_exact;
  const int tid = threadIdx.x;
  uint64_t key[CPT];
  bool valid[CPT];
  uint64_t any = 0;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int e = CPT * tid + q;
    valid[q] = e < K;
    key[q] = valid[q] ? score[e] : 0ull;
    any |= key[q];
  }
  if (tid < 512) hist[tid >> 8][tid & 255] = 0u;
  // the highest byte any key uses
  uint64_t orv = wave_or_u64(any);
  if ((tid & 63) == 0) orw[tid >> 6] = orv;
  __syncthreads();
  orv = 0;
  for (int w = 0; w < kSelectThreads / 64; ++w) orv |= orw[w];
  const int top = orv == 0 ? 0 : (63 - __builtin_clzll(orv)) >> 3;

  // Per pass (byte b, from the top): histogram the remaining candidates'
  // byte b, then one wave finds the bin holding the need-th largest.  If
  // that bin holds exactly the keys still needed, every key whose bytes
  // from the top down to b are at least the prefix is selected, and the
  // lower bytes need no pass.  Two barriers per pass: the next pass's
  // histogram buffer is cleared while this one is scanned.
  uint64_t prefix = 0, mask = 0;
  int need = k, exact = 0;
  for (int b = top, i = 0; b >= 0; --b, ++i) {
    uint32_t* h = hist[i & 1];
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      if (valid[q] && (key[q] & mask) == prefix) atomicAdd(&h[(key[q] >> (8 * b)) & 0xFFu], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255 - 4l .. 252 - 4l (descending)
      int cnt[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) sum += (cnt[j] = (int)h[255 - 4 * tid - j]);
      int incl = sum;
      for (int o = 1; o < 64; o <<= 1) {
        const int w = __shfl_up(incl, o);
        if (tid >= o) incl += w;
      }
      int c = incl - sum;                      // keys in higher bins
      if (c < need && need <= incl) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (c + cnt[j] >= need) {
            s_prefix = prefix | ((uint64_t)(255 - 4 * tid - j) << (8 * b));
            s_need = need - c;
            s_exact = c + cnt[j] == need ? 1 : 0;
            break;
          }
          c += cnt[j];
        }
      }
    } else if (tid >= 256 && tid < 512) {
      hist[(i + 1) & 1][tid - 256] = 0u;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    exact = s_exact;
    mask |= 0xFFull << (8 * b);
    if (exact) break;
  }
  // exact: the selection is every key whose masked bytes are >= prefix.
  // Otherwise prefix is the k-th largest score T: take everything above it
  // and the first `need` channels equal to it.
  int ties = 0;
  if (!exact) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) ties += (valid[q] && key[q] == prefix) ? 1 : 0;
  }
  int tie_rank = block_exclusive_scan(ties, wsum);
  bool sel[CPT];
  int nsel = 0;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    sel[q] = false;
    if (exact) {
      sel[q] = valid[q] && (key[q] & mask) >= prefix;
    } else {
      if (valid[q] && key[q] > prefix) sel[q] = true;
      if (valid[q] && key[q] == prefix) sel[q] = tie_rank++ < need;
    }
    nsel += sel[q] ? 1 : 0;
  }
  int pos = block_exclusive_scan(nsel, wsum);
#pragma unroll
  for (int q = 0; q < CPT; ++q)
    if (sel[q]) S[pos++] = CPT * tid + q;
}

// one workgroup per score vector (grid = number of vectors)
static void launch_select_topk(const uint64_t* score, int64_t K, int64_t k, int32_t* S,
                               unsigned vectors, hipStream_t s) {
  if (K <= 4 * kSelectThreads)
    k_select_topk<4><<<vectors, kSelectThreads, 0, s>>>(score, (int)K, (int)k, S);
  else if (K <= 8 * kSelectThreads)
    k_select_topk<8><<<vectors, kSelectThreads, 0, s>>>(score, (int)K, (int)k, S);
  else
    k_select_topk<16><<<vectors, kSelectThreads, 0, s>>>(score, (int)K, (int)k, S);
}

// R[m][j] = bf16(fma(-(q*s), g, x[m][S[j]])): a block owns `rpb` rows (at
// most 64); its 256 threads take the (row, channel) pairs of those rows in
// order, eight pairs in flight per thread (the gathers of one pair are three
// dependent-free loads, so they overlap across pairs).
constexpr int kGatherRows = 64;
constexpr int kGatherInFlight = 8;

__global__ void __launch_bounds__(256)
k_gather_residual(const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ codes,
                  const uint8_t* __restrict__ scales, const float* __restrict__ g_x,
                  const int32_t* __restrict__ S, int64_t M, int64_t K, int k, int rpb,
                  uint16_t* __restrict__ R) {
  const float g = *g_x;
  const int64_t m0 = (int64_t)blockIdx.x * rpb;
  const int64_t rows = M - m0 < rpb ? M - m0 : rpb;
  const int64_t n = rows * k;
  for (int64_t q0 = 0; q0 < n; q0 += 256 * kGatherInFlight) {
    uint32_t cb[kGatherInFlight], sb[kGatherInFlight], xb[kGatherInFlight];
    int sh[kGatherInFlight];
#pragma unroll
    for (int u = 0; u < kGatherInFlight; ++u) {
      const int64_t q = q0 + u * 256 + threadIdx.x;
      if (q < n) {
        const int64_t m = m0 + q / k;
        const int j = (int)(q % k);
        const int c = S[j];
        cb[u] = codes[m * (K / 2) + (c >> 1)];
        sb[u] = scales[m * (K / 16) + (c >> 4)];
        // (streaming hint: the last read of x in a forward; the codes and
        // scales are read again to build the GEMM's operand image)
        xb[u] = __builtin_nontemporal_load(x + m * ldx + c);
        sh[u] = 4 * (c & 1);
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherInFlight; ++u) {
      const int64_t q = q0 + u * 256 + threadIdx.x;
      if (q < n) {
        const float qv = e2m1_unpack2<0>((cb[u] >> sh[u]) & 0xFu).x;
        const float sv = e4m3_decode(sb[u]);
        R[m0 * k + q] = (uint16_t)f32_to_bf16_rne(
            __builtin_fmaf(-(qv * sv), g, bf16_bits_to_f32(xb[u])));
      }
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
// expert e (t = a_rows[p]).  Thread b owns channels 16 b .. 16 b + 15 of the
// workgroup's 4096-channel slice (blockIdx.y); a workgroup walks 64
// consecutive permuted rows, which belong to one
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
  const int b = (int)blockIdx.y * 256 + threadIdx.x;
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
// e, t = a_rows[p]: 64 permuted rows per workgroup, their (row, channel)
// pairs over the threads with eight in flight per thread, as in
// k_gather_residual.
__global__ void __launch_bounds__(256)
k_gather_residual_rows(const uint16_t* __restrict__ x, int64_t ldx,
                       const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       const float* __restrict__ g_x, const int32_t* __restrict__ a_rows,
                       const int32_t* __restrict__ offsets, int E, int64_t M_src, int64_t M_total,
                       int64_t K, int k, int rpb, const int32_t* __restrict__ S,
                       uint16_t* __restrict__ R) {
  const float g = *g_x;
  const int64_t p_lo = (int64_t)blockIdx.x * rpb;
  const int64_t rows = M_total - p_lo < rpb ? M_total - p_lo : rpb;
  const int64_t n = rows * k;
  for (int64_t q0 = 0; q0 < n; q0 += 256 * kGatherInFlight) {
    uint32_t cb[kGatherInFlight], sb[kGatherInFlight], xb[kGatherInFlight];
    int sh[kGatherInFlight];
#pragma unroll
    for (int u = 0; u < kGatherInFlight; ++u) {
      const int64_t q = q0 + u * 256 + threadIdx.x;
      if (q < n) {
        const int64_t p = p_lo + q / k;
        const int j = (int)(q % k);
        const int e = expert_of(offsets, E, p);
        int64_t t = a_rows ? (int64_t)a_rows[p] : p;
        t = t < 0 ? 0 : (t >= M_src ? M_src - 1 : t);
        int c = S[(int64_t)e * k + j];
        c = c < 0 ? 0 : (c >= K ? (int)K - 1 : c);
        cb[u] = codes[t * (K / 2) + (c >> 1)];
        sb[u] = scales[t * (K / 16) + (c >> 4)];
        xb[u] = x[t * ldx + c];
        sh[u] = 4 * (c & 1);
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherInFlight; ++u) {
      const int64_t q = q0 + u * 256 + threadIdx.x;
      if (q < n) {
        const float qv = e2m1_unpack2<0>((cb[u] >> sh[u]) & 0xFu).x;
        const float sv = e4m3_decode(sb[u]);
        R[p_lo * k + q] = (uint16_t)f32_to_bf16_rne(
            __builtin_fmaf(-(qv * sv), g, bf16_bits_to_f32(xb[u])));
      }
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
  launch_select_topk(score, K, k, S, 1, s);
  if (M > 0) {
    // rows per block: 64, halved while that leaves fewer than two blocks
    // per CU and a block still has more than one pair per thread (few rows:
    // the gather is then latency-bound, and more blocks overlap it)
    int rpb = kGatherRows;
    while (rpb > 1 && (M + rpb - 1) / rpb < 2LL * num_cus() && (int64_t)rpb * k > 256) rpb /= 2;
    const int64_t blocks = (M + rpb - 1) / rpb;
    k_gather_residual<<<(unsigned)blocks, 256, 0, s>>>(
        static_cast<const uint16_t*>(x_used), ldx, codes, scales, g_x, S, M, K, (int)k, rpb,
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
    k_expert_scores<<<dim3((unsigned)blocks, (unsigned)((K + 4095) / 4096)), 256, 0, s>>>(
        static_cast<const uint16_t*>(x_used), ldx, codes, scales, g_x, a_rows, expert_offsets,
        (int)E, M_src, M_total, K, score);
  launch_select_topk(score, K, k, S, (unsigned)E, s);
  if (M_total > 0) {
    // rows per block as in select_residual_channels
    int rpb = kExpertRows;
    while (rpb > 1 && (M_total + rpb - 1) / rpb < 2LL * num_cus() && (int64_t)rpb * k > 256)
      rpb /= 2;
    k_gather_residual_rows<<<(unsigned)((M_total + rpb - 1) / rpb), 256, 0, s>>>(
        static_cast<const uint16_t*>(x_used), ldx, codes, scales, g_x, a_rows, expert_offsets,
        (int)E, M_src, M_total, K, (int)k, rpb, S, static_cast<uint16_t*>(R));
  }
  return check_launch("select_residual_channels_per_expert");
}

}  // extern "C"
