// MoE routing, expert-major permutation and the weighted un-permute/combine
// around the grouped expert GEMM (the MoE model of the QUADS pages,
// gist.science technical summary §4; the router is not described there:
// top-k of logit + bias, ties to the lower expert, softmax over the chosen k).
//
// Permutation without host synchronisation or float atomics (a few tokens:
// steps 2-4 in one workgroup, k_permute_small):
//   1. k_route: one wave per token -> topk_ids, topk_w (softmax in float64).
//   2. k_route_masks: one wave per chunk of 64 tokens; per expert a 64-bit
//      mask of the chunk's tokens that chose it (LDS atomic OR), plus counts.
//   3. k_chunk_scan: one wave per expert, exclusive scan over chunks -> each
//      chunk's base inside the expert and the expert's total;
//      k_expert_offsets: exclusive scan of the totals -> expert_offsets.
//   4. k_scatter: row = offsets[e] + base[chunk][e] + popcount(mask below the
//      token), so tokens stay ascending inside an expert.
#include "device.h"
#include "runtime.h"

namespace nvfp4 {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 32;

// Routing of token t by one wave: the top-tk experts of logit + bias (ties
// to the lower expert) and their softmax weights.
// Each lane holds experts lane + 64 i, i < KPER (E <= 64 KPER).
template <int KPER>
__device__ __forceinline__ void route_token(const float* __restrict__ logits,
                                            const float* __restrict__ bias, int64_t t, int E,
                                            int tk, int32_t* __restrict__ ids,
                                            float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  constexpr int kPer = KPER;
  float v[kPer];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    int e = lane + 64 * i;
    float l = -INFINITY;
    if (e < E) {
      l = logits[t * E + e];
      if (bias) l = l + bias[e];
    }
    v[i] = l;
    if (e >= E) taken |= 1u << i;
  }
  // lane r keeps the r-th pick; the picks come out in descending order
  float my_v = -INFINITY;
  int my_e = 0;
  float top = 0.0f;
  for (int r = 0; r < tk; ++r) {
    // lane-local best among untaken (value desc, index asc)
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int e = lane + 64 * i;
      if (!(taken & (1u << i)) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o);
      int oe = __shfl_xor(be, o);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == r) { my_v = bv; my_e = be; }
    if (r == 0) top = bv;
  }
  // softmax over the picks in float64, one pick per lane
  const double z = lane < tk ? exp((double)my_v - (double)top) : 0.0;
  double sum = z;
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane < tk) {
    ids[t * tk + lane] = my_e;
    w[t * tk + lane] = (float)(z / sum);
  }
}

template <int KPER>
__global__ void __launch_bounds__(256)
k_route(const float* __restrict__ logits, const float* __restrict__ bias, int64_t T, int E,
        int tk, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int64_t t = blockIdx.x * 4LL + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<KPER>(logits, bias, t, E, tk, ids, w);
}

// masks [nchunks][E] uint64, counts [nchunks][E] int32
__global__ void __launch_bounds__(64)
k_route_masks(const int32_t* __restrict__ ids, int64_t T, int E, int tk,
              uint64_t* __restrict__ masks, int32_t* __restrict__ counts) {
  __shared__ unsigned long long m[kMaxExperts];
  const int lane = threadIdx.x;
  const int64_t c = blockIdx.x;
  for (int e = lane; e < E; e += 64) m[e] = 0ull;
  __syncthreads();
  const int64_t t = c * 64 + lane;
  if (t < T)
    for (int j = 0; j < tk; ++j) atomicOr(&m[ids[t * tk + j]], 1ull << lane);
  __syncthreads();
  for (int e = lane; e < E; e += 64) {
    masks[c * E + e] = m[e];
    counts[c * E + e] = __popcll(m[e]);
  }
}

// One wave per expert: base[c][e] = sum_{c' < c} counts[c'][e] (exclusive scan
// over chunks, lane-contiguous runs), totals[e] = the expert's row count.
__global__ void __launch_bounds__(256)
k_chunk_scan(int32_t* __restrict__ counts_to_base, int64_t nchunks, int E,
             int32_t* __restrict__ totals) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int64_t per = (nchunks + 63) / 64;
  const int64_t c0 = lane * per;
  int run = 0;
  for (int64_t c = c0; c < c0 + per && c < nchunks; ++c) run += counts_to_base[c * E + e];
  int incl = run;
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  int base = incl - run;
  for (int64_t c = c0; c < c0 + per && c < nchunks; ++c) {
    const int v = counts_to_base[c * E + e];
    counts_to_base[c * E + e] = base;
    base += v;
  }
  if (lane == 63) totals[e] = incl;
}

// One workgroup: expert_offsets = exclusive scan of totals (E <= 1024).
__global__ void __launch_bounds__(1024)
k_expert_offsets(const int32_t* __restrict__ totals, int E, int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int v = tid < E ? totals[tid] : 0;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += u;
  }
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
  if (tid < E) offsets[tid] = base + incl - v;
  if (tid == E - 1) offsets[E] = base + incl;
}

__global__ void __launch_bounds__(64)
k_scatter(const int32_t* __restrict__ ids, int64_t T, int E, int tk,
          const uint64_t* __restrict__ masks, const int32_t* __restrict__ base,
          const int32_t* __restrict__ offsets,
          int32_t* __restrict__ perm_token, int32_t* __restrict__ inv_perm) {
  const int lane = threadIdx.x;
  const int64_t c = blockIdx.x;
  const int64_t t = c * 64 + lane;
  if (t >= T) return;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int j = 0; j < tk; ++j) {
    const int e = ids[t * tk + j];
    const int p = offsets[e] + base[c * E + e] + __popcll(masks[c * E + e] & below);
    perm_token[p] = (int32_t)t;
    inv_perm[t * tk + j] = p;
  }
}

// Steps 2-4 in one workgroup for a few tokens (T <= 512, E <= 256), with
// barriers between them: the chunk masks and counts live in LDS, thread e
// scans expert e's chunks, the first E threads scan the totals, and thread t
// scatters token t.  Identical results, one launch after k_route.
constexpr int kSmallT = 512;
constexpr int kSmallE = 256;
__global__ void __launch_bounds__(1024)
k_permute_small(const int32_t* __restrict__ ids, int T, int E, int tk,
                int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
                int32_t* __restrict__ inv_perm) {
  __shared__ unsigned long long m[kSmallT / 64][kSmallE];
  __shared__ int base[kSmallT / 64][kSmallE];
  __shared__ int off[kSmallE];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int nchunks = (T + 63) / 64;
  for (int i = tid; i < nchunks * kSmallE; i += 1024) m[i / kSmallE][i % kSmallE] = 0ull;
  __syncthreads();
  if (tid < T)
    for (int j = 0; j < tk; ++j) atomicOr(&m[tid >> 6][ids[tid * tk + j]], 1ull << (tid & 63));
  __syncthreads();
  int total = 0;
  if (tid < E)
    for (int c = 0; c < nchunks; ++c) {
      base[c][tid] = total;
      total += __popcll(m[c][tid]);
    }
  // exclusive scan of the totals over the experts
  int incl = total;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += u;
  }
  if ((tid & 63) == 63) wsum[wave] = incl;
  __syncthreads();
  int wb = 0;
  for (int q = 0; q < wave; ++q) wb += wsum[q];
  if (tid < E) {
    off[tid] = wb + incl - total;
    offsets[tid] = wb + incl - total;
  }
  if (tid == E - 1) offsets[E] = wb + incl;
  __syncthreads();
  if (tid < T) {
    const int c = tid >> 6, lane = tid & 63;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    for (int j = 0; j < tk; ++j) {
      const int e = ids[tid * tk + j];
      const int p = off[e] + base[c][e] + __popcll(m[c][e] & below);
      perm_token[p] = tid;
      inv_perm[tid * tk + j] = p;
    }
  }
}

// out[t][n..n+8) = bf16(sum_j w[t][j] * y[inv_perm[t][j]][n..n+8)), float32
// in slot order.  One block per token; its routing is read once.
__global__ void __launch_bounds__(512)
k_combine(const uint16_t* __restrict__ y, const int32_t* __restrict__ inv_perm,
          const float* __restrict__ tw, int64_t T, int tk, int64_t N, uint16_t* __restrict__ out) {
  __shared__ int64_t rows[kMaxTopk];
  __shared__ float wts[kMaxTopk];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < tk) {
    rows[threadIdx.x] = inv_perm[t * tk + threadIdx.x];
    wts[threadIdx.x] = tw[t * tk + threadIdx.x];
  }
  __syncthreads();
  // acc += w_j * y_j in slot order j = 0 .. tk-1; the rows' loads are
  // issued eight at a time ahead of their multiply-adds, with the streaming
  // (nontemporal) hint: every expert output is read once (240 -> 207 us on
  // 16384 tokens x top-8 x 4096 bf16)
  auto load_nt = [](const uint16_t* src) {
    typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
    const u32x4n v = __builtin_nontemporal_load(reinterpret_cast<const u32x4n*>(src));
    return make_uint4(v.x, v.y, v.z, v.w);
  };
  auto fma8 = [](float* acc, float wj, const uint4& v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = __builtin_fmaf(wj, bf16_bits_to_f32(u[i] & 0xFFFFu), acc[2 * i]);
      acc[2 * i + 1] = __builtin_fmaf(wj, bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
    }
  };
  for (int64_t n = threadIdx.x * 8LL; n < N; n += (int64_t)blockDim.x * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int j0 = 0;
    for (; j0 + 8 <= tk; j0 += 8) {
      uint4 v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) v[jj] = load_nt(y + rows[j0 + jj] * N + n);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) fma8(acc, wts[j0 + jj], v[jj]);
    }
    for (int j = j0; j < tk; ++j) fma8(acc, wts[j], load_nt(y + rows[j] * N + n));
    uint4 o;
    o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + t * N + n) = o;
  }
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t moe_permute_workspace_size(int64_t T, int64_t E) {
  int64_t nchunks = (T + 63) / 64;
  if (nchunks < 1) nchunks = 1;
  return round_up((size_t)nchunks * (size_t)E * sizeof(uint64_t), 256) +
         round_up((size_t)(nchunks + 1) * (size_t)E * sizeof(int32_t), 256);
}

int moe_permute(const float* logits, const float* bias, int64_t T, int64_t E, int64_t tk,
                int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* perm_token,
                int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(T >= 0 && E >= 1 && E <= kMaxExperts && tk >= 1 && tk <= E && tk <= kMaxTopk &&
                 T * tk < (1LL << 31),
             NVFP4_ERR_SHAPE, "moe_permute: need T >= 0, 1 <= tk <= min(E, %d), E <= %d",
             kMaxTopk, kMaxExperts);
  NV_REQUIRE(expert_offsets && ws && (T == 0 || (logits && topk_ids && topk_w && perm_token &&
                                                 inv_perm)),
             NVFP4_ERR_NULL, "moe_permute: missing pointer");
  NV_REQUIRE(aligned(ws, 16) && aligned(logits, 4) && aligned(topk_ids, 4), NVFP4_ERR_ALIGN,
             "moe_permute: misaligned pointer");
  NV_REQUIRE(ws_bytes >= moe_permute_workspace_size(T, E), NVFP4_ERR_WORKSPACE,
             "moe_permute: workspace too small");
  hipStream_t s = as_stream(stream);
  int64_t nchunks = (T + 63) / 64;
  uint64_t* masks = static_cast<uint64_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(
      static_cast<char*>(ws) +
      round_up((size_t)(nchunks > 0 ? nchunks : 1) * (size_t)E * sizeof(uint64_t), 256));
  if (T == 0) {
    fill_u32(reinterpret_cast<uint32_t*>(expert_offsets), E + 1, 0u, s);
    return check_launch("moe_permute");
  }
  {
    // experts per lane: one or two for up to 128 experts (each pick scans
    // them; 16384 tokens x 128 experts: 48 -> 40 us), else sixteen (4 for
    // 256 experts measured no faster)
    const unsigned g = (unsigned)((T + 3) / 4);
    if (E <= 64)
      k_route<1><<<g, 256, 0, s>>>(logits, bias, T, (int)E, (int)tk, topk_ids, topk_w);
    else if (E <= 128)
      k_route<2><<<g, 256, 0, s>>>(logits, bias, T, (int)E, (int)tk, topk_ids, topk_w);
    else
      k_route<kMaxExperts / 64><<<g, 256, 0, s>>>(logits, bias, T, (int)E, (int)tk, topk_ids,
                                                  topk_w);
  }
  if (T <= kSmallT && E <= kSmallE) {
    k_permute_small<<<1, 1024, 0, s>>>(topk_ids, (int)T, (int)E, (int)tk, expert_offsets,
                                       perm_token, inv_perm);
    return check_launch("moe_permute");
  }
  int32_t* totals = counts + (size_t)nchunks * E;
  k_route_masks<<<(unsigned)nchunks, 64, 0, s>>>(topk_ids, T, (int)E, (int)tk, masks, counts);
  k_chunk_scan<<<(unsigned)((E + 3) / 4), 256, 0, s>>>(counts, nchunks, (int)E, totals);
  k_expert_offsets<<<1, 1024, 0, s>>>(totals, (int)E, expert_offsets);
  k_scatter<<<(unsigned)nchunks, 64, 0, s>>>(topk_ids, T, (int)E, (int)tk, masks, counts,
                                             expert_offsets, perm_token, inv_perm);
  return check_launch("moe_permute");
}

int moe_unpermute_combine(const void* y, const int32_t* inv_perm, const float* topk_w, int64_t T,
                          int64_t tk, int64_t N, void* out, void* stream) {
  NV_REQUIRE(T >= 0 && tk >= 1 && N >= 8 && N % 8 == 0, NVFP4_ERR_SHAPE,
             "moe_unpermute_combine: need T >= 0, tk >= 1, N %% 8 == 0");
  if (T == 0) return ok();
  NV_REQUIRE(y && inv_perm && topk_w && out, NVFP4_ERR_NULL, "moe_unpermute_combine: missing pointer");
  NV_REQUIRE(aligned(y, 16) && aligned(out, 16), NVFP4_ERR_ALIGN,
             "moe_unpermute_combine: misaligned pointer");
  hipStream_t s = as_stream(stream);
  NV_REQUIRE(T < (1LL << 31) && tk <= kMaxTopk, NVFP4_ERR_SHAPE,
             "moe_unpermute_combine: need T < 2^31 and tk <= %d", kMaxTopk);
  k_combine<<<(unsigned)T, N >= 4096 ? 512 : 256, 0, s>>>(
      static_cast<const uint16_t*>(y), inv_perm, topk_w, T, (int)tk, N,
      static_cast<uint16_t*>(out));
  return check_launch("moe_unpermute_combine");
}

}  // extern "C"
