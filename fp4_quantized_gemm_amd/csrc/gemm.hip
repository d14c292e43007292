// Expert-grouped W4A4 GEMM with Residual Activation Compensation (QUADS:
// keep the native FP4 product over all of K and add back, for the few
// channels of largest activation residual, the residual times the same FP4
// weights; gist.science technical summary §2.2 B; arXiv abstract).
//
// Mapping of NVFP4 onto CDNA4 matrix cores.  gfx950's scaled FP4 MFMA applies
// power-of-two (E8M0) scales per 32 elements; NVFP4 needs a full E4M3 scale
// per 16 elements.  An element times its block scale, q * s, has at most
// 2 + 4 significant bits, so it is exact in bf16: the kernel decodes packed
// codes and scales into bf16 operands in registers and runs the bf16 MFMA,
// which makes every product exact and leaves only float32 accumulation
// rounding.  The residual correction is a K-extension of the same
// accumulator: acc = g_x * sum_K x~ w~  +  sum_S r w~,  y = bf16(g_w * acc).
//
// Tiling: a workgroup owns one (expert, 128-row tile, 128-column tile); its
// four waves own 64x64 each.  K advances 128 at a time through LDS, one row
// of a stage being 64 bytes of codes + 8 scale bytes + 8 pad (80-byte stride:
// conflict-free 16-byte reads).  Lane l of a wave reads the 16 bytes at
// k-offset 32*(l/16) of its row and feeds four MFMA k-slices from them; the
// k order inside an MFMA is permuted identically for A and B, which leaves
// the dot products unchanged.
#include "device.h"
#include "runtime.h"

namespace nvfp4 {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 128;
constexpr int kRowBytes = 80;

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* g_x;
  const int32_t* a_rows;
  const uint16_t* R;
  const int32_t* S;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* g_w;
  const int32_t* offsets;
  const int32_t* tile_prefix;
  uint16_t* y;
  int64_t M_src, M_total, N, K;
  int E, k;
};

// tile_prefix[e] = number of 128-row tiles of experts before e; [E] = total
__global__ void __launch_bounds__(1024)
k_tile_prefix(const int32_t* __restrict__ offsets, int E, int64_t M_total, int bm,
              int32_t* __restrict__ prefix) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  int v = 0;
  if (tid < E) {
    int64_t lo = offsets[tid], hi = offsets[tid + 1];
    lo = lo < 0 ? 0 : (lo > M_total ? M_total : lo);
    hi = hi < lo ? lo : (hi > M_total ? M_total : hi);
    v = (int)((hi - lo + bm - 1) / bm);
  }
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o);
    if ((tid & 63) >= o) incl += u;
  }
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wsum[w];
  if (tid < E) prefix[tid] = base + incl - v;
  if (tid == E - 1) prefix[E] = base + incl;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__global__ void __launch_bounds__(256)
k_gemm_rac(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smA[kBM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t smB[kBN * kRowBytes];
  __shared__ int32_t rows_src[kBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r16 = lane & 15;

  // which expert / row tile
  const int gt = blockIdx.x;
  if (gt >= p.tile_prefix[p.E]) return;
  int lo = 0, hi = p.E;                       // largest e with prefix[e] <= gt
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (p.tile_prefix[mid] <= gt) lo = mid; else hi = mid;
  }
  const int e = lo;
  int64_t e_lo = p.offsets[e], e_hi = p.offsets[e + 1];
  e_lo = e_lo < 0 ? 0 : (e_lo > p.M_total ? p.M_total : e_lo);
  e_hi = e_hi < e_lo ? e_lo : (e_hi > p.M_total ? p.M_total : e_hi);
  const int64_t p0 = e_lo + (int64_t)(gt - p.tile_prefix[e]) * kBM;
  const int64_t n0 = (int64_t)blockIdx.y * kBN;
  const int64_t Kh = p.K / 2, Ks = p.K / 16;

  if (tid < kBM) {
    int64_t pr = p0 + tid;
    if (pr >= e_hi) pr = e_hi - 1;
    int64_t t = p.a_rows ? (int64_t)p.a_rows[pr] : pr;
    t = t < 0 ? 0 : (t >= p.M_src ? p.M_src - 1 : t);
    rows_src[tid] = (int32_t)t;
  }
  __syncthreads();

  const uint8_t* wc = p.w_codes + (int64_t)e * p.N * Kh;
  const uint8_t* wsc = p.w_scales + (int64_t)e * p.N * Ks;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < p.K; k0 += kBK) {
    // global -> registers
    uint4 ga[2], gb[2];
    uint2 gsa = make_uint2(0, 0), gsb = make_uint2(0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      const int r = q >> 2, part = q & 3;
      ga[i] = *reinterpret_cast<const uint4*>(p.a_codes + (int64_t)rows_src[r] * Kh + k0 / 2 + part * 16);
      int64_t n = n0 + r;
      if (n >= p.N) n = p.N - 1;
      gb[i] = *reinterpret_cast<const uint4*>(wc + n * Kh + k0 / 2 + part * 16);
    }
    if (tid < kBM) {
      gsa = *reinterpret_cast<const uint2*>(p.a_scales + (int64_t)rows_src[tid] * Ks + k0 / 16);
    } else {
      int64_t n = n0 + (tid - kBM);
      if (n >= p.N) n = p.N - 1;
      gsb = *reinterpret_cast<const uint2*>(wsc + n * Ks + k0 / 16);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      const int r = q >> 2, part = q & 3;
      *reinterpret_cast<uint4*>(smA + r * kRowBytes + part * 16) = ga[i];
      *reinterpret_cast<uint4*>(smB + r * kRowBytes + part * 16) = gb[i];
    }
    if (tid < kBM) *reinterpret_cast<uint2*>(smA + tid * kRowBytes + 64) = gsa;
    else *reinterpret_cast<uint2*>(smB + (tid - kBM) * kRowBytes + 64) = gsb;
    __syncthreads();

    // LDS -> registers (packed), decode per k-slice, MFMA
    uint4 ar[4], br[4];
    uint32_t as[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm * 64 + 16 * i + r16;
      ar[i] = *reinterpret_cast<const uint4*>(smA + ra * kRowBytes + 16 * g);
      as[i] = *reinterpret_cast<const uint16_t*>(smA + ra * kRowBytes + 64 + 2 * g);
      const int rb = wn * 64 + 16 * i + r16;
      br[i] = *reinterpret_cast<const uint4*>(smB + rb * kRowBytes + 16 * g);
      bs[i] = *reinterpret_cast<const uint16_t*>(smB + rb * kRowBytes + 64 + 2 * g);
    }
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      u32x4 A[4], B[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wa = sl == 0 ? ar[i].x : sl == 1 ? ar[i].y : sl == 2 ? ar[i].z : ar[i].w;
        const uint32_t wb = sl == 0 ? br[i].x : sl == 1 ? br[i].y : sl == 2 ? br[i].z : br[i].w;
        A[i] = decode8_bf16(wa, e4m3_decode((as[i] >> (8 * (sl >> 1))) & 0xFFu));
        B[i] = decode8_bf16(wb, e4m3_decode((bs[i] >> (8 * (sl >> 1))) & 0xFFu));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(A[i], B[j], acc[i][j]);
    }
  }

  // epilogue: x g_x, residual K-extension over S, x g_w, bf16 store
  const float gx = *p.g_x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] *= gx;

  for (int kc = 0; kc < p.k; kc += 32) {
    u32x4 A[4], B[4];
    int ch[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int slot = kc + 8 * g + t;
      int c = slot < p.k ? p.S[slot] : -1;
      ch[t] = c < 0 ? -1 : (c >= p.K ? (int)p.K - 1 : c);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = rows_src[wm * 64 + 16 * i + r16];
      const uint16_t* rr = p.R + t * p.k + kc + 8 * g;
      uint32_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = (kc + 8 * g + q < p.k) ? rr[q] : 0u;
      A[i] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t n = n0 + wn * 64 + 16 * j + r16;
      if (n >= p.N) n = p.N - 1;
      uint32_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (ch[q] < 0) { v[q] = 0u; continue; }
        const uint32_t byte = wc[n * Kh + (ch[q] >> 1)];
        const float wq = e2m1_unpack2<0>((byte >> (4 * (ch[q] & 1))) & 0xFu).x;
        const float ws = e4m3_decode(wsc[n * Ks + (ch[q] >> 4)]);
        v[q] = __float_as_uint(wq * ws) >> 16;
      }
      B[j] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(A[i], B[j], acc[i][j]);
  }

  const float gw = p.g_w[e];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int64_t prow = p0 + wm * 64 + 16 * i + 4 * g + rr;
      if (prow >= e_hi) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + 16 * j + r16;
        if (n < p.N) p.y[prow * p.N + n] = (uint16_t)f32_to_bf16_rne(acc[i][j][rr] * gw);
      }
    }
  }
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t grouped_w4a4_gemm_rac_workspace_size(int64_t E, int64_t M_total, int64_t N, int64_t K,
                                            int64_t k) {
  (void)M_total;
  (void)N;
  (void)K;
  (void)k;
  return round_up((size_t)(E + 1) * sizeof(int32_t), 256);
}

int grouped_w4a4_gemm_rac(const uint8_t* a_codes, const uint8_t* a_scales, const float* g_x,
                          const int32_t* a_rows, int64_t M_src, const void* R_S, const int32_t* S,
                          int64_t k, const uint8_t* w_codes, const uint8_t* w_scales,
                          const float* g_w, const int32_t* expert_offsets, int64_t E,
                          int64_t M_total, int64_t N, int64_t K, void* y, void* ws,
                          size_t ws_bytes, void* stream) {
  NV_REQUIRE(E >= 1 && E <= 1024 && M_total >= 0 && N >= 16 && N % 16 == 0 && K >= kBK &&
                 K % kBK == 0 && k >= 0 && k <= K && M_src >= 0,
             NVFP4_ERR_SHAPE,
             "grouped_w4a4_gemm_rac: need 1 <= E <= 1024, N %% 16 == 0, K %% 128 == 0, "
             "0 <= k <= K (E=%lld N=%lld K=%lld k=%lld)",
             (long long)E, (long long)N, (long long)K, (long long)k);
  NV_REQUIRE(a_rows != nullptr || M_src >= M_total, NVFP4_ERR_SHAPE,
             "grouped_w4a4_gemm_rac: without a_rows, M_src must be >= M_total");
  NV_REQUIRE(M_total == 0 || M_src >= 1, NVFP4_ERR_SHAPE, "grouped_w4a4_gemm_rac: M_src == 0");
  NV_REQUIRE(g_x && w_codes && w_scales && g_w && expert_offsets && ws &&
                 (M_total == 0 || (a_codes && a_scales && y)) && (k == 0 || (R_S && S)),
             NVFP4_ERR_NULL, "grouped_w4a4_gemm_rac: missing pointer");
  NV_REQUIRE(aligned(a_codes, 16) && aligned(w_codes, 16) && aligned(a_scales, 8) &&
                 aligned(w_scales, 8) && aligned(ws, 16) && aligned(y, 2) && aligned(R_S, 2),
             NVFP4_ERR_ALIGN, "grouped_w4a4_gemm_rac: misaligned pointer");
  NV_REQUIRE(ws_bytes >= grouped_w4a4_gemm_rac_workspace_size(E, M_total, N, K, k),
             NVFP4_ERR_WORKSPACE, "grouped_w4a4_gemm_rac: workspace too small");
  if (M_total == 0) return ok();
  hipStream_t s = as_stream(stream);
  int32_t* prefix = static_cast<int32_t*>(ws);
  k_tile_prefix<<<1, 1024, 0, s>>>(expert_offsets, (int)E, M_total, kBM, prefix);
  GemmArgs a;
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.g_x = g_x;
  a.a_rows = a_rows;
  a.R = static_cast<const uint16_t*>(R_S);
  a.S = S;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.g_w = g_w;
  a.offsets = expert_offsets;
  a.tile_prefix = prefix;
  a.y = static_cast<uint16_t*>(y);
  a.M_src = M_src;
  a.M_total = M_total;
  a.N = N;
  a.K = K;
  a.E = (int)E;
  a.k = (int)k;
  const int64_t m_tiles = (M_total + kBM - 1) / kBM + E;
  const int64_t n_tiles = (N + kBN - 1) / kBN;
  k_gemm_rac<<<dim3((unsigned)m_tiles, (unsigned)n_tiles), 256, 0, s>>>(a);
  return check_launch("grouped_w4a4_gemm_rac");
}

}  // extern "C"
