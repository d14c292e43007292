// NVFP4 quantize-dequantize paths: the weight QDQ shared by trainer and
// rollout (weights go through one quantize-dequantize path on both sides:
// arXiv abstract; gist.science technical summary §2.1, §2.2 A), its packed
// copy for the grouped GEMMs, the second-pass QDQ of the compensated residual
// (summary §2.2 B), the E2M1 conversion itself, and the FP8 (E4M3) baseline's
// quantizer.  The online activation quantizer is in actquant.hip.
//
// Pass structure (HBM-bound): an amax pass (integer max over bf16 bit
// patterns, exact and order-free), then a block quantizer: block max -> E4M3
// scale, codes via the hardware E2M1 conversion.
#include <cstdlib>

#include "device.h"
#include "runtime.h"

namespace nvfp4 {

// Thread -> (row sub-index, column chunk) mapping used by both passes: a
// workgroup of 256 threads covers `rows_per_iter` rows of `chunks` chunks.
struct RowTiling {
  int chunks;          // chunks per row
  int rows_per_iter;   // rows a workgroup covers per step
  int col_groups;      // gridDim.y when a row has more than 256 chunks
};

static RowTiling row_tiling(int64_t chunks) {
  RowTiling t;
  if (chunks >= 256) {
    t.chunks = (int)chunks;
    t.rows_per_iter = 1;
    t.col_groups = (int)((chunks + 255) / 256);
  } else {
    t.chunks = (int)chunks;
    t.rows_per_iter = 256 / (int)chunks;
    t.col_groups = 1;
  }
  return t;
}

// Contiguous tensors: flat loop, four independent 16-byte loads in flight
// per thread (tensor t = blockIdx.y, n8 chunks of 8 elements each).

__global__ void __launch_bounds__(256)
k_amax_flat(const uint16_t* __restrict__ x, int64_t n8, int64_t tensor_stride,
            uint32_t* __restrict__ amax) {
  const uint4* xt = reinterpret_cast<const uint4*>(x + (int64_t)blockIdx.y * tensor_stride);
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = blockIdx.x * 256LL + threadIdx.x;
  uint32_t m = 0;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    const uint4 a = xt[i], b = xt[i + stride], c = xt[i + 2 * stride], d = xt[i + 3 * stride];
    m = max(m, max(max(absmax_bf16x8(a), absmax_bf16x8(b)), max(absmax_bf16x8(c), absmax_bf16x8(d))));
  }
  for (; i < n8; i += stride) m = max(m, absmax_bf16x8(xt[i]));
  block_atomic_max<256>(m, amax + blockIdx.y);
}

// The fake-quantized value of a block's 16 codes, bf16(fp32(q * s) * g), sign
// from the code bit, as 8 dwords of bf16 pairs.
__device__ __forceinline__ void fake_quant16(const uint32_t pk[2], float s, float g,
                                             uint32_t o[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c0 = (pk[i >> 2] >> (8 * (i & 3))) & 0xFu;
    const uint32_t c1 = (pk[i >> 2] >> (8 * (i & 3) + 4)) & 0xFu;
    const f32x2 q = e2m1_unpack2<0>(c0 | (c1 << 4));
    const uint32_t h0 = f32_to_bf16_rne(__builtin_fabsf(q.x * s) * g) | ((c0 & 8u) << 12);
    const uint32_t h1 = f32_to_bf16_rne(__builtin_fabsf(q.y * s) * g) | ((c1 & 8u) << 12);
    o[i] = h0 | (h1 << 16);
  }
}

// ---------------------------------------------------------------------------
// Block quantizer of the second-pass residual QDQ: one thread per 16-element
// block of a [rows][K] tensor with amax given as bf16 bits.
//
//   A = amax, g = fp32(A / 2688)
//   s = e4m3( fp32(blockmax * 448) / A )            (fp32 divide, RNE)
//   rho = fp32(2688 / fp32(s * A)),  v = fp32(x * rho),  code = e2m1(v)
//   s == 0: every magnitude 0.   Sign of a code = sign of x.
//   out_qdq = bf16(fp32(q*s) * g)                   (the fake-quantized value)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_quantize(const uint16_t* __restrict__ x, int64_t rows, int64_t ldx, int64_t K, int blocks,
           int rows_per_iter, const uint32_t* __restrict__ amax, uint8_t* __restrict__ codes,
           uint8_t* __restrict__ scales, float* __restrict__ g_out,
           uint16_t* __restrict__ out_qdq) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *g_out = bf16_bits_to_f32(*amax) / kScaleDen;
  const int cw = blocks < 256 ? blocks : 256;
  const int rsub = tid / cw;
  const int c = blockIdx.y * 256 + tid % cw;
  if (rsub >= rows_per_iter || c >= blocks) return;
  const float A = bf16_bits_to_f32(*amax);
  const float g = A / kScaleDen;
  for (int64_t r = (int64_t)blockIdx.x * rows_per_iter + rsub; r < rows;
       r += (int64_t)gridDim.x * rows_per_iter) {
    const uint16_t* xr = x + r * ldx + (int64_t)c * 16;
    const uint4 v0 = *reinterpret_cast<const uint4*>(xr);
    const uint4 v1 = *reinterpret_cast<const uint4*>(xr + 8);
    float xf[16];
    uint32_t sbyte, pk[2];
    float s;
    quant_block16(v0, v1, A, xf, sbyte, s, pk);
    *reinterpret_cast<uint2*>(codes + r * (K / 2) + (int64_t)c * 8) = make_uint2(pk[0], pk[1]);
    scales[r * (K / 16) + c] = (uint8_t)sbyte;
    uint32_t o[8];
    fake_quant16(pk, s, g, o);
    uint16_t* wo = out_qdq + r * K + (int64_t)c * 16;
    *reinterpret_cast<uint4*>(wo) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(wo + 8) = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// ---------------------------------------------------------------------------
// Weight quantize pass (after the per-expert amax pass): one workgroup per
// 16-row slice of an expert, one thread per 16-element block with
// kQdqRound blocks' loads in flight, and the 4 scale bytes of a 64-byte
// scale tile row written as one dword.  Experts run last to first: the amax
// pass read them first to last, so the first slices here re-read the rows
// it read last, which may still be in the Infinity Cache.  Four blocks in
// flight (96 VGPRs, 5 waves per SIMD) measured 3-6% faster than eight
// (152 VGPRs, 3 waves per SIMD).
// ---------------------------------------------------------------------------
constexpr int kQdqRound = 4;

__global__ void __launch_bounds__(256)
k_qdq_slices(const uint16_t* __restrict__ w, int64_t N, int64_t K, int E,
             const uint32_t* __restrict__ amax, uint8_t* __restrict__ codes,
             uint8_t* __restrict__ scales, float* __restrict__ g_w, uint16_t* __restrict__ w_qdq,
             uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales) {
  const int tid = threadIdx.x;
  const int e = E - 1 - (int)blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t KB = K / 16;
  const uint16_t* src = w + ((int64_t)e * N + row0) * K;
  const float A = bf16_bits_to_f32(amax[e]);
  const float g = A / kScaleDen;
  if (blockIdx.x == 0 && tid == 0) g_w[e] = g;
  // block b of the slice is block c = 4 t + (b % 4) of row (b / 4) % 16,
  // t = b / 64: a wave covers one 16-row x 64-column tile, so its loads are
  // whole 128-byte row pieces, its row-major code stores 32 bytes per row,
  // and (packed copy) its code stores one contiguous 512-byte tile and its
  // scale stores one 64-byte tile.  16 * KB = K is a multiple of 64
  // (K % 64 == 0), so a wave's blocks are all in range or all out, and lanes
  // 4j..4j+3 hold blocks 4t..4t+3 of one row
  const int64_t nblk = 16 * KB;
  uint8_t* psc_e = pscales ? pscales + e * packed_scales_per_expert(N, K) : nullptr;
  for (int64_t b0 = 0; b0 < nblk; b0 += 256 * kQdqRound) {
    uint4 c0[kQdqRound], c1[kQdqRound];
#pragma unroll
    for (int u = 0; u < kQdqRound; ++u) {
      const int64_t b = b0 + u * 256 + tid;
      if (b < nblk) {
        const int64_t r = (b >> 2) & 15, c = ((b >> 6) << 2) + (b & 3);
        const uint16_t* xr = src + r * K + c * 16;
        c0[u] = *reinterpret_cast<const uint4*>(xr);
        c1[u] = *reinterpret_cast<const uint4*>(xr + 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kQdqRound; ++u) {
      const int64_t b = b0 + u * 256 + tid;
      if (b >= nblk) break;                  // wave-uniform
      const int64_t r = (b >> 2) & 15, c = ((b >> 6) << 2) + (b & 3);
      float xf[16], s;
      uint32_t sbyte, pk[2];
      quant_block16(c0[u], c1[u], A, xf, sbyte, s, pk);
      const int64_t orow = (int64_t)e * N + row0 + r;
      *reinterpret_cast<uint2*>(codes + orow * (K / 2) + c * 8) = make_uint2(pk[0], pk[1]);
      const uint32_t s4 = sbyte | (__shfl_down(sbyte, 1) << 8) | (__shfl_down(sbyte, 2) << 16) |
                          (__shfl_down(sbyte, 3) << 24);
      if ((c & 3) == 0) *reinterpret_cast<uint32_t*>(scales + orow * KB + c) = s4;
      if (pcodes != nullptr) {
        *reinterpret_cast<uint2*>(pcodes + e * packed_codes_per_expert(N, K) +
                                  wcode_offset(row0 + r, 16 * c, K)) = make_uint2(pk[0], pk[1]);
        if ((c & 3) == 0) *reinterpret_cast<uint32_t*>(psc_e + wscale_offset(row0 + r, c, K)) = s4;
      }
      if (w_qdq != nullptr) {
        uint32_t o[8];
        fake_quant16(pk, s, g, o);
        uint16_t* wo = w_qdq + orow * K + c * 16;
        *reinterpret_cast<uint4*>(wo) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(wo + 8) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Row-major NVFP4 weights -> the tiles of the grouped GEMMs' packed copy:
// codes in 512-byte tiles of 16 rows x 64 columns ([N/16][K/64][2][16][16]
// per expert: column halves, rows, bytes) and block scales in 64-byte tiles
// of the same rows and columns ([..][16][4]).  A permutation of bytes:
// thread q moves the 16-byte code chunk q of the tiles, and (q < the number
// of scale dwords) the scale dword q.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_pack_weights(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t E,
               int64_t N, int64_t K, uint8_t* __restrict__ pcodes, uint8_t* __restrict__ pscales) {
  const int64_t kt = K / 64, nt = N / 16;
  const int64_t n_chunks = E * N * K / 32;        // 16-byte code chunks
  const int64_t n_words = E * N * K / 64;         // scale dwords
  const int64_t chunks_e = N * K / 32, words_e = N * K / 64;
  for (int64_t q = blockIdx.x * 256LL + threadIdx.x; q < n_chunks; q += (int64_t)gridDim.x * 256) {
    const int64_t tile = q >> 5, within = q & 31;
    const int64_t kb = tile % kt, nb = (tile / kt) % nt, e = tile / (kt * nt);
    const int64_t row = e * N + nb * 16 + (within & 15);
    const uint4 v = *reinterpret_cast<const uint4*>(codes + row * (K / 2) + kb * 32 + (within >> 4) * 16);
    *reinterpret_cast<uint4*>(pcodes + e * packed_codes_per_expert(N, K) + (q - e * chunks_e) * 16) = v;
    if (q < n_words) {
      const int64_t st = q >> 4, r = q & 15;
      const int64_t skb = st % kt, snb = (st / kt) % nt, se = st / (kt * nt);
      const int64_t srow = se * N + snb * 16 + r;
      *reinterpret_cast<uint32_t*>(pscales + se * packed_scales_per_expert(N, K) +
                                   (q - se * words_e) * 4) =
          *reinterpret_cast<const uint32_t*>(scales + srow * (K / 16) + skb * 4);
    }
  }
}

// Row-major NVFP4 weights -> the channel-major part of the packed copy.
// One wave per tile of 64 rows x 64 columns of one expert (rows past N
// skipped; N % 16 == 0): it stages the tile's codes (32 bytes per row) and
// scales (4 bytes per row) in LDS, then lane l writes column k0 + l's
// nibbles of the tile's rows (8 bytes per 16 rows) and lanes 0..15 the 16
// scale bytes of block k0 / 16 + l / 4, rows 16 (l % 4) ..
__global__ void __launch_bounds__(256)
k_pack_channel_major(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                     int64_t E, int64_t N, int64_t K, uint8_t* __restrict__ pcodes,
                     uint8_t* __restrict__ pscales) {
  __shared__ uint8_t ct[4][64][33];               // (+1: column reads spread over banks)
  __shared__ uint8_t st[4][64][4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t rt = (N + 63) / 64, kt = K / 64;
  const int64_t tiles = E * rt * kt;
  // every wave runs the same number of iterations (the barriers)
  for (int64_t t0 = (int64_t)blockIdx.x * 4; t0 < tiles; t0 += (int64_t)gridDim.x * 4) {
    const int64_t t = t0 + w;
    const bool live = t < tiles;
    const int64_t kb = live ? t % kt : 0, nb = live ? (t / kt) % rt : 0, e = live ? t / (kt * rt) : 0;
    const int64_t n0 = nb * 64, k0 = kb * 64;
    const int64_t rows = N - n0 < 64 ? N - n0 : 64;
    if (live && lane < rows) {
      const int64_t row = e * N + n0 + lane;
      // (8-byte loads: the codes need only 8-byte alignment)
      const uint2* src = reinterpret_cast<const uint2*>(codes + row * (K / 2) + k0 / 2);
      const uint2 a = src[0], b = src[1], c = src[2], d = src[3];
      const uint32_t v[8] = {a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
#pragma unroll
      for (int j = 0; j < 32; ++j) ct[w][lane][j] = (uint8_t)(v[j >> 2] >> (8 * (j & 3)));
      const uint32_t s4 = *reinterpret_cast<const uint32_t*>(scales + row * (K / 16) + k0 / 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) st[w][lane][j] = (uint8_t)(s4 >> (8 * j));
    }
    __syncthreads();
    if (live) {
      uint8_t* pc = pcodes + e * packed_codes_per_expert(N, K) + N * K / 2;
      for (int g = 0; g < rows / 16; ++g) {
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t a = (ct[w][16 * g + 2 * j][lane >> 1] >> (4 * (lane & 1))) & 0xFu;
          const uint32_t b = (ct[w][16 * g + 2 * j + 1][lane >> 1] >> (4 * (lane & 1))) & 0xFu;
          const uint32_t byte = a | (b << 4);
          if (j < 4) lo |= byte << (8 * j);
          else hi |= byte << (8 * (j - 4));
        }
        *reinterpret_cast<uint2*>(pc + (k0 + lane) * (N / 2) + (n0 + 16 * g) / 2) = make_uint2(lo, hi);
      }
      if (lane < 16 && 16 * (lane & 3) < rows) {
        const int kk = lane >> 2, r0 = 16 * (lane & 3);
        uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) o[j >> 2] |= (uint32_t)st[w][r0 + j][kk] << (8 * (j & 3));
        uint32_t* ps = reinterpret_cast<uint32_t*>(pscales + e * packed_scales_per_expert(N, K) +
                                                   N * K / 16 + (k0 / 16 + kk) * N + n0 + r0);
#pragma unroll
        for (int j = 0; j < 4; ++j) ps[j] = o[j];   // (the scales need only 4-byte alignment)
      }
    }
    __syncthreads();
  }
}

static void launch_pack_channel_major(const uint8_t* codes, const uint8_t* scales, int64_t E,
                                      int64_t N, int64_t K, uint8_t* pcodes, uint8_t* pscales,
                                      hipStream_t s) {
  const int64_t tiles = E * ((N + 63) / 64) * (K / 64);
  int64_t nb = (tiles + 3) / 4;
  if (nb > 16LL * num_cus()) nb = 16LL * num_cus();
  k_pack_channel_major<<<(unsigned)nb, 256, 0, s>>>(codes, scales, E, N, K, pcodes, pscales);
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) quantization with one float32 scale per tensor (tensor t =
// blockIdx.y): g = A / 448, code = sign(x) | E4M3(|x| / g), every magnitude
// code 0 when A = 0.  Both divisions are correctly rounded float32.  Eight
// elements (one 16-byte load, one 8-byte store) per thread per iteration.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_fp8_quantize(const uint16_t* __restrict__ x, int64_t n8, int64_t tensor_stride,
               const uint32_t* __restrict__ amax, uint8_t* __restrict__ codes,
               float* __restrict__ g) {
  const int t = blockIdx.y;
  const float A = bf16_bits_to_f32(amax[t]);
  const float gt = A / kE4M3Max;
  if (blockIdx.x == 0 && threadIdx.x == 0) g[t] = gt;
  const uint4* xt = reinterpret_cast<const uint4*>(x + (int64_t)t * tensor_stride);
  uint2* ct = reinterpret_cast<uint2*>(codes + (int64_t)t * tensor_stride);
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const uint4 v = xt[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t h = (w[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
      const uint32_t mag = A > 0.f ? e4m3_encode_nonneg(bf16_bits_to_f32(h & 0x7FFFu) / gt) : 0u;
      out[q >> 2] |= (mag | ((h >> 8) & 0x80u)) << (8 * (q & 3));
    }
    ct[i] = make_uint2(out[0], out[1]);
  }
}

// E2M1 codes of float32 values with unit scale, one code per output byte:
// the conversion every quantizer here applies to x * rho (e2m1_pack2).
__global__ void __launch_bounds__(256)
k_e2m1_encode(const float* __restrict__ v, int64_t n, uint8_t* __restrict__ codes) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; 2 * i < n; i += (int64_t)gridDim.x * 256) {
    const float a = v[2 * i];
    const float b = 2 * i + 1 < n ? v[2 * i + 1] : 0.0f;
    const uint32_t pk = e2m1_pack2(a, b);
    codes[2 * i] = (uint8_t)(pk & 0xFu);
    if (2 * i + 1 < n) codes[2 * i + 1] = (uint8_t)(pk >> 4);
  }
}

static unsigned grid_rows(int64_t rows, int rows_per_iter, int64_t cap) {
  int64_t need = (rows + rows_per_iter - 1) / rows_per_iter;
  if (need < 1) need = 1;
  return (unsigned)(need < cap ? need : cap);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t nvfp4_qdq_weights_workspace_size(int64_t E) {
  return round_up((size_t)(E > 0 ? E : 1) * sizeof(uint32_t), 256);
}

size_t nvfp4_qdq_residual_workspace_size(int64_t M, int64_t k) {
  (void)M;
  (void)k;
  return 256;
}

// Second-pass quantization of the selected residual: the [M][k] tensor goes
// through the weight QDQ path (its own amax, 16-blocks along the selected
// channels, row-major scales) and r^ = bf16(fp32(q * s) * g_r) is written for
// the GEMM's correction.
int nvfp4_qdq_residual(const void* r, int64_t M, int64_t k, uint8_t* codes, uint8_t* scales,
                       float* g_r, void* r_qdq, void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(g_r && ws, NVFP4_ERR_NULL, "nvfp4_qdq_residual: g_r and ws are required");
  NV_REQUIRE(M >= 0 && k >= 16 && k % 16 == 0 && M * k < (1LL << 40), NVFP4_ERR_SHAPE,
             "nvfp4_qdq_residual: need M >= 0, k >= 16, k %% 16 == 0 (M=%lld k=%lld)",
             (long long)M, (long long)k);
  NV_REQUIRE(M == 0 || (r && codes && scales && r_qdq), NVFP4_ERR_NULL,
             "nvfp4_qdq_residual: r, codes, scales and r_qdq are required");
  NV_REQUIRE(aligned(r, 16) && aligned(codes, 8) && aligned(r_qdq, 16) && aligned(ws, 16),
             NVFP4_ERR_ALIGN, "nvfp4_qdq_residual: misaligned pointer");
  NV_REQUIRE(ws_bytes >= nvfp4_qdq_residual_workspace_size(M, k), NVFP4_ERR_WORKSPACE,
             "nvfp4_qdq_residual: workspace too small");
  hipStream_t s = as_stream(stream);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  fill_u32(amax, 1, 0u, s);
  const int cus = num_cus();
  const uint16_t* src = static_cast<const uint16_t*>(r);
  if (M > 0) {
    const int64_t n8 = M * k / 8;
    int64_t nb = (n8 + 1023) / 1024;
    if (nb > 8LL * cus) nb = 8LL * cus;
    k_amax_flat<<<dim3((unsigned)(nb > 0 ? nb : 1), 1, 1), 256, 0, s>>>(src, n8, 0, amax);
  }
  RowTiling t16 = row_tiling(k / 16);
  dim3 grid(grid_rows(M, t16.rows_per_iter, 8LL * cus), t16.col_groups, 1);
  k_quantize<<<grid, 256, 0, s>>>(src, M, k, k, t16.chunks, t16.rows_per_iter, amax, codes, scales,
                                  g_r, static_cast<uint16_t*>(r_qdq));
  return check_launch("nvfp4_qdq_residual");
}

int nvfp4_qdq_weights(const void* w, int64_t E, int64_t N, int64_t K, uint8_t* codes,
                      uint8_t* scales, float* g_w, void* w_qdq, uint8_t* packed_codes,
                      uint8_t* packed_scales, void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(w && codes && scales && g_w && ws, NVFP4_ERR_NULL,
             "nvfp4_qdq_weights: w, codes, scales, g_w and ws are required");
  NV_REQUIRE((packed_codes == nullptr) == (packed_scales == nullptr), NVFP4_ERR_NULL,
             "nvfp4_qdq_weights: give both packed outputs or neither");
  NV_REQUIRE(E >= 1 && E <= 65535 && N >= 16 && N % 16 == 0 && K >= 64 && K % 64 == 0,
             NVFP4_ERR_SHAPE,
             "nvfp4_qdq_weights: need 1 <= E <= 65535, N %% 16 == 0, K %% 64 == 0 "
             "(N=%lld K=%lld)", (long long)N, (long long)K);
  NV_REQUIRE(aligned(w, 16) && aligned(codes, 8) && aligned(scales, 4) && aligned(w_qdq, 16) &&
                 aligned(packed_codes, 16) && aligned(packed_scales, 4) && aligned(ws, 16),
             NVFP4_ERR_ALIGN, "nvfp4_qdq_weights: misaligned pointer");
  NV_REQUIRE(ws_bytes >= nvfp4_qdq_weights_workspace_size(E), NVFP4_ERR_WORKSPACE,
             "nvfp4_qdq_weights: workspace too small");
  hipStream_t s = as_stream(stream);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  const int cus = num_cus();
  fill_u32(amax, E, 0u, s);
  const int64_t per_e = (8LL * cus + E - 1) / E;
  {
    const int64_t n8 = N * K / 8;
    int64_t nb = (n8 + 1023) / 1024;
    if (nb > per_e) nb = per_e;
    k_amax_flat<<<dim3((unsigned)(nb > 0 ? nb : 1), (unsigned)E, 1), 256, 0, s>>>(
        static_cast<const uint16_t*>(w), n8, N * K, amax);
  }
  k_qdq_slices<<<dim3((unsigned)(N / 16), (unsigned)E, 1), 256, 0, s>>>(
      static_cast<const uint16_t*>(w), N, K, (int)E, amax, codes, scales, g_w,
      static_cast<uint16_t*>(w_qdq), packed_codes, packed_scales);
  if (packed_codes != nullptr)
    launch_pack_channel_major(codes, scales, E, N, K, packed_codes, packed_scales, s);
  return check_launch("nvfp4_qdq_weights");
}

int nvfp4_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t E, int64_t N,
                       int64_t K, uint8_t* packed_codes, uint8_t* packed_scales, void* stream) {
  NV_REQUIRE(codes && scales && packed_codes && packed_scales, NVFP4_ERR_NULL,
             "nvfp4_pack_weights: missing pointer");
  NV_REQUIRE(E >= 1 && E <= 65535 && N >= 16 && N % 16 == 0 && K >= 64 && K % 64 == 0,
             NVFP4_ERR_SHAPE,
             "nvfp4_pack_weights: need 1 <= E <= 65535, N %% 16 == 0, K %% 64 == 0 "
             "(N=%lld K=%lld)", (long long)N, (long long)K);
  NV_REQUIRE(aligned(codes, 16) && aligned(scales, 4) && aligned(packed_codes, 16) &&
                 aligned(packed_scales, 4),
             NVFP4_ERR_ALIGN, "nvfp4_pack_weights: misaligned pointer");
  const int64_t n_chunks = E * N * K / 32;
  int64_t nb = (n_chunks + 255) / 256;
  if (nb > 16LL * num_cus()) nb = 16LL * num_cus();
  k_pack_weights<<<(unsigned)nb, 256, 0, as_stream(stream)>>>(codes, scales, E, N, K,
                                                             packed_codes, packed_scales);
  launch_pack_channel_major(codes, scales, E, N, K, packed_codes, packed_scales,
                            as_stream(stream));
  return check_launch("nvfp4_pack_weights");
}

int nvfp4_e2m1_encode_f32(const float* v, int64_t n, uint8_t* codes, void* stream) {
  NV_REQUIRE(n >= 0, NVFP4_ERR_SHAPE, "nvfp4_e2m1_encode_f32: n < 0");
  if (n == 0) return ok();
  NV_REQUIRE(v && codes, NVFP4_ERR_NULL, "nvfp4_e2m1_encode_f32: missing pointer");
  NV_REQUIRE(aligned(v, 4), NVFP4_ERR_ALIGN, "nvfp4_e2m1_encode_f32: misaligned v");
  int64_t nb = (n / 2 + 256) / 256;
  if (nb > 16LL * num_cus()) nb = 16LL * num_cus();
  k_e2m1_encode<<<(unsigned)nb, 256, 0, as_stream(stream)>>>(v, n, codes);
  return check_launch("nvfp4_e2m1_encode_f32");
}

size_t fp8_quantize_workspace_size(int64_t E) {
  return round_up((size_t)(E > 0 ? E : 1) * sizeof(uint32_t), 256);
}

int fp8_quantize(const void* x, int64_t E, int64_t M, int64_t K, uint8_t* codes, float* g,
                 void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(g && ws, NVFP4_ERR_NULL, "fp8_quantize: g and ws are required");
  NV_REQUIRE(E >= 1 && E <= 65535 && M >= 0 && K >= 8 && K % 8 == 0, NVFP4_ERR_SHAPE,
             "fp8_quantize: need 1 <= E <= 65535, M >= 0, K %% 8 == 0 (E=%lld M=%lld K=%lld)",
             (long long)E, (long long)M, (long long)K);
  NV_REQUIRE(M == 0 || (x && codes), NVFP4_ERR_NULL, "fp8_quantize: x and codes are required");
  NV_REQUIRE(aligned(x, 16) && aligned(codes, 8) && aligned(ws, 16), NVFP4_ERR_ALIGN,
             "fp8_quantize: misaligned pointer");
  NV_REQUIRE(ws_bytes >= fp8_quantize_workspace_size(E), NVFP4_ERR_WORKSPACE,
             "fp8_quantize: workspace too small");
  hipStream_t s = as_stream(stream);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  fill_u32(amax, E, 0u, s);
  const int64_t n8 = M * K / 8;
  const int64_t per_e = (8LL * num_cus() + E - 1) / E;
  int64_t nb = (n8 + 1023) / 1024;
  nb = nb > per_e ? per_e : (nb < 1 ? 1 : nb);
  if (n8 > 0)
    k_amax_flat<<<dim3((unsigned)nb, (unsigned)E, 1), 256, 0, s>>>(
        static_cast<const uint16_t*>(x), n8, M * K, amax);
  k_fp8_quantize<<<dim3((unsigned)nb, (unsigned)E, 1), 256, 0, s>>>(
      static_cast<const uint16_t*>(x), n8, M * K, amax, codes, g);
  return check_launch("fp8_quantize");
}

}  // extern "C"
