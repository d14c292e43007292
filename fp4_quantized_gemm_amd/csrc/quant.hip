// NVFP4 quantizers: online activation quantization (with the per-channel
// residual statistic used to pick compensation channels) and the weight QDQ
// path shared by trainer and rollout.
//
// QUADS (arXiv abstract; gist.science technical summary §2.1, §2.2 A-B):
// activations are recomputed and quantized to E2M1 every forward; weights go
// through one quantize-dequantize path on both sides; the channels with the
// largest activation residual get compensated.
//
// Pass structure (both HBM-bound):
//   1. amax: per-tensor max |x| (integer max over bf16 bit patterns, so the
//      result is exact and order-free); for the SwiGLU input it also forms
//      h = bf16(silu(gate) * up) and writes h once.
//   2. quantize: one thread per 16-element block; block max -> E4M3 scale,
//      codes via the hardware E2M1 conversion, residual and fixed-point
//      channel score in the same pass.
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

// ---------------------------------------------------------------------------
// Pass 1a: amax over one or more [rows][K] bf16 tensors stacked by row
// (tensor id = blockIdx.z).  Chunks of 8 elements (one 16-byte load).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_amax(const uint16_t* __restrict__ x, int64_t rows, int64_t ldx, int64_t tensor_stride,
       int chunks, int rows_per_iter, uint32_t* __restrict__ amax) {
  const int tid = threadIdx.x;
  const int cw = chunks < 256 ? chunks : 256;
  const int rsub = tid / cw;
  const int c = blockIdx.y * 256 + tid % cw;
  const uint16_t* xt = x + (int64_t)blockIdx.z * tensor_stride;
  uint32_t m = 0;
  if (rsub < rows_per_iter && c < chunks) {
    for (int64_t r = (int64_t)blockIdx.x * rows_per_iter + rsub; r < rows;
         r += (int64_t)gridDim.x * rows_per_iter) {
      m = max(m, absmax_bf16x8(*reinterpret_cast<const uint4*>(xt + r * ldx + (int64_t)c * 8)));
    }
  }
  block_atomic_max<256>(m, amax + blockIdx.z);
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

// ---------------------------------------------------------------------------
// Pass 1b: h = bf16(silu(gate) * up) from y = [gate | up] ([M][2I], row stride
// ldy); writes h [M][I] and its amax.  silu(g) = g / (1 + exp(-g)), float32.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_swiglu_amax(const uint16_t* __restrict__ y, int64_t rows, int64_t ldy, int64_t inter,
              int chunks, int rows_per_iter, uint16_t* __restrict__ h,
              uint32_t* __restrict__ amax) {
  const int tid = threadIdx.x;
  const int cw = chunks < 256 ? chunks : 256;
  const int rsub = tid / cw;
  const int c = blockIdx.y * 256 + tid % cw;
  uint32_t m = 0;
  if (rsub < rows_per_iter && c < chunks) {
    for (int64_t r = (int64_t)blockIdx.x * rows_per_iter + rsub; r < rows;
         r += (int64_t)gridDim.x * rows_per_iter) {
      const uint16_t* yr = y + r * ldy + (int64_t)c * 8;
      uint4 g = *reinterpret_cast<const uint4*>(yr);
      uint4 u = *reinterpret_cast<const uint4*>(yr + inter);
      uint4 o;
      o.x = swiglu_pair(g.x, u.x);
      o.y = swiglu_pair(g.y, u.y);
      o.z = swiglu_pair(g.z, u.z);
      o.w = swiglu_pair(g.w, u.w);
      *reinterpret_cast<uint4*>(h + r * inter + (int64_t)c * 8) = o;
      m = max(m, absmax_bf16x8(o));
    }
  }
  block_atomic_max<256>(m, amax);
}

// One 16-element block (two 16-byte halves of bf16 bits) against tensor amax
// A: the elements as float32, the E4M3 scale byte and value, and the 16
// codes packed two per byte (element 2j in bits 3:0 of byte j).
__device__ __forceinline__ void quant_block16(const uint4& v0, const uint4& v1, float A,
                                              float xf[16], uint32_t& sbyte, float& s,
                                              uint32_t pk[2]) {
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t bmax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xf[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    xf[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    bmax = max(bmax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
  sbyte = 0;
  s = 0.0f;
  pk[0] = pk[1] = 0u;
  if (A > 0.0f) {
    float u = (bf16_bits_to_f32(bmax) * kE4M3Max) / A;
    sbyte = e4m3_encode_nonneg(u);
    s = e4m3_decode(sbyte);
  }
  if (s > 0.0f) {
    const float rho = kScaleDen / (s * A);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t b = e2m1_pack2(xf[2 * i] * rho, xf[2 * i + 1] * rho);
      pk[i >> 2] |= b << (8 * (i & 3));
    }
  } else {
    // magnitude 0 everywhere; keep the signs
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t b = ((w[i] >> 12) & 0x8u) | ((w[i] >> 24) & 0x80u);
      pk[i >> 2] |= b << (8 * (i & 3));
    }
  }
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
// Pass 2: block quantizer.  One thread per 16-element block; tensors stacked
// by row (blockIdx.z), each with its own amax (bf16 bits) and tensor scale.
//
//   A = amax, g = fp32(A / 2688)
//   s = e4m3( fp32(blockmax * 448) / A )            (fp32 divide, RNE)
//   rho = fp32(2688 / fp32(s * A)),  v = fp32(x * rho),  code = e2m1(v)
//   s == 0: every magnitude 0.   Sign of a code = sign of x.
//   residual r = bf16(fma(-(q*s), g, x))            (one rounding to fp32)
//   score[j] += floor(|r| * 2^(31 - E_A))           (exact, <= 2^31)
//   w_qdq = bf16(fp32(q*s) * g)                     (trainer fake-quant)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
k_quantize(const uint16_t* __restrict__ x, int64_t rows, int64_t ldx, int64_t K,
           int64_t tensor_stride, int ntensors, int blocks, int rows_per_iter,
           const uint32_t* __restrict__ amax, uint8_t* __restrict__ codes,
           uint8_t* __restrict__ scales, float* __restrict__ g_out,
           uint64_t* __restrict__ partial, uint16_t* __restrict__ w_qdq) {
  // partial: [gridDim.x][K] per-workgroup channel sums (or NULL: no scores)
  extern __shared__ uint64_t red[];               // 256 * 16 entries when rows_per_iter > 1
  uint64_t* score = partial;
  const int tid = threadIdx.x;
  const int t = blockIdx.z;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0)
    g_out[t] = bf16_bits_to_f32(amax[t]) / kScaleDen;
  const int cw = blocks < 256 ? blocks : 256;
  const int rsub = tid / cw;
  const int c = blockIdx.y * 256 + tid % cw;
  const bool active = rsub < rows_per_iter && c < blocks;

  const float A = bf16_bits_to_f32(amax[t]);
  const float g = A / kScaleDen;
  const int ea = A > 0.0f ? frexp_exponent(A) : 0;
  const uint16_t* xt = x + (int64_t)t * tensor_stride;
  const int64_t row0 = (int64_t)t * rows;     // output row offset of this tensor
  uint64_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0;

  const int64_t rstep = (int64_t)gridDim.x * rows_per_iter;
  uint4 n0 = make_uint4(0, 0, 0, 0), n1 = n0;
  int64_t r = (int64_t)blockIdx.x * rows_per_iter + rsub;
  if (active && r < rows) {
    const uint16_t* xr = xt + r * ldx + (int64_t)c * 16;
    n0 = *reinterpret_cast<const uint4*>(xr);
    n1 = *reinterpret_cast<const uint4*>(xr + 8);
  }
  for (; active && r < rows; r += rstep) {
    // the next row's loads are issued before this row's arithmetic
    const uint4 v0 = n0, v1 = n1;
    if (r + rstep < rows) {
      const uint16_t* xn = xt + (r + rstep) * ldx + (int64_t)c * 16;
      n0 = *reinterpret_cast<const uint4*>(xn);
      n1 = *reinterpret_cast<const uint4*>(xn + 8);
    }
    float xf[16];
    uint32_t sbyte, pk[2];
    float s;
    quant_block16(v0, v1, A, xf, sbyte, s, pk);
    const int64_t orow = row0 + r;
    *reinterpret_cast<uint2*>(codes + orow * (K / 2) + (int64_t)c * 8) = make_uint2(pk[0], pk[1]);
    scales[orow * (K / 16) + c] = (uint8_t)sbyte;

    if (score != nullptr || w_qdq != nullptr) {
      float qs[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x2 a0 = e2m1_unpack2<0>(pk[i >> 1] >> (16 * (i & 1)));
        f32x2 a1 = e2m1_unpack2<1>(pk[i >> 1] >> (16 * (i & 1)));
        qs[4 * i + 0] = a0.x * s;
        qs[4 * i + 1] = a0.y * s;
        qs[4 * i + 2] = a1.x * s;
        qs[4 * i + 3] = a1.y * s;
      }
      if (score != nullptr && A > 0.0f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float rr = __builtin_fmaf(-qs[i], g, xf[i]);
          float rb = bf16_bits_to_f32(f32_to_bf16_rne(rr));
          acc[i] += (uint64_t)(uint32_t)__builtin_ldexpf(__builtin_fabsf(rb), 31 - ea);
        }
      }
      if (w_qdq != nullptr) {
        uint32_t o[8];
        fake_quant16(pk, s, g, o);
        uint16_t* wo = w_qdq + orow * K + (int64_t)c * 16;
        *reinterpret_cast<uint4*>(wo) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(wo + 8) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
  }
  if (partial == nullptr) return;
  // sum the rows_per_iter row groups of this workgroup, then one write per
  // channel: exact integer sums, so any grouping gives the same bits
  if (rows_per_iter > 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[tid * 16 + i] = acc[i];
    __syncthreads();
    if (rsub == 0 && active) {
      for (int q = 1; q < rows_per_iter; ++q)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += red[(q * cw + tid) * 16 + i];
    }
  }
  if (rsub == 0 && active) {
    uint64_t* dst = partial + (int64_t)blockIdx.x * K + (int64_t)c * 16;
#pragma unroll
    for (int i = 0; i < 16; i += 2)
      *reinterpret_cast<ulonglong2*>(dst + i) = make_ulonglong2(acc[i], acc[i + 1]);
  }
}

// score[j] += sum over workgroups of partial[w][j]: a block sums a tile of
// 64 channels x 64 partial rows (four row groups, LDS combine), then one
// 64-bit integer atomic per channel.  Integer sums: any order, same bits.
__global__ void __launch_bounds__(256)
k_score_reduce(const uint64_t* __restrict__ partial, int nparts, int64_t K,
               uint64_t* __restrict__ score) {
  __shared__ uint64_t red4[4][64];
  const int ch = threadIdx.x & 63, pg = threadIdx.x >> 6;
  const int64_t j = blockIdx.x * 64LL + ch;
  const int p0 = blockIdx.y * 64;
  uint64_t s = 0;
  if (j < K)
    for (int q = pg; q < 64 && p0 + q < nparts; q += 4) s += partial[(int64_t)(p0 + q) * K + j];
  red4[pg][ch] = s;
  __syncthreads();
  if (pg == 0 && j < K) {
    s = red4[0][ch] + red4[1][ch] + red4[2][ch] + red4[3][ch];
    if (s) atomicAdd(reinterpret_cast<unsigned long long*>(score + j), (unsigned long long)s);
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
             uint8_t* __restrict__ scales, float* __restrict__ g_w, uint16_t* __restrict__ w_qdq) {
  const int tid = threadIdx.x;
  const int e = E - 1 - (int)blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t KB = K / 16;
  const uint16_t* src = w + ((int64_t)e * N + row0) * K;
  const float A = bf16_bits_to_f32(amax[e]);
  const float g = A / kScaleDen;
  if (blockIdx.x == 0 && tid == 0) g_w[e] = g;
  // block b of the slice is block c = 4 t + (b % 4) of row (b / 4) % 16,
  // t = b / 64: a wave covers one 16-row x 64-column tile, so its code
  // stores are one contiguous 512-byte tile, its scale stores one 64-byte
  // tile, and its loads whole 128-byte row pieces.  16 * KB = K is a
  // multiple of 64 (K % 64 == 0), so a wave's blocks are all in range or all
  // out, and lanes 4j..4j+3 hold blocks 4t..4t+3 of one row
  const int64_t nblk = 16 * KB;
  uint8_t* sc_e = scales + (int64_t)e * N * KB;
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
      *reinterpret_cast<uint2*>(codes + (int64_t)e * N * (K / 2) + wcode_offset(row0 + r, 16 * c, K)) =
          make_uint2(pk[0], pk[1]);
      const uint32_t s4 = sbyte | (__shfl_down(sbyte, 1) << 8) | (__shfl_down(sbyte, 2) << 16) |
                          (__shfl_down(sbyte, 3) << 24);
      if ((c & 3) == 0) *reinterpret_cast<uint32_t*>(sc_e + wscale_offset(row0 + r, c, K)) = s4;
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

static unsigned grid_rows(int64_t rows, int rows_per_iter, int64_t cap) {
  int64_t need = (rows + rows_per_iter - 1) / rows_per_iter;
  if (need < 1) need = 1;
  return (unsigned)(need < cap ? need : cap);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

// at most 4 workgroups per CU: each writes one row of channel-score
// partials ([grid][K] u64), and at 8 per CU those partials were half the
// bytes of the activation itself (4 per CU measured 6-7% faster; 2 per CU
// slower on the h of the large-prefill block)
static int quant_grid(int64_t M, int64_t K) {
  RowTiling t16 = row_tiling(K / 16);
  return (int)grid_rows(M, t16.rows_per_iter, 4LL * num_cus());
}

size_t nvfp4_quantize_act_workspace_size(int64_t M, int64_t K) {
  if (M < 0 || K < 32) return 256;
  return 256 + round_up((size_t)quant_grid(M, K) * (size_t)K * sizeof(uint64_t), 256);
}

size_t nvfp4_qdq_weights_workspace_size(int64_t E) {
  return round_up((size_t)(E > 0 ? E : 1) * sizeof(uint32_t), 256);
}

// the quantize pass (and the channel-score reduction) once the amax is known
static void quantize_pass(const uint16_t* src, int64_t M, int64_t K, int64_t ld,
                          const uint32_t* amax, uint8_t* codes, uint8_t* scales, float* g_x,
                          uint64_t* score, uint64_t* partial, hipStream_t s) {
  RowTiling t16 = row_tiling(K / 16);
  const int nq = quant_grid(M, K);
  dim3 grid(nq, t16.col_groups, 1);
  const size_t red_bytes = (score && t16.rows_per_iter > 1) ? 256 * 16 * sizeof(uint64_t) : 0;
  k_quantize<<<grid, 256, red_bytes, s>>>(src, M, ld, K, 0, 1, t16.chunks, t16.rows_per_iter,
                                          amax, codes, scales, g_x, score ? partial : nullptr,
                                          nullptr);
  if (score) {
    fill_u64(score, K, 0ull, s);
    k_score_reduce<<<dim3((unsigned)((K + 63) / 64), (unsigned)((nq + 63) / 64)), 256, 0, s>>>(
        partial, nq, K, score);
  }
}

int nvfp4_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, int glu,
                       uint8_t* codes, uint8_t* scales, float* g_x, uint64_t* score,
                       void* x_used, void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(g_x && ws, NVFP4_ERR_NULL, "nvfp4_quantize_act: g_x and ws are required");
  NV_REQUIRE(M >= 0 && K >= 32 && K % 32 == 0, NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act: need M >= 0, K >= 32, K %% 32 == 0 (M=%lld K=%lld)",
             (long long)M, (long long)K);
  NV_REQUIRE(glu == 0 || glu == 1, NVFP4_ERR_SHAPE, "nvfp4_quantize_act: glu must be 0 or 1");
  NV_REQUIRE(ldx >= (glu ? 2 * K : K) && ldx % 8 == 0, NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act: bad ldx %lld", (long long)ldx);
  NV_REQUIRE(M == 0 || (x && codes && scales), NVFP4_ERR_NULL,
             "nvfp4_quantize_act: x, codes and scales are required");
  NV_REQUIRE(!glu || x_used, NVFP4_ERR_NULL, "nvfp4_quantize_act: glu=1 needs x_used for h");
  NV_REQUIRE(aligned(x, 16) && aligned(codes, 8) && aligned(x_used, 16) && aligned(score, 8) &&
                 aligned(ws, 16),
             NVFP4_ERR_ALIGN, "nvfp4_quantize_act: misaligned pointer");
  NV_REQUIRE(ws_bytes >= nvfp4_quantize_act_workspace_size(M, K), NVFP4_ERR_WORKSPACE,
             "nvfp4_quantize_act: workspace too small");
  hipStream_t s = as_stream(stream);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  uint64_t* partial = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + 256);
  fill_u32(amax, 1, 0u, s);
  const int cus = num_cus();
  const uint16_t* src = static_cast<const uint16_t*>(x);
  int64_t ld = ldx;
  if (M > 0) {
    RowTiling t8 = row_tiling(K / 8);
    dim3 grid(grid_rows(M, t8.rows_per_iter, 8LL * cus), t8.col_groups, 1);
    if (glu) {
      k_swiglu_amax<<<grid, 256, 0, s>>>(src, M, ldx, K, t8.chunks, t8.rows_per_iter,
                                         static_cast<uint16_t*>(x_used), amax);
      src = static_cast<const uint16_t*>(x_used);
      ld = K;
    } else if (ldx == K) {
      const int64_t n8 = M * K / 8;
      int64_t nb = (n8 + 1023) / 1024;
      if (nb > 8LL * cus) nb = 8LL * cus;
      k_amax_flat<<<dim3((unsigned)(nb > 0 ? nb : 1), 1, 1), 256, 0, s>>>(src, n8, 0, amax);
    } else {
      k_amax<<<grid, 256, 0, s>>>(src, M, ldx, 0, t8.chunks, t8.rows_per_iter, amax);
    }
  }
  quantize_pass(src, M, K, ld, amax, codes, scales, g_x, score, partial, s);
  return check_launch("nvfp4_quantize_act");
}

int nvfp4_quantize_act_amax(const void* x, int64_t M, int64_t K, int64_t ldx,
                            const uint32_t* amax, uint8_t* codes, uint8_t* scales, float* g_x,
                            uint64_t* score, void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(g_x && ws && amax, NVFP4_ERR_NULL,
             "nvfp4_quantize_act_amax: g_x, amax and ws are required");
  NV_REQUIRE(M >= 0 && K >= 32 && K % 32 == 0 && ldx >= K && ldx % 8 == 0, NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act_amax: need M >= 0, K >= 32, K %% 32 == 0, ldx >= K, "
             "ldx %% 8 == 0 (M=%lld K=%lld)", (long long)M, (long long)K);
  NV_REQUIRE(M == 0 || (x && codes && scales), NVFP4_ERR_NULL,
             "nvfp4_quantize_act_amax: x, codes and scales are required");
  NV_REQUIRE(aligned(x, 16) && aligned(codes, 8) && aligned(score, 8) && aligned(ws, 16) &&
                 aligned(amax, 4),
             NVFP4_ERR_ALIGN, "nvfp4_quantize_act_amax: misaligned pointer");
  NV_REQUIRE(ws_bytes >= nvfp4_quantize_act_workspace_size(M, K), NVFP4_ERR_WORKSPACE,
             "nvfp4_quantize_act_amax: workspace too small");
  uint64_t* partial = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + 256);
  quantize_pass(static_cast<const uint16_t*>(x), M, K, ldx, amax, codes, scales, g_x, score,
                partial, as_stream(stream));
  return check_launch("nvfp4_quantize_act_amax");
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
  k_quantize<<<grid, 256, 0, s>>>(src, M, k, k, 0, 1, t16.chunks, t16.rows_per_iter, amax, codes,
                                  scales, g_r, nullptr, static_cast<uint16_t*>(r_qdq));
  return check_launch("nvfp4_qdq_residual");
}

int nvfp4_qdq_weights(const void* w, int64_t E, int64_t N, int64_t K, uint8_t* codes,
                      uint8_t* scales, float* g_w, void* w_qdq, void* ws, size_t ws_bytes,
                      void* stream) {
  NV_REQUIRE(w && codes && scales && g_w && ws, NVFP4_ERR_NULL,
             "nvfp4_qdq_weights: w, codes, scales, g_w and ws are required");
  NV_REQUIRE(E >= 1 && E <= 65535 && N >= 16 && N % 16 == 0 && K >= 64 && K % 64 == 0,
             NVFP4_ERR_SHAPE,
             "nvfp4_qdq_weights: need 1 <= E <= 65535, N %% 16 == 0, K %% 64 == 0 "
             "(N=%lld K=%lld)", (long long)N, (long long)K);
  NV_REQUIRE(aligned(w, 16) && aligned(codes, 8) && aligned(w_qdq, 16) && aligned(ws, 16),
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
      static_cast<uint16_t*>(w_qdq));
  return check_launch("nvfp4_qdq_weights");
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
