// Device helpers for the NVFP4 kernels (gfx950 only).
//
// Number formats: E2M1 element codes (sign | 3-bit magnitude index into
// {0, .5, 1, 1.5, 2, 3, 4, 6}), OCP FP8 E4M3 block scales over 16 elements,
// one float32 tensor scale.  The QUADS pages name only the E2M1 grid and
// "fine-grained scaling" (gist.science technical summary §1; arXiv
// abstract); the block layout is the public NVFP4 definition.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
constexpr float kScaleDen = 2688.0f;   // 6 * 448: largest E2M1 magnitude x largest E4M3

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two float32 values -> their bf16 bits packed (a low, b high), round to
// nearest even: one hardware conversion on gfx950.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Non-negative float32 -> E4M3 byte, round to nearest even, saturate at 448.
// Subnormal range (u < 2^-6): the code is the nearest multiple of 2^-9,
// which rintf (ties to even) gives exactly after an exact power-of-two
// scaling; a result of 8 is the smallest normal's code, as it should be.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float u) {
  if (!(u < kE4M3Max)) return 0x7Eu;
  if (u < 0.015625f) return (uint32_t)__builtin_rintf(u * 512.0f);
  uint32_t b = __float_as_uint(u);
  uint32_t e = (b >> 23) - 127u + 7u;        // biased E4M3 exponent, 1..15
  uint32_t m = b & 0x7FFFFFu;
  uint32_t f = m >> 20, rem = m & 0xFFFFFu;
  f += (rem > 0x80000u || (rem == 0x80000u && (f & 1u))) ? 1u : 0u;
  uint32_t code = (e << 3) + f;              // a mantissa carry bumps the exponent
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// Two float32 values -> one byte of two E2M1 codes (a in bits 3:0, b in
// bits 7:4): round to nearest, ties to the even code, saturating at 6, sign
// kept for values that round to zero (the hardware conversion with unit
// scale does exactly this).
__device__ __forceinline__ uint32_t e2m1_pack2(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// Byte `sel` (0..3) of w, two E2M1 codes -> their two values as float32.
// The conversion's own scale only applies a power of two, so an E4M3 block
// scale is multiplied in separately by the callers.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_unpack2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Pack the (exact) bf16 images of two float32 values whose low 16 bits are
// zero: the upper halves, a low, b high.
__device__ __forceinline__ uint32_t pack_hi16(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// 8 E2M1 codes (one dword) times one block scale -> 8 bf16 values, exact
// (a code value has 2 significant bits, an E4M3 value 4, bf16 holds 8).
__device__ __forceinline__ u32x4 decode8_bf16(uint32_t w, float s) {
  f32x2 v0 = e2m1_unpack2<0>(w), v1 = e2m1_unpack2<1>(w);
  f32x2 v2 = e2m1_unpack2<2>(w), v3 = e2m1_unpack2<3>(w);
  u32x4 r;
  r.x = pack_hi16(v0.x * s, v0.y * s);
  r.y = pack_hi16(v1.x * s, v1.y * s);
  r.z = pack_hi16(v2.x * s, v2.y * s);
  r.w = pack_hi16(v3.x * s, v3.y * s);
  return r;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// max |v| over 8 bf16 values (two per dword) as 15-bit magnitude bits: for
// finite values the bits order like the magnitudes
__device__ __forceinline__ uint32_t absmax_bf16x8(uint4 v) {
  const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu, d = v.z & 0x7FFF7FFFu,
                 e = v.w & 0x7FFF7FFFu;
  const uint32_t hi = max(max(a >> 16, b >> 16), max(d >> 16, e >> 16));
  const uint32_t lo = max(max(a & 0xFFFFu, b & 0xFFFFu), max(d & 0xFFFFu, e & 0xFFFFu));
  return max(hi, lo);
}

// Block-wide max of non-negative 32-bit values, then one device atomic per
// block (instead of one per wave, which serialises at the L2 on one address).
template <int NTHREADS>
__device__ __forceinline__ void block_atomic_max(uint32_t v, uint32_t* dst) {
  __shared__ uint32_t wm[NTHREADS / 64];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NTHREADS / 64; ++i) m = wm[i] > m ? wm[i] : m;
    if (m) atomicMax(dst, m);
  }
}

// Weight block scales are stored in 64-byte tiles, one per 16 rows x 64 k:
// [N/16][K/64][16 rows][4 blocks].  A GEMM reads a row block's scales for a
// stretch of K as whole tiles (row-major [N][K/16] would give each 64-k step
// 4 bytes of every row and a 128-byte line shared by 32 steps).  Byte offset
// of block kb (= k / 16) of row n, for K columns:
__device__ __forceinline__ int64_t wscale_offset(int64_t n, int64_t kb, int64_t K) {
  return (((n >> 4) * (K >> 6) + (kb >> 2)) << 6) + ((n & 15) << 2) + (kb & 3);
}

// Weight codes are tiled the same way, 512 bytes per 16 rows x 64 k, in two
// halves of 32 columns: [N/16][K/64][2 halves][16 rows][16 bytes].  A 64-k
// step of a row block is then one contiguous run of whole cache lines
// (row-major [N][K/2] gives each step 32 bytes of every row, half of a
// 64-byte request), and a load instruction whose lanes take 16 bytes of 16
// rows of one half reads whole 128-byte lines.  Byte offset of the code
// byte holding columns k, k + 1 (k even) of row n, for K columns:
__device__ __forceinline__ int64_t wcode_offset(int64_t n, int64_t k, int64_t K) {
  return (((n >> 4) * (K >> 6) + (k >> 6)) << 9) + (((k & 63) >> 5) << 8) + ((n & 15) << 4) +
         ((k & 31) >> 1);
}

// The grouped GEMMs' packed copy of one expert's weights is the code tiles
// above (N * K / 2 bytes) followed by a channel-major copy of the codes,
// [K][N / 2] (byte n / 2 of column k: rows n, n + 1, the lower row in bits
// 3:0); its scales are the scale tiles (N * K / 16 bytes) followed by a
// channel-major copy [K / 16][N].  The channel-major copies let the
// residual correction gather the weight columns of a few selected channels
// without reading the whole matrix.
__host__ __device__ __forceinline__ int64_t packed_codes_per_expert(int64_t N, int64_t K) {
  return N * K;
}
__host__ __device__ __forceinline__ int64_t packed_scales_per_expert(int64_t N, int64_t K) {
  return N * K / 8;
}

// SwiGLU of bf16 gate and up values: silu(g) * u in float32 with the
// hardware exp2 and reciprocal (a few float32 ulps), then one rounding to
// bf16: the correctly rounded bf16 value except when the float32 value lies
// within those ulps of a bf16 rounding boundary, i.e. at most one bf16 step
// away from it.  Shared by the quantizer's SwiGLU pass and the gate+up GEMM
// epilogue, so both give the same bits.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// two bf16 gates and two bf16 ups (packed pairs) -> two bf16 h (packed)
__device__ __forceinline__ uint32_t swiglu_pair(uint32_t g2, uint32_t u2) {
  float g0 = bf16_bits_to_f32(g2 & 0xFFFFu), g1 = bf16_bits_to_f32(g2 >> 16);
  float u0 = bf16_bits_to_f32(u2 & 0xFFFFu), u1 = bf16_bits_to_f32(u2 >> 16);
  return bf16x2_rne(silu_mul(g0, u0), silu_mul(g1, u1));
}

// One 16-element block (two 16-byte halves of bf16 bits) against tensor amax
// A: the elements as float32, the E4M3 scale byte and value, and the 16
// codes packed two per byte (element 2j in bits 3:0 of byte j).
__device__ __forceinline__ void quant_block16(const uint4& v0, const uint4& v1, float A,
                                              float xf[16], uint32_t& sbyte, float& s,
                                              uint32_t pk[2]) {
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  // largest |x| bits: a packed 16-bit max over the sign-cleared pairs
  typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
  u16x2_t m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xf[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    xf[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
  }
  const uint32_t bmax = max((uint32_t)m2.x, (uint32_t)m2.y);
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
    // each conversion writes its two codes into byte i % 4 of the word
#define NV_PK_FP4(I)                                                                    \
  pk[(I) >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(pk[(I) >> 2], xf[2 * (I)] * rho, \
                                                          xf[2 * (I) + 1] * rho, 1.0f, (I) & 3)
    NV_PK_FP4(0); NV_PK_FP4(1); NV_PK_FP4(2); NV_PK_FP4(3);
    NV_PK_FP4(4); NV_PK_FP4(5); NV_PK_FP4(6); NV_PK_FP4(7);
#undef NV_PK_FP4
  } else {
    // magnitude 0 everywhere; keep the signs
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t b = ((w[i] >> 12) & 0x8u) | ((w[i] >> 24) & 0x80u);
      pk[i >> 2] |= b << (8 * (i & 3));
    }
  }
}

__device__ __forceinline__ int frexp_exponent(float a) {
  return (int)((__float_as_uint(a) >> 23) & 0xFFu) - 126;   // a normal and > 0
}

}  // namespace nvfp4
