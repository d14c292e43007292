// Online activation quantization with the per-channel residual statistic
// that Residual Activation Compensation ranks channels by (QUADS: activations
// are recomputed and quantized to E2M1 every forward, arXiv abstract and
// gist.science technical summary §2.1; the channels of largest residual get
// compensated, summary §2.2 B).
//
// Two kernels per call (three when the amax is given and G_r > 1):
//   1. amax: every workgroup writes the largest |x| of its share (bf16 bits,
//      an integer max, so exact and order-free) to its own slot; nothing is
//      shared, so nothing needs clearing first.  For the SwiGLU input it also
//      forms h = bf16(silu(gate) * up) and writes h once.  Its first
//      workgroup zeroes the scores for step 2.
//   2. quantize: a workgroup owns one column tile of 256 channels (16 blocks
//      of 16) for every G_r-th group of 16 rows: it takes the tensor amax as
//      the largest slot, quantizes its blocks (E4M3 scale, E2M1 codes via the
//      hardware conversion), forms the residual and the fixed-point channel
//      score of its rows, and adds the 256 channel sums of its row groups to
//      the scores with 64-bit integer atomics (with G_r = 1 it writes them).
//      Integer sums: any order gives the same bits.
//   3. only when the amax is given (no pass 1 to zero the scores) and
//      G_r > 1: step 2 writes its channel sums to the scratch instead, and
//      score[j] = the G_r partial sums of channel j, as a kernel.
//
// Scratch per call: the amax slots and (amax given) G_r x K u64 partial
// sums, with G_r chosen so the grid holds about four workgroups per CU: at
// most ~2 MB at K = 4096 on 256 CUs, whatever M is.
#include <mutex>

#include "device.h"
#include "runtime.h"

namespace nvfp4 {

constexpr int kAmaxSlots = 1024;        // workgroups of the amax pass, at most
constexpr int kTileBlocks = 16;         // 16-element blocks per column tile (256 channels)
constexpr int kTileRows = 16;           // rows per workgroup step

// Workgroup max of non-negative 32-bit values (every thread returns it).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t wm[4];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t m = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
  __syncthreads();
  return m;
}

// Pass 1, contiguous x: n8 chunks of 8 bf16, four 16-byte loads in flight per
// thread; workgroup b writes its max to part[b].
__global__ void __launch_bounds__(256)
k_act_amax(const uint16_t* __restrict__ x, int64_t n8, uint32_t* __restrict__ part,
           uint64_t* __restrict__ zero, int64_t n_zero) {
  if (blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0ull;
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = blockIdx.x * 256LL + threadIdx.x;
  uint32_t m = 0;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    const uint4 a = xv[i], b = xv[i + stride], c = xv[i + 2 * stride], d = xv[i + 3 * stride];
    m = max(m, max(max(absmax_bf16x8(a), absmax_bf16x8(b)), max(absmax_bf16x8(c), absmax_bf16x8(d))));
  }
  for (; i < n8; i += stride) m = max(m, absmax_bf16x8(xv[i]));
  m = block_max_u32(m);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// Pass 1, rows of K bf16 at stride ldx (workgroup b takes rows b, b + G, ...).
__global__ void __launch_bounds__(256)
k_act_amax_rows(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                uint32_t* __restrict__ part, uint64_t* __restrict__ zero, int64_t n_zero) {
  if (blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0ull;
  uint32_t m = 0;
  for (int64_t r = blockIdx.x; r < M; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < K / 8; c += 256)
      m = max(m, absmax_bf16x8(*reinterpret_cast<const uint4*>(x + r * ldx + c * 8)));
  m = block_max_u32(m);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// Pass 1 for the SwiGLU input: h [M][I] = bf16(silu(gate) * up) of
// y = [gate | up] ([M][2I], row stride ldy), written once, with its amax.
__global__ void __launch_bounds__(256)
k_act_swiglu_amax(const uint16_t* __restrict__ y, int64_t M, int64_t ldy, int64_t I,
                  uint16_t* __restrict__ h, uint32_t* __restrict__ part,
                  uint64_t* __restrict__ zero, int64_t n_zero) {
  if (blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0ull;
  uint32_t m = 0;
  const int64_t n8 = M * (I / 8);
  for (int64_t q = blockIdx.x * 256LL + threadIdx.x; q < n8; q += (int64_t)gridDim.x * 256) {
    const int64_t r = q / (I / 8), c = (q - r * (I / 8)) * 8;
    const uint16_t* yr = y + r * ldy + c;
    const uint4 g = *reinterpret_cast<const uint4*>(yr);
    const uint4 u = *reinterpret_cast<const uint4*>(yr + I);
    const uint4 o = make_uint4(swiglu_pair(g.x, u.x), swiglu_pair(g.y, u.y), swiglu_pair(g.z, u.z),
                               swiglu_pair(g.w, u.w));
    *reinterpret_cast<uint4*>(h + r * I + c) = o;
    m = max(m, absmax_bf16x8(o));
  }
  m = block_max_u32(m);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// Pass 2.  Grid (column tiles, G_r row groups), 256 threads: thread (rs, cb)
// = (tid / 16, tid % 16) takes block cb of the tile in rows
// 16 (blockIdx.y + G_r i) + rs.  The tensor amax is amax_given (bf16 bits)
// or the largest of part[0 .. n_part).
//
//   A = amax, g = fp32(A / 2688)
//   s = e4m3( fp32(blockmax * 448) / A )            (fp32 divide, RNE)
//   rho = fp32(2688 / fp32(s * A)),  v = fp32(x * rho),  code = e2m1(v)
//   s == 0: every magnitude 0.   Sign of a code = sign of x.
//   r = bf16(fma(-(q*s), g, x))                     (one rounding to fp32)
//   score[j] += floor(|r| * 2^(31 - E_A))           (exact, < 2^32)
__global__ void __launch_bounds__(256)
k_act_quant(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
            const uint32_t* __restrict__ part, int n_part, const uint32_t* __restrict__ amax_given,
            uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ g_out,
            uint64_t* __restrict__ score, uint64_t* __restrict__ score_part,
            int score_zeroed) {
  __shared__ uint64_t red[kTileRows][kTileBlocks * 16];      // 32 KB: [row sub][channel]
  const int tid = threadIdx.x;
  const int rs = tid >> 4, cb = tid & 15;
  const int ct = blockIdx.x, gy = blockIdx.y, G_r = gridDim.y;

  uint32_t abits;
  if (amax_given != nullptr) {
    abits = *amax_given;
  } else {
    uint32_t m = 0;
    for (int i = tid; i < n_part; i += 256) m = max(m, part[i]);
    abits = block_max_u32(m);
  }
  const float A = bf16_bits_to_f32(abits);
  const float g = A / kScaleDen;
  if (ct == 0 && gy == 0 && tid == 0) *g_out = g;
  const int ea = A > 0.0f ? frexp_exponent(A) : 0;

  const int64_t nblk = K / 16;
  const int64_t blk = (int64_t)ct * kTileBlocks + cb;
  const bool active = blk < nblk;
  // four consecutive blocks of a row share one scale dword when the row's
  // scales are dword-aligned (K % 64 == 0: then a tile's blocks come in whole
  // fours)
  const bool scale_dw = (nblk & 3) == 0;
  // channel sums: 32-bit over up to 8 rows, then added to 64 bits (a term
  // is at most |r| 2^(31 - E_A) with |r| <= 0.18 A < 0.18 2^E_A, so 8 terms
  // stay below 2^32)
  uint64_t acc[16];
  uint32_t a32[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0, a32[i] = 0;
  int n32 = 0;

  const int64_t rstep = (int64_t)kTileRows * G_r;
  int64_t r = (int64_t)gy * kTileRows + rs;
  // rows two steps ahead are loaded before a row's arithmetic
  uint4 n0 = make_uint4(0, 0, 0, 0), n1 = n0, m0 = n0, m1 = n0;
  if (active && r < M) {
    const uint16_t* xr = x + r * ldx + blk * 16;
    n0 = *reinterpret_cast<const uint4*>(xr);
    n1 = *reinterpret_cast<const uint4*>(xr + 8);
  }
  if (active && r + rstep < M) {
    const uint16_t* xr = x + (r + rstep) * ldx + blk * 16;
    m0 = *reinterpret_cast<const uint4*>(xr);
    m1 = *reinterpret_cast<const uint4*>(xr + 8);
  }
  // (every thread runs the same number of iterations: the scale-dword
  // shuffles below need all lanes of a row group)
  for (int64_t r0 = (int64_t)gy * kTileRows; r0 < M; r0 += rstep, r += rstep) {
    const uint4 v0 = n0, v1 = n1;
    n0 = m0;
    n1 = m1;
    const bool live = active && r < M;
    if (active && r + 2 * rstep < M) {
      const uint16_t* xn = x + (r + 2 * rstep) * ldx + blk * 16;
      m0 = *reinterpret_cast<const uint4*>(xn);
      m1 = *reinterpret_cast<const uint4*>(xn + 8);
    }
    float xf[16];
    uint32_t sbyte, pk[2];
    float s;
    quant_block16(v0, v1, A, xf, sbyte, s, pk);
    if (live) *reinterpret_cast<uint2*>(codes + r * (K / 2) + blk * 8) = make_uint2(pk[0], pk[1]);
    if (scale_dw) {
      const uint32_t s4 = sbyte | (__shfl_down(sbyte, 1) << 8) | (__shfl_down(sbyte, 2) << 16) |
                          (__shfl_down(sbyte, 3) << 24);
      if (live && (cb & 3) == 0) *reinterpret_cast<uint32_t*>(scales + r * nblk + blk) = s4;
    } else if (live) {
      scales[r * nblk + blk] = (uint8_t)sbyte;
    }
    if (score != nullptr && live && A > 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x2 q = e2m1_unpack2<0>((pk[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        const float r0f = __builtin_fmaf(-(q.x * s), g, xf[2 * i]);
        const float r1f = __builtin_fmaf(-(q.y * s), g, xf[2 * i + 1]);
        // r = bf16(r0f), bf16(r1f): one round-to-nearest-even conversion
        const uint32_t rb = bf16x2_rne(r0f, r1f);
        const float b0 = __uint_as_float(rb << 16), b1 = __uint_as_float(rb & 0xFFFF0000u);
        a32[2 * i] += (uint32_t)__builtin_ldexpf(__builtin_fabsf(b0), 31 - ea);
        a32[2 * i + 1] += (uint32_t)__builtin_ldexpf(__builtin_fabsf(b1), 31 - ea);
      }
    }
    if (++n32 == 8) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += a32[i], a32[i] = 0;
      n32 = 0;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] += a32[i];
  if (score == nullptr) return;

  // the tile's 256 channel sums over this workgroup's rows
#pragma unroll
  for (int i = 0; i < 16; ++i) red[rs][cb * 16 + i] = acc[i];
  __syncthreads();
  uint64_t tot = 0;
#pragma unroll
  for (int q = 0; q < kTileRows; ++q) tot += red[q][tid];
  const int64_t ch = (int64_t)ct * (kTileBlocks * 16) + tid;
  if (ch >= K) return;
  if (G_r == 1)
    score[ch] = tot;
  else if (score_zeroed)
    atomicAdd(reinterpret_cast<unsigned long long*>(score + ch), (unsigned long long)tot);
  else
    score_part[(int64_t)gy * K + ch] = tot;
}

// Pass 3: score[j] = sum over q < G_r of part[q][j].  A workgroup takes 64
// channels; its 256 threads split each channel's G_r partial sums in four
// (eight independent loads in flight per thread), then four sums per channel
// are added in LDS.
__global__ void __launch_bounds__(256)
k_act_score_sum(const uint64_t* __restrict__ part, int G_r, int64_t K,
                uint64_t* __restrict__ score) {
  __shared__ uint64_t red[4][64];
  const int c = threadIdx.x & 63, sl = threadIdx.x >> 6;
  const int64_t ch = blockIdx.x * 64LL + c;
  uint64_t sum = 0;
  if (ch < K) {
    const int q0 = (int)((int64_t)G_r * sl / 4), q1 = (int)((int64_t)G_r * (sl + 1) / 4);
    int q = q0;
    for (; q + 8 <= q1; q += 8) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(q + u) * K + ch];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; q < q1; ++q) sum += part[(int64_t)q * K + ch];
  }
  red[sl][c] = sum;
  __syncthreads();
  if (sl == 0 && ch < K) score[ch] = red[0][c] + red[1][c] + red[2][c] + red[3][c];
}

// Launch plan of one call: column tiles, row groups and the scratch they use.
struct ActPlan {
  int tiles;        // column tiles of 256 channels
  int groups;       // G_r
  size_t part_off, bytes;
};

// max_part_bytes: a cap on the partial sums (the fixed scratch of the
// allocation-free entry point), or 0 for none; fewer row groups then share
// the rows
static ActPlan act_plan(int64_t M, int64_t K, int cus, size_t max_part_bytes) {
  ActPlan p;
  p.tiles = (int)((K / 16 + kTileBlocks - 1) / kTileBlocks);
  const int64_t row_groups = (M + kTileRows - 1) / kTileRows;
  int64_t gr = (4LL * cus + p.tiles - 1) / p.tiles;
  if (gr > row_groups) gr = row_groups;
  if (gr > 65535) gr = 65535;
  if (max_part_bytes > 0 && gr * K * 8 > (int64_t)max_part_bytes)
    gr = (int64_t)max_part_bytes / (K * 8);
  p.groups = (int)(gr < 1 ? 1 : gr);
  p.part_off = kAmaxSlots * sizeof(uint32_t);
  p.bytes = p.part_off + (p.groups > 1 ? (size_t)p.groups * (size_t)K * 8 : 0);
  return p;
}

// The whole call on the given scratch (`ws`, at least plan.bytes).
static int act_quantize(const char* who, const void* x, int64_t M, int64_t K, int64_t ldx,
                        int glu, const uint32_t* amax_given, uint8_t* codes, uint8_t* scales,
                        float* g_x, uint64_t* score, void* x_used, void* ws, const ActPlan& pl,
                        hipStream_t s) {
  uint32_t* part = static_cast<uint32_t*>(ws);
  uint64_t* score_part = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + pl.part_off);
  // with the amax pass in this call, it zeroes the scores and the quantize
  // pass adds each workgroup's channel sums with 64-bit integer atomics (no
  // third launch, no partial sums); with the amax given, the partial sums
  // go to the scratch and a separate pass adds them
  const bool atomic_scores = amax_given == nullptr && score != nullptr && pl.groups > 1;
  uint64_t* zero = atomic_scores ? score : nullptr;
  const int64_t n_zero = atomic_scores ? K : 0;
  const uint16_t* src = static_cast<const uint16_t*>(x);
  int64_t ld = ldx;
  int n_part = 0;
  if (amax_given == nullptr) {
    const int cus = num_cus();
    int64_t nb;
    if (glu) {
      nb = (M * (K / 8) + 1023) / 1024;
      nb = nb > 4LL * cus ? 4LL * cus : nb;
      nb = nb > kAmaxSlots ? kAmaxSlots : (nb < 1 ? 1 : nb);
      k_act_swiglu_amax<<<(unsigned)nb, 256, 0, s>>>(src, M, ldx, K,
                                                    static_cast<uint16_t*>(x_used), part,
                                                    zero, n_zero);
      src = static_cast<const uint16_t*>(x_used);
      ld = K;
    } else if (ldx == K) {
      nb = (M * K / 8 + 1023) / 1024;
      nb = nb > 4LL * cus ? 4LL * cus : nb;
      nb = nb > kAmaxSlots ? kAmaxSlots : (nb < 1 ? 1 : nb);
      k_act_amax<<<(unsigned)nb, 256, 0, s>>>(src, M * K / 8, part, zero, n_zero);
    } else {
      nb = M < 1 ? 1 : (M > 4LL * cus ? 4LL * cus : M);
      nb = nb > kAmaxSlots ? kAmaxSlots : nb;
      k_act_amax_rows<<<(unsigned)nb, 256, 0, s>>>(src, M, K, ldx, part, zero, n_zero);
    }
    n_part = (int)nb;
  }
  k_act_quant<<<dim3((unsigned)pl.tiles, (unsigned)pl.groups), 256, 0, s>>>(
      src, M, K, ld, part, n_part, amax_given, codes, scales, g_x, score, score_part,
      atomic_scores ? 1 : 0);
  if (score != nullptr && pl.groups > 1 && !atomic_scores)
    k_act_score_sum<<<(unsigned)((K + 63) / 64), 256, 0, s>>>(score_part, pl.groups, K, score);
  return check_launch(who);
}

// ---------------------------------------------------------------------------
// Allocation-free entry point: the same two kernels on a fixed scratch array
// in device memory (one copy per device, kept until the process ends), for
// callers that cannot allocate.  Every call on a device shares its copy:
// the amax slots and partial sums are written before they are read in each
// call, so nothing carries over from one call to the next; calls that
// overlap in time on one device race.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
constexpr int64_t kNoAllocMaxK = 65536;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_addr[64];

// The device address of this device's copy of `scratch`, looked up once per
// device with that device current.  (In host code the array's name is a
// host-side stand-in, not a device address.)
static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(NVFP4_ERR_HIP, "nvfp4_quantize_act_noalloc: hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(NVFP4_ERR_HIP, "nvfp4_quantize_act_noalloc: hipGetSymbolAddress: %s",
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t nvfp4_quantize_act_workspace_size(int64_t M, int64_t K) {
  if (M < 0 || K < 32) return 256;
  return act_plan(M, K, num_cus(), 0).bytes;
}

int nvfp4_quantize_act(const void* x, int64_t M, int64_t K, int64_t ldx, int glu,
                       uint8_t* codes, uint8_t* scales, float* g_x, uint64_t* score,
                       void* x_used, void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(g_x && ws, NVFP4_ERR_NULL, "nvfp4_quantize_act: g_x and ws are required");
  NV_REQUIRE(M >= 0 && K >= 32 && K % 32 == 0 && M < (1LL << 40), NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act: need M >= 0, K >= 32, K %% 32 == 0 (M=%lld K=%lld)",
             (long long)M, (long long)K);
  NV_REQUIRE(glu == 0 || glu == 1, NVFP4_ERR_SHAPE, "nvfp4_quantize_act: glu must be 0 or 1");
  NV_REQUIRE(ldx >= (glu ? 2 * K : K) && ldx % 8 == 0, NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act: bad ldx %lld", (long long)ldx);
  NV_REQUIRE(M == 0 || (x && codes && scales), NVFP4_ERR_NULL,
             "nvfp4_quantize_act: x, codes and scales are required");
  NV_REQUIRE(!glu || x_used, NVFP4_ERR_NULL, "nvfp4_quantize_act: glu=1 needs x_used for h");
  NV_REQUIRE(aligned(x, 16) && aligned(codes, 8) && aligned(scales, 4) && aligned(x_used, 16) &&
                 aligned(score, 8) && aligned(ws, 16),
             NVFP4_ERR_ALIGN, "nvfp4_quantize_act: misaligned pointer");
  const ActPlan pl = act_plan(M, K, num_cus(), 0);
  NV_REQUIRE(ws_bytes >= pl.bytes, NVFP4_ERR_WORKSPACE, "nvfp4_quantize_act: workspace too small");
  return act_quantize("nvfp4_quantize_act", x, M, K, ldx, glu, nullptr, codes, scales, g_x, score,
                      x_used, ws, pl, as_stream(stream));
}

int nvfp4_quantize_act_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx, int glu,
                               uint8_t* codes, uint8_t* scales, float* g_x, uint64_t* score,
                               void* x_used, void* stream) {
  NV_REQUIRE(g_x, NVFP4_ERR_NULL, "nvfp4_quantize_act_noalloc: g_x is required");
  NV_REQUIRE(M >= 0 && K >= 32 && K % 32 == 0 && M < (1LL << 40), NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act_noalloc: need M >= 0, K >= 32, K %% 32 == 0 (M=%lld K=%lld)",
             (long long)M, (long long)K);
  NV_REQUIRE(K <= kNoAllocMaxK, NVFP4_ERR_UNSUPPORTED,
             "nvfp4_quantize_act_noalloc: K=%lld exceeds %lld, the largest the fixed scratch "
             "takes; use nvfp4_quantize_act with a workspace",
             (long long)K, (long long)kNoAllocMaxK);
  NV_REQUIRE(glu == 0 || glu == 1, NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act_noalloc: glu must be 0 or 1");
  NV_REQUIRE(ldx >= (glu ? 2 * K : K) && ldx % 8 == 0, NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act_noalloc: bad ldx %lld", (long long)ldx);
  NV_REQUIRE(M == 0 || (x && codes && scales), NVFP4_ERR_NULL,
             "nvfp4_quantize_act_noalloc: x, codes and scales are required");
  NV_REQUIRE(!glu || x_used, NVFP4_ERR_NULL,
             "nvfp4_quantize_act_noalloc: glu=1 needs x_used for h");
  NV_REQUIRE(aligned(x, 16) && aligned(codes, 8) && aligned(scales, 4) && aligned(x_used, 16) &&
                 aligned(score, 8),
             NVFP4_ERR_ALIGN, "nvfp4_quantize_act_noalloc: misaligned pointer");
  const ActPlan pl = act_plan(M, K, num_cus(), kNoAllocScratchBytes - kAmaxSlots * 4);
  NV_REQUIRE(pl.bytes <= kNoAllocScratchBytes, NVFP4_ERR_UNSUPPORTED,
             "nvfp4_quantize_act_noalloc: needs %zu bytes of scratch, the fixed array holds %zu",
             pl.bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != NVFP4_OK) return st;
  return act_quantize("nvfp4_quantize_act_noalloc", x, M, K, ldx, glu, nullptr, codes, scales,
                      g_x, score, x_used, ws, pl, as_stream(stream));
}

int nvfp4_quantize_act_amax(const void* x, int64_t M, int64_t K, int64_t ldx,
                            const uint32_t* amax, uint8_t* codes, uint8_t* scales, float* g_x,
                            uint64_t* score, void* ws, size_t ws_bytes, void* stream) {
  NV_REQUIRE(g_x && ws && amax, NVFP4_ERR_NULL,
             "nvfp4_quantize_act_amax: g_x, amax and ws are required");
  NV_REQUIRE(M >= 0 && K >= 32 && K % 32 == 0 && ldx >= K && ldx % 8 == 0 && M < (1LL << 40),
             NVFP4_ERR_SHAPE,
             "nvfp4_quantize_act_amax: need M >= 0, K >= 32, K %% 32 == 0, ldx >= K, "
             "ldx %% 8 == 0 (M=%lld K=%lld)", (long long)M, (long long)K);
  NV_REQUIRE(M == 0 || (x && codes && scales), NVFP4_ERR_NULL,
             "nvfp4_quantize_act_amax: x, codes and scales are required");
  NV_REQUIRE(aligned(x, 16) && aligned(codes, 8) && aligned(scales, 4) && aligned(score, 8) &&
                 aligned(ws, 16) && aligned(amax, 4),
             NVFP4_ERR_ALIGN, "nvfp4_quantize_act_amax: misaligned pointer");
  const ActPlan pl = act_plan(M, K, num_cus(), 0);
  NV_REQUIRE(ws_bytes >= pl.bytes, NVFP4_ERR_WORKSPACE,
             "nvfp4_quantize_act_amax: workspace too small");
  return act_quantize("nvfp4_quantize_act_amax", x, M, K, ldx, 0, amax, codes, scales, g_x, score,
                      nullptr, ws, pl, as_stream(stream));
}

}  // extern "C"
