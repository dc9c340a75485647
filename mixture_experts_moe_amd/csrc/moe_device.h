// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Saturate to the E4M3 finite range; NaN passes through (comparisons are false).
__device__ __forceinline__ float sat448(float v) { return v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v); }

// Four fp32 values -> four OCP E4M3 codes (round to nearest even) packed
// little-endian into one word: byte i holds the code of value i.
// x combined with the x of lane ^ 16 (or lane ^ 32) through gfx950's lane-swap
// instructions (v_permlane16_swap / v_permlane32_swap: a register swaps its odd
// 16-lane rows, or its upper 32 lanes, with another's), instead of an LDS
// permute.  Called with the value in both operands, the two results hold, in
// every lane, x of the lane and of its partner (in either order); max and sum
// are commutative, so the result is bitwise that of op(x, shfl_xor(x, 16/32)).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return (uint32_t)w;
}
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false) & 0xffffu;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// SwiGLU's silu(g) = g / (1 + e^-g) in fp32 from the hardware base-2
// exponential and reciprocal (about 1 ulp each; e^-g = 2^(-g log2 e)): a few
// fp32 ulps of relative error, far below the step of the E4M3 or bf16 h that
// follows, and about a fifth of the instructions of the library exponential
// and the correctly rounded division.  Large |g|: 2^(big) = inf gives 0 for
// very negative g, 2^(-big) = 0 gives g.
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}

// A compile-time integer as a value (register-slot and run selectors).
template <int N>
struct Ic {
  static constexpr int value = N;
};

// Maximum of an unsigned value over the 64 lanes of a wave, returned to every
// lane.  DPP row shifts build each 16-lane row's maximum in its lane 15, two
// row broadcasts carry it to lane 63, and readlane returns it; lanes whose DPP
// source is out of range read 0, the identity of an unsigned maximum.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
#define MOE_DPP_MAX(ctrl, rmask, bmask) \
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, (ctrl), (rmask), (bmask), false))
  MOE_DPP_MAX(0x111, 0xf, 0xf);  // row_shr:1
  MOE_DPP_MAX(0x112, 0xf, 0xf);  // row_shr:2
  MOE_DPP_MAX(0x113, 0xf, 0xf);  // row_shr:3
  MOE_DPP_MAX(0x114, 0xf, 0xe);  // row_shr:4, banks 1-3
  MOE_DPP_MAX(0x118, 0xf, 0xc);  // row_shr:8, banks 2-3
  MOE_DPP_MAX(0x142, 0xa, 0xf);  // row_bcast:15 into rows 1 and 3
  MOE_DPP_MAX(0x143, 0xc, 0xf);  // row_bcast:31 into rows 2 and 3
#undef MOE_DPP_MAX
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, <= 1024);
// `tmp` holds 17 ints of LDS.  Returns the thread's exclusive prefix; *total
// receives the block sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < NW ? tmp[lane] : 0;
    int wi = wave_incl_scan(w);
    if (lane < NW) tmp[lane] = wi - w;
    if (lane == NW - 1) tmp[16] = wi;
  }
  __syncthreads();
  int r = inc - v + tmp[wave];
  *total = tmp[16];
  __syncthreads();
  return r;
}

// Exclusive prefix sum over a block of 1024 threads; `tmp` holds 17 ints of LDS.
// Returns the thread's exclusive prefix; *total receives the block sum.
__device__ __forceinline__ int block1024_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? tmp[lane] : 0;
    int wi = wave_incl_scan(w);
    if (lane < 16) tmp[lane] = wi - w;
    if (lane == 15) tmp[16] = wi;
  }
  __syncthreads();
  int r = inc - v + tmp[wave];
  *total = tmp[16];
  __syncthreads();
  return r;
}

// 16 E4M3 codes (bytes 0..15 of `in`) -> 16 bf16 values, exactly (every E4M3
// value is a bf16 value): lo = bytes 0..7, hi = bytes 8..15, in order.
__device__ __forceinline__ void e4m3x16_to_bf16(v4i in, v4i& lo, v4i& hi) {
#define MOE_CVT2(w, sel) __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), 1.0f, (sel)))
  lo = v4i{MOE_CVT2(in[0], false), MOE_CVT2(in[0], true), MOE_CVT2(in[1], false), MOE_CVT2(in[1], true)};
  hi = v4i{MOE_CVT2(in[2], false), MOE_CVT2(in[2], true), MOE_CVT2(in[3], false), MOE_CVT2(in[3], true)};
#undef MOE_CVT2
}

// One 128-deep K block of E4M3 codes, product accumulated at fp32 precision:
// the 32 codes per lane of each operand (two 16-byte halves) are decoded to bf16
// and fed to four chained 16x16x32 bf16 products.  The E4M3 matrix-core product
// (v_mfma_f32_16x16x128_f8f6f4) truncates its internal sum on gfx950 (measured:
// about 1e-4 of the summed magnitudes, against 3e-7 for fp32), which is enough to
// flip re-quantised h codes; the bf16 products of the decoded codes are exact and
// accumulate like fp32 (measured 2.6e-7).  Lane l's slot j of operand i
// holds the same K index for A and B, so the product is the K-block dot product
// whatever K order the hardware assigns to the slots.
__device__ __forceinline__ v4f kblock_e4m3_exact(v4i alo, v4i ahi, const v4i (&b)[4]) {
  v4i a0, a1, a2, a3;
  e4m3x16_to_bf16(alo, a0, a1);
  e4m3x16_to_bf16(ahi, a2, a3);
  v4f p = {0.f, 0.f, 0.f, 0.f};
  p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a0), __builtin_bit_cast(v8bf, b[0]), p, 0, 0, 0);
  p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a1), __builtin_bit_cast(v8bf, b[1]), p, 0, 0, 0);
  p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a2), __builtin_bit_cast(v8bf, b[2]), p, 0, 0, 0);
  p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a3), __builtin_bit_cast(v8bf, b[3]), p, 0, 0, 0);
  return p;
}

// The same product split in two: the weight codes decoded once (a[4]), then
// the four chained products against one row chunk's operands -- for tiles of
// several row chunks, which would otherwise decode the same codes per chunk.
__device__ __forceinline__ void kblock_decode(v4i alo, v4i ahi, v4i (&a)[4]) {
  e4m3x16_to_bf16(alo, a[0], a[1]);
  e4m3x16_to_bf16(ahi, a[2], a[3]);
}
__device__ __forceinline__ v4f kblock_bf16(const v4i (&a)[4], const v4i (&b)[4]) {
  v4f p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[i]), __builtin_bit_cast(v8bf, b[i]), p, 0, 0,
                                                0);
  return p;
}

// 16x16x32 bf16 matrix-core product accumulated into c.
__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

}  // namespace moe
