// Shared device helpers of the gfx950 decoder library: number formats, MFMA operand types,
// wave reductions and the launch-error plumbing used by every kernel file.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace gqa {

constexpr int kHeadDim = 128;
constexpr int kKvHeads = 8;
constexpr int kBlock = 32;          // positions per KV block
constexpr int kMaxBatch = 32;       // rows of one batched decode
constexpr float kLog2e = 1.4426950408889634f;

// Epilogues of the projection kernels.
enum Epi : int { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };

// Per-row addressing of a batched decode call: position of the new token and the
// session's block table (logical block -> physical block).
struct Rows {
  int32_t pos[kMaxBatch];
  const int32_t* table[kMaxBatch];
};

// Source of the FP16 hi/lo operand rows of a decode matvec (see k_gemv.hip).
enum XMode : int { X_RAW = 0, X_RESID = 1, X_SWIGLU = 2 };
struct XSrc {
  int mode;
  // X_RAW: hi/lo rows in global memory, row stride ld
  const f16* hi;
  const f16* lo;
  int ld;
  // X_RESID: x = res[b] + pscale * sum_{s < nsplit} part[s][b] (fixed split order);
  // operand = x * w (the RMSNorm weight; the 1/rms factor is applied by the consumer of the
  // projection). x is written to res_out and the sum of squares of x over each K range to
  // ss_out[range][b] by the workgroups of the first row tile.
  const float* res;
  float* res_out;
  const float* part;
  int nsplit;
  int64_t pstride;
  int pld;
  float pscale;
  const uint16_t* w;
  float* ss_out;
  // X_SWIGLU: c = 1 / sqrt(sum_r ss[r][b] / H + eps); g = c * sum_s gu[s][b][32*(f/16) + f%16],
  // u = c * sum_s gu[s][b][32*(f/16) + 16 + f%16]; operand = silu(g) * u.
  const float* gu;
  int gu_split;
  int64_t gu_stride;
  int gu_ld;
  const float* ss;
  int ss_n;
  int H;
  float eps;
};

// Sum-of-squares partials: ss[range][row], kMaxBatch rows per range.
__device__ __forceinline__ float inv_rms_from_ss(const float* ss, int n, int row, int H, float eps) {
  float t = 0.f;
  for (int r = 0; r < n; ++r) t += ss[r * 32 + row];
  return 1.0f / sqrtf(t / (float)H + eps);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even; the values handled here are finite.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Eight BF16 weights (one 16-byte load) -> eight FP16 MFMA operands. BF16 has 8 significant
// bits, so the conversion is exact for |w| in [2^-17, 65504]; smaller magnitudes lose at most
// 2^-25 absolutely.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(uint4 v) {
  f16x8 r;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (f16)__uint_as_float(w[i] << 16);
    r[2 * i + 1] = (f16)__uint_as_float(w[i] & 0xFFFF0000u);
  }
  return r;
}

// Split an FP32 value into FP16 hi + lo with x = hi + lo up to 2^-22 relative (2^-25 absolute
// near zero). Two FP16 MFMAs over (hi, lo) give a near-FP32 product with BF16/FP16 weights.
__device__ __forceinline__ void split_f16(float x, f16& hi, f16& lo) {
  hi = (f16)x;
  lo = (f16)(x - (float)hi);
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace gqa
