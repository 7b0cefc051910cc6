// Seeded synthetic weights generated on the device, and the Q8_0 quantiser.
//
// Generator: element i of the logical row-major [rows][cols] tensor with key `key` takes
// u = SplitMix64 finaliser of (key + (i+1) * 0x9E3779B97F4A7C15) (Steele, Lea and Flood,
// OOPSLA 2014), S = sum of the four 16-bit fields of u, z = S - 131070, and
// w = bf16_rne(fp32(z) * scale) with one FP32 multiply. The value lands at the physical row
// given by the layout mode (plain with a row offset, or the 16-row gate/up interleave), stored
// tile-major (tiled_index).
//
// Q8_0 (Kipp Model Support, "Quantization (Q8_0)"): 32-weight blocks along a row, an fp16
// scale and 32 int8 quants (stored here as a tile-major int8 matrix plus a scale array indexed by
// tiled_scale_index). d = amax / 127 (FP32 division), scale = fp16_rne(d),
// q = clamp(round_half_away(w / d), -127, 127), and q = 0 when d = 0.
//
// AFFINE4_GS32 (Kipp Model Support, "Quantization (AFFINE4_GS32)"): 32-weight groups along a row
// of 4-bit codes with an fp16 scale and an fp16 bias, w = scale * q + bias. d = (max - min) / 15
// (FP32), scale = fp16_rne(d), bias = fp16_rne(min), q = clamp(round_half_away((w - bias) /
// scale), 0, 15) from the stored scale and bias in FP32, q = 0 when the scale is 0. Codes are
// stored tile-major like the BF16 weights at half a byte each: the 8 codes an operand lane reads
// (tiled_index positions 8 i .. 8 i + 7) form the 32-bit word i, element 2 j in nibble j and
// element 2 j + 1 in nibble j + 4; scales and biases at tiled_scale_index.
#include "gqa_common.h"

namespace gqa {

__device__ __forceinline__ uint64_t splitmix_at(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// mode 0: physical row = row_off + r. mode 1: gate rows of the interleave (32*(r/16) + r%16);
// mode 2: up rows (32*(r/16) + 16 + r%16).
__global__ void gen_weights_kernel(uint16_t* __restrict__ dst, uint64_t key, int64_t rows, int64_t cols,
                                   int mode, int64_t row_off, float scale) {
  int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    uint64_t u = splitmix_at(key, (uint64_t)i);
    int64_t s = (int64_t)(u & 0xFFFF) + (int64_t)((u >> 16) & 0xFFFF) + (int64_t)((u >> 32) & 0xFFFF) +
                (int64_t)(u >> 48);
    float z = (float)(int32_t)(s - 131070);
    float w = __fmul_rn(z, scale);
    int64_t r = i / cols, c = i - r * cols;
    int64_t pr = mode == 0 ? row_off + r : (mode == 1 ? 32 * (r / 16) + (r % 16) : 32 * (r / 16) + 16 + (r % 16));
    dst[tiled_index(pr, c, cols)] = f32_to_bf16_rne(w);
  }
}

__global__ void fill_u16_kernel(uint16_t* __restrict__ dst, int64_t n, uint16_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = v;
}

// One thread per 32-weight block (row, blk) of a tile-major BF16 matrix [rows][cols] -> the
// tile-major int8 quants at the same element positions and the scale at tiled_scale_index.
__global__ void quantize_q8_0_kernel(const uint16_t* __restrict__ w, int8_t* __restrict__ q, f16* __restrict__ d,
                                     int64_t rows, int64_t cols) {
  int64_t nb = rows * (cols / 32);
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = b / (cols / 32), blk = b - row * (cols / 32);
    int64_t at[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) at[g] = tiled_index(row, blk * 32 + g * 8, cols);   // 8 contiguous columns each
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = bf16_bits_to_f32(w[at[i / 8] + i % 8]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    float dd = __fdiv_rn(amax, 127.0f);
    d[tiled_scale_index(row, blk, cols)] = (f16)dd;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float r = dd == 0.f ? 0.f : __fdiv_rn(v[i], dd);
      float qi = roundf(r);                      // half away from zero
      qi = fminf(fmaxf(qi, -127.f), 127.f);
      q[at[i / 8] + i % 8] = (int8_t)(int)qi;
    }
  }
}

// One thread per 32-weight group (row, blk) of a tile-major BF16 matrix [rows][cols].
__global__ void quantize_affine4_kernel(const uint16_t* __restrict__ w, uint32_t* __restrict__ q4,
                                        f16* __restrict__ d, f16* __restrict__ bias, int64_t rows, int64_t cols) {
  int64_t nb = rows * (cols / 32);
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = b / (cols / 32), blk = b - row * (cols / 32);
    int64_t at[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) at[g] = tiled_index(row, blk * 32 + g * 8, cols);   // 8 contiguous columns each
    float v[32];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = bf16_bits_to_f32(w[at[i / 8] + i % 8]);
      mn = fminf(mn, v[i]);
      mx = fmaxf(mx, v[i]);
    }
    const f16 sd = (f16)__fdiv_rn(__fsub_rn(mx, mn), 15.0f), sb = (f16)mn;
    d[tiled_scale_index(row, blk, cols)] = sd;
    bias[tiled_scale_index(row, blk, cols)] = sb;
    const float D = (float)sd, Bv = (float)sb;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float r = D == 0.f ? 0.f : __fdiv_rn(__fsub_rn(v[g * 8 + e], Bv), D);
        const float qf = fminf(fmaxf(roundf(r), 0.f), 15.f);   // half away from zero
        word |= (uint32_t)(int)qf << (4 * ((e & 1) * 4 + (e >> 1)));
      }
      q4[at[g] / 8] = word;
    }
  }
}

// FP16 prefill copy (prefill_weight_index) of a tile-major AFFINE4 matrix: one thread per
// 8-element piece, w = fp16_rne(fmaf(scale, q, bias)) (the prefill GEMM's operand).
__global__ void prefill_copy_affine4_kernel(const uint32_t* __restrict__ q4, const f16* __restrict__ d,
                                            const f16* __restrict__ bias, f16* __restrict__ dst, int64_t rows,
                                            int64_t cols) {
  const int64_t npieces = rows * cols / 8, ksteps = cols >> 5;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < npieces; p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bp = p >> 7, pos = p & 127;
    const int64_t row = (bp / ksteps) * 32 + (pos & 31);
    const int64_t col = (bp % ksteps) * 32 + ((pos >> 6) & 1) * 16 + ((pos >> 5) & 1) * 8;
    const uint32_t word = q4[tiled_index(row, col, cols) / 8];
    const float D = (float)d[tiled_scale_index(row, col >> 5, cols)];
    const float Bv = (float)bias[tiled_scale_index(row, col >> 5, cols)];
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = (float)((word >> (4 * ((e & 1) * 4 + (e >> 1)))) & 15u);
      o[e] = (f16)fmaf(D, q, Bv);
    }
    *(f16x8*)(dst + p * 8) = o;
  }
}

// FP16 prefill copy (prefill_weight_index) of a tile-major Q8_0 matrix: one thread per 8-element
// piece, w = fp16_rne(scale * q) (the product is exact in FP32; one FP16 rounding).
__global__ void prefill_copy_q8_kernel(const int8_t* __restrict__ q, const f16* __restrict__ d, f16* __restrict__ dst,
                                       int64_t rows, int64_t cols) {
  const int64_t npieces = rows * cols / 8, ksteps = cols >> 5;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < npieces; p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bp = p >> 7, pos = p & 127;
    const int64_t row = (bp / ksteps) * 32 + (pos & 31);
    const int64_t col = (bp % ksteps) * 32 + ((pos >> 6) & 1) * 16 + ((pos >> 5) & 1) * 8;
    const int8_t* src = q + tiled_index(row, col, cols);
    const float D = (float)d[tiled_scale_index(row, col >> 5, cols)];
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (f16)(D * (float)src[e]);
    *(f16x8*)(dst + p * 8) = o;
  }
}

hipError_t launch_prefill_copy_q8(const int8_t* q, const f16* d, f16* dst, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t n = rows * cols / 8;
  const int grid = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(prefill_copy_q8_kernel, dim3(grid), dim3(256), 0, st, q, d, dst, rows, cols);
  return hipGetLastError();
}

// FP16 prefill copy (prefill_weight_index) of a tile-major BF16 matrix: one thread per 8-element
// piece of the destination, converted exactly like the matrix-core operand path (bf16x8_to_f16x8).
__global__ void prefill_copy_kernel(const uint16_t* __restrict__ src, f16* __restrict__ dst, int64_t rows,
                                    int64_t cols) {
  const int64_t npieces = rows * cols / 8, ksteps = cols >> 5;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < npieces; p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bp = p >> 7, pos = p & 127;
    const int64_t row = (bp / ksteps) * 32 + (pos & 31);
    const int64_t col = (bp % ksteps) * 32 + ((pos >> 6) & 1) * 16 + ((pos >> 5) & 1) * 8;
    const uint4 v = *(const uint4*)(src + tiled_index(row, col, cols));
    *(f16x8*)(dst + p * 8) = bf16x8_to_f16x8(v);
  }
}

hipError_t launch_prefill_copy(const uint16_t* src, f16* dst, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t n = rows * cols / 8;
  const int grid = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(prefill_copy_kernel, dim3(grid), dim3(256), 0, st, src, dst, rows, cols);
  return hipGetLastError();
}

hipError_t launch_quantize_affine4(const uint16_t* w, uint8_t* q4, f16* d, f16* bias, int64_t rows, int64_t cols,
                                  hipStream_t st) {
  int64_t nb = rows * (cols / 32);
  int grid = (int)std::min<int64_t>((nb + 255) / 256, 65536);
  hipLaunchKernelGGL(quantize_affine4_kernel, dim3(grid), dim3(256), 0, st, w, (uint32_t*)q4, d, bias, rows, cols);
  return hipGetLastError();
}

hipError_t launch_prefill_copy_affine4(const uint8_t* q4, const f16* d, const f16* bias, f16* dst, int64_t rows,
                                       int64_t cols, hipStream_t st) {
  const int64_t n = rows * cols / 8;
  const int grid = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(prefill_copy_affine4_kernel, dim3(grid), dim3(256), 0, st, (const uint32_t*)q4, d, bias, dst, rows,
                     cols);
  return hipGetLastError();
}

hipError_t launch_gen_weights(uint16_t* dst, uint64_t key, int64_t rows, int64_t cols, int mode, int64_t row_off,
                              float scale, hipStream_t st) {
  int64_t n = rows * cols;
  int grid = (int)std::min<int64_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(gen_weights_kernel, dim3(grid), dim3(256), 0, st, dst, key, rows, cols, mode, row_off, scale);
  return hipGetLastError();
}

hipError_t launch_fill_u16(uint16_t* dst, int64_t n, uint16_t v, hipStream_t st) {
  int grid = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_u16_kernel, dim3(grid), dim3(256), 0, st, dst, n, v);
  return hipGetLastError();
}

hipError_t launch_quantize_q8_0(const uint16_t* w, int8_t* q, f16* d, int64_t rows, int64_t cols, hipStream_t st) {
  int64_t nb = rows * (cols / 32);
  int grid = (int)std::min<int64_t>((nb + 255) / 256, 65536);
  hipLaunchKernelGGL(quantize_q8_0_kernel, dim3(grid), dim3(256), 0, st, w, q, d, rows, cols);
  return hipGetLastError();
}

}  // namespace gqa
