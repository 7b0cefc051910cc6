// Row-wise kernels of the decoder block: embedding gather, RMSNorm (fused with the
// deterministic split-K reduction and residual add of the decode projections), per-head
// q/k RMSNorm + rotate-half RoPE + BF16 KV write through the block table, and argmax.
//
// Kipp Model Support, "The registry": RMS epsilon 1e-6, head width 128, 8 KV heads.
// Kipp Model Support, "Validated results" (qwen3-0.6b-base): K and V are stored rounded to
// BF16. Kipp Roadmap, status v0.0.2: per-session 32-position block table.
#include "gqa_common.h"

namespace gqa {

// x[t][:] = fp32(E[ids[t]][:]). Out-of-range ids (possible only for device-resident ids)
// poison the row with NaN and set the model's error word.
__global__ void embed_kernel(const uint16_t* __restrict__ E, const int32_t* __restrict__ ids, int H, int vocab,
                             float* __restrict__ x, int32_t* __restrict__ err) {
  int t = blockIdx.x;
  int id = ids[t];
  float* xr = x + (int64_t)t * H;
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = __builtin_nanf("");
    return;
  }
  const uint16_t* er = E + (int64_t)id * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = bf16_bits_to_f32(er[i]);
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// One 256-thread block per row. If nsplit > 0: x[r] += part_scale * sum_{s < nsplit} part[s][r][:]
// (fixed order), written back. Then y = x / sqrt(mean(x^2) + eps) * w * out_scale, stored as FP16
// hi/lo pairs (yhi, ylo) for the next projection. H <= 4096 and H % 256 == 0.
__global__ __launch_bounds__(256) void rmsnorm_kernel(float* __restrict__ x, int ldx, const float* __restrict__ part,
                                                      int nsplit, int part_stride_split, int part_ld, float part_scale,
                                                      const uint16_t* __restrict__ w, int H, float eps,
                                                      float out_scale, f16* __restrict__ yhi,
                                                      f16* __restrict__ ylo, int ldy) {
  __shared__ float red[4];
  int r = blockIdx.x;
  float* xr = x + (int64_t)r * ldx;
  constexpr int kMaxPer = 16;
  float v[kMaxPer];
  int per = H / 256;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    if (j < per) {
      int i = threadIdx.x + 256 * j;
      float a = xr[i];
      if (nsplit > 0) {
        float acc = 0.f;
        for (int s = 0; s < nsplit; ++s) acc += part[(int64_t)s * part_stride_split + (int64_t)r * part_ld + i];
        a += acc * part_scale;
        xr[i] = a;
      }
      v[j] = a;
      ss += a * a;
    }
  }
  float tot = block_sum_256(ss, red);
  float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int j = 0; j < kMaxPer; ++j) {
    if (j < per) {
      int i = threadIdx.x + 256 * j;
      float y = v[j] * inv * bf16_bits_to_f32(w[i]) * out_scale;
      f16 hi, lo;
      split_f16(y, hi, lo);
      yhi[(int64_t)r * ldy + i] = hi;
      ylo[(int64_t)r * ldy + i] = lo;
    }
  }
}

// Residual reduction only (no norm): x[r] += sum_s part[s][r][:]. Used before the final norm
// when only the last row continues.
__global__ void residual_reduce_kernel(float* __restrict__ x, int ldx, const float* __restrict__ part, int nsplit,
                                       int part_stride_split, int part_ld, float part_scale, int H) {
  int r = blockIdx.x;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) acc += part[(int64_t)s * part_stride_split + (int64_t)r * part_ld + i];
    x[(int64_t)r * ldx + i] += acc * part_scale;
  }
}

// Per (row, head) wave: head h < nq is a query head, then 8 key heads, then 8 value heads of
// the fused q|k|v projection row. Lane l owns dims l and l+64 (a RoPE pair).
//   q, k: RMSNorm over the 128 dims with w_qn / w_kn, then rotate by the row's position.
//   k, v: rounded to BF16 and written to pool[phys][kvh][slot][128], phys = table[p >> 5].
//   q: written as FP32 to qout[row][h][128].
// Input: qkv[row][n] (prefill, nsplit == 0) or sum over s of part[s][row][n] (decode).
template <bool kDecode>
__global__ __launch_bounds__(256) void qk_rope_kv_kernel(const float* __restrict__ qkv, int nsplit, int part_stride,
                                                         int ldqkv, int nq, const uint16_t* __restrict__ wqn,
                                                         const uint16_t* __restrict__ wkn, float eps,
                                                         const float* __restrict__ rcos,
                                                         const float* __restrict__ rsin, int pos0,
                                                         const int32_t* __restrict__ table0, Rows rows,
                                                         uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
                                                         float* __restrict__ qout, int nrows) {
  int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  int nheads = nq + 2 * kKvHeads;
  int gidx = blockIdx.x * 4 + wave;
  int row = gidx / nheads, h = gidx % nheads;
  if (row >= nrows) return;
  int pos;
  const int32_t* table;
  if (kDecode) {
    pos = rows.pos[row];
    table = rows.table[row];
  } else {
    pos = pos0 + row;
    table = table0;
  }
  int64_t base = (int64_t)row * ldqkv + h * kHeadDim;
  float a, b;
  if (nsplit == 0) {
    a = qkv[base + l];
    b = qkv[base + l + 64];
  } else {
    a = 0.f;
    b = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      a += qkv[(int64_t)s * part_stride + base + l];
      b += qkv[(int64_t)s * part_stride + base + l + 64];
    }
  }
  bool isq = h < nq, isk = h >= nq && h < nq + kKvHeads;
  if (isq || isk) {
    float ss = wave_sum(a * a + b * b);
    float inv = 1.0f / sqrtf(ss / (float)kHeadDim + eps);
    const uint16_t* w = isq ? wqn : wkn;
    a = a * inv * bf16_bits_to_f32(w[l]);
    b = b * inv * bf16_bits_to_f32(w[l + 64]);
    float c = rcos[(int64_t)pos * 64 + l], s = rsin[(int64_t)pos * 64 + l];
    float ra = a * c - b * s;
    float rb = b * c + a * s;
    a = ra;
    b = rb;
  }
  if (isq) {
    float* qo = qout + ((int64_t)row * nq + h) * kHeadDim;
    qo[l] = a;
    qo[l + 64] = b;
  } else {
    int kvh = isk ? h - nq : h - nq - kKvHeads;
    int phys = table[pos >> 5];
    uint16_t* dst = (isk ? kpool : vpool) + (((int64_t)phys * kKvHeads + kvh) * kBlock + (pos & 31)) * kHeadDim;
    dst[l] = f32_to_bf16_rne(a);
    dst[l + 64] = f32_to_bf16_rne(b);
  }
}

// argmax over each row of logits [B][V]; ties go to the lowest index.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ logits, int64_t ld, int V,
                                                      int32_t* __restrict__ out) {
  __shared__ float sv[1024];
  __shared__ int si[1024];
  const float* r = logits + (int64_t)blockIdx.x * ld;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = threadIdx.x; i < V; i += 1024) {
    float v = r[i];
    if (v > best) {
      best = v;
      bi = i;
    }
  }
  sv[threadIdx.x] = best;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      float ov = sv[threadIdx.x + s];
      int oi = si[threadIdx.x + s];
      if (ov > sv[threadIdx.x] || (ov == sv[threadIdx.x] && oi < si[threadIdx.x])) {
        sv[threadIdx.x] = ov;
        si[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = si[0] == 0x7FFFFFFF ? -1 : si[0];
}

hipError_t launch_embed(const uint16_t* E, const int32_t* ids, int T, int H, int vocab, float* x, int32_t* err,
                        hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(256), 0, st, E, ids, H, vocab, x, err);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(float* x, int ldx, const float* part, int nsplit, int part_stride_split, int part_ld,
                          float part_scale, const uint16_t* w, int H, float eps, float out_scale, f16* yhi, f16* ylo,
                          int ldy, int rows, hipStream_t st) {
  if (H % 256 != 0 || H > 4096) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, st, x, ldx, part, nsplit, part_stride_split, part_ld,
                     part_scale, w, H, eps, out_scale, yhi, ylo, ldy);
  return hipGetLastError();
}

hipError_t launch_residual_reduce(float* x, int ldx, const float* part, int nsplit, int part_stride_split,
                                  int part_ld, float part_scale, int H, int rows, hipStream_t st) {
  hipLaunchKernelGGL(residual_reduce_kernel, dim3(rows), dim3(256), 0, st, x, ldx, part, nsplit, part_stride_split,
                     part_ld, part_scale, H);
  return hipGetLastError();
}

hipError_t launch_qk_rope_kv(bool decode, const float* qkv, int nsplit, int part_stride, int ldqkv, int nq,
                             const uint16_t* wqn, const uint16_t* wkn, float eps, const float* rcos,
                             const float* rsin, int pos0, const int32_t* table0, const Rows& rows,
                             uint16_t* kpool, uint16_t* vpool, float* qout, int nrows, hipStream_t st) {
  int nheads = nq + 2 * kKvHeads;
  int waves = nrows * nheads;
  dim3 grid((waves + 3) / 4);
  if (decode)
    hipLaunchKernelGGL(qk_rope_kv_kernel<true>, grid, dim3(256), 0, st, qkv, nsplit, part_stride, ldqkv, nq, wqn,
                       wkn, eps, rcos, rsin, pos0, table0, rows, kpool, vpool, qout, nrows);
  else
    hipLaunchKernelGGL(qk_rope_kv_kernel<false>, grid, dim3(256), 0, st, qkv, nsplit, part_stride, ldqkv, nq, wqn,
                       wkn, eps, rcos, rsin, pos0, table0, rows, kpool, vpool, qout, nrows);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int64_t ld, int V, int B, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, st, logits, ld, V, out);
  return hipGetLastError();
}

}  // namespace gqa
