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
// poison the row with NaN and set the model's error word. Workgroup 0 also clears `zero`
// (nzero ints, e.g. the decode attention's arrival counters of a static scratch).
__global__ void embed_kernel(const uint16_t* __restrict__ E, const int32_t* __restrict__ ids, int H, int vocab,
                             float* __restrict__ x, int32_t* __restrict__ err, int32_t* __restrict__ zero, int nzero) {
  int t = blockIdx.x;
  if (t == 0)
    for (int i = threadIdx.x; i < nzero; i += blockDim.x) zero[i] = 0;
  int id = ids[t];
  float* xr = x + (int64_t)t * H;
  if (id < 0 || id >= vocab) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = __builtin_nanf("");
    return;
  }
  // the embedding is tile-major (tiled_index): 8 consecutive columns are one 16-byte piece
  for (int i = threadIdx.x * 8; i < H; i += blockDim.x * 8) {
    const uint4 v = *(const uint4*)(E + tiled_index(id, i, H));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float4 a, b;
    a.x = bf16_bits_to_f32(w[0] & 0xFFFF); a.y = bf16_bits_to_f32(w[0] >> 16);
    a.z = bf16_bits_to_f32(w[1] & 0xFFFF); a.w = bf16_bits_to_f32(w[1] >> 16);
    b.x = bf16_bits_to_f32(w[2] & 0xFFFF); b.y = bf16_bits_to_f32(w[2] >> 16);
    b.z = bf16_bits_to_f32(w[3] & 0xFFFF); b.w = bf16_bits_to_f32(w[3] >> 16);
    *(float4*)(xr + i) = a;
    *(float4*)(xr + i + 4) = b;
  }
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

// One block of H/4 threads per row (one float4 each; H % 256 == 0, H <= 4096). If NS > 0:
// x[r] += part_scale * sum_{s < NS} part[s][r][:] (fixed order), written back. Then
// y = x / sqrt(mean(x^2) + eps) * w * out_scale, stored as FP16 hi/lo pairs (yhi, ylo) for the
// next projection. Every load of a thread is issued before any is used.
template <int NS>
__global__ __launch_bounds__(1024) void rmsnorm_kernel(float* __restrict__ x, int ldx, const float* __restrict__ part,
                                                       int part_stride_split, int part_ld, float part_scale,
                                                       const uint16_t* __restrict__ w, int H, float eps,
                                                       float out_scale, f16* __restrict__ yhi,
                                                       f16* __restrict__ ylo, int ldy) {
  __shared__ float red[16];
  const int r = blockIdx.x, t = threadIdx.x, i = 4 * t;
  float* xr = x + (int64_t)r * ldx;
  float4 v = *(const float4*)(xr + i);
  float4 pv[NS > 0 ? NS : 1];
#pragma unroll
  for (int s = 0; s < NS; ++s) pv[s] = *(const float4*)(part + (int64_t)s * part_stride_split + (int64_t)r * part_ld + i);
  const uint2 wb = *(const uint2*)(w + i);
  if (NS > 0) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc.x += pv[s].x;
      acc.y += pv[s].y;
      acc.z += pv[s].z;
      acc.w += pv[s].w;
    }
    v.x += acc.x * part_scale;
    v.y += acc.y * part_scale;
    v.z += acc.z * part_scale;
    v.w += acc.w * part_scale;
    *(float4*)(xr + i) = v;
  }
  float ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  ss = wave_sum(ss);
  const int nw = blockDim.x >> 6;
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int k = 0; k < nw; ++k) tot += red[k];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  const float y[4] = {v.x * inv * bf16_bits_to_f32(wb.x & 0xFFFF) * out_scale,
                      v.y * inv * bf16_bits_to_f32(wb.x >> 16) * out_scale,
                      v.z * inv * bf16_bits_to_f32(wb.y & 0xFFFF) * out_scale,
                      v.w * inv * bf16_bits_to_f32(wb.y >> 16) * out_scale};
  f16x4 hv, lv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f16 h, l;
    split_f16(y[e], h, l);
    hv[e] = h;
    lv[e] = l;
  }
  *(f16x4*)(yhi + (int64_t)r * ldy + i) = hv;
  *(f16x4*)(ylo + (int64_t)r * ldy + i) = lv;
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
                                                         KvQ8 kq8, float* __restrict__ qout, int nrows) {
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
    float pa[8], pb[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      pa[s] = s < nsplit ? qkv[(int64_t)s * part_stride + base + l] : 0.f;
      pb[s] = s < nsplit ? qkv[(int64_t)s * part_stride + base + l + 64] : 0.f;
    }
    a = 0.f;
    b = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      a += pa[s];
      b += pb[s];
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
    const int64_t off = (((int64_t)phys * kKvHeads + kvh) * kBlock + (pos & 31)) * kHeadDim;
    if (kq8.kq) {
      // Q8_0 row: lane l holds dims l (block l / 32) and l + 64 (block 2 + l / 32); the block
      // maxima are taken over each half of the wave. Attention reads the codes and scales.
      float ma = fabsf(a), mb = fabsf(b);
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) {
        ma = fmaxf(ma, __shfl_xor(ma, m));
        mb = fmaxf(mb, __shfl_xor(mb, m));
      }
      const float da = q8kv_scale(ma), db = q8kv_scale(mb);
      const f16 sa = (f16)da, sb = (f16)db;
      const int ca = q8kv_code(a, da), cb = q8kv_code(b, db);
      int8_t* cq = (isk ? kq8.kq : kq8.vq) + off;
      cq[l] = (int8_t)ca;
      cq[l + 64] = (int8_t)cb;
      if ((l & 31) == 0) {
        f16* sc = (isk ? kq8.ks : kq8.vs) + (off >> 5);
        sc[l >> 5] = sa;
        sc[2 + (l >> 5)] = sb;
      }
    } else {
      uint16_t* dst = (isk ? kpool : vpool) + off;
      dst[l] = f32_to_bf16_rne(a);
      dst[l + 64] = f32_to_bf16_rne(b);
    }
  }
}

// argmax of each token row from the lm_head matvec's per-tile candidates cand[b][t] =
// (max value, index bits); ties go to the lowest index.
__global__ __launch_bounds__(1024) void argmax_kernel(const float2* __restrict__ cand, int ntiles,
                                                      int32_t* __restrict__ out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const float2* c = cand + (int64_t)blockIdx.x * ntiles;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = threadIdx.x; i < ntiles; i += 1024 * 4) {
    float2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = i + 1024 * u < ntiles ? c[i + 1024 * u] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int idx = __float_as_int(v[u].y);
      if (v[u].x > best || (v[u].x == best && idx < bi)) {
        best = v[u].x;
        bi = idx;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(best, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) {
      best = ov;
      bi = oi;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = best;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    best = sv[0];
    bi = si[0];
    for (int k = 1; k < 16; ++k)
      if (sv[k] > best || (sv[k] == best && si[k] < bi)) {
        best = sv[k];
        bi = si[k];
      }
    out[blockIdx.x] = bi == 0x7FFFFFFF ? -1 : bi;
  }
}

hipError_t launch_embed(const uint16_t* E, const int32_t* ids, int T, int H, int vocab, float* x, int32_t* err,
                        hipStream_t st, int32_t* zero, int nzero) {
  if (nzero < 0 || (nzero > 0 && !zero)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(256), 0, st, E, ids, H, vocab, x, err, zero, nzero);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(float* x, int ldx, const float* part, int nsplit, int part_stride_split, int part_ld,
                          float part_scale, const uint16_t* w, int H, float eps, float out_scale, f16* yhi, f16* ylo,
                          int ldy, int rows, hipStream_t st) {
  if (H % 256 != 0 || H > 4096) return hipErrorInvalidValue;
#define RMS_CASE(NS)                                                                                              \
  case NS:                                                                                                        \
    hipLaunchKernelGGL(rmsnorm_kernel<NS>, dim3(rows), dim3(H / 4), 0, st, x, ldx, part, part_stride_split, part_ld, \
                       part_scale, w, H, eps, out_scale, yhi, ylo, ldy);                                         \
    break;
  switch (nsplit) {
    RMS_CASE(0) RMS_CASE(1) RMS_CASE(2) RMS_CASE(3) RMS_CASE(4) RMS_CASE(5) RMS_CASE(6) RMS_CASE(7) RMS_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef RMS_CASE
  return hipGetLastError();
}

hipError_t launch_qk_rope_kv(bool decode, const float* qkv, int nsplit, int part_stride, int ldqkv, int nq,
                             const uint16_t* wqn, const uint16_t* wkn, float eps, const float* rcos,
                             const float* rsin, int pos0, const int32_t* table0, const Rows& rows,
                             uint16_t* kpool, uint16_t* vpool, const KvQ8& kq8, float* qout, int nrows,
                             hipStream_t st) {
  int nheads = nq + 2 * kKvHeads;
  int waves = nrows * nheads;
  dim3 grid((waves + 3) / 4);
  if (decode)
    hipLaunchKernelGGL(qk_rope_kv_kernel<true>, grid, dim3(256), 0, st, qkv, nsplit, part_stride, ldqkv, nq, wqn,
                       wkn, eps, rcos, rsin, pos0, table0, rows, kpool, vpool, kq8, qout, nrows);
  else
    hipLaunchKernelGGL(qk_rope_kv_kernel<false>, grid, dim3(256), 0, st, qkv, nsplit, part_stride, ldqkv, nq, wqn,
                       wkn, eps, rcos, rsin, pos0, table0, rows, kpool, vpool, kq8, qout, nrows);
  return hipGetLastError();
}

// Log-probability of a given next token from a row of logits (Kipp Roadmap, status v0.0.3:
// multi-row scoring): out[b] = l[t] - (m + log sum_v exp(l[v] - m)), m = max_v l[v], t =
// targets[b]. One 1024-thread workgroup per row; every sum and max in a fixed order (thread
// strides, then the 64 lanes, then the 16 waves in order), in FP32.
__global__ __launch_bounds__(1024) void score_kernel(const float* __restrict__ logits, int V,
                                                    const int32_t* __restrict__ targets, float* __restrict__ out) {
  __shared__ float red[16];
  const float* l = logits + (int64_t)blockIdx.x * V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < V; i += 1024) mx = fmaxf(mx, l[i]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float sum = 0.f;
  for (int i = threadIdx.x; i < V; i += 1024) sum += expf(l[i] - mx);
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) tot += red[w];
    out[blockIdx.x] = l[targets[blockIdx.x]] - (mx + logf(tot));
  }
}

hipError_t launch_score(const float* logits, int V, const int32_t* targets, int B, float* out, hipStream_t st) {
  if (B < 1) return hipSuccess;
  hipLaunchKernelGGL(score_kernel, dim3(B), dim3(1024), 0, st, logits, V, targets, out);
  return hipGetLastError();
}

// SwiGLU of prefill rows from the split-K partials of the fused gate|up matvec, whose output
// interleaves 16 gate and 16 up rows: m[t][f] = silu(g) * u, g and u summed over the splits in
// order, stored as FP16 hi/lo. grid (ceil(F / 256), rows).
__global__ __launch_bounds__(256) void swiglu_rows_kernel(const float* __restrict__ gu, int nsplit, int64_t stride,
                                                          int ldgu, int F, f16* __restrict__ mh,
                                                          f16* __restrict__ ml, int ldm) {
  const int t = blockIdx.y, f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const int64_t rg = (int64_t)t * ldgu + 32 * (f / 16) + (f % 16);
  float g = 0.f, u = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    g += gu[s * stride + rg];
    u += gu[s * stride + rg + 16];
  }
  const float m = __fmul_rn(__fdiv_rn(g, 1.0f + expf(-g)), u);
  f16 h, l;
  split_f16(m, h, l);
  mh[(int64_t)t * ldm + f] = h;
  ml[(int64_t)t * ldm + f] = l;
}

hipError_t launch_swiglu_rows(const float* gu, int nsplit, int64_t stride, int ldgu, int F, int rows, f16* mh, f16* ml,
                              int ldm, hipStream_t st) {
  if (rows < 1 || nsplit < 1 || F % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(swiglu_rows_kernel, dim3((F + 255) / 256, rows), dim3(256), 0, st, gu, nsplit, stride, ldgu, F,
                     mh, ml, ldm);
  return hipGetLastError();
}

// Entries of a pooled session's block table. The values travel as kernel arguments, so they are
// fixed at launch and stream-ordered with the evaluation that reads them.
__global__ __launch_bounds__(64) void table_write_kernel(int32_t* __restrict__ table, TableWrites t) {
  const int i = threadIdx.x;
  if (i < t.n) table[t.idx[i]] = t.val[i];
}

hipError_t launch_table_writes(int32_t* table, const TableWrites& t, hipStream_t st) {
  if (t.n < 1) return hipSuccess;
  if (t.n > kTableWritesMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(64), 0, st, table, t);
  return hipGetLastError();
}

// argmax of each of `rows` logit rows (row stride ld) read in full; ties go to the lowest index,
// and a row with no value above -inf (all NaN) gives -1.
__global__ __launch_bounds__(1024) void argmax_rows_kernel(const float* __restrict__ logits, int V, int64_t ld,
                                                           int32_t* __restrict__ out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const float* l = logits + (int64_t)blockIdx.x * ld;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = threadIdx.x * 4; i < V; i += 1024 * 4) {        // V % 4 == 0
    const float4 v = *(const float4*)(l + i);
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (e[u] > best) {                                       // first index of the thread's maximum
        best = e[u];
        bi = i + u;
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) {
      best = ov;
      bi = oi;
    }
  }
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = best;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    best = sv[0];
    bi = si[0];
    for (int k = 1; k < 16; ++k)
      if (sv[k] > best || (sv[k] == best && si[k] < bi)) {
        best = sv[k];
        bi = si[k];
      }
    out[blockIdx.x] = bi == 0x7FFFFFFF ? -1 : bi;
  }
}

hipError_t launch_argmax_rows(const float* logits, int V, int64_t ld, int rows, int32_t* out, hipStream_t st) {
  if (rows < 1 || V % 4 != 0 || ld % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(rows), dim3(1024), 0, st, logits, V, ld, out);
  return hipGetLastError();
}

hipError_t launch_argmax(const float2* cand, int ntiles, int B, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, st, cand, ntiles, out);
  return hipGetLastError();
}

}  // namespace gqa
