// GQA attention over the paged BF16 KV cache.
//
// Kipp Roadmap, status v0.0.3/v0.0.4: flash-attention prefill for GQA (kipp_flash_gqa_prefill);
// status v0.0.2: K/V live in 32-position blocks addressed through a per-session block table.
// For query head h the KV head is h / g (g = n_q_heads / 8); key j is visible to the query at
// position p iff j <= p; scores are q.k / sqrt(128) and the output is the softmax-weighted sum of
// V. Softmax runs in base 2 on scores pre-multiplied by log2(e) / sqrt(128).
//
// Prefill: one 256-thread workgroup per (query tile, KV head). Each wave owns 32 query positions
// of one head of the group, so the g heads that share a KV head share every K/V tile staged in
// LDS. S^T = K Q^T and O^T = V^T P^T run on the matrix cores (v_mfma_f32_16x16x32_f16): K and V
// are exact FP16 operands, Q and P enter as FP16 hi/lo pairs (near-FP32), accumulation is FP32,
// and the online softmax keeps a running max and sum per query column. P^T is consumed straight
// from the S^T accumulator layout: within each 32-key chunk a lane holds keys 4g..4g+3 and
// 16+4g..16+4g+3 (g = lane / 16), and V^T is read from LDS in the same key order.
//
// Decode: one wave per (row, KV head, 64-position chunk), FP32 on the vector ALUs; the
// per-chunk (max, sum, o) partials are merged by attn_combine_kernel. The chunking depends only
// on the row's own context length, never on the batch.
#include "gqa_common.h"

namespace gqa {

constexpr int kDecodeChunk = 64;
constexpr int kPartStride = 132;   // floats per decode partial: m, l, pad, pad, o[128]

template <int G, bool PSPLIT>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const float* __restrict__ q, int nq, int T, int pos0,
                                                           const int32_t* __restrict__ table,
                                                           const uint16_t* __restrict__ kpool,
                                                           const uint16_t* __restrict__ vpool, float out_scale,
                                                           f16* __restrict__ ohi, f16* __restrict__ olo, int ldo) {
  constexpr int WPH = 4 / G;            // waves per head
  constexpr int BQ = 32 * WPH;          // query positions per workgroup
  constexpr int KT = 64;                // keys per iteration
  constexpr int LDK = kHeadDim + 8, LDV = KT + 8;
  __shared__ f16 sK[KT * LDK];
  __shared__ f16 sVt[kHeadDim * LDV];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int qtile = gridDim.x - 1 - blockIdx.x;     // longest rows first
  const int kvh = blockIdx.y;
  const int tq0 = qtile * BQ;                        // first query row (round-relative) of the workgroup
  const int head = kvh * G + wave / WPH;
  const int tw0 = tq0 + (wave % WPH) * 32;           // first query row of this wave
  const int kend = pos0 + min(tq0 + BQ, T);          // keys needed by the workgroup's valid rows
  const float qscale = kLog2e * 0.08838834764831845f;

  // Q fragments (B operand of S^T): lane -> query column r16 of tile qt, dims kk*32 + 8*g4 .. +7.
  f16x8 qh[2][4], ql[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    int t = tw0 + qt * 16 + r16;
    const float* qr = q + ((int64_t)min(t, T - 1) * nq + head) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float4 v0 = *(const float4*)(qr + kk * 32 + g4 * 8);
      float4 v1 = *(const float4*)(qr + kk * 32 + g4 * 8 + 4);
      float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f16 h, l;
        split_f16(v[e] * qscale, h, l);
        qh[qt][kk][e] = h;
        ql[qt][kk][e] = l;
      }
    }
  }

  f32x4 o[8][2];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d][0] = o[d][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-1e30f, -1e30f}, lrow[2] = {0.f, 0.f};

  // staging: K chunk c = tid + 256*i -> key c >> 4, dims (c & 15) * 8; V chunk -> key c & 63,
  // dims ((c >> 6)) * 8 (so consecutive lanes write consecutive keys of one V^T row).
  uint4 rk[4], rv[4];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + 256 * i;
      int key = kb + (c >> 4);
      if (key < kend) {
        int phys = table[key >> 5];
        rk[i] = *(const uint4*)(kpool + (((int64_t)phys * kKvHeads + kvh) * kBlock + (key & 31)) * kHeadDim +
                                (c & 15) * 8);
      } else {
        rk[i] = uint4{0, 0, 0, 0};
      }
      int vkey = kb + (c & 63);
      if (vkey < kend) {
        int phys = table[vkey >> 5];
        rv[i] = *(const uint4*)(vpool + (((int64_t)phys * kKvHeads + kvh) * kBlock + (vkey & 31)) * kHeadDim +
                                (c >> 6) * 8);
      } else {
        rv[i] = uint4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + 256 * i;
      *(f16x8*)&sK[(c >> 4) * LDK + (c & 15) * 8] = bf16x8_to_f16x8(rk[i]);
      f16x8 v = bf16x8_to_f16x8(rv[i]);
      int key = c & 63, d0 = (c >> 6) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[(d0 + e) * LDV + key] = v[e];
    }
  };

  gload(0);
  for (int kb = 0; kb < kend; kb += KT) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kb + KT < kend) gload(kb + KT);

    // S^T tiles: s[kt][qt][r] = score of key kb + kt*16 + 4*g4 + r for query column qt*16 + r16.
    f32x4 s[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt][0] = s[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f16x8 a = *(const f16x8*)&sK[(kt * 16 + r16) * LDK + kk * 32 + g4 * 8];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          s[kt][qt] = mfma16(a, qh[qt][kk], s[kt][qt]);
          s[kt][qt] = mfma16(a, ql[qt][kk], s[kt][qt]);
        }
      }
    }
    // causal mask + online softmax per query column
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      int qpos = pos0 + tw0 + qt * 16 + r16;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int kpos = kb + kt * 16 + g4 * 4 + r;
          float v = kpos <= qpos ? s[kt][qt][r] : -INFINITY;
          s[kt][qt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float mnew = fmaxf(mrow[qt], mx);
      float alpha = exp2f(mrow[qt] - mnew);
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = exp2f(s[kt][qt][r] - mnew);
          s[kt][qt][r] = p;
          sum += p;
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      lrow[qt] = lrow[qt] * alpha + sum;
      mrow[qt] = mnew;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[d][qt] *= alpha;
    }
    // O^T += V^T P^T over two 32-key chunks
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f16x8 ph[2], pl[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f16 h, l;
          split_f16(s[2 * c][qt][r], h, l);
          ph[qt][r] = h;
          pl[qt][r] = l;
          split_f16(s[2 * c + 1][qt][r], h, l);
          ph[qt][4 + r] = h;
          pl[qt][4 + r] = l;
        }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const f16* vr = &sVt[(d * 16 + r16) * LDV + c * 32 + g4 * 4];
        f16x4 v0 = *(const f16x4*)vr;
        f16x4 v1 = *(const f16x4*)(vr + 16);
        f16x8 a = f16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          o[d][qt] = mfma16(a, ph[qt], o[d][qt]);
          if (PSPLIT) o[d][qt] = mfma16(a, pl[qt], o[d][qt]);
        }
      }
    }
  }

  // o[d][qt][r] = O^T[dim d*16 + 4*g4 + r][query qt*16 + r16]
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    int t = tw0 + qt * 16 + r16;
    if (t < T) {
      float inv = out_scale / lrow[qt];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        f16x4 hv, lv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f16 h, l;
          split_f16(o[d][qt][r] * inv, h, l);
          hv[r] = h;
          lv[r] = l;
        }
        int64_t off = (int64_t)t * ldo + head * kHeadDim + d * 16 + g4 * 4;
        *(f16x4*)&ohi[off] = hv;
        *(f16x4*)&olo[off] = lv;
      }
    }
  }
}

// Decode: grid (chunk, kv head, row); one wave. Lane: key slot ks = lane >> 4 (4 keys per step),
// dims 8*(lane & 15) .. +7. Two passes over the chunk's 64 keys (scores, then values).
template <int G>
__global__ __launch_bounds__(64) void attn_decode_kernel(const float* __restrict__ q, int nq, Rows rows,
                                                         const uint16_t* __restrict__ kpool,
                                                         const uint16_t* __restrict__ vpool,
                                                         float* __restrict__ part, int max_chunks) {
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int ctx = rows.pos[b] + 1;
  if (c * kDecodeChunk >= ctx) return;
  const int32_t* table = rows.table[b];
  const int lane = threadIdx.x, ks = lane >> 4, dg = lane & 15;
  const float qscale = kLog2e * 0.08838834764831845f;

  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float* qr = q + ((int64_t)b * nq + kvh * G + hh) * kHeadDim + dg * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[hh][e] = qr[e] * qscale;
  }
  constexpr int STEPS = kDecodeChunk / 4;
  float sc[G][STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    int j = c * kDecodeChunk + st * 4 + ks;
    bool valid = j < ctx;
    uint4 kr = uint4{0, 0, 0, 0};
    if (valid) {
      int phys = table[j >> 5];
      kr = *(const uint4*)(kpool + (((int64_t)phys * kKvHeads + kvh) * kBlock + (j & 31)) * kHeadDim + dg * 8);
    }
    float kf[8] = {bf16_bits_to_f32(kr.x & 0xFFFF), bf16_bits_to_f32(kr.x >> 16), bf16_bits_to_f32(kr.y & 0xFFFF),
                   bf16_bits_to_f32(kr.y >> 16),    bf16_bits_to_f32(kr.z & 0xFFFF), bf16_bits_to_f32(kr.z >> 16),
                   bf16_bits_to_f32(kr.w & 0xFFFF), bf16_bits_to_f32(kr.w >> 16)};
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qv[hh][e], kf[e], d);
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      d += __shfl_xor(d, 4, 64);
      d += __shfl_xor(d, 8, 64);
      sc[hh][st] = valid ? d : -INFINITY;
    }
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) mx = fmaxf(mx, sc[hh][st]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    m[hh] = mx;
    float sum = 0.f;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      float p = exp2f(sc[hh][st] - mx);
      sc[hh][st] = p;
      sum += p;
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    l[hh] = sum;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    int j = c * kDecodeChunk + st * 4 + ks;
    if (j < ctx) {
      int phys = table[j >> 5];
      uint4 vr = *(const uint4*)(vpool + (((int64_t)phys * kKvHeads + kvh) * kBlock + (j & 31)) * kHeadDim + dg * 8);
      float vf[8] = {bf16_bits_to_f32(vr.x & 0xFFFF), bf16_bits_to_f32(vr.x >> 16), bf16_bits_to_f32(vr.y & 0xFFFF),
                     bf16_bits_to_f32(vr.y >> 16),    bf16_bits_to_f32(vr.z & 0xFFFF), bf16_bits_to_f32(vr.z >> 16),
                     bf16_bits_to_f32(vr.w & 0xFFFF), bf16_bits_to_f32(vr.w >> 16)};
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(sc[hh][st], vf[e], o[hh][e]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[hh][e] += __shfl_xor(o[hh][e], 16, 64);
      o[hh][e] += __shfl_xor(o[hh][e], 32, 64);
    }
    if (ks == 0) {
      float* pp = part + (((int64_t)b * nq + kvh * G + hh) * max_chunks + c) * kPartStride;
      if (dg == 0) {
        pp[0] = m[hh];
        pp[1] = l[hh];
      }
      *(float4*)(pp + 4 + dg * 8) = make_float4(o[hh][0], o[hh][1], o[hh][2], o[hh][3]);
      *(float4*)(pp + 8 + dg * 8) = make_float4(o[hh][4], o[hh][5], o[hh][6], o[hh][7]);
    }
  }
}

// Merge the chunk partials of one (row, head): O = sum_c o_c 2^(m_c - M) / sum_c l_c 2^(m_c - M).
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part, int nq, Rows rows,
                                                           int max_chunks, float out_scale, f16* __restrict__ ohi,
                                                           f16* __restrict__ olo, int ldo) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int n = (rows.pos[b] + 1 + kDecodeChunk - 1) / kDecodeChunk;
  const float* pp = part + ((int64_t)b * nq + h) * max_chunks * kPartStride;
  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, pp[c * kPartStride]);
  float L = 0.f, O = 0.f;
  for (int c = 0; c < n; ++c) {
    float w = exp2f(pp[c * kPartStride] - M);
    L = fmaf(pp[c * kPartStride + 1], w, L);
    O = fmaf(pp[c * kPartStride + 4 + d], w, O);
  }
  f16 hi, lo;
  split_f16(O / L * out_scale, hi, lo);
  ohi[(int64_t)b * ldo + h * kHeadDim + d] = hi;
  olo[(int64_t)b * ldo + h * kHeadDim + d] = lo;
}

hipError_t launch_attn_prefill(const float* q, int nq, int T, int pos0, const int32_t* table, const uint16_t* kpool,
                               const uint16_t* vpool, float out_scale, f16* ohi, f16* olo, int ldo, hipStream_t st) {
  int G = nq / kKvHeads;
  if (G == 4) {
    dim3 grid((T + 31) / 32, kKvHeads);
    hipLaunchKernelGGL((attn_prefill_kernel<4, true>), grid, dim3(256), 0, st, q, nq, T, pos0, table, kpool, vpool,
                       out_scale, ohi, olo, ldo);
  } else if (G == 2) {
    dim3 grid((T + 63) / 64, kKvHeads);
    hipLaunchKernelGGL((attn_prefill_kernel<2, true>), grid, dim3(256), 0, st, q, nq, T, pos0, table, kpool, vpool,
                       out_scale, ohi, olo, ldo);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const float* q, int nq, const Rows& rows, int B, int max_ctx, const uint16_t* kpool,
                              const uint16_t* vpool, float* part, int max_chunks, float out_scale, f16* ohi,
                              f16* olo, int ldo, hipStream_t st) {
  int chunks = (max_ctx + kDecodeChunk - 1) / kDecodeChunk;
  if (chunks > max_chunks) return hipErrorInvalidValue;
  dim3 grid(chunks, kKvHeads, B);
  int G = nq / kKvHeads;
  if (G == 4)
    hipLaunchKernelGGL(attn_decode_kernel<4>, grid, dim3(64), 0, st, q, nq, rows, kpool, vpool, part, max_chunks);
  else if (G == 2)
    hipLaunchKernelGGL(attn_decode_kernel<2>, grid, dim3(64), 0, st, q, nq, rows, kpool, vpool, part, max_chunks);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(nq, B), dim3(128), 0, st, part, nq, rows, max_chunks, out_scale, ohi,
                     olo, ldo);
  return hipGetLastError();
}

}  // namespace gqa
