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
// Decode: one wave per (row, KV head, 32-position block), FP32 on the vector ALUs, four blocks
// per workgroup; see attn_decode_kernel.
#include "gqa_common.h"

namespace gqa {

constexpr int kDecodeChunk = 32;   // positions per decode wave (one KV block)
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

// Decode attention, one kernel per layer: grid (128-position chunk, KV head, row), four waves
// per workgroup, one 32-position block per wave (the block table is read once per wave).
//  1. q for the g query heads of the KV head: the fixed-order sum of the q|k|v projection's
//     split partials, per-head RMSNorm, rotate-half RoPE at the row's position.
//  2. The wave whose block holds the new position also builds its k (norm + RoPE) and v, rounds
//     them to BF16, writes them through the block table, and uses those register values for
//     that position.
//  3. Scores, softmax and the value sum over the wave's keys in FP32; the four waves merge
//     through LDS in wave order into one (max, sum, o) partial per chunk.
//  4. The last workgroup of a (row, KV head) to finish (device-scope release/acquire fences
//     around an atomic counter, which it resets) merges the chunk partials in chunk order and
//     writes o / l as FP16 hi/lo operands of the o projection.
// The q|k|v projection was taken of x * w_norm; its partials are scaled here by the row's 1/rms,
// recomputed from the sum-of-squares partials the projection's prologue wrote.
// The chunking depends only on the row's own context length, never on the batch.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeChunkPos = kDecodeChunk * kDecodeWaves;   // positions per workgroup
constexpr int kMergeMaxChunks = 128;                            // 16,384 positions

template <int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void attn_decode_kernel(
    const float* __restrict__ qkvp, int nsplit, int64_t pstride, int QKV, int nq, const float* __restrict__ ss,
    int ss_n, int H, const uint16_t* __restrict__ wqn, const uint16_t* __restrict__ wkn, float eps,
    const float* __restrict__ rcos, const float* __restrict__ rsin, Rows rows, uint16_t* __restrict__ kpool,
    uint16_t* __restrict__ vpool, float* __restrict__ part, int max_chunks, int* __restrict__ counters,
    float out_scale, f16* __restrict__ ohi, f16* __restrict__ olo, int ldo) {
  __shared__ float sm[kDecodeWaves][G], sl[kDecodeWaves][G];
  __shared__ float so[kDecodeWaves][G][kHeadDim];
  __shared__ float sw[G][kMergeMaxChunks];
  __shared__ float sL[G][kMergeMaxChunks];
  __shared__ int s_last;
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int pos = rows.pos[b], ctx = pos + 1;
  const int nchunk = (ctx + kDecodeChunkPos - 1) / kDecodeChunkPos;
  if (c >= nchunk) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ks = lane >> 4, dg = lane & 15;
  const int blk = c * kDecodeWaves + wave;                 // logical 32-position block of this wave
  const int kpos0 = blk * kDecodeChunk;
  const bool active = kpos0 < ctx;
  const float qscale = kLog2e * 0.08838834764831845f;
  const float* qrow = qkvp + (int64_t)b * QKV;
  // 1/rms of the normalised layer input: the projection was taken of x * w only
  const float cin = inv_rms_from_ss(ss, ss_n, b, H, eps);

  // sum of the projection's split partials for 8 consecutive dims of one head row, times cin
  auto head8 = [&](int hrow, float (&o)[8]) {
    float t[8][8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < nsplit) {
        const float* p = qrow + (int64_t)s * pstride + hrow * kHeadDim + dg * 8;
        float4 a0 = *(const float4*)p, a1 = *(const float4*)(p + 4);
        t[s][0] = a0.x; t[s][1] = a0.y; t[s][2] = a0.z; t[s][3] = a0.w;
        t[s][4] = a1.x; t[s][5] = a1.y; t[s][6] = a1.z; t[s][7] = a1.w;
      }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s < nsplit) acc += t[s][e];
      o[e] = __fmul_rn(acc, cin);
    }
  };
  // per-head RMSNorm over the 16 lanes of a key slot group, then RoPE: dims i < 64 pair with
  // i + 64, which live in lane dg ^ 8 at the same e.
  const float* cr = rcos + (int64_t)pos * 64;
  const float* sr = rsin + (int64_t)pos * 64;
  auto norm_rope = [&](float (&x)[8], const uint16_t* w) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    ss += __shfl_xor(ss, 8, 64);
    const float inv = 1.0f / sqrtf(ss / (float)kHeadDim + eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * bf16_bits_to_f32(w[dg * 8 + e]);
    const int i0 = (dg & 7) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float partner = __shfl_xor(y[e], 8, 64);
      float cs = cr[i0 + e], sn = sr[i0 + e];
      x[e] = dg < 8 ? y[e] * cs - partner * sn : y[e] * cs + partner * sn;
    }
  };

  // K/V loads of this wave's block first: they depend only on the block table
  constexpr int STEPS = kDecodeChunk / 4;
  uint4 kr[STEPS], vr[STEPS];
  if (active) {
    const int phys = rows.table[b][blk];
    const uint16_t* kbp = kpool + (((int64_t)phys * kKvHeads + kvh) * kBlock) * kHeadDim + dg * 8;
    const uint16_t* vbp = vpool + (((int64_t)phys * kKvHeads + kvh) * kBlock) * kHeadDim + dg * 8;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int j = kpos0 + st * 4 + ks;
      kr[st] = j < pos ? *(const uint4*)(kbp + (st * 4 + ks) * kHeadDim) : uint4{0, 0, 0, 0};
      vr[st] = j < pos ? *(const uint4*)(vbp + (st * 4 + ks) * kHeadDim) : uint4{0, 0, 0, 0};
    }
  }
  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    head8(kvh * G + hh, qv[hh]);
    norm_rope(qv[hh], wqn);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[hh][e] *= qscale;
  }
  // the new position's K/V (only in the wave whose block holds it)
  const bool owner = active && pos >= kpos0 && pos < kpos0 + kDecodeChunk;
  uint4 knew = uint4{0, 0, 0, 0}, vnew = uint4{0, 0, 0, 0};
  if (owner) {
    float kx[8], vx[8];
    head8(nq + kvh, kx);
    norm_rope(kx, wkn);
    head8(nq + kKvHeads + kvh, vx);
    uint32_t kb16[8], vb16[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kb16[e] = f32_to_bf16_rne(kx[e]);
      vb16[e] = f32_to_bf16_rne(vx[e]);
    }
    knew = uint4{kb16[0] | (kb16[1] << 16), kb16[2] | (kb16[3] << 16), kb16[4] | (kb16[5] << 16),
                 kb16[6] | (kb16[7] << 16)};
    vnew = uint4{vb16[0] | (vb16[1] << 16), vb16[2] | (vb16[3] << 16), vb16[4] | (vb16[5] << 16),
                 vb16[6] | (vb16[7] << 16)};
    if (ks == 0) {
      const int phys = rows.table[b][pos >> 5];
      const int64_t off = (((int64_t)phys * kKvHeads + kvh) * kBlock + (pos & 31)) * kHeadDim + dg * 8;
      *(uint4*)(kpool + off) = knew;
      *(uint4*)(vpool + off) = vnew;
    }
  }

  float m[G], l[G], o[G][8];
  if (active) {
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      if (kpos0 + st * 4 + ks == pos) {
        kr[st] = knew;
        vr[st] = vnew;
      }
    }
    float sc[G][STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const bool valid = kpos0 + st * 4 + ks < ctx;
      uint4 k4 = kr[st];
      float kf[8] = {bf16_bits_to_f32(k4.x & 0xFFFF), bf16_bits_to_f32(k4.x >> 16), bf16_bits_to_f32(k4.y & 0xFFFF),
                     bf16_bits_to_f32(k4.y >> 16),    bf16_bits_to_f32(k4.z & 0xFFFF), bf16_bits_to_f32(k4.z >> 16),
                     bf16_bits_to_f32(k4.w & 0xFFFF), bf16_bits_to_f32(k4.w >> 16)};
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
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) mx = fmaxf(mx, sc[hh][st]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        float p = exp2f(sc[hh][st] - mx);
        sum += p;
        uint4 v4 = vr[st];
        float vf[8] = {bf16_bits_to_f32(v4.x & 0xFFFF), bf16_bits_to_f32(v4.x >> 16), bf16_bits_to_f32(v4.y & 0xFFFF),
                       bf16_bits_to_f32(v4.y >> 16),    bf16_bits_to_f32(v4.z & 0xFFFF), bf16_bits_to_f32(v4.z >> 16),
                       bf16_bits_to_f32(v4.w & 0xFFFF), bf16_bits_to_f32(v4.w >> 16)};
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(p, vf[e], o[hh][e]);
      }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[hh][e] += __shfl_xor(o[hh][e], 16, 64);
        o[hh][e] += __shfl_xor(o[hh][e], 32, 64);
      }
      m[hh] = mx;
      l[hh] = sum;
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
    }
  }
  // merge the four waves (wave order) into the chunk partial
  if (ks == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (dg == 0) {
        sm[wave][hh] = m[hh];
        sl[wave][hh] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) so[wave][hh][dg * 8 + e] = o[hh][e];
    }
  }
  __syncthreads();
  {
    // thread -> (head, dim pair): G * 128 outputs over 256 threads
    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 64 * kDecodeWaves) {
      const int hh = idx / kHeadDim, d = idx % kHeadDim;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, sm[w][hh]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        const float wt = exp2f(sm[w][hh] - M);
        L = fmaf(sl[w][hh], wt, L);
        O = fmaf(so[w][hh][d], wt, O);
      }
      float* pp = part + (((int64_t)b * nq + kvh * G + hh) * max_chunks + c) * kPartStride;
      if (d == 0) {
        pp[0] = M;
        pp[1] = L;
      }
      pp[4 + d] = O;
    }
  }
  // last workgroup of this (row, KV head) merges the chunk partials
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const int old = __hip_atomic_fetch_add(&counters[b * kKvHeads + kvh], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == nchunk - 1;
    if (s_last) __threadfence();
  }
  __syncthreads();
  if (!s_last) return;
  // chunk maxima and sums into LDS (one thread per (head, chunk)), then per-head weights
  for (int i = threadIdx.x; i < G * nchunk; i += 64 * kDecodeWaves) {
    const int hh = i / nchunk, cc = i - hh * nchunk;
    const float* q = part + (((int64_t)b * nq + kvh * G + hh) * max_chunks + cc) * kPartStride;
    const float2 ml = *(const float2*)q;
    sw[hh][cc] = ml.x;
    sL[hh][cc] = ml.y;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int hh = threadIdx.x;
    float M = -INFINITY;
    for (int cc = 0; cc < nchunk; ++cc) M = fmaxf(M, sw[hh][cc]);
    float L = 0.f;
    for (int cc = 0; cc < nchunk; ++cc) {
      const float wt = exp2f(sw[hh][cc] - M);
      sw[hh][cc] = wt;
      L = fmaf(sL[hh][cc], wt, L);
    }
    sL[hh][0] = L;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 64 * kDecodeWaves) {
    const int hh = idx / kHeadDim, d = idx % kHeadDim;
    const float* pp = part + ((int64_t)b * nq + kvh * G + hh) * max_chunks * kPartStride + 4 + d;
    float O = 0.f;
    int cc = 0;
    for (; cc + 8 <= nchunk; cc += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = pp[(int64_t)(cc + u) * kPartStride];
#pragma unroll
      for (int u = 0; u < 8; ++u) O = fmaf(t[u], sw[hh][cc + u], O);
    }
    for (; cc < nchunk; ++cc) O = fmaf(pp[(int64_t)cc * kPartStride], sw[hh][cc], O);
    f16 hi, lo;
    split_f16(O / sL[hh][0] * out_scale, hi, lo);
    ohi[(int64_t)b * ldo + (kvh * G + hh) * kHeadDim + d] = hi;
    olo[(int64_t)b * ldo + (kvh * G + hh) * kHeadDim + d] = lo;
  }
  if (threadIdx.x == 0) counters[b * kKvHeads + kvh] = 0;
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

hipError_t launch_attn_decode(const float* qkvp, int nsplit, int64_t pstride, int QKV, int nq, const float* ss,
                              int ss_n, int H, const uint16_t* wqn, const uint16_t* wkn, float eps, const float* rcos,
                              const float* rsin, const Rows& rows, int B, int max_ctx, uint16_t* kpool,
                              uint16_t* vpool, float* part, int max_chunks, int* counters, float out_scale, f16* ohi,
                              f16* olo, int ldo, hipStream_t st) {
  const int chunks = (max_ctx + kDecodeChunkPos - 1) / kDecodeChunkPos;
  if (chunks > max_chunks || chunks > kMergeMaxChunks || nsplit < 1 || nsplit > 8) return hipErrorInvalidValue;
  dim3 grid(chunks, kKvHeads, B);
  const int G = nq / kKvHeads;
#define DEC_LAUNCH(GG)                                                                                           \
  hipLaunchKernelGGL(attn_decode_kernel<GG>, grid, dim3(64 * kDecodeWaves), 0, st, qkvp, nsplit, pstride, QKV, nq, \
                     ss, ss_n, H, wqn, wkn, eps, rcos, rsin, rows, kpool, vpool, part, max_chunks, counters,       \
                     out_scale, ohi, olo, ldo)
  if (G == 4)
    DEC_LAUNCH(4);
  else if (G == 2)
    DEC_LAUNCH(2);
  else
    return hipErrorInvalidValue;
#undef DEC_LAUNCH
  return hipGetLastError();
}

}  // namespace gqa
