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
// Decode: split-context attention in FP32 on the vector ALUs, then a chunk merge; see
// attn_decode_kernel.
#include "gqa_common.h"

namespace gqa {


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

// Decode attention (split context), grid (chunk, KV head, row), four waves per workgroup.
// A row's context [0, pos] is cut into chunks of decode_chunk_len(ctx) positions (a multiple of
// 64 chosen from the row's own context length only, so a row gets the same chunks whether it is
// evaluated alone or in a batch). A workgroup walks its chunk 64 positions at a time: wave w
// takes 16 consecutive positions, lane (ks, dg) = (lane / 16, lane % 16) holds dims 8dg..8dg+7 of
// positions ks, ks + 4, ks + 8, ks + 12, so one wave-wide 16-byte load covers four whole K (or V)
// rows, 1 KiB of contiguous pool memory. Each 16-lane group keeps its own online-softmax state
// (max, sum, value sum) for the g query heads of the KV head; the 16 states of the workgroup are
// merged in LDS into one chunk partial (max, sum, o[128]) per head.
//  1. q for the g query heads: the fixed-order sum of the q|k|v projection's split partials,
//     times the row's 1/rms (recomputed from the sum-of-squares partials the projection's
//     prologue wrote), per-head RMSNorm, rotate-half RoPE at the row's position, built once
//     per workgroup in LDS with every global load of the step issued together.
//  2. The workgroup whose chunk holds the new position also builds its k (norm + RoPE) and v,
//     rounds them to BF16, writes them through the block table and uses the rounded values
//     for that position.
//  3. The last workgroup of a (row, KV head) to finish combines the chunk partials of its heads in
//     chunk order (merge_head).
constexpr int kDecodeWaves = 4;
constexpr int kDecodeMaxChunks = 64;
constexpr int kPartStride = 132;   // floats per chunk partial: m, l, pad, pad, o[128]

__host__ __device__ __forceinline__ int decode_chunk_len(int ctx) {
  return 64 * ((ctx + 64 * kDecodeMaxChunks - 1) / (64 * kDecodeMaxChunks));
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float (&f)[8]) {
  f[0] = bf16_bits_to_f32(v.x & 0xFFFF); f[1] = bf16_bits_to_f32(v.x >> 16);
  f[2] = bf16_bits_to_f32(v.y & 0xFFFF); f[3] = bf16_bits_to_f32(v.y >> 16);
  f[4] = bf16_bits_to_f32(v.z & 0xFFFF); f[5] = bf16_bits_to_f32(v.z >> 16);
  f[6] = bf16_bits_to_f32(v.w & 0xFFFF); f[7] = bf16_bits_to_f32(v.w >> 16);
}

// Combine the chunk partials of one (row, query head) in chunk order: o = sum_c w_c o_c / sum_c
// w_c l_c with w_c = 2^(m_c - max m). One wave; lane t owns dims 2t, 2t + 1. The result is
// written as the FP16 hi/lo operand of the o projection, times out_scale.
__device__ __forceinline__ void merge_head(const float* pp, int nchunk, int lane, float out_scale, f16* ohi,
                                           f16* olo) {
  const float2 ml = *(const float2*)(pp + (int64_t)min(lane, nchunk - 1) * kPartStride);
  float2 ov[kDecodeMaxChunks];
#pragma unroll
  for (int cc = 0; cc < kDecodeMaxChunks; ++cc)
    ov[cc] = *(const float2*)(pp + (int64_t)min(cc, nchunk - 1) * kPartStride + 4 + 2 * lane);
  const float mv = lane < nchunk ? ml.x : -INFINITY;
  const float M = wave_max(mv);
  const float wt = lane < nchunk ? exp2f(mv - M) : 0.f;
  float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int cc = 0; cc < kDecodeMaxChunks; ++cc) {
    if (cc < nchunk) {
      const float w = __shfl(wt, cc, 64);
      L = fmaf(__shfl(ml.y, cc, 64), w, L);
      o0 = fmaf(ov[cc].x, w, o0);
      o1 = fmaf(ov[cc].y, w, o1);
    }
  }
  const float inv = out_scale / L;
  f16 h0, l0, h1, l1;
  split_f16(o0 * inv, h0, l0);
  split_f16(o1 * inv, h1, l1);
  *(f16x2*)(ohi + 2 * lane) = f16x2{h0, h1};
  *(f16x2*)(olo + 2 * lane) = f16x2{l0, l1};
}

template <int G>
__global__ __launch_bounds__(64 * kDecodeWaves) void attn_decode_kernel(
    const float* __restrict__ qkvp, int nsplit, int64_t pstride, int QKV, int nq, const float* __restrict__ ss,
    int ss_n, int H, const uint16_t* __restrict__ wqn, const uint16_t* __restrict__ wkn, float eps,
    const float* __restrict__ rcos, const float* __restrict__ rsin, Rows rows, uint16_t* __restrict__ kpool,
    uint16_t* __restrict__ vpool, float* part, int* __restrict__ counters, float out_scale, f16* __restrict__ ohi,
    f16* __restrict__ olo, int ldo) {
  constexpr int NST = 4 * kDecodeWaves;                   // softmax states per workgroup
  constexpr int NE = (G + 2) * kHeadDim;                  // q heads, then k and v of the new position
  __shared__ float sraw[NE];                              // projection sums (times 1/rms)
  __shared__ float sq[NE];                                // normed + rotated q (scaled), k; v
  __shared__ float sm[NST][G], sl[NST][G];
  __shared__ float so[NST][G][kHeadDim];
  __shared__ int s_last;
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int pos = rows.pos[b], ctx = pos + 1;
  const int CH = decode_chunk_len(ctx);
  const int nchunk = (ctx + CH - 1) / CH;
  if (c >= nchunk) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ks = lane >> 4, dg = lane & 15;
  const int p_begin = c * CH, p_end = min(p_begin + CH, ctx);
  const int niter = (p_end - p_begin + 63) / 64;
  const bool owner = pos >= p_begin && pos < p_end;     // this chunk holds the new position
  const int32_t* table = rows.table[b];
  const uint16_t* kbase = kpool + (int64_t)kvh * kBlock * kHeadDim + dg * 8;
  const uint16_t* vbase = vpool + (int64_t)kvh * kBlock * kHeadDim + dg * 8;
  constexpr int64_t kBlockElems = (int64_t)kKvHeads * kBlock * kHeadDim;

  // K/V of iteration `it` for this lane: positions p0 + 4 st + ks, all in one 32-position block.
  // The loads are unconditional (no branch between them): a position past the chunk reads a slot
  // of a block the session owns (or of the pool's block 0 when the whole group is past it) and
  // its value is discarded in step().
  auto phys_of = [&](int it) { return table[min(p_begin + it * 64 + wave * 16, p_end - 1) >> 5]; };
  auto load = [&](int it, int phys, uint4 (&kr)[4], uint4 (&vr)[4]) {
    const int p0 = p_begin + it * 64 + wave * 16;
    const int64_t off = (int64_t)phys * kBlockElems + (int64_t)(p0 & 31) * kHeadDim;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      kr[st] = *(const uint4*)(kbase + off + (st * 4 + ks) * kHeadDim);
      vr[st] = *(const uint4*)(vbase + off + (st * 4 + ks) * kHeadDim);
    }
  };
  uint4 kA[4], vA[4], kB[4], vB[4];
  // Issue order matters (vector loads complete in order): the block-table entry, the RoPE and
  // norm constants, the projection partials, then the first K/V, so q is built while the K/V
  // are in flight.
  const int phys0 = phys_of(0);
  nsplit = max(1, min(nsplit, 8));
  const float cs = rcos[(int64_t)pos * 64 + lane], sn = rsin[(int64_t)pos * 64 + lane];
  const float wq0 = bf16_bits_to_f32(wqn[lane]), wq1 = bf16_bits_to_f32(wqn[64 + lane]);
  const float wk0 = bf16_bits_to_f32(wkn[lane]), wk1 = bf16_bits_to_f32(wkn[64 + lane]);

  // 1. projection sums for the g q heads (and k, v in the owner): element e of the head rows
  //    kvh*g .. (q), nq + kvh (k), nq + 8 + kvh (v); split partials summed in split order
  {
    const float* qrow = qkvp + (int64_t)b * QKV;
    const int nel = owner ? NE : G * kHeadDim;
    constexpr int NI = (NE + 64 * kDecodeWaves - 1) / (64 * kDecodeWaves);
    float t[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) {                       // every load first
      const int e = i * 64 * kDecodeWaves + tid;
      const int hrow = e < G * kHeadDim ? kvh * G + e / kHeadDim
                                        : (e < (G + 1) * kHeadDim ? nq + kvh : nq + kKvHeads + kvh);
      const float* p = qrow + (e < nel ? hrow * kHeadDim + (e % kHeadDim) : 0);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) t[i][s2] = p[(int64_t)min(s2, nsplit - 1) * pstride];   // unconditional
    }
    load(0, phys0, kA, vA);
    const float cin = inv_rms_from_ss(ss, ss_n, b, H, eps);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = i * 64 * kDecodeWaves + tid;
      float acc = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) acc += s2 < nsplit ? t[i][s2] : 0.f;   // select, not a branch
      if (e < nel) sraw[e] = __fmul_rn(acc, cin);
    }
  }
  __syncthreads();
  // 2. per-head RMSNorm(128) and rotate-half RoPE at `pos`: wave w handles heads w, w + 4, ...;
  //    lane t owns dims t and t + 64 (a RoPE pair). q is pre-scaled by log2(e)/sqrt(128).
  {
    const float qscale = kLog2e * 0.08838834764831845f;
    const int nh = owner ? G + 1 : G;
    for (int hh = wave; hh < nh; hh += kDecodeWaves) {
      const float x0 = sraw[hh * kHeadDim + lane], x1 = sraw[hh * kHeadDim + 64 + lane];
      const float inv = 1.0f / sqrtf(wave_sum(x0 * x0 + x1 * x1) / (float)kHeadDim + eps);
      const float y0 = x0 * inv * (hh < G ? wq0 : wk0), y1 = x1 * inv * (hh < G ? wq1 : wk1);
      float r0 = y0 * cs - y1 * sn, r1 = y1 * cs + y0 * sn;
      if (hh < G) {
        r0 *= qscale;
        r1 *= qscale;
      } else {                                            // k: BF16 storage rounding
        r0 = bf16_bits_to_f32(f32_to_bf16_rne(r0));
        r1 = bf16_bits_to_f32(f32_to_bf16_rne(r1));
      }
      sq[hh * kHeadDim + lane] = r0;
      sq[hh * kHeadDim + 64 + lane] = r1;
    }
    if (owner && tid < kHeadDim) sq[(G + 1) * kHeadDim + tid] = bf16_bits_to_f32(f32_to_bf16_rne(sraw[(G + 1) * kHeadDim + tid]));
  }
  __syncthreads();
  // the new position's K/V into the pool, through the block table
  if (owner && tid < 2 * kHeadDim / 8) {
    const int kv = tid >> 4, d0 = (tid & 15) * 8;       // tid < 16: K, else V
    const float* src = sq + (G + kv) * kHeadDim + d0;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = f32_to_bf16_rne(src[e]);
    const int64_t off = (int64_t)table[pos >> 5] * kBlockElems + ((int64_t)kvh * kBlock + (pos & 31)) * kHeadDim + d0;
    *(uint4*)((kv ? vpool : kpool) + off) =
        uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[hh][e] = sq[hh * kHeadDim + dg * 8 + e];

  // 3. online softmax over the chunk, one state per 16-lane row group
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
  auto step = [&](int it, const uint4 (&kr)[4], const uint4 (&vr)[4]) {
    const int p0 = p_begin + it * 64 + wave * 16;
    float kf[4][8], vf[4][8];
    bool valid[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int p = p0 + st * 4 + ks;
      valid[st] = p < p_end;
      bf16x8_to_f32(kr[st], kf[st]);
      bf16x8_to_f32(vr[st], vf[st]);
      if (owner && p == pos) {                            // the new position, not yet in the pool
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kf[st][e] = sq[G * kHeadDim + dg * 8 + e];
          vf[st][e] = sq[(G + 1) * kHeadDim + dg * 8 + e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[st][e] = valid[st] ? vf[st][e] : 0.f;
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float sc[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qv[hh][e], kf[st][e], d);
        d = row16_sum(d);
        sc[st] = valid[st] ? d : -INFINITY;
      }
      const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      const float mn = fmaxf(m[hh], mx);
      if (mn == -INFINITY) continue;                     // nothing visible yet in this group
      const float alpha = exp2f(m[hh] - mn);
      float lsum = l[hh] * alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= alpha;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float pr = exp2f(sc[st] - mn);
        lsum += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pr, vf[st][e], o[hh][e]);
      }
      l[hh] = lsum;
      m[hh] = mn;
    }
  };
  for (int it = 0; it < niter; it += 2) {
    if (it + 1 < niter) load(it + 1, phys_of(it + 1), kB, vB);
    step(it, kA, vA);
    if (it + 1 >= niter) break;
    if (it + 2 < niter) load(it + 2, phys_of(it + 2), kA, vA);
    step(it + 1, kB, vB);
  }

  // 4. merge the 16 row-group states of the workgroup (state index 4 * wave + ks, in order)
  const int si = wave * 4 + ks;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (dg == 0) {
      sm[si][hh] = m[hh];
      sl[si][hh] = l[hh];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) so[si][hh][dg * 8 + e] = o[hh][e];
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += 64 * kDecodeWaves) {
    const int hh = idx / kHeadDim, d = idx % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NST; ++w) M = fmaxf(M, sm[w][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NST; ++w) {
      const float wt = sm[w][hh] == -INFINITY ? 0.f : exp2f(sm[w][hh] - M);
      L = fmaf(sl[w][hh], wt, L);
      O = fmaf(so[w][hh][d], wt, O);
    }
    float* pp = part + (((int64_t)b * nq + kvh * G + hh) * kDecodeMaxChunks + c) * kPartStride;
    if (d == 0) {
      pp[0] = M;
      pp[1] = L;
    }
    pp[4 + d] = O;
  }
  // 5. the last workgroup of this (row, KV head) to finish merges the chunk partials. Every wave
  //    waits until its partial stores have completed, then one thread publishes them device-wide
  //    (a device-scope release writes back this XCD's L2) and counts the workgroup in; the last
  //    workgroup acquires (invalidating its stale cache lines) before any wave reads the other
  //    workgroups' partials, and resets the count for the next call.
  __builtin_amdgcn_s_waitcnt(0);          // vmcnt = lgkmcnt = 0: this wave's stores are done
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int old = __hip_atomic_fetch_add(&counters[b * kKvHeads + kvh], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == nchunk - 1;
    if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!s_last) return;
  if (wave < G) {
    const int h = kvh * G + wave;
    merge_head(part + ((int64_t)b * nq + h) * kDecodeMaxChunks * kPartStride, nchunk, lane, out_scale,
               ohi + (int64_t)b * ldo + h * kHeadDim, olo + (int64_t)b * ldo + h * kHeadDim);
  }
  if (tid == 0) counters[b * kKvHeads + kvh] = 0;
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
                              uint16_t* vpool, float* part, int* counters, float out_scale, f16* ohi, f16* olo,
                              int ldo, hipStream_t st) {
  if (nsplit < 1 || nsplit > 8 || B < 1 || B > kMaxBatch || max_ctx < 1) return hipErrorInvalidValue;
  const int CH = decode_chunk_len(max_ctx);
  const int chunks = (max_ctx + CH - 1) / CH;          // rows with shorter contexts exit early
  dim3 grid(chunks, kKvHeads, B);
  const int G = nq / kKvHeads;
#define DEC_LAUNCH(GG)                                                                                           \
  hipLaunchKernelGGL(attn_decode_kernel<GG>, grid, dim3(64 * kDecodeWaves), 0, st, qkvp, nsplit, pstride, QKV, nq, \
                     ss, ss_n, H, wqn, wkn, eps, rcos, rsin, rows, kpool, vpool, part, counters, out_scale, ohi, olo, \
                     ldo)
  if (G == 4)
    DEC_LAUNCH(4);
  else if (G == 2)
    DEC_LAUNCH(2);
  else
    return hipErrorInvalidValue;
#undef DEC_LAUNCH
  return hipGetLastError();
}

// floats of the chunk-partial buffer for B rows of nq heads
int64_t attn_decode_part_floats(int nq) { return (int64_t)kMaxBatch * nq * kDecodeMaxChunks * kPartStride; }

}  // namespace gqa
