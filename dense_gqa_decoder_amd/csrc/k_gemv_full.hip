// Decode projections for a few token rows with the whole K range in one workgroup.
//
// Y[b][n] = sum_k W[n][k] * x[b][k] for B <= 4 rows whose FP16 hi/lo operand rows fit in LDS.
// A workgroup owns NBW 16-row weight bands; the K range of a band is cut into S = NWB equal
// ranges, one wave each (the same ranges as the split-K matvec in k_gemv.hip), so every wave
// streams one contiguous stretch of the tile-major weights with 16-byte loads, U K-steps per
// stage with two stages in flight, and multiplies them on the matrix cores
// (v_mfma_f32_16x16x32_f16, FP16 hi/lo activations, FP32 accumulate). The S range partials of a
// band are then summed in LDS in range order, starting from zero -- the same additions the
// split-K path's consumers perform on its global partials -- so a row gives bit-identical
// results on both paths (Kipp Roadmap, status v0.0.2: batched evaluation equals isolated).
//
// Operand prologues (the whole row is read by every workgroup; it is small and L2-resident, or
// for a launch of a decode chain read device-scope once the predecessors have counted in):
//   XF_RAW  copy FP16 hi/lo rows from global memory.
//   XF_NORM the RMSNorm input of a projection: x * w_norm, split hi/lo; the sum of squares of x
//           per K range is formed with the split-K path's element-to-thread mapping and order
//           (thread t of a 256-thread group takes elements t + 256 j of the range, then the
//           wave sums, then the four waves in order); workgroup 0 publishes the range sums in
//           ss_out[range][row] for later consumers. The 1/rms factor is a per-row scalar applied
//           after the projection (by the epilogue or by the consumer).
// Epilogues:
//   EPI_STORE  y = sum (q|k|v, lm_head; optional argmax candidates per band)
//   EPI_ADD    y = y + sum * yscale (residual stream update after o and down)
//   EPI_SWIGLU bands 2j, 2j+1 are gate and up of features 16j..16j+15: m = silu(g c) * (u c),
//              c = 1/rms of the layer input, written as FP16 hi/lo rows for the down projection
//              (BF16 weights: as mixed bands, EPI_SWIGLU_MIX below, the same products).
//   EPI_ADD loads its residual rows before the weight stream (its workgroup is their only writer).
#include "gqa_common.h"

namespace gqa {

constexpr int kFullMaxB = 4;
// K-steps per stage of the decode projections, two stages in flight; any value gives the same
// bits. Measured on the 4B decode: BF16 weights 3 (q|k|v, gate/up) and 6 (o, down) run 0.9%
// faster than 4 and 8, which the quantised formats keep (their smaller steps gain from depth).
constexpr int kUQkv = 3, kUGu = 3, kUOd = 6, kUQkvQ = 4, kUGuQ = 4, kUOdQ = 8, kULm = 8;
constexpr int kFullMaxLds = 64 * 1024;   // operand rows (hi + lo) in LDS
// Gate/up of BF16 weights as mixed bands: workgroup m takes rows 8 (m % 2) .. + 7 of the gate
// band 2 (m / 2) and of the up band after it (the same eight features) as the 16 rows of its
// matrix-core tiles, so the SwiGLU pairs meet in one wave and the grid has one workgroup per
// eight features (1,216 of four waves for the 4B shape, 4.75 per CU) instead of one per sixteen
// (608 of eight waves: two or three per CU, and the CUs with three set the kernel's end).
constexpr int EPI_SWIGLU_MIX = 3;
#ifndef GQA_GATEUP_MIXED
#define GQA_GATEUP_MIXED 1
#endif

// CH: membership of a decode chain (gqa_common.h). 0: none. 1: an any-order launch that waits
// for its predecessors before reading the operand rows and reads them device-scope. 2: an
// ordered launch (the queue has finished its predecessors), plain loads. 1 and 2 write what
// later launches read device-scope and count themselves in at the end.
// wsrc (the weights: a.W, or a.Wq for the quantised formats) and kdim (a.K) lead the arguments so
// that the dispatcher preloads them into scalar registers (-amdgpu-kernarg-preload-count): a
// wave issues its first weight loads without waiting for a kernel-argument load.
template <int QM, int NWB, int NBW, int U, int MODE, int EPI, int MAXB, int CH>
__global__ __launch_bounds__(64 * NWB * NBW) void gemv_full_kernel(const void* __restrict__ wsrc, int kdim, FullArgs a) {
  constexpr int NT = 64 * NWB * NBW;
  constexpr int S = NWB;
  extern __shared__ f16 sx[];                         // [2][B][K] (+ one padding piece)
  __shared__ f32x4 red[NBW][NWB][64];
  __shared__ float sred[kFullMaxB][8][4];
  __shared__ float sinv[kFullMaxB];
  // the wave index as a scalar, so the K-range bounds and every test on them are uniform branches
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bw = wave / NWB, kp = wave % NWB;
  const int band = blockIdx.x * NBW + bw;
  const int K = kdim, B = a.B, KS = K >> 5;
  const int s0 = kp * (KS / S), s1 = s0 + KS / S;
  const int r16 = lane & 15, g4 = lane >> 4;

  // weight stream of this wave: band `band`, K-steps [s0, s1); lane l loads tile row l % 16,
  // K-elements 8 (l / 16) .. + 7 (the tile-major layout), or for a mixed band that row of the
  // gate (l % 16 < 8) or up band
  static_assert(EPI != EPI_SWIGLU_MIX || (QM == WM_BF16 && NBW == 1), "mixed bands: BF16, one per workgroup");
  int64_t chunk0 = (int64_t)band * KS;
  int loff = lane * 8;
  if constexpr (EPI == EPI_SWIGLU_MIX) {
    chunk0 = (int64_t)(2 * (blockIdx.x >> 1) + (r16 >> 3)) * KS;
    loff = 8 * (16 * g4 + 8 * (blockIdx.x & 1) + (r16 & 7));
  }
  struct Buf {
    uint4 w[U];
    uint2 q[U];
    uint32_t q4[U];
    uint2 sc[U];
    uint2 bs[U];
  };
  auto fetch = [&](Buf& f, int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ch = chunk0 + min(s + u, s1 - 1);     // unconditional: no branch between loads
      if (QM == WM_Q8) {
        f.q[u] = *(const uint2*)((const int8_t*)wsrc + ch * 512 + lane * 8);
      } else if (QM == WM_A4) {
        f.q4[u] = *(const uint32_t*)((const int8_t*)wsrc + ch * 256 + lane * 4);
      } else {
        f.w[u] = *(const uint4*)((const uint16_t*)wsrc + ch * 512 + loff);
      }
    }
  };
  Buf b0, b1;
  fetch(b0, s0);
  fetch(b1, s0 + U);
  const int n = band * 16 + g4 * 4;                   // epilogue: rows n .. n + 3 of token row r16
  const bool yown = kp == 0 && r16 < B;

  // Q8_0 / AFFINE4: the scales (and biases) of the workgroup's bands, staged in LDS once, in their
  // memory order [band][K-step][16 rows] after the operand rows, so the weight stream issues one
  // load per lane and step (the scale reads, repeated by the 16 token lanes, come from LDS).
  f16* const ssc = sx + 2 * B * K + 8;
  f16* const sbs = ssc + NBW * KS * 16;
  if constexpr (QM != WM_BF16) {
    const int per = KS * 2;                             // 16-byte pieces per band
    for (int i = tid; i < NBW * per; i += NT) {
      const int bb = i / per, c = i - bb * per;
      const int64_t src = (int64_t)(blockIdx.x * NBW + bb) * KS * 16 + c * 8;
      *(uint4*)(ssc + bb * KS * 16 + c * 8) = *(const uint4*)(a.Wd + src);
      if (QM == WM_A4) *(uint4*)(sbs + bb * KS * 16 + c * 8) = *(const uint4*)(a.Wb + src);
    }
  }
  if constexpr (CH == 1) chain_wait(a.chain);
  // EPI_ADD: the residual rows this lane updates, loaded now rather than after the stream (this
  // workgroup is the only writer of its band)
  float4 yold = make_float4(0.f, 0.f, 0.f, 0.f);
  if (EPI == EPI_ADD && yown) {
    const float* src = a.y + (int64_t)r16 * a.ldy + n;
    if constexpr (CH == 1)
      yold = __builtin_bit_cast(float4, ld_dev16(src));
    else
      yold = *(const float4*)src;
  }

  // ---- operand rows into LDS: [0][b][k] = hi, [1][b][k] = lo
  const int BK = B * K;
  if constexpr (MODE == XF_RAW) {
    constexpr int CMAX = (MAXB == 1 ? kFullMaxLds / 4 : kFullMaxLds) / 16 / NT;
    const int npiece = 2 * BK / 8;
    uint4 v[CMAX];
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
      const int c = min(tid + i * NT, npiece - 1);
      const int hl = c >= BK / 8, rem = c - hl * (BK / 8), b = rem / (K / 8), q = rem - b * (K / 8);
      const f16* src = (hl ? a.xlo : a.xhi) + (int64_t)b * a.ldx + q * 8;
      if constexpr (CH == 1)
        v[i] = ld_dev16(src);
      else
        v[i] = *(const uint4*)src;
    }
#pragma unroll
    for (int i = 0; i < CMAX; ++i) *(uint4*)(sx + (int64_t)min(tid + i * NT, npiece) * 8) = v[i];
  } else {
    // thread (g, t): ranges r = g, g + G, ...; elements t + 256 j of each range
    constexpr int G = NT >= 256 ? NT / 256 : 1;
    constexpr int P = S / G;                          // ranges per 256-thread group
    constexpr int JMAX = (4096 / S + 255) / 256;      // K <= 4096 for normed inputs
    const int g = tid >> 8, t = tid & 255;
    const int klen = K / S;
    float xv[MAXB][P][JMAX], wv[P][JMAX];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int j = 0; j < JMAX; ++j) {                // every load first, unconditional
        const int r = p * G + g, off = min(t + 256 * j, klen - 1);
        wv[p][j] = bf16_bits_to_f32(a.nw[r * klen + off]);
#pragma unroll
        for (int b = 0; b < MAXB; ++b) {
          const float* src = a.xres + (int64_t)min(b, B - 1) * K + r * klen + off;
          if constexpr (CH == 1)
            xv[b][p][j] = ld_dev(src);
          else
            xv[b][p][j] = *src;
        }
      }
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
      if (b >= B) break;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int r = p * G + g;
        float ssq = 0.f;
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
          const int off = t + 256 * j;
          if (off < klen) {
            const float x = xv[b][p][j];
            f16 h, l;
            split_f16(__fmul_rn(x, wv[p][j]), h, l);
            sx[(int64_t)b * K + r * klen + off] = h;
            sx[(int64_t)BK + b * K + r * klen + off] = l;
            ssq = __fadd_rn(ssq, __fmul_rn(x, x));
          }
        }
        ssq = wave_sum(ssq);
        if (lane == 0) sred[b][r][(t >> 6)] = ssq;
      }
    }
  }
  __syncthreads();
  if constexpr (MODE == XF_NORM) {
    if (tid < kFullMaxB) {
      const int b = tid;
      float tot = 0.f;
      for (int r = 0; r < S && b < B; ++r) {
        const float sr = __fadd_rn(__fadd_rn(__fadd_rn(sred[b][r][0], sred[b][r][1]), sred[b][r][2]), sred[b][r][3]);
        if (blockIdx.x == 0 && a.ss_out) {
          if constexpr (CH != 0)
            st_dev(a.ss_out + r * 32 + b, sr);
          else
            a.ss_out[r * 32 + b] = sr;
        }
        tot += sr;
      }
      sinv[b] = 1.0f / sqrtf(tot / (float)K + a.eps);
    }
    __syncthreads();
  }

  // ---- stream the weights
  // token columns r16 >= B: their products are computed and never stored (every store, candidate and
  // shuffle below is per column and gated on r16 < B). The BF16 stream gives them zero operands by
  // masked LDS reads (only the token lanes read); the quantised streams, which issue more per step,
  // let them read row 0 unmasked, which spares the exec-mask branches and measured faster there.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f16* xh = sx + (int64_t)(r16 < B ? r16 : 0) * K + g4 * 8;
  const f16* xl = xh + BK;
  auto compute = [&](const Buf& f, int s) {
    if constexpr (QM == WM_BF16) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s + u < s1) {
          const int kk = (s + u) * 32;
          const f16x8 bh = r16 < B ? *(const f16x8*)(xh + kk) : f16x8{};
          const f16x8 bl = r16 < B ? *(const f16x8*)(xl + kk) : f16x8{};
          const f16x8 w = bf16x8_to_f16x8(f.w[u]);
          acc = mfma16(w, bh, acc);
          acc = mfma16(w, bl, acc);
        }
      }
    } else {
      // every step's block products first, then the scaled accumulation in step order
      f32x4 p[U], xs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s + u < s1) {
          const int kk = (s + u) * 32;
          const f16x8 bh = *(const f16x8*)(xh + kk);
          const f16x8 bl = *(const f16x8*)(xl + kk);
          qstep_products<QM>(qwiden<QM>(f.q[u], f.q4[u]), bh, bl, p[u], xs[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (s + u < s1) {
          const int at = (bw * KS + s + u) * 16 + g4 * 4;
          qstep_accumulate<QM>(acc, p[u], xs[u], *(const uint2*)(ssc + at), *(const uint2*)(sbs + at));
        }
    }
  };
  for (int s = s0; s < s1; s += 2 * U) {
    compute(b0, s);
    if (s + U >= s1) break;
    if (s + 2 * U < s1) fetch(b0, s + 2 * U);
    compute(b1, s + U);
    if (s + 3 * U < s1) fetch(b1, s + 3 * U);
  }

  // ---- range partials summed in range order
  red[bw][kp][lane] = acc;
  __syncthreads();
  // acc[r] of lane (r16, g4) = row 16 band + 4 g4 + r of token row r16
  if constexpr (EPI == EPI_SWIGLU_MIX) {
    // lanes g4 = 0, 1 hold gate rows 4 g4 + r (features 16 (m / 2) + 8 (m % 2) + 4 g4 + r), lanes
    // g4 + 2 the up rows of the same features
    if (wave != 0) {
      if constexpr (CH != 0) chain_signal(a.chain);
      return;
    }
    f32x4 tsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWB; ++w) {
      const f32x4 o = red[0][w][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) tsum[r] += o[r];
    }
    float us[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) us[r] = __shfl_xor(tsum[r], 32, 64);
    if (g4 < 2 && r16 < B) {
      const float c = sinv[r16];
      const int f = (blockIdx.x >> 1) * 16 + (blockIdx.x & 1) * 8 + g4 * 4;
      f16x4 hv, lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gg = __fmul_rn(tsum[r], c), uu = __fmul_rn(us[r], c);
        const float m = __fmul_rn(__fdiv_rn(gg, 1.0f + expf(-gg)), uu);
        f16 h, l;
        split_f16(m, h, l);
        hv[r] = h;
        lv[r] = l;
      }
      f16* dh = a.mhi + (int64_t)r16 * a.ldm + f;
      f16* dl = a.mlo + (int64_t)r16 * a.ldm + f;
      if constexpr (CH != 0) {
        st_dev8(dh, __builtin_bit_cast(uint64_t, hv));
        st_dev8(dl, __builtin_bit_cast(uint64_t, lv));
      } else {
        *(f16x4*)dh = hv;
        *(f16x4*)dl = lv;
      }
    }
    if constexpr (CH != 0) chain_signal(a.chain);
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
    static_assert(NBW == 2, "gate and up bands");
    if (wave != 0) {
      if constexpr (CH != 0) chain_signal(a.chain);
      return;
    }
    f32x4 gs = {0.f, 0.f, 0.f, 0.f}, us = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWB; ++w) {
      const f32x4 o0 = red[0][w][lane], o1 = red[1][w][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gs[r] += o0[r];
        us[r] += o1[r];
      }
    }
    if (r16 < B) {
      const float c = sinv[r16];
      const int f = blockIdx.x * 16 + g4 * 4;          // band pair blockIdx.x: features 16 j ..
      f16x4 hv, lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gg = __fmul_rn(gs[r], c), uu = __fmul_rn(us[r], c);
        const float m = __fmul_rn(__fdiv_rn(gg, 1.0f + expf(-gg)), uu);
        f16 h, l;
        split_f16(m, h, l);
        hv[r] = h;
        lv[r] = l;
      }
      f16* dh = a.mhi + (int64_t)r16 * a.ldm + f;
      f16* dl = a.mlo + (int64_t)r16 * a.ldm + f;
      if constexpr (CH != 0) {
        st_dev8(dh, __builtin_bit_cast(uint64_t, hv));
        st_dev8(dl, __builtin_bit_cast(uint64_t, lv));
      } else {
        *(f16x4*)dh = hv;
        *(f16x4*)dl = lv;
      }
    }
    if constexpr (CH != 0) chain_signal(a.chain);
    return;
  }
  if (kp != 0) {
    if constexpr (CH != 0) chain_signal(a.chain);
    return;
  }
  f32x4 tsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < NWB; ++w) {
    const f32x4 o = red[bw][w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) tsum[r] += o[r];
  }
  if (r16 < B) {
    float* dst = a.y + (int64_t)r16 * a.ldy + n;
    const float4 o = yold;
    const float4 out =
        EPI == EPI_ADD
            ? make_float4(__fadd_rn(o.x, __fmul_rn(tsum[0], a.yscale)), __fadd_rn(o.y, __fmul_rn(tsum[1], a.yscale)),
                          __fadd_rn(o.z, __fmul_rn(tsum[2], a.yscale)), __fadd_rn(o.w, __fmul_rn(tsum[3], a.yscale)))
            : make_float4(tsum[0], tsum[1], tsum[2], tsum[3]);
    if constexpr (CH != 0)
      st_dev16(dst, __builtin_bit_cast(uint4, out));
    else
      *(float4*)dst = out;
  }
  if (EPI == EPI_STORE && a.cand) {
    // argmax candidate of the band's 16 rows for token row r16: (value, index), lowest index on ties
    float bv = tsum[0];
    int bi = n;
#pragma unroll
    for (int r = 1; r < 4; ++r)
      if (tsum[r] > bv) {
        bv = tsum[r];
        bi = n + r;
      }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (g4 == 0 && r16 < B) a.cand[(int64_t)r16 * (a.N / 16) + band] = make_float2(bv, __int_as_float(bi));
  }
  if constexpr (CH != 0) chain_signal(a.chain);
}

// Whether the whole-K path can take B rows of a K-wide operand.
bool gemv_full_fits(int K, int B) { return B >= 1 && B <= kFullMaxB && (size_t)4 * B * K + 16 <= kFullMaxLds; }

// S = waves per band = K ranges; EPI_SWIGLU takes band pairs (gate, up). Requires
// K % (32 * S) == 0, N % (16 * bands per workgroup) == 0, and for XF_NORM K <= 4096.
// A launch of a decode chain (a.chain.cnt set) runs the CH kernels, any-order when it waits;
// *nwg (if not null) receives the number of workgroups launched.
hipError_t launch_gemv_full(int mode, int epi, int S, const FullArgs& a, hipStream_t st, int* nwg) {
  if (!gemv_full_fits(a.K, a.B) || a.K % (32 * S) != 0 || a.N % 16 != 0) return hipErrorInvalidValue;
  if (mode == XF_NORM && (a.K > 4096 || !a.xres || !a.nw)) return hipErrorInvalidValue;
  const int chm = !a.chain.cnt ? 0 : a.chain.wait ? 1 : 2;
  if (chm && (a.cand || (a.chain.wait && !a.chain.err))) return hipErrorInvalidValue;
  const int qm = a.Wb ? WM_A4 : a.Wq ? WM_Q8 : WM_BF16;
  const size_t shm = (size_t)4 * a.B * a.K + 16;
  const unsigned flags = a.chain.wait ? hipExtAnyOrderLaunch : 0u;
  const void* const wsrc_ = qm == WM_BF16 ? (const void*)a.W : (const void*)a.Wq;
#define FULL_CH(Q, NWB, NBW, U, MO, EP, MB)                                                                   \
  do {                                                                                                        \
    if (chm == 1)                                                                                             \
      GQA_LAUNCH_F((gemv_full_kernel<Q, NWB, NBW, U, MO, EP, MB, 1>), dim3(a.N / 16 / NBW),                   \
                   dim3(64 * NWB * NBW), shm_, st, flags, wsrc_, a.K, a);                                                  \
    else if (chm == 2)                                                                                        \
      GQA_LAUNCH((gemv_full_kernel<Q, NWB, NBW, U, MO, EP, MB, 2>), dim3(a.N / 16 / NBW),                     \
                 dim3(64 * NWB * NBW), shm_, st, wsrc_, a.K, a);                                                           \
    else                                                                                                      \
      GQA_LAUNCH((gemv_full_kernel<Q, NWB, NBW, U, MO, EP, MB, 0>), dim3(a.N / 16 / NBW),                     \
                 dim3(64 * NWB * NBW), shm_, st, wsrc_, a.K, a);                                                           \
  } while (0)
#define FULL(Q, NWB, NBW, U, MO, EP)                                                                          \
  do {                                                                                                        \
    const size_t shm_ = shm + (Q == WM_BF16 ? 0 : (size_t)NBW * (a.K / 32) * 32 * (Q == WM_A4 ? 2 : 1));    \
    if (nwg) *nwg = a.N / 16 / NBW;                                                                           \
    if (a.B == 1 && (size_t)4 * a.K + 16 <= kFullMaxLds / 4)                                                  \
      FULL_CH(Q, NWB, NBW, U, MO, EP, 1);                                                                     \
    else                                                                                                      \
      FULL_CH(Q, NWB, NBW, U, MO, EP, kFullMaxB);                                                             \
  } while (0)
#define FULL_NC(NWB, NBW)                                                                                     \
  do {                                                                                                        \
    if (nwg) *nwg = a.N / 16 / NBW;                                                                           \
    if (a.B == 1 && (size_t)4 * a.K + 16 <= kFullMaxLds / 4)                                                  \
      GQA_LAUNCH((gemv_full_kernel<WM_BF16, NWB, NBW, kULm, XF_RAW, EPI_STORE, 1, 0>), dim3(a.N / 16 / NBW), \
                 dim3(64 * NWB * NBW), shm, st, wsrc_, a.K, a);                                                            \
    else                                                                                                      \
      GQA_LAUNCH((gemv_full_kernel<WM_BF16, NWB, NBW, kULm, XF_RAW, EPI_STORE, kFullMaxB, 0>),            \
                 dim3(a.N / 16 / NBW), dim3(64 * NWB * NBW), shm, st, wsrc_, a.K, a);                                      \
  } while (0)
#define BY_QM(NWB, NBW, UB, UQ, MO, EP)    \
  do {                                     \
    if (qm == WM_A4)                       \
      FULL(WM_A4, NWB, NBW, UQ, MO, EP);   \
    else if (qm == WM_Q8)                  \
      FULL(WM_Q8, NWB, NBW, UQ, MO, EP);   \
    else                                   \
      FULL(WM_BF16, NWB, NBW, UB, MO, EP); \
  } while (0)
  if (epi == EPI_SWIGLU) {
    if (mode != XF_NORM || S != 4 || a.N % 32 != 0) return hipErrorInvalidValue;
    if (qm == WM_BF16 && GQA_GATEUP_MIXED)
      FULL(WM_BF16, 4, 1, kUGu, XF_NORM, EPI_SWIGLU_MIX);
    else
      BY_QM(4, 2, kUGu, kUGuQ, XF_NORM, EPI_SWIGLU);
  } else if (S == 8) {
    if (mode == XF_NORM) {
      if (epi != EPI_STORE) return hipErrorInvalidValue;
      BY_QM(8, 1, kUQkv, kUQkvQ, XF_NORM, EPI_STORE);
    } else if (epi == EPI_ADD) {
      BY_QM(8, 1, kUOd, kUOdQ, XF_RAW, EPI_ADD);
    } else {
      BY_QM(8, 1, 4, 4, XF_RAW, EPI_STORE);
    }
  } else if (S == 1) {
    if (mode != XF_RAW || epi != EPI_STORE || qm != WM_BF16) return hipErrorInvalidValue;
    if (chm) return hipErrorInvalidValue;                // the lm_head is not part of a chain
    if (a.N % 64 == 0)
      FULL_NC(1, 4);
    else
      FULL_NC(1, 1);
  } else {
    return hipErrorInvalidValue;
  }
#undef BY_QM
#undef FULL
#undef FULL_CH
#undef FULL_NC
  return hipGetLastError();
}

}  // namespace gqa
