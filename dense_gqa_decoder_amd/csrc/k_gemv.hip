// Decode projections for 1..32 token rows: P[s][b][n] = sum_{k in split s} W[n][k] * x[b][k].
//
// HBM-streaming matvec: each wave owns a 16-row weight band (tile-major, so the band is one
// contiguous stretch of memory and every wave-wide load is a whole kilobyte) and streams it over
// the workgroup's K-split with 16-byte loads in stages of eight 32-wide K-steps, double-buffered so
// the next stage's weight loads are in flight during the current stage's MFMAs, and multiplies
// them on the matrix cores against the token rows as the 16-wide N side
// (v_mfma_f32_16x16x32_f16, FP16 hi/lo activations, FP32 accumulate); the four waves of a
// workgroup share the operand rows in LDS. The token count B only widens the padded N side:
// every output column runs the same instruction sequence in the same K order whatever B is, so a
// row evaluated in a batch is bit-identical to the same row evaluated alone (Kipp Roadmap,
// status v0.0.2: batched-equals-isolated).
//
// Split-K (Kipp Roadmap, status v0.0.4: the split-K partial buffer has its own constant): each
// split writes a partial P[s][b][n]; consumers sum the splits in a fixed order. Q8_0 weights
// (Kipp Model Support, "Quantization (Q8_0)") take one MFMA per 32-weight quant block into a
// fresh accumulator, scaled by the block's fp16 scale in FP32; the 16 scales of a tile are
// contiguous, so a lane's four row scales are one 8-byte load.
//
// For B <= 4 the activation rows of the workgroup's K range are built in LDS by a prologue that
// performs the producer's elementwise step (X_RAW copy, X_RESID residual add times the norm
// weight, X_SWIGLU silu(g) * u), so no separate kernel runs between two projections. The RMSNorm
// 1/rms factor is a per-row scalar, so it is applied after the projection by its consumer; the
// prologue only touches its own K range. For B > 4 the same arithmetic runs in rows_kernel into
// global memory (same element-to-thread mapping and reduction order) and the matvec reads its
// operands there.
#include "gqa_common.h"

namespace gqa {

constexpr int kGemvWaves = 4;
constexpr int kGemvStage = 8;     // 32-wide K-steps per pipeline stage
constexpr int kXldsMaxRows = 4;

// Operand element e (absolute K index) of row b for the X_RESID / X_SWIGLU modes, and the
// residual value (X_RESID) for the sum of squares. Thread t of a 256-thread block owns elements
// k0 + t + 256 j of a K range; partial sums are added in split order.
struct ElemOut {
  float y;    // operand value before the hi/lo split
  float x;    // X_RESID: updated residual value
};

__device__ __forceinline__ void resid_elems(const XSrc& xs, int b, int k0, int klen, int jbeg, float (&xv)[4],
                                            float (&yv)[4]) {
  const int t = threadIdx.x;
  float rv[4], acc[4];
  float pv[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int off = t + 256 * (jbeg + q);
    const bool ok = off < klen;
    rv[q] = ok ? xs.res[(int64_t)b * xs.H + k0 + off] : 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < xs.nsplit) pv[q][s] = ok ? xs.part[(int64_t)s * xs.pstride + (int64_t)b * xs.pld + k0 + off] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[q] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < xs.nsplit) acc[q] += pv[q][s];
    const int off = t + 256 * (jbeg + q);
    xv[q] = xs.nsplit > 0 ? __fadd_rn(rv[q], __fmul_rn(acc[q], xs.pscale)) : rv[q];
    yv[q] = off < klen ? __fmul_rn(xv[q], bf16_bits_to_f32(xs.w[k0 + off])) : 0.f;
  }
}

__device__ __forceinline__ float swiglu_elem(const XSrc& xs, int b, int f, float c) {
  const int64_t rg = (int64_t)32 * (f / 16) + (f % 16);
  float g = 0.f, u = 0.f;
  for (int s = 0; s < xs.gu_split; ++s) {
    const float* p = xs.gu + (int64_t)s * xs.gu_stride + (int64_t)b * xs.gu_ld;
    g += p[rg];
    u += p[rg + 16];
  }
  g = __fmul_rn(g, c);
  u = __fmul_rn(u, c);
  return __fmul_rn(__fdiv_rn(g, 1.0f + expf(-g)), u);
}

// Builds the operand rows of one K range [k0, k0 + klen) of row b. dst(e_off, hi, lo) stores
// one element; with `writer`, X_RESID also stores x to res_out and returns the range's sum of
// squares (thread order, then the 64 lanes, then the four waves) in ss_out[range][b].
template <class Store>
__device__ __forceinline__ void build_range(const XSrc& xs, int b, int k0, int klen, int range, bool writer,
                                            float* red, Store dst) {
  const int nj = (klen + 255) / 256;
  if (xs.mode == X_RESID) {
    float ssq = 0.f;
    for (int j0 = 0; j0 < nj; j0 += 4) {
      float xv[4], yv[4];
      resid_elems(xs, b, k0, klen, j0, xv, yv);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int off = threadIdx.x + 256 * (j0 + q);
        if (off < klen) {
          f16 h, l;
          split_f16(yv[q], h, l);
          dst(off, h, l);
          if (writer) {
            xs.res_out[(int64_t)b * xs.H + k0 + off] = xv[q];
            ssq = __fadd_rn(ssq, __fmul_rn(xv[q], xv[q]));
          }
        }
      }
    }
    if (writer) {
      ssq = wave_sum(ssq);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ssq;
      __syncthreads();
      if (threadIdx.x == 0) xs.ss_out[range * 32 + b] = __fadd_rn(__fadd_rn(__fadd_rn(red[0], red[1]), red[2]), red[3]);
      __syncthreads();
    }
  } else if (xs.mode == X_SWIGLU) {
    const float c = inv_rms_from_ss(xs.ss, xs.ss_n, b, xs.H, xs.eps);
    for (int off = threadIdx.x; off < klen; off += 256) {
      f16 h, l;
      split_f16(swiglu_elem(xs, b, k0 + off, c), h, l);
      dst(off, h, l);
    }
  }
}

template <int QM, int NT, bool XLDS>
__global__ __launch_bounds__(64 * kGemvWaves) void gemv_kernel(const uint16_t* __restrict__ W,
                                                               const int8_t* __restrict__ Wq,
                                                               const f16* __restrict__ Wd,
                                                               const f16* __restrict__ Wb, int K, int N, XSrc xs,
                                                               int B, int klen, float* __restrict__ P,
                                                               int64_t part_stride, int ldp,
                                                               float2* __restrict__ cand) {
  constexpr int U = kGemvStage;
  constexpr int NW = kGemvWaves;
  __shared__ float red[4];
  extern __shared__ f16 sx[];                     // XLDS: [B][2][klen] (hi, lo)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int tile = blockIdx.x * NW + wave;        // 16-row tile of this wave
  const bool has_tile = tile * 16 < N;
  const int n0 = (has_tile ? tile : 0) * 16;
  const int s = blockIdx.y;
  const int k0 = s * klen;
  const int kb = k0, ke = k0 + klen;

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the wave's 16-row band is contiguous (tile-major weights): chunk ks at band + ks * 512
  const int64_t band = (int64_t)(n0 >> 4) * (K >> 5);
  struct Buf {
    uint4 wv[U];
    uint2 qv[U];
    uint32_t q4[U];
    uint2 sc[U];
    uint2 bs[U];
  };
  auto fetch = [&](Buf& f, int k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k + u * 32;
      const bool ok = kk < ke && has_tile;
      const int64_t chunk = band + (kk >> 5);
      if (QM == WM_Q8) {
        f.qv[u] = ok ? *(const uint2*)(Wq + chunk * 512 + lane * 8) : uint2{0, 0};
        f.sc[u] = ok ? *(const uint2*)(Wd + chunk * 16 + g4 * 4) : uint2{0, 0};
      } else if (QM == WM_A4) {
        f.q4[u] = ok ? *(const uint32_t*)(Wq + chunk * 256 + lane * 4) : 0u;
        f.sc[u] = ok ? *(const uint2*)(Wd + chunk * 16 + g4 * 4) : uint2{0, 0};
        f.bs[u] = ok ? *(const uint2*)(Wb + chunk * 16 + g4 * 4) : uint2{0, 0};
      } else {
        f.wv[u] = ok ? *(const uint4*)(W + chunk * 512 + lane * 8) : uint4{0, 0, 0, 0};
      }
    }
  };
  constexpr int STEP = 32 * U;
  Buf b0, b1;
  fetch(b0, kb);   // first weight stage in flight during the prologue

  const f16* xh[NT];
  const f16* xl[NT];
  bool xv[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int b = j * 16 + r16;
    xv[j] = b < B;
    if (XLDS) {
      xh[j] = sx + (int64_t)(xv[j] ? b : 0) * 2 * klen + g4 * 8 - k0;
      xl[j] = xh[j] + klen;
    } else {
      xh[j] = xs.hi + (int64_t)(xv[j] ? b : 0) * xs.ld + g4 * 8;
      xl[j] = xs.lo + (int64_t)(xv[j] ? b : 0) * xs.ld + g4 * 8;
    }
  }
  if (XLDS) {
    if (xs.mode == X_RAW) {
      const int per_row = klen / 8;
      for (int c = threadIdx.x; c < B * 2 * per_row; c += 64 * NW) {
        int b = c / (2 * per_row), rem = c - b * 2 * per_row, hl = rem / per_row, q = rem - hl * per_row;
        const f16* src = (hl ? xs.lo : xs.hi) + (int64_t)b * xs.ld + k0 + q * 8;
        *(uint4*)(sx + (int64_t)b * 2 * klen + hl * klen + q * 8) = *(const uint4*)src;
      }
    } else {
      const bool writer = blockIdx.x == 0;
      for (int b = 0; b < B; ++b) {
        f16* row = sx + (int64_t)b * 2 * klen;
        build_range(xs, b, k0, klen, s, writer, red, [&](int off, f16 h, f16 l) {
          row[off] = h;
          row[klen + off] = l;
        });
      }
    }
    __syncthreads();
  }
  if (!has_tile) return;

  auto compute = [&](const Buf& f, int k) {
    if constexpr (QM == WM_BF16) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k + u * 32;
        const bool ok = kk < ke;
        const f16x8 a = bf16x8_to_f16x8(f.wv[u]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const f16x8 bh = (ok && xv[j]) ? *(const f16x8*)(xh[j] + kk) : f16x8{};
          const f16x8 bl = (ok && xv[j]) ? *(const f16x8*)(xl[j] + kk) : f16x8{};
          acc[j] = mfma16(a, bh, acc[j]);
          acc[j] = mfma16(a, bl, acc[j]);
        }
      }
    } else {
      // four steps' block products at a time, then their scaled accumulation in step order
      constexpr int G = 4;
#pragma unroll
      for (int u0 = 0; u0 < U; u0 += G) {
        f32x4 p[G][NT], xs[G][NT];
#pragma unroll
        for (int v = 0; v < G; ++v) {
          const int u = u0 + v, kk = k + u * 32;
          const bool ok = kk < ke;
          const f16x8 a = qwiden<QM>(f.qv[u], f.q4[u]);
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const f16x8 bh = (ok && xv[j]) ? *(const f16x8*)(xh[j] + kk) : f16x8{};
            const f16x8 bl = (ok && xv[j]) ? *(const f16x8*)(xl[j] + kk) : f16x8{};
            qstep_products<QM>(a, bh, bl, p[v][j], xs[v][j]);
          }
        }
#pragma unroll
        for (int v = 0; v < G; ++v)
#pragma unroll
          for (int j = 0; j < NT; ++j) qstep_accumulate<QM>(acc[j], p[v][j], xs[v][j], f.sc[u0 + v], f.bs[u0 + v]);
      }
    }
  };
  // Steps past ke load zeros (weights and activations), so they add exact zeros.
  int k = kb;
  while (true) {
    if (k + STEP < ke) fetch(b1, k + STEP);
    compute(b0, k);
    k += STEP;
    if (k >= ke) break;
    if (k + STEP < ke) fetch(b0, k + STEP);
    compute(b1, k);
    k += STEP;
    if (k >= ke) break;
  }

  // acc[j][r] = value of weight row n0 + 4*g4 + r for token row j*16 + r16.
  const int n = n0 + g4 * 4;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int b = j * 16 + r16;
    if (b < B) {
      float4 v = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      *(float4*)&P[(int64_t)s * part_stride + (int64_t)b * ldp + n] = v;
    }
    if (cand) {
      // argmax candidate of these 16 rows for token row b: (value, index), lowest index on ties
      float bv = acc[j][0];
      int bi = n;
#pragma unroll
      for (int r = 1; r < 4; ++r)
        if (acc[j][r] > bv) {
          bv = acc[j][r];
          bi = n + r;
        }
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (g4 == 0 && b < B) cand[(int64_t)b * (N / 16) + tile] = make_float2(bv, __int_as_float(bi));
    }
  }
}

// B > 4 token rows (X_RAW operands in global memory). The operand rows of the workgroup's K
// range pass through LDS kRowsStageK K-elements at a time: per stage each staged row is one
// wave-wide direct-to-LDS copy (hi then lo half), double-buffered, shared by the eight waves (eight 16-row
// bands) of the workgroup, so the activations cross the L2-to-CU path once per workgroup instead
// of once per wave. Each wave streams its band's weights one stage ahead in registers and runs
// the same MFMA chain per (band, K range) as gemv_kernel, so the partials are bit-identical to
// the B <= 4 paths. The weight loads and copies are unconditional (clamped addresses; steps past
// the range are skipped in compute), so a wave issues exactly the same number per stage and one
// vmcnt wait covers a stage's operand copies and the weights of the stage before.
constexpr int kRowsWaves = 8;
#ifndef GQA_ROWS_STAGE_K
#define GQA_ROWS_STAGE_K 128
#endif
constexpr int kRowsStageK = GQA_ROWS_STAGE_K;   // 128: 34 KB of staged rows for 32 tokens, four workgroups per CU
static_assert(kRowsStageK % 128 == 0 && kRowsStageK <= 256, "whole groups of four K-steps, one copy per row");
constexpr int kRowsPitch = 2 * kRowsStageK + 8;   // f16 per staged row: hi | lo | 16 bytes pad

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int QM, int NT>
__global__ __launch_bounds__(64 * kRowsWaves) void gemv_rows_kernel(const uint16_t* __restrict__ W,
                                                                   const int8_t* __restrict__ Wq,
                                                                   const f16* __restrict__ Wd,
                                                                   const f16* __restrict__ Wb, int K, int N, XSrc xs,
                                                                   int B, int klen, float* __restrict__ P,
                                                                   int64_t part_stride, int ldp,
                                                                   float2* __restrict__ cand) {
  constexpr int U = kRowsStageK / 32;                 // K-steps per stage
  constexpr int ROWS = 16 * NT;                       // staged token rows
  constexpr int RPW = ROWS / kRowsWaves;              // staged rows copied per wave
  constexpr int BUF = ROWS * kRowsPitch;              // f16 per buffer
  constexpr int NF = QM == WM_Q8 ? 2 * U : QM == WM_A4 ? 3 * U : U;   // weight loads per stage and wave
  __shared__ __attribute__((aligned(16))) f16 sx[2 * BUF];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int tile = blockIdx.x * kRowsWaves + wave;
  const bool has_tile = tile * 16 < N;
  const int n0 = (has_tile ? tile : 0) * 16;
  const int s = blockIdx.y;
  const int k0 = s * klen, ke = k0 + klen;
  const int nstage = (klen + kRowsStageK - 1) / kRowsStageK;
  const int64_t band = (int64_t)(n0 >> 4) * (K >> 5);

  struct Buf {
    uint4 wv[U];
    uint2 qv[U];
    uint32_t q4[U];
    uint2 sc[U];
    uint2 bs[U];
  };
  auto fetch = [&](Buf& f, int t) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(k0 + t * kRowsStageK + u * 32, ke - 32);
      const int64_t chunk = band + (kk >> 5);
      if (QM == WM_Q8) {
        f.qv[u] = *(const uint2*)(Wq + chunk * 512 + lane * 8);
        f.sc[u] = *(const uint2*)(Wd + chunk * 16 + g4 * 4);
      } else if (QM == WM_A4) {
        f.q4[u] = *(const uint32_t*)(Wq + chunk * 256 + lane * 4);
        f.sc[u] = *(const uint2*)(Wd + chunk * 16 + g4 * 4);
        f.bs[u] = *(const uint2*)(Wb + chunk * 16 + g4 * 4);
      } else {
        f.wv[u] = *(const uint4*)(W + chunk * 512 + lane * 8);
      }
    }
  };
  // stage t's operand rows into buffer t & 1, one wave-wide copy per row: lane l brings 16 bytes
  // to byte 16 l of the row's slot, lanes [0, P) the hi piece and [P, 2 P) the lo piece with
  // P = kRowsStageK / 8; lanes past 2 P (a stage shorter than 256) copy nothing, which leaves the
  // number of copies a wave issues per stage unchanged
  constexpr int P8 = kRowsStageK / 8;
  static_assert(2 * P8 <= 64 && 16 * 2 * P8 <= 2 * kRowsPitch, "one copy per staged row");
  auto issue_x = [&](int t) {
    const int hl = lane >= P8;
    const int kk = min(k0 + t * kRowsStageK + (lane % P8) * 8, ke - 8);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = wave * RPW + i;
      const f16* src = (hl ? xs.lo : xs.hi) + (int64_t)min(row, B - 1) * xs.ld + kk;
      if (2 * P8 == 64 || lane < 2 * P8) lds_dma16(src, sx + (t & 1) * BUF + row * kRowsPitch);
    }
  };

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Buf& f, int t) {
    const f16* xb = sx + (t & 1) * BUF + r16 * kRowsPitch + g4 * 8;
    if constexpr (QM == WM_BF16) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k0 + t * kRowsStageK + u * 32 >= ke) break;
        const f16x8 a = bf16x8_to_f16x8(f.wv[u]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const f16x8 bh = *(const f16x8*)(xb + j * 16 * kRowsPitch + u * 32);
          const f16x8 bl = *(const f16x8*)(xb + j * 16 * kRowsPitch + kRowsStageK + u * 32);
          acc[j] = mfma16(a, bh, acc[j]);
          acc[j] = mfma16(a, bl, acc[j]);
        }
      }
    } else {
      // four steps' block products at a time, then their scaled accumulation in step order
      constexpr int G = 4;
#pragma unroll
      for (int u0 = 0; u0 < U; u0 += G) {
        f32x4 p[G][NT], xs[G][NT];
#pragma unroll
        for (int v = 0; v < G; ++v) {
          const int u = u0 + v;
          if (k0 + t * kRowsStageK + u * 32 >= ke) break;
          const f16x8 a = qwiden<QM>(f.qv[u], f.q4[u]);
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const f16x8 bh = *(const f16x8*)(xb + j * 16 * kRowsPitch + u * 32);
            const f16x8 bl = *(const f16x8*)(xb + j * 16 * kRowsPitch + kRowsStageK + u * 32);
            qstep_products<QM>(a, bh, bl, p[v][j], xs[v][j]);
          }
        }
#pragma unroll
        for (int v = 0; v < G; ++v) {
          if (k0 + t * kRowsStageK + (u0 + v) * 32 >= ke) break;
#pragma unroll
          for (int j = 0; j < NT; ++j) qstep_accumulate<QM>(acc[j], p[v][j], xs[v][j], f.sc[u0 + v], f.bs[u0 + v]);
        }
      }
    }
  };

  // issue order per wave: weights(0), x(0), weights(1), then per stage t: x(t+1), weights(t+2);
  // so when stage t starts, only weights(t+1) may still be in flight after x(t).
  // Every stage issues the same copies and loads (past the range they repeat the last piece, an
  // L2 hit, into the buffer not being read), so every path has the same number in flight.
  Buf b0, b1;
  fetch(b0, 0);
  issue_x(0);
  fetch(b1, 1);
  auto stage = [&](Buf& f, int t) {
    vm_wait<NF>();                                    // x(t) and everything before it have landed
    __syncthreads();                                  // stage t's rows are in LDS; buffer (t+1)&1 is free
    issue_x(t + 1);
    compute(f, t);
    fetch(f, t + 2);
  };
  for (int t = 0; t < nstage; t += 2) {               // unrolled by two: b0 and b1 keep their registers
    stage(b0, t);
    if (t + 1 >= nstage) break;
    stage(b1, t + 1);
  }
  vm_wait<0>();                                       // no copy into LDS outlives the workgroup
  if (!has_tile) return;

  // acc[j][r] = value of weight row n0 + 4*g4 + r for token row j*16 + r16.
  const int n = n0 + g4 * 4;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int b = j * 16 + r16;
    if (b < B) {
      const float4 v = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      *(float4*)&P[(int64_t)s * part_stride + (int64_t)b * ldp + n] = v;
    }
    if (cand) {
      float bv = acc[j][0];
      int bi = n;
#pragma unroll
      for (int r = 1; r < 4; ++r)
        if (acc[j][r] > bv) {
          bv = acc[j][r];
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
      if (g4 == 0 && b < B) cand[(int64_t)b * (N / 16) + tile] = make_float2(bv, __int_as_float(bi));
    }
  }
}

// B > 4: the prologue arithmetic of one K range of one row into global hi/lo rows
// (grid: ranges x rows, 256 threads) -- the same element mapping and order as the LDS path.
__global__ __launch_bounds__(256) void rows_kernel(XSrc xs, int klen, f16* __restrict__ yhi, f16* __restrict__ ylo,
                                                   int ldy) {
  __shared__ float red[4];
  const int s = blockIdx.x, b = blockIdx.y, k0 = s * klen;
  f16* hrow = yhi + (int64_t)b * ldy + k0;
  f16* lrow = ylo + (int64_t)b * ldy + k0;
  build_range(xs, b, k0, klen, s, true, red, [&](int off, f16 h, f16 l) {
    hrow[off] = h;
    lrow[off] = l;
  });
}

// Requires K % (32 * nsplit) == 0 and N % 16 == 0. Each wave streams one 16-row tile over the
// workgroup's K range; a workgroup holds four tiles that share one operand prologue. With
// B <= 4 the operand rows are built in LDS by the xs.mode prologue; with B > 4 xs must be X_RAW
// over global FP16 hi/lo rows.
// cand (optional, nsplit == 1): per token row b and 16-row tile t, the tile's (max value, index
// as float bits) at cand[b * (N / 16) + t], for a following argmax reduction.
// staged: use the LDS-staged kernel for any B (X_RAW rows only).
hipError_t launch_gemv(const uint16_t* W, const int8_t* Wq, const f16* Wd, const f16* Wb, int K, int N, const XSrc& xs,
                       int B, int nsplit, float* P, int64_t part_stride, int ldp, float2* cand, hipStream_t st,
                       bool staged) {
  if (B < 1 || B > kMaxBatch || nsplit < 1 || K % (32 * nsplit) != 0 || N % 16 != 0) return hipErrorInvalidValue;
  if (cand && nsplit != 1) return hipErrorInvalidValue;
  const bool lds = B <= kXldsMaxRows && !staged;
  if (!lds && xs.mode != X_RAW) return hipErrorInvalidValue;
  if (xs.mode == X_RESID && (xs.nsplit > 8 || xs.H != K)) return hipErrorInvalidValue;
  dim3 grid((N / 16 + kGemvWaves - 1) / kGemvWaves, nsplit);
  const int klen = K / nsplit;
  const size_t shm = lds ? (size_t)B * klen * 4 : 0;
  if (shm > 64 * 1024) return hipErrorInvalidValue;
  const dim3 blk(64 * kGemvWaves);
#define GEMV_LAUNCH(QM, NT, L)                                                                                   \
  GQA_LAUNCH((gemv_kernel<QM, NT, L>), grid, blk, shm, st, W, Wq, Wd, Wb, K, N, xs, B, klen, P, part_stride, ldp, cand)
  const int qm = Wb ? WM_A4 : Wq ? WM_Q8 : WM_BF16;
  if (lds) {
    if (qm == WM_A4) GEMV_LAUNCH(WM_A4, 1, true);
    else if (qm == WM_Q8) GEMV_LAUNCH(WM_Q8, 1, true);
    else GEMV_LAUNCH(WM_BF16, 1, true);
  } else {
    const dim3 rgrid((N / 16 + kRowsWaves - 1) / kRowsWaves, nsplit), rblk(64 * kRowsWaves);
#define ROWS_LAUNCH(QM, NT)                                                                                      \
  GQA_LAUNCH((gemv_rows_kernel<QM, NT>), rgrid, rblk, 0, st, W, Wq, Wd, Wb, K, N, xs, B, klen, P, part_stride, ldp, \
             cand)
    if (B <= 16) {
      if (qm == WM_A4) ROWS_LAUNCH(WM_A4, 1);
      else if (qm == WM_Q8) ROWS_LAUNCH(WM_Q8, 1);
      else ROWS_LAUNCH(WM_BF16, 1);
    } else {
      if (qm == WM_A4) ROWS_LAUNCH(WM_A4, 2);
      else if (qm == WM_Q8) ROWS_LAUNCH(WM_Q8, 2);
      else ROWS_LAUNCH(WM_BF16, 2);
    }
#undef ROWS_LAUNCH
  }
#undef GEMV_LAUNCH
  return hipGetLastError();
}

// Operand rows for B > 4 (same K ranges as the matvec that will consume them: nsplit ranges).
hipError_t launch_rows(const XSrc& xs, int K, int nsplit, int B, f16* yhi, f16* ylo, int ldy, hipStream_t st) {
  if (xs.mode == X_RAW || K % nsplit != 0 || (xs.mode == X_RESID && xs.nsplit > 8)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rows_kernel, dim3(nsplit, B), dim3(256), 0, st, xs, K / nsplit, yhi, ylo, ldy);
  return hipGetLastError();
}

// Full RMSNorm of B rows (res + partials, times w, times 1/rms) into global hi/lo: one
// 256-thread block per row; used before the lm_head.
__global__ __launch_bounds__(256) void final_norm_kernel(XSrc xs, f16* __restrict__ yhi, f16* __restrict__ ylo,
                                                         int ldy) {
  __shared__ float red[4];
  const int b = blockIdx.x, H = xs.H;
  float ssq = 0.f;
  const int nj = (H + 255) / 256;
  float xvals[16];
#pragma unroll
  for (int j0 = 0; j0 < 16; j0 += 4) {
    if (j0 < nj) {
      float xv[4], yv[4];
      resid_elems(xs, b, 0, H, j0, xv, yv);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xvals[j0 + q] = xv[q];
        if (threadIdx.x + 256 * (j0 + q) < H) ssq = __fadd_rn(ssq, __fmul_rn(xv[q], xv[q]));
      }
    }
  }
  ssq = wave_sum(ssq);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ssq;
  __syncthreads();
  const float tot = __fadd_rn(__fadd_rn(__fadd_rn(red[0], red[1]), red[2]), red[3]);
  const float inv = 1.0f / sqrtf(tot / (float)H + xs.eps);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = threadIdx.x + 256 * j;
    if (j < nj && e < H) {
      f16 h, l;
      split_f16(__fmul_rn(__fmul_rn(xvals[j], inv), bf16_bits_to_f32(xs.w[e])), h, l);
      yhi[(int64_t)b * ldy + e] = h;
      ylo[(int64_t)b * ldy + e] = l;
    }
  }
}

hipError_t launch_final_norm(const XSrc& xs, int B, f16* yhi, f16* ylo, int ldy, hipStream_t st) {
  if (xs.mode != X_RESID || xs.H > 4096 || xs.nsplit > 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(final_norm_kernel, dim3(B), dim3(256), 0, st, xs, yhi, ylo, ldy);
  return hipGetLastError();
}

}  // namespace gqa
