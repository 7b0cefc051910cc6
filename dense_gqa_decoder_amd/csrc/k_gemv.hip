// Decode projections for 1..32 token rows: P[s][b][n] = sum_{k in split s} W[n][k] * x[b][k].
//
// HBM-streaming matvec: each one-wave workgroup owns 16 weight rows (32 for the fused
// gate/up SwiGLU epilogue) and one K-split, streams its weight bytes once with 16-byte loads
// (eight K-steps of 32 in flight per lane), and multiplies them on the matrix cores against
// the token rows as the 16-wide N side (v_mfma_f32_16x16x32_f16, FP16 hi/lo activations, FP32
// accumulate). The token count B only widens the padded N side: every output column runs the
// same instruction sequence in the same K order whatever B is, so a row evaluated in a batch
// is bit-identical to the same row evaluated alone (Kipp Roadmap, status v0.0.2:
// batched-equals-isolated).
//
// Split-K (Kipp Roadmap, status v0.0.4: the split-K partial buffer has its own constant)
// writes one partial per split; the consumer kernel sums the splits in a fixed order, so the
// result does not depend on scheduling. Q8_0 weights (Kipp Model Support, "Quantization
// (Q8_0)") take one MFMA per quant block into a fresh accumulator, scaled in FP32.
#include "gqa_common.h"

namespace gqa {

template <int EPI, bool Q8, int NT>
__global__ __launch_bounds__(64) void gemv_kernel(const uint16_t* __restrict__ W, const int8_t* __restrict__ Wq,
                                                  const f16* __restrict__ Wd, int K, int N,
                                                  const f16* __restrict__ Xhi, const f16* __restrict__ Xlo, int ldx,
                                                  int B, int klen, float* __restrict__ P, int64_t part_stride,
                                                  int ldp, f16* __restrict__ Mhi, f16* __restrict__ Mlo, int ldm,
                                                  float m_scale) {
  constexpr int NA = EPI == EPI_SWIGLU ? 2 : 1;  // weight tiles per wave (gate, up)
  const int lane = threadIdx.x;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int n0 = blockIdx.x * 16 * NA;
  const int s = blockIdx.y;
  const int kb = s * klen, ke = kb + klen;

  f32x4 acc[NA][NT];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[a][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const f16* xh[NT];
  const f16* xl[NT];
  bool xv[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    int b = j * 16 + r16;
    xv[j] = b < B;
    xh[j] = Xhi + (int64_t)(xv[j] ? b : 0) * ldx + g4 * 8;
    xl[j] = Xlo + (int64_t)(xv[j] ? b : 0) * ldx + g4 * 8;
  }

  auto step = [&](const f16x8 (&a)[NA], int k, const float (&sc)[NA][4]) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      f16x8 bh = f16x8{}, bl = f16x8{};
      if (xv[j]) {
        bh = *(const f16x8*)(xh[j] + k);
        bl = *(const f16x8*)(xl[j] + k);
      }
#pragma unroll
      for (int aa = 0; aa < NA; ++aa) {
        if (Q8) {
          f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
          p = mfma16(a[aa], bh, p);
          p = mfma16(a[aa], bl, p);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[aa][j][r] = fmaf(sc[aa][r], p[r], acc[aa][j][r]);
        } else {
          acc[aa][j] = mfma16(a[aa], bh, acc[aa][j]);
          acc[aa][j] = mfma16(a[aa], bl, acc[aa][j]);
        }
      }
    }
  };

  constexpr int U = 8;
  int k = kb;
  for (; k + 32 * U <= ke; k += 32 * U) {
    uint4 wv[NA][U];
    uint2 qv[NA][U];
    float sc[NA][U][4];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int64_t row = n0 + aa * 16 + r16;
        int kk = k + u * 32 + g4 * 8;
        if (Q8) {
          qv[aa][u] = *(const uint2*)(Wq + row * K + kk);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sc[aa][u][r] = (float)Wd[(int64_t)(n0 + aa * 16 + g4 * 4 + r) * (K / 32) + (k + u * 32) / 32];
        } else {
          wv[aa][u] = *(const uint4*)(W + row * K + kk);
        }
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f16x8 a[NA];
      float scu[NA][4];
#pragma unroll
      for (int aa = 0; aa < NA; ++aa) {
        if (Q8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[aa][e] = (f16)(float)(int8_t)((qv[aa][u].x >> (8 * e)) & 0xFF);
            a[aa][4 + e] = (f16)(float)(int8_t)((qv[aa][u].y >> (8 * e)) & 0xFF);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) scu[aa][r] = sc[aa][u][r];
        } else {
          a[aa] = bf16x8_to_f16x8(wv[aa][u]);
        }
      }
      step(a, k + u * 32, scu);
    }
  }
  for (; k < ke; k += 32) {
    f16x8 a[NA];
    float scu[NA][4];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa) {
      int64_t row = n0 + aa * 16 + r16;
      int kk = k + g4 * 8;
      if (Q8) {
        uint2 q = *(const uint2*)(Wq + row * K + kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[aa][e] = (f16)(float)(int8_t)((q.x >> (8 * e)) & 0xFF);
          a[aa][4 + e] = (f16)(float)(int8_t)((q.y >> (8 * e)) & 0xFF);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) scu[aa][r] = (float)Wd[(int64_t)(n0 + aa * 16 + g4 * 4 + r) * (K / 32) + k / 32];
      } else {
        a[aa] = bf16x8_to_f16x8(*(const uint4*)(W + row * K + kk));
      }
    }
    step(a, k, scu);
  }

  // acc[aa][j][r] = value of weight row n0 + aa*16 + 4*g4 + r for token row j*16 + r16.
  if (EPI == EPI_SWIGLU) {
    const int f = (n0 / 32) * 16 + g4 * 4;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      int b = j * 16 + r16;
      if (b < B) {
        f16x4 hv, lv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float g = acc[0][j][r], u = acc[NA - 1][j][r];
          float m = g / (1.0f + expf(-g)) * u * m_scale;
          f16 h, l;
          split_f16(m, h, l);
          hv[r] = h;
          lv[r] = l;
        }
        *(f16x4*)&Mhi[(int64_t)b * ldm + f] = hv;
        *(f16x4*)&Mlo[(int64_t)b * ldm + f] = lv;
      }
    }
  } else {
    const int n = n0 + g4 * 4;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      int b = j * 16 + r16;
      if (b < B) {
        float4 v = make_float4(acc[0][j][0], acc[0][j][1], acc[0][j][2], acc[0][j][3]);
        *(float4*)&P[(int64_t)s * part_stride + (int64_t)b * ldp + n] = v;
      }
    }
  }
}

template <int EPI, bool Q8>
static hipError_t launch_gemv_e(const uint16_t* W, const int8_t* Wq, const f16* Wd, int K, int N, const f16* Xhi,
                                const f16* Xlo, int ldx, int B, int nsplit, float* P, int64_t part_stride, int ldp,
                                f16* Mhi, f16* Mlo, int ldm, float m_scale, hipStream_t st) {
  constexpr int NA = EPI == EPI_SWIGLU ? 2 : 1;
  dim3 grid(N / (16 * NA), nsplit);
  int klen = K / nsplit;
  if (B <= 16)
    hipLaunchKernelGGL((gemv_kernel<EPI, Q8, 1>), grid, dim3(64), 0, st, W, Wq, Wd, K, N, Xhi, Xlo, ldx, B, klen, P,
                       part_stride, ldp, Mhi, Mlo, ldm, m_scale);
  else
    hipLaunchKernelGGL((gemv_kernel<EPI, Q8, 2>), grid, dim3(64), 0, st, W, Wq, Wd, K, N, Xhi, Xlo, ldx, B, klen, P,
                       part_stride, ldp, Mhi, Mlo, ldm, m_scale);
  return hipGetLastError();
}

// B <= 16 and B in 17..32 use the same per-column arithmetic (one or two 16-column tiles).
hipError_t launch_gemv(int epi, const uint16_t* W, const int8_t* Wq, const f16* Wd, int K, int N, const f16* Xhi,
                       const f16* Xlo, int ldx, int B, int nsplit, float* P, int64_t part_stride, int ldp, f16* Mhi,
                       f16* Mlo, int ldm, float m_scale, hipStream_t st) {
  if (B < 1 || B > kMaxBatch || nsplit < 1 || K % (32 * nsplit) != 0) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU) {
    if (N % 32 != 0 || nsplit != 1) return hipErrorInvalidValue;
    return Wq ? launch_gemv_e<EPI_SWIGLU, true>(W, Wq, Wd, K, N, Xhi, Xlo, ldx, B, 1, P, part_stride, ldp, Mhi, Mlo,
                                                ldm, m_scale, st)
              : launch_gemv_e<EPI_SWIGLU, false>(W, Wq, Wd, K, N, Xhi, Xlo, ldx, B, 1, P, part_stride, ldp, Mhi, Mlo,
                                                 ldm, m_scale, st);
  }
  if (N % 16 != 0) return hipErrorInvalidValue;
  return Wq ? launch_gemv_e<EPI_STORE, true>(W, Wq, Wd, K, N, Xhi, Xlo, ldx, B, nsplit, P, part_stride, ldp, Mhi,
                                             Mlo, ldm, m_scale, st)
            : launch_gemv_e<EPI_STORE, false>(W, Wq, Wd, K, N, Xhi, Xlo, ldx, B, nsplit, P, part_stride, ldp, Mhi,
                                              Mlo, ldm, m_scale, st);
}

}  // namespace gqa
