// Prefill projections: C[t][n] = sum_k W[n][k] * x[t][k] on the gfx950 matrix cores.
//
// W is BF16 (or Q8_0: int8 quants with an fp16 scale per 32-weight block, Kipp Model
// Support, "Quantization (Q8_0)") [N][K], tile-major (tiled_index): a workgroup's weight tile
// for one K-step is BN/16 contiguous 2 KiB pieces, copied to LDS unchanged, and each 16x32
// MFMA operand is one conflict-free 16-byte LDS read per lane. x is the FP32 activation, held as an
// FP16 hi/lo pair so that two FP16 MFMAs (v_mfma_f32_16x16x32_f16) per K-step give a
// near-FP32 product; accumulation is FP32. BF16 weights become FP16 operands exactly.
// For Q8_0 each 32-wide K-step is one quant block: the int8 quants are exact FP16 operands,
// the MFMA sums q*x over the block into a fresh accumulator and the block scale is applied
// in FP32 afterwards (the dequantisation is done once per LDS tile and reused by every token
// column of the tile).
//
// Tiling: a 256-thread workgroup computes a BN x BT tile (weights rows x tokens), each of its
// four waves a (BN/2) x (BT/2) quadrant built from 16x16 MFMA tiles. K advances 64 per step
// through LDS; the next step's global loads are issued into registers before the MFMAs of the
// current step. N % BN == 0 and K % 64 == 0 are required; T (tokens) may be ragged.
//
// Epilogues: EPI_STORE C = acc * out_scale; EPI_ADD C += acc * out_scale (residual);
// EPI_SWIGLU: the weight rows interleave gate and up in 16-row groups
// (physical rows 32j..32j+15 = gate features 16j.., 32j+16.. = up features 16j..), so each
// lane holds matching gate/up values and writes m = silu(g) * u * m_scale as an FP16 hi/lo
// pair for the down projection.
#include "gqa_common.h"

namespace gqa {

template <int BN, int BT, int EPI, bool Q8>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t* __restrict__ W, const int8_t* __restrict__ Wq,
                                                   const f16* __restrict__ Wd, int K, int N,
                                                   const f16* __restrict__ Xhi, const f16* __restrict__ Xlo, int ldx,
                                                   int T, float* __restrict__ C, int ldc, float out_scale,
                                                   f16* __restrict__ Mhi, f16* __restrict__ Mlo, int ldm,
                                                   float m_scale) {
  constexpr int BK = 64, LD = BK + 8;
  constexpr int WN = BN / 2, WT = BT / 2;        // per-wave quadrant
  constexpr int TN = WN / 16, TT = WT / 16;      // 16x16 tiles per wave
  constexpr int CW = BN * BK / 8 / 256;          // 16-byte weight chunks per thread
  constexpr int CX = BT * BK / 8 / 256;          // 16-byte activation chunks per thread (each of hi, lo)
  static_assert(CW >= 1 && CX >= 1, "tile too small");
  static_assert(BN <= 256, "one scale row per thread");
  __shared__ f16 sW[BN * BK];                    // tile-major, as in memory: [band][k-chunk][lane][8]
  __shared__ f16 sXh[BT * LD];
  __shared__ f16 sXl[BT * LD];
  __shared__ float sD[Q8 ? BN * 2 : 1];          // Q8: block scales of this K-step (2 blocks x BN rows)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = blockIdx.x * BN, t0 = blockIdx.y * BT;
  const int wn = (wave & 1) * WN, wt = (wave >> 1) * WT;

  f32x4 acc[TN][TT];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 rw[CW];
  uint2 rq[Q8 ? CW : 1];
  uint4 rxh[CX], rxl[CX];
  f16 rd0 = (f16)0.f, rd1 = (f16)0.f;

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      // unit c: band c / 128, then 128 consecutive 8-element pieces (two 32-wide chunks)
      const int c = tid + 256 * i;
      const int64_t at = ((int64_t)((n0 >> 4) + (c >> 7)) * (K >> 5) + (k0 >> 5)) * 512 + (c & 127) * 8;
      if (Q8)
        rq[i] = *(const uint2*)(Wq + at);
      else
        rw[i] = *(const uint4*)(W + at);
    }
    if (Q8 && tid < BN) {                          // scales of the two quant blocks of this K-step
      const int64_t at = ((int64_t)((n0 >> 4) + (tid >> 4)) * (K >> 5) + (k0 >> 5)) * 16 + (tid & 15);
      rd0 = Wd[at];
      rd1 = Wd[at + 16];
    }
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      int t = t0 + row;
      if (t < T) {
        rxh[i] = *(const uint4*)(Xhi + (int64_t)t * ldx + k0 + col);
        rxl[i] = *(const uint4*)(Xlo + (int64_t)t * ldx + k0 + col);
      } else {
        rxh[i] = uint4{0, 0, 0, 0};
        rxl[i] = uint4{0, 0, 0, 0};
      }
    }
  };

  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int c = tid + 256 * i;
      f16x8 v;
      if (Q8) {
        uint32_t lo = rq[i].x, hi = rq[i].y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = (f16)(float)(int8_t)((lo >> (8 * e)) & 0xFF);
          v[4 + e] = (f16)(float)(int8_t)((hi >> (8 * e)) & 0xFF);
        }
      } else {
        v = bf16x8_to_f16x8(rw[i]);
      }
      *(f16x8*)&sW[c * 8] = v;
    }
    if (Q8 && tid < BN) {
      sD[tid * 2] = (float)rd0;
      sD[tid * 2 + 1] = (float)rd1;
    }
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      *(uint4*)&sXh[row * LD + col] = rxh[i];
      *(uint4*)&sXl[row * LD + col] = rxl[i];
    }
  };

  gload(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (k0 + BK < K) gload(k0 + BK);
    const int r16 = lane & 15;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int koff = kk * 32 + (lane >> 4) * 8;
      f16x8 a[TN], bh[TT], bl[TT];
#pragma unroll
      for (int i = 0; i < TN; ++i) a[i] = *(const f16x8*)&sW[((((wn >> 4) + i) * 2 + kk) * 64 + lane) * 8];
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        bh[j] = *(const f16x8*)&sXh[(wt + j * 16 + r16) * LD + koff];
        bl[j] = *(const f16x8*)&sXl[(wt + j * 16 + r16) * LD + koff];
      }
      if (Q8) {
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          float sc[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] = sD[(wn + i * 16 + (lane >> 4) * 4 + r) * 2 + kk];
#pragma unroll
          for (int j = 0; j < TT; ++j) {
            f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
            p = mfma16(a[i], bh[j], p);
            p = mfma16(a[i], bl[j], p);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc[r], p[r], acc[i][j][r]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TT; ++j) {
            acc[i][j] = mfma16(a[i], bh[j], acc[i][j]);
            acc[i][j] = mfma16(a[i], bl[j], acc[i][j]);
          }
      }
    }
  }

  // D[n][t]: lane holds rows n = base + 4*(lane>>4) + r of column t = base + (lane & 15).
  const int tl = lane & 15, nq4 = (lane >> 4) * 4;
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < TN; i += 2) {
      int pt = (n0 + wn + i * 16) / 16;          // even physical 16-row tile: gate
      int f = (pt / 2) * 16 + nq4;
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        int t = t0 + wt + j * 16 + tl;
        if (t < T) {
          f16x4 hv, lv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float g = acc[i][j][r], u = acc[i + 1][j][r];
            float m = g / (1.0f + expf(-g)) * u * m_scale;
            f16 h, lo;
            split_f16(m, h, lo);
            hv[r] = h;
            lv[r] = lo;
          }
          *(f16x4*)&Mhi[(int64_t)t * ldm + f] = hv;
          *(f16x4*)&Mlo[(int64_t)t * ldm + f] = lv;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      int n = n0 + wn + i * 16 + nq4;
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        int t = t0 + wt + j * 16 + tl;
        if (t < T) {
          float4* dst = (float4*)&C[(int64_t)t * ldc + n];
          float4 v = make_float4(acc[i][j][0] * out_scale, acc[i][j][1] * out_scale, acc[i][j][2] * out_scale,
                                 acc[i][j][3] * out_scale);
          if (EPI == EPI_ADD) {
            float4 o = *dst;
            v.x += o.x;
            v.y += o.y;
            v.z += o.z;
            v.w += o.w;
          }
          *dst = v;
        }
      }
    }
  }
}

template <int BN, int BT, bool Q8>
static hipError_t launch_gemm_t(int epi, const uint16_t* W, const int8_t* Wq, const f16* Wd, int K, int N,
                                const f16* Xhi, const f16* Xlo, int ldx, int T, float* C, int ldc, float out_scale,
                                f16* Mhi, f16* Mlo, int ldm, float m_scale, hipStream_t st) {
  dim3 grid(N / BN, (T + BT - 1) / BT);
  if (epi == EPI_STORE)
    hipLaunchKernelGGL((gemm_kernel<BN, BT, EPI_STORE, Q8>), grid, dim3(256), 0, st, W, Wq, Wd, K, N, Xhi, Xlo, ldx,
                       T, C, ldc, out_scale, Mhi, Mlo, ldm, m_scale);
  else if (epi == EPI_ADD)
    hipLaunchKernelGGL((gemm_kernel<BN, BT, EPI_ADD, Q8>), grid, dim3(256), 0, st, W, Wq, Wd, K, N, Xhi, Xlo, ldx, T,
                       C, ldc, out_scale, Mhi, Mlo, ldm, m_scale);
  else
    hipLaunchKernelGGL((gemm_kernel<BN, BT, EPI_SWIGLU, Q8>), grid, dim3(256), 0, st, W, Wq, Wd, K, N, Xhi, Xlo, ldx,
                       T, C, ldc, out_scale, Mhi, Mlo, ldm, m_scale);
  return hipGetLastError();
}

// Weight tile 256 rows x 128 tokens per workgroup.
constexpr int kGemmBN = 256, kGemmBT = 128;

hipError_t launch_gemm(int epi, const uint16_t* W, const int8_t* Wq, const f16* Wd, int K, int N, const f16* Xhi,
                       const f16* Xlo, int ldx, int T, float* C, int ldc, float out_scale, f16* Mhi, f16* Mlo,
                       int ldm, float m_scale, hipStream_t st) {
  if (N % kGemmBN != 0 || K % 64 != 0 || T <= 0) return hipErrorInvalidValue;
  if (Wq)
    return launch_gemm_t<kGemmBN, kGemmBT, true>(epi, W, Wq, Wd, K, N, Xhi, Xlo, ldx, T, C, ldc, out_scale, Mhi, Mlo,
                                                 ldm, m_scale, st);
  return launch_gemm_t<kGemmBN, kGemmBT, false>(epi, W, Wq, Wd, K, N, Xhi, Xlo, ldx, T, C, ldc, out_scale, Mhi, Mlo,
                                                ldm, m_scale, st);
}

}  // namespace gqa
