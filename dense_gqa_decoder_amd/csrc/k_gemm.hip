// Prefill projections: C[t][n] = sum_k W[n][k] * x[t][k] on the gfx950 matrix cores.
//
// W is the FP16 prefill copy of a BF16 matrix [N][K] (prefill_weight_index: per 32-row block and
// 32-wide K-step one contiguous 2 KiB piece in the MFMA operand order, copied to LDS unchanged),
// or Q8_0 (Kipp Model Support, "Quantization (Q8_0)": int8 quants, tile-major, with an fp16 scale
// per 32-weight block).
// x is the FP32 activation held as an FP16 hi/lo pair (split_f16). With SPLIT, two FP16 MFMAs
// (hi, then lo) per operand pair give a near-FP32 product; without it only hi enters (one MFMA,
// FP16-rounded activations). Accumulation is FP32 throughout; BF16 weights are exact FP16
// operands. For Q8_0 each 32-wide K-step is one quant block: the int8 quants are exact FP16
// operands, the MFMAs sum q*x over the block into a fresh accumulator and the block's scale is
// applied in FP32 afterwards.
//
// Tiling: a 256-thread workgroup computes a 256 (weight rows) x 128 (tokens) tile; each wave a
// 128 x 64 quadrant of 4 x 2 v_mfma_f32_32x32x16_f16 tiles (A = 32 weight rows, B = 32 tokens).
// K advances 32 per step through two LDS buffers filled by direct-to-LDS loads: the next step's
// copies are in flight during the current step's MFMAs, one barrier per step. Q8_0 quants are
// copied as bytes (half the traffic of FP16) and widened to FP16 when the A operand is read
// (exact: 0x6400 | (q + 128) is the FP16 value 1152 + q).
// Workgroups walk the output tiles in groups of 8 weight-row blocks x all token blocks, and the
// tiles are dealt to the eight XCDs in contiguous runs, so the workgroups resident on one XCD at
// a time share their weight and activation tiles in that XCD's L2.
// N % 256 == 0 and K % 32 == 0 are required; T (tokens) may be ragged.
//
// Epilogues: EPI_STORE C = acc * out_scale; EPI_ADD C += acc * out_scale (residual);
// EPI_SWIGLU: the weight rows interleave gate and up in 16-row bands (physical band 2j = gate
// features 16j.., band 2j+1 = up features 16j..), so the top and bottom halves of every 32-row
// MFMA tile are matching gate and up rows, and each lane writes m = silu(g) * u * m_scale for
// its own values as an FP16 hi/lo pair for the down projection.
#include "gqa_common.h"

namespace gqa {

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

struct GemmArgs {
  const f16* W;              // BF16 models: the FP16 prefill copy (prefill_weight_index layout)
  const int8_t* Wq;
  const f16* Wd;
  int K, N;
  const f16* Xhi;
  const f16* Xlo;
  int ldx, T;
  float* C;
  int ldc;
  float out_scale;
  f16* Mhi;
  f16* Mlo;
  int ldm;
  float m_scale;
  int ksplit;                // K ranges (EPI_STORE only): range s writes C + s * split_stride
  int64_t split_stride;
  int Nvalid;                // EPI_STORE: columns >= Nvalid are not stored (N padded to the tile)
};

constexpr int kGemmBN = 256, kGemmBT = 128, kGemmBK = 32;
constexpr int kGemmGroup = 8;        // weight-row blocks per tile group

// The Q8_0 instances decode quants and apply per-block scales in registers; bounding them to one workgroup per CU
// gives them the full register file (no spills), which measured 2.3-2.8x faster than two spilling workgroups.
template <int EPI, bool Q8, bool SPLIT>
__global__ __launch_bounds__(256, Q8 ? 1 : 2) void gemm_kernel(GemmArgs g) {
  constexpr int BN = kGemmBN, BT = kGemmBT, BK = kGemmBK;
  constexpr int TN = 4, TT = 2;                  // 32x32 tiles per wave
  // Per buffer: weights (FP16 in operand order, or Q8_0 int8 quants: 16 bands x 512 bytes, the
  // odd bands rotated by 128 bytes so that the two bands a half-wave reads hit different banks),
  // the Q8_0 scales of the step (256 fp16), and the activation hi / lo rows (token t's 16-byte
  // pieces swizzled by xswz).
  __shared__ __attribute__((aligned(16))) f16 sW[2][BN * BK];
  __shared__ __attribute__((aligned(16))) f16 sS[2][Q8 ? 512 : 8];
  __shared__ __attribute__((aligned(16))) f16 sXh[2][BT * BK];
  __shared__ __attribute__((aligned(16))) f16 sXl[SPLIT ? 2 : 1][SPLIT ? BT * BK : 8];
  auto bufW = [&](int b) -> f16* { return sW[b]; };
  auto bufXh = [&](int b) -> f16* { return sXh[b]; };
  auto bufXl = [&](int b) -> f16* { return sXl[SPLIT ? b : 0]; };

  // ---- tile and K range of this workgroup: XCD-contiguous runs of a grouped order of
  //      (K range, tile) items, tiles of one K range consecutive
  const int K = g.K, T = g.T;
  const int nnb = g.N / BN, ntb = (T + BT - 1) / BT, total = nnb * ntb, items = total * g.ksplit;
  const int per_xcd = (items + 7) / 8;
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= items || (blockIdx.x >> 3) >= per_xcd) return;
  const int kr = item / total, tile = item - kr * total;
  const int ns_all = K / BK;
  const int s_begin = kr * ns_all / g.ksplit, s_end = (kr + 1) * ns_all / g.ksplit;
  const int kbase = s_begin * BK;
  float* const Cout = g.C ? g.C + (int64_t)kr * g.split_stride : nullptr;
  const int grp = tile / (kGemmGroup * ntb), rem = tile - grp * kGemmGroup * ntb;
  const int gsz = min(kGemmGroup, nnb - grp * kGemmGroup);
  const int nb = grp * kGemmGroup + rem % gsz, tb = rem / gsz;
  const int n0 = nb * BN, t0 = tb * BT;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = (wave & 1) * 128, wt = (wave >> 1) * 64;
  const int l32 = lane & 31, hf = lane >> 5;

  const int64_t band0 = (int64_t)(n0 >> 4) * (K >> 5);   // Q8_0: first 16-row band's chunk index
  const int64_t blk0 = (int64_t)(n0 >> 5) * (K >> 5);    // FP16: first 32-row block's piece index

  f32x16 acc[TN][TT];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // MFMA operands of one 16-wide half (kh) of a K-step
  // LDS weight order per 32-row block and K-step: [kh][hf][row 0..31][8 halves], so the 32 lanes
  // of each half-wave read 512 contiguous bytes (no bank conflicts)
  auto a_op = [&](int buf, int i, int kh) {
    return *(const f16x8*)&bufW(buf)[((wn >> 5) + i) * 1024 + kh * 512 + hf * 256 + l32 * 8];
  };
  // DMA layout: piece kc of token t at slot 4 t + (kc ^ xswz(t)); the XOR spreads the 16 (or 32)
  // tokens a half-wave reads over all banks
  auto xswz = [](int t) { return ((t >> 2) ^ (t >> 3)) & 3; };
  auto b_op = [&](const f16* sx, int j, int kh) {
    const int t = wt + 32 * j + l32;
    return *(const f16x8*)&sx[(t * 4 + ((2 * kh + hf) ^ xswz(t))) * 8];
  };

  auto compute = [&](int cur) {
    const f16* sxh = bufXh(cur);
    const f16* sxl = SPLIT ? bufXl(cur) : nullptr;
    if (Q8) {
      f16x8 bh[TT][2], bl[TT][2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int j = 0; j < TT; ++j) {
          bh[j][kh] = b_op(sxh, j, kh);
          if (SPLIT) bl[j][kh] = b_op(sxl, j, kh);
        }
      const uint8_t* wq = (const uint8_t*)bufW(cur);
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        // rows wn + 32 i + l32: band 2 ((wn >> 5) + i) + l32 / 16, row l32 % 16 of it; the quants
        // of K-half kh for lane half hf are chunk position (16 (2 kh + hf) + row) * 8
        const int band = 2 * ((wn >> 5) + i) + (l32 >> 4), r = l32 & 15;
        f16x8 a[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int slot = ((8 * (2 * kh + hf) + (r >> 1)) + 8 * (band & 1)) & 31;
          a[kh] = i8x8_to_f16x8(*(const uint2*)(wq + band * 512 + slot * 16 + (r & 1) * 8));
        }
        // scales of the accumulator rows 32 i + 8 q + 4 hf + 0..3 of this wave's quadrant
        f16 sc[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x4 v = *(const f16x4*)&sS[cur][wn + 32 * i + 8 * q + 4 * hf];
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * q + e] = v[e];
        }
#pragma unroll
        for (int j = 0; j < TT; ++j) {
          f32x16 p = f32x16{};
          p = mfma32(a[0], bh[j][0], p);
          if (SPLIT) p = mfma32(a[0], bl[j][0], p);
          p = mfma32(a[1], bh[j][1], p);
          if (SPLIT) p = mfma32(a[1], bl[j][1], p);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = fmaf((float)sc[e], p[e], acc[i][j][e]);
        }
      }
    } else {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        f16x8 a[TN], bh[TT], bl[TT];
#pragma unroll
        for (int i = 0; i < TN; ++i) a[i] = a_op(cur, i, kh);
#pragma unroll
        for (int j = 0; j < TT; ++j) {
          bh[j] = b_op(sxh, j, kh);
          if (SPLIT) bl[j] = b_op(sxl, j, kh);
        }
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TT; ++j) {
            acc[i][j] = mfma32(a[i], bh[j], acc[i][j]);
            if (SPLIT) acc[i][j] = mfma32(a[i], bl[j], acc[i][j]);
          }
      }
    }
  };

  const int nsteps = s_end - s_begin;
  int cur = 0;
  // Pipeline: LDS buffer s % 2 holds step s; step s + 1 streams into the other buffer by
  // direct-to-LDS loads during step s's MFMAs. Per step each wave copies 2 KiB of activation
  // hi (and lo) rows, and 4 KiB of FP16 weights or 2 KiB of Q8_0 quants (wave 0 also the 512
  // bytes of scales); the LDS destination of a wave-wide load is contiguous in lane order.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dw[4], dx[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (Q8) {
      // quants: load 2 wv + i (i < 2) covers bands 2 (2 wv + i) + l / 32; LDS slot l % 32 holds
      // chunk slot (l % 32 - 8 (band & 1)) & 31
      const int b = 2 * (2 * wv + (i & 1)) + (lane >> 5), slot = ((lane & 31) - 8 * (b & 1)) & 31;
      dw[i] = (uint32_t)(b * (K >> 5)) * 512u + (uint32_t)slot * 16u;
    } else {
      const int c = (wv * 4 + i) * 64 + lane;    // piece c of the step, as in memory
      dw[i] = (uint32_t)((c >> 7) * (K >> 5)) * 1024u + (uint32_t)(c & 127) * 8u;
    }
  }
  // scales: lane l < 32 brings half l % 2 of band l / 2's 16 scales (lanes 32.. repeat them)
  const uint32_t ds = (uint32_t)(((lane & 31) >> 1) * (K >> 5)) * 16u + (uint32_t)(lane & 1) * 8u;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = (wv * 2 + i) * 64 + lane, t = slot >> 2, kc = (slot & 3) ^ xswz(t);
    dx[i] = (uint32_t)(min(t0 + t, T - 1) * g.ldx + kc * 8);      // rows past T: a valid row, never stored
  }
  // Direct-to-LDS copies: every barrier that publishes a filled buffer follows dma_wait().
  auto dma = [&](int buf, int k0) {
    if (Q8) {
      const int8_t* qsrc = g.Wq + (band0 + (k0 >> 5)) * 512;
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16(qsrc + dw[i], (const uint8_t*)bufW(buf) + (2 * wv + i) * 1024);
      if (wv == 0) lds_dma16(g.Wd + (band0 + (k0 >> 5)) * 16 + ds, sS[buf]);
    } else {
      const f16* wsrc = g.W + (blk0 + (k0 >> 5)) * 1024;
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma16(wsrc + dw[i], &bufW(buf)[(wv * 4 + i) * 512]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lds_dma16(g.Xhi + k0 + dx[i], &bufXh(buf)[(wv * 2 + i) * 512]);
      if (SPLIT) lds_dma16(g.Xlo + k0 + dx[i], &bufXl(buf)[(wv * 2 + i) * 512]);
    }
  };
  auto dma_wait = []() { vm_wait_all(); };
  dma(0, kbase);
  dma_wait();
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {            // buffer cur holds step s
    const bool more = s + 1 < nsteps;
    if (more) dma(cur ^ 1, kbase + (s + 1) * BK);
    compute(cur);
    if (more) {
      dma_wait();                               // this wave's loads of step s + 1 have landed
      __syncthreads();                          // ... and every other wave's
      cur ^= 1;
    }
  }

  // acc[i][j][e] = D[row wn + 32 i + 8 (e / 4) + 4 hf + e % 4][token wt + 32 j + l32]
#pragma unroll
  for (int j = 0; j < TT; ++j) {
    const int t = t0 + wt + 32 * j + l32;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int nbase = n0 + wn + 32 * i + 4 * hf;
      if (EPI == EPI_SWIGLU) {
        // rows 0..15 of the tile are gate, 16..31 the matching up rows
        const int f = ((n0 + wn + 32 * i) >> 5) * 16 + 4 * hf;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          f16x4 hv, lv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gg = acc[i][j][q * 4 + r], uu = acc[i][j][(q + 2) * 4 + r];
            const float m = gg / (1.0f + expf(-gg)) * uu * g.m_scale;
            f16 h, l;
            split_f16(m, h, l);
            hv[r] = h;
            lv[r] = l;
          }
          *(f16x4*)&g.Mhi[(int64_t)t * g.ldm + f + 8 * q] = hv;
          *(f16x4*)&g.Mlo[(int64_t)t * g.ldm + f + 8 * q] = lv;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (EPI == EPI_STORE && nbase + 8 * q >= g.Nvalid) continue;   // Nvalid % 4 == 0
          float4* dst = (float4*)&Cout[(int64_t)t * g.ldc + nbase + 8 * q];
          float4 v = make_float4(acc[i][j][q * 4 + 0] * g.out_scale, acc[i][j][q * 4 + 1] * g.out_scale,
                                 acc[i][j][q * 4 + 2] * g.out_scale, acc[i][j][q * 4 + 3] * g.out_scale);
          if (EPI == EPI_ADD) {
            const float4 o = *dst;
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

template <bool Q8, bool SPLIT>
static hipError_t launch_gemm_t(int epi, const GemmArgs& a, hipStream_t st) {
  const int items = (a.N / kGemmBN) * ((a.T + kGemmBT - 1) / kGemmBT) * a.ksplit;
  dim3 grid(8 * ((items + 7) / 8));
  if (epi == EPI_STORE)
    GQA_LAUNCH((gemm_kernel<EPI_STORE, Q8, SPLIT>), grid, dim3(256), 0, st, a);
  else if (epi == EPI_ADD)
    GQA_LAUNCH((gemm_kernel<EPI_ADD, Q8, SPLIT>), grid, dim3(256), 0, st, a);
  else
    GQA_LAUNCH((gemm_kernel<EPI_SWIGLU, Q8, SPLIT>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// split: FP16 hi/lo activations (two MFMAs per operand pair); otherwise hi only.
// ksplit > 1 (EPI_STORE only): the K steps are cut into ksplit consecutive ranges and range s
// stores its partial product at C + s * split_stride; the consumer sums them in range order.
// nvalid (EPI_STORE): only columns below it are stored (0: all N); a multiple of 4.
hipError_t launch_gemm(int epi, bool split, const f16* W, const int8_t* Wq, const f16* Wd, int K, int N,
                       const f16* Xhi, const f16* Xlo, int ldx, int T, float* C, int ldc, float out_scale, f16* Mhi,
                       f16* Mlo, int ldm, float m_scale, int ksplit, int64_t split_stride, hipStream_t st, int nvalid) {
  if (N % kGemmBN != 0 || K % kGemmBK != 0 || T <= 0) return hipErrorInvalidValue;
  if (ksplit < 1 || ksplit > K / kGemmBK || (ksplit > 1 && epi != EPI_STORE)) return hipErrorInvalidValue;
  if (nvalid == 0) nvalid = N;
  if (nvalid % 4 != 0 || nvalid > N || (nvalid != N && epi != EPI_STORE)) return hipErrorInvalidValue;
  GemmArgs a{W, Wq, Wd, K, N, Xhi, Xlo, ldx, T, C, ldc, out_scale, Mhi, Mlo, ldm, m_scale, ksplit, split_stride,
             nvalid};
  if (Wq) return split ? launch_gemm_t<true, true>(epi, a, st) : launch_gemm_t<true, false>(epi, a, st);
  return split ? launch_gemm_t<false, true>(epi, a, st) : launch_gemm_t<false, false>(epi, a, st);
}

}  // namespace gqa
