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
// K advances 32 per step through two LDS buffers: the next step's global loads are in flight
// during the current step's MFMAs and are written to the other buffer, one barrier per step.
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
};

constexpr int kGemmBN = 256, kGemmBT = 128, kGemmBK = 32;
constexpr int kGemmGroup = 8;        // weight-row blocks per tile group

template <int EPI, bool Q8, bool SPLIT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  constexpr int BN = kGemmBN, BT = kGemmBT, BK = kGemmBK;
  // BF16 models (FP16 prefill copy): global -> LDS by direct-to-LDS loads (no registers, no
  // conversion), activation rows swizzled instead of padded. Q8_0 models: through registers
  // (int8 -> FP16), activation rows padded to 80 bytes. Both give conflict-free operand reads.
  constexpr bool DMA = !Q8;
  constexpr int XLD = DMA ? BK : BK + 8;         // halves per token row in LDS
  constexpr int TN = 4, TT = 2;                  // 32x32 tiles per wave
  __shared__ __attribute__((aligned(16))) f16 sW[2][BN * BK];
  __shared__ __attribute__((aligned(16))) f16 sXh[2][BT * XLD];
  __shared__ __attribute__((aligned(16))) f16 sXl[SPLIT ? 2 : 1][SPLIT ? BT * XLD : 8];
  auto bufW = [&](int b) -> f16* { return sW[b]; };
  auto bufXh = [&](int b) -> f16* { return sXh[b]; };
  auto bufXl = [&](int b) -> f16* { return sXl[SPLIT ? b : 0]; };
  __shared__ float sD[2][Q8 ? BN : 1];

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

  // ---- global -> register staging of one K-step
  constexpr int PW = BN * BK / 8 / 256;          // 16-byte weight pieces per thread (4)
  constexpr int PX = BT * BK / 8 / 256;          // 16-byte activation pieces per thread and half (2)
  struct Stage {
    uint4 w[PW];
    uint2 q[Q8 ? PW : 1];
    uint4 xh[PX], xl[SPLIT ? PX : 1];
    f16 d;
  };
  // 32-bit per-thread offsets from workgroup-uniform bases (one scalar base + one VGPR per load)
  // BF16 models read the FP16 prefill copy: piece c = 32-row block c / 128, position c % 128 of
  // its 2 KiB K-step (already in LDS order). Q8_0 models read the tile-major quants: piece c =
  // 16-row band c / 64, lane-order position c % 64.
  const int64_t band0 = (int64_t)(n0 >> 4) * (K >> 5);
  const int64_t blk0 = (int64_t)(n0 >> 5) * (K >> 5);
  uint32_t woff[PW], xoff[PX];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int c = tid + 256 * i;
    woff[i] = Q8 ? (uint32_t)((c >> 6) * (K >> 5)) * 512u + (uint32_t)(c & 63) * 8u
                 : (uint32_t)((c >> 7) * (K >> 5)) * 1024u + (uint32_t)(c & 127) * 8u;
  }
#pragma unroll
  for (int i = 0; i < PX; ++i) {
    const int c = tid + 256 * i, tok = c >> 2, kc = c & 3;
    xoff[i] = (uint32_t)(min(t0 + tok, T - 1) * g.ldx + kc * 8);   // rows past T: a valid row, never stored
  }
  const uint32_t doff = (uint32_t)((tid >> 4) * (K >> 5)) * 16u + (uint32_t)(tid & 15);
  auto gload = [&](Stage& r, int k0) {
    k0 = min(k0, K - BK);                        // past the end: reload the last step (never used)
    const int64_t kw = band0 + (k0 >> 5), kb = blk0 + (k0 >> 5);
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      if (Q8)
        r.q[i] = *(const uint2*)(g.Wq + kw * 512 + woff[i]);
      else
        r.w[i] = *(const uint4*)(g.W + kb * 1024 + woff[i]);
    }
    if (Q8) r.d = g.Wd[kw * 16 + doff];
#pragma unroll
    for (int i = 0; i < PX; ++i) {
      r.xh[i] = *(const uint4*)(g.Xhi + k0 + xoff[i]);
      if (SPLIT) r.xl[i] = *(const uint4*)(g.Xlo + k0 + xoff[i]);
    }
  };
  auto sstore = [&](const Stage& r, int buf) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int c = tid + 256 * i;
      if (Q8) {
        f16x8 v;
        const uint32_t lo = r.q[i].x, hi = r.q[i].y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = (f16)(float)(int8_t)((lo >> (8 * e)) & 0xFF);      // exact small integers
          v[4 + e] = (f16)(float)(int8_t)((hi >> (8 * e)) & 0xFF);
        }
        // band c / 64, position g * 16 + r -> LDS order [block][kh][hf][row 32][8]
        const int band = c >> 6, gq = (c >> 4) & 3, rr = c & 15;
        *(f16x8*)&bufW(buf)[(band >> 1) * 1024 + (gq >> 1) * 512 + (gq & 1) * 256 + ((band & 1) * 16 + rr) * 8] = v;
      } else {
        *(uint4*)&bufW(buf)[c * 8] = r.w[i];
      }
    }
    if (Q8) sD[buf][tid] = (float)r.d;
#pragma unroll
    for (int i = 0; i < PX; ++i) {
      const int c = tid + 256 * i, tok = c >> 2, kc = c & 3;
      *(uint4*)&bufXh(buf)[tok * XLD + kc * 8] = r.xh[i];
      if (SPLIT) *(uint4*)&bufXl(buf)[tok * XLD + kc * 8] = r.xl[i];
    }
  };

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
    if (DMA) return *(const f16x8*)&sx[(t * 4 + ((2 * kh + hf) ^ xswz(t))) * 8];
    return *(const f16x8*)&sx[t * XLD + kh * 16 + hf * 8];
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
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const f16x8 a0 = a_op(cur, i, 0), a1 = a_op(cur, i, 1);
        float sc[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *(const float4*)&sD[cur][wn + 32 * i + q * 8 + hf * 4];
          sc[4 * q] = v.x;
          sc[4 * q + 1] = v.y;
          sc[4 * q + 2] = v.z;
          sc[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < TT; ++j) {
          f32x16 p;
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] = 0.f;
          p = mfma32(a0, bh[j][0], p);
          if (SPLIT) p = mfma32(a0, bl[j][0], p);
          p = mfma32(a1, bh[j][1], p);
          if (SPLIT) p = mfma32(a1, bl[j][1], p);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = fmaf(sc[e], p[e], acc[i][j][e]);
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
  if constexpr (DMA) {
    // Pipeline: LDS buffer s % 2 holds step s; step s + 1 streams into the other buffer by
    // direct-to-LDS loads during step s's MFMAs. Each wave issues 4 + 2 (+ 2) kilobyte loads per
    // step; the LDS destination of a wave-wide load is contiguous in lane order.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint32_t dw[4], dx[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (wv * 4 + i) * 64 + lane;    // piece c of the step, as in memory
      dw[i] = (uint32_t)((c >> 7) * (K >> 5)) * 1024u + (uint32_t)(c & 127) * 8u;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = (wv * 2 + i) * 64 + lane, t = slot >> 2, kc = (slot & 3) ^ xswz(t);
      dx[i] = (uint32_t)(min(t0 + t, T - 1) * g.ldx + kc * 8);      // rows past T: a valid row, never stored
    }
    // Direct-to-LDS copies: every barrier that publishes a filled buffer follows dma_wait().
    auto dma1 = [](const f16* src, const f16* lds_dst) { lds_dma16(src, lds_dst); };
    auto dma = [&](int buf, int k0) {
      const f16* wsrc = g.W + (blk0 + (k0 >> 5)) * 1024;
#pragma unroll
      for (int i = 0; i < 4; ++i) dma1(wsrc + dw[i], &bufW(buf)[(wv * 4 + i) * 512]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dma1(g.Xhi + k0 + dx[i], &bufXh(buf)[(wv * 2 + i) * 512]);
        if (SPLIT) dma1(g.Xlo + k0 + dx[i], &bufXl(buf)[(wv * 2 + i) * 512]);
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
  } else {
    // Pipeline: LDS buffer s % 2 holds step s; the registers hold step s + 1, whose global loads
    // are in flight during step s's MFMAs.
    Stage r;
    gload(r, kbase);
    sstore(r, 0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      const bool more = s + 1 < nsteps;
      if (more) gload(r, kbase + (s + 1) * BK);
      compute(cur);
      if (more) {
        sstore(r, cur ^ 1);
        __syncthreads();
        cur ^= 1;
      }
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
hipError_t launch_gemm(int epi, bool split, const f16* W, const int8_t* Wq, const f16* Wd, int K, int N,
                       const f16* Xhi, const f16* Xlo, int ldx, int T, float* C, int ldc, float out_scale, f16* Mhi,
                       f16* Mlo, int ldm, float m_scale, int ksplit, int64_t split_stride, hipStream_t st) {
  if (N % kGemmBN != 0 || K % kGemmBK != 0 || T <= 0) return hipErrorInvalidValue;
  if (ksplit < 1 || ksplit > K / kGemmBK || (ksplit > 1 && epi != EPI_STORE)) return hipErrorInvalidValue;
  GemmArgs a{W, Wq, Wd, K, N, Xhi, Xlo, ldx, T, C, ldc, out_scale, Mhi, Mlo, ldm, m_scale, ksplit, split_stride};
  if (Wq) return split ? launch_gemm_t<true, true>(epi, a, st) : launch_gemm_t<true, false>(epi, a, st);
  return split ? launch_gemm_t<false, true>(epi, a, st) : launch_gemm_t<false, false>(epi, a, st);
}

}  // namespace gqa
