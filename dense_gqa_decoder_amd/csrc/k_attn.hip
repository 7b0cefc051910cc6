// GQA attention over the paged KV cache (BF16, or Q8_0 codes read as bf16(scale * code)).
//
// Kipp Roadmap, status v0.0.3/v0.0.4: flash-attention prefill for GQA (kipp_flash_gqa_prefill);
// status v0.0.2: K/V live in 32-position blocks addressed through a per-session block table.
// For query head h the KV head is h / g (g = n_q_heads / 8); key j is visible to the query at
// position p iff j <= p; scores are q.k / sqrt(128) and the output is the softmax-weighted sum of
// V. Softmax runs in base 2 on scores pre-multiplied by log2(e) / sqrt(128).
//
// Prefill (attn_prefill_kernel): 512-thread workgroups, one per (KV head, pair of 32-query
// tiles). The pair is tile i and tile n-1-i of the n tiles of the round, so every workgroup
// walks the same number of causal key tiles (the round costs n + 1 key sweeps per pair whatever
// i is), and workgroup b serves KV head b % 8, so all workgroups of one KV head run on one XCD
// and share its L2. The eight waves are g heads x 8/g key splits: wave (h, s) owns the 32
// queries of head h and, of every staged tile of 32 * 8/g keys, the 32-key subtile s, with its
// own online-softmax state; the split states are merged in LDS at the end of the query tile.
//  - K and V tiles go from the pool to LDS by direct-to-LDS loads (no register staging), double
//    buffered; the block ids of the keys are staged in LDS once per workgroup. With a Q8_0 cache
//    each copy's codes and block scale pass through registers and are widened into the same
//    LDS slots. K runs one tile
//    ahead of V, so each iteration issues the score MFMAs of the next subtile in the same
//    straight-line block as the softmax and P V products of the current one.
//  - S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K is the exact BF16 A operand (one 16-byte LDS
//    read per lane and step), Q^T the B operand held in registers as a BF16 hi/lo pair
//    (hi = RNE(x), lo = RNE of the exact remainder: about 2^-17 relative).
//  - The accumulator gives each lane one query and 16 keys, which is already the B-operand
//    layout of O^T = V^T P^T once the keys of each 16-key step are taken in the order
//    (4 hf + 0..3, 8 + 4 hf + 0..3) for lane half hf; P enters as a BF16 hi/lo pair too.
//  - V^T, the A operand, comes straight from the row-major V tile through the transposing LDS
//    read ds_read_b64_tr_b16: lane i of each 16-lane group addresses key row i / 4, 8-byte piece
//    i % 4 of a 4-key x 16-dim block and receives the 4 keys of dim i.
//  - The running max is kept lazily: the accumulator and sum are rescaled only when a new score
//    exceeds the reference max by more than 2^8, so p = 2^(s - m) stays below 256.
//
// Decode: split-context attention on the matrix cores into chunk partials, then a chunk merge in
// chunk order; see attn_decode_kernel.
#include "gqa_common.h"

#include <algorithm>

namespace gqa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32_bf16(bf16v8 a, bf16v8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// BF16 hi/lo of two FP32 values, packed two per dword: hi = RNE(x), lo = RNE(x - hi) (the
// remainder is exact in FP32), so hi + lo = x to about 2^-17 relative.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(a, b);
  lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ __forceinline__ bf16v8 as_bf16v8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16v8, uint4{a, b, c, d});
}

// max and sum of a lane's value with the value of lane l ^ 32 (same result in both lanes)
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

constexpr int kDecodeMaxChunks = 64;
constexpr int kPartStride = 132;   // floats per chunk partial: m, l, pad, pad, o[128]

// LDS of the prefill kernel. A staged tile holds KT keys. K tile: 8 planes, one per 16-dim step
// st, each KT rows x 32 bytes, the two 16-byte halves of row r swapped when bit 3 of r is set
// (16 consecutive rows read at one half then cover all 64 banks). V tile: 4 planes, one per
// 32-dim tile dt, each KT rows x 64 bytes (4 consecutive rows are 256 contiguous bytes, the
// footprint of a transposing read by 32 lanes). Both layouts put every step, dim tile and key
// offset of a lane's reads into the instruction's immediate offset.
template <int G>
struct PrefillLds {
  static constexpr int NS = 8 / G;                       // key splits
  static constexpr int KT = 32 * NS;                     // keys per staged tile
  static constexpr int TILE = KT * kHeadDim;             // BF16 elements of one K (or V) tile
  static constexpr int KPLANE = KT * 16, VPLANE = KT * 32;
  static constexpr int KV_BYTES = 4 * TILE * 2;          // two buffers of K, two of V
  static constexpr int MERGE_BYTES = G * (NS - 1) * 66 * 64 * 4;   // per lane: m, l, o[64]
  static constexpr int MAX_BLOCKS = 4096;                // block-table entries staged in LDS
  static constexpr int AREA = KV_BYTES > MERGE_BYTES ? KV_BYTES : MERGE_BYTES;   // K/V buffers, or the merge
  static constexpr int BYTES = AREA + MAX_BLOCKS * 4;
};

// part == nullptr: o of each query row written as FP16 hi/lo. Otherwise (one query tile, T <= 32)
// the keys are split over gridDim.y workgroups: split c takes its share of the key tiles and
// writes, per query row t and head h, the partial (m, l, o[128]) of its keys at
// part[((t * nq + h) * kDecodeMaxChunks + c) * kPartStride] (the decode chunk-partial layout; m in
// log2 units, o relative to m), merged afterwards by attn_merge_rows_kernel.
// KQ8: the cache is Q8_0 (kq8); a copy's 8 codes and their block scale go through registers and
// are widened to the values attention reads, bf16(fp32(scale) * code), into the same LDS slots
// the BF16 cache's direct copies fill. They are loaded where the copies are issued and written
// before the barrier that publishes the tile.
template <int G, bool PSPLIT, bool KQ8>
__global__ __launch_bounds__(512) void attn_prefill_kernel(const float* __restrict__ q, int nq, int T, int pos0,
                                                           const int32_t* __restrict__ table,
                                                           const uint16_t* kpool, const uint16_t* vpool,
                                                           float out_scale, f16* __restrict__ ohi,
                                                           f16* __restrict__ olo, int ldo, float* __restrict__ part,
                                                           KvQ8 kq8) {
  using L = PrefillLds<G>;
  constexpr int NS = L::NS, KT = L::KT, TILE = L::TILE, KPLANE = L::KPLANE, VPLANE = L::VPLANE;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[L::BYTES / 2];
  int* const tbl = (int*)(lds + L::AREA / 2);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = wave % G, ks = wave / G;
  const int kvh = blockIdx.x & 7, pair = blockIdx.x >> 3;
  const int head = kvh * G + hh;
  const int nt = (T + 31) >> 5;
  const int hf = lane >> 5, c32 = lane & 31;
  const float qscale = kLog2e * 0.08838834764831845f;
  const int64_t blk_elems = (int64_t)kKvHeads * kBlock * kHeadDim;

  // Staging: wave w copies the 1 KiB segments w + 8 i (i < NS) of each tile. A K segment is 32
  // rows (one pool block) of plane (w + 8 i) / NS, rows 32 (w % NS) ..; lane l brings row l / 2,
  // half l % 2. A V segment is 16 rows of plane (w + 8 i) / (2 NS), rows 16 (w % 2NS) ..; lane l
  // brings row l / 4, chunk l % 4. Each wave's segments of a tile lie in one pool block.
  const int krg = wave % NS, vrg = wave % (2 * NS);
  const int kchunk = (((lane & 1) ^ ((lane >> 4) & 1)) << 3);
  // K operand: row 32 ks + c32 of the tile, dims 16 st + 8 hf ..
  const int kl = (ks * 32 + c32) * 16 + ((hf ^ ((c32 >> 3) & 1)) << 3);
  // V^T operand: 16-lane group g reads dims 16 (g % 2) .. of a 4-key block at rows 4 hf + ..
  const int vi = lane & 15;
  const int vl = (ks * 32 + 4 * hf + (vi >> 2)) * 32 + ((lane >> 4) & 1) * 16 + (vi & 3) * 4;

  // the block ids of every key the workgroup reads (the first query tile is the longer one)
  {
    const int nblk = (pos0 + min(32 * (nt - pair), T) + 31) >> 5;
    for (int i = tid; i < nblk; i += 512) tbl[i] = table[i];
  }
  __syncthreads();

  for (int which = 0; which < 2; ++which) {
    const int qt = which == 0 ? nt - 1 - pair : pair;
    if (which == 1 && qt == nt - 1 - pair) break;
    const int t0 = qt * 32;
    const int qfirst = pos0 + t0, qlast = pos0 + min(t0 + 32, T) - 1;
    const int kend = qlast + 1;
    const int ntile_all = (kend + KT - 1) / KT;
    // this workgroup's key tiles [tb, ntile): all of them, or split c's share
    const int per_split = (ntile_all + gridDim.y - 1) / gridDim.y;
    const int tb = part ? min((int)blockIdx.y * per_split, ntile_all) : 0;
    const int ntile = part ? min(tb + per_split, ntile_all) : ntile_all;
    const int myq = pos0 + min(t0 + c32, T - 1);

    // Pipeline over staged tiles: iteration t needs K(t + 1) (for S(t + 1)) and V(t) (for
    // P(t) V(t)), so the K stream runs one tile ahead of the V stream; tile u of a stream sits
    // in buffer u & 1. Iteration t issues the copies of K(t + 2) and V(t + 1) into the buffers
    // that iteration t - 1 finished with; they land while it computes.
    // Q8_0: one tile of each stream in registers between issue and land
    uint2 kc[NS], vc[NS];
    uint16_t ksc[NS], vsc[NS];
    auto issue_k = [&](int u) {
      const int ph = tbl[min(u * KT + krg * 32, kend - 1) >> 5];
      const int key = min(u * KT + krg * 32 + (lane >> 1), kend - 1);   // rows past the last query: a valid row
      const int64_t e0 = (int64_t)ph * blk_elems + ((int64_t)kvh * kBlock + (key & 31)) * kHeadDim + kchunk;
      uint16_t* dst = lds + (u & 1) * TILE;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int sg = wave + 8 * i;
        const int64_t e = e0 + 16 * (sg / NS);
        if constexpr (KQ8) {
          kc[i] = *(const uint2*)(kq8.kq + e);
          ksc[i] = __builtin_bit_cast(uint16_t, kq8.ks[e >> 5]);
        } else {
          lds_dma16(kpool + e, dst + sg * 512);
        }
      }
    };
    auto issue_v = [&](int u) {
      const int ph = tbl[min(u * KT + vrg * 16, kend - 1) >> 5];
      const int key = min(u * KT + vrg * 16 + (lane >> 2), kend - 1);
      const int64_t e0 = (int64_t)ph * blk_elems + ((int64_t)kvh * kBlock + (key & 31)) * kHeadDim + (lane & 3) * 8;
      uint16_t* dst = lds + (2 + (u & 1)) * TILE;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int sg = wave + 8 * i;
        const int64_t e = e0 + 32 * (sg / (2 * NS));
        if constexpr (KQ8) {
          vc[i] = *(const uint2*)(kq8.vq + e);
          vsc[i] = __builtin_bit_cast(uint16_t, kq8.vs[e >> 5]);
        } else {
          lds_dma16(vpool + e, dst + sg * 512);
        }
      }
    };
    auto land_k = [&](int u) {
      uint16_t* dst = lds + (u & 1) * TILE;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        *(uint4*)(dst + (wave + 8 * i) * 512 + 8 * lane) = q8kv_bf16x8(kc[i], __builtin_bit_cast(f16, ksc[i]));
    };
    auto land_v = [&](int u) {
      uint16_t* dst = lds + (2 + (u & 1)) * TILE;
#pragma unroll
      for (int i = 0; i < NS; ++i)
        *(uint4*)(dst + (wave + 8 * i) * 512 + 8 * lane) = q8kv_bf16x8(vc[i], __builtin_bit_cast(f16, vsc[i]));
    };
    // first copies, then the Q loads (their latencies overlap); Q8_0: K(tb) lands before K(tb + 1)
    // reuses the registers
    if (tb < ntile) {
      issue_k(tb);
      issue_v(tb);
      if constexpr (KQ8) {
        land_k(tb);
        land_v(tb);
      }
      if (tb + 1 < ntile) {
        issue_k(tb + 1);
        if constexpr (KQ8) land_k(tb + 1);
      }
    }

    // Q^T operand: lane holds query c32, dims 16 st + 8 hf .. +7, pre-scaled, as BF16 hi/lo
    bf16v8 qh[8], ql[8];
    {
      const float* qr = q + ((int64_t)min(t0 + c32, T - 1) * nq + head) * kHeadDim + 8 * hf;
      float4 qa[8], qb[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        qa[st] = *(const float4*)(qr + 16 * st);
        qb[st] = *(const float4*)(qr + 16 * st + 4);
      }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const float4 a = qa[st], b = qb[st];
        uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
        split_bf16x2(a.x * qscale, a.y * qscale, h0, l0);
        split_bf16x2(a.z * qscale, a.w * qscale, h1, l1);
        split_bf16x2(b.x * qscale, b.y * qscale, h2, l2);
        split_bf16x2(b.z * qscale, b.w * qscale, h3, l3);
        qh[st] = as_bf16v8(h0, h1, h2, h3);
        ql[st] = as_bf16v8(l0, l1, l2, l3);
      }
    }

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float m = -1e30f, lsum = 0.f;

    // S^T of subtile ks of K tile u: sc[e] = score of key u KT + 32 ks + 8 (e / 4) + 4 hf + e % 4
    auto scores = [&](int u) {
      const uint16_t* kp = lds + (u & 1) * TILE + kl;
      f32x16 sc = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16v8 a = *(const bf16v8*)(kp + st * KPLANE);
        sc = mfma32_bf16(a, qh[st], sc);
        sc = mfma32_bf16(a, ql[st], sc);
      }
      return sc;
    };

    vm_wait_all();                     // K(tb) (and everything else issued so far)
    __syncthreads();
    f32x16 sc = scores(tb);
    for (int t = tb; t < ntile; ++t) {
      if constexpr (KQ8) {             // the tiles loaded during iteration t - 1
        if (t > tb) {
          if (t + 1 < ntile) land_k(t + 1);
          land_v(t);
        }
      }
      vm_wait_all();                   // this wave's copies of K(t + 1) and V(t)
      __syncthreads();                 // ... and every wave's; the buffers of K(t), V(t - 1) are free
      if (t + 2 < ntile) issue_k(t + 2);
      if (t + 1 < ntile) issue_v(t + 1);

      const int sub = t * KT + ks * 32;
      if (sub > qlast) continue;       // every key of this and later subtiles is masked
      if (sub + 31 > qfirst) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = sub + 8 * (e >> 2) + 4 * hf + (e & 3);
          sc[e] = key <= myq ? sc[e] : -INFINITY;
        }
      }
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
      const float mnew = fmaxf(m, xhalf_max(mx));
      if (__any(mnew > m + 8.f)) {
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      }
      // S(t + 1) (on the last tile it reads a stale buffer and is discarded), P(t), O += V(t)^T P(t)^T
      const f32x16 sn = scores(t + 1);
      uint32_t ph[8], pl[8];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sc[e] - m), p1 = __builtin_amdgcn_exp2f(sc[e + 1] - m);
        ps += p0;
        ps += p1;
        if (PSPLIT)
          split_bf16x2(p0, p1, ph[e >> 1], pl[e >> 1]);
        else
          ph[e >> 1] = pk_bf16(p0, p1);
      }
      lsum += ps;
      const uint16_t* vt = lds + (2 + (t & 1)) * TILE + vl;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16v8 bh = as_bf16v8(ph[4 * j], ph[4 * j + 1], ph[4 * j + 2], ph[4 * j + 3]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const s16x4 v0 = lds_read_tr16(vt + dt * VPLANE + 16 * j * 32);
          const s16x4 v1 = lds_read_tr16(vt + dt * VPLANE + (16 * j + 8) * 32);
          const bf16v8 a = __builtin_bit_cast(bf16v8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt] = mfma32_bf16(a, bh, o[dt]);
          if (PSPLIT) {
            const bf16v8 bl = as_bf16v8(pl[4 * j], pl[4 * j + 1], pl[4 * j + 2], pl[4 * j + 3]);
            o[dt] = mfma32_bf16(a, bl, o[dt]);
          }
        }
      }
      sc = sn;
    }
    lsum = xhalf_sum(lsum);

    auto store = [&](float Lsum) {
      const int t = t0 + c32;
      if (t >= T) return;
      const float inv = out_scale / Lsum;
      const int64_t base = (int64_t)t * ldo + head * kHeadDim + 4 * hf;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f16x4 hv, lv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            f16 h, l;
            split_f16(o[dt][4 * g4 + r] * inv, h, l);
            hv[r] = h;
            lv[r] = l;
          }
          *(f16x4*)&ohi[base + dt * 32 + 8 * g4] = hv;
          *(f16x4*)&olo[base + dt * 32 + 8 * g4] = lv;
        }
    };

    if constexpr (NS == 1) {
      store(lsum);
      __syncthreads();                 // the next query tile's first copies reuse buffer 0
    } else {
      float* sm = (float*)lds;
      __syncthreads();                 // every wave is done with the K/V buffers
      if (ks > 0) {
        float* d = sm + (hh * (NS - 1) + ks - 1) * 66 * 64 + lane;
        d[0] = m;
        d[64] = lsum;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) d[(2 + dt * 16 + e) * 64] = o[dt][e];
      }
      __syncthreads();
      if (ks == 0) {
        const float* src = sm + hh * (NS - 1) * 66 * 64 + lane;
        float M = m;
#pragma unroll
        for (int k = 0; k < NS - 1; ++k) M = fmaxf(M, src[k * 66 * 64]);
        const float w0 = __builtin_amdgcn_exp2f(m - M);
        float Ls = lsum * w0;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= w0;
#pragma unroll
        for (int k = 0; k < NS - 1; ++k) {
          const float* sk = src + k * 66 * 64;
          const float w = __builtin_amdgcn_exp2f(sk[0] - M);
          Ls = fmaf(sk[64], w, Ls);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] = fmaf(sk[(2 + dt * 16 + e) * 64], w, o[dt][e]);
        }
        if (part) {
          const int t = t0 + c32;
          if (t < T) {
            float* pp = part + (((int64_t)t * nq + head) * kDecodeMaxChunks + blockIdx.y) * kPartStride;
            if (hf == 0) {
              pp[0] = M;
              pp[1] = Ls;
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4)
                *(float4*)(pp + 4 + dt * 32 + 8 * g4 + 4 * hf) =
                    make_float4(o[dt][4 * g4], o[dt][4 * g4 + 1], o[dt][4 * g4 + 2], o[dt][4 * g4 + 3]);
          }
        } else {
          store(Ls);
        }
      }
      __syncthreads();                 // the merge area is the next query tile's K/V buffer
    }
  }
}

// Decode attention (split context), grid (chunk group, KV head, row), kDecodeWaves (four) waves
// per workgroup. A row's context [0, pos] is cut into chunks of decode_chunk_len(ctx) positions
// (a multiple of the 64-position step chosen from the row's own context length only, so a row
// gets the same chunks whether it is evaluated alone or in a batch). A workgroup walks its chunk
// one step at a time, wave w taking 16 consecutive keys on the matrix cores (section 3 below);
// each wave keeps its own online-softmax state (max, sum, value sum) for the g query heads of the
// KV head, and the wave states are merged in LDS, in wave order, into one chunk partial (max,
// sum, o[128]) per head. A Q8_0 cache is read as codes and block scales, widened to
// bf16(scale * code) as a step is computed.
//  1. q for the g query heads: the fixed-order sum of the q|k|v projection's split partials,
//     times the row's 1/rms (recomputed from the sum-of-squares partials the projection's
//     prologue wrote), per-head RMSNorm, rotate-half RoPE at the row's position, built once
//     per workgroup in LDS with every global load of the step issued together.
//  2. The workgroup whose chunk holds the new position also builds its k (norm + RoPE) and v,
//     rounds them to BF16, writes them through the block table and uses the rounded values
//     for that position.
//  3. The last workgroup of a (row, KV head) to finish combines the chunk partials of its heads in
//     chunk order (merge_head).
#ifndef GQA_DECODE_WAVES
#define GQA_DECODE_WAVES 4
#endif
constexpr int kDecodeWaves = GQA_DECODE_WAVES;
constexpr int kDecodeStep = 16 * kDecodeWaves;          // positions per step: 16 keys per wave
#ifndef GQA_BATCH_CHUNKS_PER_WG
#define GQA_BATCH_CHUNKS_PER_WG 3
#endif
constexpr int kBatchChunksPerWorkgroup = GQA_BATCH_CHUNKS_PER_WG;

#ifndef GQA_DECODE_TARGET_CHUNKS
#define GQA_DECODE_TARGET_CHUNKS 32
#endif
// Chunk length of a row's context: the smallest multiple of a step (kDecodeStep positions) that
// cuts it into at most GQA_DECODE_TARGET_CHUNKS chunks (<= kDecodeMaxChunks). A function of the
// row's own context only, so a row's partials and merge do not depend on the batch.
__host__ __device__ __forceinline__ int decode_chunk_len(int ctx) {
  static_assert(GQA_DECODE_TARGET_CHUNKS >= 1 && GQA_DECODE_TARGET_CHUNKS <= kDecodeMaxChunks, "chunk count");
  return kDecodeStep * ((ctx + kDecodeStep * GQA_DECODE_TARGET_CHUNKS - 1) / (kDecodeStep * GQA_DECODE_TARGET_CHUNKS));
}

// Device-scope (sc1) accesses: coherent across the XCDs' L2 caches without an L2 writeback or
// invalidate. The fused chunk merge passes its partials through these, so the only ordering it
// needs is that the stores have completed before the workgroup is counted in.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_dev2(const float* p) {
  const uint64_t v = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(float2, v);
}

// Combine the chunk partials of one (row, query head) in chunk order: o = sum_c w_c o_c / sum_c
// w_c l_c with w_c = 2^(m_c - max m). One wave; lane t owns dims 2t, 2t + 1. The result is
// written as the FP16 hi/lo operand of the o projection, times out_scale. DEV: the partials
// were written by other workgroups of the same launch (device-scope loads).
template <bool DEV, int NC, bool STDEV = false>
__device__ __forceinline__ void merge_head_n(const float* pp, int nchunk, int lane, float out_scale, f16* ohi,
                                             f16* olo) {
  auto ld2 = [](const float* p) { return DEV ? load_dev2(p) : *(const float2*)p; };
  const float2 ml = ld2(pp + (int64_t)min(lane, nchunk - 1) * kPartStride);
  float2 ov[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc)
    ov[cc] = ld2(pp + (int64_t)min(cc, nchunk - 1) * kPartStride + 4 + 2 * lane);
  const float mv = lane < nchunk ? ml.x : -INFINITY;
  const float M = wave_max(mv);
  const float wt = lane < nchunk ? exp2f(mv - M) : 0.f;
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  // Every chunk slot enters the chains: past nchunk the weight is exactly 0 and the (clamped)
  // values are finite, so those steps add +0 to sums that started at +0 and cannot be -0, which
  // leaves them unchanged. No branch per chunk, so the compiler cannot sink each load next to
  // its use (which serialised the loads).
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {                      // chunk cc's weight and sum, read as scalars
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), cc));
    L = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml.y), cc)), w, L);
    o0 = fmaf(ov[cc].x, w, o0);
    o1 = fmaf(ov[cc].y, w, o1);
  }
  const float inv = out_scale / L;
  f16 h0, l0, h1, l1;
  split_f16(o0 * inv, h0, l0);
  split_f16(o1 * inv, h1, l1);
  if constexpr (STDEV) {                                  // read by the next launch of a chain
    __hip_atomic_store((uint32_t*)(ohi + 2 * lane), __builtin_bit_cast(uint32_t, f16x2{h0, h1}), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store((uint32_t*)(olo + 2 * lane), __builtin_bit_cast(uint32_t, f16x2{l0, l1}), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *(f16x2*)(ohi + 2 * lane) = f16x2{h0, h1};
    *(f16x2*)(olo + 2 * lane) = f16x2{l0, l1};
  }
}

// merge_head_n over the slots a context can use: NC = 32 when it has at most 32 chunks (half the
// partial loads), else all 64. The slots past nchunk enter with weight 0 and add exact zeros, so
// both give the same bits.
template <bool DEV, bool STDEV = false>
__device__ __forceinline__ void merge_head(const float* pp, int nchunk, int lane, float out_scale, f16* ohi,
                                           f16* olo) {
  if (nchunk <= 32)
    merge_head_n<DEV, 32, STDEV>(pp, nchunk, lane, out_scale, ohi, olo);
  else
    merge_head_n<DEV, kDecodeMaxChunks, STDEV>(pp, nchunk, lane, out_scale, ohi, olo);
}

// K/V of one wave's 16 keys of a 64-position step, in flight: BF16 K rows in registers (the V
// planes travel by direct-to-LDS copies), or with a Q8_0 cache the K and V codes and their block
// scales in registers, widened to the same BF16 values when the step is computed.
struct DecStage {
  uint4 kr[4];      // K rows: the MFMA A operand (BF16), one uint4 per 32-dim step
  uint2 kc[4];      // Q8_0: K codes of the same elements
  uint2 ksc;        // Q8_0: the key's four block scales
  uint4 vc[2];      // Q8_0: V codes of one key, 32 dims
  uint16_t vsc;     // Q8_0: their block scale
};

// Dispatch order of a batch's rows: grid slice z serves row b[z]. Workgroups are dispatched in
// index order, so the launcher puts the rows with the longest workgroups first and the short ones
// fill the tail. Which row a workgroup serves does not change what it computes.
struct RowOrder {
  uint8_t b[kMaxBatch];
};
static_assert(kMaxBatch <= 256, "row indices fit a byte");

// Shared memory of one decode-attention workgroup.
template <int G, int NBUF>
struct AttnSmem {
  float sraw[(G + 2) * kHeadDim];                         // projection sums (times 1/rms)
  float sq[(G + 2) * kHeadDim];                           // normed + rotated q (scaled), k; v
  float wm[kDecodeWaves][G], wl[kDecodeWaves][G];
  float wo[kDecodeWaves][G][kHeadDim];
  __attribute__((aligned(16))) uint16_t vlds[kDecodeWaves][NBUF][16 * kHeadDim];   // V planes, NBUF steps
  int stab[64 * kDecodeWaves];                            // block-table entries of the workgroup's chunks
  int s_last;
};

// The arguments of a decode-attention launch.
struct AttnArgs {
  const float* qkvp;
  int nsplit;
  int64_t pstride;
  int QKV, nq;
  const float* ss;
  int ss_n, H;
  const uint16_t *wqn, *wkn;
  float eps;
  const float *rcos, *rsin;
  Rows rows;
  RowOrder order;
  int cpw;
  uint16_t *kpool, *vpool;
  KvQ8 kq8;
  float* part;
  int* counters;
  float out_scale;
  f16 *ohi, *olo;
  int ldo;
  Chain chain;                                            // a launch of a decode chain (or none)
};

// One workgroup of the decode attention: chunk group bx, KV head kvh, grid row slot zs.
// CHAIN: a launch of a decode chain (gqa_common.h): issues its first K/V, waits for its
// predecessors, reads the projection device-scope and writes the merged rows device-scope.
// Steps in flight of a decode-attention workgroup: K/V of NBUF steps (registers and V planes)
// are held at once, so while a step is computed the next NBUF - 1 are loading. Three for the
// single workgroup per CU of a few-row decode (one wave per SIMD: latency is all there is to
// hide), two for the row-batched launch (three workgroups per CU).
#ifndef GQA_DECODE_BUFFERS_FUSED
#define GQA_DECODE_BUFFERS_FUSED 3
#endif
constexpr int decode_buffers(bool fused) { return fused ? GQA_DECODE_BUFFERS_FUSED : 2; }

// LTAB: every workgroup's block-table entries fit the LDS table (one per thread), which the
// launcher checks; the steps then read their block ids from LDS only. (A step reading "LDS or
// global" through one pointer becomes a generic load, which waits for every vector load in
// flight.)
template <int G, bool FUSED, bool KQ8, bool CHAIN, bool LTAB>
__device__ __forceinline__ void attn_decode_body(AttnSmem<G, decode_buffers(FUSED)>& sm, int bx, int kvh, int zs,
                                                 const AttnArgs& A) {
  constexpr int NBUF = decode_buffers(FUSED);
  static_assert(NBUF == 2 || NBUF == 3, "two or three steps in flight");
  constexpr int NW = kDecodeWaves;                        // softmax states per workgroup (one per wave)
  constexpr int NE = (G + 2) * kHeadDim;                  // q heads, then k and v of the new position
  const float* __restrict__ qkvp = A.qkvp;
  int nsplit = A.nsplit;
  const int64_t pstride = A.pstride;
  const int QKV = A.QKV, nq = A.nq, ss_n = A.ss_n, H = A.H, cpw = A.cpw, ldo = A.ldo;
  const float* __restrict__ ss = A.ss;
  const uint16_t* __restrict__ wqn = A.wqn;
  const uint16_t* __restrict__ wkn = A.wkn;
  const float eps = A.eps, out_scale = A.out_scale;
  const float* __restrict__ rcos = A.rcos;
  const float* __restrict__ rsin = A.rsin;
  const Rows& rows = A.rows;
  uint16_t* __restrict__ kpool = A.kpool;
  uint16_t* __restrict__ vpool = A.vpool;
  const KvQ8& kq8 = A.kq8;
  float* part = A.part;
  int* __restrict__ counters = A.counters;
  f16* __restrict__ ohi = A.ohi;
  f16* __restrict__ olo = A.olo;
  float (&sraw)[NE] = sm.sraw;
  float (&sq)[NE] = sm.sq;
  float (&wm)[NW][G] = sm.wm;
  float (&wl)[NW][G] = sm.wl;
  float (&wo)[NW][G][kHeadDim] = sm.wo;
  uint16_t (&vlds)[NW][NBUF][16 * kHeadDim] = sm.vlds;
  int& s_last = sm.s_last;
  const int b = A.order.b[zs];
  const int pos = rows.pos[b], ctx = pos + 1;
  const int CH = decode_chunk_len(ctx);
  const int nchunk = (ctx + CH - 1) / CH;
  const int c0 = bx * cpw;                                // this workgroup's chunks [c0, c1)
  if (c0 >= nchunk) return;
  const int c1 = min(c0 + cpw, nchunk);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int hq = lane & 15, g4 = lane >> 4;
  const bool owner = c1 == nchunk;                        // the last chunk holds the new position
  auto p_end_of = [&](int cc) { return min(cc * CH + CH, ctx); };
  auto niter_of = [&](int cc) { return (p_end_of(cc) - cc * CH + kDecodeStep - 1) / kDecodeStep; };
  const int32_t* table = rows.table[b];
  constexpr int64_t kBlockElems = (int64_t)kKvHeads * kBlock * kHeadDim;

  // Keys of 64-position step `it` for this wave: p0 .. p0 + 15 with p0 = chunk start + 64 it + 16 w,
  // all in one 32-position block. The loads are unconditional: a key past the chunk reads a slot
  // of a block the session owns (or the pool's block 0 when the whole wave is past it); its score
  // is masked and its V row zeroed in LDS before use.
  //   K: lane l loads key l % 16, dims 32 s + 8 (l / 16) .. + 7 for s = 0..3 (the A operand rows).
  //   V: four 1 KiB direct-to-LDS copies into 16-dim planes (16 keys x 32 bytes each); copy j
  //      fills planes 2 j, 2 j + 1, lane l bringing key (l % 32) / 2, half l % 2 of the plane.
  // The block-table entries of the workgroup's positions are staged in LDS (LTAB; one per thread,
  // loaded with the first K/V and stored before the barrier that publishes q), so a step's K/V
  // loads do not wait for a table load; the first step reads the table directly.
  const int blk0 = (c0 * CH) >> 5, nblk = ((min(c1 * CH, ctx) - 1) >> 5) - blk0 + 1;
  const int tabv = LTAB && tid < nblk ? table[blk0 + tid] : 0;
  auto blk_of = [&](int cc, int it) { return min(cc * CH + it * kDecodeStep + wave * 16, p_end_of(cc) - 1) >> 5; };
  auto phys_first = [&](int cc, int it) { return table[blk_of(cc, it)]; };
  auto phys_of = [&](int cc, int it) {
    if constexpr (LTAB)
      return sm.stab[blk_of(cc, it) - blk0];
    else
      return table[blk_of(cc, it)];
  };
  //   Q8_0 cache: K as above but the codes (8 bytes per lane and 32-dim step) and the key's four
  //   block scales; V: lane l brings the 32 codes of key l / 4, dims 32 (l % 4) .. + 31, and their
  //   scale, widened into the same LDS planes when the step is computed.
  auto issue = [&](int phys, DecStage& sg, int buf) {
    const int64_t rows = (int64_t)phys * kBlockElems + ((int64_t)kvh * kBlock + ((wave * 16) & 31)) * kHeadDim;
    if constexpr (KQ8) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) sg.kc[s4] = *(const uint2*)(kq8.kq + rows + hq * kHeadDim + 32 * s4 + 8 * g4);
      sg.ksc = *(const uint2*)(kq8.ks + ((rows + hq * kHeadDim) >> 5));
      const int64_t vo = rows + (lane >> 2) * kHeadDim + 32 * (lane & 3);
      sg.vc[0] = *(const uint4*)(kq8.vq + vo);
      sg.vc[1] = *(const uint4*)(kq8.vq + vo + 16);
      sg.vsc = __builtin_bit_cast(uint16_t, kq8.vs[vo >> 5]);
    } else {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) sg.kr[s4] = *(const uint4*)(kpool + rows + hq * kHeadDim + 32 * s4 + 8 * g4);
      const int vrow = (lane & 31) >> 1, vhalf = lane & 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int plane = 2 * j + (lane >> 5);
        lds_dma16(vpool + rows + vrow * kHeadDim + 16 * plane + 8 * vhalf, &vlds[wave][buf][j * 512]);
      }
    }
  };
  DecStage kA, kB, kC;                                   // kC: third buffer (NBUF == 3)
  // Issue order matters (vector loads complete in order): the block-table entry, the RoPE and
  // norm constants, the projection partials, then the first K/V, so q is built while the K/V
  // are in flight.
  const int phys0 = phys_first(c0, 0);
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
    if constexpr (CHAIN) {                               // one projection range (nsplit == 1)
      issue(phys0, kA, 0);
      chain_wait(A.chain);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {                       // every load first
      const int e = i * 64 * kDecodeWaves + tid;
      const int hrow = e < G * kHeadDim ? kvh * G + e / kHeadDim
                                        : (e < (G + 1) * kHeadDim ? nq + kvh : nq + kKvHeads + kvh);
      const float* p = qrow + (e < nel ? hrow * kHeadDim + (e % kHeadDim) : 0);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        if constexpr (CHAIN)
          t[i][s2] = s2 == 0 ? ld_dev(p) : 0.f;
        else
          t[i][s2] = p[(int64_t)min(s2, nsplit - 1) * pstride];   // unconditional
      }
    }
    if constexpr (!CHAIN) issue(phys0, kA, 0);
    const float cin = CHAIN ? inv_rms_from_ss_dev(ss, ss_n, b, H, eps) : inv_rms_from_ss(ss, ss_n, b, H, eps);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = i * 64 * kDecodeWaves + tid;
      float acc = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) acc += s2 < nsplit ? t[i][s2] : 0.f;   // select, not a branch
      if (e < nel) sraw[e] = __fmul_rn(acc, cin);
    }
  }
  if (LTAB && tid < nblk) sm.stab[tid] = tabv;
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
      } else if (!kq8.kq) {                               // k: BF16 storage rounding
        r0 = bf16_bits_to_f32(f32_to_bf16_rne(r0));
        r1 = bf16_bits_to_f32(f32_to_bf16_rne(r1));
      }
      sq[hh * kHeadDim + lane] = r0;
      sq[hh * kHeadDim + 64 + lane] = r1;
    }
    if (owner && tid < kHeadDim) {
      const float vr = sraw[(G + 1) * kHeadDim + tid];
      sq[(G + 1) * kHeadDim + tid] = kq8.kq ? vr : bf16_bits_to_f32(f32_to_bf16_rne(vr));
    }
  }
  __syncthreads();
  // the new position's K/V into the pool, through the block table. Q8_0 cache: thread t < 256
  // quantises element t % 128 of the K (t < 128) or V row; each 32-dim block is one half-wave, whose
  // maximum comes from lane exchanges. Codes and scales go to the pool, and the row in LDS is
  // replaced by the values attention reads back, bf16(scale * code).
  if (kq8.kq) {
    static_assert(64 * kDecodeWaves >= 2 * kHeadDim, "one thread per K and V element");
    if (owner) {
      if (tid < 2 * kHeadDim) {
        const int kv = tid / kHeadDim, e = tid % kHeadDim;
        float* src = sq + (G + kv) * kHeadDim;
        const float x = src[e];
        float amax = fabsf(x);
#pragma unroll
        for (int msk = 16; msk >= 1; msk >>= 1) amax = fmaxf(amax, __shfl_xor(amax, msk));
        const float d = q8kv_scale(amax);
        const f16 sc = (f16)d;
        const int c = q8kv_code(x, d);
        const int64_t off =
            (int64_t)table[pos >> 5] * kBlockElems + ((int64_t)kvh * kBlock + (pos & 31)) * kHeadDim;
        (kv ? kq8.vq : kq8.kq)[off + e] = (int8_t)c;
        if ((e & 31) == 0) (kv ? kq8.vs : kq8.ks)[(off >> 5) + (e >> 5)] = sc;
        src[e] = bf16_bits_to_f32(q8kv_read_bf16(sc, c));
      }
      __syncthreads();
    }
  } else if (owner && tid < 2 * kHeadDim / 8) {
    const int kv = tid >> 4, d0 = (tid & 15) * 8;       // tid < 16: K, else V
    const float* src = sq + (G + kv) * kHeadDim + d0;
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = f32_to_bf16_rne(src[e]);
    const int64_t off = (int64_t)table[pos >> 5] * kBlockElems + ((int64_t)kvh * kBlock + (pos & 31)) * kHeadDim + d0;
    const uint4 row8 = uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    if constexpr (CHAIN)                                  // no dirty L2 lines from a chained launch
      st_dev16((kv ? vpool : kpool) + off, row8);
    else
      *(uint4*)((kv ? vpool : kpool) + off) = row8;
  }
  // 3. attention over the chunk on the matrix cores; wave w takes keys 16 w .. 16 w + 15 of every
  //    64-position step and keeps its own online-softmax state per head.
  //    Scores S^T[key][head] = K q^T by v_mfma_f32_16x16x32_bf16: A = the 16 keys' K rows, B = q as
  //    BF16 hi/lo (lane l: head l % 16, zero for heads >= g), four 32-dim steps x hi/lo. The score
  //    accumulator (lane l: keys 4 (l / 16) + i, head l % 16) is, as BF16 hi/lo, the A operand of
  //    v_mfma_f32_16x16x16_bf16 for O[head][dim] += P[head][key] V[key][dim]; V is read from its
  //    LDS planes transposed (ds_read_b64_tr_b16: lane i of a 16-lane group addresses key i / 4,
  //    piece i % 4, and receives dim i of the group's four keys).
  bf16v8 qh[4], ql[4];
  {
    const int hc = min(hq, G - 1);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      uint32_t h[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * s4 + 8 * g4 + 2 * j;
        const float a0 = hq < G ? sq[hc * kHeadDim + d] : 0.f, a1 = hq < G ? sq[hc * kHeadDim + d + 1] : 0.f;
        split_bf16x2(a0, a1, h[j], lo[j]);
      }
      qh[s4] = as_bf16v8(h[0], h[1], h[2], h[3]);
      ql[s4] = as_bf16v8(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  f32x4 O[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;                   // head hq: the wave's running max and sum
  auto xrow_max = [](float v) {                            // max over lanes l, l ^ 16
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto xrow_sum = [](float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
  auto compute = [&](int cc, int it, DecStage& sg, int buf) {
    const int p0 = cc * CH + it * kDecodeStep + wave * 16, p_end = p_end_of(cc);
    uint16_t* vl = vlds[wave][buf];
    uint4 (&kr)[4] = sg.kr;
    if constexpr (KQ8) {                                  // widen the step's codes (before the new row's overrides)
      const f16 ksc[4] = {__builtin_bit_cast(f16, (uint16_t)(sg.ksc.x & 0xFFFFu)),
                          __builtin_bit_cast(f16, (uint16_t)(sg.ksc.x >> 16)),
                          __builtin_bit_cast(f16, (uint16_t)(sg.ksc.y & 0xFFFFu)),
                          __builtin_bit_cast(f16, (uint16_t)(sg.ksc.y >> 16))};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) kr[s4] = q8kv_bf16x8(sg.kc[s4], ksc[s4]);
      const f16 vsc = __builtin_bit_cast(f16, sg.vsc);
      const int kk = lane >> 2, qd = lane & 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {                       // dims 32 qd + 16 h .. + 15: plane 2 qd + h
        uint16_t* dst = vl + (2 * qd + h) * 256 + kk * 16;
        *(uint4*)dst = q8kv_bf16x8(uint2{sg.vc[h].x, sg.vc[h].y}, vsc);
        *(uint4*)(dst + 8) = q8kv_bf16x8(uint2{sg.vc[h].z, sg.vc[h].w}, vsc);
      }
    }
    if (owner && p0 + hq == pos) {                        // the new position: K from LDS, not the pool
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float* kq = sq + G * kHeadDim + 32 * s4 + 8 * g4;
        uint32_t w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w4[j] = f32_to_bf16_rne(kq[2 * j]) | (f32_to_bf16_rne(kq[2 * j + 1]) << 16);
        kr[s4] = uint4{w4[0], w4[1], w4[2], w4[3]};
      }
    }
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const bf16v8 ka = as_bf16v8(kr[s4].x, kr[s4].y, kr[s4].z, kr[s4].w);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[s4], st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[s4], st, 0, 0, 0);
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = p0 + 4 * g4 + i < p_end ? st[i] : -INFINITY;
    const float mx = xhalf_max(xrow_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]))));
    const float mnew = fmaxf(m_run, mx);
    const bool any = mnew != -INFINITY;                   // a visible key so far for this head
    const float alpha = any ? exp2f(m_run - mnew) : 1.f;
    float pv[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = any ? exp2f(sc[i] - mnew) : 0.f;
      ps += pv[i];
    }
    ps = xhalf_sum(xrow_sum(ps));
    l_run = l_run * alpha + ps;
    m_run = mnew;
    // O rows 0 .. g - 1 (lanes 0..15) are the heads; head r's alpha sits in lane r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r < G ? r : 0));
#pragma unroll
      for (int n = 0; n < 8; ++n) O[n][r] *= ar;
    }
    uint32_t ph0, pl0, ph1, pl1;
    split_bf16x2(pv[0], pv[1], ph0, pl0);
    split_bf16x2(pv[2], pv[3], ph1, pl1);
    const s16x4 pah = __builtin_bit_cast(s16x4, uint2{ph0, ph1}), pal = __builtin_bit_cast(s16x4, uint2{pl0, pl1});
    // V rows of keys past the chunk to zero (masked keys must add 0 * finite), the new position's
    // row from LDS; lane l covers key l % 16, planes 2 (l / 16), 2 (l / 16) + 1
    {
      const int key = hq, pl2 = 2 * g4;
      if (p0 + key >= p_end) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          *(uint4*)(vl + (pl2 + q2) * 256 + key * 16) = uint4{0, 0, 0, 0};
          *(uint4*)(vl + (pl2 + q2) * 256 + key * 16 + 8) = uint4{0, 0, 0, 0};
        }
      } else if (owner && p0 + key == pos) {
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const float* vq = sq + (G + 1) * kHeadDim + 16 * (pl2 + q2);
          uint32_t w8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) w8[j] = f32_to_bf16_rne(vq[2 * j]) | (f32_to_bf16_rne(vq[2 * j + 1]) << 16);
          *(uint4*)(vl + (pl2 + q2) * 256 + key * 16) = uint4{w8[0], w8[1], w8[2], w8[3]};
          *(uint4*)(vl + (pl2 + q2) * 256 + key * 16 + 8) = uint4{w8[4], w8[5], w8[6], w8[7]};
        }
      }
    }
    const uint16_t* vt = vl + (4 * g4 + (hq >> 2)) * 16 + (hq & 3) * 4;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const s16x4 vb = lds_read_tr16(vt + n * 256);
      O[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pah, vb, O[n], 0, 0, 0);
      O[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pal, vb, O[n], 0, 0, 0);
    }
  };
  // 4. per chunk: merge the wave states of the workgroup (in wave order) into the chunk partial,
  //    then start the next chunk from empty states
  auto finish = [&](int cc) {
    if (lane < G) {
      wm[wave][lane] = m_run;
      wl[wave][lane] = l_run;
    }
    if (lane < 16) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < G; ++r) wo[wave][r][16 * n + lane] = O[n][r];
    }
    __syncthreads();
    // per (head, dim): the max over the wave states, the state weights 2^(m_w - max), the
    // weighted sums, in wave order; each thread forms its head's max and weights itself, so one
    // barrier publishes the wave states and no second pass is needed
    for (int idx = tid; idx < G * kHeadDim; idx += 64 * kDecodeWaves) {
      const int hh = idx / kHeadDim, d = idx % kHeadDim;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w][hh]);
      float wt[NW], L = 0.f, Ov = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        wt[w] = wm[w][hh] == -INFINITY ? 0.f : exp2f(wm[w][hh] - M);
        L = fmaf(wl[w][hh], wt[w], L);
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) Ov = fmaf(wo[w][hh][d], wt[w], Ov);
      float* pp = part + (((int64_t)b * nq + kvh * G + hh) * kDecodeMaxChunks + cc) * kPartStride;
      if (FUSED) {                          // read by another workgroup of this launch
        if (d == 0) {
          store_dev(pp, M);
          store_dev(pp + 1, L);
        }
        store_dev(pp + 4 + d, Ov);
      } else {                              // read by attn_merge_kernel after this launch
        if (d == 0) {
          pp[0] = M;
          pp[1] = L;
        }
        pp[4 + d] = Ov;
      }
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) O[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
    if (cc + 1 < c1) __syncthreads();     // the wave-state arrays are reused by the next chunk
  };

  // The workgroup's steps (chunk, 64-position step) in order through a ring of NBUF buffers (K in
  // registers, V planes in LDS per wave) across chunk boundaries, so the next chunk's first
  // copies are in flight during a chunk's merge. Before a step is computed the step NBUF - 1
  // ahead is issued into the buffer the previous step used; the step's own copies and loads
  // have landed once at most the eight of each later issued step are in flight. (lc, lit): next
  // step to issue; (cc, cit): next step to compute; `ahead`: issued steps not yet computed.
  int lc = c0, lit = 0, cc = c0, cit = 0;
  auto advance = [&](int& ch, int& it) {
    if (++it >= niter_of(ch)) {
      it = 0;
      ++ch;
    }
  };
  advance(lc, lit);                                      // step (c0, 0) was issued into kA, buffer 0
  int ahead = 1;
  if constexpr (NBUF == 3) {
    if (lc < c1) {                                       // step 2 of the ring, into kB
      issue(phys_of(lc, lit), kB, 1);
      advance(lc, lit);
      ahead = 2;
    }
  }
  auto run = [&](DecStage& sg, int buf) {
    compute(cc, cit, sg, buf);
    if (cit + 1 == niter_of(cc)) finish(cc);
    advance(cc, cit);
  };
  // compute the step in (cur, cb) after issuing the next one into (fre, fb)
  auto one = [&](DecStage& cur, int cb, DecStage& fre, int fb) {
    if (lc < c1) {
      issue(phys_of(lc, lit), fre, fb);
      advance(lc, lit);
      ++ahead;
    }
    if (ahead >= 3)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (ahead == 2)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      vm_wait_all();
    run(cur, cb);
    --ahead;
  };
  if constexpr (NBUF == 3) {
    while (true) {
      one(kA, 0, kC, 2);
      if (ahead == 0) break;
      one(kB, 1, kA, 0);
      if (ahead == 0) break;
      one(kC, 2, kB, 1);
      if (ahead == 0) break;
    }
  } else {
    while (true) {
      one(kA, 0, kB, 1);
      if (ahead == 0) break;
      one(kB, 1, kA, 0);
      if (ahead == 0) break;
    }
  }
  if (!FUSED) return;                     // attn_merge_kernel combines the partials
  // 5. the last workgroup of this (row, KV head) to finish merges the chunk partials. The
  //    partials went out as device-scope stores and are read back with device-scope loads, so
  //    no cache writeback or invalidate is needed: every wave waits until its stores have
  //    completed, then one thread counts the workgroup in; the last workgroup merges and resets
  //    the count for the next call.
  __builtin_amdgcn_s_waitcnt(0);          // vmcnt = lgkmcnt = 0: this wave's stores are done
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&counters[b * kKvHeads + kvh], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == nchunk - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (wave < G) {
    const int h = kvh * G + wave;
    merge_head<true, CHAIN>(part + ((int64_t)b * nq + h) * kDecodeMaxChunks * kPartStride, nchunk, lane, out_scale,
                     ohi + (int64_t)b * ldo + h * kHeadDim, olo + (int64_t)b * ldo + h * kHeadDim);
  }
  // in a chain the count goes back to zero with a device-scope store, which the arrivals of a
  // later any-order launch cannot overtake through a cache writeback
  if (tid == 0) {
    if constexpr (CHAIN)
      __hip_atomic_store(&counters[b * kKvHeads + kvh], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      counters[b * kKvHeads + kvh] = 0;
  }
}

template <int G, bool FUSED, bool KQ8, bool CHAIN, bool LTAB>
__global__ __launch_bounds__(64 * kDecodeWaves, FUSED ? 1 : (KQ8 ? 2 : 3)) void attn_decode_kernel(AttnArgs A) {
  __shared__ AttnSmem<G, decode_buffers(FUSED)> sm;
  attn_decode_body<G, FUSED, KQ8, CHAIN, LTAB>(sm, blockIdx.x, blockIdx.y, blockIdx.z, A);
  if constexpr (CHAIN) chain_signal(A.chain);
}

// Chunk merge as a kernel of its own, for large batches: grid (KV head, row), one wave per query
// head of the group. The kernel boundary orders it after every chunk partial, so no workgroup
// of the attention kernel needs a device-scope fence (with thousands of workgroups those
// fences, each writing back an XCD's L2, serialise). Same arithmetic as the fused merge.
template <int G>
__global__ __launch_bounds__(64 * G) void attn_merge_kernel(const float* __restrict__ part, int nq, Rows rows,
                                                           float out_scale, f16* __restrict__ ohi,
                                                           f16* __restrict__ olo, int ldo) {
  const int kvh = blockIdx.x, b = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ctx = rows.pos[b] + 1, CH = decode_chunk_len(ctx), nchunk = (ctx + CH - 1) / CH;
  const int h = kvh * G + wave;
  merge_head<false>(part + ((int64_t)b * nq + h) * kDecodeMaxChunks * kPartStride, nchunk, lane, out_scale,
                    ohi + (int64_t)b * ldo + h * kHeadDim, olo + (int64_t)b * ldo + h * kHeadDim);
}

// Merge of a split prefill attention: grid (KV head, query row), one wave per query head of the
// group; the same arithmetic as the decode chunk merge.
template <int G>
__global__ __launch_bounds__(64 * G) void attn_merge_rows_kernel(const float* __restrict__ part, int nq, int nchunk,
                                                                float out_scale, f16* __restrict__ ohi,
                                                                f16* __restrict__ olo, int ldo) {
  const int kvh = blockIdx.x, t = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = kvh * G + wave;
  merge_head<false>(part + ((int64_t)t * nq + h) * kDecodeMaxChunks * kPartStride, nchunk, lane, out_scale,
                    ohi + (int64_t)t * ldo + h * kHeadDim, olo + (int64_t)t * ldo + h * kHeadDim);
}

// part (optional): chunk-partial scratch for up to 32 rows (attn_decode_part_floats). With it, a
// round of at most 32 rows over a long context splits the keys over several workgroups per KV
// head (a single query tile would otherwise run on eight workgroups) and merges them after.
hipError_t launch_attn_prefill(const float* q, int nq, int T, int pos0, const int32_t* table, const uint16_t* kpool,
                               const uint16_t* vpool, const KvQ8& kq8, float out_scale, f16* ohi, f16* olo, int ldo,
                               float* part, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if ((pos0 + T + 31) / 32 > PrefillLds<4>::MAX_BLOCKS) return hipErrorInvalidValue;   // context too long
  const int G = nq / kKvHeads;
  if (G != 4 && G != 2) return hipErrorInvalidValue;
  const int pairs = ((T + 31) / 32 + 1) / 2;
  // key splits: about four 64-key tiles each, at most kDecodeMaxChunks
  const int kt = G == 4 ? PrefillLds<4>::KT : PrefillLds<2>::KT;
  const int ntile = (pos0 + T + kt - 1) / kt;
  const int csplit = (part && T <= 32) ? std::min(kDecodeMaxChunks, std::max(1, (ntile * kt + 255) / 256)) : 1;
  float* const pp = csplit > 1 ? part : nullptr;
  const dim3 grid(pairs * kKvHeads, csplit);
  if (!kq8.kq && (!kpool || !vpool)) return hipErrorInvalidValue;
#define PF_LAUNCH(GG, Q) \
  GQA_LAUNCH((attn_prefill_kernel<GG, true, Q>), grid, dim3(512), 0, st, q, nq, T, pos0, table, kpool, vpool, out_scale, \
             ohi, olo, ldo, pp, kq8)
  if (G == 4) {
    if (kq8.kq) PF_LAUNCH(4, true);
    else PF_LAUNCH(4, false);
  } else {
    if (kq8.kq) PF_LAUNCH(2, true);
    else PF_LAUNCH(2, false);
  }
#undef PF_LAUNCH
  if (pp) {
    if (G == 4)
      hipLaunchKernelGGL(attn_merge_rows_kernel<4>, dim3(kKvHeads, T), dim3(256), 0, st, pp, nq, csplit, out_scale, ohi,
                         olo, ldo);
    else
      hipLaunchKernelGGL(attn_merge_rows_kernel<2>, dim3(kKvHeads, T), dim3(128), 0, st, pp, nq, csplit, out_scale, ohi,
                         olo, ldo);
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const float* qkvp, int nsplit, int64_t pstride, int QKV, int nq, const float* ss,
                              int ss_n, int H, const uint16_t* wqn, const uint16_t* wkn, float eps, const float* rcos,
                              const float* rsin, const Rows& rows, int B, int max_ctx, uint16_t* kpool,
                              uint16_t* vpool, const KvQ8& kq8, float* part, int* counters, float out_scale, f16* ohi,
                              f16* olo, int ldo, hipStream_t st, const Chain& chain, int* nwg) {
  if (nsplit < 1 || nsplit > 8 || B < 1 || B > kMaxBatch || max_ctx < 1) return hipErrorInvalidValue;
  const bool ch = chain.cnt != nullptr;                   // chained: fused path, one projection range
  if (ch && (B > 4 || nsplit != 1 || (chain.wait && !chain.err))) return hipErrorInvalidValue;
  // the grid covers the largest chunk count of any row: the count is not monotonic in the
  // context (the chunk length grows in steps), so a shorter row can need more chunks than the
  // longest one; workgroups past a row's own count exit early
  int chunks = 1;
  for (int b = 0; b < B; ++b) {
    const int ctx = rows.pos[b] + 1, ch = decode_chunk_len(ctx);
    if (ctx > max_ctx) return hipErrorInvalidValue;
    chunks = std::max(chunks, (ctx + ch - 1) / ch);
  }
  const int G = nq / kKvHeads;
  // up to four rows: the last workgroup of a (row, KV head) merges; more rows: a merge kernel
  const bool fused = B <= 4;
  // chunks per workgroup: one for few rows (parallelism; the fused merge counts one workgroup per
  // chunk), several for many rows (q is built once per workgroup and the K/V stream runs on
  // across its chunks); the chunks and their partials are the same either way
  const int cpw = fused ? 1 : kBatchChunksPerWorkgroup;
  dim3 grid((chunks + cpw - 1) / cpw, kKvHeads, B);
  // the LDS block table holds one entry per thread: a workgroup spans at most cpw chunks of
  // 32-position blocks (chunk starts are block aligned)
  bool ltab = true;
  for (int b = 0; b < B; ++b)
    if (cpw * decode_chunk_len(rows.pos[b] + 1) / kBlock > 64 * kDecodeWaves) ltab = false;
  // rows by decreasing workgroup length (positions one workgroup walks), then by decreasing
  // context, then by index
  RowOrder order;
  int wl[kMaxBatch];
  for (int b = 0; b < B; ++b) {
    const int ctx = rows.pos[b] + 1, ch = decode_chunk_len(ctx);
    wl[b] = std::min(ctx, cpw * ch);
    order.b[b] = (uint8_t)b;
  }
  std::stable_sort(order.b, order.b + B, [&](uint8_t x, uint8_t y) {
    return wl[x] != wl[y] ? wl[x] > wl[y] : rows.pos[x] > rows.pos[y];
  });
  const AttnArgs A{qkvp, nsplit, pstride, QKV, nq, ss, ss_n, H, wqn, wkn, eps, rcos, rsin, rows, order, cpw,
                   kpool, vpool, kq8, part, counters, out_scale, ohi, olo, ldo, chain};
  const unsigned flags = chain.wait ? hipExtAnyOrderLaunch : 0u;
  if (nwg) *nwg = (int)(grid.x * grid.y * grid.z);
#define DEC_LAUNCH(GG, FU)                                                                                         \
  do {                                                                                                             \
    if (kq8.kq) {                                                                                                  \
      DEC_LAUNCH_Q(GG, FU, true);                                                                                  \
    } else {                                                                                                       \
      DEC_LAUNCH_Q(GG, FU, false);                                                                                 \
    }                                                                                                              \
  } while (0)
#define DEC_LAUNCH_Q(GG, FU, Q)          \
  do {                                   \
    if (ltab)                            \
      DEC_LAUNCH_T(GG, FU, Q, true);     \
    else                                 \
      DEC_LAUNCH_T(GG, FU, Q, false);    \
  } while (0)
#define DEC_LAUNCH_T(GG, FU, Q, LT)                                                                               \
  do {                                                                                                            \
    if (FU && ch)                                                                                                 \
      GQA_LAUNCH_F((attn_decode_kernel<GG, FU, Q, FU, LT>), grid, dim3(64 * kDecodeWaves), 0, st, flags, A);      \
    else                                                                                                          \
      hipLaunchKernelGGL((attn_decode_kernel<GG, FU, Q, false, LT>), grid, dim3(64 * kDecodeWaves), 0, st, A);    \
  } while (0)
  if (G != 4 && G != 2) return hipErrorInvalidValue;
  if (fused) {
    if (G == 4) DEC_LAUNCH(4, true);
    else DEC_LAUNCH(2, true);
  } else {
    if (G == 4) {
      DEC_LAUNCH(4, false);
      hipLaunchKernelGGL(attn_merge_kernel<4>, dim3(kKvHeads, B), dim3(256), 0, st, part, nq, rows, out_scale, ohi, olo,
                         ldo);
    } else {
      DEC_LAUNCH(2, false);
      hipLaunchKernelGGL(attn_merge_kernel<2>, dim3(kKvHeads, B), dim3(128), 0, st, part, nq, rows, out_scale, ohi, olo,
                         ldo);
    }
  }
#undef DEC_LAUNCH
#undef DEC_LAUNCH_Q
#undef DEC_LAUNCH_T
  return hipGetLastError();
}

// floats of the chunk-partial buffer for B rows of nq heads
int64_t attn_decode_part_floats(int nq) { return (int64_t)kMaxBatch * nq * kDecodeMaxChunks * kPartStride; }

}  // namespace gqa
