// Shared device helpers of the gfx950 decoder library: number formats, MFMA operand types,
// wave reductions and the launch-error plumbing used by every kernel file.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace gqa {

// Timing of single launches: when armed, the next kernel launched through GQA_LAUNCH records
// `start` and `stop` from its own dispatch packet (hipExtLaunchKernelGGL), so the interval is the
// kernel's execution and nothing else; the pair is consumed by that launch.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;
// GQA_LAUNCH_F passes dispatch flags (hipExtAnyOrderLaunch for the chained decode launches).
#define GQA_LAUNCH_F(kernel, grid, block, shm, st, flags, ...)                                                \
  do {                                                                                                      \
    if (::gqa::g_launch_events.start) {                                                                     \
      const ::gqa::LaunchEvents ev_ = ::gqa::g_launch_events;                                               \
      ::gqa::g_launch_events = ::gqa::LaunchEvents{};                                                       \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, st, ev_.start, ev_.stop, flags, __VA_ARGS__);        \
    } else if (flags) {                                                                                     \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, st, nullptr, nullptr, flags, __VA_ARGS__);           \
    } else {                                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, shm, st, __VA_ARGS__);                                        \
    }                                                                                                       \
  } while (0)
#define GQA_LAUNCH(kernel, grid, block, shm, st, ...) GQA_LAUNCH_F(kernel, grid, block, shm, st, 0u, __VA_ARGS__)


constexpr int kHeadDim = 128;
constexpr int kKvHeads = 8;
constexpr int kBlock = 32;          // positions per KV block
constexpr int kMaxBatch = 32;       // rows of one batched decode

// Block-table entries written by one launch (values passed as kernel arguments).
constexpr int kTableWritesMax = 32;
struct TableWrites {
  int32_t idx[kTableWritesMax];
  int32_t val[kTableWritesMax];
  int32_t n;
};
constexpr float kLog2e = 1.4426950408889634f;

// Epilogues of the projection kernels.
enum Epi : int { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };

// Per-row addressing of a batched decode call: position of the new token and the
// session's block table (logical block -> physical block).
struct Rows {
  int32_t pos[kMaxBatch];
  const int32_t* table[kMaxBatch];
};

// Source of the FP16 hi/lo operand rows of a decode matvec (see k_gemv.hip).
enum XMode : int { X_RAW = 0, X_RESID = 1, X_SWIGLU = 2 };
struct XSrc {
  int mode;
  // X_RAW: hi/lo rows in global memory, row stride ld
  const f16* hi;
  const f16* lo;
  int ld;
  // X_RESID: x = res[b] + pscale * sum_{s < nsplit} part[s][b] (fixed split order);
  // operand = x * w (the RMSNorm weight; the 1/rms factor is applied by the consumer of the
  // projection). x is written to res_out and the sum of squares of x over each K range to
  // ss_out[range][b] by the workgroups of the first row tile.
  const float* res;
  float* res_out;
  const float* part;
  int nsplit;
  int64_t pstride;
  int pld;
  float pscale;
  const uint16_t* w;
  float* ss_out;
  // X_SWIGLU: c = 1 / sqrt(sum_r ss[r][b] / H + eps); g = c * sum_s gu[s][b][32*(f/16) + f%16],
  // u = c * sum_s gu[s][b][32*(f/16) + 16 + f%16]; operand = silu(g) * u.
  const float* gu;
  int gu_split;
  int64_t gu_stride;
  int gu_ld;
  const float* ss;
  int ss_n;
  int H;
  float eps;
};

enum FullMode : int { XF_RAW = 0, XF_NORM = 1 };

// ---- Dependent decode launches without a queue barrier
// The per-layer launches of a decode of a few rows go out with hipExtAnyOrderLaunch: the queue
// then neither holds a launch until its predecessor has finished nor writes back and
// invalidates the L2 caches between the two, which removes the 1-1.5 us gap between dependent
// launches (most of a launch's fixed cost, its first loads and its tail, lies inside it and
// stays). Each launch orders itself against its predecessors instead:
//  * a producer writes what later launches of the chain read with device-scope stores (through
//    the non-coherent per-XCD L2 to memory); at its end every wave waits until its stores have
//    completed, then one thread adds 1 to arrival counter (workgroup index) % kChainLanes;
//  * a consumer first issues the loads that do not depend on its predecessors (weights, block
//    table, constants), then one wave polls the counters until each has reached the target the
//    host passed (the arrivals of every earlier launch of the chain), and then reads the
//    predecessors' outputs with device-scope loads.
// A wait is bounded: after kChainSpinMax polls (about 0.1 s) the workgroup sets kErrChainWait in
// the model's error word and goes on, and every later wait that sees the flag gives up at once
// (wrong results, reported by gqa_model_check_device_error; no hang). The counters are cleared
// by the first (ordered) launch of each call.
constexpr int kChainLanes = 16;
constexpr int kChainStride = 64;          // ints between counters: one 256-byte line each
constexpr int kChainInts = kChainLanes * kChainStride;
constexpr int kChainSpinMax = 1 << 16;
constexpr int32_t kErrChainWait = 2;
struct Chain {
  int32_t* cnt = nullptr;                 // arrival counters, or null: not chained
  int32_t* err = nullptr;                 // error word
  int wait = 0;                           // 1: wait for target[] first (any-order launch)
  int32_t target[kChainLanes] = {};
};

// Device-scope (sc1) accesses of the chained buffers.
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev8(const void* p) {
  return __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ld_dev16(const void* p) {
  const uint64_t a = ld_dev8(p), b = ld_dev8((const char*)p + 8);
  return uint4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev8(void* p, uint64_t v) {
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev16(void* p, uint4 v) {
  st_dev8(p, (uint64_t)v.x | ((uint64_t)v.y << 32));
  st_dev8((char*)p + 8, (uint64_t)v.z | ((uint64_t)v.w << 32));
}

// Wait until every counter has reached its target (all threads of the workgroup call this).
__device__ __forceinline__ void chain_wait(const Chain& c) {
  if (!c.wait) return;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // lanes 0..15 poll the counters, lane 16 the error word
    const int32_t want = lane < kChainLanes ? c.target[lane] : 0;
    const int32_t* at = lane < kChainLanes ? c.cnt + lane * kChainStride : c.err;
    for (int spin = 0;; ++spin) {
      const int32_t v = __hip_atomic_load(at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__all(lane >= kChainLanes || v >= want)) break;
      if (__any(lane >= kChainLanes && (v & kErrChainWait))) break;   // an earlier wait gave up
      if (spin >= kChainSpinMax) {
        if (lane == 0) __hip_atomic_fetch_or(c.err, kErrChainWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// Count this workgroup in once all of its stores have completed (all threads call this).
__device__ __forceinline__ void chain_signal(const Chain& c) {
  if (!c.cnt) return;
  __builtin_amdgcn_s_waitcnt(0);          // vmcnt = lgkmcnt = 0: this wave's stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    const int wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    __hip_atomic_fetch_add(c.cnt + (wg % kChainLanes) * kChainStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Host side: the targets of the next launch of a chain, and the arrivals of each launch.
struct ChainTrack {
  int32_t* cnt = nullptr;
  int32_t* err = nullptr;
  int32_t arrived[kChainLanes] = {};
  int launches = 0;
  int32_t offset = 0;                     // added to every target (a test of the bounded wait)
  // Arguments of the next launch: the first one is an ordinary launch (the queue holds it until
  // the call's earlier, unchained work has finished) that only signals; the others go out
  // any-order and wait. (An ordinary launch in the middle of a chain would cost more than the
  // chain saves: the queue would hold it until all any-order launches before it had finished.)
  Chain next() const {
    Chain c;
    if (!cnt) return c;
    c.cnt = cnt;
    c.err = err;
    c.wait = launches > 0;
    for (int i = 0; i < kChainLanes; ++i) c.target[i] = arrived[i] + offset;
    return c;
  }
  void launched(int nwg) {
    if (!cnt) return;
    for (int i = 0; i < kChainLanes; ++i) arrived[i] += nwg / kChainLanes + (i < nwg % kChainLanes ? 1 : 0);
    ++launches;
  }
};

// Arguments of the whole-K decode matvec (k_gemv_full.hip).
struct FullArgs {
  const uint16_t* W;
  const int8_t* Wq;        // Q8_0 quants, or AFFINE4 packed codes when Wb is set
  const f16* Wd;           // Q8_0 / AFFINE4 scales
  const f16* Wb;           // AFFINE4 biases (null otherwise)
  int K, N, B;
  const f16* xhi;          // XF_RAW: [B][ldx]
  const f16* xlo;
  int ldx;
  const float* xres;       // XF_NORM: [B][K] residual stream
  const uint16_t* nw;      // XF_NORM: norm weight [K]
  float eps;
  float* ss_out;           // XF_NORM: [range][32] sums of squares (written by workgroup 0)
  float* y;                // EPI_STORE / EPI_ADD: [B][ldy]
  int ldy;
  float yscale;
  f16* mhi;                // EPI_SWIGLU: [B][ldm]
  f16* mlo;
  int ldm;
  float2* cand;            // EPI_STORE: argmax candidates [B][N / 16] or null
  Chain chain;             // chained decode launch (or none)
};

// Sum-of-squares partials: ss[range][row], kMaxBatch rows per range.
// n <= 8; the loads are issued together and summed in range order.
__device__ __forceinline__ float inv_rms_from_ss(const float* ss, int n, int row, int H, float eps) {
  float v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = ss[min(r, n - 1) * 32 + row];   // unconditional, no branches
  float t = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) t += r < n ? v[r] : 0.f;
  return 1.0f / sqrtf(t / (float)H + eps);
}
// The same from device-scope loads (partials written by a chained predecessor).
__device__ __forceinline__ float inv_rms_from_ss_dev(const float* ss, int n, int row, int H, float eps) {
  float v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = ld_dev(ss + min(r, n - 1) * 32 + row);
  float t = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) t += r < n ? v[r] : 0.f;
  return 1.0f / sqrtf(t / (float)H + eps);
}

// Data-parallel-primitive (DPP) lane moves within rows of 16 lanes: no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i within each half row
constexpr int kDppMirror = 0x140;       // lane i <- 15 - i within each row
constexpr int kDppRor8 = 0x128;         // lane i <- (i + 8) mod 16 within each row

// Sum over the 16 lanes of each row; every lane of the row gets the same value.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}

// Weight matrices [rows][cols] (rows % 16 == 0, cols % 32 == 0) are stored tile-major: each
// 16-row x 32-column tile is one contiguous 512-element chunk laid out in the operand order of
// v_mfma_f32_16x16x32_f16 (lane l = 16 * g + r holds row r, columns 8g..8g+7), and the chunks of
// one 16-row band follow each other along the columns. A wave streaming a band therefore reads
// whole contiguous kilobytes (BF16) and needs no LDS transpose for the matrix operand.
__host__ __device__ __forceinline__ int64_t tiled_index(int64_t row, int64_t col, int64_t cols) {
  return ((((row >> 4) * (cols >> 5) + (col >> 5)) << 9) + ((((col & 31) >> 3) * 16 + (row & 15)) << 3) +
          (col & 7));
}
// FP16 prefill copy of a BF16 weight matrix [rows][cols] (rows % 32 == 0, cols % 32 == 0): per
// 32-row block and 32-column step one contiguous 1024-element piece ordered [kh][hf][row][8], the
// A-operand order of v_mfma_f32_32x32x16_f16 for the two 16-wide halves kh of the step.
__host__ __device__ __forceinline__ int64_t prefill_weight_index(int64_t row, int64_t col, int64_t cols) {
  return ((((row >> 5) * (cols >> 5) + (col >> 5)) << 10) + (((col >> 4) & 1) << 9) + (((col >> 3) & 1) << 8) +
          ((row & 31) << 3) + (col & 7));
}
// Q8_0 scale of (row, 32-column block): [row band][block][row within band].
__host__ __device__ __forceinline__ int64_t tiled_scale_index(int64_t row, int64_t blk, int64_t cols) {
  return (((row >> 4) * (cols >> 5) + blk) << 4) + (row & 15);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even; the values handled here are finite.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Q8_0 KV cache (Kipp Roadmap, status v0.0.4: opt-in Q8_0 KV). Each head row of 128 K or V values
// is stored as four blocks of 32 int8 codes with an fp16 scale, the Q8_0 weight format and rule:
// d = max|x| / 127 (FP32), scale = fp16(d), code = clamp(round_half_away(x / d), -127, 127), 0 when
// d = 0. The codes sit at the element offsets of the BF16 pool (one byte each), scale j of the row
// at element offset / 32. Attention reads bf16(fp32(scale) * code), the BF16 cache's operand format.
struct KvQ8 {
  int8_t* kq;      // nullptr: the cache is BF16
  int8_t* vq;
  f16* ks;
  f16* vs;
};
__device__ __forceinline__ float q8kv_scale(float amax) { return __fdiv_rn(amax, 127.0f); }
__device__ __forceinline__ int q8kv_code(float x, float d) {
  if (d == 0.f) return 0;
  return (int)fminf(fmaxf(roundf(__fdiv_rn(x, d)), -127.f), 127.f);
}
__device__ __forceinline__ uint16_t q8kv_read_bf16(f16 scale, int code) {
  return f32_to_bf16_rne((float)scale * (float)code);
}
// Eight Q8_0 KV codes of one 32-value block (two dwords, code j in byte j) -> the eight BF16
// values attention reads, bf16(fp32(scale) * code) each (q8kv_read_bf16), packed in pairs. The
// product is exact in FP32 (11 + 7 significant bits); v_cvt_pk_bf16_f32 rounds each to nearest
// even, as f32_to_bf16_rne does, two per instruction.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 q8kv_bf16x8(uint2 codes, f16 scale) {
  const float s = (float)scale;
  const uint32_t x[2] = {codes.x, codes.y};
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = x[i >> 1];
    const int sh = 16 * (i & 1);
    const float c0 = (float)(int8_t)((word >> sh) & 0xFFu), c1 = (float)(int8_t)((word >> (sh + 8)) & 0xFFu);
    const f32x2v p = {s * c0, s * c1};
    w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2v));
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// FP32 -> FP16 conversions of MFMA operands go through explicit instructions, never through a
// plain cast: the compiler is free to lower a cast to different instructions in different
// kernels (mixed-precision FMA forms fuse a preceding product), and every kernel that builds an
// operand must produce the same bits for the same value. Activations use cvt_rne2 (below);
// BF16 weights, exact in FP16 over their range, use v_cvt_pkrtz_f16_f32.
__device__ __forceinline__ f16x2 cvt_rtz2(float a, float b) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Eight BF16 weights (one 16-byte load) -> eight FP16 MFMA operands. BF16 has 8 significant
// bits, so the conversion is exact for |w| in [2^-17, 65504]; smaller magnitudes lose at most
// 2^-25 absolutely.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(uint4 v) {
  f16x8 r;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 p = cvt_rtz2(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xFFFF0000u));
    r[2 * i] = p[0];
    r[2 * i + 1] = p[1];
  }
  return r;
}

// FP32 pair -> FP16 pair rounded to nearest even, always by the one instruction
// v_cvt_pk_f16_f32 (written out so that no kernel lowers it differently).
__device__ __forceinline__ f16x2 cvt_rne2(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return __builtin_bit_cast(f16x2, r);
}

// Split an FP32 value into FP16 hi + lo: hi = rne(x), lo = rne(x - hi) (the difference is exact
// in FP32), so x = hi + lo to about 2^-22 relative (2^-25 absolute near zero). Two FP16 MFMAs
// over (hi, lo) give a near-FP32 product with BF16/FP16 weights; hi alone is the FP16 operand
// of the single-operand prefill mode (unbiased rounding, 2^-11 relative).
__device__ __forceinline__ void split_f16(float x, f16& hi, f16& lo) {
  hi = cvt_rne2(x, 0.f)[0];
  lo = cvt_rne2(x - (float)hi, 0.f)[0];
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16v8 __attribute__((ext_vector_type(8)));

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane l's 16 bytes land at
// lds_dst + 16 l, where lds_dst is the same for the whole wave. Issued as inline assembly: the
// compiler cannot tell which LDS bytes such a load writes and would otherwise wait for it before
// every LDS read. Being invisible to the compiler, the copies are also not covered by the waits
// it places before a barrier: a barrier that publishes them must follow vm_wait_all().
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds_dst) {
  // the destination is the same for the whole wave; readfirstlane keeps it in a scalar register
  // also where the copy sits under a lane condition
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
  // one wait state between the M0 write and the load that reads it
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(la), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Eight int8 quants (two dwords) -> eight exact FP16 values: the byte q + 128 (q ^ 0x80) below the
// FP16 pattern 0x64 is the value 1152 + q, and subtracting 1152 is exact.
// Weight formats of the matvec kernels.
enum WeightMode : int { WM_BF16 = 0, WM_Q8 = 1, WM_A4 = 2 };

// AFFINE4 codes of one operand lane, 8 K-elements of one weight row in a 32-bit word: nibble j
// holds element 2 j and nibble j + 4 element 2 j + 1 (j = 0..3), so (w >> 4 j) & 0x000F000F puts
// a pair under the FP16 exponent bits 0x6400 (the value 1024 + q) and one packed subtraction of
// 1024 leaves the exact codes.
__device__ __forceinline__ f16x8 u4x8_to_f16x8(uint32_t w) {
  const f16x2 base = {(f16)1024.0f, (f16)1024.0f};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 q = __builtin_bit_cast(f16x2, ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u) - base;
    r[2 * j] = q[0];
    r[2 * j + 1] = q[1];
  }
  return r;
}

// Four fp16 values (two 32-bit words) as FP32.
__device__ __forceinline__ void f16x4_bits_to_f32(uint2 v, float (&o)[4]) {
  o[0] = (float)__builtin_bit_cast(f16, (uint16_t)(v.x & 0xFFFF));
  o[1] = (float)__builtin_bit_cast(f16, (uint16_t)(v.x >> 16));
  o[2] = (float)__builtin_bit_cast(f16, (uint16_t)(v.y & 0xFFFF));
  o[3] = (float)__builtin_bit_cast(f16, (uint16_t)(v.y >> 16));
}

__device__ __forceinline__ f16x8 i8x8_to_f16x8(uint2 v) {
  const uint32_t x0 = v.x ^ 0x80808080u, x1 = v.y ^ 0x80808080u;
  const uint32_t h[4] = {__builtin_amdgcn_perm(0x64646464u, x0, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, x0, 0x05030402u),
                         __builtin_amdgcn_perm(0x64646464u, x1, 0x05010400u),
                         __builtin_amdgcn_perm(0x64646464u, x1, 0x05030402u)};
  const f16x2 bias = {(f16)1152.0f, (f16)1152.0f};
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 q = __builtin_bit_cast(f16x2, h[i]) - bias;
    r[2 * i] = q[0];
    r[2 * i + 1] = q[1];
  }
  return r;
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// One 32-wide K-step of a quantised band against one token column's operand (hi, lo), in two
// parts that every matvec path uses in the same order, so a row's result does not depend on the
// path. qstep_products: the codes' block products into a fresh accumulator p, and for AFFINE4 the
// operand's sum over the step xs (an all-ones A operand) -- both on the matrix cores.
// qstep_accumulate: per weight row acc += scale * p (Q8_0), or acc += scale * p + bias * xs
// (AFFINE4, w = scale * q + bias), in FP32. The kernels issue the products of several steps
// before accumulating them in step order, so no FMA waits on the MFMA just before it.
template <int QM>
__device__ __forceinline__ void qstep_products(f16x8 a, f16x8 bh, f16x8 bl, f32x4& p, f32x4& xs) {
  p = f32x4{0.f, 0.f, 0.f, 0.f};
  p = mfma16(a, bh, p);
  p = mfma16(a, bl, p);
  if constexpr (QM == WM_A4) {
    const f16 one = (f16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};
    xs = f32x4{0.f, 0.f, 0.f, 0.f};
    xs = mfma16(ones, bh, xs);
    xs = mfma16(ones, bl, xs);
  }
}

template <int QM>
__device__ __forceinline__ void qstep_accumulate(f32x4& acc, const f32x4& p, const f32x4& xs, uint2 sc2, uint2 bs2) {
  float sc[4];
  f16x4_bits_to_f32(sc2, sc);
  if constexpr (QM == WM_A4) {
    float bs[4];
    f16x4_bits_to_f32(bs2, bs);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(sc[r], p[r], fmaf(bs[r], xs[r], acc[r]));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(sc[r], p[r], acc[r]);
  }
}

// Widened codes of one operand lane.
template <int QM>
__device__ __forceinline__ f16x8 qwiden(uint2 q8, uint32_t q4) {
  if constexpr (QM == WM_A4) return u4x8_to_f16x8(q4);
  else return i8x8_to_f16x8(q8);
}

// Wave-wide sum / max: DPP within each 16-lane row, then the four row results read as scalars
// and combined in row order (the same value in every lane).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((a + b) + c) + d;
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

}  // namespace gqa
