// Host runtime and C ABI of the decoder library: model (weights, KV block pool, per-model
// scratch), sessions (block table, position), and the launch sequences of prefill rounds,
// single-row decode and batched decode. Declared in include/gqa.h.
//
// Kipp Roadmap, status v0.0.4: prefill runs in device-derived rounds, activation scratch is
// one per model and the split-K partial count is its own constant. Status v0.0.3: sessions
// take their KV blocks from one model-owned pool. Kipp Reproducing, "Build": failures are
// fatal errors, never a fallback.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gqa.h"
#include "_build/build_info.h"   // GQA_BUILD_INFO, written by build.py before every build
#include "gqa_common.h"
#include "kv_pool.h"

namespace gqa {
hipError_t launch_gen_weights(uint16_t* dst, uint64_t key, int64_t rows, int64_t cols, int mode, int64_t row_off,
                              float scale, hipStream_t st);
hipError_t launch_fill_u16(uint16_t* dst, int64_t n, uint16_t v, hipStream_t st);
hipError_t launch_quantize_q8_0(const uint16_t* w, int8_t* q, f16* d, int64_t rows, int64_t cols, hipStream_t st);
hipError_t launch_quantize_affine4(const uint16_t* w, uint8_t* q4, f16* d, f16* bias, int64_t rows, int64_t cols,
                                  hipStream_t st);
hipError_t launch_prefill_copy_q8(const int8_t* q, const f16* d, f16* dst, int64_t rows, int64_t cols, hipStream_t st);
hipError_t launch_prefill_copy_affine4(const uint8_t* q4, const f16* d, const f16* bias, f16* dst, int64_t rows,
                                       int64_t cols, hipStream_t st);
hipError_t launch_embed(const uint16_t* E, const int32_t* ids, int T, int H, int vocab, float* x, int32_t* err,
                        hipStream_t st, int32_t* zero = nullptr, int nzero = 0);
hipError_t launch_rmsnorm(float* x, int ldx, const float* part, int nsplit, int part_stride_split, int part_ld,
                          float part_scale, const uint16_t* w, int H, float eps, float out_scale, f16* yhi, f16* ylo,
                          int ldy, int rows, hipStream_t st);
hipError_t launch_qk_rope_kv(bool decode, const float* qkv, int nsplit, int part_stride, int ldqkv, int nq,
                             const uint16_t* wqn, const uint16_t* wkn, float eps, const float* rcos,
                             const float* rsin, int pos0, const int32_t* table0, const Rows& rows, uint16_t* kpool,
                             uint16_t* vpool, const KvQ8& kq8, float* qout, int nrows, hipStream_t st);
hipError_t launch_argmax(const float2* cand, int ntiles, int B, int32_t* out, hipStream_t st);
hipError_t launch_argmax_rows(const float* logits, int V, int64_t ld, int rows, int32_t* out, hipStream_t st);
hipError_t launch_score(const float* logits, int V, const int32_t* targets, int B, float* out, hipStream_t st);
hipError_t launch_table_writes(int32_t* table, const TableWrites& t, hipStream_t st);
hipError_t launch_swiglu_rows(const float* gu, int nsplit, int64_t stride, int ldgu, int F, int rows, f16* mh, f16* ml,
                              int ldm, hipStream_t st);
hipError_t launch_prefill_copy(const uint16_t* src, f16* dst, int64_t rows, int64_t cols, hipStream_t st);
hipError_t launch_gemm(int epi, bool split, const f16* W, const int8_t* Wq, const f16* Wd, int K, int N, const f16* Xhi,
                       const f16* Xlo, int ldx, int T, float* C, int ldc, float out_scale, f16* Mhi, f16* Mlo,
                       int ldm, float m_scale, int ksplit, int64_t split_stride, hipStream_t st,
                       int nvalid = 0);
hipError_t launch_gemv(const uint16_t* W, const int8_t* Wq, const f16* Wd, const f16* Wb, int K, int N, const XSrc& xs, int B,
                       int nsplit, float* P, int64_t part_stride, int ldp, float2* cand, hipStream_t st,
                       bool staged = false);
hipError_t launch_rows(const XSrc& xs, int K, int nsplit, int B, f16* yhi, f16* ylo, int ldy, hipStream_t st);
bool gemv_full_fits(int K, int B);
hipError_t launch_gemv_full(int mode, int epi, int S, const FullArgs& a, hipStream_t st, int* nwg = nullptr);
hipError_t launch_final_norm(const XSrc& xs, int B, f16* yhi, f16* ylo, int ldy, hipStream_t st);
hipError_t launch_attn_prefill(const float* q, int nq, int T, int pos0, const int32_t* table, const uint16_t* kpool,
                               const uint16_t* vpool, const KvQ8& kq8, float out_scale, f16* ohi, f16* olo, int ldo,
                               float* part, hipStream_t st);
hipError_t launch_attn_decode(const float* qkvp, int nsplit, int64_t pstride, int QKV, int nq, const float* ss,
                              int ss_n, int H, const uint16_t* wqn, const uint16_t* wkn, float eps, const float* rcos,
                              const float* rsin, const Rows& rows, int B, int max_ctx, uint16_t* kpool,
                              uint16_t* vpool, const KvQ8& kq8, float* part, int* counters, float out_scale, f16* ohi,
                              f16* olo, int ldo, hipStream_t st, const Chain& chain = Chain{}, int* nwg = nullptr);
int64_t attn_decode_part_floats(int nq);
}  // namespace gqa

namespace gqa {
thread_local LaunchEvents g_launch_events;

// The whole-K decode path's per-layer launches go out as one chain of any-order launches
// (gqa_common.h); 0 launches them as ordinary dependent launches (same kernels, same results).
#ifndef GQA_DECODE_CHAIN
#define GQA_DECODE_CHAIN 1
#endif
constexpr bool kDecodeChain = GQA_DECODE_CHAIN != 0;
}

using namespace gqa;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                         \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(GQA_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
uint64_t splitmix(uint64_t key, uint64_t i) {
  uint64_t z = key + (i + 1ull) * kGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Scale of the generator: 0.02 / std of the sum of four uniform 16-bit integers.
float weight_scale() { return (float)(0.02 / sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0)); }

// Attention output enters the o projection multiplied by this power of two (and the
// projection result is divided by it), keeping the FP16 lo half of small outputs normal.
constexpr float kAttnOutScale = 16.0f;

// Rows of one scoring GEMM (the logits scratch holds this many rows).
constexpr int kScoreRows = 256;

struct LayerW {
  uint16_t *attn_norm = nullptr, *ffn_norm = nullptr, *q_norm = nullptr, *k_norm = nullptr;
  uint16_t *wqkv = nullptr, *wo = nullptr, *wgu = nullptr, *wd = nullptr;                  // BF16
  f16 *pqkv = nullptr, *po = nullptr, *pgu = nullptr, *pd = nullptr;                       // FP16 prefill copies
  int8_t *qqkv = nullptr, *qo = nullptr, *qgu = nullptr, *qd = nullptr;   // Q8_0 quants / AFFINE4 codes
  f16 *sqkv = nullptr, *so = nullptr, *sgu = nullptr, *sd = nullptr;       // Q8_0 / AFFINE4 scales
  f16 *bqkv = nullptr, *bo = nullptr, *bgu = nullptr, *bd = nullptr;       // AFFINE4 biases
  uint16_t *kpool = nullptr, *vpool = nullptr;   // BF16 cache; with a Q8_0 cache: null
  KvQ8 kq8{nullptr, nullptr, nullptr, nullptr};   // Q8_0 cache: codes and scales
};

}  // namespace

struct gqa_model {
  gqa_model_desc d{};
  int dev = 0, cu = 0, R = 0;
  int QKV = 0, QD = 0;          // fused q|k|v rows, attention width
  int s_qkv = 1, s_o = 1, s_gu = 1, s_d = 1;  // decode split-K counts
  std::vector<LayerW> L;
  uint16_t *embed = nullptr, *lm_head = nullptr, *final_norm = nullptr;
  f16* plm = nullptr;           // FP16 prefill copy of the lm_head, rows padded with zeros to Vpad
  int Vpad = 0;                 // vocab rounded up to the GEMM's 256-row tile
  float *rcos = nullptr, *rsin = nullptr;
  float *x = nullptr, *x2 = nullptr, *qkv = nullptr, *q = nullptr, *part = nullptr, *part2 = nullptr,
        *apart = nullptr;
  float* ppart = nullptr;       // prefill: K-range partials of the o and down projections [<= 4 R][H]
  int32_t* counters = nullptr;  // decode attention: finished chunks per (row, KV head)
  int32_t* chain = nullptr;     // decode: arrival counters of the chained launches (kChainInts)
  float* ss = nullptr;          // decode: sum-of-squares partials [2][8][32] (q|k|v input, gate|up input)
  float2* cand = nullptr;   // lm_head argmax candidates [32][vocab / 16]
  float* slog = nullptr;    // logits of up to kScoreRows rows being scored [kScoreRows][vocab]
  f16 *xh = nullptr, *xl = nullptr, *oh = nullptr, *ol = nullptr, *mh = nullptr, *ml = nullptr;
  int32_t *ids_dev = nullptr, *err = nullptr;
  int32_t* ids_host = nullptr;  // pinned staging
  hipEvent_t ids_evt = nullptr;
  int64_t part_floats = 0;
  std::vector<void*> allocs;
  std::unique_ptr<KvPool> pool;   // block states and the prefix cache
  int sessions = 0;
  int64_t weight_bytes = 0, kv_bytes = 0, scratch_bytes = 0, prefill_copy_bytes = 0;
  std::mutex mu;
  // kernel timing (gqa_model_profile)
  int prof_cls = GQA_PROF_NONE;
  std::vector<hipEvent_t> prof_ev;
  int64_t prof_used = 0, prof_dropped = 0;
  int32_t chain_offset = 0;     // gqa_model_debug_chain_offset
};

struct gqa_session {
  gqa_model* m = nullptr;
  int max_pos = 0, pos = 0;
  std::vector<int32_t> blocks;          // fixed table (sessions created with gqa_session_create)
  std::unique_ptr<PooledSeq> seq;       // on-demand table with prefix sharing (pooled sessions)
  int32_t reused = 0;                   // positions the last eval_prefill took from the cache
  int32_t* d_table = nullptr;
};

namespace {

void free_model(gqa_model* m) {
  if (!m) return;
  for (hipEvent_t e : m->prof_ev) (void)hipEventDestroy(e);
  for (void* p : m->allocs) (void)hipFree(p);
  if (m->ids_host) (void)hipHostFree(m->ids_host);
  if (m->ids_evt) (void)hipEventDestroy(m->ids_evt);
  delete m;
}

template <class T>
int dalloc(gqa_model* m, T** p, int64_t count, int64_t* counter) {
  void* v = nullptr;
  size_t bytes = (size_t)std::max<int64_t>(count, 1) * sizeof(T);
  hipError_t e = hipMalloc(&v, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(GQA_E_OOM, "hipMalloc of %zu bytes failed: %s", bytes, hipGetErrorString(e));
  }
  m->allocs.push_back(v);
  *p = (T*)v;
  if (counter) *counter += (int64_t)bytes;
  return GQA_OK;
}

int check_desc(const gqa_model_desc* d) {
  if (!d) return fail(GQA_E_INVALID, "null descriptor");
  if (d->n_kv_heads != kKvHeads || d->head_dim != kHeadDim)
    return fail(GQA_E_INVALID, "n_kv_heads must be 8 and head_dim 128");
  if (d->n_q_heads != 16 && d->n_q_heads != 32) return fail(GQA_E_INVALID, "n_q_heads must be 16 or 32");
  if (d->n_layers < 1 || d->hidden < 256 || d->hidden > 4096 || d->hidden % 256 || d->ffn < 128 ||
      (2 * d->ffn) % 256 || d->vocab < 16 || d->vocab % 16)
    return fail(GQA_E_INVALID, "unsupported shape (hidden %% 256, hidden <= 4096, 2*ffn %% 256, vocab %% 16)");
  if (d->scheme != GQA_SCHEME_BF16 && d->scheme != GQA_SCHEME_Q8_0 && d->scheme != GQA_SCHEME_AFFINE4)
    return fail(GQA_E_INVALID, "unknown scheme");
  if (d->prefill_operands != GQA_PREFILL_SPLIT && d->prefill_operands != GQA_PREFILL_FP16)
    return fail(GQA_E_INVALID, "unknown prefill_operands");
  if (d->prefill_q8_direct != 0 && d->prefill_q8_direct != 1) return fail(GQA_E_INVALID, "prefill_q8_direct must be 0 or 1");
  if (d->kv_quant != GQA_KV_BF16 && d->kv_quant != GQA_KV_Q8_0) return fail(GQA_E_INVALID, "kv_quant must be 0 or 1");
  if (d->kv_pool_blocks < 1 || d->max_positions < 1 || d->max_round_tokens < 0)
    return fail(GQA_E_INVALID, "kv_pool_blocks and max_positions must be positive");
  if (!(d->rope_theta > 1.0f) || !(d->rms_eps > 0.0f)) return fail(GQA_E_INVALID, "bad rope_theta or rms_eps");
  return GQA_OK;
}

// Generator tensor ids: embedding 0; layer l, kind j (attn_norm, q, k, v, q_norm, k_norm, o,
// ffn_norm, gate, up, down) -> 1 + 11 l + j; final norm 1 + 11 L; lm_head 2 + 11 L.
uint64_t tensor_key(uint64_t seed, int L, int kind, int layer) {
  int tid;
  if (kind == GQA_T_EMBED)
    tid = 0;
  else if (kind == GQA_T_FINAL_NORM)
    tid = 1 + 11 * L;
  else if (kind == GQA_T_LM_HEAD)
    tid = 2 + 11 * L;
  else
    tid = 1 + 11 * layer + (kind - GQA_T_ATTN_NORM);
  return splitmix(seed, (uint64_t)tid);
}

// Per-call scratch of a decode: the residual stream (two buffers for the split-K path), the
// projection outputs or split partials, the operand rows, the attention chunk partials and
// arrival counters, the sum-of-squares partials, the argmax candidates and the arrival counters
// of the chained launches. The model's own buffers by default; gqa_session_eval_decode_static
// carves them from a static device array. `zero` (nzero ints, or null) is cleared by the first
// kernel of the call.
struct DecodeScratch {
  float *x = nullptr, *x2 = nullptr, *part = nullptr, *part2 = nullptr, *ss = nullptr, *apart = nullptr;
  int32_t* counters = nullptr;
  int32_t* chain = nullptr;
  f16 *oh = nullptr, *ol = nullptr, *mh = nullptr, *ml = nullptr, *xh = nullptr, *xl = nullptr;
  float2* cand = nullptr;
  int64_t pstride = 0;     // stride of split-K partial ranges (floats)
  int32_t* zero = nullptr;
  int nzero = 0;
};

DecodeScratch model_scratch(gqa_model* m) {
  DecodeScratch sc;
  sc.x = m->x;
  sc.x2 = m->x2;
  sc.part = m->part;
  sc.part2 = m->part2;
  sc.ss = m->ss;
  sc.apart = m->apart;
  sc.counters = m->counters;
  sc.chain = m->chain;
  sc.zero = m->chain;
  sc.nzero = kChainInts;
  sc.oh = m->oh;
  sc.ol = m->ol;
  sc.mh = m->mh;
  sc.ml = m->ml;
  sc.xh = m->xh;
  sc.xl = m->xl;
  sc.cand = m->cand;
  sc.pstride = m->part_floats / 8;
  return sc;
}

// ---- allocation-free decode (gqa_session_eval_decode_static)
// The per-call decode scratch of one row lives in this file-scope device array, one copy per
// device, held until the process ends. Host code never uses the name `scratch` as an address
// (on the host it is only a stand-in): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in g_scratch_base.
constexpr size_t kStaticScratchBytes = (size_t)2 << 20;   // 2 MiB
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_base[kMaxDevices] = {};

int static_scratch_base(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(GQA_E_INVALID, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_base[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GQA_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_base[dev] = p;
  }
  *out = g_scratch_base[dev];
  return GQA_OK;
}

// Lay one row's decode scratch out from `base` (256-byte aligned pieces) and return the bytes
// it spans; with base == nullptr only the size is computed. Whole-K matvec path only (no split
// partials, no second residual buffer); the attention partials of row 0 and its eight arrival
// counters, then the chain's arrival counters, which the call's embedding launch clears.
size_t carve_static_scratch(const gqa_model* m, void* base, DecodeScratch* sc) {
  const gqa_model_desc& d = m->d;
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? (void*)((char*)base + off) : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  *sc = DecodeScratch{};
  sc->x = (float*)take(4 * (size_t)d.hidden);
  sc->part = (float*)take(4 * (size_t)m->QKV);
  sc->ss = (float*)take(4 * 2 * 8 * 32);
  sc->apart = (float*)take(4 * (size_t)(attn_decode_part_floats(d.n_q_heads) / kMaxBatch));
  sc->counters = (int32_t*)take(4 * kKvHeads);       // 256 bytes, then the chain counters
  sc->chain = (int32_t*)take(4 * kChainInts);
  sc->oh = (f16*)take(2 * (size_t)m->QD);
  sc->ol = (f16*)take(2 * (size_t)m->QD);
  sc->mh = (f16*)take(2 * (size_t)d.ffn);
  sc->ml = (f16*)take(2 * (size_t)d.ffn);
  sc->xh = (f16*)take(2 * (size_t)d.hidden);
  sc->xl = (f16*)take(2 * (size_t)d.hidden);
  sc->cand = (float2*)take(sizeof(float2) * (size_t)(d.vocab / 16));
  sc->pstride = m->QKV;
  sc->zero = sc->counters;
  sc->nzero = 64 + kChainInts;
  return off;
}

int eval_rows(gqa_session* const* ss, int32_t B, const int32_t* ids, int32_t ids_on_device, float* logits,
              int32_t* argmax, const DecodeScratch* scr, hipStream_t st);

}  // namespace

extern "C" {

const char* gqa_last_error(void) { return g_err.c_str(); }

const char* gqa_build_info(void) { return GQA_BUILD_INFO; }

int gqa_device_describe(int32_t device, gqa_device_desc* out) {
  g_err.clear();
  if (!out) return fail(GQA_E_INVALID, "null out pointer");
  int n = 0;
  HIP_TRY(hipGetDeviceCount(&n));
  if (device < 0 || device >= n) return fail(GQA_E_INVALID, "device %d outside [0, %d)", device, n);
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, device));
  memset(out, 0, sizeof(*out));
  snprintf(out->name, sizeof(out->name), "%s", prop.name);
  snprintf(out->arch, sizeof(out->arch), "%s", prop.gcnArchName);
  out->cu_count = prop.multiProcessorCount;
  out->clock_khz = prop.clockRate;
  out->memory_clock_khz = prop.memoryClockRate;
  out->memory_bus_bits = prop.memoryBusWidth;
  out->total_memory = (int64_t)prop.totalGlobalMem;
  out->l2_bytes = prop.l2CacheSize;
  out->lds_per_cu = (int64_t)prop.maxSharedMemoryPerMultiProcessor;
  HIP_TRY(hipRuntimeGetVersion(&out->runtime_version));
  HIP_TRY(hipDriverGetVersion(&out->driver_version));
  return GQA_OK;
}

int gqa_model_create(const gqa_model_desc* desc, uint64_t seed, gqa_model** out) {
  g_err.clear();
  if (!out) return fail(GQA_E_INVALID, "null out pointer");
  int rc = check_desc(desc);
  if (rc) return rc;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(GQA_E_DEVICE, "device %d is %s, this library is built for gfx950 only", dev, prop.gcnArchName);

  gqa_model* m = new gqa_model();
  m->d = *desc;
  m->dev = dev;
  m->cu = prop.multiProcessorCount;
  const gqa_model_desc& d = m->d;
  const int H = d.hidden, F = d.ffn, V = d.vocab, NQ = d.n_q_heads;
  m->QD = NQ * kHeadDim;
  m->QKV = m->QD + 2 * kKvHeads * kHeadDim;
  m->R = d.max_round_tokens > 0 ? d.max_round_tokens : std::max(64, m->cu * 8);
  // K ranges of the decode matvecs, fixed per model and shared by the whole-K path (one wave
  // per range) and the split-K path (one workgroup column per range), so every row sums the
  // same range partials in the same order on both paths
  m->s_qkv = 8;
  m->s_o = 8;
  m->s_gu = 4;
  m->s_d = (F / 32) % 8 == 0 ? 8 : 4;
  const bool q8 = d.scheme == GQA_SCHEME_Q8_0, a4 = d.scheme == GQA_SCHEME_AFFINE4;
  const bool q8copy = q8 && !d.prefill_q8_direct;       // Q8_0 prefill over FP16 copies
  int64_t* wb = &m->weight_bytes;

#define ALLOC(p, n, ctr)                      \
  do {                                        \
    int r_ = dalloc(m, &(p), (int64_t)(n), ctr); \
    if (r_) {                                 \
      free_model(m);                          \
      return r_;                              \
    }                                         \
  } while (0)

  ALLOC(m->embed, (int64_t)V * H, wb);
  ALLOC(m->final_norm, H, wb);
  if (!d.tied)
    ALLOC(m->lm_head, (int64_t)V * H, wb);
  else
    m->lm_head = m->embed;
  m->L.resize(d.n_layers);
  const int64_t pool_elems = (int64_t)d.kv_pool_blocks * kKvHeads * kBlock * kHeadDim;
  for (int l = 0; l < d.n_layers; ++l) {
    LayerW& w = m->L[l];
    ALLOC(w.attn_norm, H, wb);
    ALLOC(w.ffn_norm, H, wb);
    ALLOC(w.q_norm, kHeadDim, wb);
    ALLOC(w.k_norm, kHeadDim, wb);
    if (q8) {
      ALLOC(w.qqkv, (int64_t)m->QKV * H, wb);
      ALLOC(w.sqkv, (int64_t)m->QKV * H / 32, wb);
      ALLOC(w.qo, (int64_t)H * m->QD, wb);
      ALLOC(w.so, (int64_t)H * m->QD / 32, wb);
      ALLOC(w.qgu, (int64_t)2 * F * H, wb);
      ALLOC(w.sgu, (int64_t)2 * F * H / 32, wb);
      ALLOC(w.qd, (int64_t)H * F, wb);
      ALLOC(w.sd, (int64_t)H * F / 32, wb);
      if (q8copy) {
        ALLOC(w.pqkv, (int64_t)m->QKV * H, &m->prefill_copy_bytes);
        ALLOC(w.po, (int64_t)H * m->QD, &m->prefill_copy_bytes);
        ALLOC(w.pgu, (int64_t)2 * F * H, &m->prefill_copy_bytes);
        ALLOC(w.pd, (int64_t)H * F, &m->prefill_copy_bytes);
      }
    } else if (a4) {
      // codes (half a byte per weight), scales and biases; FP16 dequantised copies for prefill
      ALLOC(w.qqkv, (int64_t)m->QKV * H / 2, wb);
      ALLOC(w.sqkv, (int64_t)m->QKV * H / 32, wb);
      ALLOC(w.bqkv, (int64_t)m->QKV * H / 32, wb);
      ALLOC(w.qo, (int64_t)H * m->QD / 2, wb);
      ALLOC(w.so, (int64_t)H * m->QD / 32, wb);
      ALLOC(w.bo, (int64_t)H * m->QD / 32, wb);
      ALLOC(w.qgu, (int64_t)2 * F * H / 2, wb);
      ALLOC(w.sgu, (int64_t)2 * F * H / 32, wb);
      ALLOC(w.bgu, (int64_t)2 * F * H / 32, wb);
      ALLOC(w.qd, (int64_t)H * F / 2, wb);
      ALLOC(w.sd, (int64_t)H * F / 32, wb);
      ALLOC(w.bd, (int64_t)H * F / 32, wb);
      ALLOC(w.pqkv, (int64_t)m->QKV * H, &m->prefill_copy_bytes);
      ALLOC(w.po, (int64_t)H * m->QD, &m->prefill_copy_bytes);
      ALLOC(w.pgu, (int64_t)2 * F * H, &m->prefill_copy_bytes);
      ALLOC(w.pd, (int64_t)H * F, &m->prefill_copy_bytes);
    } else {
      ALLOC(w.wqkv, (int64_t)m->QKV * H, wb);
      ALLOC(w.wo, (int64_t)H * m->QD, wb);
      ALLOC(w.wgu, (int64_t)2 * F * H, wb);
      ALLOC(w.wd, (int64_t)H * F, wb);
      ALLOC(w.pqkv, (int64_t)m->QKV * H, &m->prefill_copy_bytes);
      ALLOC(w.po, (int64_t)H * m->QD, &m->prefill_copy_bytes);
      ALLOC(w.pgu, (int64_t)2 * F * H, &m->prefill_copy_bytes);
      ALLOC(w.pd, (int64_t)H * F, &m->prefill_copy_bytes);
    }
    if (d.kv_quant == GQA_KV_Q8_0) {
      ALLOC(w.kq8.kq, pool_elems, &m->kv_bytes);
      ALLOC(w.kq8.vq, pool_elems, &m->kv_bytes);
      ALLOC(w.kq8.ks, pool_elems / 32, &m->kv_bytes);
      ALLOC(w.kq8.vs, pool_elems / 32, &m->kv_bytes);
    } else {
      ALLOC(w.kpool, pool_elems, &m->kv_bytes);
      ALLOC(w.vpool, pool_elems, &m->kv_bytes);
    }
  }
  const int rows = std::max(m->R, kMaxBatch);
  int64_t* sb = &m->scratch_bytes;
  ALLOC(m->x, (int64_t)rows * H, sb);
  ALLOC(m->x2, (int64_t)kMaxBatch * H, sb);
  ALLOC(m->xh, (int64_t)rows * H, sb);
  ALLOC(m->xl, (int64_t)rows * H, sb);
  ALLOC(m->qkv, (int64_t)m->R * m->QKV, sb);
  ALLOC(m->q, (int64_t)rows * m->QD, sb);
  ALLOC(m->oh, (int64_t)rows * m->QD, sb);
  ALLOC(m->ol, (int64_t)rows * m->QD, sb);
  ALLOC(m->mh, (int64_t)rows * F, sb);
  ALLOC(m->ml, (int64_t)rows * F, sb);
  m->part_floats = (int64_t)8 * kMaxBatch * std::max(std::max(m->QKV, 2 * F), H);
  ALLOC(m->part, m->part_floats, sb);
  ALLOC(m->part2, m->part_floats, sb);
  ALLOC(m->apart, attn_decode_part_floats(NQ), sb);
  ALLOC(m->ppart, (int64_t)4 * m->R * H, sb);
  ALLOC(m->counters, kMaxBatch * kKvHeads, sb);
  ALLOC(m->chain, kChainInts, sb);
  ALLOC(m->ss, 2 * 8 * 32, sb);
  ALLOC(m->ids_dev, std::max(d.max_positions, kMaxBatch), sb);
  ALLOC(m->cand, (int64_t)kMaxBatch * (V / 16), sb);
  ALLOC(m->slog, (int64_t)kScoreRows * V, sb);
  m->Vpad = (V + 255) / 256 * 256;
  ALLOC(m->plm, (int64_t)m->Vpad * H, &m->prefill_copy_bytes);
  ALLOC(m->err, 1, sb);
  ALLOC(m->rcos, (int64_t)d.max_positions * 64, sb);
  ALLOC(m->rsin, (int64_t)d.max_positions * 64, sb);
#undef ALLOC
  hipError_t e = hipHostMalloc((void**)&m->ids_host, sizeof(int32_t) * std::max(d.max_positions, kMaxBatch),
                               hipHostMallocDefault);
  if (e != hipSuccess) {
    free_model(m);
    return fail(GQA_E_OOM, "pinned staging allocation failed: %s", hipGetErrorString(e));
  }
  if ((e = hipEventCreateWithFlags(&m->ids_evt, hipEventDisableTiming)) != hipSuccess) {
    free_model(m);
    return fail(GQA_E_HIP, "hipEventCreate failed: %s", hipGetErrorString(e));
  }

  // weights
  hipStream_t st = nullptr;
  const float sc = weight_scale();
  uint16_t* tmp = nullptr;
  if (q8 || a4) {
    int64_t biggest = std::max<int64_t>(std::max<int64_t>((int64_t)2 * F * H, (int64_t)m->QKV * H),
                                        std::max<int64_t>((int64_t)H * m->QD, (int64_t)H * F));
    void* v = nullptr;
    if (hipMalloc(&v, biggest * 2) != hipSuccess) {
      (void)hipGetLastError();
      free_model(m);
      return fail(GQA_E_OOM, "temporary BF16 buffer for quantisation does not fit");
    }
    tmp = (uint16_t*)v;
  }
  auto gen = [&](uint16_t* dst, int kind, int layer, int64_t r, int64_t c, int mode, int64_t off) {
    return launch_gen_weights(dst, tensor_key(seed, d.n_layers, kind, layer), r, c, mode, off, sc, st);
  };
  hipError_t ge = hipSuccess;
  auto chk = [&](hipError_t x) {
    if (x != hipSuccess && ge == hipSuccess) ge = x;
  };
  chk(gen(m->embed, GQA_T_EMBED, -1, V, H, 0, 0));
  if (!d.tied) chk(gen(m->lm_head, GQA_T_LM_HEAD, -1, V, H, 0, 0));
  chk(launch_prefill_copy(m->lm_head, m->plm, V, H, st));
  chk(hipMemsetAsync(m->plm + (int64_t)V * H, 0, (size_t)(m->Vpad - V) * H * 2, st));
  chk(launch_fill_u16(m->final_norm, H, 0x3F80, st));
  const int KVD = kKvHeads * kHeadDim;
  for (int l = 0; l < d.n_layers && ge == hipSuccess; ++l) {
    LayerW& w = m->L[l];
    chk(launch_fill_u16(w.attn_norm, H, 0x3F80, st));
    chk(launch_fill_u16(w.ffn_norm, H, 0x3F80, st));
    chk(launch_fill_u16(w.q_norm, kHeadDim, 0x3F80, st));
    chk(launch_fill_u16(w.k_norm, kHeadDim, 0x3F80, st));
    // quantised schemes generate each projection into tmp and quantise it from there
    auto quant = [&](int8_t* q, f16* sc_, f16* b_, f16* pcopy, int64_t r, int64_t c) {
      if (q8) chk(launch_quantize_q8_0(tmp, q, sc_, r, c, st));
      if (q8copy) chk(launch_prefill_copy_q8(q, sc_, pcopy, r, c, st));
      if (a4) {
        chk(launch_quantize_affine4(tmp, (uint8_t*)q, sc_, b_, r, c, st));
        chk(launch_prefill_copy_affine4((const uint8_t*)q, sc_, b_, pcopy, r, c, st));
      }
    };
    const bool qs = q8 || a4;
    uint16_t* dqkv = qs ? tmp : w.wqkv;
    chk(gen(dqkv, GQA_T_Q, l, m->QD, H, 0, 0));
    chk(gen(dqkv, GQA_T_K, l, KVD, H, 0, m->QD));
    chk(gen(dqkv, GQA_T_V, l, KVD, H, 0, m->QD + KVD));
    if (qs) quant(w.qqkv, w.sqkv, w.bqkv, w.pqkv, m->QKV, H);
    uint16_t* dO = qs ? tmp : w.wo;
    chk(gen(dO, GQA_T_O, l, H, m->QD, 0, 0));
    if (qs) quant(w.qo, w.so, w.bo, w.po, H, m->QD);
    uint16_t* dgu = qs ? tmp : w.wgu;
    chk(gen(dgu, GQA_T_GATE, l, F, H, 1, 0));
    chk(gen(dgu, GQA_T_UP, l, F, H, 2, 0));
    if (qs) quant(w.qgu, w.sgu, w.bgu, w.pgu, 2 * F, H);
    uint16_t* dD = qs ? tmp : w.wd;
    chk(gen(dD, GQA_T_DOWN, l, H, F, 0, 0));
    if (qs) quant(w.qd, w.sd, w.bd, w.pd, H, F);
    if (!qs) {
      chk(launch_prefill_copy(w.wqkv, w.pqkv, m->QKV, H, st));
      chk(launch_prefill_copy(w.wo, w.po, H, m->QD, st));
      chk(launch_prefill_copy(w.wgu, w.pgu, 2 * F, H, st));
      chk(launch_prefill_copy(w.wd, w.pd, H, F, st));
    }
    if (qs) chk(hipStreamSynchronize(st));
    if (d.kv_quant == GQA_KV_Q8_0) {
      chk(hipMemsetAsync(w.kq8.kq, 0, pool_elems, st));
      chk(hipMemsetAsync(w.kq8.vq, 0, pool_elems, st));
      chk(hipMemsetAsync(w.kq8.ks, 0, pool_elems / 32 * 2, st));
      chk(hipMemsetAsync(w.kq8.vs, 0, pool_elems / 32 * 2, st));
    } else {
      chk(hipMemsetAsync(w.kpool, 0, pool_elems * 2, st));
      chk(hipMemsetAsync(w.vpool, 0, pool_elems * 2, st));
    }
  }
  chk(hipMemsetAsync(m->err, 0, 4, st));
  chk(hipMemsetAsync(m->counters, 0, sizeof(int32_t) * kMaxBatch * kKvHeads, st));
  chk(hipMemsetAsync(m->chain, 0, sizeof(int32_t) * kChainInts, st));
  chk(hipDeviceSynchronize());
  if (tmp) (void)hipFree(tmp);
  if (ge != hipSuccess) {
    free_model(m);
    return fail(GQA_E_HIP, "weight generation failed: %s", hipGetErrorString(ge));
  }

  // RoPE: angle p * theta^(-2i/128) in double, cos/sin rounded to FP32.
  {
    std::vector<float> c((size_t)d.max_positions * 64), s((size_t)d.max_positions * 64);
    for (int p = 0; p < d.max_positions; ++p)
      for (int i = 0; i < 64; ++i) {
        double inv = pow((double)d.rope_theta, -2.0 * i / 128.0);
        double a = (double)p * inv;
        c[(size_t)p * 64 + i] = (float)cos(a);
        s[(size_t)p * 64 + i] = (float)sin(a);
      }
    e = hipMemcpy(m->rcos, c.data(), c.size() * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(m->rsin, s.data(), s.size() * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      free_model(m);
      return fail(GQA_E_HIP, "RoPE table upload failed: %s", hipGetErrorString(e));
    }
  }
  m->pool.reset(new KvPool(d.kv_pool_blocks));
  *out = m;
  return GQA_OK;
}

void gqa_model_destroy(gqa_model* model) {
  if (!model) return;
  (void)hipDeviceSynchronize();
  free_model(model);
}

int gqa_model_get_info(const gqa_model* m, gqa_model_info* info) {
  if (!m || !info) return fail(GQA_E_INVALID, "null argument");
  info->round_tokens = m->R;
  info->cu_count = m->cu;
  info->weight_bytes = m->weight_bytes;
  info->kv_pool_bytes = m->kv_bytes;
  info->scratch_bytes = m->scratch_bytes;
  info->prefill_copy_bytes = m->prefill_copy_bytes;
  info->free_blocks = m->pool->available();
  info->cached_blocks = m->pool->cached_count();
  info->prefix_lookups = (int64_t)m->pool->lookups;
  info->prefix_hits = (int64_t)m->pool->hits;
  info->prefix_evictions = (int64_t)m->pool->evictions;
  return GQA_OK;
}

int gqa_session_create(gqa_model* m, int32_t max_positions, const int32_t* block_ids, gqa_session** out) {
  g_err.clear();
  if (!m || !out) return fail(GQA_E_INVALID, "null argument");
  if (max_positions < 1 || max_positions > m->d.max_positions)
    return fail(GQA_E_INVALID, "max_positions %d outside [1, %d]", max_positions, m->d.max_positions);
  int nb = (max_positions + kBlock - 1) / kBlock;
  std::lock_guard<std::mutex> lk(m->mu);
  std::vector<int32_t> blocks(nb);
  KvPool& pool = *m->pool;
  if (block_ids) {
    std::vector<char> seen(m->d.kv_pool_blocks, 0);
    for (int i = 0; i < nb; ++i) {
      int b = block_ids[i];
      if (b < 0 || b >= m->d.kv_pool_blocks) return fail(GQA_E_INVALID, "block id %d outside the pool", b);
      if (seen[b]) return fail(GQA_E_INVALID, "block id %d repeated", b);
      if (pool.state(b) == KvPool::PRIVATE || pool.refs(b) > 0)
        return fail(GQA_E_INVALID, "block id %d already owned by a session", b);
      seen[b] = 1;
      blocks[i] = b;
    }
    for (int b : blocks) pool.take(b);
  } else {
    if (pool.available() < nb) return fail(GQA_E_OOM, "KV pool has %d free blocks, %d needed", pool.available(), nb);
    for (int i = 0; i < nb; ++i) blocks[i] = pool.take_any();
  }
  gqa_session* s = new gqa_session();
  s->m = m;
  s->max_pos = max_positions;
  s->blocks = blocks;
  void* v = nullptr;
  hipError_t e = hipMalloc(&v, sizeof(int32_t) * nb);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete s;
    return fail(GQA_E_OOM, "block table allocation failed");
  }
  s->d_table = (int32_t*)v;
  e = hipMemcpy(s->d_table, blocks.data(), sizeof(int32_t) * nb, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(v);
    for (int b : blocks) pool.unref(b);
    delete s;
    return fail(GQA_E_HIP, "block table upload failed: %s", hipGetErrorString(e));
  }
  m->sessions++;
  *out = s;
  return GQA_OK;
}

void gqa_session_destroy(gqa_session* s) {
  if (!s) return;
  gqa_model* m = s->m;
  (void)hipDeviceSynchronize();
  {
    std::lock_guard<std::mutex> lk(m->mu);
    if (s->seq) s->seq->finish(s->pos);   // publish at finish
    for (int b : s->blocks) m->pool->unref(b);
    m->sessions--;
  }
  (void)hipFree(s->d_table);
  delete s;
}

int gqa_session_create_pooled(gqa_model* m, int32_t max_positions, gqa_session** out) {
  g_err.clear();
  if (!m || !out) return fail(GQA_E_INVALID, "null argument");
  if (max_positions < 1 || max_positions > m->d.max_positions)
    return fail(GQA_E_INVALID, "max_positions %d outside [1, %d]", max_positions, m->d.max_positions);
  const int nb = (max_positions + kBlock - 1) / kBlock;
  void* v = nullptr;
  hipError_t e = hipMalloc(&v, sizeof(int32_t) * nb);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(GQA_E_OOM, "block table allocation failed");
  }
  // unmapped entries point at block 0: never read below the session's position, and a valid
  // address if a kernel's rounding ever reads one
  e = hipMemset(v, 0, sizeof(int32_t) * nb);
  if (e != hipSuccess) {
    (void)hipFree(v);
    return fail(GQA_E_HIP, "block table initialisation failed: %s", hipGetErrorString(e));
  }
  gqa_session* s = new gqa_session();
  s->m = m;
  s->max_pos = max_positions;
  s->d_table = (int32_t*)v;
  std::lock_guard<std::mutex> lk(m->mu);
  s->seq.reset(new PooledSeq(*m->pool, max_positions));
  m->sessions++;
  *out = s;
  return GQA_OK;
}

int gqa_session_reset(gqa_session* s) {
  if (!s) return fail(GQA_E_INVALID, "null session");
  if (s->seq) {
    std::lock_guard<std::mutex> lk(s->m->mu);
    s->seq->finish(s->pos);
  }
  s->pos = 0;
  s->reused = 0;
  return GQA_OK;
}

int gqa_session_publish(gqa_session* s) {
  g_err.clear();
  if (!s) return fail(GQA_E_INVALID, "null session");
  if (!s->seq) return fail(GQA_E_INVALID, "not a pooled session");
  std::lock_guard<std::mutex> lk(s->m->mu);
  s->seq->publish(s->pos);
  return GQA_OK;
}

int32_t gqa_session_reused(const gqa_session* s) { return s ? s->reused : -1; }

int32_t gqa_session_position(const gqa_session* s) { return s ? s->pos : -1; }

}  // extern "C"

namespace {

// Stage host ids into pinned memory and copy them to the device on `st`. The staging buffer is
// reused, so wait for the previous copy first.
int upload_ids(gqa_model* m, const int32_t* ids, int n, hipStream_t st) {
  HIP_TRY(hipEventSynchronize(m->ids_evt));
  memcpy(m->ids_host, ids, sizeof(int32_t) * n);
  HIP_TRY(hipMemcpyAsync(m->ids_dev, m->ids_host, sizeof(int32_t) * n, hipMemcpyHostToDevice, st));
  HIP_TRY(hipEventRecord(m->ids_evt, st));
  return GQA_OK;
}

// Apply a pooled session's block changes on `st` before its evaluation: whole-block K/V copies
// (copy on write) in every layer, then the table entries.
int apply_pool_changes(gqa_session* s, const std::vector<TableWrite>& tw, const std::vector<BlockCopy>& cp,
                       hipStream_t st) {
  gqa_model* m = s->m;
  const size_t blk = (size_t)kKvHeads * kBlock * kHeadDim;
  for (const BlockCopy& c : cp)
    for (const LayerW& w : m->L) {
      if (w.kq8.kq) {
        HIP_TRY(hipMemcpyAsync(w.kq8.kq + c.dst * blk, w.kq8.kq + c.src * blk, blk, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(w.kq8.vq + c.dst * blk, w.kq8.vq + c.src * blk, blk, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(w.kq8.ks + c.dst * blk / 32, w.kq8.ks + c.src * blk / 32, blk / 32 * 2,
                               hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(w.kq8.vs + c.dst * blk / 32, w.kq8.vs + c.src * blk / 32, blk / 32 * 2,
                               hipMemcpyDeviceToDevice, st));
      } else {
        HIP_TRY(hipMemcpyAsync(w.kpool + c.dst * blk, w.kpool + c.src * blk, blk * 2, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(w.vpool + c.dst * blk, w.vpool + c.src * blk, blk * 2, hipMemcpyDeviceToDevice, st));
      }
    }
  for (size_t i = 0; i < tw.size(); i += kTableWritesMax) {
    TableWrites t{};
    t.n = (int)std::min(tw.size() - i, (size_t)kTableWritesMax);
    for (int k = 0; k < t.n; ++k) {
      t.idx[k] = tw[i + k].idx;
      t.val[k] = tw[i + k].val;
    }
    HIP_TRY(launch_table_writes(s->d_table, t, st));
  }
  return GQA_OK;
}

// Map and make private the blocks a pooled session writes for positions [p0, p1), recording
// the ids (nullptr: not known on the host). GQA_E_OOM, with nothing changed, if the pool is
// exhausted. No-op for sessions with a fixed table.
int prepare_write(gqa_session* s, int p0, int p1, const int32_t* ids, hipStream_t st) {
  if (!s->seq) return GQA_OK;
  std::vector<TableWrite> tw;
  std::vector<BlockCopy> cp;
  {
    std::lock_guard<std::mutex> lk(s->m->mu);
    if (!s->seq->prepare_write(p0, p1, tw, cp))
      return fail(GQA_E_OOM, "KV pool exhausted: no block free or evictable for positions [%d, %d)", p0, p1);
    s->seq->record(p0, ids, p1 - p0);
  }
  return apply_pool_changes(s, tw, cp, st);
}

constexpr int64_t kProfMax = 65536;

// Time the next launch of kernel class `cls` when that class is being recorded: the launch
// stamps a start/stop event pair from its own dispatch (GQA_LAUNCH). A pair that no launch
// consumed (a failed launch, or a kernel started another way) is not counted.
struct ProfScope {
  gqa_model* m;
  hipStream_t st;
  bool armed = false;
  ProfScope(gqa_model* m_, int cls, hipStream_t st_) : m(m_), st(st_) {
    if (m->prof_cls != cls) return;
    if (m->prof_used >= kProfMax) {
      m->prof_dropped++;
      return;
    }
    while ((int64_t)m->prof_ev.size() < 2 * (m->prof_used + 1)) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return;
      m->prof_ev.push_back(e);
    }
    g_launch_events.start = m->prof_ev[2 * m->prof_used];
    g_launch_events.stop = m->prof_ev[2 * m->prof_used + 1];
    m->prof_used++;
    armed = true;
  }
  ~ProfScope() {
    if (armed && g_launch_events.start) m->prof_used--;
    g_launch_events = LaunchEvents{};
  }
};

#define LAUNCH(expr)                                                                                   \
  do {                                                                                                 \
    hipError_t e_ = (expr);                                                                            \
    if (e_ != hipSuccess) return fail(GQA_E_HIP, "launch failed at %s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)


// Decode / batched decode over B rows; ids already on the device. Per layer: q|k|v matvec (its
// prologue adds the previous down projection to the residual stream and multiplies by the
// norm weight), fused attention (1/rms scale, q/k norm, RoPE, KV write, attention, chunk
// merge), o matvec, gate|up matvec (prologue: residual add of the o projection times the norm
// weight), down matvec (prologue: 1/rms scale and SwiGLU). The residual stream alternates
// between two buffers so a prologue can write the updated stream while other workgroups still
// read the previous one. With B > 4 the prologue work runs in rows_kernel with the same
// arithmetic.
int run_decode(gqa_model* m, const DecodeScratch& sc, const Rows& rows, int B, int max_ctx, const int32_t* ids_dev,
               float* logits, int32_t* argmax, hipStream_t st) {
  const gqa_model_desc& d = m->d;
  const int H = d.hidden, F = d.ffn, V = d.vocab, NQ = d.n_q_heads, QD = m->QD, QKV = m->QKV;
  const float eps = d.rms_eps;
  // the decode attention reads the BF16 cache, or a Q8_0 cache's codes and scales directly (w.kq8)
  auto kv_k = [](const LayerW& w) { return w.kpool; };
  auto kv_v = [](const LayerW& w) { return w.vpool; };
  const bool fused = B <= 4;
  const int64_t pstride = sc.pstride;
  float* xa = sc.x;
  float* xb = sc.x2;
  float* P0 = sc.part;
  float* P1 = sc.part2;
  float* ss_qkv = sc.ss;
  float* ss_gu = sc.ss + 8 * 32;
  LAUNCH(launch_embed(m->embed, ids_dev, B, H, V, xa, m->err, st, sc.zero, sc.nzero));

  auto resid_src = [&](float* res, float* res_out, const float* part, int nsplit, float pscale, const uint16_t* w,
                       float* ss_out) {
    XSrc x{};
    x.mode = X_RESID;
    x.res = res;
    x.res_out = res_out;
    x.part = part;
    x.nsplit = part ? nsplit : 0;
    x.pstride = pstride;
    x.pld = H;
    x.pscale = pscale;
    x.w = w;
    x.ss_out = ss_out;
    x.H = H;
    x.eps = eps;
    return x;
  };
  auto raw_src = [&](const f16* hi, const f16* lo, int ld) {
    XSrc x{};
    x.mode = X_RAW;
    x.hi = hi;
    x.lo = lo;
    x.ld = ld;
    return x;
  };
  // matvec over an operand built by a prologue: in LDS (B <= 4) or by rows_kernel first
  auto gemv_built = [&](const uint16_t* W, const int8_t* Wq, const f16* Wd, const f16* Wb, int K, int N, const XSrc& xs,
                        int nsplit, float* P, int ldp, f16* hi, f16* lo) -> hipError_t {
    if (fused) return launch_gemv(W, Wq, Wd, Wb, K, N, xs, B, nsplit, P, pstride, ldp, nullptr, st);
    hipError_t e = launch_rows(xs, K, nsplit, B, hi, lo, K, st);
    if (e != hipSuccess) return e;
    return launch_gemv(W, Wq, Wd, Wb, K, N, raw_src(hi, lo, K), B, nsplit, P, pstride, ldp, nullptr, st);
  };

  // Whole-K path (few rows): the residual stream xa is final after every projection, no split
  // partials; bit-identical per row to the split-K path below.
  if (gemv_full_fits(std::max(std::max(H, QD), F), B)) {
    auto fa = [&]() {
      FullArgs a{};
      a.B = B;
      a.eps = eps;
      return a;
    };
    // The layers' launches form one chain (any-order launches that order themselves through
    // arrival counters, cleared by the embedding launch above); the final norm after it is an
    // ordinary launch, which the queue holds until every launch before it has finished. While
    // the decode gate/up matvec is being timed the chain is off: a chained launch starts before
    // its predecessor ends and waits, so its events would not bracket its own execution.
    ChainTrack ct;
    if (kDecodeChain && m->prof_cls != GQA_PROF_DECODE_GATEUP) {
      ct.cnt = sc.chain;
      ct.err = m->err;
      ct.offset = m->chain_offset;
    }
    int nwg = 0;
    for (int l = 0; l < d.n_layers; ++l) {
      const LayerW& w = m->L[l];
      FullArgs q = fa();
      q.W = w.wqkv; q.Wq = w.qqkv; q.Wd = w.sqkv; q.Wb = w.bqkv; q.K = H; q.N = QKV;
      q.xres = xa; q.nw = w.attn_norm; q.ss_out = ss_qkv; q.y = P0; q.ldy = QKV;
      q.chain = ct.next();
      LAUNCH(launch_gemv_full(XF_NORM, EPI_STORE, m->s_qkv, q, st, &nwg));
      ct.launched(nwg);
      LAUNCH(launch_attn_decode(P0, 1, pstride, QKV, NQ, ss_qkv, m->s_qkv, H, w.q_norm, w.k_norm, eps, m->rcos,
                                m->rsin, rows, B, max_ctx, kv_k(w), kv_v(w), w.kq8, sc.apart, sc.counters, kAttnOutScale,
                                sc.oh, sc.ol, QD, st, ct.next(), &nwg));
      ct.launched(nwg);
      FullArgs o = fa();
      o.W = w.wo; o.Wq = w.qo; o.Wd = w.so; o.Wb = w.bo; o.K = QD; o.N = H;
      o.xhi = sc.oh; o.xlo = sc.ol; o.ldx = QD; o.y = xa; o.ldy = H; o.yscale = 1.f / kAttnOutScale;
      o.chain = ct.next();
      LAUNCH(launch_gemv_full(XF_RAW, EPI_ADD, m->s_o, o, st, &nwg));
      ct.launched(nwg);
      FullArgs g = fa();
      g.W = w.wgu; g.Wq = w.qgu; g.Wd = w.sgu; g.Wb = w.bgu; g.K = H; g.N = 2 * F;
      g.xres = xa; g.nw = w.ffn_norm; g.ss_out = ss_gu; g.mhi = sc.mh; g.mlo = sc.ml; g.ldm = F;
      g.chain = ct.next();
      {
        ProfScope ps(m, GQA_PROF_DECODE_GATEUP, st);
        LAUNCH(launch_gemv_full(XF_NORM, EPI_SWIGLU, m->s_gu, g, st, &nwg));
      }
      ct.launched(nwg);
      FullArgs dn = fa();
      dn.W = w.wd; dn.Wq = w.qd; dn.Wd = w.sd; dn.Wb = w.bd; dn.K = F; dn.N = H;
      dn.xhi = sc.mh; dn.xlo = sc.ml; dn.ldx = F; dn.y = xa; dn.ldy = H; dn.yscale = 1.f;
      dn.chain = ct.next();
      LAUNCH(launch_gemv_full(XF_RAW, EPI_ADD, m->s_d, dn, st, &nwg));
      ct.launched(nwg);
    }
    LAUNCH(launch_final_norm(resid_src(xa, nullptr, nullptr, 0, 1.f, m->final_norm, nullptr), B, sc.xh, sc.xl, H,
                             st));
    FullArgs lm = fa();
    lm.W = m->lm_head; lm.K = H; lm.N = V; lm.xhi = sc.xh; lm.xlo = sc.xl; lm.ldx = H; lm.y = logits; lm.ldy = V;
    lm.cand = argmax ? sc.cand : nullptr;
    {
      ProfScope ps(m, GQA_PROF_DECODE_LMHEAD, st);
      LAUNCH(launch_gemv_full(XF_RAW, EPI_STORE, 1, lm, st));
    }
    if (argmax) LAUNCH(launch_argmax(sc.cand, V / 16, B, argmax, st));
    return GQA_OK;
  }

  const float* prev = nullptr;
  int prev_split = 0;
  for (int l = 0; l < d.n_layers; ++l) {
    const LayerW& w = m->L[l];
    LAUNCH(gemv_built(w.wqkv, w.qqkv, w.sqkv, w.bqkv, H, QKV, resid_src(xa, xb, prev, prev_split, 1.f, w.attn_norm, ss_qkv),
                      m->s_qkv, P0, QKV, sc.xh, sc.xl));
    std::swap(xa, xb);
    LAUNCH(launch_attn_decode(P0, m->s_qkv, pstride, QKV, NQ, ss_qkv, m->s_qkv, H, w.q_norm, w.k_norm, eps, m->rcos,
                              m->rsin, rows, B, max_ctx, kv_k(w), kv_v(w), w.kq8, sc.apart, sc.counters, kAttnOutScale,
                              sc.oh, sc.ol, QD, st));
    LAUNCH(launch_gemv(w.wo, w.qo, w.so, w.bo, QD, H, raw_src(sc.oh, sc.ol, QD), B, m->s_o, P1, pstride, H, nullptr,
                       st));
    {
      ProfScope ps(m, GQA_PROF_DECODE_GATEUP, st);
      LAUNCH(gemv_built(w.wgu, w.qgu, w.sgu, w.bgu, H, 2 * F,
                        resid_src(xa, xb, P1, m->s_o, 1.f / kAttnOutScale, w.ffn_norm, ss_gu), m->s_gu, P0, 2 * F,
                        sc.xh, sc.xl));
    }
    std::swap(xa, xb);
    XSrc sw{};
    sw.mode = X_SWIGLU;
    sw.gu = P0;
    sw.gu_split = m->s_gu;
    sw.gu_stride = pstride;
    sw.gu_ld = 2 * F;
    sw.ss = ss_gu;
    sw.ss_n = m->s_gu;
    sw.H = H;
    sw.eps = eps;
    LAUNCH(gemv_built(w.wd, w.qd, w.sd, w.bd, F, H, sw, m->s_d, P1, H, sc.mh, sc.ml));
    prev = P1;
    prev_split = m->s_d;
  }
  LAUNCH(launch_final_norm(resid_src(xa, nullptr, prev, prev_split, 1.f, m->final_norm, nullptr), B, sc.xh, sc.xl, H,
                           st));
  {
    ProfScope ps(m, GQA_PROF_DECODE_LMHEAD, st);
    LAUNCH(launch_gemv(m->lm_head, nullptr, nullptr, nullptr, H, V, raw_src(sc.xh, sc.xl, H), B, 1, logits, pstride, V,
                       argmax ? sc.cand : nullptr, st));
  }
  if (argmax) LAUNCH(launch_argmax(sc.cand, V / 16, B, argmax, st));
  return GQA_OK;
}

// K ranges of a prefill projection onto the residual stream (N = hidden outputs over T rows):
// about two workgroups per CU when the output tiles alone are too few, at most 8 ranges, at
// least 4 K-steps per range, and at most 4 R rows of partials.
int prefill_ksplit(const gqa_model* m, int N, int K, int T) {
  const int tiles = (N / 256) * ((T + 127) / 128);
  const int want = (2 * m->cu + tiles / 2) / tiles;
  return std::max(1, std::min({want, 8, 4 * m->R / T, K / 32 / 4}));
}

constexpr int kProfNever = -1;   // a ProfScope class no recording selects

// Prefill rounds over n ids already in device memory (ids_dev); see gqa_session_eval_prefill.
// Per layer: q|k|v GEMM, q/k norm + RoPE + KV write, attention, o GEMM (K-range partials),
// residual add of the partials + RMSNorm, gate|up GEMM with SwiGLU, down GEMM (partials), and
// the next layer's residual add + RMSNorm. Rounds of at most 32 rows run the projections as
// matvecs (gate|up then a SwiGLU pass over its partials). The logits need only the last row of the last layer:
// after writing that layer's K/V, its attention, o and MLP run for the last row alone (and are
// skipped in rounds before the last).
// What a prefill call returns: the last row's logits (and argmax), every row's, or the
// log-probability of each next token.
enum PrefillOut { kOutLast = 0, kOutAll = 1, kOutScores = 2 };

int run_prefill(gqa_session* s, const int32_t* ids_dev, int n, int out, float* logits, int32_t* argmax,
                float* scores, hipStream_t st) {
  gqa_model* m = s->m;
  const gqa_model_desc& d = m->d;
  const int H = d.hidden, F = d.ffn, V = d.vocab, NQ = d.n_q_heads, QD = m->QD, QKV = m->QKV;
  const float eps = d.rms_eps;
  Rows none{};
  // a Q8_0 cache has no BF16 pools: K/V are written and read as codes and scales (w.kq8)
  auto kv_k = [](const LayerW& w) { return w.kpool; };
  auto kv_v = [](const LayerW& w) { return w.vpool; };
  const bool split = d.prefill_operands == GQA_PREFILL_SPLIT;
  // the GEMM reads Q8_0 quants directly if so configured; otherwise every scheme uses the FP16
  // prefill copies
  auto gq = [&](const int8_t* q) { return d.scheme == GQA_SCHEME_Q8_0 && d.prefill_q8_direct ? q : nullptr; };
  // Projection of `rows` operand rows (FP16 hi/lo, row stride ldx) for a round of at most 32
  // rows: the LDS-staged matvec over the decode weights with the decode K ranges, partials
  // P[range][row][N] (range stride rows * N) summed in range order by the consumer. A 128-row
  // GEMM tile would leave most of the chip idle and stream each weight tile on few CUs.
  auto matvec = [&](const uint16_t* W, const int8_t* Wq, const f16* Wd, const f16* Wb, int K, int N, const f16* xh,
                    const f16* xl, int ldx, int rows, int nsplit, float* P) -> int {
    XSrc raw{};
    raw.mode = X_RAW;
    raw.hi = xh;
    raw.lo = xl;
    raw.ld = ldx;
    LAUNCH(launch_gemv(W, Wq, Wd, Wb, K, N, raw, rows, nsplit, P, (int64_t)rows * N, N, nullptr, st, true));
    return GQA_OK;
  };
  for (int off = 0; off < n; off += m->R) {
    const int T = std::min(m->R, n - off);
    const int pos0 = s->pos + off;
    const bool final_round = off + T == n;
    const bool mv = T <= kMaxBatch;   // matvec projections for this round
    LAUNCH(launch_embed(m->embed, ids_dev + off, T, H, d.vocab, m->x, m->err, st));
    LAUNCH(launch_rmsnorm(m->x, H, nullptr, 0, 0, 0, 1.f, m->L[0].attn_norm, H, eps, 1.f, m->xh, m->xl, H, T, st));
    for (int l = 0; l < d.n_layers; ++l) {
      const LayerW& w = m->L[l];
      const bool last = l + 1 == d.n_layers;
      if (mv) {
        int rc = matvec(w.wqkv, w.qqkv, w.sqkv, w.bqkv, H, QKV, m->xh, m->xl, H, T, m->s_qkv, m->part);
        if (rc) return rc;
        LAUNCH(launch_qk_rope_kv(false, m->part, m->s_qkv, T * QKV, QKV, NQ, w.q_norm, w.k_norm, eps, m->rcos,
                                 m->rsin, pos0, s->d_table, none, kv_k(w), kv_v(w), w.kq8, m->q, T, st));
      } else {
        LAUNCH(launch_gemm(EPI_STORE, split, w.pqkv, gq(w.qqkv), w.sqkv, H, QKV, m->xh, m->xl, H, T, m->qkv, QKV, 1.f,
                           nullptr, nullptr, 0, 1.f, 1, 0, st));
        LAUNCH(launch_qk_rope_kv(false, m->qkv, 0, 0, QKV, NQ, w.q_norm, w.k_norm, eps, m->rcos, m->rsin, pos0,
                                 s->d_table, none, kv_k(w), kv_v(w), w.kq8, m->q, T, st));
      }
      const bool one = last && out == kOutLast;                // only the final row feeds the logits
      if (one && !final_round) break;
      const int rows = one ? 1 : T, r0 = one ? T - 1 : 0;
      {
        ProfScope ps(m, last ? kProfNever : GQA_PROF_PREFILL_ATTN, st);
        LAUNCH(launch_attn_prefill(m->q + (int64_t)r0 * QD, NQ, rows, pos0 + r0, s->d_table, kv_k(w), kv_v(w), w.kq8,
                                   kAttnOutScale, m->oh, m->ol, QD, m->apart, st));
      }
      float* pp = mv ? m->part2 : m->ppart;     // o and down partials
      int so = 0, sd = 0;
      if (mv) {
        so = m->s_o;
        int rc = matvec(w.wo, w.qo, w.so, w.bo, QD, H, m->oh, m->ol, QD, rows, so, pp);
        if (rc) return rc;
      } else {
        so = prefill_ksplit(m, H, QD, rows);
        LAUNCH(launch_gemm(EPI_STORE, split, w.po, gq(w.qo), w.so, QD, H, m->oh, m->ol, QD, rows, pp, H, 1.f, nullptr,
                           nullptr, 0, 1.f, so, (int64_t)rows * H, st));
      }
      LAUNCH(launch_rmsnorm(m->x + (int64_t)r0 * H, H, pp, so, rows * H, H, 1.f / kAttnOutScale, w.ffn_norm, H, eps,
                            1.f, m->xh, m->xl, H, rows, st));
      if (mv) {
        int rc = matvec(w.wgu, w.qgu, w.sgu, w.bgu, H, 2 * F, m->xh, m->xl, H, rows, m->s_gu, m->part);
        if (rc) return rc;
        LAUNCH(launch_swiglu_rows(m->part, m->s_gu, (int64_t)rows * 2 * F, 2 * F, F, rows, m->mh, m->ml, F, st));
        sd = m->s_d;
        rc = matvec(w.wd, w.qd, w.sd, w.bd, F, H, m->mh, m->ml, F, rows, sd, pp);
        if (rc) return rc;
      } else {
        {
          ProfScope ps(m, last ? kProfNever : GQA_PROF_PREFILL_GATEUP, st);
          LAUNCH(launch_gemm(EPI_SWIGLU, split, w.pgu, gq(w.qgu), w.sgu, H, 2 * F, m->xh, m->xl, H, rows, nullptr, 0, 1.f,
                             m->mh, m->ml, F, 1.f, 1, 0, st));
        }
        sd = prefill_ksplit(m, H, F, rows);
        LAUNCH(launch_gemm(EPI_STORE, split, w.pd, gq(w.qd), w.sd, F, H, m->mh, m->ml, F, rows, pp, H, 1.f, nullptr,
                           nullptr, 0, 1.f, sd, (int64_t)rows * H, st));
      }
      const uint16_t* next_norm = last ? m->final_norm : m->L[l + 1].attn_norm;
      LAUNCH(launch_rmsnorm(m->x + (int64_t)r0 * H, H, pp, sd, rows * H, H, 1.f, next_norm, H, eps, 1.f, m->xh, m->xl,
                            H, rows, st));
      if (last && out != kOutLast && !mv) {
        // lm_head over every row of a GEMM round: one GEMM over the padded FP16 copy (only the
        // vocab's columns stored); scores go through the logits scratch kScoreRows rows at a time
        if (out == kOutAll) {
          ProfScope ps(m, GQA_PROF_ROWS_LMHEAD, st);
          LAUNCH(launch_gemm(EPI_STORE, split, m->plm, nullptr, nullptr, H, m->Vpad, m->xh, m->xl, H, rows,
                             logits + (int64_t)off * V, V, 1.f, nullptr, nullptr, 0, 1.f, 1, 0, st, V));
          if (argmax) LAUNCH(launch_argmax_rows(logits + (int64_t)off * V, V, V, rows, argmax + off, st));
        } else {
          for (int c0 = 0; c0 < rows; c0 += kScoreRows) {
            const int i0 = off + c0, Bc = std::min(std::min(kScoreRows, rows - c0), n - 1 - i0);
            if (Bc < 1) break;
            {
              ProfScope ps(m, GQA_PROF_ROWS_LMHEAD, st);
              LAUNCH(launch_gemm(EPI_STORE, split, m->plm, nullptr, nullptr, H, m->Vpad, m->xh + (int64_t)c0 * H,
                                 m->xl + (int64_t)c0 * H, H, Bc, m->slog, V, 1.f, nullptr, nullptr, 0, 1.f, 1, 0, st,
                                 V));
            }
            LAUNCH(launch_score(m->slog, V, ids_dev + i0 + 1, Bc, scores + i0, st));
          }
        }
      } else if (last) {
        // lm_head over the rows, up to 32 at a time (the batched decode matvec)
        for (int g0 = 0; g0 < rows; g0 += kMaxBatch) {
          const int i0 = off + r0 + g0;                       // call-relative index of the group's first row
          int Bg = std::min(kMaxBatch, rows - g0);
          if (out == kOutScores) Bg = std::min(Bg, n - 1 - i0);   // rows with a next token
          if (Bg < 1) break;
          XSrc raw{};
          raw.mode = X_RAW;
          raw.hi = m->xh + (int64_t)g0 * H;
          raw.lo = m->xl + (int64_t)g0 * H;
          raw.ld = H;
          ProfScope ps(m, out == kOutLast ? kProfNever : GQA_PROF_ROWS_LMHEAD, st);
          if (out == kOutScores) {
            LAUNCH(launch_gemv(m->lm_head, nullptr, nullptr, nullptr, H, V, raw, Bg, 1, m->slog, 0, V, nullptr, st));
            LAUNCH(launch_score(m->slog, V, ids_dev + i0 + 1, Bg, scores + i0, st));
          } else {
            float* dst = logits + (int64_t)(out == kOutAll ? i0 : 0) * V;
            LAUNCH(launch_gemv(m->lm_head, nullptr, nullptr, nullptr, H, V, raw, Bg, 1, dst, 0, V,
                               argmax ? m->cand : nullptr,
                               st));
            if (argmax) LAUNCH(launch_argmax(m->cand, V / 16, Bg, argmax + (out == kOutAll ? i0 : 0), st));
          }
        }
      }
    }
  }
  s->pos += n;
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_session_eval_prefill(gqa_session* s, const int32_t* ids, int32_t n, float* logits, int32_t* argmax,
                             hipStream_t st) {
  g_err.clear();
  if (!s || !ids || !logits) return fail(GQA_E_INVALID, "null argument");
  gqa_model* m = s->m;
  const gqa_model_desc& d = m->d;
  if (n < 1) return fail(GQA_E_INVALID, "n must be >= 1");
  if ((int64_t)s->pos + n > s->max_pos)
    return fail(GQA_E_RANGE, "context overflow: %d + %d > %d", s->pos, n, s->max_pos);
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= d.vocab) return fail(GQA_E_RANGE, "token id %d at %d outside [0, %d)", ids[i], i, d.vocab);
  // a pooled session at position 0 first maps the cached blocks of its prompt's leading whole
  // blocks and evaluates only the rest
  int reuse = 0;
  if (s->seq && s->pos == 0) {
    std::vector<TableWrite> tw;
    {
      std::lock_guard<std::mutex> lk(m->mu);
      reuse = s->seq->map_prefix(ids, n, tw);
    }
    int rc = apply_pool_changes(s, tw, {}, st);
    if (rc) return rc;
    s->pos = reuse;
  }
  s->reused = reuse;
  int rc = prepare_write(s, s->pos, s->pos + n - reuse, ids + reuse, st);
  if (rc) {
    if (reuse) {
      std::lock_guard<std::mutex> lk(m->mu);
      s->seq->release();
      s->pos = 0;
      s->reused = 0;
    }
    return rc;
  }
  rc = upload_ids(m, ids, n, st);
  if (rc) return rc;
  return run_prefill(s, m->ids_dev + reuse, n - reuse, kOutLast, logits, argmax, nullptr, st);
}

int gqa_session_eval_prefill_device(gqa_session* s, const int32_t* ids_dev, int32_t n, float* logits,
                                    int32_t* argmax, hipStream_t st) {
  g_err.clear();
  if (!s || !ids_dev || !logits) return fail(GQA_E_INVALID, "null argument");
  if (n < 1) return fail(GQA_E_INVALID, "n must be >= 1");
  if ((int64_t)s->pos + n > s->max_pos)
    return fail(GQA_E_RANGE, "context overflow: %d + %d > %d", s->pos, n, s->max_pos);
  int rc = prepare_write(s, s->pos, s->pos + n, nullptr, st);
  if (rc) return rc;
  return run_prefill(s, ids_dev, n, kOutLast, logits, argmax, nullptr, st);
}

int gqa_session_eval_n(gqa_session* s, const int32_t* ids, int32_t n, float* logits, int32_t* argmax, hipStream_t st) {
  g_err.clear();
  if (!s || !ids || !logits) return fail(GQA_E_INVALID, "null argument");
  if (n < 1) return fail(GQA_E_INVALID, "n must be >= 1");
  if ((int64_t)s->pos + n > s->max_pos)
    return fail(GQA_E_RANGE, "context overflow: %d + %d > %d", s->pos, n, s->max_pos);
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= s->m->d.vocab)
      return fail(GQA_E_RANGE, "token id %d at %d outside [0, %d)", ids[i], i, s->m->d.vocab);
  int rc = prepare_write(s, s->pos, s->pos + n, ids, st);
  if (rc) return rc;
  rc = upload_ids(s->m, ids, n, st);
  if (rc) return rc;
  return run_prefill(s, s->m->ids_dev, n, kOutAll, logits, argmax, nullptr, st);
}

int gqa_session_eval_scored(gqa_session* s, const int32_t* ids, int32_t n, float* scores, hipStream_t st) {
  g_err.clear();
  if (!s || !ids || !scores) return fail(GQA_E_INVALID, "null argument");
  if (n < 2) return fail(GQA_E_INVALID, "n must be >= 2 (a token to score needs the one before it)");
  if ((int64_t)s->pos + n > s->max_pos)
    return fail(GQA_E_RANGE, "context overflow: %d + %d > %d", s->pos, n, s->max_pos);
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= s->m->d.vocab)
      return fail(GQA_E_RANGE, "token id %d at %d outside [0, %d)", ids[i], i, s->m->d.vocab);
  int rc = prepare_write(s, s->pos, s->pos + n, ids, st);
  if (rc) return rc;
  rc = upload_ids(s->m, ids, n, st);
  if (rc) return rc;
  return run_prefill(s, s->m->ids_dev, n, kOutScores, nullptr, nullptr, scores, st);
}

int gqa_session_truncate(gqa_session* s, int32_t pos) {
  g_err.clear();
  if (!s) return fail(GQA_E_INVALID, "null session");
  if (pos < 0 || pos > s->pos) return fail(GQA_E_RANGE, "position %d outside [0, %d]", pos, s->pos);
  s->pos = pos;
  return GQA_OK;
}

int gqa_session_eval_batch(gqa_session* const* ss, int32_t B, const int32_t* ids, int32_t ids_on_device,
                           float* logits, int32_t* argmax, hipStream_t st) {
  g_err.clear();
  return eval_rows(ss, B, ids, ids_on_device, logits, argmax, nullptr, st);
}

int gqa_session_eval_decode_static(gqa_session* s, const int32_t* id, int32_t id_on_device, float* logits,
                                   int32_t* argmax, hipStream_t st) {
  g_err.clear();
  if (!s || !id || !logits) return fail(GQA_E_INVALID, "null argument");
  gqa_model* m = s->m;
  const gqa_model_desc& d = m->d;
  if (!gemv_full_fits(std::max(std::max(d.hidden, m->QD), d.ffn), 1))
    return fail(GQA_E_INVALID, "the static-scratch decode needs the whole-K matvec path (hidden, attention width and "
                               "ffn <= %d)", 16380);
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != m->dev) return fail(GQA_E_INVALID, "current device %d is not the model's device %d", dev, m->dev);
  DecodeScratch sc;
  const size_t need = carve_static_scratch(m, nullptr, &sc);
  if (need > kStaticScratchBytes)
    return fail(GQA_E_INVALID, "this model's decode needs %zu bytes of scratch; the static scratch holds %zu", need,
                kStaticScratchBytes);
  void* base = nullptr;
  int rc = static_scratch_base(dev, &base);
  if (rc) return rc;
  carve_static_scratch(m, base, &sc);
  return eval_rows(&s, 1, id, id_on_device, logits, argmax, &sc, st);
}

}  // extern "C"

namespace {

// Rows of one batched (or single) decode: checks, id upload, KV block mapping, then run_decode
// over the model's scratch or the given one.
int eval_rows(gqa_session* const* ss, int32_t B, const int32_t* ids, int32_t ids_on_device, float* logits,
              int32_t* argmax, const DecodeScratch* scr, hipStream_t st) {
  if (!ss || !ids || !logits) return fail(GQA_E_INVALID, "null argument");
  if (B < 1 || B > kMaxBatch) return fail(GQA_E_INVALID, "B = %d outside [1, %d]", B, kMaxBatch);
  gqa_model* m = ss[0] ? ss[0]->m : nullptr;
  if (!m) return fail(GQA_E_INVALID, "null session");
  Rows rows{};
  int max_ctx = 0;
  for (int b = 0; b < B; ++b) {
    if (!ss[b]) return fail(GQA_E_INVALID, "null session at %d", b);
    if (ss[b]->m != m) return fail(GQA_E_INVALID, "sessions of different models");
    for (int c = 0; c < b; ++c)
      if (ss[c] == ss[b]) return fail(GQA_E_INVALID, "session repeated at rows %d and %d", c, b);
    if (ss[b]->pos + 1 > ss[b]->max_pos) return fail(GQA_E_RANGE, "context overflow in row %d", b);
    rows.pos[b] = ss[b]->pos;
    rows.table[b] = ss[b]->d_table;
    max_ctx = std::max(max_ctx, ss[b]->pos + 1);
  }
  const int32_t* ids_dev = ids;
  if (!ids_on_device) {
    for (int b = 0; b < B; ++b)
      if (ids[b] < 0 || ids[b] >= m->d.vocab)
        return fail(GQA_E_RANGE, "token id %d in row %d outside [0, %d)", ids[b], b, m->d.vocab);
    int rc = upload_ids(m, ids, B, st);
    if (rc) return rc;
    ids_dev = m->ids_dev;
  }
  for (int b = 0; b < B; ++b) {
    int rc = prepare_write(ss[b], ss[b]->pos, ss[b]->pos + 1, ids_on_device ? nullptr : ids + b, st);
    if (rc) return rc;
  }
  int rc = run_decode(m, scr ? *scr : model_scratch(m), rows, B, max_ctx, ids_dev, logits, argmax, st);
  if (rc) return rc;
  for (int b = 0; b < B; ++b) ss[b]->pos++;
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_session_eval_decode(gqa_session* s, const int32_t* id, int32_t id_on_device, float* logits, int32_t* argmax,
                            hipStream_t st) {
  return gqa_session_eval_batch(&s, 1, id, id_on_device, logits, argmax, st);
}

int gqa_model_profile(gqa_model* m, int32_t cls) {
  if (!m) return fail(GQA_E_INVALID, "null model");
  if (cls < GQA_PROF_NONE || cls > GQA_PROF_ROWS_LMHEAD) return fail(GQA_E_INVALID, "unknown kernel class %d", cls);
  HIP_TRY(hipDeviceSynchronize());
  m->prof_cls = cls;
  m->prof_used = 0;
  m->prof_dropped = 0;
  return GQA_OK;
}

int gqa_model_debug_chain_offset(gqa_model* m, int32_t offset) {
  if (!m) return fail(GQA_E_INVALID, "null model");
  if (offset < 0 || offset > (1 << 20)) return fail(GQA_E_INVALID, "chain offset %d outside [0, 2^20]", offset);
  m->chain_offset = offset;
  return GQA_OK;
}

int gqa_model_profile_read(gqa_model* m, int64_t* launches, double* total_ms, int64_t* dropped) {
  if (!m || !launches || !total_ms) return fail(GQA_E_INVALID, "null argument");
  HIP_TRY(hipDeviceSynchronize());
  double tot = 0.0;
  for (int64_t i = 0; i < m->prof_used; ++i) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, m->prof_ev[2 * i], m->prof_ev[2 * i + 1]));
    tot += ms;
  }
  *launches = m->prof_used;
  *total_ms = tot;
  if (dropped) *dropped = m->prof_dropped;
  return GQA_OK;
}

int gqa_model_check_device_error(gqa_model* m, hipStream_t st) {
  if (!m) return fail(GQA_E_INVALID, "null model");
  HIP_TRY(hipStreamSynchronize(st));
  int32_t v = 0;
  HIP_TRY(hipMemcpy(&v, m->err, 4, hipMemcpyDeviceToHost));
  if (v) {
    HIP_TRY(hipMemset(m->err, 0, 4));
    if (v & kErrChainWait)
      return fail(GQA_E_HIP, "a chained decode launch gave up waiting for its predecessor (results invalid)");
    return fail(GQA_E_RANGE, "a device-resident token id was outside [0, %d)", m->d.vocab);
  }
  return GQA_OK;
}

static int physical_row(const gqa_model* m, int kind, int r, const void** base, int* cols, bool q8, int layer) {
  const gqa_model_desc& d = m->d;
  const int H = d.hidden, F = d.ffn;
  const LayerW* w = layer >= 0 && layer < d.n_layers ? &m->L[layer] : nullptr;
  switch (kind) {
    case GQA_T_Q: *cols = H; *base = q8 ? (const void*)w->qqkv : w->wqkv; return r;
    case GQA_T_K: *cols = H; *base = q8 ? (const void*)w->qqkv : w->wqkv; return m->QD + r;
    case GQA_T_V: *cols = H; *base = q8 ? (const void*)w->qqkv : w->wqkv; return m->QD + kKvHeads * kHeadDim + r;
    case GQA_T_O: *cols = m->QD; *base = q8 ? (const void*)w->qo : w->wo; return r;
    case GQA_T_GATE: *cols = H; *base = q8 ? (const void*)w->qgu : w->wgu; return 32 * (r / 16) + (r % 16);
    case GQA_T_UP: *cols = H; *base = q8 ? (const void*)w->qgu : w->wgu; return 32 * (r / 16) + 16 + (r % 16);
    case GQA_T_DOWN: *cols = F; *base = q8 ? (const void*)w->qd : w->wd; return r;
    default: return -1;
  }
}

static int logical_rows(const gqa_model* m, int kind) {
  const gqa_model_desc& d = m->d;
  switch (kind) {
    case GQA_T_Q: return m->QD;
    case GQA_T_K: case GQA_T_V: return kKvHeads * kHeadDim;
    case GQA_T_O: case GQA_T_DOWN: return d.hidden;
    case GQA_T_GATE: case GQA_T_UP: return d.ffn;
    case GQA_T_EMBED: case GQA_T_LM_HEAD: return d.vocab;
    case GQA_T_ATTN_NORM: case GQA_T_FFN_NORM: case GQA_T_FINAL_NORM: return 1;
    case GQA_T_Q_NORM: case GQA_T_K_NORM: return 1;
    default: return -1;
  }
}

}  // extern "C"

namespace {

// Copy logical row `prow` of a tile-major matrix [*][cols] with elements of `esize` bytes (and,
// for Q8_0, its cols/32 scales) to host memory: the row's 16-row band is copied, then the row is
// gathered with tiled_index.
int read_tiled_row(const void* base, int esize, int64_t prow, int cols, void* dst, const f16* scales,
                   uint16_t* sdst) {
  const int64_t band_elems = (int64_t)16 * cols;
  std::vector<char> band((size_t)band_elems * esize);
  HIP_TRY(hipMemcpy(band.data(), (const char*)base + (prow >> 4) * band_elems * esize, band.size(),
                    hipMemcpyDeviceToHost));
  for (int c = 0; c < cols; ++c)
    memcpy((char*)dst + (int64_t)c * esize, band.data() + tiled_index(prow & 15, c, cols) * esize, esize);
  if (scales) {
    std::vector<uint16_t> sb((size_t)(cols / 32) * 16);
    HIP_TRY(hipMemcpy(sb.data(), scales + (prow >> 4) * (cols / 32) * 16, sb.size() * 2, hipMemcpyDeviceToHost));
    for (int k = 0; k < cols / 32; ++k) sdst[k] = sb[tiled_scale_index(prow & 15, k, cols)];
  }
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_debug_read_weight(gqa_model* m, int32_t kind, int32_t layer, int32_t row0, int32_t rows, uint16_t* dst) {
  if (!m || !dst) return fail(GQA_E_INVALID, "null argument");
  const gqa_model_desc& d = m->d;
  int nrow = logical_rows(m, kind);
  if (nrow < 0) return fail(GQA_E_INVALID, "unknown tensor kind %d", kind);
  bool per_layer = !(kind == GQA_T_EMBED || kind == GQA_T_LM_HEAD || kind == GQA_T_FINAL_NORM);
  if (per_layer && (layer < 0 || layer >= d.n_layers)) return fail(GQA_E_INVALID, "layer %d out of range", layer);
  if (row0 < 0 || rows < 1 || row0 + rows > nrow) return fail(GQA_E_INVALID, "rows out of range");
  HIP_TRY(hipDeviceSynchronize());
  const uint16_t* src = nullptr;
  int cols = d.hidden;
  switch (kind) {
    case GQA_T_EMBED:
    case GQA_T_LM_HEAD: {
      if (kind == GQA_T_LM_HEAD && d.tied) return fail(GQA_E_INVALID, "tied model has no separate lm_head");
      const uint16_t* base = kind == GQA_T_EMBED ? m->embed : m->lm_head;
      for (int r = 0; r < rows; ++r) {
        int rc = read_tiled_row(base, 2, row0 + r, cols, dst + (int64_t)r * cols, nullptr, nullptr);
        if (rc) return rc;
      }
      return GQA_OK;
    }
    case GQA_T_FINAL_NORM: src = m->final_norm; break;
    case GQA_T_ATTN_NORM: src = m->L[layer].attn_norm; break;
    case GQA_T_FFN_NORM: src = m->L[layer].ffn_norm; break;
    case GQA_T_Q_NORM: src = m->L[layer].q_norm; cols = kHeadDim; break;
    case GQA_T_K_NORM: src = m->L[layer].k_norm; cols = kHeadDim; break;
    default: break;
  }
  if (src) {
    HIP_TRY(hipMemcpy(dst, src + (int64_t)row0 * cols, (size_t)rows * cols * 2, hipMemcpyDeviceToHost));
    return GQA_OK;
  }
  if (d.scheme != GQA_SCHEME_BF16) return fail(GQA_E_INVALID, "a quantised model keeps no BF16 projections");
  for (int r = 0; r < rows; ++r) {
    const void* base = nullptr;
    int pr = physical_row(m, kind, row0 + r, &base, &cols, false, layer);
    int rc = read_tiled_row(base, 2, pr, cols, dst + (int64_t)r * cols, nullptr, nullptr);
    if (rc) return rc;
  }
  return GQA_OK;
}

int gqa_debug_read_q8(gqa_model* m, int32_t kind, int32_t layer, int32_t row0, int32_t rows, int8_t* quants,
                      uint16_t* scales) {
  if (!m || !quants || !scales) return fail(GQA_E_INVALID, "null argument");
  const gqa_model_desc& d = m->d;
  if (d.scheme != GQA_SCHEME_Q8_0) return fail(GQA_E_INVALID, "not a Q8_0 model");
  if (layer < 0 || layer >= d.n_layers) return fail(GQA_E_INVALID, "layer out of range");
  int nrow = logical_rows(m, kind);
  const void* base = nullptr;
  int cols = 0;
  if (nrow < 0 || physical_row(m, kind, 0, &base, &cols, true, layer) < 0)
    return fail(GQA_E_INVALID, "not a projection kind");
  if (row0 < 0 || rows < 1 || row0 + rows > nrow) return fail(GQA_E_INVALID, "rows out of range");
  HIP_TRY(hipDeviceSynchronize());
  const LayerW& w = m->L[layer];
  const f16* sb = kind == GQA_T_O ? w.so : kind == GQA_T_DOWN ? w.sd : (kind == GQA_T_GATE || kind == GQA_T_UP) ? w.sgu : w.sqkv;
  for (int r = 0; r < rows; ++r) {
    int pr = physical_row(m, kind, row0 + r, &base, &cols, true, layer);
    int rc = read_tiled_row(base, 1, pr, cols, quants + (int64_t)r * cols, sb, scales + (int64_t)r * (cols / 32));
    if (rc) return rc;
  }
  return GQA_OK;
}

int gqa_debug_read_affine4(gqa_model* m, int32_t kind, int32_t layer, int32_t row0, int32_t rows, uint8_t* codes,
                           uint16_t* scales, uint16_t* biases) {
  if (!m || !codes || !scales || !biases) return fail(GQA_E_INVALID, "null argument");
  const gqa_model_desc& d = m->d;
  if (d.scheme != GQA_SCHEME_AFFINE4) return fail(GQA_E_INVALID, "not an AFFINE4 model");
  if (layer < 0 || layer >= d.n_layers) return fail(GQA_E_INVALID, "layer out of range");
  int nrow = logical_rows(m, kind);
  const void* base = nullptr;
  int cols = 0;
  if (nrow < 0 || physical_row(m, kind, 0, &base, &cols, true, layer) < 0)
    return fail(GQA_E_INVALID, "not a projection kind");
  if (row0 < 0 || rows < 1 || row0 + rows > nrow) return fail(GQA_E_INVALID, "rows out of range");
  HIP_TRY(hipDeviceSynchronize());
  const LayerW& w = m->L[layer];
  const bool gu = kind == GQA_T_GATE || kind == GQA_T_UP;
  const f16* sp = kind == GQA_T_O ? w.so : kind == GQA_T_DOWN ? w.sd : gu ? w.sgu : w.sqkv;
  const f16* bp = kind == GQA_T_O ? w.bo : kind == GQA_T_DOWN ? w.bd : gu ? w.bgu : w.bqkv;
  std::vector<uint32_t> band;
  std::vector<uint16_t> sb, bb;
  for (int r = 0; r < rows; ++r) {
    const int pr = physical_row(m, kind, row0 + r, &base, &cols, true, layer);
    const int64_t band_words = (int64_t)16 * cols / 8;            // 8 codes per 32-bit word
    band.resize((size_t)band_words);
    HIP_TRY(hipMemcpy(band.data(), (const uint32_t*)base + (pr >> 4) * band_words, band.size() * 4,
                      hipMemcpyDeviceToHost));
    for (int c = 0; c < cols; ++c) {
      const int64_t t = tiled_index(pr & 15, c, cols);
      const int e = (int)(t & 7);
      codes[(int64_t)r * cols + c] = (uint8_t)((band[(size_t)(t >> 3)] >> (4 * ((e & 1) * 4 + (e >> 1)))) & 15u);
    }
    sb.resize((size_t)(cols / 32) * 16);
    bb.resize(sb.size());
    HIP_TRY(hipMemcpy(sb.data(), sp + (int64_t)(pr >> 4) * (cols / 32) * 16, sb.size() * 2, hipMemcpyDeviceToHost));
    HIP_TRY(hipMemcpy(bb.data(), bp + (int64_t)(pr >> 4) * (cols / 32) * 16, bb.size() * 2, hipMemcpyDeviceToHost));
    for (int k = 0; k < cols / 32; ++k) {
      scales[(int64_t)r * (cols / 32) + k] = sb[tiled_scale_index(pr & 15, k, cols)];
      biases[(int64_t)r * (cols / 32) + k] = bb[tiled_scale_index(pr & 15, k, cols)];
    }
  }
  return GQA_OK;
}

int gqa_debug_read_kv(gqa_session* s, int32_t layer, int32_t pos0, int32_t n, uint16_t* k, uint16_t* v) {
  if (!s || !k || !v) return fail(GQA_E_INVALID, "null argument");
  gqa_model* m = s->m;
  if (layer < 0 || layer >= m->d.n_layers) return fail(GQA_E_INVALID, "layer out of range");
  if (pos0 < 0 || n < 1 || pos0 + n > s->max_pos) return fail(GQA_E_INVALID, "positions out of range");
  HIP_TRY(hipDeviceSynchronize());
  const LayerW& w = m->L[layer];
  const std::vector<int32_t>& table = s->seq ? s->seq->blocks : s->blocks;
  for (int i = 0; i < n; ++i) {
    int p = pos0 + i;
    int phys = table[p / kBlock];
    if (phys < 0) return fail(GQA_E_INVALID, "position %d is in no block of the session", p);
    for (int h = 0; h < kKvHeads; ++h) {
      int64_t off = (((int64_t)phys * kKvHeads + h) * kBlock + (p % kBlock)) * kHeadDim;
      uint16_t* kd = k + ((int64_t)i * kKvHeads + h) * kHeadDim;
      uint16_t* vd = v + ((int64_t)i * kKvHeads + h) * kHeadDim;
      if (w.kq8.kq) {                          // bf16(scale * code), as attention reads it
        int8_t c[2][kHeadDim];
        _Float16 sc[2][kHeadDim / 32];
        HIP_TRY(hipMemcpy(c[0], w.kq8.kq + off, kHeadDim, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(c[1], w.kq8.vq + off, kHeadDim, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(sc[0], w.kq8.ks + off / 32, kHeadDim / 32 * 2, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(sc[1], w.kq8.vs + off / 32, kHeadDim / 32 * 2, hipMemcpyDeviceToHost));
        for (int e = 0; e < kHeadDim; ++e) {
          for (int kv = 0; kv < 2; ++kv) {
            float x = (float)sc[kv][e / 32] * (float)c[kv][e];
            uint32_t u;
            memcpy(&u, &x, 4);
            u += 0x7FFFu + ((u >> 16) & 1u);
            (kv ? vd : kd)[e] = (uint16_t)(u >> 16);
          }
        }
      } else {
        HIP_TRY(hipMemcpy(kd, w.kpool + off, kHeadDim * 2, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(vd, w.vpool + off, kHeadDim * 2, hipMemcpyDeviceToHost));
      }
    }
  }
  return GQA_OK;
}

int gqa_debug_read_kv_q8(gqa_session* s, int32_t layer, int32_t pos0, int32_t n, int8_t* kc, uint16_t* ks,
                         int8_t* vc, uint16_t* vs) {
  if (!s || !kc || !ks || !vc || !vs) return fail(GQA_E_INVALID, "null argument");
  gqa_model* m = s->m;
  if (layer < 0 || layer >= m->d.n_layers) return fail(GQA_E_INVALID, "layer out of range");
  if (pos0 < 0 || n < 1 || pos0 + n > s->max_pos) return fail(GQA_E_INVALID, "positions out of range");
  const LayerW& w = m->L[layer];
  if (!w.kq8.kq) return fail(GQA_E_INVALID, "the model's KV cache is BF16");
  HIP_TRY(hipDeviceSynchronize());
  const std::vector<int32_t>& table = s->seq ? s->seq->blocks : s->blocks;
  for (int i = 0; i < n; ++i) {
    int p = pos0 + i;
    int phys = table[p / kBlock];
    if (phys < 0) return fail(GQA_E_INVALID, "position %d is in no block of the session", p);
    for (int h = 0; h < kKvHeads; ++h) {
      const int64_t off = (((int64_t)phys * kKvHeads + h) * kBlock + (p % kBlock)) * kHeadDim;
      const int64_t o = (int64_t)i * kKvHeads + h;
      HIP_TRY(hipMemcpy(kc + o * kHeadDim, w.kq8.kq + off, kHeadDim, hipMemcpyDeviceToHost));
      HIP_TRY(hipMemcpy(vc + o * kHeadDim, w.kq8.vq + off, kHeadDim, hipMemcpyDeviceToHost));
      HIP_TRY(hipMemcpy(ks + o * 4, w.kq8.ks + off / 32, 8, hipMemcpyDeviceToHost));
      HIP_TRY(hipMemcpy(vs + o * 4, w.kq8.vs + off / 32, 8, hipMemcpyDeviceToHost));
    }
  }
  return GQA_OK;
}

int gqa_debug_read_scratch(gqa_model* m, int32_t which, int64_t offset, int64_t count, void* dst) {
  if (!m || !dst) return fail(GQA_E_INVALID, "null argument");
  const gqa_model_desc& d = m->d;
  const int rows = std::max(m->R, kMaxBatch);
  const void* base = nullptr;
  int64_t n = 0, esize = 4;
  switch (which) {
    case GQA_S_RESID_A: base = m->x; n = (int64_t)rows * d.hidden; break;
    case GQA_S_RESID_B: base = m->x2; n = (int64_t)kMaxBatch * d.hidden; break;
    case GQA_S_PART_A: base = m->part; n = m->part_floats; break;
    case GQA_S_PART_B: base = m->part2; n = m->part_floats; break;
    case GQA_S_ATTN_HI: base = m->oh; n = (int64_t)rows * m->QD; esize = 2; break;
    case GQA_S_ATTN_LO: base = m->ol; n = (int64_t)rows * m->QD; esize = 2; break;
    case GQA_S_MLP_HI: base = m->mh; n = (int64_t)rows * d.ffn; esize = 2; break;
    case GQA_S_MLP_LO: base = m->ml; n = (int64_t)rows * d.ffn; esize = 2; break;
    case GQA_S_NORM_HI: base = m->xh; n = (int64_t)rows * d.hidden; esize = 2; break;
    case GQA_S_NORM_LO: base = m->xl; n = (int64_t)rows * d.hidden; esize = 2; break;
    case GQA_S_SUMSQ: base = m->ss; n = 2 * 8 * 32; break;
    case GQA_S_QROT: base = m->q; n = (int64_t)rows * m->QD; break;
    case GQA_S_QKV: base = m->qkv; n = (int64_t)m->R * m->QKV; break;
    default: return fail(GQA_E_INVALID, "unknown scratch buffer %d", which);
  }
  if (offset < 0 || count < 1 || offset + count > n) return fail(GQA_E_INVALID, "range outside the buffer");
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(dst, (const char*)base + offset * esize, (size_t)(count * esize), hipMemcpyDeviceToHost));
  return GQA_OK;
}

int gqa_debug_read_rope(gqa_model* m, int32_t n, float* c, float* s) {
  if (!m || !c || !s) return fail(GQA_E_INVALID, "null argument");
  if (n < 1 || n > m->d.max_positions) return fail(GQA_E_INVALID, "n out of range");
  HIP_TRY(hipMemcpy(c, m->rcos, (size_t)n * 64 * 4, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(s, m->rsin, (size_t)n * 64 * 4, hipMemcpyDeviceToHost));
  return GQA_OK;
}

}  // extern "C"
