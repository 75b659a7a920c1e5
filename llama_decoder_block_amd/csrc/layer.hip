// C ABI of the decoder-layer library: argument checks, weight packing, the
// RoPE table, scratch memory, and the launch sequence of one layer call.
//
// Launch sequence (bf16), one pre-norm layer as on the "LMDrive LLM core
// inference unit" page §2.5 and the "LLM mechanics lecture notes" Ch.02 block
// equation:
//   1  RMSNorm(x)                        -> xn          (bf16)
//   2  xn Wqkv^T, RoPE, cache append     -> q scratch, K/V cache slots
//   3  causal attention over the cache   -> o           (flash kernel for T > 1,
//                                                        split-K kernel for T = 1)
//   4  o Wo^T + x                        -> X'          (fp32 residual stream)
//   5  RMSNorm(X')                       -> xn          (bf16)
//   6  SiLU(xn Wg^T) * (xn Wu^T)         -> h           (bf16)
//   7  h Wd^T + X'                       -> y           (bf16)
// Steps 2, 4, 6, 7 use the tiled MFMA GEMMs when the call has more than 64
// tokens and the weight-streaming GEMMs otherwise; in the latter case the
// activations xn, o and h are written in fragment order by their producers
// (steps 1, 3, 5, 6), which is the operand layout the streaming GEMMs load.
// bf16 weights are converted to fragment order once, at creation.
#include "common.h"
#include "../../include/llama_layer.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

using namespace llama;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(LLAMA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_OR_RETURN(expr, what)              \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr int kDecodeChunk = 64;  // sequences per split-K attention launch

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int llama::set_error(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

struct llama_layer {
  llama_layer_config cfg;
  int device = 0;
  size_t es = 2;  // element size of the layer dtype
  // weights (owned)
  // (bf16: fragment order; fp32: row-major)
  void* wqkv = nullptr;  // [(H + 2 Hkv) dh, d]
  void* wo = nullptr;    // [d, H dh]
  void* wgu = nullptr;   // bf16: [2f, d] in 64-row blocks [gate | up]; fp32: [gate; up]
  void* wd = nullptr;    // [d, f]
  void* g1 = nullptr;
  void* g2 = nullptr;
  float* rope_cos = nullptr;  // [max_pos, dh/2]
  float* rope_sin = nullptr;
  // scratch (owned); bf16 activations hold max(max_tokens, 128) rows so that
  // the fragment-order form (whole 32-row blocks) always fits
  void* xn = nullptr;     // [max_tokens, d]
  void* q = nullptr;      // bf16: [max_tokens, H dh]; fp32: qkv [max_tokens, (H+2Hkv) dh]
  void* o = nullptr;      // [max_tokens, H dh]
  float* x1 = nullptr;    // [max_tokens, d] fp32
  void* h = nullptr;      // [max_tokens, f]
  float* gu = nullptr;    // fp32 path: [max_tokens, 2f]
  float* part = nullptr;  // split-K partials
  int part_seqs = 0;      // sequences the partial buffer holds at once
  void* kv_stage = nullptr;  // bf16 layers: [2, rows, Hkv, 128] new keys / values for the int8 cache's append
  SkinnyScratch sk{};     // split column groups of the weight-streaming GEMMs
  GemmSplit gs{};         // split K of the tiled GEMMs (bf16 layers taking more than 128 tokens)
  int* check_flag = nullptr;  // LLAMA_LAYER_CHECK=1 at create: position validation result
  // per-step event timing (measurement aid)
  static constexpr int kRing = 256;
  bool prof_on = false;
  int prof_step = -1;  // -1: every step; else only this step is bracketed
  bool prof_events = false;
  hipEvent_t ev[kRing][LLAMA_LAYER_STEPS + 1];
  long long prof_next = 0, prof_done = 0;  // calls recorded / harvested
  double prof_ms[LLAMA_LAYER_STEPS] = {};
};

namespace {

// Scratch memory of one layer call: the handle's own buffers, or slices of
// the library's static device array (llama_layer_decode_noalloc).
struct CallScratch {
  void* xn;
  void* q;
  void* o;
  float* x1;
  void* h;
  float* gu;
  float* part;     // decode attention split partials
  int part_seqs;   // sequences whose partials fit at once
  SkinnyScratch sk;
  void* kv_stage;  // [2, rows, Hkv, 128] bf16 (the int8 cache's append), or null
  GemmSplit gs;    // split K of the tiled GEMMs (null: no split)
};

// The call's cache: contiguous [B, Hkv, max_pos, 128] K and V (pg null), or
// page pools with a block table; span = the slots a sequence can hold.
struct KvArgs {
  void* k;
  void* v;
  KvPaging pg;
  int span;
  // int8 cache: k and v hold int8 codes [B, Hkv, max_pos, 128] and these one
  // fp32 scale per row [B, Hkv, max_pos] (paged: code pools [n_pages, Hkv,
  // page, 128] and scale pools [n_pages, Hkv, page]); null for bf16/fp32
  float* k_scale = nullptr;
  float* v_scale = nullptr;
};

CallScratch handle_scratch(llama_layer* L) {
  return CallScratch{L->xn, L->q, L->o, L->x1, L->h, L->gu, L->part, L->part_seqs, L->sk, L->kv_stage, L->gs};
}

}  // namespace

namespace {

const char* const kStepNames[LLAMA_LAYER_STEPS] = {
    "rmsnorm_attn", "qkv_rope_cache", "attention", "o_proj_residual",
    "rmsnorm_mlp", "gate_up_swiglu", "down_residual"};

// add the step times of the oldest recorded call to the totals
hipError_t harvest_one(llama_layer* L) {
  hipEvent_t* e = L->ev[L->prof_done % llama_layer::kRing];
  const int lo = L->prof_step < 0 ? 0 : L->prof_step, hi = L->prof_step < 0 ? LLAMA_LAYER_STEPS : L->prof_step + 1;
  hipError_t r = hipEventSynchronize(e[hi]);
  if (r != hipSuccess) return r;
  for (int i = lo; i < hi; ++i) {
    float ms = 0.f;
    r = hipEventElapsedTime(&ms, e[i], e[i + 1]);
    if (r != hipSuccess) return r;
    L->prof_ms[i] += ms;
  }
  ++L->prof_done;
  return hipSuccess;
}

void release(llama_layer* L) {
  if (L->prof_events)
    for (auto& row : L->ev)
      for (auto& e : row) (void)hipEventDestroy(e);
  void* bufs[] = {L->wqkv, L->wo, L->wgu, L->wd, L->g1, L->g2, L->rope_cos, L->rope_sin,
                  L->xn, L->q, L->o, L->x1, L->h, L->gu, L->part, L->sk.part, L->sk.cnt, L->check_flag,
                  L->kv_stage, L->gs.part, L->gs.cnt};
  for (void* p : bufs)
    if (p) (void)hipFree(p);
}

int alloc(void** p, size_t bytes) {
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    return fail(LLAMA_ERR_ALLOC, "hipMalloc(%zu bytes): %s", bytes, hipGetErrorString(e));
  }
  return LLAMA_OK;
}

int check_config(const llama_layer_config* c) {
  if (c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->d_ff <= 0 ||
      c->max_pos <= 0 || c->max_tokens <= 0)
    return fail(LLAMA_ERR_INVALID, "sizes must be positive");
  if (c->n_heads % c->n_kv_heads != 0)
    return fail(LLAMA_ERR_INVALID, "n_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_heads,
                c->n_kv_heads);
  if (c->head_dim % 2 != 0) return fail(LLAMA_ERR_INVALID, "head_dim must be even");
  if (!(c->rms_eps >= 0.f) || !isfinite(c->rms_eps) || !(c->rope_base > 0.f) || !isfinite(c->rope_base))
    return fail(LLAMA_ERR_INVALID, "rms_eps must be finite and >= 0, rope_base finite and > 0");
  if (c->dtype != LLAMA_F32 && c->dtype != LLAMA_BF16) return fail(LLAMA_ERR_INVALID, "unknown dtype");
  if (c->bidirectional != 0 && c->bidirectional != 1) return fail(LLAMA_ERR_INVALID, "bidirectional must be 0 or 1");
  if (c->dtype == LLAMA_BF16) {
    if (c->head_dim != 128) return fail(LLAMA_ERR_UNSUPPORTED, "bf16 kernels need head_dim 128");
    if (c->d_model % 128 || c->d_ff % 128)
      return fail(LLAMA_ERR_UNSUPPORTED, "bf16 kernels need d_model and d_ff multiples of 128");
    // calls of <= 128 tokens normalise into fragment order: one wavefront per
    // row up to d = 8192, a workgroup per row at d = 16384 (2048 x 8)
    if (c->d_model > 8192 && c->d_model != 16384)
      return fail(LLAMA_ERR_UNSUPPORTED, "bf16 kernels need d_model <= 8192 or d_model = 16384");
    // kernels address every operand with 32-bit byte offsets
    const double lim = 4294967295.0;
    const double d = c->d_model, f = c->d_ff, qd = 128.0 * c->n_heads,
                 nqkv = 128.0 * (c->n_heads + 2 * c->n_kv_heads), mt = c->max_tokens + 256.0;
    if (nqkv * d * 2 > lim || 2 * f * d * 2 > lim || d * qd * 2 > lim || d * f * 2 > lim ||
        mt * f * 2 > lim || mt * d * 4 > lim || mt * qd * 2 > lim || 256.0 * c->max_pos > lim)
      return fail(LLAMA_ERR_UNSUPPORTED, "an operand exceeds 4 GiB (32-bit buffer offsets)");
  }
  return LLAMA_OK;
}

int part_floats(const llama_layer_config& c, int* seqs) {
  const int s = c.max_tokens < kDecodeChunk ? c.max_tokens : kDecodeChunk;
  long long best = 0;
  for (int b = 1; b <= s; ++b) {
    // (the bound over every span <= max_pos: a paged call's span can be smaller)
    const long long n = static_cast<long long>(b) * c.n_heads * decode_attn_max_splits(c.max_pos, b, c.n_heads, c.n_kv_heads) * 130;
    if (n > best) best = n;
  }
  *seqs = s;
  return static_cast<int>(best);
}

}  // namespace

// ---- the allocation-free decode: scratch in a static device array ----
namespace {

// Holds the scratch of one llama_layer_decode_noalloc call; each GPU the
// library runs on keeps its own copy until the process ends.  Host code uses
// the per-device address from hipGetSymbolAddress (the array's name on the
// host is only a stand-in).
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(32) << 20;
constexpr int kNoAllocMaxSeqs = 64;  // sequences per allocation-free decode call
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the array's device address on device dev (the current device); looked up once
int noalloc_scratch(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(LLAMA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(LLAMA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return LLAMA_OK;
}

// fill kernel: clears the split-group counters at the start of a call (a
// kernel rather than hipMemsetAsync, so the call can sit in a captured graph)
__global__ void zero_words_kernel(unsigned* __restrict__ p, int n) {
  const int i = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

}  // namespace

extern "C" {

const char* llama_layer_strerror(int status) {
  switch (status) {
    case LLAMA_OK: return "ok";
    case LLAMA_ERR_NULL: return "null pointer argument";
    case LLAMA_ERR_INVALID: return "invalid argument";
    case LLAMA_ERR_UNSUPPORTED: return "unsupported shape";
    case LLAMA_ERR_CAPACITY: return "call exceeds the handle's capacity";
    case LLAMA_ERR_HIP: return "HIP runtime error";
    case LLAMA_ERR_ALLOC: return "allocation failed";
    default: return "unknown status";
  }
}

const char* llama_layer_last_error(void) { return g_last_error.c_str(); }

int llama_layer_create(const llama_layer_config* cfg, const llama_layer_weights* w, void* stream,
                       llama_layer** out) {
  g_last_error.clear();
  if (!cfg || !w || !out) return fail(LLAMA_ERR_NULL, "cfg, weights and out must be non-null");
  *out = nullptr;
  const void* wp[] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->ffn_norm, w->w_gate, w->w_up, w->w_down};
  for (const void* p : wp)
    if (!p) return fail(LLAMA_ERR_NULL, "every weight pointer must be non-null");
  int st = check_config(cfg);
  if (st != LLAMA_OK) return st;
  for (const void* p : wp)
    if (!aligned16(p)) return fail(LLAMA_ERR_INVALID, "weight pointers must be 16-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  llama_layer* L = new (std::nothrow) llama_layer();
  if (!L) return fail(LLAMA_ERR_ALLOC, "host allocation failed");
  L->cfg = *cfg;
  L->es = cfg->dtype == LLAMA_BF16 ? 2 : 4;
  hipError_t e = hipGetDevice(&L->device);
  if (e != hipSuccess) { delete L; return hip_fail(e, "hipGetDevice"); }

  const size_t es = L->es;
  const size_t d = cfg->d_model, H = cfg->n_heads, Hkv = cfg->n_kv_heads, dh = cfg->head_dim,
               f = cfg->d_ff, mp = cfg->max_pos;
  const size_t mt = cfg->dtype == LLAMA_BF16 && cfg->max_tokens < kSkinnyMaxTokens ? kSkinnyMaxTokens
                                                                                   : cfg->max_tokens;
  const size_t nq = H * dh, nkv = Hkv * dh;
#define ALLOC_OR_FAIL(ptr, bytes)                               \
  do {                                                          \
    int a_ = alloc(reinterpret_cast<void**>(&(ptr)), (bytes));  \
    if (a_ != LLAMA_OK) { release(L); delete L; return a_; }    \
  } while (0)
#define HIP_OR_FAIL(expr, what)                                      \
  do {                                                               \
    hipError_t e_ = (expr);                                          \
    if (e_ != hipSuccess) { release(L); delete L; return hip_fail(e_, what); } \
  } while (0)

  ALLOC_OR_FAIL(L->wqkv, (nq + 2 * nkv) * d * es);
  ALLOC_OR_FAIL(L->wo, d * nq * es);
  ALLOC_OR_FAIL(L->wgu, 2 * f * d * es);
  ALLOC_OR_FAIL(L->wd, d * f * es);
  ALLOC_OR_FAIL(L->g1, d * es);
  ALLOC_OR_FAIL(L->g2, d * es);
  ALLOC_OR_FAIL(L->rope_cos, mp * (dh / 2) * sizeof(float));
  ALLOC_OR_FAIL(L->rope_sin, mp * (dh / 2) * sizeof(float));
  ALLOC_OR_FAIL(L->xn, mt * d * es);
  ALLOC_OR_FAIL(L->o, mt * nq * es);
  ALLOC_OR_FAIL(L->x1, mt * d * sizeof(float));
  ALLOC_OR_FAIL(L->h, mt * f * es);
  if (const char* chk = getenv("LLAMA_LAYER_CHECK"); chk && strcmp(chk, "1") == 0)
    ALLOC_OR_FAIL(L->check_flag, sizeof(int));
  if (cfg->dtype == LLAMA_BF16) {
    ALLOC_OR_FAIL(L->q, mt * nq * es);
    ALLOC_OR_FAIL(L->kv_stage, 2 * mt * nkv * es);
    const int pf = part_floats(*cfg, &L->part_seqs);
    ALLOC_OR_FAIL(L->part, static_cast<size_t>(pf) * sizeof(float));
    ALLOC_OR_FAIL(L->sk.part, skinny_scratch_floats() * sizeof(float));
    // one counter per column group: 32-row blocks (QKV, o_proj, down) or
    // pairs of them (gate/up)
    const size_t groups = std::max({(nq + 2 * nkv) / 32, 2 * f / 64, d / 32});
    ALLOC_OR_FAIL(L->sk.cnt, groups * sizeof(unsigned));
    L->sk.cnt_len = static_cast<int>(groups);
    L->sk.part_len = skinny_scratch_floats();
    HIP_OR_FAIL(hipMemsetAsync(L->sk.cnt, 0, groups * sizeof(unsigned), s), "clear counters");
    if (cfg->max_tokens > kSkinnyMaxTokens) {  // calls of more than 128 tokens take the tiled GEMMs
      ALLOC_OR_FAIL(L->gs.part, gemm_split_part_floats() * sizeof(float));
      ALLOC_OR_FAIL(L->gs.cnt, static_cast<size_t>(device_cu_count()) * sizeof(unsigned));
      HIP_OR_FAIL(hipMemsetAsync(L->gs.cnt, 0, static_cast<size_t>(device_cu_count()) * sizeof(unsigned), s),
                  "clear counters");
    }
  } else {
    ALLOC_OR_FAIL(L->q, mt * (nq + 2 * nkv) * es);
    ALLOC_OR_FAIL(L->gu, mt * 2 * f * sizeof(float));
  }

  const hipMemcpyKind dd = hipMemcpyDeviceToDevice;
  HIP_OR_FAIL(hipMemcpyAsync(L->g1, w->attn_norm, d * es, dd, s), "copy attn_norm");
  HIP_OR_FAIL(hipMemcpyAsync(L->g2, w->ffn_norm, d * es, dd, s), "copy ffn_norm");
  if (cfg->dtype == LLAMA_BF16) {
    // fragment order; rows of a 32-row-aligned range sit where they would in
    // row-major order, so q, k and v rows are converted straight into their
    // place in the concatenated matrix (each head in rotary-pair order, so
    // that a rotation's two inputs are neighbouring output columns).  Wo and
    // Wdown become fp16: their activations (the attention output, h) are fp16.
    const int di = static_cast<int>(d), fi = static_cast<int>(f), nqi = static_cast<int>(nq),
              nkvi = static_cast<int>(nkv);
    auto* wqkv = static_cast<bf16_t*>(L->wqkv);
    auto* wgu = static_cast<bf16_t*>(L->wgu);
    auto src = [](const void* p) { return static_cast<const bf16_t*>(p); };
    HIP_OR_FAIL(launch_pack_rows(src(w->wq), nqi, di, wqkv, 0, 0, 0, s), "convert wq");
    HIP_OR_FAIL(launch_pack_rows(src(w->wk), nkvi, di, wqkv + nq * d, 0, 0, 0, s), "convert wk");
    HIP_OR_FAIL(launch_pack_rows(src(w->wv), nkvi, di, wqkv + (nq + nkv) * d, 0, 0, 0, s), "convert wv");
    HIP_OR_FAIL(launch_pack_rows(src(w->wo), di, nqi, static_cast<bf16_t*>(L->wo), di, di, 1, s), "convert wo");
    HIP_OR_FAIL(launch_pack_rows(src(w->w_down), di, fi, static_cast<bf16_t*>(L->wd), di, di, 1, s), "convert w_down");
    // 64-row blocks: rows [128 j, 128 j + 64) = gate rows [64 j, 64 j + 64),
    // rows [128 j + 64, 128 j + 128) = up rows [64 j, 64 j + 64)
    HIP_OR_FAIL(launch_pack_rows(src(w->w_gate), fi, di, wgu, 64, 128, 0, s), "convert w_gate");
    HIP_OR_FAIL(launch_pack_rows(src(w->w_up), fi, di, wgu + 64 * d, 64, 128, 0, s), "convert w_up");
  } else {
    char* qkv = static_cast<char*>(L->wqkv);
    HIP_OR_FAIL(hipMemcpyAsync(qkv, w->wq, nq * d * es, dd, s), "copy wq");
    HIP_OR_FAIL(hipMemcpyAsync(qkv + nq * d * es, w->wk, nkv * d * es, dd, s), "copy wk");
    HIP_OR_FAIL(hipMemcpyAsync(qkv + (nq + nkv) * d * es, w->wv, nkv * d * es, dd, s), "copy wv");
    HIP_OR_FAIL(hipMemcpyAsync(L->wo, w->wo, d * nq * es, dd, s), "copy wo");
    HIP_OR_FAIL(hipMemcpyAsync(L->wd, w->w_down, d * f * es, dd, s), "copy w_down");
    HIP_OR_FAIL(hipMemcpyAsync(L->wgu, w->w_gate, f * d * es, dd, s), "copy w_gate");
    HIP_OR_FAIL(hipMemcpyAsync(static_cast<char*>(L->wgu) + f * d * es, w->w_up, f * d * es, dd, s),
                "copy w_up");
  }

  // RoPE table: angle p * base^(-2i/dh), evaluated in fp64, stored fp32
  {
    const size_t half = dh / 2;
    std::vector<float> cb(mp * half), sb(mp * half);
    for (size_t i = 0; i < half; ++i) {
      const double theta = pow(static_cast<double>(cfg->rope_base), -2.0 * static_cast<double>(i) / dh);
      for (size_t p = 0; p < mp; ++p) {
        const double a = static_cast<double>(p) * theta;
        cb[p * half + i] = static_cast<float>(cos(a));
        sb[p * half + i] = static_cast<float>(sin(a));
      }
    }
    HIP_OR_FAIL(hipMemcpyAsync(L->rope_cos, cb.data(), cb.size() * sizeof(float), hipMemcpyHostToDevice, s),
                "upload rope cos");
    HIP_OR_FAIL(hipMemcpyAsync(L->rope_sin, sb.data(), sb.size() * sizeof(float), hipMemcpyHostToDevice, s),
                "upload rope sin");
    HIP_OR_FAIL(hipStreamSynchronize(s), "synchronize after create");
  }
#undef ALLOC_OR_FAIL
#undef HIP_OR_FAIL
  *out = L;
  return LLAMA_OK;
}

void llama_layer_destroy(llama_layer* L) {
  if (!L) return;
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  if (have && cur != L->device) (void)hipSetDevice(L->device);
  (void)hipDeviceSynchronize();
  release(L);
  if (have && cur != L->device) (void)hipSetDevice(cur);
  delete L;
}

// Debug validation of the positions (LLAMA_LAYER_CHECK=1 when the handle is
// created): bit 0 of *bad if a position lies outside [0, span), bit 1 if a
// position repeats within its sequence (token i against the earlier tokens
// of its sequence: O(T^2) per sequence, a debug aid only), bit 2 (paged) if
// a page the token writes or reads (slots 0 .. its position) has an id
// outside [0, n_pages).
static __global__ void check_positions_kernel(const int32_t* __restrict__ pos, int B, int T, int span, KvPaging pg,
                                              int* bad) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(B) * T) return;
  const int p = pos[i];
  if (p < 0 || p >= span) {
    atomicOr(bad, 1);
    return;
  }
  for (long long j = i - i % T; j < i; ++j)
    if (pos[j] == p) {
      atomicOr(bad, 2);
      return;
    }
  if (pg.block_table) {
    const int32_t* row = pg.block_table + (i / T) * pg.blocks_per_seq;
    for (int bi = 0; bi <= p / pg.page; ++bi)
      if (row[bi] < 0 || row[bi] >= pg.n_pages) {
        atomicOr(bad, 4);
        return;
      }
  }
}

static int check_positions(llama_layer* L, const int32_t* pos, int B, int T, const KvArgs& kv, hipStream_t s) {
  const long long n = static_cast<long long>(B) * T;
  int bad = 0;
  HIP_OR_RETURN(hipMemsetAsync(L->check_flag, 0, sizeof(int), s), "clear check flag");
  hipLaunchKernelGGL(check_positions_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, pos, B, T,
                     kv.span, kv.pg, L->check_flag);
  HIP_OR_RETURN(hipGetLastError(), "position check launch");
  HIP_OR_RETURN(hipMemcpyAsync(&bad, L->check_flag, sizeof(int), hipMemcpyDeviceToHost, s), "read check flag");
  HIP_OR_RETURN(hipStreamSynchronize(s), "position check");
  if (bad & 1) return fail(LLAMA_ERR_INVALID, "a position lies outside [0, %d)", kv.span);
  if (bad & 2) return fail(LLAMA_ERR_INVALID, "a position repeats within a sequence");
  if (bad & 4) return fail(LLAMA_ERR_INVALID, "a block table entry in use lies outside [0, n_pages = %d)", kv.pg.n_pages);
  return LLAMA_OK;
}

static int run_layer(llama_layer* L, const CallScratch& S, const void* x, void* y, const int32_t* pos, int B,
                     int T, const KvArgs& kv, hipStream_t s) {
  void* kc = kv.k;
  void* vc = kv.v;
  const llama_layer_config& c = L->cfg;
  const int M = B * T;
  const int d = c.d_model, H = c.n_heads, Hkv = c.n_kv_heads, f = c.d_ff;
  if (L->check_flag) {
    const int st = check_positions(L, pos, B, T, kv, s);
    if (st != LLAMA_OK) return st;
  }

  if (c.dtype == LLAMA_F32) {
    F32Layer F{};
    F.d = d; F.H = H; F.Hkv = Hkv; F.dh = c.head_dim; F.f = f; F.max_pos = c.max_pos; F.eps = c.rms_eps;
    F.bidir = c.bidirectional;
    F.g1 = static_cast<const float*>(L->g1); F.g2 = static_cast<const float*>(L->g2);
    F.wqkv = static_cast<const float*>(L->wqkv); F.wo = static_cast<const float*>(L->wo);
    F.wgu = static_cast<const float*>(L->wgu); F.wd = static_cast<const float*>(L->wd);
    F.rope_cos = L->rope_cos; F.rope_sin = L->rope_sin;
    F.xn = static_cast<float*>(S.xn); F.qkv = static_cast<float*>(S.q); F.attn = static_cast<float*>(S.o);
    F.x1 = S.x1; F.gu = S.gu; F.h = static_cast<float*>(S.h);
    HIP_OR_RETURN(run_f32_layer(F, static_cast<const float*>(x), static_cast<float*>(y), pos, B, T,
                                static_cast<float*>(kc), static_cast<float*>(vc), s),
                  "fp32 layer launch");
    return LLAMA_OK;
  }

  const bf16_t* xb = static_cast<const bf16_t*>(x);
  bf16_t* yb = static_cast<bf16_t*>(y);
  bf16_t* xn = static_cast<bf16_t*>(S.xn);
  bf16_t* q = static_cast<bf16_t*>(S.q);
  bf16_t* o = static_cast<bf16_t*>(S.o);
  bf16_t* h = static_cast<bf16_t*>(S.h);
  const bf16_t* wqkv = static_cast<const bf16_t*>(L->wqkv);
  const bf16_t* wo = static_cast<const bf16_t*>(L->wo);
  const bf16_t* wgu = static_cast<const bf16_t*>(L->wgu);
  const bf16_t* wd = static_cast<const bf16_t*>(L->wd);
  const int nqkv = (H + 2 * Hkv) * 128;
  const bool skinny = M <= kSkinnyMaxTokens;

  QkvEpilogue ep{};
  ep.q = q;
  ep.k_cache = static_cast<bf16_t*>(kc);
  ep.v_cache = static_cast<bf16_t*>(vc);
  ep.pos = pos;
  ep.rope_cos = L->rope_cos;
  ep.rope_sin = L->rope_sin;
  ep.T = T;
  ep.n_heads = H;
  ep.n_kv_heads = Hkv;
  ep.max_pos = c.max_pos;
  ep.span = kv.span;
  ep.pg = kv.pg;
  // int8 cache: the projection stages the new rows in bf16, the append
  // quantizes them into their slots
  const bool q8 = kv.k_scale != nullptr;
  bf16_t* k_stage = static_cast<bf16_t*>(S.kv_stage);
  bf16_t* v_stage = q8 ? k_stage + static_cast<size_t>(M) * Hkv * 128 : nullptr;
  if (q8) {
    ep.stage = 1;
    ep.k_cache = k_stage;
    ep.v_cache = v_stage;
  }

  hipEvent_t* ev = nullptr;
  if (L->prof_on) {
    if (L->prof_next - L->prof_done == llama_layer::kRing) HIP_OR_RETURN(harvest_one(L), "profile harvest");
    ev = L->ev[L->prof_next % llama_layer::kRing];
  }
  const int ps = L->prof_step;
  auto mark = [&](int i) -> hipError_t {
    return ev && (ps < 0 || i == ps || i == ps + 1) ? hipEventRecord(ev[i], s) : hipSuccess;
  };

  HIP_OR_RETURN(mark(0), "event record");
  HIP_OR_RETURN(launch_rmsnorm(xb, 0, L->g1, 0, xn, 0, skinny, M, d, c.rms_eps, s), "rmsnorm 1");
  HIP_OR_RETURN(mark(1), "event record");
  HIP_OR_RETURN(skinny ? launch_skinny_qkv(xn, wqkv, M, nqkv, d, ep, S.sk, s)
                       : launch_gemm_qkv(xn, wqkv, M, nqkv, d, ep, S.gs, s),
                "qkv projection");
  if (q8)
    HIP_OR_RETURN(launch_kv_int8_append(k_stage, v_stage, pos, B, T, Hkv, c.max_pos, kv.span, kv.pg, static_cast<int8_t*>(kc),
                                        static_cast<int8_t*>(vc), kv.k_scale, kv.v_scale, s),
                  "int8 cache append");
  HIP_OR_RETURN(mark(2), "event record");
  if (T == 1) {
    // sequences in chunks of part_seqs (64: a chunk starts on a 32-row block,
    // where fragment order and row-major order agree, so o, in fragment order
    // for <= 128 tokens, moves with b0 as well); contiguous caches or
    // block-table rows move with b0
    const bool paged = kv.pg.block_table != nullptr;
    const size_t kv_seq = paged ? 0 : static_cast<size_t>(Hkv) * c.max_pos * 128;  // elements per sequence
    const size_t kv_es = q8 ? 1 : 2;
    for (int b0 = 0; b0 < B; b0 += S.part_seqs) {
      const int nb = B - b0 < S.part_seqs ? B - b0 : S.part_seqs;
      const int ns = decode_attn_splits(kv.span, nb, H, Hkv);
      KvPaging pgc = kv.pg;
      if (paged) pgc.block_table += static_cast<size_t>(b0) * pgc.blocks_per_seq;
      const size_t sc0 = q8 && !paged ? static_cast<size_t>(b0) * Hkv * c.max_pos : 0;  // scale rows before sequence b0
      HIP_OR_RETURN(launch_attn_decode(q + static_cast<size_t>(b0) * H * 128,
                                       static_cast<const char*>(kc) + b0 * kv_seq * kv_es,
                                       static_cast<const char*>(vc) + b0 * kv_seq * kv_es, pos + b0,
                                       o + static_cast<size_t>(b0) * H * 128, skinny, S.part, ns, nb, H, Hkv,
                                       c.max_pos, kv.span, pgc, s, q8 ? kv.k_scale + sc0 : nullptr,
                                       q8 ? kv.v_scale + sc0 : nullptr),
                    "decode attention");
    }
  } else {
    HIP_OR_RETURN(launch_attn_prefill(q, kc, vc, pos, o, skinny, B, T, H, Hkv, c.max_pos, kv.span, kv.pg,
                                      c.bidirectional, s, kv.k_scale, kv.v_scale),
                  "prefill attention");
  }
  HIP_OR_RETURN(mark(3), "event record");
  HIP_OR_RETURN(skinny ? launch_skinny_resid_f32out(o, wo, M, d, H * 128, xb, S.x1, S.sk, s)
                       : launch_gemm_resid_f32out(o, wo, M, d, H * 128, xb, S.x1, S.gs, s),
                "o_proj");
  HIP_OR_RETURN(mark(4), "event record");
  HIP_OR_RETURN(launch_rmsnorm(S.x1, 1, L->g2, 0, xn, 0, skinny, M, d, c.rms_eps, s), "rmsnorm 2");
  HIP_OR_RETURN(mark(5), "event record");
  HIP_OR_RETURN(skinny ? launch_skinny_swiglu(xn, wgu, M, f, d, h, S.sk, s)
                       : launch_gemm_swiglu(xn, wgu, M, 2 * f, d, h, S.gs, s),
                "gate/up projection");
  HIP_OR_RETURN(mark(6), "event record");
  HIP_OR_RETURN(skinny ? launch_skinny_resid_bf16out(h, wd, M, d, f, S.x1, yb, S.sk, s)
                       : launch_gemm_resid_bf16out(h, wd, M, d, f, S.x1, yb, S.gs, s),
                "down projection");
  HIP_OR_RETURN(mark(7), "event record");
  if (ev) ++L->prof_next;
  return LLAMA_OK;
}

// Argument checks shared by every call; kv.pg.block_table non-null for the
// paged calls (their page arguments are checked by the caller).
static int checked_call(llama_layer* L, const void* x, void* y, const int32_t* pos, int B, int T,
                        const KvArgs& kv, void* stream) {
  if (!L || !x || !y || !pos || !kv.k || !kv.v)
    return fail(LLAMA_ERR_NULL, "layer, x, y, positions and caches must be non-null");
  if (B < 1 || T < 1) return fail(LLAMA_ERR_INVALID, "B and T must be >= 1 (got %d, %d)", B, T);
  if (static_cast<long long>(B) * T > L->cfg.max_tokens)
    return fail(LLAMA_ERR_CAPACITY, "B*T = %lld exceeds max_tokens = %d", static_cast<long long>(B) * T,
                L->cfg.max_tokens);
  if (T > kv.span) return fail(LLAMA_ERR_CAPACITY, "T = %d exceeds the %d slots a sequence holds", T, kv.span);
  if (!aligned16(x) || !aligned16(y) || !aligned16(kv.k) || !aligned16(kv.v))
    return fail(LLAMA_ERR_INVALID, "x, y and the caches must be 16-byte aligned");
  int cur = 0;
  HIP_OR_RETURN(hipGetDevice(&cur), "hipGetDevice");
  if (cur != L->device) HIP_OR_RETURN(hipSetDevice(L->device), "hipSetDevice");
  const int st = run_layer(L, handle_scratch(L), x, y, pos, B, T, kv, static_cast<hipStream_t>(stream));
  if (cur != L->device) (void)hipSetDevice(cur);
  return st;
}

static KvArgs contiguous_kv(const llama_layer* L, void* kc, void* vc) {
  return KvArgs{kc, vc, KvPaging{nullptr, 0, 0, 0}, L ? L->cfg.max_pos : 0};
}

static int paged_kv(const llama_layer* L, void* kp, void* vp, const int32_t* block_table, int blocks_per_seq,
                    int page_size, int n_pages, KvArgs* out) {
  if (!L || !block_table) return fail(LLAMA_ERR_NULL, "layer and block_table must be non-null");
  if (L->cfg.dtype != LLAMA_BF16) return fail(LLAMA_ERR_UNSUPPORTED, "the paged cache serves bf16 layers");
  if (page_size <= 0 || page_size % 64)
    return fail(LLAMA_ERR_INVALID, "page_size must be a positive multiple of 64 (got %d)", page_size);
  if (blocks_per_seq < 1 || n_pages < 1)
    return fail(LLAMA_ERR_INVALID, "blocks_per_seq and n_pages must be >= 1 (got %d, %d)", blocks_per_seq, n_pages);
  const long long cap = static_cast<long long>(blocks_per_seq) * page_size;
  if (static_cast<long long>(n_pages) * L->cfg.n_kv_heads * page_size * 256 > 4294967295LL)
    return fail(LLAMA_ERR_UNSUPPORTED, "a page pool exceeds 4 GiB (32-bit buffer offsets)");
  *out = KvArgs{kp, vp, KvPaging{block_table, blocks_per_seq, page_size, n_pages},
                static_cast<int>(cap < L->cfg.max_pos ? cap : L->cfg.max_pos)};
  return LLAMA_OK;
}

int llama_layer_profile(llama_layer* L, int enable) {
  g_last_error.clear();
  if (!L) return fail(LLAMA_ERR_NULL, "layer must be non-null");
  if (enable < 0 || enable >= 2 + LLAMA_LAYER_STEPS)
    return fail(LLAMA_ERR_INVALID, "profile mode %d: 0 off, 1 every step, 2 + i step i only", enable);
  if (enable) {
    if (!L->prof_events) {
      for (auto& row : L->ev)
        for (auto& e : row) HIP_OR_RETURN(hipEventCreate(&e), "hipEventCreate");
      L->prof_events = true;
    }
    while (L->prof_done < L->prof_next) HIP_OR_RETURN(harvest_one(L), "profile harvest");
    for (double& v : L->prof_ms) v = 0.0;
    L->prof_next = L->prof_done = 0;
  }
  L->prof_on = enable != 0;
  L->prof_step = enable >= 2 ? enable - 2 : -1;
  return LLAMA_OK;
}

int llama_layer_profile_read(llama_layer* L, double* step_ms, int n_steps, long long* calls) {
  g_last_error.clear();
  if (!L || !step_ms || !calls) return fail(LLAMA_ERR_NULL, "layer, step_ms and calls must be non-null");
  while (L->prof_done < L->prof_next) HIP_OR_RETURN(harvest_one(L), "profile harvest");
  for (int i = 0; i < n_steps && i < LLAMA_LAYER_STEPS; ++i) step_ms[i] = L->prof_ms[i];
  *calls = L->prof_done;
  return LLAMA_OK;
}

const char* llama_layer_step_name(int step) {
  return step >= 0 && step < LLAMA_LAYER_STEPS ? kStepNames[step] : "";
}

int llama_layer_prefill(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B,
                        int32_t T, void* k_cache, void* v_cache, void* stream) {
  g_last_error.clear();
  return checked_call(L, x, y, positions, B, T, contiguous_kv(L, k_cache, v_cache), stream);
}

int llama_layer_decode(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B,
                       void* k_cache, void* v_cache, void* stream) {
  g_last_error.clear();
  return checked_call(L, x, y, positions, B, 1, contiguous_kv(L, k_cache, v_cache), stream);
}

int llama_layer_kv_quantize(llama_layer* L, const void* k_cache, const void* v_cache, int32_t B, int32_t n_slots,
                            void* k_codes, void* v_codes, float* k_scale, float* v_scale, void* stream) {
  g_last_error.clear();
  if (!L || !k_cache || !v_cache || !k_codes || !v_codes || !k_scale || !v_scale)
    return fail(LLAMA_ERR_NULL, "layer, caches, codes and scales must be non-null");
  if (L->cfg.dtype != LLAMA_BF16) return fail(LLAMA_ERR_UNSUPPORTED, "the int8 cache serves bf16 layers");
  if (B < 1 || n_slots < 0 || n_slots > L->cfg.max_pos)
    return fail(LLAMA_ERR_INVALID, "B must be >= 1 and n_slots in [0, max_pos] (got %d, %d)", B, n_slots);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_codes) || !aligned16(v_codes) ||
      ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3u))
    return fail(LLAMA_ERR_INVALID, "caches and codes must be 16-byte aligned, scales 4-byte aligned");
  int cur = 0;
  HIP_OR_RETURN(hipGetDevice(&cur), "hipGetDevice");
  if (cur != L->device) HIP_OR_RETURN(hipSetDevice(L->device), "hipSetDevice");
  const hipError_t e = launch_kv_int8_convert(static_cast<const bf16_t*>(k_cache), static_cast<const bf16_t*>(v_cache),
                                              B, L->cfg.n_kv_heads, L->cfg.max_pos, n_slots,
                                              static_cast<int8_t*>(k_codes), static_cast<int8_t*>(v_codes), k_scale,
                                              v_scale, static_cast<hipStream_t>(stream));
  if (cur != L->device) (void)hipSetDevice(cur);
  return e != hipSuccess ? hip_fail(e, "int8 cache conversion") : LLAMA_OK;
}

// The int8 calls' own argument checks, made before anything reads the handle.
static int int8_args(const llama_layer* L, const float* k_scale, const float* v_scale) {
  if (!L || !k_scale || !v_scale) return fail(LLAMA_ERR_NULL, "layer and scales must be non-null");
  if (L->cfg.dtype != LLAMA_BF16) return fail(LLAMA_ERR_UNSUPPORTED, "the int8 cache serves bf16 layers");
  if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3u)
    return fail(LLAMA_ERR_INVALID, "scales must be 4-byte aligned");
  return LLAMA_OK;
}

// kv: the call's codes (contiguous or paged); the scales are added here
static int int8_call(llama_layer* L, const void* x, void* y, const int32_t* positions, int B, int T, KvArgs kv,
                     float* k_scale, float* v_scale, void* stream) {
  kv.k_scale = k_scale;
  kv.v_scale = v_scale;
  return checked_call(L, x, y, positions, B, T, kv, stream);
}

int llama_layer_prefill_int8(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B, int32_t T,
                             void* k_codes, void* v_codes, float* k_scale, float* v_scale, void* stream) {
  g_last_error.clear();
  const int st = int8_args(L, k_scale, v_scale);
  return st != LLAMA_OK ? st
                        : int8_call(L, x, y, positions, B, T, contiguous_kv(L, k_codes, v_codes), k_scale, v_scale,
                                    stream);
}

int llama_layer_decode_int8(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B,
                            void* k_codes, void* v_codes, float* k_scale, float* v_scale, void* stream) {
  g_last_error.clear();
  const int st = int8_args(L, k_scale, v_scale);
  return st != LLAMA_OK ? st
                        : int8_call(L, x, y, positions, B, 1, contiguous_kv(L, k_codes, v_codes), k_scale, v_scale,
                                    stream);
}

int llama_layer_prefill_paged_int8(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B,
                                   int32_t T, void* k_pages, void* v_pages, float* k_scale_pages,
                                   float* v_scale_pages, const int32_t* block_table, int32_t blocks_per_seq,
                                   int32_t page_size, int32_t n_pages, void* stream) {
  g_last_error.clear();
  KvArgs kv{};
  int st = int8_args(L, k_scale_pages, v_scale_pages);
  if (st == LLAMA_OK) st = paged_kv(L, k_pages, v_pages, block_table, blocks_per_seq, page_size, n_pages, &kv);
  return st != LLAMA_OK ? st : int8_call(L, x, y, positions, B, T, kv, k_scale_pages, v_scale_pages, stream);
}

int llama_layer_decode_paged_int8(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B,
                                  void* k_pages, void* v_pages, float* k_scale_pages, float* v_scale_pages,
                                  const int32_t* block_table, int32_t blocks_per_seq, int32_t page_size,
                                  int32_t n_pages, void* stream) {
  g_last_error.clear();
  KvArgs kv{};
  int st = int8_args(L, k_scale_pages, v_scale_pages);
  if (st == LLAMA_OK) st = paged_kv(L, k_pages, v_pages, block_table, blocks_per_seq, page_size, n_pages, &kv);
  return st != LLAMA_OK ? st : int8_call(L, x, y, positions, B, 1, kv, k_scale_pages, v_scale_pages, stream);
}

int llama_layer_prefill_paged(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B, int32_t T,
                              void* k_pages, void* v_pages, const int32_t* block_table, int32_t blocks_per_seq,
                              int32_t page_size, int32_t n_pages, void* stream) {
  g_last_error.clear();
  KvArgs kv{};
  const int st = paged_kv(L, k_pages, v_pages, block_table, blocks_per_seq, page_size, n_pages, &kv);
  return st != LLAMA_OK ? st : checked_call(L, x, y, positions, B, T, kv, stream);
}

int llama_layer_decode_paged(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B,
                             void* k_pages, void* v_pages, const int32_t* block_table, int32_t blocks_per_seq,
                             int32_t page_size, int32_t n_pages, void* stream) {
  g_last_error.clear();
  KvArgs kv{};
  const int st = paged_kv(L, k_pages, v_pages, block_table, blocks_per_seq, page_size, n_pages, &kv);
  return st != LLAMA_OK ? st : checked_call(L, x, y, positions, B, 1, kv, stream);
}

int llama_layer_decode_noalloc(llama_layer* L, const void* x, void* y, const int32_t* positions, int32_t B,
                               void* k_cache, void* v_cache, void* stream) {
  g_last_error.clear();
  if (!L || !x || !y || !positions || !k_cache || !v_cache)
    return fail(LLAMA_ERR_NULL, "layer, x, y, positions and caches must be non-null");
  const llama_layer_config& c = L->cfg;
  if (c.dtype != LLAMA_BF16) return fail(LLAMA_ERR_UNSUPPORTED, "the allocation-free decode serves bf16 layers");
  if (B < 1) return fail(LLAMA_ERR_INVALID, "B must be >= 1 (got %d)", B);
  if (B > kNoAllocMaxSeqs)
    return fail(LLAMA_ERR_CAPACITY, "the allocation-free decode takes at most %d sequences (got %d)",
                kNoAllocMaxSeqs, B);
  if (!aligned16(x) || !aligned16(y) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(LLAMA_ERR_INVALID, "x, y and the caches must be 16-byte aligned");
  // slices of the static array, 256-byte aligned; activations in fragment
  // order hold whole 32-row blocks, i.e. 64 rows
  const size_t d = c.d_model, nq = static_cast<size_t>(c.n_heads) * 128, f = c.d_ff;
  const size_t nkv = static_cast<size_t>(c.n_kv_heads) * 128, rows = kNoAllocMaxSeqs;
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~static_cast<size_t>(255);
    return at;
  };
  const size_t o_xn = take(rows * d * 2), o_q = take(rows * nq * 2), o_o = take(rows * nq * 2),
               o_x1 = take(rows * d * 4), o_h = take(rows * f * 2);
  const int ns = decode_attn_splits(c.max_pos, B, c.n_heads, c.n_kv_heads);
  const size_t o_part = take(static_cast<size_t>(B) * c.n_heads * ns * 130 * sizeof(float));
  const int g_max = std::min(device_cu_count(), kSkinnyGrid);
  const size_t sk_floats = static_cast<size_t>(2) * g_max * 2 * (B <= 32 ? 1 : 2) * 1024;
  const size_t o_skp = take(sk_floats * sizeof(float));
  const size_t groups = std::max({(nq + 2 * nkv) / 32, 2 * f / 64, d / 32});
  const size_t o_cnt = take(groups * sizeof(unsigned));
  if (off > kNoAllocScratchBytes)
    return fail(LLAMA_ERR_CAPACITY, "this call needs %zu bytes of scratch; the static array holds %zu", off,
                kNoAllocScratchBytes);
  int cur = 0;
  HIP_OR_RETURN(hipGetDevice(&cur), "hipGetDevice");
  if (cur != L->device) HIP_OR_RETURN(hipSetDevice(L->device), "hipSetDevice");
  unsigned char* base = nullptr;
  int st = noalloc_scratch(L->device, &base);
  if (st == LLAMA_OK) {
    CallScratch S{};
    S.xn = base + o_xn;
    S.q = base + o_q;
    S.o = base + o_o;
    S.x1 = reinterpret_cast<float*>(base + o_x1);
    S.h = base + o_h;
    S.gu = nullptr;
    S.part = reinterpret_cast<float*>(base + o_part);
    S.part_seqs = B;
    S.sk.part = reinterpret_cast<float*>(base + o_skp);
    S.sk.part_len = sk_floats;
    S.sk.cnt = reinterpret_cast<unsigned*>(base + o_cnt);
    S.sk.cnt_len = static_cast<int>(groups);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int n = static_cast<int>(groups);
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, s, S.sk.cnt, n);
    const hipError_t e = hipGetLastError();
    st = e != hipSuccess ? hip_fail(e, "clear counters")
                         : run_layer(L, S, x, y, positions, B, 1, contiguous_kv(L, k_cache, v_cache), s);
  }
  if (cur != L->device) (void)hipSetDevice(cur);
  return st;
}

}  // extern "C"
