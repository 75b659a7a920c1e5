// The generation stack around the decoder layer: token embedding, L layers,
// final RMSNorm, LM head, the sampling step and a native generation loop
// (the C ABI in include/llama_model.h).
//
// Sources: "LLM mechanics lecture notes" Ch.02 (X_0 = E[ids], L pre-norm
// blocks, [B,T,V] logits, generation reads the last position), Ch.04
// (prefill fills every layer's cache, decode feeds one token per sequence),
// Ch.05 (temperature, greedy as an explicit argmax, the top-p nucleus, the
// sign-aware repetition penalty, EOS as a per-row stop, max tokens, the
// end-to-end loop); "LMDrive LLM core inference unit" page §2.1 (RMSNorm).
//
// gfx950 design.
//   * The logits are needed for the last position of each sequence only:
//     those B <= 128 rows are gathered, normalised into fragment order and
//     multiplied by the LM head with the weight-streaming GEMM (its fp32
//     epilogue); the LM head rows are padded to a multiple of 128 at create.
//   * Sampling runs one 1024-thread workgroup per row and never writes the
//     logits: the penalty is applied on the fly through an LDS bitmap of the
//     penalised ids (deduplicated with atomic ORs), probabilities are
//     recomputed from the logits in every pass (they stay in L2), and every
//     reduction walks fixed contiguous chunks in a fixed tree, so the result
//     is deterministic.  The nucleus is found without a sort: a bisection on
//     the bit pattern of a probability threshold t finds the largest t whose
//     mass sum(p_i >= t) reaches top_p * sum(p); tokens above t are in, and of
//     the tokens equal to t the smallest ids are taken until the mass is
//     reached — exactly the descending-probability prefix with ties by id.
//     The draw is an inverse CDF in ascending id over the nucleus (a block
//     prefix sum over the chunks).
//   * The loop keeps each row's state (generated ids, count, finished) on
//     the device; the sampling kernel updates it, and the host reads the
//     finished flags once per step to stop early.
#include "common.h"
#include "../../include/llama_model.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

using namespace llama;

namespace {

#define MODEL_HIP(expr, what)                                                   \
  do {                                                                          \
    hipError_t e_ = (expr);                                                     \
    if (e_ != hipSuccess) return set_error(LLAMA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)

constexpr int kMaxRows = kSkinnyMaxTokens;  // logits rows per call
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / 64;
constexpr int kMaxVocab = 1 << 20;

// ---------------------------------------------------------------- small kernels

// x[n, :] = table[ids[n], :] (zeros for an id outside [0, V))
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ table, const int32_t* __restrict__ ids,
                                                    T* __restrict__ x, int d, int vocab) {
  const int n = blockIdx.x;
  const int id = ids[n];
  const bool ok = id >= 0 && id < vocab;
  const T* src = table + static_cast<size_t>(ok ? id : 0) * d;
  T* dst = x + static_cast<size_t>(n) * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) dst[i] = ok ? src[i] : T(0);
}

// last[b, :] = x[b*T + T-1, :]
template <typename T>
__global__ __launch_bounds__(256) void gather_last_kernel(const T* __restrict__ x, T* __restrict__ last, int T_,
                                                          int d) {
  const int b = blockIdx.x;
  const T* src = x + (static_cast<size_t>(b) * T_ + T_ - 1) * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) last[static_cast<size_t>(b) * d + i] = src[i];
}

__global__ void positions_kernel(int32_t* __restrict__ pos, int n, int T_) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) pos[i] = i % T_;
}

// ---------------------------------------------------------------- sampling

struct SampleArgs {
  const float* logits;
  int vocab, ld;
  float temperature, top_p, penalty;
  const int32_t* hist;  // [B, hist_ld]
  const int32_t* hist_len;
  int hist_ld;
  const float* uniforms;
  int32_t* out;
  // generation state (nullable): the sampled id is appended to hist[b] unless
  // it is eos_id or the row is finished; a row finishes at eos_id or when its
  // count reaches max_len
  int32_t* gen_hist;
  int32_t* gen_len;
  int32_t* done;
  int eos_id, max_len;
};

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < kSampleWaves; ++i) t += red[i];  // fixed order
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < kSampleWaves; ++i) t = fmaxf(t, red[i]);
  return t;
}

__device__ __forceinline__ int block_max_int(int v, int* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = max(v, __shfl_xor(v, s, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int t = INT32_MIN;
  for (int i = 0; i < kSampleWaves; ++i) t = max(t, red[i]);
  return t;
}

// exclusive prefix over the block's threads (in thread order) and the total
__device__ __forceinline__ float block_exclusive_scan(float v, float* red, float& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float inc = v;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const float o = __shfl_up(inc, s, 64);
    if (lane >= s) inc += o;
  }
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  float before = 0.f;
  total = 0.f;
  for (int i = 0; i < kSampleWaves; ++i) {
    if (i < w) before += red[i];
    total += red[i];
  }
  return before + inc - v;
}

__device__ __forceinline__ int block_exclusive_scan_int(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int o = __shfl_up(inc, s, 64);
    if (lane >= s) inc += o;
  }
  __syncthreads();
  if (lane == 63) red[w] = inc;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += red[i];
  return before + inc - v;
}

// one workgroup per row; dynamic LDS: the penalty bitmap, ceil(V / 32) words
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleArgs a) {
  extern __shared__ unsigned pen_bits[];
  __shared__ float redf[kSampleWaves];
  __shared__ int redi[kSampleWaves];
  __shared__ int s_pick;
  __shared__ float s_before[kSampleThreads];
  const int b = blockIdx.x, t = threadIdx.x;
  if (a.done && a.done[b]) return;  // uniform per workgroup
  const int V = a.vocab;
  const float* z = a.logits + static_cast<size_t>(b) * a.ld;
  const int words = (V + 31) >> 5;

  // penalised ids: the distinct generated ids (history)
  const bool use_pen = a.penalty != 1.f && a.hist != nullptr;
  if (use_pen) {
    for (int i = t; i < words; i += kSampleThreads) pen_bits[i] = 0u;
    __syncthreads();
    const int n = a.hist_len[b];
    for (int i = t; i < n; i += kSampleThreads) {
      const int id = a.hist[static_cast<size_t>(b) * a.hist_ld + i];
      if (id >= 0 && id < V) atomicOr(&pen_bits[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
  }
  auto val = [&](int i) {
    const float zi = z[i];
    if (use_pen && ((pen_bits[i >> 5] >> (i & 31)) & 1u)) return zi > 0.f ? zi / a.penalty : zi * a.penalty;
    return zi;
  };
  // thread t owns the contiguous ids [c0, c1)
  const int chunk = (V + kSampleThreads - 1) / kSampleThreads;
  const int c0 = min(t * chunk, V), c1 = min(c0 + chunk, V);

  int pick;
  if (a.temperature == 0.f) {
    // greedy: the largest value, the smallest id among equals
    float bv = -INFINITY;
    int bi = INT32_MAX;
    for (int i = c0; i < c1; ++i) {
      const float v = val(i);
      if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
    }
    const float mx = block_max(bv, redf);
    pick = -block_max_int(bv == mx ? -bi : INT32_MIN, redi);
  } else {
    float lm = -INFINITY;
    for (int i = c0; i < c1; ++i) lm = fmaxf(lm, val(i));
    const float mx = block_max(lm, redf);
    const float k = 1.4426950408889634f / a.temperature;  // exp(x / tau) = 2^(x log2(e) / tau)
    auto prob = [&](int i) { return exp2f((val(i) - mx) * k); };
    float ls = 0.f;
    for (int i = c0; i < c1; ++i) ls += prob(i);
    const float S = block_sum(ls, redf);

    // nucleus: threshold t* and the number of ties at t* taken (smallest ids)
    float thr = 0.f;   // members: p > thr, plus the first n_tie ids with p == thr
    int n_tie = 0;
    float Z = S;       // nucleus mass
    if (a.top_p < 1.f) {
      const float target = a.top_p * S;
      auto mass_ge = [&](float th) {
        float m = 0.f;
        for (int i = c0; i < c1; ++i) {
          const float p = prob(i);
          if (p >= th) m += p;
        }
        return block_sum(m, redf);
      };
      uint32_t lo = 0u, hi = 0x7f800000u;  // mass(lo) >= target > mass(hi) = 0
      while (hi - lo > 1u) {
        const uint32_t mid = lo + (hi - lo) / 2u;
        if (mass_ge(__uint_as_float(mid)) >= target) lo = mid; else hi = mid;
      }
      thr = __uint_as_float(lo);
      // mass strictly above the threshold (below target), and how many of the
      // tokens equal to it complete the prefix
      float mg = 0.f;
      for (int i = c0; i < c1; ++i) {
        const float p = prob(i);
        if (p > thr) mg += p;
      }
      const float above = block_sum(mg, redf);
      if (thr > 0.f) n_tie = max(1, static_cast<int>(ceilf((target - above) / thr - 1e-4f)));
      Z = above + static_cast<float>(n_tie) * thr;
    }
    // inverse CDF in ascending id over the members
    const bool nucleus = a.top_p < 1.f;
    int tie_before = 0;
    if (nucleus) {
      int ties_here = 0;
      for (int i = c0; i < c1; ++i) ties_here += prob(i) == thr ? 1 : 0;
      tie_before = block_exclusive_scan_int(ties_here, redi);
    }
    auto member = [&](float p, int& tie_rank) {
      if (!nucleus) return true;
      if (p > thr) return true;
      if (p == thr) return tie_rank++ < n_tie;
      return false;
    };
    float mine = 0.f;
    int last_member = -1;
    {
      int tr = tie_before;
      for (int i = c0; i < c1; ++i) {
        const float p = prob(i);
        if (member(p, tr)) { mine += p; last_member = i; }
      }
    }
    float total;
    const float before = block_exclusive_scan(mine, redf, total);
    (void)total;
    const float u = a.uniforms ? a.uniforms[b] : 0.f;
    const float r = u * Z;
    // the chunks' intervals [before_t, before_t+1) partition [0, inf) exactly
    // (the last one is open): exactly one thread owns r
    s_before[t] = before;
    if (t == 0) s_pick = -1;
    __syncthreads();
    const float end = t + 1 < kSampleThreads ? s_before[t + 1] : INFINITY;
    if (r >= before && r < end) {
      float run = before;
      int tr = tie_before;
      int found = last_member;  // past the chunk's rounded sum: its last member
      for (int i = c0; i < c1; ++i) {
        const float p = prob(i);
        if (member(p, tr)) {
          run += p;
          if (run > r) { found = i; break; }
        }
      }
      s_pick = found;
    }
    __syncthreads();
    pick = s_pick;
    if (pick < 0) pick = block_max_int(last_member, redi);  // an empty last chunk: the last member
  }
  if (t == 0) {
    a.out[b] = pick;
    if (a.done) {
      const int n = a.gen_len[b];
      if (pick == a.eos_id) {
        a.done[b] = 1;
      } else {
        a.gen_hist[static_cast<size_t>(b) * a.hist_ld + n] = pick;
        a.gen_len[b] = n + 1;
        if (n + 1 >= a.max_len) a.done[b] = 1;
      }
    }
  }
}

int check_sampling(const llama_sampling* p, int vocab) {
  if (!p) return set_error(LLAMA_ERR_NULL, "sampling parameters must be non-null");
  if (vocab < 2 || vocab > kMaxVocab) return set_error(LLAMA_ERR_INVALID, "vocab must be in [2, 2^20] (got %d)", vocab);
  if (!(p->temperature >= 0.f) || !isfinite(p->temperature))
    return set_error(LLAMA_ERR_INVALID, "temperature must be finite and >= 0");
  if (!(p->top_p > 0.f && p->top_p <= 1.f)) return set_error(LLAMA_ERR_INVALID, "top_p must be in (0, 1]");
  if (!(p->repetition_penalty >= 1.f) || !isfinite(p->repetition_penalty))
    return set_error(LLAMA_ERR_INVALID, "repetition_penalty must be finite and >= 1");
  return LLAMA_OK;
}

hipError_t launch_sample(const SampleArgs& a, int B, hipStream_t s) {
  const size_t lds = static_cast<size_t>((a.vocab + 31) / 32) * sizeof(unsigned);
  hipLaunchKernelGGL(sample_kernel, dim3(B), dim3(kSampleThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------- the handle

struct llama_model {
  llama_model_config cfg;
  int device = 0;
  size_t es = 2;
  int Vp = 0;  // LM head rows, padded to a multiple of 128 (bf16)
  std::vector<llama_layer*> layers;
  void* embed = nullptr;       // [V, d]
  void* final_norm = nullptr;  // [d]
  void* lm = nullptr;          // bf16: [Vp, d] fragment order; fp32: [V, d] row-major
  void* x = nullptr;           // [max_tokens, d] activations between layers (in place)
  void* last = nullptr;        // [64, d] last positions
  void* xn = nullptr;          // [64, d] normalised last positions (bf16: fragment order)
  int32_t* ids = nullptr;      // [max_tokens]
  int32_t* pos = nullptr;      // [max_tokens]
  SkinnyScratch sk{};
};

namespace {

void release(llama_model* m) {
  for (llama_layer* l : m->layers) llama_layer_destroy(l);
  void* bufs[] = {m->embed, m->final_norm, m->lm, m->x, m->last, m->xn, m->ids, m->pos, m->sk.part, m->sk.cnt};
  for (void* p : bufs)
    if (p) (void)hipFree(p);
}

int dev_alloc(void** p, size_t bytes) {
  if (hipMalloc(p, bytes ? bytes : 16) != hipSuccess) {
    *p = nullptr;
    return set_error(LLAMA_ERR_ALLOC, "device allocation of %zu bytes failed", bytes);
  }
  return LLAMA_OK;
}

// embedding, the layers' prefill or decode, the last rows, final norm, LM head
int run_stack(llama_model* m, int B, int T, const int32_t* pos, void* const* kc, void* const* vc, float* logits,
              hipStream_t s) {
  const llama_layer_config& c = m->cfg.layer;
  const int d = c.d_model, V = m->cfg.vocab, M = B * T;
  const bool bf = c.dtype == LLAMA_BF16;
  if (bf)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(M), dim3(256), 0, s, static_cast<const bf16_t*>(m->embed),
                       m->ids, static_cast<bf16_t*>(m->x), d, V);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, s, static_cast<const float*>(m->embed), m->ids,
                       static_cast<float*>(m->x), d, V);
  MODEL_HIP(hipGetLastError(), "embedding");
  for (int l = 0; l < m->cfg.n_layers; ++l) {
    if (!kc[l] || !vc[l]) return set_error(LLAMA_ERR_NULL, "cache pointers of layer %d are null", l);
    const int st = T == 1 ? llama_layer_decode(m->layers[l], m->x, m->x, pos, B, kc[l], vc[l], s)
                          : llama_layer_prefill(m->layers[l], m->x, m->x, pos, B, T, kc[l], vc[l], s);
    if (st != LLAMA_OK) return st;
  }
  const void* last = m->x;
  if (T > 1) {
    if (bf)
      hipLaunchKernelGGL(gather_last_kernel<bf16_t>, dim3(B), dim3(256), 0, s, static_cast<const bf16_t*>(m->x),
                         static_cast<bf16_t*>(m->last), T, d);
    else
      hipLaunchKernelGGL(gather_last_kernel<float>, dim3(B), dim3(256), 0, s, static_cast<const float*>(m->x),
                         static_cast<float*>(m->last), T, d);
    MODEL_HIP(hipGetLastError(), "gather last positions");
    last = m->last;
  }
  if (bf) {
    MODEL_HIP(launch_rmsnorm(last, 0, m->final_norm, 0, m->xn, 0, 1, B, d, c.rms_eps, s), "final RMSNorm");
    MODEL_HIP(launch_skinny_f32out(static_cast<const bf16_t*>(m->xn), static_cast<const bf16_t*>(m->lm), B, m->Vp,
                                   d, logits, V, V, m->sk, s),
              "LM head");
  } else {
    MODEL_HIP(launch_rmsnorm(last, 1, m->final_norm, 1, m->xn, 1, 0, B, d, c.rms_eps, s), "final RMSNorm");
    MODEL_HIP(launch_f32_gemm(static_cast<const float*>(m->xn), static_cast<const float*>(m->lm), nullptr, logits,
                              B, V, d, s),
              "LM head");
  }
  return LLAMA_OK;
}

int check_call(llama_model* m, int B, int T, void* const* kc, void* const* vc, const float* logits) {
  if (!m || !kc || !vc || !logits) return set_error(LLAMA_ERR_NULL, "model, caches and logits must be non-null");
  if (B < 1 || T < 1) return set_error(LLAMA_ERR_INVALID, "B and T must be >= 1 (got %d, %d)", B, T);
  if (B > kMaxRows) return set_error(LLAMA_ERR_CAPACITY, "at most %d sequences per call (got %d)", kMaxRows, B);
  if (static_cast<long long>(B) * T > m->cfg.layer.max_tokens)
    return set_error(LLAMA_ERR_CAPACITY, "B*T = %lld exceeds max_tokens = %d", static_cast<long long>(B) * T,
                     m->cfg.layer.max_tokens);
  if (T > m->cfg.layer.max_pos) return set_error(LLAMA_ERR_CAPACITY, "T = %d exceeds max_pos", T);
  return LLAMA_OK;
}

}  // namespace

extern "C" {

int llama_model_create(const llama_model_config* cfg, const llama_model_weights* w, void* stream,
                       llama_model** out) {
  set_error(LLAMA_OK, "");
  if (!cfg || !w || !out || !w->embed || !w->final_norm || !w->lm_head || !w->layers)
    return set_error(LLAMA_ERR_NULL, "cfg, weights (embed, final_norm, lm_head, layers) and out must be non-null");
  *out = nullptr;
  if (cfg->n_layers < 1) return set_error(LLAMA_ERR_INVALID, "n_layers must be >= 1");
  if (cfg->vocab < 2 || cfg->vocab > kMaxVocab) return set_error(LLAMA_ERR_INVALID, "vocab must be in [2, 2^20]");
  hipStream_t s = static_cast<hipStream_t>(stream);
  llama_model* m = new (std::nothrow) llama_model();
  if (!m) return set_error(LLAMA_ERR_ALLOC, "host allocation failed");
  m->cfg = *cfg;
  const llama_layer_config& c = cfg->layer;
  m->es = c.dtype == LLAMA_BF16 ? 2 : 4;
#define MODEL_FAIL(st)  \
  do {                  \
    release(m);         \
    delete m;           \
    return (st);        \
  } while (0)
#define MODEL_HIP_FAIL(expr, what)                                                        \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) MODEL_FAIL(set_error(LLAMA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_))); \
  } while (0)
#define MODEL_ALLOC(ptr, bytes)                                   \
  do {                                                            \
    int a_ = dev_alloc(reinterpret_cast<void**>(&(ptr)), (bytes)); \
    if (a_ != LLAMA_OK) MODEL_FAIL(a_);                           \
  } while (0)
  MODEL_HIP_FAIL(hipGetDevice(&m->device), "hipGetDevice");
  for (int l = 0; l < cfg->n_layers; ++l) {
    llama_layer* L = nullptr;
    const int st = llama_layer_create(&c, &w->layers[l], stream, &L);
    if (st != LLAMA_OK) MODEL_FAIL(st);
    m->layers.push_back(L);
  }
  const size_t d = c.d_model, V = cfg->vocab, es = m->es;
  const bool bf = c.dtype == LLAMA_BF16;
  m->Vp = bf ? static_cast<int>((V + 127) / 128 * 128) : static_cast<int>(V);
  MODEL_ALLOC(m->embed, V * d * es);
  MODEL_ALLOC(m->final_norm, d * es);
  MODEL_ALLOC(m->lm, static_cast<size_t>(m->Vp) * d * es);
  MODEL_ALLOC(m->x, static_cast<size_t>(c.max_tokens) * d * es);
  MODEL_ALLOC(m->last, kMaxRows * d * es);
  MODEL_ALLOC(m->xn, kMaxRows * d * es);
  MODEL_ALLOC(m->ids, static_cast<size_t>(c.max_tokens) * sizeof(int32_t));
  MODEL_ALLOC(m->pos, static_cast<size_t>(c.max_tokens) * sizeof(int32_t));
  const hipMemcpyKind dd = hipMemcpyDeviceToDevice;
  MODEL_HIP_FAIL(hipMemcpyAsync(m->embed, w->embed, V * d * es, dd, s), "copy embedding");
  MODEL_HIP_FAIL(hipMemcpyAsync(m->final_norm, w->final_norm, d * es, dd, s), "copy final norm");
  if (bf) {
    // zero-padded row-major copy, then fragment order for the streaming GEMM
    void* tmp = nullptr;
    MODEL_ALLOC(tmp, static_cast<size_t>(m->Vp) * d * es);
    hipError_t e = hipMemsetAsync(tmp, 0, static_cast<size_t>(m->Vp) * d * es, s);
    if (e == hipSuccess) e = hipMemcpyAsync(tmp, w->lm_head, V * d * es, dd, s);
    if (e == hipSuccess)
      e = launch_pack_rows(static_cast<const bf16_t*>(tmp), m->Vp, static_cast<int>(d), static_cast<bf16_t*>(m->lm),
                           m->Vp, m->Vp, 0, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)hipFree(tmp);
    MODEL_HIP_FAIL(e, "convert LM head");
    MODEL_ALLOC(m->sk.part, skinny_scratch_floats() * sizeof(float));
    const size_t groups = static_cast<size_t>(m->Vp) / 32;
    MODEL_ALLOC(m->sk.cnt, groups * sizeof(unsigned));
    m->sk.cnt_len = static_cast<int>(groups);
    m->sk.part_len = skinny_scratch_floats();
    MODEL_HIP_FAIL(hipMemsetAsync(m->sk.cnt, 0, groups * sizeof(unsigned), s), "clear counters");
  } else {
    MODEL_HIP_FAIL(hipMemcpyAsync(m->lm, w->lm_head, V * d * es, dd, s), "copy LM head");
  }
  MODEL_HIP_FAIL(hipStreamSynchronize(s), "create");
#undef MODEL_ALLOC
#undef MODEL_HIP_FAIL
#undef MODEL_FAIL
  *out = m;
  return LLAMA_OK;
}

void llama_model_destroy(llama_model* m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  release(m);
  delete m;
}

int llama_model_prefill(llama_model* m, const int32_t* ids, int32_t B, int32_t T, void* const* kc,
                        void* const* vc, float* logits, void* stream) {
  set_error(LLAMA_OK, "");
  int st = check_call(m, B, T, kc, vc, logits);
  if (st != LLAMA_OK) return st;
  if (!ids) return set_error(LLAMA_ERR_NULL, "ids must be non-null");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = B * T;
  MODEL_HIP(hipMemcpyAsync(m->ids, ids, M * sizeof(int32_t), hipMemcpyDeviceToDevice, s), "copy ids");
  hipLaunchKernelGGL(positions_kernel, dim3((M + 255) / 256), dim3(256), 0, s, m->pos, M, T);
  MODEL_HIP(hipGetLastError(), "positions");
  return run_stack(m, B, T, m->pos, kc, vc, logits, s);
}

int llama_model_decode(llama_model* m, const int32_t* ids, const int32_t* positions, int32_t B, void* const* kc,
                       void* const* vc, float* logits, void* stream) {
  set_error(LLAMA_OK, "");
  int st = check_call(m, B, 1, kc, vc, logits);
  if (st != LLAMA_OK) return st;
  if (!ids || !positions) return set_error(LLAMA_ERR_NULL, "ids and positions must be non-null");
  hipStream_t s = static_cast<hipStream_t>(stream);
  MODEL_HIP(hipMemcpyAsync(m->ids, ids, B * sizeof(int32_t), hipMemcpyDeviceToDevice, s), "copy ids");
  return run_stack(m, B, 1, positions, kc, vc, logits, s);
}

int llama_sample(const float* logits, int32_t B, int32_t vocab, int32_t ld, const llama_sampling* params,
                 const int32_t* history, const int32_t* history_len, int32_t history_ld, const float* uniforms,
                 int32_t* out_ids, void* stream) {
  set_error(LLAMA_OK, "");
  if (!logits || !out_ids) return set_error(LLAMA_ERR_NULL, "logits and out_ids must be non-null");
  int st = check_sampling(params, vocab);
  if (st != LLAMA_OK) return st;
  if (B < 1 || ld < vocab || history_ld < 0) return set_error(LLAMA_ERR_INVALID, "B >= 1, ld >= vocab, history_ld >= 0");
  if (params->temperature > 0.f && !uniforms) return set_error(LLAMA_ERR_NULL, "uniforms are needed when temperature > 0");
  if (params->repetition_penalty != 1.f && (!history || !history_len))
    return set_error(LLAMA_ERR_NULL, "history and history_len are needed with a repetition penalty");
  SampleArgs a{};
  a.logits = logits;
  a.vocab = vocab;
  a.ld = ld;
  a.temperature = params->temperature;
  a.top_p = params->top_p;
  a.penalty = params->repetition_penalty;
  a.hist = history;
  a.hist_len = history_len;
  a.hist_ld = history_ld;
  a.uniforms = uniforms;
  a.out = out_ids;
  MODEL_HIP(launch_sample(a, B, static_cast<hipStream_t>(stream)), "sampling");
  return LLAMA_OK;
}

int llama_model_generate(llama_model* m, const int32_t* prompt, int32_t B, int32_t T, int32_t max_new,
                         const llama_sampling* params, const float* uniforms, void* const* kc, void* const* vc,
                         int32_t* out_ids, int32_t* out_len, void* stream) {
  set_error(LLAMA_OK, "");
  if (!m || !prompt || !out_ids || !out_len || !kc || !vc)
    return set_error(LLAMA_ERR_NULL, "model, prompt, caches, out_ids and out_len must be non-null");
  int st = check_sampling(params, m ? m->cfg.vocab : 0);
  if (st != LLAMA_OK) return st;
  if (max_new < 1) return set_error(LLAMA_ERR_INVALID, "max_new must be >= 1");
  if (B < 1 || T < 1) return set_error(LLAMA_ERR_INVALID, "B and T must be >= 1");
  if (static_cast<long long>(T) + max_new > m->cfg.layer.max_pos)
    return set_error(LLAMA_ERR_INVALID, "T + max_new = %lld exceeds max_pos = %d",
                     static_cast<long long>(T) + max_new, m->cfg.layer.max_pos);
  if (params->temperature > 0.f && !uniforms) return set_error(LLAMA_ERR_NULL, "uniforms are needed when temperature > 0");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int V = m->cfg.vocab;
  // per-call device state: prompt, logits, history, counts, finished flags, ids, positions, uniforms
  int32_t *d_prompt = nullptr, *d_hist = nullptr, *d_len = nullptr, *d_done = nullptr, *d_ids = nullptr,
          *d_pos = nullptr;
  float *d_logits = nullptr, *d_u = nullptr;
  auto free_all = [&]() {
    void* ps[] = {d_prompt, d_hist, d_len, d_done, d_ids, d_pos, d_logits, d_u};
    for (void* p : ps)
      if (p) (void)hipFree(p);
  };
  const size_t nB = static_cast<size_t>(B);
  if (dev_alloc(reinterpret_cast<void**>(&d_prompt), nB * T * 4) || dev_alloc(reinterpret_cast<void**>(&d_hist), nB * max_new * 4) ||
      dev_alloc(reinterpret_cast<void**>(&d_len), nB * 4) || dev_alloc(reinterpret_cast<void**>(&d_done), nB * 4) ||
      dev_alloc(reinterpret_cast<void**>(&d_ids), nB * 4) || dev_alloc(reinterpret_cast<void**>(&d_pos), nB * 4) ||
      dev_alloc(reinterpret_cast<void**>(&d_logits), nB * V * 4) ||
      (uniforms && dev_alloc(reinterpret_cast<void**>(&d_u), nB * max_new * 4))) {
    free_all();
    return LLAMA_ERR_ALLOC;
  }
#define GEN_HIP(expr, what)                                                              \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) { free_all(); return set_error(LLAMA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); } \
  } while (0)
  GEN_HIP(hipMemcpyAsync(d_prompt, prompt, nB * T * 4, hipMemcpyHostToDevice, s), "copy prompt");
  if (uniforms) GEN_HIP(hipMemcpyAsync(d_u, uniforms, nB * max_new * 4, hipMemcpyHostToDevice, s), "copy uniforms");
  GEN_HIP(hipMemsetAsync(d_len, 0, nB * 4, s), "clear counts");
  GEN_HIP(hipMemsetAsync(d_done, 0, nB * 4, s), "clear flags");
  GEN_HIP(hipMemsetAsync(d_hist, 0xff, nB * max_new * 4, s), "clear history");
  st = llama_model_prefill(m, d_prompt, B, T, kc, vc, d_logits, stream);
  if (st != LLAMA_OK) { free_all(); return st; }
  std::vector<int32_t> done(nB, 0), pos_h(nB);
  for (int step = 0; step < max_new; ++step) {
    SampleArgs a{};
    a.logits = d_logits;
    a.vocab = V;
    a.ld = V;
    a.temperature = params->temperature;
    a.top_p = params->top_p;
    a.penalty = params->repetition_penalty;
    a.hist = d_hist;
    a.hist_len = d_len;
    a.hist_ld = max_new;
    a.uniforms = d_u ? d_u + static_cast<size_t>(step) * B : nullptr;
    a.out = d_ids;
    a.gen_hist = d_hist;
    a.gen_len = d_len;
    a.done = d_done;
    a.eos_id = params->eos_id;
    a.max_len = max_new;
    GEN_HIP(launch_sample(a, B, s), "sampling");
    GEN_HIP(hipMemcpyAsync(done.data(), d_done, nB * 4, hipMemcpyDeviceToHost, s), "read flags");
    GEN_HIP(hipStreamSynchronize(s), "sampling step");
    if (std::all_of(done.begin(), done.end(), [](int32_t v) { return v != 0; })) break;
    // the new tokens sit at position T + step (a finished row's slot is
    // written too, with whatever id it last had; its output is never read)
    for (size_t b = 0; b < nB; ++b) pos_h[b] = T + step;
    GEN_HIP(hipMemcpyAsync(d_pos, pos_h.data(), nB * 4, hipMemcpyHostToDevice, s), "copy positions");
    st = llama_model_decode(m, d_ids, d_pos, B, kc, vc, d_logits, stream);
    if (st != LLAMA_OK) { free_all(); return st; }
  }
  std::vector<int32_t> len(nB);
  GEN_HIP(hipMemcpyAsync(len.data(), d_len, nB * 4, hipMemcpyDeviceToHost, s), "read counts");
  GEN_HIP(hipMemcpyAsync(out_ids, d_hist, nB * max_new * 4, hipMemcpyDeviceToHost, s), "read tokens");
  GEN_HIP(hipStreamSynchronize(s), "generate");
  for (size_t b = 0; b < nB; ++b) out_len[b] = len[b];
#undef GEN_HIP
  free_all();
  return LLAMA_OK;
}

}  // extern "C"
