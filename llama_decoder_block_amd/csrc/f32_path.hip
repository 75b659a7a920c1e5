// fp32 decoder layer for any shape (small layers; no tiling or MFMA).  Same
// computation and sources as the bf16 path: "LMDrive LLM core inference unit"
// page §2.1-§2.5 and the "LLM mechanics lecture notes" Ch.02 (block equation,
// causal mask before the softmax, RoPE, RMSNorm, SwiGLU) and Ch.04 (KV cache).
// Everything stays in fp32; nothing is rounded to a narrower type.
#include "common.h"

#include <math.h>

namespace llama {
namespace {

// out[m, n] = sum_k A[m, k] W[n, k] (+ resid[m, n])
__global__ void f32_gemm_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                const float* __restrict__ resid, float* __restrict__ out, int M,
                                int N, int K) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(M) * N) return;
  const int m = static_cast<int>(i / N), n = static_cast<int>(i % N);
  const float* a = A + static_cast<size_t>(m) * K;
  const float* w = W + static_cast<size_t>(n) * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], w[k], s);
  if (resid) s += resid[i];
  out[i] = s;
}

// qkv [M, (H + 2 Hkv) dh] -> q (RoPE, in place) and rotated k / raw v into the caches
__global__ void f32_rope_scatter_kernel(float* __restrict__ qkv, float* __restrict__ k_cache,
                                        float* __restrict__ v_cache, const int32_t* __restrict__ pos,
                                        const float* __restrict__ cosb, const float* __restrict__ sinb,
                                        int T, int H, int Hkv, int dh, int max_pos) {
  const int m = blockIdx.x;
  const int half = dh / 2;
  const int width = (H + 2 * Hkv) * dh;
  float* row = qkv + static_cast<size_t>(m) * width;
  const int p = pos[m];
  const bool in_range = p >= 0 && p < max_pos;
  const int b = m / T;
  // rotate q and k heads
  for (int i = threadIdx.x; i < (H + Hkv) * half; i += blockDim.x) {
    const int head = i / half, e = i % half;
    float* x = row + head * dh;
    const float c = in_range ? cosb[static_cast<size_t>(p) * half + e] : 1.f;
    const float s = in_range ? sinb[static_cast<size_t>(p) * half + e] : 0.f;
    const float x1 = x[e], x2 = x[e + half];
    x[e] = x1 * c - x2 * s;
    x[e + half] = x2 * c + x1 * s;
  }
  __syncthreads();
  if (!in_range) return;
  for (int i = threadIdx.x; i < Hkv * dh; i += blockDim.x) {
    const int g = i / dh, e = i % dh;
    const size_t slot = (static_cast<size_t>(b * Hkv + g) * max_pos + p) * dh + e;
    k_cache[slot] = row[(H + g) * dh + e];
    v_cache[slot] = row[(H + Hkv + g) * dh + e];
  }
}

// one wavefront per (token, query head); bidir: the token sees every slot up
// to its sequence's largest position in the call, not only up to its own
__global__ __launch_bounds__(64) void f32_attention_kernel(const float* __restrict__ qkv,
                                                           const float* __restrict__ k_cache,
                                                           const float* __restrict__ v_cache,
                                                           const int32_t* __restrict__ pos,
                                                           float* __restrict__ o, int T, int H,
                                                           int Hkv, int dh, int max_pos, int bidir) {
  const int m = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int g = h / (H / Hkv);
  const int b = m / T;
  const float* q = qkv + static_cast<size_t>(m) * (H + 2 * Hkv) * dh + h * dh;
  int lim = pos[m];
  if (bidir) {
    for (int t = lane; t < T; t += 64) lim = max(lim, pos[b * T + t]);
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) lim = max(lim, __shfl_xor(lim, sft, 64));
  }
  const int p = min(lim, max_pos - 1);
  const float* K = k_cache + static_cast<size_t>(b * Hkv + g) * max_pos * dh;
  const float* V = v_cache + static_cast<size_t>(b * Hkv + g) * max_pos * dh;
  const float scale = 1.f / sqrtf(static_cast<float>(dh));
  auto score = [&](int j) {
    float s = 0.f;
    for (int e = lane; e < dh; e += 64) s = fmaf(q[e], K[static_cast<size_t>(j) * dh + e], s);
    return warp_sum(s) * scale;
  };
  float mx = -INFINITY;
  for (int j = 0; j <= p; ++j) mx = fmaxf(mx, score(j));
  float l = 0.f;
  constexpr int kMaxPerLane = 8;  // dh <= 512
  float acc[kMaxPerLane];
  for (int i = 0; i < kMaxPerLane; ++i) acc[i] = 0.f;
  for (int j = 0; j <= p; ++j) {
    const float e = expf(score(j) - mx);
    l += e;
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int d = lane + 64 * i;
      if (d < dh) acc[i] = fmaf(e, V[static_cast<size_t>(j) * dh + d], acc[i]);
    }
  }
  float* out = o + static_cast<size_t>(m) * H * dh + h * dh;
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int d = lane + 64 * i;
    if (d < dh) out[d] = p >= 0 ? acc[i] / l : 0.f;
  }
}

// gu [M, 2f] = [gate | up] -> h [M, f]
__global__ void f32_swiglu_kernel(const float* __restrict__ gu, float* __restrict__ h, int M, int f) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<long long>(M) * f) return;
  const int m = static_cast<int>(i / f), j = static_cast<int>(i % f);
  const float g = gu[static_cast<size_t>(m) * 2 * f + j];
  const float u = gu[static_cast<size_t>(m) * 2 * f + f + j];
  h[i] = g / (1.f + expf(-g)) * u;
}

hipError_t gemm(const float* A, const float* W, const float* resid, float* out, int M, int N, int K,
                hipStream_t s) {
  const long long n = static_cast<long long>(M) * N;
  hipLaunchKernelGGL(f32_gemm_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     A, W, resid, out, M, N, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_f32_gemm(const float* A, const float* W, const float* resid, float* out, int M, int N, int K,
                           hipStream_t s) {
  return gemm(A, W, resid, out, M, N, K, s);
}

hipError_t run_f32_layer(const F32Layer& L, const float* x, float* y, const int32_t* pos, int B,
                         int T, float* k_cache, float* v_cache, hipStream_t s) {
  const int M = B * T;
  const int nqkv = (L.H + 2 * L.Hkv) * L.dh;
  hipError_t e;
#define LLAMA_TRY(expr) \
  if ((e = (expr)) != hipSuccess) return e
  LLAMA_TRY(launch_rmsnorm(x, 1, L.g1, 1, L.xn, 1, 0, M, L.d, L.eps, s));
  LLAMA_TRY(gemm(L.xn, L.wqkv, nullptr, L.qkv, M, nqkv, L.d, s));
  hipLaunchKernelGGL(f32_rope_scatter_kernel, dim3(M), dim3(256), 0, s, L.qkv, k_cache, v_cache, pos,
                     L.rope_cos, L.rope_sin, T, L.H, L.Hkv, L.dh, L.max_pos);
  LLAMA_TRY(hipGetLastError());
  hipLaunchKernelGGL(f32_attention_kernel, dim3(M, L.H), dim3(64), 0, s, L.qkv, k_cache, v_cache, pos,
                     L.attn, T, L.H, L.Hkv, L.dh, L.max_pos, L.bidir);
  LLAMA_TRY(hipGetLastError());
  LLAMA_TRY(gemm(L.attn, L.wo, x, L.x1, M, L.d, L.H * L.dh, s));
  LLAMA_TRY(launch_rmsnorm(L.x1, 1, L.g2, 1, L.xn, 1, 0, M, L.d, L.eps, s));
  LLAMA_TRY(gemm(L.xn, L.wgu, nullptr, L.gu, M, 2 * L.f, L.d, s));
  {
    const long long n = static_cast<long long>(M) * L.f;
    hipLaunchKernelGGL(f32_swiglu_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                       L.gu, L.h, M, L.f);
    LLAMA_TRY(hipGetLastError());
  }
  LLAMA_TRY(gemm(L.h, L.wd, L.x1, y, M, L.d, L.f, s));
#undef LLAMA_TRY
  return hipSuccess;
}

}  // namespace llama
