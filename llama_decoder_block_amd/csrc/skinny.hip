// Weight-streaming GEMMs for few tokens (decode: M = batch <= 64), with the
// same fused epilogues as the tiled prefill GEMMs (RoPE + cache append,
// residual adds, SwiGLU).  Sources as for the prefill projections: "LMDrive
// LLM core inference unit" page §2.3-§2.5, "Llama MLP deep dive" page §2.2,
// and the "LLM mechanics lecture notes" Ch.04 (decode reads every weight once
// per step and is memory bound).
//
// gfx950 design.  A workgroup owns 16 weight rows and all M tokens and runs
// v_mfma_f32_16x16x32_bf16 with the weight rows as the A operand (16 rows x
// 32 k) and the tokens as B (32 k x 16 tokens), so each lane streams 16
// bytes of one weight row per step straight from HBM into registers — no LDS
// staging, every weight byte read exactly once.  Eight wavefronts split K
// (round-robin 32-wide steps, 8 steps in flight per lane) and add their
// partial 16x16 tiles through LDS at the end.  The 16 rows are chosen per
// epilogue so that the pairs it needs sit in lanes l and l^32 of the
// accumulator layout: RoPE partners (dims i and i+64 of one head) and the
// gate/up pair (gate row j and up row j).  The activations (<= 64 x K bf16)
// are re-read by every workgroup but stay resident in L2.
#include "common.h"

namespace llama {
namespace {

enum { SK_QKV = 0, SK_RESID32 = 1, SK_RESID16 = 2, SK_SWIGLU = 3 };

constexpr int kWaves = 8;
constexpr int kUnroll = 8;

struct SkinnyArgs {
  QkvEpilogue qkv;
  const void* resid;
  void* out;
};

template <int TB, int EPI>
__global__ __launch_bounds__(kWaves * 64) void skinny_kernel(const bf16_t* __restrict__ X,
                                                              const bf16_t* __restrict__ W, int M,
                                                              int N, int K, SkinnyArgs ep) {
  __shared__ float red[kWaves][TB][64][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = blockIdx.x;
  const int lr = lane & 15;      // A row (weight row slot) / B column (token) of this lane
  const int kq = (lane >> 4) * 8;  // k offset of this lane inside a 32-wide step

  // weight row streamed by this lane (A operand row lr)
  int wrow;
  if constexpr (EPI == SK_QKV) {
    const int head = wg >> 3, j8 = wg & 7;
    wrow = head * 128 + (lr < 8 ? 8 * j8 + lr : 64 + 8 * j8 + (lr - 8));
  } else if constexpr (EPI == SK_SWIGLU) {
    const int c = wg * 8 + (lr & 7);  // h column
    wrow = (c >> 6) * 128 + (lr < 8 ? 0 : 64) + (c & 63);
  } else {
    wrow = wg * 16 + lr;
  }
  const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(W, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(X, static_cast<uint32_t>(M) * K * 2u);
  const uint32_t w_off = (static_cast<uint32_t>(wrow) * K + kq) * 2u;
  uint32_t x_off[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) x_off[tb] = (static_cast<uint32_t>(tb * 16 + lr) * K + kq) * 2u;

  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K / 32;
  for (int s0 = wave; s0 < nsteps; s0 += kWaves * kUnroll) {
    uint4 wv[kUnroll], xv[kUnroll][TB];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int st = s0 + u * kWaves;
      if (st < nsteps) {
        const uint32_t ko = static_cast<uint32_t>(st) * 64u;  // 32 bf16
        wv[u] = buf_load16(w_rs, w_off, ko);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) xv[u][tb] = buf_load16(x_rs, x_off[tb], ko);
      } else {
        wv[u] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) xv[u][tb] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[u]),
                                                          __builtin_bit_cast(bf16x8, xv[u][tb]),
                                                          acc[tb], 0, 0, 0);
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][tb][lane][e] = acc[tb][e];
  __syncthreads();
  if (wave != 0) return;

  // lane holds rows 4*(lane/16) + e, token tb*16 + lane%16
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) a += red[w][tb][lane][e];
      v[e] = a;
    }
    const int tok = tb * 16 + lr;
    const int rq = lane >> 4;  // row quad 0..3
    if constexpr (EPI == SK_QKV) {
      const QkvEpilogue& q = ep.qkv;
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = __shfl_xor(v[e], 32, 64);
      if (tok >= M) continue;
      const int head = wg >> 3, j8 = wg & 7;
      const int kind = head < q.n_heads ? 0 : (head < q.n_heads + q.n_kv_heads ? 1 : 2);
      const int hh = kind == 0 ? head : (kind == 1 ? head - q.n_heads : head - q.n_heads - q.n_kv_heads);
      const int p = q.pos[tok];
      const int pt = min(max(p, 0), q.max_pos - 1);
      const bool second = rq >= 2;  // rows 8..15: dims 64 + ...
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dd = 8 * j8 + 4 * (rq & 1) + e;  // first-half dim of the pair
        if (kind == 2) {
          o[e] = v[e];
        } else {
          const float c = q.rope_cos[static_cast<size_t>(pt) * 64 + dd];
          const float s = q.rope_sin[static_cast<size_t>(pt) * 64 + dd];
          const float x1 = second ? pv[e] : v[e];
          const float x2 = second ? v[e] : pv[e];
          o[e] = second ? x2 * c + x1 * s : x1 * c - x2 * s;
        }
      }
      const int d0 = (second ? 64 : 0) + 8 * j8 + 4 * (rq & 1);
      bf16_t* dst;
      if (kind == 0) {
        dst = q.q + static_cast<size_t>(tok) * q.n_heads * 128 + hh * 128 + d0;
      } else {
        if (p < 0 || p >= q.max_pos) continue;
        const int b = tok / q.T;
        bf16_t* cache = kind == 1 ? q.k_cache : q.v_cache;
        dst = cache + (static_cast<size_t>(b * q.n_kv_heads + hh) * q.max_pos + p) * 128 + d0;
      }
      uint2 w2;
      w2.x = pack_bf16x2(o[0], o[1]);
      w2.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<uint2*>(dst) = w2;
    } else if constexpr (EPI == SK_SWIGLU) {
      float up[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) up[e] = __shfl_xor(v[e], 32, 64);
      if (tok >= M || rq >= 2) continue;
      const int f = N;  // number of h columns
      const int c0 = wg * 8 + 4 * rq;
      uint2 w2;
      w2.x = pack_bf16x2(silu(v[0]) * up[0], silu(v[1]) * up[1]);
      w2.y = pack_bf16x2(silu(v[2]) * up[2], silu(v[3]) * up[3]);
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(ep.out) + static_cast<size_t>(tok) * f + c0) = w2;
    } else {
      if (tok >= M) continue;
      const int c0 = wg * 16 + 4 * rq;
      const size_t base = static_cast<size_t>(tok) * N + c0;
      if constexpr (EPI == SK_RESID32) {
        const uint2 r2 = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(ep.resid) + base);
        float4 o4 = make_float4(v[0] + lo_bf16(r2.x), v[1] + hi_bf16(r2.x), v[2] + lo_bf16(r2.y),
                                v[3] + hi_bf16(r2.y));
        *reinterpret_cast<float4*>(static_cast<float*>(ep.out) + base) = o4;
      } else {
        const float4 r4 = *reinterpret_cast<const float4*>(static_cast<const float*>(ep.resid) + base);
        uint2 w2;
        w2.x = pack_bf16x2(v[0] + r4.x, v[1] + r4.y);
        w2.y = pack_bf16x2(v[2] + r4.z, v[3] + r4.w);
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(ep.out) + base) = w2;
      }
    }
  }
}

template <int EPI>
hipError_t launch(const bf16_t* X, const bf16_t* W, int M, int N, int K, int blocks,
                  const SkinnyArgs& a, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int tb = (M + 15) / 16;
  const dim3 grid(blocks), block(kWaves * 64);
  if (tb == 1)
    hipLaunchKernelGGL((skinny_kernel<1, EPI>), grid, block, 0, s, X, W, M, N, K, a);
  else if (tb == 2)
    hipLaunchKernelGGL((skinny_kernel<2, EPI>), grid, block, 0, s, X, W, M, N, K, a);
  else if (tb <= 4)
    hipLaunchKernelGGL((skinny_kernel<4, EPI>), grid, block, 0, s, X, W, M, N, K, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                             const QkvEpilogue& ep, hipStream_t s) {
  SkinnyArgs a{};
  a.qkv = ep;
  return launch<SK_QKV>(A, W, M, N, K, N / 16, a, s);
}

hipError_t launch_skinny_resid_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                      const bf16_t* resid, float* out, hipStream_t s) {
  SkinnyArgs a{};
  a.resid = resid;
  a.out = out;
  return launch<SK_RESID32>(A, W, M, N, K, N / 16, a, s);
}

hipError_t launch_skinny_resid_bf16out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                       const float* resid, bf16_t* out, hipStream_t s) {
  SkinnyArgs a{};
  a.resid = resid;
  a.out = out;
  return launch<SK_RESID16>(A, W, M, N, K, N / 16, a, s);
}

hipError_t launch_skinny_swiglu(const bf16_t* A, const bf16_t* Wgu, int M, int f, int K,
                                bf16_t* out, hipStream_t s) {
  SkinnyArgs a{};
  a.out = out;
  return launch<SK_SWIGLU>(A, Wgu, M, f, K, f / 8, a, s);
}

}  // namespace llama
