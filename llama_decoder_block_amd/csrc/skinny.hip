// Weight-streaming GEMMs for few tokens (decode: M = batch <= 64), with the
// same fused epilogues as the tiled prefill GEMMs (RoPE + cache append,
// residual adds, SwiGLU).  Sources as for the prefill projections: "LMDrive
// LLM core inference unit" page §2.3-§2.5, "Llama MLP deep dive" page §2.2,
// and the "LLM mechanics lecture notes" Ch.04 (decode reads every weight once
// per step and is memory bound).
//
// gfx950 design.  Both operands are in fragment order, so every load is one
// contiguous 1 KB wavefront load straight into registers: a 32 x 16 weight
// fragment (A operand of v_mfma_f32_32x32x16_bf16, rows = output features)
// and a 32-token x 16 activation fragment (B operand, columns = tokens).  A
// workgroup owns NB 32-row blocks of W and all tokens; its NW wavefronts take
// the 16-wide k steps round-robin and keep DEPTH steps of loads in flight in
// a register ring (branch-free: steps past the end point the load past the
// buffer's range, which reads zeros).  The partial tiles of the waves are
// added through LDS at the end.  Each weight byte is read exactly once; the
// activations (<= 64 x K bf16) are re-read by every workgroup from L2.
//
// Pairing: with NB = 2 the blocks are nb and nb + 2, so one lane holds
// feature i and feature i + 64 of the same 128-row group for the same token
// in the same accumulator slot — the RoPE partners of one head (dims i and
// i + dh/2) and, over the [gate 64 | up 64] interleaved gate/up matrix, gate
// column j and up column j.
#include "common.h"

namespace llama {
namespace {

enum { SK_QKV = 0, SK_RESID32 = 1, SK_RESID16 = 2, SK_SWIGLU = 3 };

struct SkinnyArgs {
  QkvEpilogue qkv;
  const void* resid;
  void* out;
};

template <int NB, int TB, int NW, int DEPTH, int EPI>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(const bf16_t* __restrict__ Xp,
                                                         const bf16_t* __restrict__ Wp, int M, int N,
                                                         int K, SkinnyArgs ep) {
  __shared__ float red[NW][NB * TB][64][17];
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar, so that everything derived from it stays uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K >> 4;
  const int grp = blockIdx.x;
  const int nb0 = NB == 2 ? (grp >> 1) * 4 + (grp & 1) : grp;
  const uint32_t w_bytes = static_cast<uint32_t>(N) * K * 2u;
  const uint32_t x_bytes = static_cast<uint32_t>(TB) * 32u * K * 2u;
  const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(Wp, w_bytes);
  const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(Xp, x_bytes);

  f32x16 acc[NB][TB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][t][r] = 0.f;

  const int nsteps = (KB - wave + NW - 1) / NW;  // k steps wave, wave + NW, ...
  uint4 wv[DEPTH][NB], xv[DEPTH][TB];
  auto issue = [&](int slot, int st) {
    const uint32_t kb = static_cast<uint32_t>(wave + st * NW);
    const bool ok = st < nsteps;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint32_t off = ((static_cast<uint32_t>(nb0 + 2 * j) * KB + kb) << 10) + lane * 16u;
      wv[slot][j] = buf_load16(w_rs, ok ? off : w_bytes, 0);
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const uint32_t off = ((static_cast<uint32_t>(t) * KB + kb) << 10) + lane * 16u;
      xv[slot][t] = buf_load16(x_rs, ok ? off : x_bytes, 0);
    }
  };
  // the sched barriers keep every step's loads in issue order, which lets
  // the compiler wait for exactly the oldest step instead of draining the ring
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    issue(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int st = 0; st < nsteps; st += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int t = 0; t < TB; ++t)
          acc[j][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv[d][j]),
                                                              __builtin_bit_cast(bf16x8, xv[d][t]),
                                                              acc[j][t], 0, 0, 0);
      issue(d, st + d + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][j * TB + t][lane][r] = acc[j][t][r];
  __syncthreads();

  // epilogue: wave t finishes token block t.  Accumulator slot r of a lane
  // is feature 8 (r/4) + 4 (lane/32) + r%4 of its block, token lane % 32, so
  // four consecutive slots are four consecutive features.
  for (int t = wave; t < TB; t += NW) {
    float v[NB][16];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) a += red[w][j * TB + t][lane][r];
        v[j][r] = a;
      }
    const int tok = t * 32 + (lane & 31);
    if (tok >= M) continue;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int fib = 8 * r4 + 4 * (lane >> 5);  // first of the 4 features in the block
      if constexpr (EPI == SK_QKV) {
        static_assert(NB == 2, "RoPE needs the partner block");
        const QkvEpilogue& q = ep.qkv;
        const int head = nb0 >> 2;
        const int i = (nb0 & 3) * 32 + fib;  // dim in the head, < 64; partner i + 64
        const int kind = head < q.n_heads ? 0 : (head < q.n_heads + q.n_kv_heads ? 1 : 2);
        const int hh = kind == 0 ? head : (kind == 1 ? head - q.n_heads : head - q.n_heads - q.n_kv_heads);
        const int p = q.pos[tok];
        const int pt = min(max(p, 0), q.max_pos - 1);
        float lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) { lo[e] = v[0][4 * r4 + e]; hi[e] = v[1][4 * r4 + e]; }
        if (kind != 2) {
          const float4 c = *reinterpret_cast<const float4*>(q.rope_cos + static_cast<size_t>(pt) * 64 + i);
          const float4 s = *reinterpret_cast<const float4*>(q.rope_sin + static_cast<size_t>(pt) * 64 + i);
          const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x1 = lo[e], x2 = hi[e];
            lo[e] = x1 * cc[e] - x2 * ss[e];
            hi[e] = x2 * cc[e] + x1 * ss[e];
          }
        }
        bf16_t* dst;
        if (kind == 0) {
          dst = q.q + static_cast<size_t>(tok) * (q.n_heads * 128) + hh * 128;
        } else {
          if (p < 0 || p >= q.max_pos) continue;
          const int b = tok / q.T;
          bf16_t* cache = kind == 1 ? q.k_cache : q.v_cache;
          dst = cache + (static_cast<size_t>(b * q.n_kv_heads + hh) * q.max_pos + p) * 128;
        }
        *reinterpret_cast<uint2*>(dst + i) = make_uint2(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]));
        *reinterpret_cast<uint2*>(dst + i + 64) = make_uint2(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
      } else if constexpr (EPI == SK_SWIGLU) {
        static_assert(NB == 2, "SwiGLU needs the up block");
        const int f = N >> 1;
        const int c = (nb0 >> 2) * 64 + (nb0 & 3) * 32 + fib;  // h column
        float hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = silu(v[0][4 * r4 + e]) * v[1][4 * r4 + e];
        bf16_t* out = static_cast<bf16_t*>(ep.out);
        *reinterpret_cast<uint2*>(out + frag_index(tok, c, f)) =
            make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = (nb0 + 2 * j) * 32 + fib;
          const size_t at = static_cast<size_t>(tok) * N + col;
          if constexpr (EPI == SK_RESID32) {
            const uint2 rb = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(ep.resid) + at);
            *reinterpret_cast<float4*>(static_cast<float*>(ep.out) + at) =
                make_float4(v[j][4 * r4] + lo_bf16(rb.x), v[j][4 * r4 + 1] + hi_bf16(rb.x),
                            v[j][4 * r4 + 2] + lo_bf16(rb.y), v[j][4 * r4 + 3] + hi_bf16(rb.y));
          } else {
            const float4 rf = *reinterpret_cast<const float4*>(static_cast<const float*>(ep.resid) + at);
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(ep.out) + at) =
                make_uint2(pack_bf16x2(v[j][4 * r4] + rf.x, v[j][4 * r4 + 1] + rf.y),
                           pack_bf16x2(v[j][4 * r4 + 2] + rf.z, v[j][4 * r4 + 3] + rf.w));
          }
        }
      }
    }
  }
}

// Paired epilogues (QKV, SwiGLU) stream two blocks per workgroup; the
// residual GEMMs one, which doubles the workgroups for the narrow N = d.
template <int EPI>
hipError_t launch(const bf16_t* X, const bf16_t* W, int M, int N, int K, const SkinnyArgs& ep,
                  hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (M > kSkinnyMaxTokens || K % 16 || N % 128) return hipErrorInvalidValue;
  constexpr bool paired = EPI == SK_QKV || EPI == SK_SWIGLU;
  constexpr int NW = 2;
  if constexpr (paired) {
    const dim3 grid(N / 64);
    if (M <= 32)
      hipLaunchKernelGGL((skinny_kernel<2, 1, NW, 12, EPI>), grid, dim3(NW * 64), 0, s, X, W, M, N, K, ep);
    else
      hipLaunchKernelGGL((skinny_kernel<2, 2, NW, 8, EPI>), grid, dim3(NW * 64), 0, s, X, W, M, N, K, ep);
  } else {
    const dim3 grid(N / 32);
    if (M <= 32)
      hipLaunchKernelGGL((skinny_kernel<1, 1, NW, 16, EPI>), grid, dim3(NW * 64), 0, s, X, W, M, N, K, ep);
    else
      hipLaunchKernelGGL((skinny_kernel<1, 2, NW, 12, EPI>), grid, dim3(NW * 64), 0, s, X, W, M, N, K, ep);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                             const QkvEpilogue& q, hipStream_t s) {
  SkinnyArgs ep{};
  ep.qkv = q;
  return launch<SK_QKV>(A, W, M, N, K, ep, s);
}
hipError_t launch_skinny_resid_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                      const bf16_t* resid, float* out, hipStream_t s) {
  SkinnyArgs ep{};
  ep.resid = resid;
  ep.out = out;
  return launch<SK_RESID32>(A, W, M, N, K, ep, s);
}
hipError_t launch_skinny_resid_bf16out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                       const float* resid, bf16_t* out, hipStream_t s) {
  SkinnyArgs ep{};
  ep.resid = resid;
  ep.out = out;
  return launch<SK_RESID16>(A, W, M, N, K, ep, s);
}
hipError_t launch_skinny_swiglu(const bf16_t* A, const bf16_t* Wgu, int M, int f, int K, bf16_t* out,
                                hipStream_t s) {
  SkinnyArgs ep{};
  ep.out = out;
  return launch<SK_SWIGLU>(A, Wgu, M, 2 * f, K, ep, s);
}

}  // namespace llama
