// Weight-streaming GEMMs for few tokens (decode: M = batch <= 128), with the
// same fused epilogues as the tiled prefill GEMMs (RoPE + cache append,
// residual adds, SwiGLU).  Sources as for the prefill projections: "LMDrive
// LLM core inference unit" page §2.3-§2.5, "Llama MLP deep dive" page §2.2,
// and the "LLM mechanics lecture notes" Ch.04 (decode reads every weight once
// per step and is memory bound).
//
// gfx950 design.  Both operands are in fragment order, so every load is one
// contiguous 1 KB wavefront load straight into registers: a 32 x 16 weight
// fragment (A operand of the 32x32x16 MFMA, rows = output features) and a
// 32-token x 16 activation fragment (B operand, columns = tokens).  QKV and
// gate/up multiply bf16 operands, o_proj and down fp16 ones (the attention
// output and h are fp16), as in the tiled GEMMs.
//
// Work split.  A column group is NB 32-row blocks of W; its work is K/16 k
// steps.  The groups' k steps are laid end to end and the grid's G workgroups
// take equal contiguous ranges of them (G = groups x S, each group cut into S
// ranges, when there are too few groups to cover the CUs; else one workgroup
// per CU, whose range spans parts of several groups).  Inside a workgroup the NW
// wavefronts take the k steps of a group round-robin and keep DEPTH steps of
// loads in flight in a register ring (branch-free: steps past the end point
// the load past the buffer's range, which reads zeros); their partial tiles
// are added through LDS.  A group that lies wholly in one workgroup's range is
// finished there.  A group cut between workgroups is finished by whichever
// of them arrives last: each writes its partial tile with agent-scope atomic
// stores (coherent across the XCDs' L2s without an L2 write-back), waits for
// them to complete, and counts itself in on the group's counter; the last
// one reads all partials back, adds them in range order (so the result does
// not depend on arrival order) and runs the epilogue, then re-arms the
// counter.  Each weight byte is read exactly once (nontemporal loads); the
// activations (<= 128 x K bf16) are re-read by every workgroup from L2.
// Calls of 65-128 tokens take four 32-token blocks with 4 wavefronts (a
// wavefront finishes one token block).
//
// Pairing: the QKV weight's heads are in rotary-pair order (dims x and x + 64
// on rows 2x and 2x + 1), so a rotation's two inputs are neighbouring
// accumulator slots of one lane.  For SwiGLU, NB = 2 with blocks nb and
// nb + 2 of the [gate 64 | up 64] interleaved gate/up matrix puts gate
// column j and up column j in the same slot of the two blocks.
#include "common.h"

namespace llama {
namespace {

enum { SK_QKV = 0, SK_RESID32 = 1, SK_RESID16 = 2, SK_SWIGLU = 3, SK_F32OUT = 4 };

struct SkinnyArgs {
  QkvEpilogue qkv;
  const void* resid;
  void* out;
  float* part;     // 2 G partial slots of NB * TB * 1024 floats
  size_t part_len; // floats at part
  unsigned* cnt;   // per column group, zero between launches
  int cnt_len;
  int n_valid, ld; // SK_F32OUT: columns written (< N) and the output's row stride
};

template <int NB, int TB, int NW, int DEPTH, int EPI>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(const bf16_t* __restrict__ Xp,
                                                         const bf16_t* __restrict__ Wp, int M, int N,
                                                         int K, int G, SkinnyArgs ep) {
  constexpr int NT = NB * TB;  // 32 x 32 tiles per column group
  // o_proj and down multiply fp16 operands, the others bf16
  constexpr bool F16 = EPI == SK_RESID32 || EPI == SK_RESID16;
  __shared__ float red[NW][NT][64][17];
  __shared__ unsigned s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar, so that everything derived from it stays uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K >> 4;
  const long long W = static_cast<long long>(N / (32 * NB)) * KB;  // k steps of all groups
  auto start_of = [&](int w) -> long long { return W * w / G; };
  auto owner = [&](long long x) -> int {  // the workgroup whose range holds step x
    int w = static_cast<int>(x * G / W);
    while (w + 1 < G && start_of(w + 1) <= x) ++w;
    return w;
  };
  const int wg = blockIdx.x;
  const long long u0 = start_of(wg), u1 = start_of(wg + 1);
  const uint32_t w_bytes = static_cast<uint32_t>(N) * K * 2u;
  const uint32_t x_bytes = static_cast<uint32_t>(TB) * 32u * K * 2u;
  const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(Wp, w_bytes);
  const __amdgpu_buffer_rsrc_t x_rs = make_rsrc(Xp, x_bytes);

  // The epilogue's inputs that do not depend on the sums (the position and
  // RoPE cos/sin, or the residual), for token block t of group g: fetched
  // when the workgroup starts on the group, so the epilogue at the end of the
  // kernel does not wait on them.  rr[j][r4]: the cos and sin pairs (QKV),
  // 4 bf16 (o_proj) or 4 fp32 (down) of the residual.
  static_assert(TB <= NW, "a wavefront finishes at most one token block of a group");
  struct EpiIn {
    int p;
    uint4 rr[NB][4];
  };
  auto epi_fetch = [&](int g, int t) {
    EpiIn in{};
    const int nb0 = NB == 2 ? (g >> 1) * 4 + (g & 1) : g;
    const int tok = t * 32 + (lane & 31);
    const int tk = tok < M ? tok : 0;
    if constexpr (EPI == SK_QKV) {
      const QkvEpilogue& q = ep.qkv;
      in.p = q.pos[tk];
      const int pt = min(max(in.p, 0), q.max_pos - 1);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int x0 = ((nb0 & 3) * 32 + 8 * r4 + 4 * (lane >> 5)) >> 1;
        const float2 c = *reinterpret_cast<const float2*>(q.rope_cos + static_cast<size_t>(pt) * 64 + x0);
        const float2 sn = *reinterpret_cast<const float2*>(q.rope_sin + static_cast<size_t>(pt) * 64 + x0);
        in.rr[0][r4] = make_uint4(__float_as_uint(c.x), __float_as_uint(c.y), __float_as_uint(sn.x),
                                  __float_as_uint(sn.y));
      }
    } else if constexpr (EPI == SK_RESID32 || EPI == SK_RESID16) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const size_t at = static_cast<size_t>(tk) * N + (nb0 + 2 * j) * 32 + 8 * r4 + 4 * (lane >> 5);
          if constexpr (EPI == SK_RESID32) {
            const uint2 rb = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(ep.resid) + at);
            in.rr[j][r4] = make_uint4(rb.x, rb.y, 0u, 0u);
          } else {
            in.rr[j][r4] = *reinterpret_cast<const uint4*>(static_cast<const float*>(ep.resid) + at);
          }
        }
    }
    return in;
  };

  // the epilogue of token block t of group g, from the finished sums v[j][r]
  auto finish = [&](int g, int t, const float (&v)[NB][16], const EpiIn& in) {
    const int nb0 = NB == 2 ? (g >> 1) * 4 + (g & 1) : g;
    const int tok = t * 32 + (lane & 31);
    if (tok >= M) return;
    // accumulator slot r of a lane is feature 8 (r/4) + 4 (lane/32) + r%4 of
    // its block, token lane % 32: four consecutive slots, four consecutive features
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int fib = 8 * r4 + 4 * (lane >> 5);  // first of the 4 features in the block
      if constexpr (EPI == SK_QKV) {
        // rotary-pair order: feature 2x of a head is dim x, 2x + 1 dim x + 64;
        // the 4 features are dims x0, x0 + 64, x0 + 1, x0 + 65
        const QkvEpilogue& q = ep.qkv;
        const int head = nb0 >> 2;
        const int x0 = ((nb0 & 3) * 32 + fib) >> 1;
        const int kind = head < q.n_heads ? 0 : (head < q.n_heads + q.n_kv_heads ? 1 : 2);
        const int hh = kind == 0 ? head : (kind == 1 ? head - q.n_heads : head - q.n_heads - q.n_kv_heads);
        const int p = in.p;
        float lo[2] = {v[0][4 * r4], v[0][4 * r4 + 2]}, hi[2] = {v[0][4 * r4 + 1], v[0][4 * r4 + 3]};
        if (kind != 2) {
          const uint4 w = in.rr[0][r4];
          const float cc[2] = {__uint_as_float(w.x), __uint_as_float(w.y)};
          const float ss[2] = {__uint_as_float(w.z), __uint_as_float(w.w)};
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float x1 = lo[e], x2 = hi[e];
            lo[e] = x1 * cc[e] - x2 * ss[e];
            hi[e] = x2 * cc[e] + x1 * ss[e];
          }
        }
        bf16_t* dst;
        if (kind == 0) {
          dst = q.q + static_cast<size_t>(tok) * (q.n_heads * 128) + hh * 128;
        } else {
          if (p < 0 || p >= q.span) continue;
          const long long kr = q.stage ? static_cast<long long>(tok) * q.n_kv_heads + hh
                                       : kv_row(q.pg, tok / q.T, hh, q.n_kv_heads, q.max_pos, p);
          if (kr < 0) continue;  // no valid page for this slot
          dst = (kind == 1 ? q.k_cache : q.v_cache) + kr * 128;
        }
        *reinterpret_cast<uint32_t*>(dst + x0) = pack_bf16x2(lo[0], lo[1]);
        *reinterpret_cast<uint32_t*>(dst + x0 + 64) = pack_bf16x2(hi[0], hi[1]);
      } else if constexpr (EPI == SK_SWIGLU) {
        static_assert(NB == 2, "SwiGLU needs the up block");
        const int f = N >> 1;
        const int c = (nb0 >> 2) * 64 + (nb0 & 3) * 32 + fib;  // h column
        float hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = silu(v[0][4 * r4 + e]) * v[1][4 * r4 + e];
        bf16_t* out = static_cast<bf16_t*>(ep.out);  // fp16 h
        *reinterpret_cast<uint2*>(out + frag_index(tok, c, f)) =
            make_uint2(pack_f16x2_sat(hv[0], hv[1]), pack_f16x2_sat(hv[2], hv[3]));
      } else if constexpr (EPI == SK_F32OUT) {
        // plain fp32 rows (LM head logits): columns past n_valid are padding
        float* out = static_cast<float*>(ep.out) + static_cast<size_t>(tok) * ep.ld;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nb0 * 32 + fib + e < ep.n_valid) out[nb0 * 32 + fib + e] = v[0][4 * r4 + e];
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = (nb0 + 2 * j) * 32 + fib;
          const size_t at = static_cast<size_t>(tok) * N + col;
          if constexpr (EPI == SK_RESID32) {
            const uint2 rb = make_uint2(in.rr[j][r4].x, in.rr[j][r4].y);
            *reinterpret_cast<float4*>(static_cast<float*>(ep.out) + at) =
                make_float4(v[j][4 * r4] + lo_bf16(rb.x), v[j][4 * r4 + 1] + hi_bf16(rb.x),
                            v[j][4 * r4 + 2] + lo_bf16(rb.y), v[j][4 * r4 + 3] + hi_bf16(rb.y));
          } else {
            const float4 rf = make_float4(__uint_as_float(in.rr[j][r4].x), __uint_as_float(in.rr[j][r4].y),
                                          __uint_as_float(in.rr[j][r4].z), __uint_as_float(in.rr[j][r4].w));
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(ep.out) + at) =
                make_uint2(pack_bf16x2(v[j][4 * r4] + rf.x, v[j][4 * r4 + 1] + rf.y),
                           pack_bf16x2(v[j][4 * r4 + 2] + rf.z, v[j][4 * r4 + 3] + rf.w));
          }
        }
      }
    }
  };

  // partial slot of workgroup w's segment of group g: 2w if w's range starts
  // inside g, 2w + 1 if g is where it ends
  auto slot_of = [&](int w, int g) { return 2 * w + (start_of(w) >= static_cast<long long>(g) * KB ? 0 : 1); };

  for (long long u = u0; u < u1;) {
    const int g = static_cast<int>(u / KB);
    const int k0 = static_cast<int>(u - static_cast<long long>(g) * KB);
    const int k1 = static_cast<int>(min(static_cast<long long>(KB), u1 - static_cast<long long>(g) * KB));
    u = static_cast<long long>(g) * KB + k1;
    const int nb0 = NB == 2 ? (g >> 1) * 4 + (g & 1) : g;
    // this wave's token block of the group: its epilogue inputs, in flight during the stream
    const EpiIn pre = wave < TB ? epi_fetch(g, wave) : EpiIn{};

    f32x16 acc[NB][TB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][t][r] = 0.f;

    const int nsteps = max(0, (k1 - k0 - wave + NW - 1) / NW);  // k steps k0 + wave, + NW, ...
    uint4 wv[DEPTH][NB], xv[DEPTH][TB];
    auto issue = [&](int slot, int st) {
      const uint32_t kb = static_cast<uint32_t>(k0 + wave + st * NW);
      const bool ok = st < nsteps;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint32_t off = ((static_cast<uint32_t>(nb0 + 2 * j) * KB + kb) << 10) + lane * 16u;
        wv[slot][j] = buf_load16_nt(w_rs, ok ? off : w_bytes, 0);
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
            acc[j][t] = mfma_32x32x16<F16>(__builtin_bit_cast(bf16x8, wv[d][j]), __builtin_bit_cast(bf16x8, xv[d][t]),
                                           acc[j][t]);
        issue(d, st + d + DEPTH);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    __syncthreads();  // the previous segment's reads of red are done
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[wave][j * TB + t][lane][r] = acc[j][t][r];
    __syncthreads();

    // wave t owns token block t: the sum over waves of its NB tiles
    auto wave_sum = [&](int t, float (&v)[NB][16]) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) a += red[w][j * TB + t][lane][r];
          v[j][r] = a;
        }
    };
    if (k0 == 0 && k1 == KB) {
      for (int t = wave; t < TB; t += NW) {
        float v[NB][16];
        wave_sum(t, v);
        finish(g, t, v, pre);
      }
      continue;
    }

    // group g is shared with other workgroups
    float* mine = ep.part + static_cast<size_t>(slot_of(wg, g)) * (NT * 1024);
    for (int t = wave; t < TB; t += NW) {
      float v[NB][16];
      wave_sum(t, v);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __hip_atomic_store(mine + ((j * TB + t) * 16 + r) * 64 + lane, v[j][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partial has reached the coherent level
    __syncthreads();
    const int w_first = owner(static_cast<long long>(g) * KB);
    const int w_last = owner(static_cast<long long>(g + 1) * KB - 1);
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(ep.cnt + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               static_cast<unsigned>(w_last - w_first);
    __syncthreads();
    if (!s_last) continue;
    for (int t = wave; t < TB; t += NW) {
      float v[NB][16];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[j][r] = 0.f;
      for (int w = w_first; w <= w_last; ++w) {
        const float* src = ep.part + static_cast<size_t>(slot_of(w, g)) * (NT * 1024);
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            v[j][r] += __hip_atomic_load(src + ((j * TB + t) * 16 + r) * 64 + lane, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      }
      finish(g, t, v, pre);
    }
    if (tid == 0) __hip_atomic_store(ep.cnt + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

constexpr int kNW = 2;  // wavefronts per workgroup

// Grid size.  With fewer column groups than CUs each group is split into S
// equal k ranges, S = n_cu / groups (at most 8, each range at least 8 k
// steps), so narrow projections still cover every CU.  With more groups than
// CUs the grid is one workgroup per CU, each streaming an equal contiguous
// share of all the groups' k steps (a group cut at a share's end is finished
// by the fixup): one workgroup per group would leave some CUs with twice the
// bytes of others.  Measured on the 7B (M = 32) and 70B (M = 1) decode shapes,
// the 70B QKV and gate/up projections (320 and 896 groups) run 17% and 4%
// faster this way, the 7B ones within 4% either side.
int grid_for(int groups, int KB, int n_cu) {
  if (n_cu > kSkinnyGrid) n_cu = kSkinnyGrid;
  if (groups > n_cu) return n_cu;
  int S = n_cu / groups;
  if (S > 8) S = 8;
  while (S > 1 && KB / S < 8) --S;
  if (S < 1) S = 1;
  return groups * S;
}

template <int EPI>
hipError_t launch(const bf16_t* X, const bf16_t* W, int M, int N, int K, SkinnyArgs ep, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (M > kSkinnyMaxTokens || K % 16 || N % 128) return hipErrorInvalidValue;
  constexpr bool paired = EPI == SK_SWIGLU;
  constexpr int NB = paired ? 2 : 1;
  const int groups = N / (32 * NB);
  const int G = grid_for(groups, K / 16, device_cu_count());
  // split groups need 2 G partial slots of NB x TB tiles and a counter each
  const int TBn = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
  if (G != groups && (G > kSkinnyGrid || groups > ep.cnt_len ||
                      static_cast<size_t>(2) * G * NB * TBn * 1024 > ep.part_len))
    return hipErrorInvalidValue;
  if (M <= 32)
    hipLaunchKernelGGL((skinny_kernel<NB, 1, kNW, paired ? 12 : 16, EPI>), dim3(G), dim3(kNW * 64), 0, s, X, W, M,
                       N, K, G, ep);
  else if (M <= 64)
    hipLaunchKernelGGL((skinny_kernel<NB, 2, kNW, paired ? 8 : 12, EPI>), dim3(G), dim3(kNW * 64), 0, s, X, W, M,
                       N, K, G, ep);
  else  // 4 token blocks: a wavefront per block, so 4 wavefronts
    hipLaunchKernelGGL((skinny_kernel<NB, 4, 4, paired ? 6 : 8, EPI>), dim3(G), dim3(4 * 64), 0, s, X, W, M, N, K,
                       G, ep);
  return hipGetLastError();
}

}  // namespace

size_t skinny_scratch_floats() { return static_cast<size_t>(2) * kSkinnyGrid * 8 * 1024; }  // NB x TB <= 8

hipError_t launch_skinny_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K, const QkvEpilogue& q,
                             const SkinnyScratch& sc, hipStream_t s) {
  SkinnyArgs ep{};
  ep.qkv = q;
  ep.part = sc.part;
  ep.part_len = sc.part_len;
  ep.cnt = sc.cnt;
  ep.cnt_len = sc.cnt_len;
  return launch<SK_QKV>(A, W, M, N, K, ep, s);
}
hipError_t launch_skinny_resid_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                      const bf16_t* resid, float* out, const SkinnyScratch& sc, hipStream_t s) {
  SkinnyArgs ep{};
  ep.resid = resid;
  ep.out = out;
  ep.part = sc.part;
  ep.part_len = sc.part_len;
  ep.cnt = sc.cnt;
  ep.cnt_len = sc.cnt_len;
  return launch<SK_RESID32>(A, W, M, N, K, ep, s);
}
hipError_t launch_skinny_resid_bf16out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                       const float* resid, bf16_t* out, const SkinnyScratch& sc, hipStream_t s) {
  SkinnyArgs ep{};
  ep.resid = resid;
  ep.out = out;
  ep.part = sc.part;
  ep.part_len = sc.part_len;
  ep.cnt = sc.cnt;
  ep.cnt_len = sc.cnt_len;
  return launch<SK_RESID16>(A, W, M, N, K, ep, s);
}
hipError_t launch_skinny_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K, float* out, int n_valid,
                                int ld, const SkinnyScratch& sc, hipStream_t s) {
  if (n_valid > N || ld < n_valid) return hipErrorInvalidValue;
  SkinnyArgs ep{};
  ep.out = out;
  ep.part = sc.part;
  ep.part_len = sc.part_len;
  ep.cnt = sc.cnt;
  ep.cnt_len = sc.cnt_len;
  ep.n_valid = n_valid;
  ep.ld = ld;
  return launch<SK_F32OUT>(A, W, M, N, K, ep, s);
}
hipError_t launch_skinny_swiglu(const bf16_t* A, const bf16_t* Wgu, int M, int f, int K, bf16_t* out,
                                const SkinnyScratch& sc, hipStream_t s) {
  SkinnyArgs ep{};
  ep.out = out;
  ep.part = sc.part;
  ep.part_len = sc.part_len;
  ep.cnt = sc.cnt;
  ep.cnt_len = sc.cnt_len;
  return launch<SK_SWIGLU>(A, Wgu, M, 2 * f, K, ep, s);
}

}  // namespace llama
