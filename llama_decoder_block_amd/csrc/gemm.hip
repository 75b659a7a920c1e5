// Tiled bf16 MFMA GEMM for the prefill projections, C = A[M,K] . W[N,K]^T,
// with the layer's elementwise work fused into the epilogue:
//   QKV     rotate-half RoPE of q and k at each token's position, bf16 round,
//           q -> scratch, k and v -> their cache slot (no concatenation pass);
//   RESID32 X' = x + O Wo^T kept in fp32 (the residual add of the attention half);
//   SWIGLU  h = SiLU(gate) * up from one GEMM over the gate/up matrix packed in
//           64-row blocks [gate 64 | up 64], so a lane holds gate column j and
//           up column j in the same accumulator slot;
//   RESID16 y = bf16(X' + h Wdown^T) (the residual add of the MLP half).
//
// Sources: "LMDrive LLM core inference unit" page, §2.3 LlamaAttention (q/k/v
// projections, RoPE, cache append, o_proj) and §2.4 LlamaMLP
// (down(SiLU(gate(x)) * up(x)), no bias), §2.5 (both residual adds); §2.2 for
// the rotate-half pairing of dimension i with i + dh/2; "Llama MLP deep dive"
// page §2.2 (gate branch activated, up branch linear).
//
// gfx950 design.  Both operands are K-contiguous ("NT"), which is exactly the
// per-lane layout of v_mfma_f32_32x32x16_bf16 (a lane feeds 8 consecutive k of
// one row), so tiles are staged to LDS unchanged.  256 threads = 4 wavefronts
// in a 2x2 grid; each wave owns a (BM/2) x (BN/2) block of 32x32 accumulator
// tiles.  BK = 64; LDS rows are padded to 144 bytes so the 16-byte fragment
// reads of 16 consecutive rows fall in distinct banks.  Two LDS stages: the
// next K-slab is fetched into registers while the current one feeds the MFMAs,
// one barrier per slab.  Tiles are numbered so that each XCD (blocks are
// dealt round-robin over 8 XCDs) gets a contiguous, M-grouped range, which
// keeps the A and W panels it shares inside its own L2.
#include "common.h"

namespace llama {
namespace {

enum { EPI_QKV = 0, EPI_RESID32 = 1, EPI_RESID16 = 2, EPI_SWIGLU = 3 };

struct EpiArgs {
  QkvEpilogue qkv;
  const void* resid;
  void* out;
};

constexpr int BK = 64;
constexpr int SK = BK + 8;  // padded LDS row, in bf16 elements (144 bytes)
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

template <int BM, int BN>
struct Tile {
  static constexpr int TM = BM / 2, TN = BN / 2;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_CH = BM * (BK / 8) / kThreads;  // 16-byte chunks per thread
  static constexpr int B_CH = BN * (BK / 8) / kThreads;
};

__device__ __forceinline__ void tile_coords(int M, int N, int BM, int BN, int& m0, int& n0) {
  const int nt_m = (M + BM - 1) / BM, nt_n = (N + BN - 1) / BN;
  const int nt = nt_m * nt_n;
  int bid = blockIdx.x;
  if ((nt & 7) == 0) bid = (bid & 7) * (nt >> 3) + (bid >> 3);  // contiguous range per XCD
  const int group = kGroupM * nt_n;
  const int first_m = (bid / group) * kGroupM;
  const int gm = min(nt_m - first_m, kGroupM);
  const int in_group = bid % group;
  m0 = (first_m + in_group % gm) * BM;
  n0 = (in_group / gm) * BN;
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(const bf16_t* __restrict__ A,
                                                              const bf16_t* __restrict__ W,
                                                              int M, int N, int K, EpiArgs ep) {
  using TL = Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * SK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * SK];

  int m0, n0;
  tile_coords(M, N, BM, BN, m0, n0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: raw buffer loads with one 32-bit offset per
  // chunk; rows past M or N read as zeros and are never stored.
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(A, static_cast<uint32_t>(M) * K * 2u);
  const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(W, static_cast<uint32_t>(N) * K * 2u);
  const int ld_r = tid >> 3, ld_c = (tid & 7) * 8;
  uint32_t a_off[TL::A_CH], b_off[TL::B_CH];
#pragma unroll
  for (int i = 0; i < TL::A_CH; ++i)
    a_off[i] = (static_cast<uint32_t>(m0 + ld_r + i * 32) * K + ld_c) * 2u;
#pragma unroll
  for (int i = 0; i < TL::B_CH; ++i)
    b_off[i] = (static_cast<uint32_t>(n0 + ld_r + i * 32) * K + ld_c) * 2u;
  const int st_base = ld_r * SK + ld_c;

  uint4 ra[TL::A_CH], rb[TL::B_CH];
  f32x16 acc[TL::FM][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto gload = [&](int k0) {
    const uint32_t sk = static_cast<uint32_t>(k0) * 2u;
#pragma unroll
    for (int i = 0; i < TL::A_CH; ++i) ra[i] = buf_load16(a_rs, a_off[i], sk);
#pragma unroll
    for (int i = 0; i < TL::B_CH; ++i) rb[i] = buf_load16(b_rs, b_off[i], sk);
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < TL::A_CH; ++i)
      *reinterpret_cast<uint4*>(&As[st][st_base + i * 32 * SK]) = ra[i];
#pragma unroll
    for (int i = 0; i < TL::B_CH; ++i)
      *reinterpret_cast<uint4*>(&Bs[st][st_base + i * 32 * SK]) = rb[i];
  };

  const int nk = K / BK;
  const int a_row = (wm * TL::TM + (lane & 31)) * SK + (lane >> 5) * 8;
  const int b_row = (wn * TL::TN + (lane & 31)) * SK + (lane >> 5) * 8;
  bf16x8 fa[2][TL::FM], fb[2][TL::FN];
  auto frag_a = [&](int st, int kk, int i) {
    return *reinterpret_cast<const bf16x8*>(&As[st][a_row + i * 32 * SK + kk * 16]);
  };
  auto frag_b = [&](int st, int kk, int j) {
    return *reinterpret_cast<const bf16x8*>(&Bs[st][b_row + j * 32 * SK + kk * 16]);
  };
  // staging chunk c (A chunks first, then B): LDS write of slab kt+1 from the
  // registers, then the load of slab kt+2 into the same registers
  auto stage_chunk = [&](int c, int st_w, int k0_next) {
    const uint32_t sk = static_cast<uint32_t>(k0_next) * 2u;
    if (c < TL::A_CH) {
      *reinterpret_cast<uint4*>(&As[st_w][st_base + c * 32 * SK]) = ra[c];
      ra[c] = buf_load16(a_rs, a_off[c], sk);
    } else {
      const int cb = c - TL::A_CH;
      *reinterpret_cast<uint4*>(&Bs[st_w][st_base + cb * 32 * SK]) = rb[cb];
      rb[cb] = buf_load16(b_rs, b_off[cb], sk);
    }
  };

  // Software pipeline, fixed instruction order.  While LDS stage kt&1 feeds
  // the MFMAs of slab kt: the registers (loaded during the previous slab) are
  // written to the other stage and refilled with slab kt+2, spread over the
  // first three 16-wide k steps; each MFMA slot also reads one fragment of the
  // next k step.  The barrier sits before the last k step, whose MFMA slots
  // then read the first fragments of slab kt+1.  Past the last slab the loads
  // read in-range data of the next row or zeros and that stage is never used.
  constexpr int kSlots = TL::FM * TL::FN;
  constexpr int kChunks = TL::A_CH + TL::B_CH;
  constexpr int kPerStep = (kChunks + 2) / 3;
  gload(0);
  lstore(0);
  gload(BK);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) fa[0][i] = frag_a(0, 0, i);
#pragma unroll
  for (int j = 0; j < TL::FN; ++j) fb[0][j] = frag_b(0, 0, j);

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    const int k_next2 = (kt + 2) * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      const int rd_st = kk < 3 ? st : st ^ 1;
      const int rd_kk = kk < 3 ? kk + 1 : 0;
      if (kk == 3) __syncthreads();
#pragma unroll
      for (int m = 0; m < kSlots; ++m) {
        const int i = m / TL::FN, j = m % TL::FN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        if (m < TL::FM)
          fa[cur ^ 1][m] = frag_a(rd_st, rd_kk, m);
        else if (m < TL::FM + TL::FN)
          fb[cur ^ 1][m - TL::FM] = frag_b(rd_st, rd_kk, m - TL::FM);
        if (kk < 3) {
          // chunk placed in slot m: spread kPerStep chunks over the slots
#pragma unroll
          for (int q = 0; q < kPerStep; ++q) {
            const int c = kk * kPerStep + q;
            if (c < kChunks && (q * kSlots) / kPerStep == m) stage_chunk(c, st ^ 1, k_next2);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  // accumulator register r of tile (i, j) holds row 8*(r/4) + 4*(lane/32) + r%4
  // and column lane%32 of that 32x32 tile.
  const int row_base = m0 + wm * TL::TM + 4 * (lane >> 5);
  const int col0 = n0 + wn * TL::TN;
  const int lc = lane & 31;
  if (col0 >= N) return;

  if constexpr (EPI == EPI_QKV) {
    static_assert(TL::TN == 128, "QKV epilogue needs one 128-wide head per wave");
    const QkvEpilogue& q = ep.qkv;
    const int head = col0 >> 7;
    const int kind = head < q.n_heads ? 0 : (head < q.n_heads + q.n_kv_heads ? 1 : 2);
    const int hh = kind == 0 ? head : (kind == 1 ? head - q.n_heads : head - q.n_heads - q.n_kv_heads);
    const int qstride = q.n_heads * 128;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= M) continue;
        const int p = q.pos[row];
        const int pt = min(max(p, 0), q.max_pos - 1);  // table row (out-of-range p is never stored)
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = acc[i][j][r];
        if (kind != 2) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int dd = j * 32 + lc;
            const float c = q.rope_cos[static_cast<size_t>(pt) * 64 + dd];
            const float s = q.rope_sin[static_cast<size_t>(pt) * 64 + dd];
            const float x1 = v[j], x2 = v[j + 2];
            v[j] = x1 * c - x2 * s;
            v[j + 2] = x2 * c + x1 * s;
          }
        }
        bf16_t* dst;
        if (kind == 0) {
          dst = q.q + static_cast<size_t>(row) * qstride + hh * 128;
        } else {
          if (p < 0 || p >= q.max_pos) continue;
          const int b = row / q.T;
          bf16_t* cache = kind == 1 ? q.k_cache : q.v_cache;
          dst = cache + (static_cast<size_t>(b * q.n_kv_heads + hh) * q.max_pos + p) * 128;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j * 32 + lc] = f32_to_bf16(v[j]);
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    static_assert(TL::TN == 128, "SwiGLU epilogue needs a [gate 64 | up 64] block per wave");
    bf16_t* out = static_cast<bf16_t*>(ep.out);
    const int f = N >> 1;
    const int hcol0 = (col0 >> 7) * 64;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= M) continue;
        bf16_t* dst = out + static_cast<size_t>(row) * f + hcol0;
#pragma unroll
        for (int j = 0; j < 2; ++j) dst[j * 32 + lc] = f32_to_bf16(silu(acc[i][j][r]) * acc[i][j + 2][r]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
        if (row >= M) continue;
        const size_t base = static_cast<size_t>(row) * N + col0 + lc;
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) {
          if (col0 + j * 32 >= N) break;
          if constexpr (EPI == EPI_RESID32) {
            const bf16_t* res = static_cast<const bf16_t*>(ep.resid);
            static_cast<float*>(ep.out)[base + j * 32] = acc[i][j][r] + bf16_to_f32(res[base + j * 32]);
          } else {
            const float* res = static_cast<const float*>(ep.resid);
            static_cast<bf16_t*>(ep.out)[base + j * 32] = f32_to_bf16(acc[i][j][r] + res[base + j * 32]);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int EPI>
hipError_t launch(const bf16_t* A, const bf16_t* W, int M, int N, int K, const EpiArgs& ep,
                  hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, EPI>), dim3(tiles), dim3(kThreads), 0, s, A, W, M, N,
                     K, ep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                           const QkvEpilogue& q, hipStream_t s) {
  EpiArgs ep{};
  ep.qkv = q;
  return launch<256, 256, EPI_QKV>(A, W, M, N, K, ep, s);
}

hipError_t launch_gemm_resid_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                    const bf16_t* resid, float* out, hipStream_t s) {
  EpiArgs ep{};
  ep.resid = resid;
  ep.out = out;
  return launch<256, 128, EPI_RESID32>(A, W, M, N, K, ep, s);
}

hipError_t launch_gemm_resid_bf16out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                     const float* resid, bf16_t* out, hipStream_t s) {
  EpiArgs ep{};
  ep.resid = resid;
  ep.out = out;
  return launch<256, 128, EPI_RESID16>(A, W, M, N, K, ep, s);
}

hipError_t launch_gemm_swiglu(const bf16_t* A, const bf16_t* Wgu, int M, int N, int K,
                              bf16_t* out, hipStream_t s) {
  EpiArgs ep{};
  ep.out = out;
  return launch<256, 256, EPI_SWIGLU>(A, Wgu, M, N, K, ep, s);
}

}  // namespace llama
