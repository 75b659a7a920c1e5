// Causal flash attention for prefill, bf16 in and out, head_dim 128.
//
// Computes, for every query token m (sequence b, position p_m) and query head
// h, o = sum_j softmax_j(q.k_j / sqrt(128)) v_j over the cache slots
// j = 0 .. p_m of sequence b and kv head g = h / (H / Hkv).  The
// bidirectional variant (the SigLIP encoder's attention on the "LARQL
// multimodal support" page: the causal kernel without its mask condition)
// uses j = 0 .. P_b for every query, P_b = the largest position of sequence b
// among the call's tokens.
//
// Sources: "LMDrive LLM core inference unit" page, §2.3 LlamaAttention
// (scores q k^T / sqrt(head_dim), additive mask, softmax, weights times v;
// repeat_kv for grouped-query attention, which here is plain kv-head
// indexing); "LLM mechanics lecture notes" §02.1 (M_ij = -inf for j > i,
// added before the softmax, so future weights are exactly zero) and Ch.04
// (a query reads every visible cached K/V).  The mask compares cache slot
// (= position) with the query's position, which equals the notes' index mask
// when positions are 0..T-1 and extends it to a prefill that continues a cache.
//
// gfx950 design.  One workgroup = 128 queries of one head; each of its 4
// query wavefronts owns 32 queries.  When the grid holds at most two
// workgroups per CU, the kernel time is set by the longest query tiles'
// serial chains, so a second group of 4 wavefronts takes every other K/V tile
// and the two running states (max, sum, O) are merged through LDS at the end;
// such a workgroup needs 140 KB of LDS, so a CU runs one at a time and the
// heaviest-first order balances the two rounds.  K/V tiles of 64 slots are staged in LDS (two
// stages, register prefetch of the next tile).  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so each lane owns
// one query: its row max / row sum need only a lane-pair exchange.  The K rows
// fed to the MFMA are permuted (bits 2 and 3 of the row index swapped) so that
// a lane's 16 score registers are two runs of 8 consecutive keys — exactly the
// B operand of the next MFMA, O^T += V^T P^T, with no register shuffling.  V
// is transposed to [dd][slot] while it is written to LDS.  P stays in fp32 in
// the online softmax and is fed to the PV product in fp16 (11 significant bits
// against bf16's 8), with V converted to fp16 as it is staged.  The weights
// are taken against a reference max that moves only when a tile's max
// exceeds it by more than 8 (log2 units), so the output is rarely rescaled,
// and the row sum adds the same fp16 weights the product multiplies.  The
// row-max exchange between the two lanes of a query is a permlane32 swap.
// Query tiles are launched heaviest first across all heads and sequences (the
// causal workload grows with the tile index).  Tiles that lie wholly above a wave's diagonal are skipped, and
// the -inf mask is applied only on tiles that cross it.
#include "common.h"

#include <math.h>

#include <type_traits>

namespace llama {
namespace {

constexpr int DH = 128;
constexpr int BQ = 128;          // queries per workgroup
constexpr int BKV = 64;          // cache slots per tile
constexpr int KSTR = DH + 8;     // LDS row of K, bf16 elements (272 B)
constexpr int VSTR = BKV + 8;    // LDS row of V^T, bf16 elements (144 B)

__device__ __forceinline__ int kappa(int m) {  // swap bits 2 and 3
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// two bf16 (one 32-bit word) -> two fp16: exact for |v| in [2^-14, 65504]
// (fp16 carries bf16's 8 significant bits with 3 to spare); below that fp16's
// subnormals keep the value to within 2^-25
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  typedef __fp16 h16x2 __attribute__((ext_vector_type(2)));
  const h16x2 h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  return __builtin_bit_cast(uint32_t, h);
}

// two fp32 -> two fp16, round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}

// NGRP wave groups of 4 share the query tile and take every NGRP-th K/V tile
// (NGRP = 2 halves the longest serial chains when the grid holds at most two
// workgroups per CU; with more, two independent 4-wavefront workgroups per CU
// overlap better)
template <int NGRP>
__global__ __launch_bounds__(256 * NGRP, 3 - NGRP) void attn_prefill_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ pos, bf16_t* __restrict__ o,
    int o_frag, int n_seq, int T, int H, int Hkv, int max_pos, int bidir, float scale_log2) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[NGRP][2][BKV * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[NGRP][2][DH * VSTR];

  // 1-D grid, heaviest query tiles of every (sequence, head) first
  const int n_qt = (T + BQ - 1) / BQ;
  const int per_qt = H * n_seq;
  const int qt = n_qt - 1 - static_cast<int>(blockIdx.x) / per_qt;
  const int h = static_cast<int>(blockIdx.x) % per_qt % H, b = static_cast<int>(blockIdx.x) % per_qt / H;
  const int g = h / (H / Hkv);
  // group grp takes tiles grp, grp + NGRP, ...; wave w of either group owns
  // queries 32 w .. 32 w + 31 of the tile
  // (group and wave as scalars, so that what derives from them stays uniform)
  const int grp = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 8);
  const int tid = threadIdx.x & 255, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, lq = lane & 31;

  // ---- this lane's query
  const int t = qt * BQ + wave * 32 + lq;
  const bool valid = t < T;
  const size_t row = static_cast<size_t>(b) * T + (valid ? t : 0);
  int pq = valid ? pos[row] : -1;
  if (bidir) {  // uniform: every query of the sequence sees up to its largest position in the call
    int sm = -1;
    for (int i = static_cast<int>(threadIdx.x); i < T; i += static_cast<int>(blockDim.x))
      sm = max(sm, pos[static_cast<size_t>(b) * T + i]);
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) sm = max(sm, __shfl_xor(sm, sft, 64));
    __shared__ int s_seq[4 * NGRP];
    if (lane == 0) s_seq[threadIdx.x >> 6] = sm;
    __syncthreads();
    for (int w = 0; w < 4 * NGRP; ++w) sm = max(sm, s_seq[w]);
    if (valid) pq = sm;
  }
  pq = min(pq, max_pos - 1);

  // wave / workgroup position range
  int wmax = pq, wmin = valid ? pq : 0x7fffffff;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    wmax = max(wmax, __shfl_xor(wmax, s, 64));
    wmin = min(wmin, __shfl_xor(wmin, s, 64));
  }
  __shared__ int s_max[4];
  if (lane == 0 && grp == 0) s_max[wave] = wmax;
  __syncthreads();
  const int gmax = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  if (gmax < 0) return;  // no valid query in the whole tile (uniform)
  const int ntiles = gmax / BKV + 1;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query lq, dims s*16 + hl*8 .. +8
  const size_t qstride = static_cast<size_t>(H) * DH;
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + row * qstride + static_cast<size_t>(h) * DH + hl * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 u = valid ? *reinterpret_cast<const uint4*>(qrow + s * 16) : make_uint4(0, 0, 0, 0);
      qf[s] = as_bf16x8(u);
    }
  }

  // ---- K / V tile staging (buffer loads over this (b, g) cache slice), each
  // group for its own tiles: every thread loads 4 K and 4 V chunks of 16 bytes.
  const size_t slice = (static_cast<size_t>(b) * Hkv + g) * max_pos * DH;
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k_cache + slice, static_cast<uint32_t>(max_pos) * DH * 2u);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v_cache + slice, static_cast<uint32_t>(max_pos) * DH * 2u);
  // V: thread (vkg, vdg) loads slots 4 vkg .. 4 vkg + 3 at dims 8 vdg .. 8 vdg + 7
  // and writes them transposed as 8 rows (dims) of 4 slots, 8 bytes per row.
  // K: thread (kr, kc) loads 16-byte chunk kc of rows kr + 16 i, i < 4.
  // Every wave stages both, so the fp16 conversion work is spread evenly.
  const int vkg = tid & 15, vdg = tid >> 4;
  const int kr = tid >> 4, kc = tid & 15;
  uint4 kreg[4], vreg[4];
  auto gload = [&](int j0) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(j0) * DH * 2u);  // tile offset, uniform
#pragma unroll
    for (int i = 0; i < 4; ++i) vreg[i] = buf_load16(v_rs, ((4 * vkg + i) * DH + vdg * 8) * 2u, so);
#pragma unroll
    for (int i = 0; i < 4; ++i) kreg[i] = buf_load16(k_rs, ((kr + 16 * i) * DH + kc * 8) * 2u, so);
  };
  auto lstore = [&](int st) {
    // V goes to LDS as fp16 (the P.V product runs in fp16 so that P keeps
    // 11 significant bits in one operand)
    uint32_t w[16];  // w[4 * slot + dim/2]
    {
      const uint32_t* wb = reinterpret_cast<const uint32_t*>(vreg);
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = bf16x2_to_f16x2(wb[i]);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
      uint2 o;
      o.x = __builtin_amdgcn_perm(w[4 * 1 + (d >> 1)], w[4 * 0 + (d >> 1)], sel);
      o.y = __builtin_amdgcn_perm(w[4 * 3 + (d >> 1)], w[4 * 2 + (d >> 1)], sel);
      *reinterpret_cast<uint2*>(&Vt[grp][st][(vdg * 8 + d) * VSTR + 4 * vkg]) = o;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&Ks[grp][st][(kr + 16 * i) * KSTR + kc * 8]) = kreg[i];
  };

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (grp < ntiles) {
    gload(grp * BKV);
    lstore(0);
  }
  __syncthreads();

  const int k_row0 = kappa(lq) * KSTR + hl * 8;
  const int v_row0 = lq * VSTR + hl * 8;

  // the trip count is the same for both groups (they share the barrier)
  for (int i = 0; i * NGRP < ntiles; ++i) {
    const int it = i * NGRP + grp;
    const int st = i & 1;
    const int j0 = it * BKV;
    if (it + NGRP < ntiles) gload(j0 + NGRP * BKV);

    // one 64-slot tile; MASK: the tile crosses the diagonal of some query of this wave
    auto tile = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // S^T for 2 blocks of 32 slots (unscaled scores)
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[grp][st][k_row0 + kb * 32 * KSTR + s * 16]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
        }
      }
      // mask and tile max.  Register r of block kb is slot
      // j0 + 32 kb + 16 (r/8) + 8 hl + r%8.
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (MASK) {
            const int j = j0 + 32 * kb + 16 * (r >> 3) + 8 * hl + (r & 7);
            if (j > pq) sacc[kb][r] = -INFINITY;
          }
          mt = fmaxf(mt, sacc[kb][r]);
        }
      {  // lanes l and l ^ 32 hold the two halves of a query's slots
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // Reference max m_run (log2 units; the scale is positive, so max and
      // scaling commute).  It moves only when a tile's max exceeds it by more
      // than 8, so the running output is rarely rescaled; the weights
      // 2^(s - m_run + 7) then stay within 2^15 (fp16 range) and are fp16
      // normals down to 2^-21 of the reference.  Output and sum carry the
      // same factor, which the final division cancels.
      const float m_tile = mt * scale_log2;
      if (__any(m_tile > m_run + 8.f)) {  // wave-uniform
        const float m_new = m_tile > m_run + 8.f ? m_tile : m_run;
        const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);  // 0 from -inf
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        m_run = m_new;
      }
      const float m_sh = (m_run == -INFINITY ? 0.f : m_run) - 7.f;
      // the row sum adds the fp16 weights the P.V product multiplies
      const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
      float lsum[2] = {0.f, 0.f};
      uint32_t ph[2][2][4];  // [kb][half][packed fp16 pair]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(sacc[kb][r], scale_log2, -m_sh));
          const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], scale_log2, -m_sh));
          const uint32_t pp = pack_f16x2(p0, p1);
          ph[kb][r >> 3][(r & 7) >> 1] = pp;
          lsum[kb] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pp), ones, lsum[kb], false);
        }
      l_run += lsum[0] + lsum[1];
      // O^T += V^T P^T over 4 blocks of 16 slots
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f16x8 bp = __builtin_bit_cast(f16x8, make_uint4(ph[kb][half][0], ph[kb][half][1], ph[kb][half][2], ph[kb][half][3]));
          const int kcol = (kb * 2 + half) * 16;
#pragma unroll
          for (int fd = 0; fd < 4; ++fd) {
            const f16x8 a = *reinterpret_cast<const f16x8*>(&Vt[grp][st][v_row0 + fd * 32 * VSTR + kcol]);
            oacc[fd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bp, oacc[fd], 0, 0, 0);
          }
        }
    };
    if (it < ntiles && j0 <= wmax) {  // wave-uniform: skip tiles wholly above this wave's diagonal
      if (j0 + BKV - 1 > wmin)
        tile(std::true_type{});
      else
        tile(std::false_type{});
    }
    if (it + NGRP < ntiles) lstore(st ^ 1);
    __syncthreads();
  }

  // ---- merge group 1's running state (max, sum, O) into group 0's.  The K
  // stages are free after the loop's last barrier.
  if constexpr (NGRP == 2) {
    static_assert(sizeof(Ks) >= 4 * 66 * 64 * sizeof(float), "merge buffer");
    float* mb = reinterpret_cast<float*>(&Ks[0][0][0]) + wave * 66 * 64 + lane;  // [wave][66][lane]
    if (grp == 1) {
      mb[0] = m_run;
      mb[64] = l_run;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb[(2 + 16 * i + r) * 64] = oacc[i][r];
    }
    __syncthreads();
    if (grp == 1) return;
    {
      const float m1 = mb[0], l1 = mb[64];
      const float m = fmaxf(m_run, m1);
      const float mu = m == -INFINITY ? 0.f : m;
      const float a0 = fast_exp2(m_run - mu), a1 = fast_exp2(m1 - mu);
      l_run = l_run * a0 + l1 * a1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = oacc[i][r] * a0 + mb[(2 + 16 * i + r) * 64] * a1;
    }
    }

  // ---- normalise and store: oacc[fd] register r is dim fd*32 + 8(r/4) + 4 hl + r%4
  if (!valid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  bf16_t* orow = o + row * qstride + static_cast<size_t>(h) * DH;
#pragma unroll
  for (int fd = 0; fd < 4; ++fd)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      uint2 w;
      w.x = pack_bf16x2(oacc[fd][4 * rq] * inv, oacc[fd][4 * rq + 1] * inv);
      w.y = pack_bf16x2(oacc[fd][4 * rq + 2] * inv, oacc[fd][4 * rq + 3] * inv);
      // four consecutive dims stay contiguous in fragment order as well
      const int col = fd * 32 + 8 * rq + 4 * hl;
      bf16_t* dst = o_frag ? o + frag_index(static_cast<int>(row), h * DH + col, static_cast<int>(qstride)) : orow + col;
      *reinterpret_cast<uint2*>(dst) = w;
    }
}

}  // namespace

hipError_t launch_attn_prefill(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache,
                               const int32_t* pos, bf16_t* o, int o_frag, int B, int T, int n_heads,
                               int n_kv_heads, int max_pos, int bidir, hipStream_t s) {
  if (o_frag && B * T > kSkinnyMaxTokens) return hipErrorInvalidValue;
  const int n_wg = (T + BQ - 1) / BQ * n_heads * B;
  const dim3 grid(static_cast<unsigned>(n_wg));
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(DH)));
  if (n_wg <= 2 * n_cu)  // few workgroups: halve each query tile's chain
    hipLaunchKernelGGL(attn_prefill_kernel<2>, grid, dim3(512), 0, s, q, k_cache, v_cache, pos, o, o_frag, B, T,
                       n_heads, n_kv_heads, max_pos, bidir, scale_log2);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<1>, grid, dim3(256), 0, s, q, k_cache, v_cache, pos, o, o_frag, B, T,
                       n_heads, n_kv_heads, max_pos, bidir, scale_log2);
  return hipGetLastError();
}

}  // namespace llama
