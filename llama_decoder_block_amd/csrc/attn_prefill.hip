// Causal flash attention for prefill, head_dim 128: bf16 q and cache in, the
// output o in fp16 (the A operand of the fp16 o_proj GEMM).
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
// the online softmax and is fed to the PV product as two fp16 parts (hi + lo,
// about 22 significant bits; one fp16 alone keeps 11, and its rounding
// error, carried through the bf16 rounding of the attention output and
// amplified by the MLP, put the 70B-shape layer output beyond the bf16
// tolerance), with V converted to fp16 (exact) as it is staged.  The weights
// are taken against a reference max that lags the running max by at most 8
// (log2 units), so the output is rescaled only when some query's max moves
// past it, which after the first tile is rare; the weights then stay below
// 2^15, inside fp16's range.  The row-max exchange between the two lanes of a
// query is a permlane32 swap.  The Q fragments and each group's first K/V
// tile are loaded before the positions are read, so the kernel's start does
// not wait on three memory round trips in a row.  Query tiles are launched
// heaviest first across all heads and sequences (the causal workload grows
// with the tile index).  Tiles that lie wholly above a wave's diagonal are
// skipped, and the -inf mask is applied only on tiles that cross it.
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

// two bf16 (one 32-bit word) -> two fp16: exact for |v| in [2^-14, 65504]
// (fp16 carries bf16's 8 significant bits with 3 to spare); below that fp16's
// subnormals keep the value to within 2^-25
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  typedef __fp16 h16x2 __attribute__((ext_vector_type(2)));
  const h16x2 h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  return __builtin_bit_cast(uint32_t, h);
}

// p0, p1 -> fp16 pairs hi = p rounded toward zero, lo = fp16(p - hi) (the
// difference is exact in fp32; one rounding to fp16, to nearest even)
__device__ __forceinline__ void split_f16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
  uint32_t l;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(l) : "v"(p0), "v"(hi));
  asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(l) : "v"(p1), "v"(hi));
  lo = l;
}

// p0, p1 -> bf16 pairs hi = p rounded to nearest even, lo = bf16(p - hi)
// (the difference is exact in fp32): about 16 significant bits of p, and
// fp32's range
__device__ __forceinline__ void split_bf16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, b16x2));
  const float l0 = p0 - __uint_as_float(hi << 16), l1 = p1 - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){l0, l1}, b16x2));
}

// an int8 code as a float (exact), from byte i of w
__device__ __forceinline__ float code_f(uint32_t w, int i) {
  return static_cast<float>(static_cast<int>(static_cast<int8_t>(w >> (8 * i))));
}
// two exact floats -> their bf16 bits packed (the low halves are zero)
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// lazy rescaling: the reference max a wave's weights are taken against moves
// only when some query's tile max exceeds it by more than kLazy (log2 units);
// weights are 2^(s - ref + 15 - kLazy) <= 2^15, within fp16's range
constexpr float kLazy = 8.f;

// NGRP wave groups of 4 share the query tile and take every NGRP-th K/V tile
// (NGRP = 2 halves the longest serial chains when the grid holds at most two
// workgroups per CU; with more, two independent 4-wavefront workgroups per CU
// overlap better)
//
// Q8: the int8 cache (contiguous, or paged: code pools [n_pages, Hkv, page,
// 128] with scale pools [n_pages, Hkv, page]).  A row stands for code *
// scale; the codes are staged as bf16 (exact), so S^T = K_code Q^T is exact
// up to fp32 accumulation and each score is then multiplied by its row's K
// scale (times the softmax scale); the weight of slot j enters the P.V
// product as p_j * s_v(j) (bf16 hi + lo, fp32's range) against the V codes,
// while the row sum adds p_j.  The tile's 64 K and 64 V scales are staged in
// LDS.
template <int NGRP, bool PAGED, bool Q8>
__global__ __launch_bounds__(256 * NGRP, 3 - NGRP) void attn_prefill_kernel(
    const bf16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ pos, bf16_t* __restrict__ o,
    int o_frag, int n_seq, int T, int H, int Hkv, int max_pos, int span, KvPaging pg, int bidir,
    float scale_log2, const float* __restrict__ k_scale, const float* __restrict__ v_scale) {
  constexpr uint32_t ES = Q8 ? 1u : 2u;  // bytes per cached element
  __shared__ __attribute__((aligned(16))) bf16_t Ks[NGRP][2][BKV * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[NGRP][2][DH * VSTR];
  // Q8: [0, 64) the tile's K scales times the softmax scale, [64, 128) its V scales
  __shared__ __attribute__((aligned(16))) float Sc[NGRP][2][Q8 ? 2 * BKV : 4];

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
  // (paged: one page per tile at most, since pages hold a multiple of 64
  // slots; a tile whose page id is out of range reads zeros)
  const size_t srow = PAGED ? 0 : (static_cast<size_t>(b) * Hkv + g) * max_pos;  // the slice's first row
  const char* const kbase = static_cast<const char*>(k_cache);
  const char* const vbase = static_cast<const char*>(v_cache);
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(kbase + srow * DH * ES, static_cast<uint32_t>(max_pos) * DH * ES);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(vbase + srow * DH * ES, static_cast<uint32_t>(max_pos) * DH * ES);
  // Q8 scales: wave 0 of a group stages the tile's K scales, wave 1 its V scales
  // (16 lanes, 16 bytes each)
  const __amdgpu_buffer_rsrc_t sc_rs =
      make_rsrc(Q8 ? (wave == 0 ? k_scale : v_scale) + srow : nullptr, Q8 ? static_cast<uint32_t>(max_pos) * 4u : 0u);
  const bool sc_lane = Q8 && wave < 2 && lane < 16;
  // V: thread (vkg, vdg) loads slots 4 vkg .. 4 vkg + 3 at dims 8 vdg .. 8 vdg + 7
  // and writes them transposed as 8 rows (dims) of 4 slots, 8 bytes per row.
  // K: thread (kr, kc) loads 16-byte chunk kc of rows kr + 16 i, i < 4.
  // Every wave stages both, so the fp16 conversion work is spread evenly.
  // Q8: K thread (kr8, kc8) loads the 16 codes (bytes) kc8 of rows kr8 and
  // kr8 + 32; V thread (vkg, vdg) loads 8 codes per slot, 4 slots.
  const int vkg = tid & 15, vdg = tid >> 4;
  const int kr = tid >> 4, kc = tid & 15;
  const int kr8 = tid >> 3, kc8 = tid & 7;
  uint4 kreg[Q8 ? 2 : 4], vreg[Q8 ? 2 : 4];  // Q8: vreg holds the 4 slots' 8-byte code runs
  uint4 sreg = make_uint4(0, 0, 0, 0);
  auto gload = [&](int j0) {
    if constexpr (Q8) {
      __amdgpu_buffer_rsrc_t krs = k_rs, vrs = v_rs, srs = sc_rs;
      uint32_t row0 = static_cast<uint32_t>(j0);  // the tile's first row in the resources
      if constexpr (PAGED) {  // the tile's page (uniform); its scales sit at its code rows' indices
        const int bi = j0 / pg.page;
        const int blk = __builtin_amdgcn_readfirstlane(pg.block_table[static_cast<size_t>(b) * pg.blocks_per_seq + bi]);
        const bool ok = blk >= 0 && blk < pg.n_pages;
        const size_t prow = ok ? (static_cast<size_t>(blk) * Hkv + g) * pg.page : 0;
        const uint32_t nrow = ok ? static_cast<uint32_t>(pg.page) : 0u;
        krs = make_rsrc(kbase + prow * DH, nrow * DH);
        vrs = make_rsrc(vbase + prow * DH, nrow * DH);
        srs = make_rsrc((wave == 0 ? k_scale : v_scale) + prow, nrow * 4u);
        row0 = static_cast<uint32_t>(j0 % pg.page);
      }
      row0 = __builtin_amdgcn_readfirstlane(row0);
      const uint32_t so = row0 * DH;
#pragma unroll
      for (int i = 0; i < 2; ++i) kreg[i] = buf_load16(krs, static_cast<uint32_t>(kr8 * DH + kc8 * 16), so + 32 * i * DH);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint2 a = buf_load8(vrs, static_cast<uint32_t>((4 * vkg + 2 * i) * DH + vdg * 8), so);
        const uint2 c = buf_load8(vrs, static_cast<uint32_t>((4 * vkg + 2 * i + 1) * DH + vdg * 8), so);
        vreg[i] = make_uint4(a.x, a.y, c.x, c.y);
      }
      if (sc_lane) sreg = buf_load16(srs, static_cast<uint32_t>(lane) * 16u, row0 * 4u);
    } else {
      __amdgpu_buffer_rsrc_t krs = k_rs, vrs = v_rs;
      uint32_t so = static_cast<uint32_t>(j0) * DH * 2u;
      if constexpr (PAGED) {  // the tile's page (uniform)
        const int bi = j0 / pg.page;
        const int blk = __builtin_amdgcn_readfirstlane(pg.block_table[static_cast<size_t>(b) * pg.blocks_per_seq + bi]);
        const bool ok = blk >= 0 && blk < pg.n_pages;
        const size_t base = ok ? (static_cast<size_t>(blk) * Hkv + g) * pg.page * DH : 0;
        const uint32_t bytes = ok ? static_cast<uint32_t>(pg.page) * DH * 2u : 0u;
        krs = make_rsrc(kbase + base * 2, bytes);
        vrs = make_rsrc(vbase + base * 2, bytes);
        so = static_cast<uint32_t>(j0 % pg.page) * DH * 2u;
      }
      so = __builtin_amdgcn_readfirstlane(so);  // tile offset, uniform
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = buf_load16(vrs, (4 * vkg * DH + vdg * 8) * 2u, so + i * DH * 2u);
#pragma unroll
      for (int i = 0; i < 4; ++i) kreg[i] = buf_load16(krs, (kr * DH + kc * 8) * 2u, so + 16 * i * DH * 2u);
    }
  };
  auto lstore = [&](int st) {
    if constexpr (Q8) {  // codes -> bf16 (exact); V transposed as below
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t c[4] = {kreg[i].x, kreg[i].y, kreg[i].z, kreg[i].w};
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = pack_bf16_exact(code_f(c[e >> 1], 2 * (e & 1)), code_f(c[e >> 1], 2 * (e & 1) + 1));
        bf16_t* dst = &Ks[grp][st][(kr8 + 32 * i) * KSTR + kc8 * 16];
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
      }
      // vreg[i] = slots 4 vkg + 2 i (x, y) and 4 vkg + 2 i + 1 (z, w), dims 8 vdg ..
      const uint32_t vw[4][2] = {{vreg[0].x, vreg[0].y}, {vreg[0].z, vreg[0].w},
                                 {vreg[1].x, vreg[1].y}, {vreg[1].z, vreg[1].w}};
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint2 o;
        o.x = pack_bf16_exact(code_f(vw[0][d >> 2], d & 3), code_f(vw[1][d >> 2], d & 3));
        o.y = pack_bf16_exact(code_f(vw[2][d >> 2], d & 3), code_f(vw[3][d >> 2], d & 3));
        *reinterpret_cast<uint2*>(&Vt[grp][st][(vdg * 8 + d) * VSTR + 4 * vkg]) = o;
      }
      if (sc_lane) {
        float4 f = make_float4(__uint_as_float(sreg.x), __uint_as_float(sreg.y), __uint_as_float(sreg.z),
                               __uint_as_float(sreg.w));
        if (wave == 0) f = make_float4(f.x * scale_log2, f.y * scale_log2, f.z * scale_log2, f.w * scale_log2);
        *reinterpret_cast<float4*>(&Sc[grp][st][wave * BKV + 4 * lane]) = f;
      }
    } else {
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
    }
  };

  // the group's first K/V tile, in flight while the positions are read (a
  // tile at or past the span is not needed: every tile a query sees starts
  // below it, and a paged table has no entry there)
  if (grp * BKV < span) gload(grp * BKV);

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
  pq = min(pq, span - 1);

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

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (grp < ntiles) lstore(0);
  __syncthreads();

  const int k_row0 = kappa(lq) * KSTR + hl * 8;
  const float sl = Q8 ? 1.f : scale_log2;  // Q8 scores already carry the softmax scale
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
      if constexpr (Q8) {  // scores times the rows' K scales (which carry the softmax scale)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const float* c = &Sc[grp][st][32 * kb + 16 * hh + 8 * hl];
            const float4 c0 = *reinterpret_cast<const float4*>(c), c1 = *reinterpret_cast<const float4*>(c + 4);
            const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) sacc[kb][8 * hh + e] *= cs[e];
          }
      }
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
      // scaling commute).  Output and sum carry the same factor
      // 2^(15 - kLazy - m_run), which the final division cancels.  The
      // rescale is skipped unless some query of the wave has a tile max more
      // than kLazy above its reference m_run.
      const float m_tile = mt * sl;
      if (__any(m_tile > m_run + kLazy)) {  // wave-uniform
        const float m_new = fmaxf(m_tile, m_run);
        const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);  // 0 from -inf
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        m_run = m_new;
      }
      const float m_sh = (m_run == -INFINITY ? 0.f : m_run) - (15.f - kLazy);
      // Each weight p = 2^(s - m_run + 15 - kLazy) <= 2^15 goes to the P.V
      // product as two fp16 parts: hi = p cut to fp16's 11 significant bits,
      // lo = fp16(p - hi), so hi + lo keeps about 22 bits of p (fp16
      // alone keeps 11, which flips the bf16 rounding of the attention output
      // far more often than fp32 weights would).  The row sum adds p in fp32.
      // (Q8: the weights enter P.V times the rows' V scales, as bf16 hi + lo.)
      float lsum = 0.f;
      uint32_t ph[2][2][4], pl[2][2][4];  // [kb][half][packed fp16 (Q8: bf16) pair]
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float vs[8];
          if constexpr (Q8) {
            const float* c = &Sc[grp][st][BKV + 32 * kb + 16 * hh + 8 * hl];
            const float4 c0 = *reinterpret_cast<const float4*>(c), c1 = *reinterpret_cast<const float4*>(c + 4);
            vs[0] = c0.x; vs[1] = c0.y; vs[2] = c0.z; vs[3] = c0.w;
            vs[4] = c1.x; vs[5] = c1.y; vs[6] = c1.z; vs[7] = c1.w;
          }
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int r = 8 * hh + e;
            const float p0 = fast_exp2(fmaf(sacc[kb][r], sl, -m_sh));
            const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], sl, -m_sh));
            if constexpr (Q8)
              split_bf16(p0 * vs[e], p1 * vs[e + 1], ph[kb][hh][e >> 1], pl[kb][hh][e >> 1]);
            else
              split_f16(p0, p1, ph[kb][hh][e >> 1], pl[kb][hh][e >> 1]);
            lsum += p0 + p1;
          }
        }
      l_run += lsum;
      // O^T += V^T (P_hi + P_lo)^T over 4 blocks of 16 slots
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint4 uh = make_uint4(ph[kb][half][0], ph[kb][half][1], ph[kb][half][2], ph[kb][half][3]);
          const uint4 ul = make_uint4(pl[kb][half][0], pl[kb][half][1], pl[kb][half][2], pl[kb][half][3]);
          const int kcol = (kb * 2 + half) * 16;
          if constexpr (Q8) {
            bf16x8 a[4];
#pragma unroll
            for (int fd = 0; fd < 4; ++fd) {
              a[fd] = *reinterpret_cast<const bf16x8*>(&Vt[grp][st][v_row0 + fd * 32 * VSTR + kcol]);
              oacc[fd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fd], as_bf16x8(uh), oacc[fd], 0, 0, 0);
            }
#pragma unroll
            for (int fd = 0; fd < 4; ++fd)
              oacc[fd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fd], as_bf16x8(ul), oacc[fd], 0, 0, 0);
          } else {
            const f16x8 bh = __builtin_bit_cast(f16x8, uh), bl = __builtin_bit_cast(f16x8, ul);
            f16x8 a[4];
#pragma unroll
            for (int fd = 0; fd < 4; ++fd) {
              a[fd] = *reinterpret_cast<const f16x8*>(&Vt[grp][st][v_row0 + fd * 32 * VSTR + kcol]);
              oacc[fd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[fd], bh, oacc[fd], 0, 0, 0);
            }
#pragma unroll
            for (int fd = 0; fd < 4; ++fd) oacc[fd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[fd], bl, oacc[fd], 0, 0, 0);
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
      w.x = pack_f16x2_sat(oacc[fd][4 * rq] * inv, oacc[fd][4 * rq + 1] * inv);
      w.y = pack_f16x2_sat(oacc[fd][4 * rq + 2] * inv, oacc[fd][4 * rq + 3] * inv);
      // four consecutive dims stay contiguous in fragment order as well
      const int col = fd * 32 + 8 * rq + 4 * hl;
      bf16_t* dst = o_frag ? o + frag_index(static_cast<int>(row), h * DH + col, static_cast<int>(qstride)) : orow + col;
      *reinterpret_cast<uint2*>(dst) = w;
    }
}

}  // namespace

hipError_t launch_attn_prefill(const bf16_t* q, const void* k_cache, const void* v_cache,
                               const int32_t* pos, bf16_t* o, int o_frag, int B, int T, int n_heads,
                               int n_kv_heads, int max_pos, int span, const KvPaging& pg, int bidir,
                               hipStream_t s, const float* k_scale, const float* v_scale) {
  if (pg.block_table && (pg.page % BKV || pg.page <= 0 || span > pg.blocks_per_seq * pg.page))
    return hipErrorInvalidValue;
  const bool q8 = k_scale != nullptr;
  if (q8 && !v_scale) return hipErrorInvalidValue;
  if (o_frag && B * T > kSkinnyMaxTokens) return hipErrorInvalidValue;
  const int n_wg = (T + BQ - 1) / BQ * n_heads * B;
  const dim3 grid(static_cast<unsigned>(n_wg));
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(DH)));
#define LLAMA_ATTN_LAUNCH(NG, PG, Q8)                                                                          \
  hipLaunchKernelGGL((attn_prefill_kernel<NG, PG, Q8>), grid, dim3(256 * NG), 0, s, q, k_cache, v_cache, pos, o, \
                     o_frag, B, T, n_heads, n_kv_heads, max_pos, span, pg, bidir, scale_log2, k_scale, v_scale)
  const bool two = n_wg <= 2 * n_cu;  // few workgroups: halve each query tile's chain
  if (pg.block_table && q8) {
    if (two) LLAMA_ATTN_LAUNCH(2, true, true); else LLAMA_ATTN_LAUNCH(1, true, true);
  } else if (pg.block_table) {
    if (two) LLAMA_ATTN_LAUNCH(2, true, false); else LLAMA_ATTN_LAUNCH(1, true, false);
  } else if (q8) {
    if (two) LLAMA_ATTN_LAUNCH(2, false, true); else LLAMA_ATTN_LAUNCH(1, false, true);
  } else {
    if (two) LLAMA_ATTN_LAUNCH(2, false, false); else LLAMA_ATTN_LAUNCH(1, false, false);
  }
#undef LLAMA_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace llama
