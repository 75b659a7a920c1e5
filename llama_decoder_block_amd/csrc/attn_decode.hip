// Decode attention: one new query per sequence over its whole cache,
// o_h = softmax(q_h K_{0..p}^T / sqrt(128)) V_{0..p}, bf16 cache, fp32 math,
// o stored as fp16 (the A operand of the fp16 o_proj GEMM).
//
// Sources: "LLM mechanics lecture notes" Ch.04 (decode appends k_t, v_t and
// lets q_t read every visible cached K/V; decode stays memory bound and grows
// with context) and "LMDrive LLM core inference unit" page §2.3 (scores,
// softmax, weighted sum of values; repeat_kv grouped-query attention, here
// kv-head indexing so a K/V row read serves all query heads of its group).
//
// gfx950 design: the cache is streamed once at HBM rate, K and V together,
// with nontemporal loads (each row is read once per call).
//   * workgroup (split s, kv head g, sequence b) takes slots
//     [s L, (s+1) L) ∩ [0, p]; the split length is chosen so the grid holds
//     about 1024 workgroups (4 per CU; at 3 or 4 query heads per workgroup
//     their wavefronts need more than 128 VGPRs and 3 or 2 are resident at
//     a time), or 256 when a workgroup serves 5 or more query heads (its
//     wavefronts then need more than 256 VGPRs, one workgroup per CU).  With that many (sequence, kv head) pairs already,
//     there is one split and the workgroup writes the normalised output
//     itself; otherwise each split writes (max, sum, unnormalised o[128]) per
//     head and a second kernel merges them (the standard split-softmax merge);
//   * a K or V row (128 dims = 256 B) is read by 16 lanes with 16-byte loads,
//     so a wavefront reads 4 consecutive rows = 1 KB contiguous per load; each
//     lane keeps the next iteration's 4 K and 4 V loads in flight while it
//     works on the current ones;
//   * 16 row groups of 16 lanes each own the slots of one residue mod 16 and
//     run an online softmax over them (running max and sum in fp32, base-2
//     exponent with the scale folded into q): per 4 slots, the scores come
//     from a 16-lane DPP reduction, the running output (8 dims x heads per
//     lane) is rescaled once and the 4 weighted V rows are added;
//   * the 16 row-group states are merged with the same rule (shuffles within a
//     wave, LDS across the 4 waves).
#include "common.h"

#include <math.h>

namespace llama {
namespace {

constexpr int DH = 128;
constexpr int kMaxRep = 8;  // query heads handled per workgroup
// workgroups wanted per call: four per CU (of 256) while a wavefront fits in
// 256 VGPRs; one per CU once R >= 5 query heads push it past that
__host__ __device__ constexpr int target_wgs(int R) { return R <= 4 ? 1024 : 256; }

// (m1, l1, a1) <- merge with (m2, l2, a2): both scaled to the larger max
__device__ __forceinline__ void softmax_merge(float& m1, float& l1, float* a1, float m2, float l2,
                                              const float* a2, int n) {
  const float m = fmaxf(m1, m2);
  const float mu = m == -INFINITY ? 0.f : m;
  const float c1 = fast_exp2(m1 - mu), c2 = fast_exp2(m2 - mu);
  l1 = l1 * c1 + l2 * c2;
  for (int e = 0; e < n; ++e) a1[e] = a1[e] * c1 + a2[e] * c2;
  m1 = m;
}

// Q8: the int8 cache (codes [B, Hkv, max_pos, 128], one fp32 scale per row
// in ksc / vsc [B, Hkv, max_pos]; paged: code pools [n_pages, Hkv, page, 128]
// and scale pools [n_pages, Hkv, page], a slot's scale at its code row's
// index): a row group's 16 lanes read its 128 codes with 8-byte loads (a
// wavefront: 4 rows = 512 contiguous bytes per load) and the row's scale;
// the score is the code dot product times the key row's scale, and a weight
// multiplies the value codes after taking the value row's scale.
template <int R, bool PAGED, bool Q8>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const bf16_t* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, const int32_t* __restrict__ pos, float* __restrict__ part,
    bf16_t* __restrict__ o, int o_frag, int H, int Hkv, int max_pos, int span, KvPaging pg, int L, int n_split,
    float scale_log2, const float* __restrict__ ksc, const float* __restrict__ vsc) {
  __shared__ float red_ml[4][R][2];
  __shared__ float red_o[4][R][DH];

  const int s = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int n_rep = H / Hkv;
  const int chunks = n_rep / R;            // workgroups per kv head
  const int g = hg / chunks;
  const int h0 = g * n_rep + (hg % chunks) * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dc = lane & 15;                // 8-dim chunk of a row
  const int sub = wave * 4 + (lane >> 4);  // row group: slots = sub (mod 16)

  const int p = min(pos[b], span - 1);
  const int j_begin = s * L;
  const int j_end = min(j_begin + L, p + 1);
  const int n = j_end - j_begin;
  float* out = part + ((static_cast<size_t>(b) * H + h0) * n_split + s) * (DH + 2);
  if (n <= 0) {  // nothing visible in this split (only with several splits)
    for (int i = tid; i < R * (DH + 2); i += 256) {
      const int r = i / (DH + 2), e = i % (DH + 2);
      out[static_cast<size_t>(r) * n_split * (DH + 2) + e] = e == 0 ? -INFINITY : 0.f;
    }
    return;
  }

  // query slices, 8 dims per lane per head, pre-scaled so scores are in log2 units
  float qv[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint4 u = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(b) * H + h0 + r) * DH + dc * 8);
    qv[r][0] = lo_bf16(u.x); qv[r][1] = hi_bf16(u.x); qv[r][2] = lo_bf16(u.y); qv[r][3] = hi_bf16(u.y);
    qv[r][4] = lo_bf16(u.z); qv[r][5] = hi_bf16(u.z); qv[r][6] = lo_bf16(u.w); qv[r][7] = hi_bf16(u.w);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[r][e] *= scale_log2;
  }

  const size_t slice = PAGED ? 0 : (static_cast<size_t>(b) * Hkv + g) * max_pos * DH;
  // (element offsets: 2-byte bf16 or 1-byte int8 elements)
  constexpr int ES = Q8 ? 1 : 2;
  const char* K = static_cast<const char*>(k_cache) + (slice + static_cast<size_t>(j_begin) * DH + dc * 8) * ES;
  const char* V = static_cast<const char*>(v_cache) + (slice + static_cast<size_t>(j_begin) * DH + dc * 8) * ES;
  // int8: the scales of this (sequence, kv head)'s slots from j_begin on
  // (paged: indexed by the same pool rows as the codes)
  const float* KS = Q8 ? ksc + slice / DH + j_begin : nullptr;
  const float* VS = Q8 ? vsc + slice / DH + j_begin : nullptr;
  // Paged: the 64 slots of one iteration, s0 .. s0 + 63 with s0 = j_begin +
  // j - sub (j_begin and L are multiples of 64), lie in one page.  Slot s0 + i
  // is row (page Hkv + g) page + s0 % page + i of the pool; as an offset from
  // K's row for slot j_begin + j (the contiguous case's offset j), add this.
  auto page_shift = [&](int j) -> long long {
    const int s0 = j_begin + (j - sub);  // uniform
    const int bi = min(s0 / pg.page, pg.blocks_per_seq - 1);  // (a slot past the split reads nothing)
    int blk = __builtin_amdgcn_readfirstlane(pg.block_table[static_cast<size_t>(b) * pg.blocks_per_seq + bi]);
    blk = min(max(blk, 0), pg.n_pages - 1);  // an invalid page id reads some page, never out of bounds
    return (static_cast<long long>(blk) * Hkv + g) * pg.page + s0 % pg.page - s0;
  };

  float m[R], l[R], acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  // the 4 K and 4 V rows of this row group's next slots j, j + 16, ...
  // (int8: 8 codes per lane in .x / .y, and the rows' scales)
  // (int8: of a row group's 16 lanes, lane u < 4 loads the key scale of its
  // u-th row and lane 4 + u the value scale; the rest of the group takes them
  // by lane shuffles, one scale load per lane instead of eight)
  const float* const SS = (dc & 4) ? VS : KS;
  auto fetch = [&](int j, uint4 (&ku)[4], uint4 (&vu)[4], float& sw) {
    const long long base = PAGED ? page_shift(j) : 0;
    if constexpr (Q8) {
      const int js = j + 16 * (dc & 3);
      sw = dc < 8 && js < n ? SS[base + js] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = j + 16 * u < n;
      const long long r = base + j + 16 * u;
      if constexpr (Q8) {
        const uint2 k8 = ok ? load8_nt(K + r * DH) : make_uint2(0, 0);
        const uint2 v8 = ok ? load8_nt(V + r * DH) : make_uint2(0, 0);
        ku[u] = make_uint4(k8.x, k8.y, 0, 0);
        vu[u] = make_uint4(v8.x, v8.y, 0, 0);
      } else {
        ku[u] = ok ? load16_nt(K + r * DH * 2) : make_uint4(0, 0, 0, 0);
        vu[u] = ok ? load16_nt(V + r * DH * 2) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // 8 values of a lane's row slice: bf16 pairs, or (int8) signed bytes
  auto unpack8 = [&](const uint4& u, float (&f)[8]) {
    if constexpr (Q8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = static_cast<float>(static_cast<int8_t>(u.x >> (8 * e)));
        f[4 + e] = static_cast<float>(static_cast<int8_t>(u.y >> (8 * e)));
      }
    } else {
      f[0] = lo_bf16(u.x); f[1] = hi_bf16(u.x); f[2] = lo_bf16(u.y); f[3] = hi_bf16(u.y);
      f[4] = lo_bf16(u.z); f[5] = hi_bf16(u.z); f[6] = lo_bf16(u.w); f[7] = hi_bf16(u.w);
    }
  };
  // the rows of the next iteration are fetched before this one's arithmetic
  // (register prefetch): with R >= 5 heads a CU holds one workgroup only, and
  // with fewer, where up to four share a CU, it still measured 1% (R = 1, 2)
  // to 6% (R = 4) faster than fetching at the top of each iteration
  uint4 ku[4], vu[4];  // this iteration's rows
  float sw = 0.f;        // (int8) one of their scales (see fetch)
  fetch(sub, ku, vu, sw);
  for (int j = sub; j < n; j += 64) {
    uint4 kn[4], vn[4];  // the next iteration's rows (prefetch)
    float swn = 0.f;
    fetch(j + 64, kn, vn, swn);
    float kss[4], vss[4];  // (int8) the scales of this row group's rows
    if constexpr (Q8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kss[u] = __shfl(sw, (lane & 48) + u, 64);
        vss[u] = __shfl(sw, (lane & 48) + 4 + u, 64);
      }
    }
    float sc[R][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float kf[8];
      unpack8(ku[u], kf);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += qv[r][e] * kf[e];
        d = sum16_dpp(d);  // the 16 lanes of the row group
        if constexpr (Q8) d *= kss[u];
        sc[r][u] = j + 16 * u < n ? d : -INFINITY;  // slots past the split are masked
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float mx = fmaxf(fmaxf(sc[r][0], sc[r][1]), fmaxf(sc[r][2], sc[r][3]));
      const float m_new = fmaxf(m[r], mx);  // finite: slot j itself is visible
      const float c = fast_exp2(m[r] - m_new);
#pragma unroll
      for (int u = 0; u < 4; ++u) sc[r][u] = fast_exp2(sc[r][u] - m_new);  // weights; 0 where masked
      l[r] = l[r] * c + ((sc[r][0] + sc[r][1]) + (sc[r][2] + sc[r][3]));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= c;
      m[r] = m_new;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float vf[8];
      unpack8(vu[u], vf);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float wgt = Q8 ? sc[r][u] * vss[u] : sc[r][u];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] += wgt * vf[e];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ku[u] = kn[u];
      vu[u] = vn[u];
    }
    sw = swn;
  }

  // merge the 4 row groups of a wave (lanes 16 and 32 apart), then the 4 waves
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float m2 = __shfl_xor(m[r], x, 64), l2 = __shfl_xor(l[r], x, 64);
      float a2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(acc[r][e], x, 64);
      softmax_merge(m[r], l[r], acc[r], m2, l2, a2, 8);
    }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][r][dc * 8 + e] = acc[r][e];
      if (dc == 0) { red_ml[wave][r][0] = m[r]; red_ml[wave][r][1] = l[r]; }
    }
  }
  __syncthreads();
  for (int i = tid; i < R * DH; i += 256) {
    const int r = i / DH, d = i % DH;
    float mm = red_ml[0][r][0], ll = red_ml[0][r][1], aa = red_o[0][r][d];
#pragma unroll
    for (int w = 1; w < 4; ++w) softmax_merge(mm, ll, &aa, red_ml[w][r][0], red_ml[w][r][1], &red_o[w][r][d], 1);
    if (n_split == 1) {
      const int hh = h0 + r;
      const size_t at = o_frag ? frag_index(b, hh * DH + d, H * DH) : (static_cast<size_t>(b) * H + hh) * DH + d;
      o[at] = f32_to_f16_sat(ll > 0.f ? aa / ll : 0.f);
    } else {
      float* po = out + static_cast<size_t>(r) * n_split * (DH + 2);
      po[2 + d] = aa;
      if (d == 0) { po[0] = mm; po[1] = ll; }
    }
  }
}

// Merge the splits: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One workgroup per (sequence, head); the splits are read in parallel: the
// 256 threads take the maxima and the weighted sums of the split range in a
// fixed order (so the result does not depend on timing), then thread pairs
// (d, half) add the weighted partial outputs of their half of the splits.
constexpr int kCombineThreads = 256;
__global__ __launch_bounds__(kCombineThreads) void attn_decode_combine_kernel(const float* __restrict__ part,
                                                                             bf16_t* __restrict__ o, int o_frag,
                                                                             int H, int n_split) {
  __shared__ float red[kCombineThreads];
  __shared__ float half_sum[DH];
  const int bh = blockIdx.x;  // b * H + h
  const int t = threadIdx.x;
  const float* pp = part + static_cast<size_t>(bh) * n_split * (DH + 2);
  // global max over the splits
  float M = -INFINITY;
  for (int s = t; s < n_split; s += kCombineThreads) M = fmaxf(M, pp[static_cast<size_t>(s) * (DH + 2)]);
  red[t] = M;
  __syncthreads();
  for (int w = kCombineThreads / 2; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  const bool any = M != -INFINITY;
  // denominator: sum over splits of 2^(m_s - M) l_s (exactly 0 for empty splits)
  float den = 0.f;
  if (any)
    for (int s = t; s < n_split; s += kCombineThreads) {
      const float* e = pp + static_cast<size_t>(s) * (DH + 2);
      den += fast_exp2(e[0] - M) * e[1];
    }
  red[t] = den;
  __syncthreads();
  for (int w = kCombineThreads / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  den = red[0];
  // numerator for dim d over half hf of the splits
  const int d = t & (DH - 1), hf = t / DH;
  float num = 0.f;
  if (any)
    for (int s = hf; s < n_split; s += kCombineThreads / DH) {
      const float* e = pp + static_cast<size_t>(s) * (DH + 2);
      num += fast_exp2(e[0] - M) * e[2 + d];
    }
  if (hf == 1) half_sum[d] = num;
  __syncthreads();
  if (hf == 0) {
    num += half_sum[d];
    const size_t at = o_frag ? frag_index(bh / H, (bh % H) * DH + d, H * DH) : static_cast<size_t>(bh) * DH + d;
    o[at] = f32_to_f16_sat(den > 0.f ? num / den : 0.f);
  }
}

// slots per split: one split when the (sequence, kv head, head chunk)
// workgroups already number target_wgs(R), else enough splits to get there
int split_len(int max_pos, int B, int Hkv, int chunks, int R) {
  const long long wgs = static_cast<long long>(B) * Hkv * chunks;
  const long long target = target_wgs(R);
  if (wgs >= target) return max_pos;
  long long L = (static_cast<long long>(max_pos) * wgs + target - 1) / target;
  L = (L + 63) / 64 * 64;  // whole iterations (so a paged iteration stays in one page)
  if (L < 64) L = 64;
  if (L > max_pos) L = max_pos;
  return static_cast<int>(L);
}

int heads_per_block(int n_rep) {
  for (int r = kMaxRep; r >= 1; --r)
    if (n_rep % r == 0) return r;
  return 1;
}

}  // namespace

int decode_attn_splits(int span, int B, int n_heads, int n_kv_heads) {
  const int n_rep = n_heads / n_kv_heads;
  const int R = heads_per_block(n_rep);
  const int L = split_len(span, B, n_kv_heads, n_rep / R, R);
  return (span + L - 1) / L;
}

// A split is at least 64 slots and at least span * wgs / target_wgs slots,
// so any span <= max_pos has at most min(ceil(max_pos / 64),
// ceil(target_wgs / wgs)) splits.
int decode_attn_max_splits(int max_pos, int B, int n_heads, int n_kv_heads) {
  const int n_rep = n_heads / n_kv_heads;
  const int R = heads_per_block(n_rep);
  const long long wgs = static_cast<long long>(B) * n_kv_heads * (n_rep / R);
  const long long target = target_wgs(R);
  if (wgs >= target) return 1;
  const long long a = (max_pos + 63) / 64, c = (target + wgs - 1) / wgs;
  return static_cast<int>(a < c ? a : c);
}

hipError_t launch_attn_decode(const bf16_t* q, const void* k_cache, const void* v_cache,
                              const int32_t* pos, bf16_t* o, int o_frag, float* part, int n_split,
                              int B, int n_heads, int n_kv_heads, int max_pos, int span, const KvPaging& pg,
                              hipStream_t s, const float* k_scale, const float* v_scale) {
  if (o_frag && B > kSkinnyMaxTokens) return hipErrorInvalidValue;
  if (pg.block_table && (pg.page % 64 || pg.page <= 0 || span > pg.blocks_per_seq * pg.page))
    return hipErrorInvalidValue;
  const int n_rep = n_heads / n_kv_heads;
  const int R = heads_per_block(n_rep);
  const int L = split_len(span, B, n_kv_heads, n_rep / R, R);
  if ((span + L - 1) / L != n_split) return hipErrorInvalidValue;
  const dim3 grid(n_split, n_kv_heads * (n_rep / R), B);
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(DH)));
  const bool paged = pg.block_table != nullptr;
  const bool q8 = k_scale != nullptr;
  if (q8 && !v_scale) return hipErrorInvalidValue;
  switch (R) {
#define LLAMA_DEC_CASE(RR)                                                                                      \
  case RR:                                                                                                      \
    if (paged && q8)                                                                                            \
      hipLaunchKernelGGL((attn_decode_kernel<RR, true, true>), grid, dim3(256), 0, s, q, k_cache, v_cache, pos,  \
                         part, o, o_frag, n_heads, n_kv_heads, max_pos, span, pg, L, n_split, scale_log2,       \
                         k_scale, v_scale);                                                                     \
    else if (paged)                                                                                             \
      hipLaunchKernelGGL((attn_decode_kernel<RR, true, false>), grid, dim3(256), 0, s, q, k_cache, v_cache, pos, \
                         part, o, o_frag, n_heads, n_kv_heads, max_pos, span, pg, L, n_split, scale_log2,       \
                         nullptr, nullptr);                                                                     \
    else if (q8)                                                                                                \
      hipLaunchKernelGGL((attn_decode_kernel<RR, false, true>), grid, dim3(256), 0, s, q, k_cache, v_cache, pos, \
                         part, o, o_frag, n_heads, n_kv_heads, max_pos, span, pg, L, n_split, scale_log2,       \
                         k_scale, v_scale);                                                                     \
    else                                                                                                        \
      hipLaunchKernelGGL((attn_decode_kernel<RR, false, false>), grid, dim3(256), 0, s, q, k_cache, v_cache,    \
                         pos, part, o, o_frag, n_heads, n_kv_heads, max_pos, span, pg, L, n_split, scale_log2,  \
                         nullptr, nullptr);                                                                     \
    break;
    LLAMA_DEC_CASE(1) LLAMA_DEC_CASE(2) LLAMA_DEC_CASE(3) LLAMA_DEC_CASE(4)
    LLAMA_DEC_CASE(5) LLAMA_DEC_CASE(6) LLAMA_DEC_CASE(7) LLAMA_DEC_CASE(8)
#undef LLAMA_DEC_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(B * n_heads), dim3(kCombineThreads), 0, s, part, o, o_frag,
                     n_heads, n_split);
  return hipGetLastError();
}

}  // namespace llama
