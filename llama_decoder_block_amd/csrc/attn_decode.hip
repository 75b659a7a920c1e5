// Decode attention: one new query per sequence over its whole cache,
// o_h = softmax(q_h K_{0..p}^T / sqrt(128)) V_{0..p}, bf16 cache, fp32 math.
//
// Sources: "LLM mechanics lecture notes" Ch.04 (decode appends k_t, v_t and
// lets q_t read every visible cached K/V; decode stays memory bound and grows
// with context) and "LMDrive LLM core inference unit" page §2.3 (scores,
// softmax, weighted sum of values; repeat_kv grouped-query attention, here
// kv-head indexing so a K/V row read serves all query heads of its group).
//
// gfx950 design: the cache is streamed once at HBM rate.
//   * split-K: workgroup (split s, kv head g, sequence b) takes slots
//     [s L, (s+1) L) ∩ [0, p]; L is chosen so the grid holds well over 256
//     workgroups even at batch 1 with 8 kv heads;
//   * a K or V row (128 dims = 256 B) is read by 16 lanes with 16-byte loads,
//     so a wavefront reads 4 consecutive rows = 1 KB contiguous per load;
//   * scores: each lane dots its 8 dims with the query slice of every head of
//     the group, then a 16-lane shuffle reduction; scores live in LDS;
//   * a local softmax (max and sum in fp32, base-2 exponent with the scale
//     folded in), then P V accumulated per lane over 8 dims x heads;
//   * each split writes (max, sum, unnormalised o[128]) per head; a second
//     kernel rescales and adds the splits (the standard split-softmax merge).
#include "common.h"

#include <math.h>

namespace llama {
namespace {

constexpr int DH = 128;
constexpr int kMaxRep = 8;    // query heads handled per workgroup
constexpr int kMaxL = 512;    // slots per split (upper bound)

template <int R>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ pos, float* __restrict__ part,
    int H, int Hkv, int max_pos, int L, int n_split, float scale_log2) {
  __shared__ float sc[R][kMaxL];
  __shared__ float red[4][R][DH];
  __shared__ float stat[R][2];

  const int s = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int n_rep = H / Hkv;
  const int chunks = n_rep / R;            // workgroups per kv head
  const int g = hg / chunks;
  const int h0 = g * n_rep + (hg % chunks) * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dc = lane & 15;                // 8-dim chunk of a row
  const int sub = wave * 4 + (lane >> 4);  // 16 row groups per workgroup

  const int p = min(pos[b], max_pos - 1);
  const int j_begin = s * L;
  const int j_end = min(j_begin + L, p + 1);
  const int n = j_end - j_begin;
  float* out = part + ((static_cast<size_t>(b) * H + h0) * n_split + s) * (DH + 2);
  if (n <= 0) {  // nothing visible in this split
    for (int i = tid; i < R * (DH + 2); i += 256) {
      const int r = i / (DH + 2), e = i % (DH + 2);
      out[static_cast<size_t>(r) * n_split * (DH + 2) + e] = e == 0 ? -INFINITY : 0.f;
    }
    return;
  }

  // query slices: 8 dims per lane for each of the R heads
  float qv[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint4 u = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(b) * H + h0 + r) * DH + dc * 8);
    qv[r][0] = lo_bf16(u.x); qv[r][1] = hi_bf16(u.x); qv[r][2] = lo_bf16(u.y); qv[r][3] = hi_bf16(u.y);
    qv[r][4] = lo_bf16(u.z); qv[r][5] = hi_bf16(u.z); qv[r][6] = lo_bf16(u.w); qv[r][7] = hi_bf16(u.w);
  }

  const size_t slice = (static_cast<size_t>(b) * Hkv + g) * max_pos * DH;
  const bf16_t* K = k_cache + slice + static_cast<size_t>(j_begin) * DH + dc * 8;
  const bf16_t* V = v_cache + slice + static_cast<size_t>(j_begin) * DH + dc * 8;

  // ---- scores
  for (int j = sub; j < n; j += 16 * 4) {
    uint4 ku[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ku[u] = (j + 16 * u < n) ? *reinterpret_cast<const uint4*>(K + static_cast<size_t>(j + 16 * u) * DH)
                               : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float kf[8];
      kf[0] = lo_bf16(ku[u].x); kf[1] = hi_bf16(ku[u].x); kf[2] = lo_bf16(ku[u].y); kf[3] = hi_bf16(ku[u].y);
      kf[4] = lo_bf16(ku[u].z); kf[5] = hi_bf16(ku[u].z); kf[6] = lo_bf16(ku[u].w); kf[7] = hi_bf16(ku[u].w);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += qv[r][e] * kf[e];
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        d += __shfl_xor(d, 4, 64);
        d += __shfl_xor(d, 8, 64);
        if (dc == 0 && j + 16 * u < n) sc[r][j + 16 * u] = d * scale_log2;
      }
    }
  }
  __syncthreads();

  // ---- local softmax per head (one wave per head, heads strided by 4)
  for (int r = wave; r < R; r += 4) {
    float m = -INFINITY;
    for (int j = lane; j < n; j += 64) m = fmaxf(m, sc[r][j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float l = 0.f;
    for (int j = lane; j < n; j += 64) {
      const float e = fast_exp2(sc[r][j] - m);
      sc[r][j] = e;
      l += e;
    }
    l = warp_sum(l);
    if (lane == 0) { stat[r][0] = m; stat[r][1] = l; }
  }
  __syncthreads();

  // ---- P V: lane accumulates 8 dims x R heads over its rows
  float acc[R][8];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  for (int j = sub; j < n; j += 16 * 4) {
    uint4 vu[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vu[u] = (j + 16 * u < n) ? *reinterpret_cast<const uint4*>(V + static_cast<size_t>(j + 16 * u) * DH)
                               : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (j + 16 * u >= n) break;
      float vf[8];
      vf[0] = lo_bf16(vu[u].x); vf[1] = hi_bf16(vu[u].x); vf[2] = lo_bf16(vu[u].y); vf[3] = hi_bf16(vu[u].y);
      vf[4] = lo_bf16(vu[u].z); vf[5] = hi_bf16(vu[u].z); vf[6] = lo_bf16(vu[u].w); vf[7] = hi_bf16(vu[u].w);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pr = sc[r][j + 16 * u];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] += pr * vf[e];
      }
    }
  }
  // reduce the 4 row groups of a wave (lanes 16 apart), then the 4 waves via LDS
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[r][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[r][e] = v;
    }
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][r][dc * 8 + e] = acc[r][e];
  }
  __syncthreads();
  for (int i = tid; i < R * DH; i += 256) {
    const int r = i / DH, d = i % DH;
    const float v = red[0][r][d] + red[1][r][d] + red[2][r][d] + red[3][r][d];
    float* o = out + static_cast<size_t>(r) * n_split * (DH + 2);
    o[2 + d] = v;
    if (d == 0) { o[0] = stat[r][0]; o[1] = stat[r][1]; }
  }
}

// Merge the splits: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(128) void attn_decode_combine_kernel(const float* __restrict__ part,
                                                                  bf16_t* __restrict__ o, int o_frag,
                                                                  int H, int n_split) {
  const int bh = blockIdx.x;  // b * H + h
  const int d = threadIdx.x;
  const float* pp = part + static_cast<size_t>(bh) * n_split * (DH + 2);
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, pp[s * (DH + 2)]);
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const float* e = pp + s * (DH + 2);
      const float w = fast_exp2(e[0] - M);  // exactly 0 for empty splits (m = -inf)
      den += w * e[1];
      num += w * e[2 + d];
    }
  }
  const size_t at = o_frag ? frag_index(bh / H, (bh % H) * DH + d, H * DH) : static_cast<size_t>(bh) * DH + d;
  o[at] = f32_to_bf16(den > 0.f ? num / den : 0.f);
}

int split_len(int max_pos, int B, int Hkv) {
  // aim for >= ~2048 split workgroups in all
  const long long rows = static_cast<long long>(max_pos) * B * Hkv;
  long long L = (rows + 2047) / 2048;
  L = (L + 63) / 64 * 64;
  if (L < 64) L = 64;
  if (L > kMaxL) L = kMaxL;
  return static_cast<int>(L);
}

int heads_per_block(int n_rep) {
  for (int r = kMaxRep; r >= 1; --r)
    if (n_rep % r == 0) return r;
  return 1;
}

}  // namespace

int decode_attn_splits(int max_pos, int B, int n_kv_heads) {
  const int L = split_len(max_pos, B, n_kv_heads);
  return (max_pos + L - 1) / L;
}

hipError_t launch_attn_decode(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache,
                              const int32_t* pos, bf16_t* o, int o_frag, float* part, int n_split,
                              int B, int n_heads, int n_kv_heads, int max_pos, hipStream_t s) {
  if (o_frag && B > kSkinnyMaxTokens) return hipErrorInvalidValue;
  const int L = split_len(max_pos, B, n_kv_heads);
  if ((max_pos + L - 1) / L != n_split) return hipErrorInvalidValue;
  const int n_rep = n_heads / n_kv_heads;
  const int R = heads_per_block(n_rep);
  const dim3 grid(n_split, n_kv_heads * (n_rep / R), B);
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(DH)));
  switch (R) {
#define LLAMA_DEC_CASE(RR)                                                                              \
  case RR:                                                                                              \
    hipLaunchKernelGGL(attn_decode_split_kernel<RR>, grid, dim3(256), 0, s, q, k_cache, v_cache, pos,  \
                       part, n_heads, n_kv_heads, max_pos, L, n_split, scale_log2);                     \
    break;
    LLAMA_DEC_CASE(1) LLAMA_DEC_CASE(2) LLAMA_DEC_CASE(3) LLAMA_DEC_CASE(4)
    LLAMA_DEC_CASE(5) LLAMA_DEC_CASE(6) LLAMA_DEC_CASE(7) LLAMA_DEC_CASE(8)
#undef LLAMA_DEC_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(B * n_heads), dim3(DH), 0, s, part, o, o_frag, n_heads,
                     n_split);
  return hipGetLastError();
}

}  // namespace llama
