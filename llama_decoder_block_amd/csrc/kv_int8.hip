// int8 KV cache rows: symmetric int8 codes with one fp32 scale per cached
// row (one token's 128 dims of one kv head).
//
// Sources: "LLM mechanics lecture notes" Ch.04 (the KV cache's memory is
// 2 B T Hkv dh times the element size, and decode streams all of it every
// step; quantising the cache is named as a lever beside GQA/MQA) and "Llama
// MLP deep dive" page §6.4 (KV-cache quantisation named).  Neither gives a
// scheme; this one keeps the decision simple enough to state exactly:
//   amax = max |x| over the row's bf16 values (exact in fp32);
//   scale = amax / 127, inv = 127 / amax (correctly rounded fp32 divisions);
//   code = rint(x * inv) (one fp32 product, round half to even), which lies
//   in [-127, 127] since |x| <= amax; a row whose amax is below 2^-100
//   (zeros among them) has scale 0 and codes 0, so 127 / amax stays finite.
// The row stands for code * scale.
//
// gfx950 design: 16 lanes per row, lane l of its row group holding dims
// 8l .. 8l + 7 (one 16-byte bf16 load, one 8-byte code store), so a
// wavefront quantizes 4 rows per instruction; the row's amax is a 16-lane
// max by DPP lane moves.  The append (B * T * Hkv rows of K and of V per layer
// call) takes 16 rows per 256-thread workgroup; the conversion of a whole
// cache strides a fixed grid over the rows, with 4 row groups (16 rows) of
// loads in flight per wavefront.
#include "common.h"

#include <math.h>

#include <algorithm>

namespace llama {
namespace {

constexpr int DH = 128;

__device__ __forceinline__ float max16_dpp(float v) {  // max over the 16 lanes of a row (the moves of sum16_dpp)
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  return v;
}

__device__ __forceinline__ uint32_t code_of(float x, float inv) {
  const float c = fminf(fmaxf(rintf(x * inv), -127.f), 127.f);
  return static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(c)));
}

// quantize one row from its 16 lanes: u holds this lane's 8 bf16 dims; the
// lane stores its 8 codes at dst (8 bytes) and the row's first lane the scale
__device__ __forceinline__ void quantize8(const uint4& u, int8_t* __restrict__ dst, float* __restrict__ scale,
                                          bool first) {
  const float x[8] = {lo_bf16(u.x), hi_bf16(u.x), lo_bf16(u.y), hi_bf16(u.y),
                      lo_bf16(u.z), hi_bf16(u.z), lo_bf16(u.w), hi_bf16(u.w)};
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  m = max16_dpp(m);
  uint32_t lo = 0, hi = 0;
  float sc = 0.f;
  if (m >= 0x1p-100f) {  // uniform over the row (smaller rows are stored as zeros)
    const float inv = __fdiv_rn(127.f, m);
    sc = __fdiv_rn(m, 127.f);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= code_of(x[e], inv) << (8 * e);
      hi |= code_of(x[4 + e], inv) << (8 * e);
    }
  }
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  if (first) *scale = sc;
}

// rows r = (kv 0 / 1) * M * Hkv + m * Hkv + g (M = B * T tokens): the staged
// row of token m = b * T + t, kv head g goes to slot pos[m] of sequence b
// (paged: row (page Hkv + g) page_size + pos % page_size of the pools, the
// page from the block table; a page id outside [0, n_pages) writes nothing);
// 16 lanes per row
__global__ __launch_bounds__(256) void kv_int8_append_kernel(
    const bf16_t* __restrict__ ks, const bf16_t* __restrict__ vs, const int32_t* __restrict__ pos, int M,
    int T, int Hkv, int max_pos, int span, KvPaging pg, int8_t* __restrict__ kq, int8_t* __restrict__ vq,
    float* __restrict__ ksc, float* __restrict__ vsc) {
  const int dc = threadIdx.x & 15;
  const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int rows = M * Hkv;
  if (r >= 2 * rows) return;  // whole row groups leave together
  const bool is_v = r >= rows;
  const int mg = is_v ? r - rows : r;  // staging row m * Hkv + g
  const int m = mg / Hkv, g = mg - m * Hkv;
  const int p = pos[m];
  if (p < 0 || p >= span) return;
  size_t slot;
  if (pg.block_table) {
    const int blk = pg.block_table[static_cast<size_t>(m / T) * pg.blocks_per_seq + p / pg.page];
    if (blk < 0 || blk >= pg.n_pages) return;
    slot = (static_cast<size_t>(blk) * Hkv + g) * pg.page + p % pg.page;
  } else {
    slot = (static_cast<size_t>(m / T) * Hkv + g) * max_pos + p;
  }
  const uint4 u = *reinterpret_cast<const uint4*>((is_v ? vs : ks) + static_cast<size_t>(mg) * DH + dc * 8);
  quantize8(u, (is_v ? vq : kq) + slot * DH + dc * 8, (is_v ? vsc : ksc) + slot, dc == 0);
}

// rows r = (kv 0 / 1) * B * Hkv * n_slots + (b * Hkv + g) * n_slots + j; a
// grid of at most kConvertBlocks workgroups strides over them: a row group
// (16 lanes) takes one row per pass, and issues kConvertPasses passes' loads
// before quantizing any
constexpr int kConvertPasses = 4;
constexpr int kConvertBlocks = 4096;
__global__ __launch_bounds__(256) void kv_int8_convert_kernel(
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, int B, int Hkv, int max_pos, int n_slots,
    int8_t* __restrict__ kq, int8_t* __restrict__ vq, float* __restrict__ ksc, float* __restrict__ vsc) {
  const int dc = threadIdx.x & 15;
  const long long rows = static_cast<long long>(B) * Hkv * n_slots;
  const long long groups = static_cast<long long>(gridDim.x) * 16;  // row groups in the grid
  const long long g0 = static_cast<long long>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  for (long long base = 0; base < 2 * rows; base += groups * kConvertPasses) {
    uint4 u[kConvertPasses];
    size_t slot[kConvertPasses];
    bool is_v[kConvertPasses];
#pragma unroll
    for (int k = 0; k < kConvertPasses; ++k) {  // loads first
      const long long r0 = base + g0 + k * groups;
      const long long r = r0 < 2 * rows ? r0 : 2 * rows - 1;  // past the end: reload the last row, store nothing
      is_v[k] = r >= rows;
      const long long i = is_v[k] ? r - rows : r;
      slot[k] = static_cast<size_t>(i / n_slots) * max_pos + static_cast<size_t>(i % n_slots);
      u[k] = *reinterpret_cast<const uint4*>((is_v[k] ? vc : kc) + slot[k] * DH + dc * 8);
    }
#pragma unroll
    for (int k = 0; k < kConvertPasses; ++k)
      if (base + g0 + k * groups < 2 * rows)  // uniform over the row group
        quantize8(u[k], (is_v[k] ? vq : kq) + slot[k] * DH + dc * 8, (is_v[k] ? vsc : ksc) + slot[k], dc == 0);
  }
}

}  // namespace

hipError_t launch_kv_int8_append(const bf16_t* k_stage, const bf16_t* v_stage, const int32_t* pos, int B,
                                 int T, int n_kv_heads, int max_pos, int span, const KvPaging& pg,
                                 int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale, hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  if (pg.block_table && (pg.page <= 0 || span > pg.blocks_per_seq * pg.page)) return hipErrorInvalidValue;
  const long long rows = 2LL * B * T * n_kv_heads;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_int8_append_kernel, dim3(static_cast<unsigned>((rows + 15) / 16)), dim3(256), 0, s,
                     k_stage, v_stage, pos, B * T, T, n_kv_heads, max_pos, span, pg, k_codes, v_codes, k_scale,
                     v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_int8_convert(const bf16_t* k_cache, const bf16_t* v_cache, int B, int n_kv_heads,
                                  int max_pos, int n_slots, int8_t* k_codes, int8_t* v_codes, float* k_scale,
                                  float* v_scale, hipStream_t s) {
  if (B <= 0 || n_slots <= 0) return hipSuccess;
  const long long rows = 2LL * B * n_kv_heads * n_slots;
  const long long blocks = std::min<long long>((rows + 16 * kConvertPasses - 1) / (16 * kConvertPasses),
                                               kConvertBlocks);
  hipLaunchKernelGGL(kv_int8_convert_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, k_cache,
                     v_cache, B, n_kv_heads, max_pos, n_slots, k_codes, v_codes, k_scale, v_scale);
  return hipGetLastError();
}

}  // namespace llama
