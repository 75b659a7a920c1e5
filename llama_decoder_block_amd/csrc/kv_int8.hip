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
// gfx950 design: one wavefront per row, lane i holding dims 2i and 2i + 1
// (one 32-bit word of the bf16 row: 256 B per wavefront load, 128 B of codes
// per store); the row's amax is a wavefront max.  The work is tiny (a decode
// step appends B * Hkv rows of K and of V), so the kernel is one launch with
// four rows per 256-thread workgroup.
#include "common.h"

#include <math.h>

namespace llama {
namespace {

constexpr int DH = 128;

__device__ __forceinline__ int8_t code_of(float x, float inv) {
  const float c = rintf(x * inv);
  return static_cast<int8_t>(fminf(fmaxf(c, -127.f), 127.f));
}

// quantize one row (the calling wavefront's): src 128 bf16, dst 128 int8 + a scale
__device__ __forceinline__ void quantize_row(const bf16_t* __restrict__ src, int8_t* __restrict__ dst,
                                             float* __restrict__ scale, int lane) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(src)[lane];
  const float a = lo_bf16(w), b = hi_bf16(w);
  float m = fmaxf(fabsf(a), fabsf(b));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  int8_t ca = 0, cb = 0;
  float sc = 0.f;
  if (m >= 0x1p-100f) {  // uniform over the wavefront (smaller rows are stored as zeros)
    const float inv = __fdiv_rn(127.f, m);
    sc = __fdiv_rn(m, 127.f);
    ca = code_of(a, inv);
    cb = code_of(b, inv);
  }
  reinterpret_cast<uint16_t*>(dst)[lane] =
      static_cast<uint16_t>(static_cast<uint8_t>(ca) | (static_cast<uint16_t>(static_cast<uint8_t>(cb)) << 8));
  if (lane == 0) *scale = sc;
}

// rows r = (kv 0 / 1) * B * Hkv + b * Hkv + g: the staged row of sequence b,
// kv head g goes to slot pos[b]
__global__ __launch_bounds__(256) void kv_int8_append_kernel(
    const bf16_t* __restrict__ ks, const bf16_t* __restrict__ vs, const int32_t* __restrict__ pos, int B,
    int Hkv, int max_pos, int span, int8_t* __restrict__ kq, int8_t* __restrict__ vq,
    float* __restrict__ ksc, float* __restrict__ vsc) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = B * Hkv;
  if (r >= 2 * rows) return;
  const bool is_v = r >= rows;
  const int bg = is_v ? r - rows : r;
  const int b = bg / Hkv;
  const int p = pos[b];
  if (p < 0 || p >= span) return;
  const size_t slot = static_cast<size_t>(bg) * max_pos + p;
  quantize_row((is_v ? vs : ks) + static_cast<size_t>(bg) * DH, (is_v ? vq : kq) + slot * DH,
               (is_v ? vsc : ksc) + slot, lane);
}

// rows r = (kv 0 / 1) * B * Hkv * n_slots + (b * Hkv + g) * n_slots + j
__global__ __launch_bounds__(256) void kv_int8_convert_kernel(
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, int B, int Hkv, int max_pos, int n_slots,
    int8_t* __restrict__ kq, int8_t* __restrict__ vq, float* __restrict__ ksc, float* __restrict__ vsc) {
  const int lane = threadIdx.x & 63;
  const long long r = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const long long rows = static_cast<long long>(B) * Hkv * n_slots;
  if (r >= 2 * rows) return;
  const bool is_v = r >= rows;
  const long long i = is_v ? r - rows : r;
  const long long bg = i / n_slots, j = i % n_slots;
  const size_t slot = static_cast<size_t>(bg) * max_pos + static_cast<size_t>(j);
  quantize_row((is_v ? vc : kc) + slot * DH, (is_v ? vq : kq) + slot * DH, (is_v ? vsc : ksc) + slot, lane);
}

}  // namespace

hipError_t launch_kv_int8_append(const bf16_t* k_stage, const bf16_t* v_stage, const int32_t* pos, int B,
                                 int n_kv_heads, int max_pos, int span, int8_t* k_codes, int8_t* v_codes,
                                 float* k_scale, float* v_scale, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const long long rows = 2LL * B * n_kv_heads;
  hipLaunchKernelGGL(kv_int8_append_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s, k_stage,
                     v_stage, pos, B, n_kv_heads, max_pos, span, k_codes, v_codes, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_int8_convert(const bf16_t* k_cache, const bf16_t* v_cache, int B, int n_kv_heads,
                                  int max_pos, int n_slots, int8_t* k_codes, int8_t* v_codes, float* k_scale,
                                  float* v_scale, hipStream_t s) {
  if (B <= 0 || n_slots <= 0) return hipSuccess;
  const long long rows = 2LL * B * n_kv_heads * n_slots;
  if ((rows + 3) / 4 > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_int8_convert_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s, k_cache,
                     v_cache, B, n_kv_heads, max_pos, n_slots, k_codes, v_codes, k_scale, v_scale);
  return hipGetLastError();
}

}  // namespace llama
