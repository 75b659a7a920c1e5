// Ceilings of the GPU the layer runs on, measured beside the layer so that
// its MFMA and HBM fractions can be read against what this chip sustains as
// well as against the published peaks.
//
//   * MFMA loop: every wavefront (8 per CU, two per SIMD) issues rounds of 8
//     independent v_mfma_f32_32x32x16_bf16 on register operands, with no
//     memory traffic (the result is stored only if it hits a fixed value,
//     which keeps the work from being optimised away).  The operands are
//     pseudo-random and differ between consecutive MFMAs, so the matrix
//     cores see data that toggles like real operands (their power draw, and
//     so the clock they hold, depends on it).
//   * Streaming read: the grid (4 blocks per CU) reads a buffer once, each
//     block a contiguous region of it, its 4 wavefronts loading consecutive
//     1 KB chunks (16 bytes per lane) with 4 loads in flight each and the
//     nontemporal hint.  Of the patterns measured on a 2 GB buffer (a
//     grid-strided sweep, 512-2048 regions, 1 or 4 loads in flight, with and
//     without the hint) this one read fastest: 6.8-7.0 TB/s, against
//     6.3-6.4 TB/s for the best sweep without the hint.
//
// The prefill's dense contractions are bounded by the first, the decode's
// weight and cache streaming by the second ("LLM mechanics lecture notes"
// Ch.04: prefill is compute bound, decode memory bound).
#include "common.h"
#include "../../include/llama_layer.h"

namespace llama {
namespace {

constexpr int kMfmaChains = 8;

// bf16 pairs with random signs and mantissas and exponents in [2^-2, 2^1):
// operand bits toggle like those of real activations and weights
__device__ __forceinline__ uint32_t random_bf16x2(uint32_t r) { return (r & 0x80ff80ffu) | 0x3e003e00u; }

__device__ __forceinline__ uint32_t xorshift32(uint32_t x) {
  x ^= x << 13;
  x ^= x >> 17;
  return x ^ (x << 5);
}

__global__ __launch_bounds__(256) void ceiling_mfma_kernel(int n_iter, float* __restrict__ sink) {
  // four random A and four random B operands per lane, made once; consecutive
  // MFMAs take different pairs, so the operands toggle with no VALU work in
  // the loop
  bf16x8 a[4], b[4];
  uint32_t r = 0x9e3779b9u * (blockIdx.x * 256 + threadIdx.x + 1);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = random_bf16x2(r = xorshift32(r));
    a[k] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    b[k] = __builtin_bit_cast(bf16x8, make_uint4(w[4], w[5], w[6], w[7]));
  }
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c & 3], b[(c + (c >> 2)) & 3], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  // the value depends on every product; written only if it hits a fixed pattern
  if (s == 1234.5f) sink[0] = s;
}

// block b reads chunks [b per, (b + 1) per) (clipped to the buffer); wave w
// of the block takes chunks w, w + 4, ... of it, four per iteration
__global__ __launch_bounds__(256) void ceiling_read_kernel(const uint4* __restrict__ p, uint64_t n_chunks,
                                                           uint64_t per, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t c0 = static_cast<uint64_t>(blockIdx.x) * per;
  const uint64_t c1 = c0 + per < n_chunks ? c0 + per : n_chunks;
  uint32_t x = 0;
  for (uint64_t c = c0 + wave; c < c1; c += 16) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t cc = c + 4 * u;
      v[u] = cc < c1 ? load16_nt(p + cc * 64 + lane) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the value depends on every load; written only if it hits a fixed pattern
  if (x == 0x9e3779b9u) sink[0] = x;
}

int cu_count(int* n_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *n_cu < 1)
    return set_error(LLAMA_ERR_HIP, "cannot query the compute unit count");
  return LLAMA_OK;
}

}  // namespace
}  // namespace llama

using namespace llama;

constexpr int kMfmaBlocksPerCu = 2;  // 8 wavefronts per CU
constexpr int kReadBlocksPerCu = 4;

extern "C" int llama_layer_ceiling_mfma(int32_t n_iter, void* sink, double* flops, void* stream) {
  if (!sink || !flops) return set_error(LLAMA_ERR_NULL, "sink and flops must be non-null");
  if (n_iter < 1) return set_error(LLAMA_ERR_INVALID, "n_iter must be >= 1 (got %d)", n_iter);
  int n_cu = 0;
  if (int st = cu_count(&n_cu)) return st;
  const int blocks = n_cu * kMfmaBlocksPerCu;
  hipLaunchKernelGGL(ceiling_mfma_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), n_iter,
                     static_cast<float*>(sink));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(LLAMA_ERR_HIP, "ceiling_mfma launch: %s", hipGetErrorString(e));
  *flops = static_cast<double>(blocks) * 4 * n_iter * kMfmaChains * (2.0 * 32 * 32 * 16);
  return LLAMA_OK;
}

extern "C" int llama_layer_ceiling_read(const void* buf, uint64_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return set_error(LLAMA_ERR_NULL, "buf and sink must be non-null");
  if (bytes == 0 || bytes % 1024) return set_error(LLAMA_ERR_INVALID, "bytes must be a positive multiple of 1024");
  if (reinterpret_cast<uintptr_t>(buf) & 15u) return set_error(LLAMA_ERR_INVALID, "buf must be 16-byte aligned");
  int n_cu = 0;
  if (int st = cu_count(&n_cu)) return st;
  // whole 1 KB chunks only (a tail below 1 KB is not read)
  const uint64_t blocks = static_cast<uint64_t>(n_cu) * kReadBlocksPerCu, chunks = bytes / 1024;
  hipLaunchKernelGGL(ceiling_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), chunks, (chunks + blocks - 1) / blocks,
                     static_cast<uint32_t*>(sink));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(LLAMA_ERR_HIP, "ceiling_read launch: %s", hipGetErrorString(e));
  return LLAMA_OK;
}
