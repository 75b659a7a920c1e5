// RMSNorm over rows: out = g * x / sqrt(mean(x^2) + eps).
//
// Source: "LMDrive LLM core inference unit" page, §2.1 LlamaRMSNorm (fp32
// statistics, eps added to the mean square inside the root, learnable gain),
// and the "LLM mechanics lecture notes", §02.3 RMSNorm.  The gain multiplies
// in fp32 and the result is rounded once to the output type.
//
// One 64-wide wavefront per row.  Each lane keeps its share of the row in
// registers (NV vectors of 8 elements, 16-byte bf16 or 32-byte fp32 loads,
// consecutive lanes on consecutive vectors so a wave reads 1 KB contiguous per
// load), so HBM sees exactly one read of x and one write of out.  The sum of
// squares is reduced in fp32 with wavefront shuffles; no LDS, no barriers.
#include "common.h"

namespace llama {
namespace {

__device__ __forceinline__ void load8(const bf16_t* p, float v[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = lo_bf16(u.x); v[1] = hi_bf16(u.x); v[2] = lo_bf16(u.y); v[3] = hi_bf16(u.y);
  v[4] = lo_bf16(u.z); v[5] = hi_bf16(u.z); v[6] = lo_bf16(u.w); v[7] = hi_bf16(u.w);
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, const float v[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ void store1(bf16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }

constexpr int kRowsPerBlock = 4;  // 4 waves, one row each

// d % 8 == 0 and d <= NV * 512.  FRAG: bf16 out in fragment order (the
// 16-byte vector of k = 8 vi .. 8 vi + 7 stays contiguous there).
template <typename TIn, typename TG, typename TOut, int NV, bool FRAG>
__global__ __launch_bounds__(256) void rmsnorm_vec_kernel(const TIn* __restrict__ in,
                                                          const TG* __restrict__ g,
                                                          TOut* __restrict__ out, int rows,
                                                          int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TIn* x = in + static_cast<size_t>(row) * d;
  const int nvec = d >> 3;
  // the row and the gain are fetched together (one memory round trip)
  float v[NV][8], gv[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = lane + j * kWave;
    if (vi < nvec) {
      load8(x + vi * 8, v[j]);
      load8(g + vi * 8, gv[j]);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = lane + j * kWave;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
    }
  }
  ss = warp_sum(ss);
  const float inv = rsqrtf(ss / static_cast<float>(d) + eps);
  TOut* y = out + (FRAG ? 0 : static_cast<size_t>(row) * d);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = lane + j * kWave;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = gv[j][e] * (v[j][e] * inv);
      store8(y + (FRAG ? frag_index(row, vi * 8, d) : vi * 8), v[j]);
    }
  }
}

// Few rows (decode): one 256-thread workgroup per row, so a call of B rows
// spreads over B CUs and each lane issues d / 2048 loads of the row (and of
// the gain) instead of d / 512; the sum of squares goes through the four
// waves' partial sums in LDS, added in a fixed order.  d % 2048 == 0; for 32
// rows of 4096 the decode norm step went from ~10 to ~6.6 us (event timed).
template <typename TIn, typename TG, typename TOut, int NV, bool FRAG>
__global__ __launch_bounds__(256) void rmsnorm_row_kernel(const TIn* __restrict__ in, const TG* __restrict__ g,
                                                          TOut* __restrict__ out, int d, float eps) {
  __shared__ float part[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const TIn* x = in + static_cast<size_t>(row) * d;
  float v[NV][8], gv[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = tid + j * 256;
    load8(x + vi * 8, v[j]);
    load8(g + vi * 8, gv[j]);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
  ss = warp_sum(ss);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  ss = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = rsqrtf(ss / static_cast<float>(d) + eps);
  TOut* y = out + (FRAG ? 0 : static_cast<size_t>(row) * d);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = tid + j * 256;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[j][e] = gv[j][e] * (v[j][e] * inv);
    store8(y + (FRAG ? frag_index(row, vi * 8, d) : vi * 8), v[j]);
  }
}

// Any d: two passes over the row (the second read hits the cache).
template <typename TIn, typename TG, typename TOut>
__global__ __launch_bounds__(256) void rmsnorm_any_kernel(const TIn* __restrict__ in,
                                                          const TG* __restrict__ g,
                                                          TOut* __restrict__ out, int rows,
                                                          int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TIn* x = in + static_cast<size_t>(row) * d;
  float ss = 0.f;
  for (int i = lane; i < d; i += kWave) {
    const float a = load1(x + i);
    ss += a * a;
  }
  ss = warp_sum(ss);
  const float inv = rsqrtf(ss / static_cast<float>(d) + eps);
  TOut* y = out + static_cast<size_t>(row) * d;
  for (int i = lane; i < d; i += kWave) store1(y + i, load1(g + i) * (load1(x + i) * inv));
}

template <typename TIn, typename TG, typename TOut, bool FRAG = false>
hipError_t dispatch(const void* in, const void* g, void* out, int rows, int d, float eps,
                    hipStream_t s) {
  const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
  const TIn* x = static_cast<const TIn*>(in);
  const TG* gg = static_cast<const TG*>(g);
  TOut* y = static_cast<TOut*>(out);
  const int nv = (d + 511) / 512;
  if (rows <= 64 && d % 2048 == 0) {  // few rows: one workgroup per row
    switch (d / 2048) {
      case 1:
        hipLaunchKernelGGL((rmsnorm_row_kernel<TIn, TG, TOut, 1, FRAG>), dim3(rows), block, 0, s, x, gg, y, d, eps);
        return hipGetLastError();
      case 2:
        hipLaunchKernelGGL((rmsnorm_row_kernel<TIn, TG, TOut, 2, FRAG>), dim3(rows), block, 0, s, x, gg, y, d, eps);
        return hipGetLastError();
      case 4:
        hipLaunchKernelGGL((rmsnorm_row_kernel<TIn, TG, TOut, 4, FRAG>), dim3(rows), block, 0, s, x, gg, y, d, eps);
        return hipGetLastError();
      case 8:
        hipLaunchKernelGGL((rmsnorm_row_kernel<TIn, TG, TOut, 8, FRAG>), dim3(rows), block, 0, s, x, gg, y, d, eps);
        return hipGetLastError();
      default:
        break;  // other widths take the one-wave-per-row kernel
    }
  }
  if (d % 8 == 0 && nv <= 16) {
    if (nv <= 8)
      hipLaunchKernelGGL((rmsnorm_vec_kernel<TIn, TG, TOut, 8, FRAG>), grid, block, 0, s, x, gg, y, rows, d, eps);
    else if (nv <= 10)
      hipLaunchKernelGGL((rmsnorm_vec_kernel<TIn, TG, TOut, 10, FRAG>), grid, block, 0, s, x, gg, y, rows, d, eps);
    else
      hipLaunchKernelGGL((rmsnorm_vec_kernel<TIn, TG, TOut, 16, FRAG>), grid, block, 0, s, x, gg, y, rows, d, eps);
  } else {
    if (FRAG) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rmsnorm_any_kernel<TIn, TG, TOut>), grid, block, 0, s, x, gg, y, rows, d, eps);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const void* in, int in_f32, const void* gain, int gain_f32, void* out,
                          int out_f32, int out_frag, int rows, int d, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (out_frag) {
    if (out_f32 || gain_f32 || d % 128 != 0) return hipErrorInvalidValue;
    return in_f32 ? dispatch<float, bf16_t, bf16_t, true>(in, gain, out, rows, d, eps, s)
                  : dispatch<bf16_t, bf16_t, bf16_t, true>(in, gain, out, rows, d, eps, s);
  }
  if (!in_f32 && !gain_f32 && !out_f32) return dispatch<bf16_t, bf16_t, bf16_t>(in, gain, out, rows, d, eps, s);
  if (in_f32 && !gain_f32 && !out_f32) return dispatch<float, bf16_t, bf16_t>(in, gain, out, rows, d, eps, s);
  if (in_f32 && gain_f32 && out_f32) return dispatch<float, float, float>(in, gain, out, rows, d, eps, s);
  return hipErrorInvalidValue;
}

}  // namespace llama
