// RMSNorm over rows: out = g * x / sqrt(mean(x^2) + eps).
//
// Source: "LMDrive LLM core inference unit" page, §2.1 LlamaRMSNorm (fp32
// statistics, eps added to the mean square inside the root, learnable gain),
// and the "LLM mechanics lecture notes", §02.3 RMSNorm.  The gain multiplies
// after normalising and the result is rounded once to the output type.
//
// Precision.  A bf16 output is the rounding point of the matrix products
// that follow, and bf16 inputs repeat values (8 significant bits): when a
// row's 1/rms lands a repeated input value within ~2^-24 of a bf16 rounding
// midpoint, fp32 arithmetic rounds every copy of it the wrong way at once,
// and the whole row's projections move.  So for a bf16 output the sum of
// squares (exact products) and 1/sqrt run in fp64, and each element is
// rounded to bf16 as its exact value would be: from fp32 where the fp32
// value is provably on the right side of the rounding midpoint, else
// recomputed in fp64 and rounded correctly (to odd into fp32, then to
// nearest even: no double rounding).  An fp32 output (the fp32 layer) stays
// in fp32.
//
// A workgroup of d / 512 wavefronts per row for calls of <= 64 rows (d =
// 2048, 4096, 5120 or 8192), else of 4 (d a multiple of 2048) or 2 (d =
// 3072, 5120, 6144 or 7168) wavefronts per row, else one 64-wide wavefront
// per row.  Each lane
// keeps its share of the row in registers (NV vectors of 8 elements, 16-byte
// bf16 or 32-byte fp32 loads, consecutive lanes on consecutive vectors so a
// wave reads 1 KB contiguous per load), so HBM sees exactly one read of x and
// one write of out.  The sum of squares is reduced with wavefront shuffles
// and, across the waves of a row, through LDS in a fixed order.
#include "common.h"

namespace llama {
namespace {

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
// fp64 -> fp32 rounded to odd: truncate, then set the last bit if anything
// was cut.  A later fp32 -> bf16 rounding to nearest even then gives exactly
// the fp64 -> bf16 rounding (fp32 keeps 16 more bits than bf16; Boldo and
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd", IEEE Trans. Computers 2008).
__device__ __forceinline__ float f64_to_f32_odd(double v) {
  const float t = __double2float_rz(v);
  return __uint_as_float(__float_as_uint(t) | (static_cast<double>(t) != v ? 1u : 0u));
}

// Statistics and scaling type: fp64 for a bf16 output, fp32 for an fp32 one.
template <typename TOut> struct NormAcc { typedef double type; };
template <> struct NormAcc<float> { typedef float type; };

// 8 consecutive elements as loaded (bf16 stays packed: half the registers)
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float operator[](int e) const {
    const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return (e & 1) ? hi_bf16(w) : lo_bf16(w);
  }
};
template <> struct Raw8<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) { load8(p, v); }
  __device__ __forceinline__ float operator[](int e) const { return v[e]; }
};

// g * (x * inv) for 8 elements, as fp32 values whose bf16 rounding (to
// nearest even) is the rounding of the exact product.  fp32 output: plain
// fp32.  bf16 output (A = double): computed in fp32 from inv rounded to fp32,
// three roundings of 2^-24 each, so the fp32 value is within 3 fp32 ulps of
// the exact one; unless it lies within 8 ulps of a bf16 rounding midpoint
// (low 16 bits 0x8000), both round to the same bf16 value.  The rare ones
// near a midpoint are redone in fp64 and rounded to odd (see f64_to_f32_odd).
template <typename A, typename X, typename G>
__device__ __forceinline__ void scale8(const X& x, const G& gv, A inv, float out[8]) {
  if constexpr (sizeof(A) == 8) {
    const float inv32 = static_cast<float>(inv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = gv[e] * (x[e] * inv32);
      const int off = static_cast<int>(__float_as_uint(v) & 0xffffu) - 0x8000;
      out[e] = (off < -8 || off > 8) ? v
                                     : f64_to_f32_odd(static_cast<double>(gv[e]) * (static_cast<double>(x[e]) * inv));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = gv[e] * (x[e] * inv);
  }
}

template <typename A>
__device__ __forceinline__ A wave_sum(A v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ void store1(bf16_t* p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }

constexpr int kRowsPerBlock = 4;  // 4 waves, one row each

// 1 / sqrt(ss / d + eps): fp32 with the hardware rsqrt, or fp64
template <typename A> __device__ __forceinline__ A inv_rms(A ss, int d, float eps);
template <> __device__ __forceinline__ float inv_rms<float>(float ss, int d, float eps) {
  return rsqrtf(ss / static_cast<float>(d) + eps);
}
template <> __device__ __forceinline__ double inv_rms<double>(double ss, int d, float eps) {
  return 1.0 / sqrt(ss / static_cast<double>(d) + static_cast<double>(eps));
}

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
  Raw8<TIn> v[NV];
  Raw8<TG> gv[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = lane + j * kWave;
    if (vi < nvec) {
      v[j].load(x + vi * 8);
      gv[j].load(g + vi * 8);
    }
  }
  typedef typename NormAcc<TOut>::type A;
  A ss = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = lane + j * kWave;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += static_cast<A>(v[j][e]) * static_cast<A>(v[j][e]);
    }
  }
  ss = wave_sum(ss);
  const A inv = inv_rms<A>(ss, d, eps);
  TOut* y = out + (FRAG ? 0 : static_cast<size_t>(row) * d);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = lane + j * kWave;
    if (vi < nvec) {
      float r[8];
      scale8(v[j], gv[j], inv, r);
      store8(y + (FRAG ? frag_index(row, vi * 8, d) : vi * 8), r);
    }
  }
}

// One workgroup of W wavefronts per row: each lane issues d / (512 W) loads
// of the row (and of the gain) instead of d / 512, so a CU has several
// times the loads in flight of the one-wave-per-row kernel; the sum of
// squares goes through the waves' partial sums in LDS, added in a fixed
// order.  d = NV * 512 * W.  Measured against one wave per row: 32 decode
// rows of 4096 ~10 -> ~6.6 us (event timed); the 7B prefill norms (2048
// rows) 16.2 / 16.4 -> 12.0 / 13.3 us, the 70B ones (4096 rows of 8192)
// 50.2 / 52.8 -> 29.7 / 37.1 us.
template <typename TIn, typename TG, typename TOut, int NV, bool FRAG, int W>
__global__ __launch_bounds__(64 * W) void rmsnorm_row_kernel(const TIn* __restrict__ in, const TG* __restrict__ g,
                                                             TOut* __restrict__ out, int d, float eps) {
  typedef typename NormAcc<TOut>::type A;
  __shared__ A part[W];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const TIn* x = in + static_cast<size_t>(row) * d;
  Raw8<TIn> v[NV];
  Raw8<TG> gv[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = tid + j * 64 * W;
    v[j].load(x + vi * 8);
    gv[j].load(g + vi * 8);
  }
  A ss = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += static_cast<A>(v[j][e]) * static_cast<A>(v[j][e]);
  ss = wave_sum(ss);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  ss = part[0];
#pragma unroll
  for (int w = 1; w < W; ++w) ss += part[w];
  const A inv = inv_rms<A>(ss, d, eps);
  TOut* y = out + (FRAG ? 0 : static_cast<size_t>(row) * d);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int vi = tid + j * 64 * W;
    float r[8];
    scale8(v[j], gv[j], inv, r);
    store8(y + (FRAG ? frag_index(row, vi * 8, d) : vi * 8), r);
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
  typedef typename NormAcc<TOut>::type A;
  A ss = 0;
  for (int i = lane; i < d; i += kWave) {
    const A a = static_cast<A>(load1(x + i));
    ss += a * a;
  }
  ss = wave_sum(ss);
  const A inv = inv_rms<A>(ss, d, eps);
  TOut* y = out + static_cast<size_t>(row) * d;
  for (int i = lane; i < d; i += kWave) {
    const A v = static_cast<A>(load1(g + i)) * (static_cast<A>(load1(x + i)) * inv);
    if constexpr (sizeof(A) == 8)
      store1(y + i, f64_to_f32_odd(v));  // (any-width fallback: fp64 throughout)
    else
      store1(y + i, v);
  }
}

template <typename TIn, typename TG, typename TOut, bool FRAG = false>
hipError_t dispatch(const void* in, const void* g, void* out, int rows, int d, float eps,
                    hipStream_t s) {
  const dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock), block(256);
  const TIn* x = static_cast<const TIn*>(in);
  const TG* gg = static_cast<const TG*>(g);
  TOut* y = static_cast<TOut*>(out);
  const int nv = (d + 511) / 512;
#define LLAMA_NORM_ROW_W(W)                                                                                \
  case W:                                                                                                    \
    hipLaunchKernelGGL((rmsnorm_row_kernel<TIn, TG, TOut, 1, FRAG, W>), dim3(rows), dim3(64 * W), 0, s, x, gg, \
                       y, d, eps);                                                                           \
    return hipGetLastError();
#define LLAMA_NORM_ROW(NV, W)                                                                              \
  case NV:                                                                                                   \
    hipLaunchKernelGGL((rmsnorm_row_kernel<TIn, TG, TOut, NV, FRAG, W>), dim3(rows), dim3(64 * W), 0, s, x, gg, \
                       y, d, eps);                                                                           \
    return hipGetLastError();
  // decode-sized calls (few rows, each a workgroup): one 16-byte vector per
  // lane, d / 512 wavefronts per row, so a row's loads all go out at once
  // (a single 70B row, 8192 wide: 9.7 / 9.4 -> 8.3 / 8.7 us per norm)
  if (rows <= 64 && d % 512 == 0) {
    switch (d / 512) {
      LLAMA_NORM_ROW_W(4) LLAMA_NORM_ROW_W(8) LLAMA_NORM_ROW_W(10) LLAMA_NORM_ROW_W(16)
      default: break;
    }
  }
  if (d % 2048 == 0) {  // a workgroup of 4 wavefronts per row
    switch (d / 2048) {
      LLAMA_NORM_ROW(1, 4) LLAMA_NORM_ROW(2, 4) LLAMA_NORM_ROW(4, 4) LLAMA_NORM_ROW(8, 4)
      default: break;
    }
  }
  if (d % 1024 == 0) {  // 2 wavefronts per row
    switch (d / 1024) {
      LLAMA_NORM_ROW(3, 2) LLAMA_NORM_ROW(5, 2) LLAMA_NORM_ROW(6, 2) LLAMA_NORM_ROW(7, 2)
      default: break;  // other widths take the one-wave-per-row kernel
    }
  }
#undef LLAMA_NORM_ROW
#undef LLAMA_NORM_ROW_W
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
