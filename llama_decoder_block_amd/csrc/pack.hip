// Weight layout conversion at layer creation: row-major bf16 -> fragment
// order (the 32x32x16 MFMA operand layout, one contiguous 1 KB wavefront load
// per 32 x 16 chunk), optionally converting the elements to fp16 (the o_proj
// and down weights, whose activations are fp16).  Runs once per layer; not on
// the hot path.
#include "common.h"

namespace llama {
namespace {

// one thread per 16-byte vector (8 consecutive k of one row)
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint4* __restrict__ src, int rows, int K,
                                                        bf16_t* __restrict__ dst, int group, int group_stride,
                                                        int to_f16) {
  const size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  const int kv = K >> 3;
  if (i >= static_cast<size_t>(rows) * kv) return;
  const int r = static_cast<int>(i / kv), k = static_cast<int>(i % kv) * 8;
  int dr;
  if (group == 0) {  // heads of 128 rows, dims x and x + 64 to rows 2x and 2x + 1
    const int d = r & 127;
    dr = (r & ~127) + (d < 64 ? 2 * d : 2 * (d - 64) + 1);
  } else {
    dr = (r / group) * group_stride + r % group;
  }
  uint4 v = src[i];
  if (to_f16) {  // bf16 -> fp32 is exact; fp32 -> fp16 rounds to nearest even
    v.x = pack_f16x2_sat(lo_bf16(v.x), hi_bf16(v.x));
    v.y = pack_f16x2_sat(lo_bf16(v.y), hi_bf16(v.y));
    v.z = pack_f16x2_sat(lo_bf16(v.z), hi_bf16(v.z));
    v.w = pack_f16x2_sat(lo_bf16(v.w), hi_bf16(v.w));
  }
  *reinterpret_cast<uint4*>(dst + frag_index(dr, k, K)) = v;
}

}  // namespace

hipError_t launch_pack_rows(const bf16_t* src, int rows, int K, bf16_t* dst, int group, int group_stride,
                            int to_f16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rows % 32 || group % 32 || K % 16 || group < 0 || (group == 0 && rows % 128)) return hipErrorInvalidValue;
  const size_t n = static_cast<size_t>(rows) * (K / 8);
  hipLaunchKernelGGL(pack_rows_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(src), rows, K, dst, group, group_stride, to_f16);
  return hipGetLastError();
}

}  // namespace llama
