// Shared device helpers and internal launch entry points of the gfx950
// decoder-layer kernels.  Everything here is internal to libllama_layer.so;
// the public surface is include/llama_layer.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llama {

typedef uint16_t bf16_t;  // bf16 bit pattern as stored in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 with gfx950's v_cvt_pk_bf16_f32 (round to nearest even,
// NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two fp32 -> packed pair of bf16 (lo in bits 0..15), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the bare v_exp_f32 (results below the normal range flush to 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw buffer resource over [base, base + bytes): loads at or past the end
// return zeros (hardware range check), which is how tiles handle ragged edges.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Fragment order of a bf16 matrix [R, K] (K % 16 == 0): the operand layout of
// v_mfma_f32_32x32x16_bf16.  The matrix is cut into 1 KB chunks of 32 rows x
// 16 k; chunk (rb, kb) sits at element (rb * K/16 + kb) * 512, and inside it
// lane l's 16 bytes hold row 32 rb + l % 32, k = 16 kb + 8 (l / 32) + 0..7.  A
// wavefront reads one chunk with one contiguous 1 KB load, and rows
// [32 rb, 32 rb + n) of the matrix occupy elements [32 rb K, (32 rb + n) K),
// exactly where they sit in row-major order.  The weights of every bf16 layer
// are stored this way, and so are the activations of calls with <= 64 tokens.
__device__ __forceinline__ uint32_t frag_index(int row, int k, int K) {
  return ((static_cast<uint32_t>(row >> 5) * static_cast<uint32_t>(K >> 4) + static_cast<uint32_t>(k >> 4)) << 9) +
         (static_cast<uint32_t>((row & 31) + ((k >> 3) & 1) * 32) << 3) + static_cast<uint32_t>(k & 7);
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over each aligned group of 16 lanes, result in every lane of the group,
// with DPP lane moves (one VALU add each) instead of LDS-routed shuffles:
// swap neighbours, swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float sum16_dpp(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// -------------------------------------------------------------------------
// Internal launchers (each returns hipGetLastError() of its launch).
// -------------------------------------------------------------------------

// RMSNorm rows: out[r, :] = g * in[r, :] / sqrt(mean(in[r,:]^2) + eps).
// in is bf16 (in_f32 = 0) or fp32 (in_f32 = 1); out is bf16 or fp32.
// out_frag = 1 writes a bf16 out in fragment order (d % 128 == 0).
hipError_t launch_rmsnorm(const void* in, int in_f32, const void* gain, int gain_f32, void* out,
                          int out_f32, int out_frag, int rows, int d, float eps, hipStream_t s);

// Row-major bf16 src [rows, K] -> fragment order.  Source row r lands on row
// (r / group) * group_stride + r % group of the fragment-ordered dst
// (group = rows for a plain copy); rows and group are multiples of 32 and
// K % 16 == 0.  group = 0 is the rotary-pair order of projection heads: in
// every 128-row head, dims x and x + 64 land on rows 2x and 2x + 1.
hipError_t launch_pack_rows(const bf16_t* src, int rows, int K, bf16_t* dst, int group,
                            int group_stride, hipStream_t s);

// Tiled bf16 MFMA GEMM, C = A[M,K] . W[N,K]^T with a fused epilogue; A
// row-major, W in fragment order (K % 128 == 0).  The QKV weight is in
// rotary-pair order (see launch_pack_rows), the gate/up weight interleaved in
// 64-row blocks; the epilogues write q, the cache and h in the natural order.
struct QkvEpilogue {
  bf16_t* q;               // [M, H*dh]
  bf16_t* k_cache;         // [B, Hkv, max_pos, dh]
  bf16_t* v_cache;
  const int32_t* pos;      // [M]
  const float* rope_cos;   // [max_pos, dh/2]
  const float* rope_sin;
  int T, n_heads, n_kv_heads, max_pos;
};

hipError_t launch_gemm_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                           const QkvEpilogue& ep, hipStream_t s);
// out_f32[M,N] = A.W^T + resid_bf16[M,N]
hipError_t launch_gemm_resid_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                    const bf16_t* resid, float* out, hipStream_t s);
// out_bf16[M,N] = bf16(A.W^T + resid_f32[M,N])
hipError_t launch_gemm_resid_bf16out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                     const float* resid, bf16_t* out, hipStream_t s);
// W is the gate/up matrix interleaved in blocks of 64 rows [gate 64 | up 64]
// (N = 2f); out[M, f] = bf16(SiLU(gate) * up)
hipError_t launch_gemm_swiglu(const bf16_t* A, const bf16_t* Wgu, int M, int N, int K,
                              bf16_t* out, hipStream_t s);

// compute units of the current device (256 if the query fails)
int device_cu_count();

// Weight-streaming versions of the same four GEMMs for M <= 64 tokens: A and
// W both in fragment order (A holds ceil(M/32)*32 rows; rows >= M are never
// written out, whatever they hold).  The SwiGLU output h is written in
// fragment order, ready to be the A operand of the down projection.
// Scratch for column groups split between workgroups: part holds
// skinny_scratch_floats() floats, cnt cnt_len counters (one per column
// group: N / 32 or N / 64 for the paired SwiGLU), all zero before the first
// call; each call leaves them zero.
// Calls that share a scratch must not overlap.
constexpr int kSkinnyMaxTokens = 64;
constexpr int kSkinnyGrid = 512;  // workgroups per call, at most
struct SkinnyScratch {
  float* part;
  unsigned* cnt;
  int cnt_len;  // counters available
};
size_t skinny_scratch_floats();
hipError_t launch_skinny_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                             const QkvEpilogue& ep, const SkinnyScratch& sc, hipStream_t s);
hipError_t launch_skinny_resid_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                      const bf16_t* resid, float* out, const SkinnyScratch& sc,
                                      hipStream_t s);
hipError_t launch_skinny_resid_bf16out(const bf16_t* A, const bf16_t* W, int M, int N, int K,
                                       const float* resid, bf16_t* out, const SkinnyScratch& sc,
                                       hipStream_t s);
hipError_t launch_skinny_swiglu(const bf16_t* A, const bf16_t* Wgu, int M, int f, int K,
                                bf16_t* out, const SkinnyScratch& sc, hipStream_t s);
// out[m, n] = (A W^T)[m, n] in fp32 for n < n_valid, row stride ld (N, the
// weight's padded row count, a multiple of 128); the LM head
hipError_t launch_skinny_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K, float* out,
                                int n_valid, int ld, const SkinnyScratch& sc, hipStream_t s);

// Causal flash attention over the cache for prefill (bf16, dh = 128).
// q/o [B*T, H*128]; the query of token m sees cache slots 0..pos[m], or with
// bidir = 1 slots 0..max over t of pos[b*T + t] (its sequence's largest).
// o_frag = 1 writes o in fragment order instead of row-major.
hipError_t launch_attn_prefill(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache,
                               const int32_t* pos, bf16_t* o, int o_frag, int B, int T, int n_heads,
                               int n_kv_heads, int max_pos, int bidir, hipStream_t s);

// Decode attention (bf16, dh = 128) for one query per sequence, split over
// the cache when the grid would otherwise be small, followed by the merge of
// the splits (n_split > 1 only).  part holds B*H*n_split*(128+2) floats;
// o_frag as for the prefill kernel.
int decode_attn_splits(int max_pos, int B, int n_heads, int n_kv_heads);
hipError_t launch_attn_decode(const bf16_t* q, const bf16_t* k_cache, const bf16_t* v_cache,
                              const int32_t* pos, bf16_t* o, int o_frag, float* part, int n_split,
                              int B, int n_heads, int n_kv_heads, int max_pos, hipStream_t s);

// fp32 path (any shape).
struct F32Layer {
  int d, H, Hkv, dh, f, max_pos;
  int bidir;  // attention without the causal mask (each token sees up to its sequence's largest position)
  float eps;
  const float* g1; const float* g2;
  const float* wqkv; const float* wo; const float* wgu; const float* wd;  // wgu: [gate; up]
  const float* rope_cos; const float* rope_sin;  // [max_pos, dh/2]
  // scratch: xn [M,d], qkv [M,(H+2Hkv)dh], attn [M,H dh], x1 [M,d], gu [M,2f], h [M,f]
  float* xn; float* qkv; float* attn; float* x1; float* gu; float* h;
};
hipError_t run_f32_layer(const F32Layer& L, const float* x, float* y, const int32_t* pos, int B,
                         int T, float* k_cache, float* v_cache, hipStream_t s);
// out[m, n] = sum_k A[m, k] W[n, k] (+ resid[m, n]), fp32, all row-major
hipError_t launch_f32_gemm(const float* A, const float* W, const float* resid, float* out, int M, int N, int K,
                           hipStream_t s);
// the calling thread's last-error text (shared by every C entry point)
int set_error(int status, const char* fmt, ...);

}  // namespace llama
