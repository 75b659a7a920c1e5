// Tiled 16-bit MFMA GEMM for the prefill projections, C = A[M,K] . W[N,K]^T,
// with the layer's elementwise work fused into the epilogue:
//   QKV     rotate-half RoPE of q and k at each token's position, bf16 round,
//           q -> scratch, k and v -> their cache slot (no concatenation pass);
//           the weight's heads are in rotary-pair order (dims x and x + 64 on
//           neighbouring rows), so every even-width tile holds whole pairs;
//   RESID32 X' = x + O Wo^T kept in fp32 (the residual add of the attention half);
//   SWIGLU  h = SiLU(gate) * up from one GEMM over the gate/up matrix
//           interleaved in 64-row blocks [gate 64 | up 64], so a 128-wide wave
//           tile holds gate column j and up column j; h is stored as fp16;
//   RESID16 y = bf16(X' + h Wdown^T) (the residual add of the MLP half).
// QKV and gate/up multiply bf16 operands (v_mfma_f32_32x32x16_bf16); o_proj
// and down multiply fp16 ones (v_mfma_f32_32x32x16_f16: the attention output
// and h are fp16, with 3 more significant bits, and Wo / Wdown are converted
// to fp16 at creation).  The kernel moves operands as raw 16-bit data, so the
// two differ only in the MFMA instruction.
//
// Sources: "LMDrive LLM core inference unit" page, §2.3 LlamaAttention (q/k/v
// projections, RoPE, cache append, o_proj) and §2.4 LlamaMLP
// (down(SiLU(gate(x)) * up(x)), no bias), §2.5 (both residual adds); §2.2 for
// the rotate-half pairing of dimension i with i + dh/2; "Llama MLP deep dive"
// page §2.2 (gate branch activated, up branch linear).
//
// gfx950 design.  256 threads = 4 wavefronts over a BM x BN tile, each wave
// owning a block of 32x32 accumulator tiles of the 32x32x16 MFMA:
//   * BM = 256: a 2x2 wave grid, wave tile 128 x (BN/2) (QKV: 256 x 192);
//   * BM = 128: a 1x4 wave grid, wave tile 128 x (BN/4) (o_proj and down:
//     128 x 256 or 128 x 512; gate/up: 128 x 512; QKV at large M: 128 x 512).  No two waves load the
//     same weight fragment, so the L1 carries (BM + BN) x 32 bytes per k step
//     instead of (BM + 2 BN) x 32; the wide tiles also halve the weight and
//     activation bytes per flop at large K.
// K advances in 64-wide slabs.
//   * W is stored in fragment order, so a wave fetches each 32 x 16 weight
//     fragment it needs with one contiguous 1 KB buffer load straight into
//     registers (a ring two or four slabs deep); W never touches LDS.
//   * A (activations, row-major) is staged through registers into two LDS
//     stages of BM rows x 128 bytes; the 16-byte column chunk c of row r is
//     stored at c ^ ((r >> 1) & 7) so the fragment reads of 32 consecutive
//     rows hit distinct banks.  Rows past M read as zeros (buffer range
//     check).  (Direct buffer->LDS loads would save the register hop, but a
//     partial vmcnt wait does not order them against other waves' reads, and
//     a full drain at every barrier costs more than the hop.)
//   * The slab loop is an explicit software pipeline: while slab kt feeds the
//     MFMAs, A slab kt+1 is written to LDS, A slab kt+2 and W k-steps kt+2 are
//     in flight, and the A fragments of the next k step are read from LDS one
//     MFMA slot ahead.  One barrier per slab.
//   * Tiles are numbered so that each XCD (blocks are dealt round-robin over 8
//     XCDs) gets a contiguous, M-grouped range, which keeps the A and W panels
//     it shares inside its own L2.
//   * Split K: when the tiles fill at most half the CUs (few tokens: chunked
//     prefill, batched decode of more than 128 sequences), each tile's slabs
//     are cut into ks <= 4 ranges of whole ring cycles, one workgroup each
//     (more would leave the last arriver too many partials to read alone).  Every
//     split writes its fp32 partial tile with coherent 16-byte stores, waits
//     for them, and counts itself in on the tile's counter; the last arriver
//     adds the ks partials in split order (the result does not depend on
//     arrival order), re-arms the counter and runs the epilogue.
// Requires K % 128 == 0 (an even number of slabs) and N % BN == 0 except for
// the QKV and resid epilogues, which bounds-check columns (weight fragments
// past N read as zeros).
#include "common.h"

#include <type_traits>

namespace llama {
namespace {

enum { EPI_QKV = 0, EPI_RESID32 = 1, EPI_RESID16 = 2, EPI_SWIGLU = 3 };

struct EpiArgs {
  QkvEpilogue qkv;
  const void* resid;
  void* out;
  // split K (ks > 1): partial tiles [tiles][ks][BM * BN] fp32 and one counter
  // per tile (zero between launches)
  float* part;
  unsigned* cnt;
  int ks;
};

constexpr int BK = 64;
constexpr int kGroupM = 8;
// QKV: N = 128 (H + 2 Hkv); 192-wide tiles make 64 column tiles at 32 heads
// (512 tiles at 2048 tokens: two full rounds of 256 CUs, where 256-wide
// tiles leave the second round half empty)
constexpr int kQkvBN = 192;

__device__ __forceinline__ void tile_coords(int M, int N, int BM, int BN, int bid, int& m0, int& n0) {
  const int nt_m = (M + BM - 1) / BM, nt_n = (N + BN - 1) / BN;
  const int nt = nt_m * nt_n;
  if ((nt & 7) == 0) bid = (bid & 7) * (nt >> 3) + (bid >> 3);  // contiguous range per XCD
  const int group = kGroupM * nt_n;
  const int first_m = (bid / group) * kGroupM;
  const int gm = min(nt_m - first_m, kGroupM);
  const int in_group = bid % group;
  m0 = (first_m + in_group % gm) * BM;
  n0 = (in_group / gm) * BN;
}


__device__ __forceinline__ int a_swz(int r) { return (r >> 1) & 7; }


// the residual GEMMs (o_proj, down) multiply fp16 operands, QKV and gate/up bf16
template <int EPI> constexpr bool kF16Operands = EPI == EPI_RESID32 || EPI == EPI_RESID16;

// SPLIT: the split-K form (ep.ks > 1 workgroups per tile)
template <int BM, int BN, int EPI, int RING, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ Wp,
                                                    int M, int N, int K, EpiArgs ep) {
  constexpr bool F16 = kF16Operands<EPI>;
  constexpr int WM = BM == 256 ? 2 : 1, WN = 4 / WM;  // wave grid
  constexpr int TM = BM / WM, TN = BN / WN;           // wave tile
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int NA = BM / 32;                         // A chunks per thread per slab
  constexpr int STAGE = BM * 128;               // bytes per LDS stage (BM rows x 64 k)
  // epilogue: a wave's 32-row block in fp32, rows TN + 8 floats apart, so
  // rows r and r + 4 (the two halves of a wavefront store) start 32 banks apart
  constexpr int TNP = TN + 8;
  constexpr int EPI_WAVE = 32 * TNP * 4;
  constexpr int LDS_STAGE = STAGE > 2 * EPI_WAVE ? STAGE : 2 * EPI_WAVE;
  __shared__ __attribute__((aligned(1024))) unsigned char As0[LDS_STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char As1[LDS_STAGE];
  __shared__ unsigned s_last;
  auto stage_base = [&](int st) -> unsigned char* { return st == 0 ? As0 : As1; };
  const int ks = SPLIT ? ep.ks : 1;
  const int tile = static_cast<int>(blockIdx.x) / ks, split = static_cast<int>(blockIdx.x) - tile * ks;
  int m0, n0;
  tile_coords(M, N, BM, BN, tile, m0, n0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = WM == 2 ? wave >> 1 : 0, wn = WM == 2 ? wave & 1 : wave;
  const int KB = K >> 4;
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(A, static_cast<uint32_t>(M) * K * 2u);
  const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(Wp, static_cast<uint32_t>(N) * K * 2u);

  // A staging through registers: 16-byte chunk i of this thread is row
  // 32 i + tid / 8, column chunk tid % 8 (eight threads read one 128-byte row
  // segment); it is stored at column chunk (tid % 8) ^ swz(row), and swz(row)
  // = (row >> 1) & 7 = (tid >> 4) & 7 for every i.
  uint32_t a_goff[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i)
    a_goff[i] = (static_cast<uint32_t>(m0 + 32 * i + (tid >> 3)) * K + (tid & 7) * 8) * 2u;
  const int a_woff = (tid >> 3) * 128 + (((tid & 7) ^ ((tid >> 4) & 7)) << 4);
  // AD register sets: with RING == 4 two, so an A load is issued 2.25 slabs
  // before its LDS store (slab s is held in set s & 1), else one (1.25 slabs)
  constexpr int AD = RING == 4 ? 2 : 1;
  uint4 sa[AD][NA];
  auto a_gload = [&](int set, int i, int kt) {
    sa[set][i] = buf_load16(a_rs, a_goff[i], static_cast<uint32_t>(kt) * (BK * 2u));
  };
  auto a_lstore = [&](int set, int i, int st) {
    *reinterpret_cast<uint4*>(stage_base(st) + a_woff + i * 32 * 128) = sa[set][i];
  };
  // B fragments: this wave's FN n-blocks, straight from the fragment-ordered weights
  uint32_t b_off[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) b_off[j] = static_cast<uint32_t>((n0 >> 5) + wn * FN + j) * KB * 1024u + lane * 16u;
  uint4 bq[RING][4][FN];
  auto b_load = [&](int set, int kt, int kk, int j) {
    bq[set][kk][j] = buf_load16(b_rs, b_off[j], static_cast<uint32_t>(kt * 4 + kk) * 1024u);
  };
  // A fragment reads
  int a_rd[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_rd[i] = (wm * TM + i * 32 + (lane & 31)) * 128;
  const int a_sw = a_swz(lane & 31);  // (row >> 1) & 7 depends only on lane & 31 here (row base is a multiple of 32)
  auto frag_a = [&](int stage, int kk, int i) {
    const int c = (2 * kk + (lane >> 5)) ^ a_sw;
    return *reinterpret_cast<const bf16x8*>(stage_base(stage) + a_rd[i] + c * 16);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8 fa[2][FM];

  // this split's slabs [s0, s1): whole ring cycles (K / BK is a multiple of RING)
  const int cycles = K / BK / RING;
  const int s0 = SPLIT ? split * cycles / ks * RING : 0;
  const int s1 = SPLIT ? (split + 1) * cycles / ks * RING : K / BK;
  // prologue: A slab s0 -> stage 0, A slabs s0+1 .. s0+AD -> registers; B
  // slabs s0 .. s0+RING-1 -> ring
#pragma unroll
  for (int i = 0; i < NA; ++i) a_gload(0, i, s0);
#pragma unroll
  for (int i = 0; i < NA; ++i) a_lstore(0, i, 0);
#pragma unroll
  for (int i = 0; i < NA; ++i) a_gload(AD == 2 ? 1 : 0, i, s0 + 1);
  if constexpr (AD == 2) {
#pragma unroll
    for (int i = 0; i < NA; ++i) a_gload(0, i, s0 + 2);
  }
#pragma unroll
  for (int b = 0; b < RING; ++b)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int j = 0; j < FN; ++j) b_load(b, s0 + b, kk, j);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[0][i] = frag_a(0, 0, i);

  // Slab kt (LDS stage kt & 1, B ring set kt % RING).  k steps 0-1: A slab
  // kt+1 goes from registers into the other stage (free: its last reads
  // finished before the previous barrier), each register refilled with slab
  // kt+1+AD right after; k steps 0-3: B slab kt+RING replaces the ring slots
  // it frees, so a weight load has RING - 1 slabs of MFMA work to arrive.
  // The A fragments of the next k step are read one MFMA slot ahead.  One
  // barrier per slab, before k step 3: it publishes the other stage (the
  // LDS writes are complete: lgkmcnt) and retires this stage's reads; then
  // the first fragments of slab kt+1 are read.  Every wait on a global load
  // is the compiler's own (register dependencies), so none depends on load
  // timing.
  auto slab = [&](const int st, const int bs, int kt) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      if (kk == 3) __syncthreads();
#pragma unroll
      for (int m = 0; m < FM * FN; ++m) {
        const int i = m / FN, j = m % FN;
        acc[i][j] = mfma_32x32x16<F16>(fa[cur][i], __builtin_bit_cast(bf16x8, bq[bs][kk][j]), acc[i][j]);
        if (m < FM) fa[cur ^ 1][m] = kk < 3 ? frag_a(st, kk + 1, m) : frag_a(st ^ 1, 0, m);
        if (m >= FM * FN - FN) b_load(bs, kt + RING, kk, m - (FM * FN - FN));
        // A chunk i (k step i / 4): stored to LDS, then its register is
        // refilled with the same chunk of slab kt+1+AD two slots later, so
        // every A load has AD slabs to arrive
        if (kk < 2) {
          constexpr int s2 = FM * FN / (NA / 2);  // slots per chunk
          const int i = kk * (NA / 2) + m / s2;
          const int as = AD == 2 ? (st ^ 1) : 0;  // the set holding slab kt+1
          if (m % s2 == s2 / 2 - 1) a_lstore(as, i, st ^ 1);
          if (m % s2 == s2 - 1) a_gload(as, i, kt + 1 + AD);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int kt = s0; kt < s1; kt += RING) {
    slab(0, 0, kt);
    slab(1, 1, kt + 1);
    if constexpr (RING == 4) {
      slab(0, 2, kt + 2);
      slab(1, 3, kt + 3);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  // split K: partial tile of split t at part + (tile ks + t) BM BN; chunk q =
  // (i FN + j) 4 + r4 of thread tid (4 floats) at ((q * 256) + tid) * 16
  // bytes, so each store and load of a wavefront is 1 KB contiguous
  constexpr uint32_t TILE_BYTES = BM * BN * 4u;
  const __amdgpu_buffer_rsrc_t all =
      make_rsrc(SPLIT ? ep.part + static_cast<size_t>(tile) * ks * (BM * BN) : nullptr,
                SPLIT ? TILE_BYTES * static_cast<uint32_t>(ks) : 0u);
  if constexpr (SPLIT) {  // hand the partial tile over; only the last split goes on
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
          buf_store16_sc1(all, v, static_cast<uint32_t>((((i * FN + j) * 4 + r4) * 256 + tid) * 16) +
                                      static_cast<uint32_t>(split) * TILE_BYTES);
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partial has reached the coherent level
    __syncthreads();
    if (tid == 0) {
      s_last = __hip_atomic_fetch_add(ep.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               static_cast<unsigned>(ks - 1);
      if (s_last) __hip_atomic_store(ep.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // re-arm
    }
    __syncthreads();
    if (!s_last) return;
  }

  // ---------------------------------------------------------------- epilogue
  // Each wave moves its tile through LDS one 32-row block at a time, so the
  // elementwise work and the global traffic run on row-contiguous data:
  // 8 consecutive columns per task, 16/32-byte loads and stores.
  __syncthreads();  // every wave is done with the A stages
  float* ebuf = reinterpret_cast<float*>((wave < 2 ? As0 : As1) + (wave & 1) * EPI_WAVE);
  const int lc = lane & 31, hr = 4 * (lane >> 5);
  const int col0 = n0 + wn * TN;  // first column of this wave's tile
  if (col0 >= N) return;
  auto ld8 = [&](int R, int c) {  // 8 fp32 of row R from column c
    const float4 a = *reinterpret_cast<const float4*>(ebuf + R * TNP + c);
    const float4 b = *reinterpret_cast<const float4*>(ebuf + R * TNP + c + 4);
    return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  };
  auto bf8 = [](const f32x8& v) {
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
  };
  // QKV: a lane's tasks keep their row offset and columns in every pass, so
  // the positions of all its task rows are fetched once, before the first
  // pass, and the RoPE cos/sin of pass i + 1 are fetched while pass i runs
  // (in place of two dependent global loads per task and pass)
  constexpr int NTQ = EPI == EPI_QKV ? TN / 16 : 1;  // tasks per lane and pass
  int qpos[FM][NTQ];
  f32x4 qcos[2][NTQ], qsin[2][NTQ];
  auto qkv_cs = [&](int i, int buf) {
    const QkvEpilogue& q = ep.qkv;
#pragma unroll
    for (int k = 0; k < NTQ; ++k) {
      const int task = lane + 64 * k, c = 8 * (task % (TN / 8));
      const int x0 = ((col0 + c) & 127) >> 1;
      const int pt = min(max(qpos[i][k], 0), q.max_pos - 1);
      const float4 c4 = *reinterpret_cast<const float4*>(q.rope_cos + static_cast<size_t>(pt) * 64 + x0);
      const float4 s4 = *reinterpret_cast<const float4*>(q.rope_sin + static_cast<size_t>(pt) * 64 + x0);
      qcos[buf][k] = f32x4{c4.x, c4.y, c4.z, c4.w};
      qsin[buf][k] = f32x4{s4.x, s4.y, s4.z, s4.w};
    }
  };
  if constexpr (EPI == EPI_QKV) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int k = 0; k < NTQ; ++k) {
        const int row = m0 + wm * TM + i * 32 + (lane + 64 * k) / (TN / 8);
        qpos[i][k] = row < M ? ep.qkv.pos[row] : 0;
      }
    qkv_cs(0, 0);
  }
  // residual epilogues: the residual rows of pass i + 1 are fetched while
  // pass i runs (8 bf16 or 8 fp32 per task: one or two 16-byte loads)
  constexpr bool RESID = EPI == EPI_RESID32 || EPI == EPI_RESID16;
  constexpr int NTR = RESID ? TN / 16 : 1, RW = EPI == EPI_RESID16 ? 2 : 1;
  uint4 rres[2][NTR][RW];
  auto resid_fetch = [&](int i, int buf) {
#pragma unroll
    for (int k = 0; k < NTR; ++k) {
      const int task = lane + 64 * k, R = task / (TN / 8), c = 8 * (task % (TN / 8));
      const int row = m0 + wm * TM + i * 32 + R, col = col0 + c;
      const bool ok = row < M && col < N;
      const size_t at = ok ? static_cast<size_t>(row) * N + col : 0;
#pragma unroll
      for (int w = 0; w < RW; ++w)
        rres[buf][k][w] = EPI == EPI_RESID16
                              ? *reinterpret_cast<const uint4*>(static_cast<const float*>(ep.resid) + at + 4 * w)
                              : *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(ep.resid) + at);
    }
  };
  if constexpr (RESID) resid_fetch(0, 0);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if constexpr (EPI == EPI_QKV) {
      if (i + 1 < FM) qkv_cs(i + 1, (i + 1) & 1);
    }
    if constexpr (RESID) {
      if (i + 1 < FM) resid_fetch(i + 1, (i + 1) & 1);
    }
    // registers -> LDS: acc[i][j][r] is row 8 (r/4) + hr + r%4, column 32 j + lc
    if constexpr (SPLIT) {
      // the last split: the same values as the sum of the ks partials, added
      // in split order (its own partial read back like the others), one
      // 32 x 32 block (4 chunks x ks loads) at a time
      auto put = [&](auto ks_tag) {
        constexpr int KS = decltype(ks_tag)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          f32x4 v[4][KS];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
            for (int t = 0; t < KS; ++t)
              v[r4][t] = buf_load16_sc1(all, static_cast<uint32_t>((((i * FN + j) * 4 + r4) * 256 + tid) * 16) +
                                                 static_cast<uint32_t>(t) * TILE_BYTES);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 sum = v[r4][0];
#pragma unroll
            for (int t = 1; t < KS; ++t) sum += v[r4][t];
#pragma unroll
            for (int e = 0; e < 4; ++e) ebuf[(8 * r4 + hr + e) * TNP + 32 * j + lc] = sum[e];
          }
        }
      };
      if (ks == 2) put(std::integral_constant<int, 2>{});
      else if (ks == 3) put(std::integral_constant<int, 3>{});
      else put(std::integral_constant<int, 4>{});
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) ebuf[(8 * (r >> 2) + hr + (r & 3)) * TNP + 32 * j + lc] = acc[i][j][r];
    }
    // the same wave reads the block back: its LDS accesses complete in order
    const int row0 = m0 + wm * TM + i * 32;
    if constexpr (EPI == EPI_QKV) {
      // rotary-pair order: column 2x of a head is dim x, column 2x + 1 dim
      // x + 64.  Task: row R, 8 columns = dims x0 .. x0 + 3 and their partners.
      const QkvEpilogue& q = ep.qkv;
#pragma unroll
      for (int k = 0; k < TN / 16; ++k) {
        const int task = lane + 64 * k, R = task / (TN / 8), c = 8 * (task % (TN / 8));
        const int row = row0 + R, col = col0 + c;
        if (row >= M || col >= N) continue;
        const f32x8 a = ld8(R, c);
        f32x4 x1 = {a[0], a[2], a[4], a[6]}, x2 = {a[1], a[3], a[5], a[7]};
        const int head = col >> 7, x0 = (col & 127) >> 1;
        const int kind = head < q.n_heads ? 0 : (head < q.n_heads + q.n_kv_heads ? 1 : 2);
        const int hh = kind == 0 ? head : (kind == 1 ? head - q.n_heads : head - q.n_heads - q.n_kv_heads);
        const int p = qpos[i][k];
        if (kind != 2) {
          const f32x4 cs = qcos[i & 1][k], sn = qsin[i & 1][k];
          const f32x4 y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
          x1 = y1;
          x2 = y2;
        }
        bf16_t* dst;
        if (kind == 0) {
          dst = q.q + static_cast<size_t>(row) * (q.n_heads * 128) + hh * 128;
        } else {
          if (p < 0 || p >= q.span) continue;
          const long long kr = q.stage ? static_cast<long long>(row) * q.n_kv_heads + hh
                                       : kv_row(q.pg, row / q.T, hh, q.n_kv_heads, q.max_pos, p);
          if (kr < 0) continue;  // no valid page for this slot
          dst = (kind == 1 ? q.k_cache : q.v_cache) + kr * 128;
        }
        *reinterpret_cast<uint2*>(dst + x0) = make_uint2(pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3]));
        *reinterpret_cast<uint2*>(dst + x0 + 64) = make_uint2(pack_bf16x2(x2[0], x2[1]), pack_bf16x2(x2[2], x2[3]));
      }
    } else if constexpr (EPI == EPI_SWIGLU) {
      static_assert(TN == 128, "SwiGLU tiles are one [gate 64 | up 64] block per wave");
      // task: row R, gate columns 8c .. 8c + 7 and the up columns 64 later
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int task = lane + 64 * k, R = task >> 3, c = 8 * (task & 7);
        const int row = row0 + R;
        if (row >= M) continue;
        const f32x8 x1 = ld8(R, c), x2 = ld8(R, c + 64);
        f32x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = silu(x1[e]) * x2[e];
        const int f = N >> 1;
        *reinterpret_cast<uint4*>(static_cast<bf16_t*>(ep.out) + static_cast<size_t>(row) * f + (col0 >> 7) * 64 + c) =
            make_uint4(pack_f16x2_sat(h[0], h[1]), pack_f16x2_sat(h[2], h[3]), pack_f16x2_sat(h[4], h[5]),
                       pack_f16x2_sat(h[6], h[7]));
      }
    } else {
      // task: row R, columns 8c .. 8c + 7
#pragma unroll
      for (int k = 0; k < TN / 16; ++k) {
        const int task = lane + 64 * k, R = task / (TN / 8), c = 8 * (task % (TN / 8));
        const int row = row0 + R, col = col0 + c;
        if (row >= M || col >= N) continue;
        const f32x8 a = ld8(R, c);
        const size_t at = static_cast<size_t>(row) * N + col;
        if constexpr (EPI == EPI_RESID32) {
          const uint4 rb = rres[i & 1][k][0];
          float* o = static_cast<float*>(ep.out) + at;
          *reinterpret_cast<float4*>(o) = make_float4(a[0] + lo_bf16(rb.x), a[1] + hi_bf16(rb.x), a[2] + lo_bf16(rb.y), a[3] + hi_bf16(rb.y));
          *reinterpret_cast<float4*>(o + 4) = make_float4(a[4] + lo_bf16(rb.z), a[5] + hi_bf16(rb.z), a[6] + lo_bf16(rb.w), a[7] + hi_bf16(rb.w));
        } else {
          const uint4 r0 = rres[i & 1][k][0], r1 = rres[i & 1][k][RW - 1];
          const f32x8 rs = {__uint_as_float(r0.x), __uint_as_float(r0.y), __uint_as_float(r0.z), __uint_as_float(r0.w),
                            __uint_as_float(r1.x), __uint_as_float(r1.y), __uint_as_float(r1.z), __uint_as_float(r1.w)};
          *reinterpret_cast<uint4*>(static_cast<bf16_t*>(ep.out) + at) = bf8(a + rs);
        }
      }
    }
  }
}

// K splits for `tiles` tiles of `cycles` ring cycles each: as many as keep the
// grid within one round (at most 4, each split at least two cycles) when the
// tiles fill at most half the CUs; else 1
int split_count(int tiles, int cycles, const GemmSplit& gs) {
  if (!gs.part || !gs.cnt) return 1;
  const int n_cu = device_cu_count();
  if (2 * tiles > n_cu) return 1;
  int ks = n_cu / tiles < 4 ? n_cu / tiles : 4;
  if (ks > cycles / 2) ks = cycles / 2;
  return ks >= 2 ? ks : 1;
}

// Weight ring depth: a wave tile with 8 MFMAs per k step (128 x 256 tiles)
// gets a 4-slab ring, so a weight load that misses L2 still has ~3 slabs of
// MFMA work (~0.4 us per slab) to arrive; wider tiles do 12-16 MFMAs per k step and
// keep 2 slabs (their registers go to the accumulators).  A 4-slab ring
// needs K % 256 == 0, else the 2-slab ring runs.
template <int BM, int BN, int EPI>
hipError_t launch_tiled(const bf16_t* A, const bf16_t* Wp, int M, int N, int K, EpiArgs ep, const GemmSplit& gs,
                        hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const bool ring4 = BM == 128 && BN == 256 && K % 256 == 0;
  ep.ks = split_count(tiles, K / BK / (ring4 ? 4 : 2), gs);
  ep.part = gs.part;
  ep.cnt = gs.cnt;
  const dim3 grid(static_cast<unsigned>(tiles * ep.ks));
  const bool split = ep.ks > 1;
  if constexpr (BM == 128 && BN == 256) {
    if (ring4) {
      if (split) hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI, 4, true>), grid, dim3(256), 0, s, A, Wp, M, N, K, ep);
      else hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI, 4, false>), grid, dim3(256), 0, s, A, Wp, M, N, K, ep);
      return hipGetLastError();
    }
  }
  if (split) hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI, 2, true>), grid, dim3(256), 0, s, A, Wp, M, N, K, ep);
  else hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI, 2, false>), grid, dim3(256), 0, s, A, Wp, M, N, K, ep);
  return hipGetLastError();
}

// rounds of one tile per CU for BM x BN tiles
long rounds(int M, int N, int BM, int BN, int n_cu) {
  return ((static_cast<long>(M + BM - 1) / BM) * ((N + BN - 1) / BN) + n_cu - 1) / n_cu;
}

// 128 x 512 tiles do a 128 x 256 tile's work in ~1.6x its time (measured on
// the 13B / 70B o_proj and down shapes); take them when that wins after
// rounding each choice up to whole rounds of one tile per CU.
bool wide_resid_tiles(int M, int N) {
  const int n_cu = device_cu_count();
  return 8 * rounds(M, N, 128, 512, n_cu) < 5 * rounds(M, N, 128, 256, n_cu);
}

// QKV: a 128 x 512 tile (one head per wave) does 4/3 of a 256 x 192 tile's
// work in ~1.2x its time (measured at the 13B and 70B shapes); the same
// rounding rule decides.
bool wide_qkv_tiles(int M, int N) {
  const int n_cu = device_cu_count();
  return 40 * rounds(M, N, 128, 512, n_cu) < 33 * rounds(M, N, 256, 192, n_cu);
}
}  // namespace

int device_cu_count() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    n_cu = 256;
  return n_cu;
}

size_t gemm_split_part_floats() { return static_cast<size_t>(device_cu_count()) * 128 * 512; }

hipError_t launch_gemm_qkv(const bf16_t* A, const bf16_t* W, int M, int N, int K, const QkvEpilogue& q,
                           const GemmSplit& gs, hipStream_t s) {
  EpiArgs ep{}; ep.qkv = q;
  return wide_qkv_tiles(M, N) ? launch_tiled<128, 512, EPI_QKV>(A, W, M, N, K, ep, gs, s)
                              : launch_tiled<256, kQkvBN, EPI_QKV>(A, W, M, N, K, ep, gs, s);
}
hipError_t launch_gemm_resid_f32out(const bf16_t* A, const bf16_t* W, int M, int N, int K, const bf16_t* resid,
                                    float* out, const GemmSplit& gs, hipStream_t s) {
  EpiArgs ep{}; ep.resid = resid; ep.out = out;
  return wide_resid_tiles(M, N) ? launch_tiled<128, 512, EPI_RESID32>(A, W, M, N, K, ep, gs, s)
                                : launch_tiled<128, 256, EPI_RESID32>(A, W, M, N, K, ep, gs, s);
}
hipError_t launch_gemm_resid_bf16out(const bf16_t* A, const bf16_t* W, int M, int N, int K, const float* resid,
                                     bf16_t* out, const GemmSplit& gs, hipStream_t s) {
  EpiArgs ep{}; ep.resid = resid; ep.out = out;
  return wide_resid_tiles(M, N) ? launch_tiled<128, 512, EPI_RESID16>(A, W, M, N, K, ep, gs, s)
                                : launch_tiled<128, 256, EPI_RESID16>(A, W, M, N, K, ep, gs, s);
}
hipError_t launch_gemm_swiglu(const bf16_t* A, const bf16_t* Wgu, int M, int N, int K, bf16_t* out,
                              const GemmSplit& gs, hipStream_t s) {
  EpiArgs ep{}; ep.out = out;
  return N % 512 == 0 ? launch_tiled<128, 512, EPI_SWIGLU>(A, Wgu, M, N, K, ep, gs, s)
                      : launch_tiled<256, 256, EPI_SWIGLU>(A, Wgu, M, N, K, ep, gs, s);
}
}  // namespace llama
