// MFMA GEMM  Y[M,N] = A[M,K] . W[N,K]^T  with fused epilogues.
//
// Every linear layer of the model is y = x W^T + b with W stored [out, in]
// ("第 25 章 从小 GPT 到 GPT-2" §25.5), so A and W are both K-contiguous and
// the same kernel serves c_attn, c_proj, c_fc, mlp.c_proj and the tied head
// (whose W is the token table E [V, C] itself, §25.4).
//
// Block tile BM x BN, K step BK, staged through LDS (double-buffered, one
// barrier per K step, global loads for step k+1 in flight while step k is
// multiplied).  Each wave owns a WM x WN sub-tile made of 32x32 MFMA tiles.
// Epilogues run on the fp32 accumulators:
//   EpiQKV   : + bias, scatter Q -> [B,H,T,D], K and U -> [B,H,Tk,D]
//   EpiResid : + bias, x += (fp32 residual stream)
//   EpiAct   : + bias, optional tanh-GELU, store in the output dtype
//   head     : optional logits store + per-(row, N-tile) softmax partials
//              (max, sum exp) and the target logit, all from fp32 accumulators.
#include "gemm_core.h"

namespace gptmi {

// ---------------------------------------------------------------------------
// Skinny products: at most 64 rows (one token per sequence in a decode step,
// or the last position of each prompt).  Every weight is used by at most 64
// rows, so the weight stream from HBM sets the time.  Two kernels:
//  * the LDS-staged one (rows contiguous, K a multiple of 128; further below)
//    for every product of the model;
//  * a register path for the rest: a block owns 32 output columns and all
//    rows; its 8 waves split K into contiguous ranges and load their MFMA
//    fragments straight from global memory (no LDS staging; U k-steps of
//    loads in flight per wave).
// Both sum the eight waves' partial 64 x 32 tiles through LDS; wave 0 then
// holds the block's sum in the usual accumulator layout (rows 0-31 in
// acc[0], 32-63 in acc[1]) and runs the epilogue.
constexpr int SK_WAVES = 8;
constexpr int SK_RED = 2 * 16 * 64;   // floats of one wave's partial tile
constexpr int SK_SMEM = SK_WAVES * SK_RED * 4;

// Split K over blocks (S = gridDim.y > 1), called by wave 0 with the block's
// partial tile: publish it and count it on the column tile's counter.  Returns
// true in the block that arrives last, which then holds the sum of the S
// partials in split order and has reset the counter to zero.
__device__ __forceinline__ bool skinny_split_finish(f32x16 (&acc)[2][1], float* __restrict__ part,
                                                    int* __restrict__ cnt) {
  const int lane = threadIdx.x & 63, S = gridDim.y;
  float* const tile = part + (size_t)blockIdx.x * S * SK_RED;
  float* const mine = tile + (size_t)blockIdx.y * SK_RED;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    mine[e * 64 + lane] = acc[0][0][e];
    mine[1024 + e * 64 + lane] = acc[1][0][e];
  }
  // device scope: the blocks of one column tile may run on different XCDs
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(cnt + blockIdx.x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, 64);
  if (old != S - 1) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc[0][0][e] = tile[e * 64 + lane];
    acc[1][0][e] = tile[1024 + e * 64 + lane];
  }
  for (int y = 1; y < S; ++y) {
    const float* py = tile + (size_t)y * SK_RED;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[0][0][e] += py[e * 64 + lane];
      acc[1][0][e] += py[1024 + e * 64 + lane];
    }
  }
  if (lane == 0) cnt[blockIdx.x] = 0;
  return true;
}

// Sum of the eight waves' partial tiles through LDS (`red`, SK_SMEM bytes, free
// on entry); wave 0 receives the total.  Returns true in wave 0 only.
__device__ __forceinline__ bool skinny_block_sum(const f32x16& c0, const f32x16& c1, float* red, f32x16 (&acc)[2][1]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* mine = red + wave * SK_RED;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    mine[e * 64 + lane] = c0[e];
    mine[1024 + e * 64 + lane] = c1[e];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < SK_RED; e += SK_WAVES * 64) {
    float t = red[e];
#pragma unroll
    for (int w2 = 1; w2 < SK_WAVES; ++w2) t += red[w2 * SK_RED + e];
    red[e] = t;
  }
  __syncthreads();
  if (wave != 0) return false;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc[0][0][e] = red[e * 64 + lane];
    acc[1][0][e] = red[1024 + e * 64 + lane];
  }
  return true;
}

// A [M, K] bf16 in global memory (lda); `smem` holds the partial-sum
// reduction.  U k-steps of loads are in flight per wave.
template <int U>
__device__ __forceinline__ bool skinny_mainloop(const bf16* __restrict__ A, int lda, const bf16* __restrict__ W,
                                                int ldw, int M, int N, int K, int n0, char* smem,
                                                f32x16 (&acc)[2][1]) {
  typedef Mfma<bf16> MF;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int steps = (K + 15) >> 4;
  const int per = (steps + SK_WAVES - 1) / SK_WAVES;
  const int s_begin = wave * per, s_end = min(steps, s_begin + per);
  const int nrows = min(32, N - n0);
  // rows past M (A) and past N (W) lie outside the resources and read as zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((size_t)M * lda * sizeof(bf16)));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * ldw, (uint32_t)((size_t)nrows * ldw * sizeof(bf16)));
  const int r = lane & 31, kh = (lane >> 5) * MF::KPL;
  const uint32_t oa0 = (uint32_t)(r * lda + kh) * 2, oa1 = (uint32_t)((r + 32) * lda + kh) * 2;
  const uint32_t ow = (uint32_t)(r * ldw + kh) * 2;
  const uint4 z = make_uint4(0, 0, 0, 0);
  uint4 w[U];
  auto load_w = [&](int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 16;
      const bool ok = s + u < s_end && k + kh < K;   // K % 8 == 0: a lane's 8 values are all in or all out
      w[u] = ok ? buf_load16(rw, ow, k * 2) : z;
    }
  };
  load_w(s_begin);
  f32x16 c0, c1;
#pragma unroll
  for (int e = 0; e < 16; ++e) { c0[e] = 0.f; c1[e] = 0.f; }
  for (int s = s_begin; s < s_end; s += U) {
    if (s != s_begin) load_w(s);
    uint4 a0[U], a1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 16;
      const bool ok = s + u < s_end && k + kh < K;
      a0[u] = ok ? buf_load16(ra, oa0, k * 2) : z;
      a1[u] = ok ? buf_load16(ra, oa1, k * 2) : z;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const MF::frag wf = __builtin_bit_cast(MF::frag, w[u]);
      c0 = MF::mma(__builtin_bit_cast(MF::frag, a0[u]), wf, c0);
      c1 = MF::mma(__builtin_bit_cast(MF::frag, a1[u]), wf, c1);
    }
  }
  return skinny_block_sum(c0, c1, reinterpret_cast<float*>(smem), acc);
}

template <typename Epi, int U>
__global__ void __launch_bounds__(SK_WAVES * 64) gemm_skinny_kernel(const bf16* __restrict__ A, int lda,
                                                                   const bf16* __restrict__ W, int ldw, int M, int N,
                                                                   int K, Epi epi) {
  __shared__ __align__(16) char smem[SK_SMEM];
  const int n0 = blockIdx.x * 32;
  float2 pre[2][1][8];
  typename Epi::Col colv[1];
  if ((threadIdx.x >> 6) == 0) preload_pairs<2, 1>(pre, colv, 0, n0, M, N, epi);
  f32x16 acc[2][1];
  if (!skinny_mainloop<U>(A, lda, W, ldw, M, N, K, n0, smem, acc)) return;
  epilogue_pairs<2, 1>(acc, pre, colv, 0, n0, M, N, epi);
}

// Skinny products whose K range is staged in LDS with full-line DMA loads
// (rows contiguous: lda = ldw = K, K a multiple of 64 NSTG).  The register
// path above reads 32 bytes of 32 different rows per load instruction; here
// every instruction reads eight whole 128-byte lines.  Block: 32 output
// columns, all rows (<= 64), K range [k0, k0 + 64 NSTG) of split
// blockIdx.y.  LDS: NSTG stages of 96 rows x 128 bytes (A rows 0-63, W rows
// 64-95), chunk c of row r at slot swz<8>(r, c).  Every load is issued at
// once; then each wave multiplies its share of the 4 NSTG k-substeps and the
// eight partial tiles are summed in the (then free) stages.
template <int NSTG>
struct SkLds {
  static constexpr int ROWS = 96, STAGE = ROWS * 128, NI = NSTG * ROWS / 8, DPW = NI / SK_WAVES;
  static constexpr int BYTES = NSTG * STAGE > SK_SMEM ? NSTG * STAGE : SK_SMEM;
  static_assert(NI % SK_WAVES == 0 && DPW < 64, "loads must split evenly over the waves");
};

template <typename Epi, int NSTG>
__global__ void __launch_bounds__(SK_WAVES * 64) gemm_skinny_lds_kernel(const bf16* __restrict__ A,
                                                                       const bf16* __restrict__ W, int M, int N, int K,
                                                                       Epi epi, float* __restrict__ part,
                                                                       int* __restrict__ cnt) {
  typedef SkLds<NSTG> L;
  __shared__ __align__(1024) char lds[L::BYTES];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * NSTG * 64;
  const int nrows = min(32, N - n0);
  // rows past M (A) and past N (W) lie outside the resources and read as zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((size_t)M * K * sizeof(bf16)));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * K, (uint32_t)((size_t)nrows * K * sizeof(bf16)));
#pragma unroll
  for (int d = 0; d < L::DPW; ++d) {
    const int ins = wave + d * SK_WAVES;           // uniform: stage ins / 12, rows 8 (ins % 12) ..
    const int st = ins / 12, ri = ins % 12;
    const int row = ri * 8 + lane / 8, slot = lane % 8;
    const int grow = ri < 8 ? row : row - 64;
    dma16(ri < 8 ? ra : rw, as_lds(lds) + st * L::STAGE + ri * 1024, (uint32_t)((grow * K + swz<8>(row, slot) * 8) * 2),
          (uint32_t)((k0 + st * 64) * 2));
  }
  float2 pre[2][1][8];
  typename Epi::Col colv[1];
  if (wave == 0) preload_pairs<2, 1>(pre, colv, 0, n0, M, N, epi);
  wait_vmcnt<0>();
  lds_barrier();
  typedef Mfma<bf16> MF;
  f32x16 c0, c1;
#pragma unroll
  for (int e = 0; e < 16; ++e) { c0[e] = 0.f; c1[e] = 0.f; }
  const int lrow = lane & 31, g = lane >> 5;
#pragma unroll
  for (int it = 0; it < NSTG * 4 / SK_WAVES; ++it) {
    const int j = it * SK_WAVES + wave, c = (j & 3) * 2 + g;
    const char* s = lds + (j >> 2) * L::STAGE;
    const MF::frag a0 = __builtin_bit_cast(MF::frag, *reinterpret_cast<const uint4*>(s + lrow * 128 + swz<8>(lrow, c) * 16));
    const MF::frag a1 = __builtin_bit_cast(
        MF::frag, *reinterpret_cast<const uint4*>(s + (lrow + 32) * 128 + swz<8>(lrow + 32, c) * 16));
    const MF::frag wf = __builtin_bit_cast(
        MF::frag, *reinterpret_cast<const uint4*>(s + (lrow + 64) * 128 + swz<8>(lrow + 64, c) * 16));
    c0 = MF::mma(a0, wf, c0);
    c1 = MF::mma(a1, wf, c1);
  }
  __syncthreads();   // the stages become the reduction buffer
  f32x16 acc[2][1];
  if (!skinny_block_sum(c0, c1, reinterpret_cast<float*>(lds), acc)) return;
  if (gridDim.y > 1 && !skinny_split_finish(acc, part, cnt)) return;
  epilogue_pairs<2, 1>(acc, pre, colv, 0, n0, M, N, epi);
}

// Split-K skinny product without an epilogue: slice s = blockIdx.y of K
// (columns [64 NSTG s, 64 NSTG (s + 1))) of a 32-column tile is written as a
// raw fp32 partial product, part[(s M + m) N + n].  The block stages and
// multiplies exactly as gemm_skinny_lds_kernel; its eight waves' partial tiles
// are summed in wave order through the freed stages and every thread stores
// the four sums it made (two rows of 32 columns per wave and instruction).
// No block waits on another: the consumer adds the slices in slice order
// together with the bias (and the residual), so the result does not depend
// on which block finishes first.
template <int NSTG>
__global__ void __launch_bounds__(SK_WAVES * 64) gemm_skinny_slices_kernel(const bf16* __restrict__ A,
                                                                          const bf16* __restrict__ W, int M, int N,
                                                                          int K, float* __restrict__ part) {
  typedef SkLds<NSTG> L;
  __shared__ __align__(1024) char lds[L::BYTES];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * NSTG * 64;
  const int nrows = min(32, N - n0);
  // rows past M (A) and past N (W) lie outside the resources and read as zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((size_t)M * K * sizeof(bf16)));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * K, (uint32_t)((size_t)nrows * K * sizeof(bf16)));
#pragma unroll
  for (int d = 0; d < L::DPW; ++d) {
    const int ins = wave + d * SK_WAVES;           // uniform: stage ins / 12, rows 8 (ins % 12) ..
    const int st = ins / 12, ri = ins % 12;
    const int row = ri * 8 + lane / 8, slot = lane % 8;
    const int grow = ri < 8 ? row : row - 64;
    dma16(ri < 8 ? ra : rw, as_lds(lds) + st * L::STAGE + ri * 1024, (uint32_t)((grow * K + swz<8>(row, slot) * 8) * 2),
          (uint32_t)((k0 + st * 64) * 2));
  }
  wait_vmcnt<0>();
  lds_barrier();
  typedef Mfma<bf16> MF;
  f32x16 c0, c1;
#pragma unroll
  for (int e = 0; e < 16; ++e) { c0[e] = 0.f; c1[e] = 0.f; }
  const int lrow = lane & 31, g = lane >> 5;
#pragma unroll
  for (int it = 0; it < NSTG * 4 / SK_WAVES; ++it) {
    const int j = it * SK_WAVES + wave, c = (j & 3) * 2 + g;
    const char* s = lds + (j >> 2) * L::STAGE;
    const MF::frag a0 = __builtin_bit_cast(MF::frag, *reinterpret_cast<const uint4*>(s + lrow * 128 + swz<8>(lrow, c) * 16));
    const MF::frag a1 = __builtin_bit_cast(
        MF::frag, *reinterpret_cast<const uint4*>(s + (lrow + 32) * 128 + swz<8>(lrow + 32, c) * 16));
    const MF::frag wf = __builtin_bit_cast(
        MF::frag, *reinterpret_cast<const uint4*>(s + (lrow + 64) * 128 + swz<8>(lrow + 64, c) * 16));
    c0 = MF::mma(a0, wf, c0);
    c1 = MF::mma(a1, wf, c1);
  }
  __syncthreads();   // the stages become the reduction buffer
  float* red = reinterpret_cast<float*>(lds);
  float* mine = red + wave * SK_RED;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    mine[e * 64 + lane] = c0[e];
    mine[1024 + e * 64 + lane] = c1[e];
  }
  __syncthreads();
  float* out = part + (size_t)blockIdx.y * M * N;
  for (int e = threadIdx.x; e < SK_RED; e += SK_WAVES * 64) {
    float t = red[e];
#pragma unroll
    for (int w2 = 1; w2 < SK_WAVES; ++w2) t += red[w2 * SK_RED + e];
    // element e: accumulator half e / 1024, register r, lane l of the MFMA layout
    const int r = (e >> 6) & 15, l = e & 63;
    const int m = (e >> 10) * 32 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3), n = n0 + (l & 31);
    if (m < M && n < N) out[(size_t)m * N + n] = t;
  }
}

template <int NSTG>
static hipError_t run_skinny_slices(const bf16* A, const bf16* W, int M, int N, int K, float* part, hipStream_t st) {
  const int tiles = (N + 31) / 32, S = K / (64 * NSTG);
  hipLaunchKernelGGL((gemm_skinny_slices_kernel<NSTG>), dim3(tiles, S), dim3(SK_WAVES * 64), 0, st, A, W, M, N, K,
                     part);
  return hipGetLastError();
}

// The same product for 33..64 rows split into two 32-row halves
// (blockIdx.y): a block stages only its half of A next to its 32 weight rows
// (64 rows x 128 bytes per stage; 96 KB instead of 144 KB for K = 768), so
// twice as many blocks each bring in two thirds of the bytes.  Each wave
// multiplies a share of the k-substeps into one 32 x 32 tile; the eight
// partial tiles are summed in wave order in the freed stages and wave 0 runs
// the epilogue on rows 32 h ...
template <int NSTG>
struct SkHalf {
  static constexpr int ROWS = 64, STAGE = ROWS * 128, NI = NSTG * ROWS / 8, DPW = NI / SK_WAVES;
  static constexpr int RED = SK_WAVES * 16 * 64 * 4;   // eight 32 x 32 fp32 tiles
  static constexpr int BYTES = NSTG * STAGE > RED ? NSTG * STAGE : RED;
  static_assert(NI % SK_WAVES == 0 && DPW < 64, "loads must split evenly over the waves");
};

template <typename Epi, int NSTG>
__global__ void __launch_bounds__(SK_WAVES * 64) gemm_skinny_half_kernel(const bf16* __restrict__ A,
                                                                        const bf16* __restrict__ W, int M, int N, int K,
                                                                        Epi epi) {
  typedef SkHalf<NSTG> L;
  __shared__ __align__(1024) char lds[L::BYTES];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * 32;
  const int nrows = min(32, N - n0), mrows = min(32, M - m0);
  // rows past M (A) and past N (W) lie outside the resources and read as zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)((size_t)mrows * K * sizeof(bf16)));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * K, (uint32_t)((size_t)nrows * K * sizeof(bf16)));
#pragma unroll
  for (int d = 0; d < L::DPW; ++d) {
    const int ins = wave + d * SK_WAVES;           // uniform: stage ins / 8, rows 8 (ins % 8) ..
    const int st = ins / 8, ri = ins % 8;
    const int row = ri * 8 + lane / 8, slot = lane % 8;
    const int grow = ri < 4 ? row : row - 32;
    dma16(ri < 4 ? ra : rw, as_lds(lds) + st * L::STAGE + ri * 1024, (uint32_t)((grow * K + swz<8>(row, slot) * 8) * 2),
          (uint32_t)(st * 64 * 2));
  }
  float2 pre[1][1][8];
  typename Epi::Col colv[1];
  if (wave == 0) preload_pairs<1, 1>(pre, colv, m0, n0, M, N, epi);
  wait_vmcnt<0>();
  lds_barrier();
  typedef Mfma<bf16> MF;
  f32x16 c0;
#pragma unroll
  for (int e = 0; e < 16; ++e) c0[e] = 0.f;
  const int lrow = lane & 31, g = lane >> 5;
#pragma unroll
  for (int it = 0; it < NSTG * 4 / SK_WAVES; ++it) {
    const int j = it * SK_WAVES + wave, c = (j & 3) * 2 + g;
    const char* s = lds + (j >> 2) * L::STAGE;
    const MF::frag a0 = __builtin_bit_cast(MF::frag, *reinterpret_cast<const uint4*>(s + lrow * 128 + swz<8>(lrow, c) * 16));
    const MF::frag wf = __builtin_bit_cast(
        MF::frag, *reinterpret_cast<const uint4*>(s + (lrow + 32) * 128 + swz<8>(lrow + 32, c) * 16));
    c0 = MF::mma(a0, wf, c0);
  }
  __syncthreads();   // the stages become the reduction buffer
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int e = 0; e < 16; ++e) red[wave * 1024 + e * 64 + lane] = c0[e];
  __syncthreads();
  if (wave != 0) return;
  f32x16 acc[1][1];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float t = red[e * 64 + lane];
#pragma unroll
    for (int w2 = 1; w2 < SK_WAVES; ++w2) t += red[w2 * 1024 + e * 64 + lane];
    acc[0][0][e] = t;
  }
  epilogue_pairs<1, 1>(acc, pre, colv, m0, n0, M, N, epi);
}

// K-slices of 33..64 rows in two 32-row halves (blockIdx.z): the staging of
// gemm_skinny_half_kernel, the partial tile stored as gemm_skinny_slices_kernel
// stores it (rows 32 h ..).
template <int NSTG>
__global__ void __launch_bounds__(SK_WAVES * 64) gemm_skinny_slices_half_kernel(const bf16* __restrict__ A,
                                                                               const bf16* __restrict__ W, int M,
                                                                               int N, int K, float* __restrict__ part) {
  typedef SkHalf<NSTG> L;
  __shared__ __align__(1024) char lds[L::BYTES];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 32, k0 = blockIdx.y * NSTG * 64, m0 = blockIdx.z * 32;
  const int nrows = min(32, N - n0), mrows = min(32, M - m0);
  // rows past M (A) and past N (W) lie outside the resources and read as zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)((size_t)mrows * K * sizeof(bf16)));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * K, (uint32_t)((size_t)nrows * K * sizeof(bf16)));
#pragma unroll
  for (int d = 0; d < L::DPW; ++d) {
    const int ins = wave + d * SK_WAVES;           // uniform: stage ins / 8, rows 8 (ins % 8) ..
    const int st = ins / 8, ri = ins % 8;
    const int row = ri * 8 + lane / 8, slot = lane % 8;
    const int grow = ri < 4 ? row : row - 32;
    dma16(ri < 4 ? ra : rw, as_lds(lds) + st * L::STAGE + ri * 1024, (uint32_t)((grow * K + swz<8>(row, slot) * 8) * 2),
          (uint32_t)((k0 + st * 64) * 2));
  }
  wait_vmcnt<0>();
  lds_barrier();
  typedef Mfma<bf16> MF;
  f32x16 c0;
#pragma unroll
  for (int e = 0; e < 16; ++e) c0[e] = 0.f;
  const int lrow = lane & 31, g = lane >> 5;
#pragma unroll
  for (int it = 0; it < NSTG * 4 / SK_WAVES; ++it) {
    const int j = it * SK_WAVES + wave, c = (j & 3) * 2 + g;
    const char* s = lds + (j >> 2) * L::STAGE;
    const MF::frag a0 = __builtin_bit_cast(MF::frag, *reinterpret_cast<const uint4*>(s + lrow * 128 + swz<8>(lrow, c) * 16));
    const MF::frag wf = __builtin_bit_cast(
        MF::frag, *reinterpret_cast<const uint4*>(s + (lrow + 32) * 128 + swz<8>(lrow + 32, c) * 16));
    c0 = MF::mma(a0, wf, c0);
  }
  __syncthreads();   // the stages become the reduction buffer
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int e = 0; e < 16; ++e) red[wave * 1024 + e * 64 + lane] = c0[e];
  __syncthreads();
  float* out = part + (size_t)blockIdx.y * M * N;
  for (int e = threadIdx.x; e < 1024; e += SK_WAVES * 64) {
    float t = red[e];
#pragma unroll
    for (int w2 = 1; w2 < SK_WAVES; ++w2) t += red[w2 * 1024 + e];
    // element e: register r, lane l of the MFMA layout
    const int r = e >> 6, l = e & 63;
    const int m = m0 + (r >> 2) * 8 + (l >> 5) * 4 + (r & 3), n = n0 + (l & 31);
    if (m < M && n < N) out[(size_t)m * N + n] = t;
  }
}

template <int NSTG>
static hipError_t run_skinny_slices_any(const bf16* A, const bf16* W, int M, int N, int K, float* part,
                                        hipStream_t st) {
  if (M <= 32) return run_skinny_slices<NSTG>(A, W, M, N, K, part, st);
  const int tiles = (N + 31) / 32, S = K / (64 * NSTG);
  hipLaunchKernelGGL((gemm_skinny_slices_half_kernel<NSTG>), dim3(tiles, S, 2), dim3(SK_WAVES * 64), 0, st, A, W, M,
                     N, K, part);
  return hipGetLastError();
}

hipError_t launch_skinny_slices(const void* A, const void* W, int M, int N, int K, int S, float* part,
                                size_t part_floats, hipStream_t st) {
  if (!A || !W || !part || M <= 0 || M > 64 || N <= 0 || K <= 0 || S <= 0 || K % S != 0) return hipErrorInvalidValue;
  if ((size_t)S * M * N > part_floats) return hipErrorInvalidValue;
  const bf16* a = static_cast<const bf16*>(A);
  const bf16* w = static_cast<const bf16*>(W);
  switch (K / S) {   // the slice depth: NSTG stages of 64
    case 128: return run_skinny_slices_any<2>(a, w, M, N, K, part, st);
    case 256: return run_skinny_slices_any<4>(a, w, M, N, K, part, st);
    case 384: return run_skinny_slices_any<6>(a, w, M, N, K, part, st);
    case 512: return run_skinny_slices_any<8>(a, w, M, N, K, part, st);
    case 768: return run_skinny_slices_any<12>(a, w, M, N, K, part, st);
    default: return hipErrorInvalidValue;
  }
}

template <int NSTG, typename Epi>
static hipError_t run_skinny_lds(const bf16* A, const bf16* W, int M, int N, int K, const Epi& epi,
                                 const SkinnyWs* sk, hipStream_t st) {
  const int tiles = (N + 31) / 32, S = K / (64 * NSTG);
  if (K % (64 * NSTG) != 0) return hipErrorInvalidValue;
  if (S > 1 && (!sk || !sk->part || !sk->cnt || tiles > sk->cnt_len || tiles * S > sk->part_tiles))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_skinny_lds_kernel<Epi, NSTG>), dim3(tiles, S), dim3(SK_WAVES * 64), 0, st, A, W, M, N, K,
                     epi, S > 1 ? sk->part : nullptr, S > 1 ? sk->cnt : nullptr);
  return hipGetLastError();
}

// The LDS-staged kernel takes every product with contiguous rows and K a
// multiple of 128: up to 768 columns of K in one block, longer K split over
// blocks in ranges of 768 (or 512) when the caller gave split-K scratch.
template <typename Epi>
static hipError_t run_skinny(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int K, const Epi& epi,
                             const SkinnyWs* sk, hipStream_t st) {
  if (lda == K && ldw == K && K % 128 == 0) {
    const int n = K / 64, tiles = (N + 31) / 32;
    if (n == 12 && M > 32 && tiles <= 128) {   // two row halves: at most 256 blocks of 96 KB
      hipLaunchKernelGGL((gemm_skinny_half_kernel<Epi, 12>), dim3(tiles, 2), dim3(SK_WAVES * 64), 0, st, A, W, M, N,
                         K, epi);
      return hipGetLastError();
    }
    switch (n) {
      case 2: return run_skinny_lds<2>(A, W, M, N, K, epi, sk, st);
      case 4: return run_skinny_lds<4>(A, W, M, N, K, epi, sk, st);
      case 6: return run_skinny_lds<6>(A, W, M, N, K, epi, sk, st);
      case 8: return run_skinny_lds<8>(A, W, M, N, K, epi, sk, st);
      case 10: return run_skinny_lds<10>(A, W, M, N, K, epi, sk, st);
      case 12: return run_skinny_lds<12>(A, W, M, N, K, epi, sk, st);
      default: break;
    }
    const bool room = sk && sk->part && sk->cnt && tiles <= sk->cnt_len;
    if (room && n % 12 == 0 && tiles * (n / 12) <= sk->part_tiles) return run_skinny_lds<12>(A, W, M, N, K, epi, sk, st);
    if (room && n % 8 == 0 && tiles * (n / 8) <= sk->part_tiles) return run_skinny_lds<8>(A, W, M, N, K, epi, sk, st);
  }
  const int steps = (K + 15) / 16, per_wave = (steps + SK_WAVES - 1) / SK_WAVES;
  const dim3 grid((N + 31) / 32);
  if (per_wave <= 4)
    hipLaunchKernelGGL((gemm_skinny_kernel<Epi, 4>), grid, dim3(SK_WAVES * 64), 0, st, A, lda, W, ldw, M, N, K, epi);
  else if (per_wave <= 8)
    hipLaunchKernelGGL((gemm_skinny_kernel<Epi, 8>), grid, dim3(SK_WAVES * 64), 0, st, A, lda, W, ldw, M, N, K, epi);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<Epi, 12>), grid, dim3(SK_WAVES * 64), 0, st, A, lda, W, ldw, M, N, K, epi);
  return hipGetLastError();
}

// bf16 tied head computed transposed, Z^T = E . A^T: the MFMA rows are vocab
// entries and the columns are tokens, so every lane owns whole tokens.  The
// softmax partials of a token over this block's vocab entries are then a
// reduction over the lane's own registers, one exchange with the lane holding
// the other half of the rows (l ^ 32), and a combine over the waves along the
// vocab axis.  The target ids are read before the main loop.
//
// LDS after the main loop (the stages are free): every wave owns a slot of
// SW bytes where it gathers one 32-token column of its logits at a time as
// [token][vocab] rows (WM entries, a pitch of WM * 2 + 8 bytes, so the quad
// stores of 32 consecutive tokens meet no bank twice) and writes them out as
// 16-byte pieces of whole row spans: in the accumulators a lane holds 4
// consecutive vocab entries of one token, so direct stores would scatter
// 8 bytes over 32 token rows per instruction.  (The rows are only 2-byte
// aligned, V being odd; the 16-byte stores are unaligned.)  Slots fill the
// stages in order; the per-wave partials follow the last slot.
template <int BM, int BN, int WM, int WN, int NST, int BK>
struct HeadPlan {
  typedef DmaCfg<BM, BN, WM, WN, NST, BK> D;
  static constexpr int PITCH = WM * 2 + 8, SW = 32 * PITCH, WPS = D::STAGE / SW;
  static constexpr int PART = D::NWM * BN * 3 * 4;          // float max, sum; int argmax
  static constexpr int PST = D::NW / WPS, POFF = (D::NW % WPS) * SW;
  static_assert(WPS >= 1 && PST < NST && POFF + PART <= D::STAGE, "epilogue LDS plan must fit the stages");
  static_assert(WM % 8 == 0 && (32 * (WM / 8)) % 64 == 0, "whole 16-byte units per row, whole rounds per wave");
};

template <int K, int BM, int BN, int WM, int WN, int NST, int BK>   // BM: vocab, BN: tokens
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(dma_waves_per_eu<BM, BN, WM, WN, NST, BK>())))
head_ce_dma_kernel(const bf16* __restrict__ wte, const bf16* __restrict__ act, int V, int Mtok, HeadArgs ha) {
  typedef DmaCfg<BM, BN, WM, WN, NST, BK> D;
  typedef HeadPlan<BM, BN, WM, WN, NST, BK> P;
  __shared__ __align__(1024) char s0[D::STAGE];
  __shared__ __align__(1024) char s1[D::STAGE];
  __shared__ __align__(1024) char s2[NST > 2 ? D::STAGE : 16];
  __shared__ __align__(1024) char s3[NST > 3 ? D::STAGE : 16];
  static_assert(NST <= 4, "stage count");
  const Stages stages{{as_lds(s0), as_lds(s1), NST > 2 ? as_lds(s2) : as_lds(s0), NST > 3 ? as_lds(s3) : as_lds(s0),
                       as_lds(s0), as_lds(s0), as_lds(s0), as_lds(s0)}};
  const int num_v = (V + BM - 1) / BM, num_t = (Mtok + BN - 1) / BN;
  int tt, vt;
  tile_of(blockIdx.x, gridDim.x, num_t, num_v, tt, vt);   // groups of token tiles sweep the vocab
  const int v0 = vt * BM, t0 = tt * BN;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / D::NWN, wn = wave % D::NWN;
  const int vw0 = v0 + wm * WM;   // first vocab row of this wave
  const bool full = vw0 + WM <= V;   // no vocab row of this wave is past V

  int ytok[D::TN];                // target of each of this lane's tokens (-1: none)
#pragma unroll
  for (int j = 0; j < D::TN; ++j) {
    const int m = t0 + wn * WN + j * 32 + (lane & 31);
    ytok[j] = m < Mtok ? head_target(ha, m) : -1;
  }

  f32x16 acc[D::TM][D::TN];
  dma_mainloop<BM, BN, WM, WN, K, NST, BK>(wte, K, act, K, K, V, Mtok, v0, t0, stages, acc);

  // (stage k by selects: indexing the pointer array with a run-time value
  // would place the array itself in memory)
  auto stage = [&](int k) {
    if constexpr (NST == 2) return k == 0 ? as_lds(s0) : as_lds(s1);
    else if constexpr (NST == 3) return k == 0 ? as_lds(s0) : k == 1 ? as_lds(s1) : as_lds(s2);
    else return k == 0 ? as_lds(s0) : k == 1 ? as_lds(s1) : k == 2 ? as_lds(s2) : as_lds(s3);
  };
  lds_char* const part = stage(P::PST) + P::POFF;
  lds_float* const red = reinterpret_cast<lds_float*>(part);                        // [NWM][BN][2]
  lds_int* const redi = reinterpret_cast<lds_int*>(part + D::NWM * BN * 2 * 4);   // [NWM][BN]
  lds_char* const wl = stage(wave / P::WPS) + (wave % P::WPS) * P::SW;
  const bool amax = ha.part_idx != nullptr;
  constexpr float LOG2E = 1.4426950408889634f;
#pragma unroll
  for (int j = 0; j < D::TN; ++j) {
    const int tl = wn * WN + j * 32 + (lane & 31);
    const int m = t0 + tl;
    if (amax) {
      // greedy choice: the largest logit and its lowest vocab index.  Register
      // order i, r visits this lane's vocab rows in increasing order.
      float mx = -INFINITY;
      int mi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < D::TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = vw0 + i * 32 + acc_row(r, lane);
          if (v < V && acc[i][j][r] > mx) { mx = acc[i][j][r]; mi = v; }
        }
      const float v2 = __shfl_xor(mx, 32, 64);
      const int i2 = __shfl_xor(mi, 32, 64);
      if (better(v2, i2, mx, mi)) { mx = v2; mi = i2; }
      if (g == 0) { red[(wm * BN + tl) * 2] = mx; redi[wm * BN + tl] = mi; }
    } else {
      // softmax partials and target logit
      float mx = -INFINITY, sum = 0.f;
      if (full) {
#pragma unroll
        for (int i = 0; i < D::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mxl = mx * LOG2E;
#pragma unroll
        for (int i = 0; i < D::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) sum += fast_exp2(fmaf(acc[i][j][r], LOG2E, -mxl));
      } else {
#pragma unroll
        for (int i = 0; i < D::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vw0 + i * 32 + acc_row(r, lane) < V) mx = fmaxf(mx, acc[i][j][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (mx > -INFINITY) {
          const float mxl = mx * LOG2E;
#pragma unroll
          for (int i = 0; i < D::TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (vw0 + i * 32 + acc_row(r, lane) < V) sum += fast_exp2(fmaf(acc[i][j][r], LOG2E, -mxl));
        }
      }
      sum += __shfl_xor(sum, 32, 64);
      if (g == 0) { red[(wm * BN + tl) * 2] = mx; red[(wm * BN + tl) * 2 + 1] = sum; }
      const int y = ytok[j];
      if (m < Mtok && y >= vw0 && y < vw0 + WM) {
#pragma unroll
        for (int i = 0; i < D::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vw0 + i * 32 + acc_row(r, lane) == y) ha.tgt[m] = acc[i][j][r];
      }
    }
    if (ha.logits) {   // uniform: this column's bf16 logits through the wave's slot
      constexpr int NU = WM / 8;
#pragma unroll
      for (int i = 0; i < D::TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int vl = i * 32 + q * 8 + g * 4;
          lds_st8(wl + (lane & 31) * P::PITCH + vl * 2,
                  make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                             pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])));
        }
      // the slot is this wave's alone: LDS operations of one wave take effect
      // in issue order, so a wave-level fence orders the reads after the stores
      // (and the next column's stores after these reads)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      bf16* const L = reinterpret_cast<bf16*>(ha.logits);
#pragma unroll
      for (int u0 = 0; u0 < 32 * NU; u0 += 64) {
        const int u = u0 + lane, r = u / NU, k = u - r * NU;
        const int mr = t0 + wn * WN + j * 32 + r, v = vw0 + k * 8;
        const uint2 a = lds_ld8(wl + r * P::PITCH + k * 16);
        const uint2 b = lds_ld8(wl + r * P::PITCH + k * 16 + 8);
        if (mr >= Mtok || v >= V) continue;
        bf16* const p = L + (long long)mr * ha.ld_logits + v;
        if (v + 8 <= V) {
          if (ha.nt) {   // aligned rows: 16-byte pieces of whole lines, kept out of L2
            const u32x4_t w4 = {a.x, a.y, b.x, b.y};
            __builtin_nontemporal_store(w4, reinterpret_cast<u32x4_t*>(p));
          } else {
            const uint4 w4 = make_uint4(a.x, a.y, b.x, b.y);
            __builtin_memcpy(p, &w4, 16);
          }
        } else {
          for (int e = 0; v + e < V; ++e) {
            const uint32_t h = e < 2 ? a.x : e < 4 ? a.y : e < 6 ? b.x : b.y;
            p[e] = bf16(h >> (16 * (e & 1)));
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  __syncthreads();
  for (int tl = tid; tl < BN; tl += D::NT) {
    const int m = t0 + tl;
    if (m >= Mtok) continue;
    if (amax) {
      float mx = red[tl * 2];
      int mi = redi[tl];
#pragma unroll
      for (int w = 1; w < D::NWM; ++w)
        if (better(red[(w * BN + tl) * 2], redi[w * BN + tl], mx, mi)) {
          mx = red[(w * BN + tl) * 2];
          mi = redi[w * BN + tl];
        }
      ha.part_max[(long long)m * ha.ntiles + vt] = mx;
      ha.part_idx[(long long)m * ha.ntiles + vt] = mi;
      continue;
    }
    float M_ = red[tl * 2];
#pragma unroll
    for (int w = 1; w < D::NWM; ++w) M_ = fmaxf(M_, red[(w * BN + tl) * 2]);
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < D::NWM; ++w) {
      const float mw = red[(w * BN + tl) * 2];
      if (mw > -INFINITY) S += red[(w * BN + tl) * 2 + 1] * fast_exp2((mw - M_) * LOG2E);
    }
    ha.part_max[(long long)m * ha.ntiles + vt] = M_;
    ha.part_sum[(long long)m * ha.ntiles + vt] = S;
  }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool KTAIL>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
head_ce_kernel(const T* __restrict__ A, int lda, const T* __restrict__ W, int ldw, int M, int N, int K, HeadArgs ha) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  __shared__ __align__(16) T smem[G::SMEM_ELEMS];
  __shared__ float red[G::NWN][BM];
  __shared__ int redi[G::NWN][BM];
  __shared__ float rowmax[BM];
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, gridDim.x, num_m, num_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  f32x16 acc[G::TM][G::TN];
  gemm_mainloop<T, BM, BN, BK, WM, WN, KTAIL>(A, lda, W, ldw, M, N, K, m0, n0, smem, acc);
  const bool amax = ha.part_idx != nullptr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int ncol0 = n0 + wn * WN + (lane & 31);

  // logits store and target pick-up
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * WM + i * 32 + acc_row(r, lane);
      if (m >= M) continue;
      const int y = head_target(ha, m);
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int n = ncol0 + j * 32;
        if (n < N) {
          if (ha.logits) reinterpret_cast<T*>(ha.logits)[(long long)m * ha.ld_logits + n] = from_f32<T>(acc[i][j][r]);
          if (n == y) ha.tgt[m] = acc[i][j][r];
        }
      }
    }

  // row max (and, in argmax mode, its lowest column) over this block's columns
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float mx = -INFINITY;
      int mi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
        if (ncol0 + j * 32 < N && acc[i][j][r] > mx) { mx = acc[i][j][r]; mi = ncol0 + j * 32; }
      if (amax) {
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) {
          const float v2 = __shfl_xor(mx, o, 64);
          const int i2 = __shfl_xor(mi, o, 64);
          if (better(v2, i2, mx, mi)) { mx = v2; mi = i2; }
        }
      } else {
        mx = half_max(mx);
      }
      if ((lane & 31) == 0) {
        red[wn][wm * WM + i * 32 + acc_row(r, lane)] = mx;
        redi[wn][wm * WM + i * 32 + acc_row(r, lane)] = mi;
      }
    }
  __syncthreads();
  for (int rr = threadIdx.x; rr < BM; rr += G::NT) {
    float mx = red[0][rr];
    int mi = redi[0][rr];
#pragma unroll
    for (int w = 1; w < G::NWN; ++w)
      if (better(red[w][rr], redi[w][rr], mx, mi)) { mx = red[w][rr]; mi = redi[w][rr]; }
    rowmax[rr] = mx;
    const int m = m0 + rr;
    if (amax && m < M) {
      ha.part_max[(long long)m * ha.ntiles + nt] = mx;
      ha.part_idx[(long long)m * ha.ntiles + nt] = mi;
    }
  }
  if (amax) return;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * WM + i * 32 + acc_row(r, lane);
      const float mx = rowmax[rl];
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
        if (ncol0 + j * 32 < N) s += fast_exp2((acc[i][j][r] - mx) * 1.4426950408889634f);
      s = half_sum(s);
      if ((lane & 31) == 0) red[wn][rl] = s;
    }
  __syncthreads();
  for (int rr = threadIdx.x; rr < BM; rr += G::NT) {
    const int m = m0 + rr;
    if (m >= M) continue;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < G::NWN; ++w) s += red[w][rr];
    ha.part_max[(long long)m * ha.ntiles + nt] = rowmax[rr];
    ha.part_sum[(long long)m * ha.ntiles + nt] = s;
  }
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int BK, int WM, int WN, typename Epi>
static hipError_t run_gemm(const T* A, int lda, const T* W, int ldw, int M, int N, int K, const Epi& epi,
                           hipStream_t st) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (K % BK == 0)
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, false, Epi>), dim3(blocks), dim3(G::NT), 0, st, A, lda, W,
                       ldw, M, N, K, epi);
  else
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, true, Epi>), dim3(blocks), dim3(G::NT), 0, st, A, lda, W,
                       ldw, M, N, K, epi);
  return hipGetLastError();
}

// Tile choice.  Large bf16 products use 256x256 tiles (128x128 per wave); the
// fp32 path serves the small correctness configurations.
template <int BM, int BN, int WM, int WN, int K, int NST, int BK, typename Epi>
static hipError_t run_gemm_dma(const bf16* A, const bf16* W, int M, int N, const Epi& epi, hipStream_t st) {
  const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, K, NST, BK, Epi>), dim3(blocks),
                     dim3(DmaCfg<BM, BN, WM, WN, NST, BK>::NT), 0, st, A, K, W, K, M, N, K, 0LL, epi);
  return hipGetLastError();
}

// Run-time depth: S slices of Ks columns (grid.y), slice z's output zstride
// elements after slice z - 1's (fp32 epilogues with shift()).
template <int BM, int BN, int WM, int WN, int NST, int BK, typename Epi>
static hipError_t run_gemm_dma_rt(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int Ks, int S,
                                  long long zstride, const Epi& epi, hipStream_t st) {
  const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, 0, NST, BK, Epi>), dim3(blocks, S),
                     dim3(DmaCfg<BM, BN, WM, WN, NST, BK>::NT), 0, st, A, lda, W, ldw, M, N, Ks, zstride, epi);
  return hipGetLastError();
}

// 128 x 192 tiles make every block GEMM of the 124M
// model a whole number of rounds over 256 CUs at M = 8192 (N = 2304: 768
// tiles, 3072: 1024, 768: 256); 256 x 256 (8 waves of 64 x 128) otherwise.
template <int K, typename Epi>
static hipError_t run_gemm_dma_k(const bf16* A, const bf16* W, int M, int N, const Epi& epi, hipStream_t st) {
  // 128 x 192 also when 256 x 256 tiles could not fill the 256 CUs (a ragged
  // last column tile is cheaper than idle CUs, e.g. N = 1280)
  const long long blocks256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
  if (N % 192 == 0 || blocks256 < 256) {
    // 8 waves of 32 x 96; 64-deep stages.  Short K with an epilogue that keeps
    // little in registers across the main loop (kCompact): two stages (80 KB)
    // and two blocks per CU (128 registers per lane); otherwise three stages
    // and one block per CU.
    if (K <= 768 && Epi::kCompact) return run_gemm_dma<128, 192, 32, 96, K, 2, 64>(A, W, M, N, epi, st);
    return run_gemm_dma<128, 192, 32, 96, K, 3, 64>(A, W, M, N, epi, st);
  }
  return run_gemm_dma<256, 256, 64, 128, K, 4, 32>(A, W, M, N, epi, st);
}

// Block-tiled products (any M; K a multiple of 64 for the pipelined path,
// otherwise chunks past K read as zero)
template <typename Epi>
static hipError_t dispatch_gemm_tiled(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int K,
                                      const Epi& epi, hipStream_t st) {
  const long long tiles256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
  if (tiles256 >= 64 && lda == K && ldw == K) {
    if (K == 768) return run_gemm_dma_k<768>(A, W, M, N, epi, st);
    if (K == 2048) return run_gemm_dma_k<2048>(A, W, M, N, epi, st);   // SwiGLU down projection at F = 8/3 C
    if (K == 3072) return run_gemm_dma_k<3072>(A, W, M, N, epi, st);
  }
  if (tiles256 >= 192) return run_gemm<bf16, 256, 256, 64, 128, 64>(A, lda, W, ldw, M, N, K, epi, st);
  if ((long long)M * N >= (long long)256 * 1024 * 16)
    return run_gemm<bf16, 128, 128, 64, 64, 64>(A, lda, W, ldw, M, N, K, epi, st);
  return run_gemm<bf16, 64, 64, 64, 32, 32>(A, lda, W, ldw, M, N, K, epi, st);
}

template <typename Epi>
static hipError_t dispatch_gemm(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int K, const Epi& epi,
                                const SkinnyWs* sk, hipStream_t st) {
  if (M <= 64 && lda % 8 == 0 && ldw % 8 == 0) return run_skinny(A, lda, W, ldw, M, N, K, epi, sk, st);
  return dispatch_gemm_tiled(A, lda, W, ldw, M, N, K, epi, st);
}

template <typename Epi>
static hipError_t dispatch_gemm_tiled(const float* A, int lda, const float* W, int ldw, int M, int N, int K,
                                      const Epi& epi, hipStream_t st) {
  return run_gemm<float, 64, 64, 32, 32, 32>(A, lda, W, ldw, M, N, K, epi, st);
}

template <typename Epi>
static hipError_t dispatch_gemm(const float* A, int lda, const float* W, int ldw, int M, int N, int K, const Epi& epi,
                                const SkinnyWs*, hipStream_t st) {
  return run_gemm<float, 64, 64, 32, 32, 32>(A, lda, W, ldw, M, N, K, epi, st);
}

template <typename T>
static hipError_t linear_t(const void* A, int lda, const void* W, int ldw, const void* bias, int M, int N, int K,
                           void* out, int ldo, int act, int out_f32, const SkinnyWs* sk, hipStream_t st) {
  if (act == 3) return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K, EpiSwiGLU<T>{(T*)out, ldo}, sk, st);
  if (act == 2 && !out_f32) return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K,
                                                 EpiAct<T, 2, false>{(const T*)bias, out, ldo}, sk, st);
  if (act == 2) return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K,
                                     EpiAct<T, 2, true>{(const T*)bias, out, ldo}, sk, st);
  if (act == 1 && !out_f32) return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K,
                                                 EpiAct<T, 1, false>{(const T*)bias, out, ldo}, sk, st);
  if (act == 1) return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K,
                                     EpiAct<T, 1, true>{(const T*)bias, out, ldo}, sk, st);
  if (!out_f32) return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K,
                                     EpiAct<T, 0, false>{(const T*)bias, out, ldo}, sk, st);
  return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K, EpiAct<T, 0, true>{(const T*)bias, out, ldo}, sk,
                       st);
}

hipError_t launch_linear(int dtype, const void* A, int lda, const void* W, int ldw, const void* bias, int M, int N,
                         int K, void* out, int ldo, int act, int out_f32, hipStream_t st, const SkinnyWs* sk) {
  if (dtype == 0) return linear_t<float>(A, lda, W, ldw, bias, M, N, K, out, ldo, act, out_f32, sk, st);
  return linear_t<bf16>(A, lda, W, ldw, bias, M, N, K, out, ldo, act, out_f32, sk, st);
}

template <typename T>
static hipError_t resid_t(const void* A, int lda, const void* W, int ldw, const void* bias, int M, int N, int K,
                          float* x, int ldx, const SkinnyWs* sk, hipStream_t st) {
  EpiResid<T> e{(const T*)bias, x, ldx};
  return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K, e, sk, st);
}

hipError_t launch_linear_resid(int dtype, const void* A, int lda, const void* W, int ldw, const void* bias, int M,
                               int N, int K, float* x, int ldx, hipStream_t st, const SkinnyWs* sk) {
  if (dtype == 0) return resid_t<float>(A, lda, W, ldw, bias, M, N, K, x, ldx, sk, st);
  return resid_t<bf16>(A, lda, W, ldw, bias, M, N, K, x, ldx, sk, st);
}

template <typename T>
static hipError_t qkv_t(const QKVArgs& a, const SkinnyWs* sk, hipStream_t st) {
  EpiQKV<T> e{(const T*)a.bias, a.C, a.H, a.D, a.T_seq, 1.0f / (float)a.T_seq, (T*)a.q, a.q_bh, (T*)a.k, a.k_bh,
              (T*)a.v, a.v_bh, a.pos, a.Tk, a.Hkv, a.rope};
  return dispatch_gemm((const T*)a.A, a.C, (const T*)a.W, a.C, a.M, a.C + 2 * a.Hkv * a.D, a.C, e, sk, st);
}

hipError_t launch_qkv(int dtype, const QKVArgs& a, hipStream_t st, const SkinnyWs* sk) {
  if (dtype == 0) return qkv_t<float>(a, sk, st);
  return qkv_t<bf16>(a, sk, st);
}

// Batched products for the attention backward: grid.y runs over z = b * H + h,
// and every operand and the fp32 output start at b * (stride_b) + h * (stride_h)
// (BatchStrides).

template <typename T, int BM, int BN, int BK, int WM, int WN, bool KTAIL, typename Epi>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_batched_kernel(const T* __restrict__ A, int lda, const T* __restrict__ W, int ldw, int M, int N, int K,
                    Epi epi_z, BatchStrides bs, int causal) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  __shared__ __align__(16) T smem[G::SMEM_ELEMS];
  const int z = blockIdx.y, b = z / bs.H, h = z - b * bs.H;
  A += b * bs.ab + h * bs.ah;
  W += b * bs.wb + h * bs.wh;
  const Epi epi = epi_z.at(b, h, bs);   // this product's outputs
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, gridDim.x, num_m, num_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  // causal 1 (score products): a tile wholly above the diagonal (every column
  // n > every row m) is never read, so it is not computed (uniform exit).
  // causal 2 / 3 (contractions against a causal [rows][keys] operand, BM a
  // multiple of BK): row m's terms vanish for k < m (2) or k > m (3), so the
  // tile contracts only over [m0, K) or [0, min(K, m0 + BM)).
  if (causal == 1 && n0 > m0 + BM - 1) return;
  const int k0 = causal == 2 ? m0 : 0, k1 = causal == 3 ? min(K, m0 + BM) : K;
  const int wave = threadIdx.x >> 6;
  const int mb = m0 + (wave / G::NWN) * WM, nb = n0 + (wave % G::NWN) * WN;
  float2 pre[G::TM][G::TN][8];
  typename Epi::Col colv[G::TN];
  preload_pairs<G::TM, G::TN>(pre, colv, mb, nb, M, N, epi);
  f32x16 acc[G::TM][G::TN];
  if constexpr (IsRaw<Epi>::value) {
    // the epilogue's own inputs are requested before the main loop, so their
    // latency overlaps the operand loads
    const auto rp = epi.template raw_preload<G::TM, G::TN>(mb, nb);
    gemm_mainloop<T, BM, BN, BK, WM, WN, KTAIL>(A + k0, lda, W + k0, ldw, M, N, k1 - k0, m0, n0, smem, acc);
    constexpr int WLB = (int)(G::SMEM_ELEMS * sizeof(T) / (G::NWM * G::NWN)) & ~15;
    __syncthreads();   // the tiles of the last K step are read: the LDS is free
    epi.template raw<G::TM, G::TN, WLB>(acc, mb, nb, M, N, as_lds(smem) + wave * WLB, rp);
  } else {
    gemm_mainloop<T, BM, BN, BK, WM, WN, KTAIL>(A + k0, lda, W + k0, ldw, M, N, k1 - k0, m0, n0, smem, acc);
    epilogue_pairs<G::TM, G::TN>(acc, pre, colv, mb, nb, M, N, epi);
  }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, typename Epi>
static hipError_t run_batched(const T* A, int lda, const T* W, int ldw, int M, int N, int K, const Epi& epi,
                              const BatchStrides& bs, int Z, int causal, hipStream_t st) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  const dim3 grid(((M + BM - 1) / BM) * ((N + BN - 1) / BN), Z);
  if (K % BK == 0)
    hipLaunchKernelGGL((gemm_batched_kernel<T, BM, BN, BK, WM, WN, false, Epi>), grid, dim3(G::NT), 0, st, A, lda, W,
                       ldw, M, N, K, epi, bs, causal);
  else
    hipLaunchKernelGGL((gemm_batched_kernel<T, BM, BN, BK, WM, WN, true, Epi>), grid, dim3(G::NT), 0, st, A, lda, W,
                       ldw, M, N, K, epi, bs, causal);
  return hipGetLastError();
}

// out_z [M, N] fp32 = A_z [M, K] . W_z [N, K]^T for z < Z (K a multiple of 8, or of 4 in fp32).
// causal 1: tiles wholly above the diagonal are left unwritten; 2 / 3: A_z[m, k]
// is zero for k < m (2) or k > m (3) and K is a multiple of 64, so each row
// tile contracts over its nonzero range only.
hipError_t launch_gemm_batched(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                               float* out, int ldo, const BatchStrides& bs, int Z, hipStream_t st, int causal) {
  const EpiF32<false> epi{out, ldo};
  if (dtype == 0)
    return run_batched<float, 64, 64, 32, 32, 32>((const float*)A, lda, (const float*)W, ldw, M, N, K, epi, bs, Z,
                                                  causal, st);
  if (N >= 128)
    return run_batched<bf16, 128, 128, 64, 64, 64>((const bf16*)A, lda, (const bf16*)W, ldw, M, N, K, epi, bs, Z,
                                                   causal, st);
  return run_batched<bf16, 64, 64, 64, 32, 32>((const bf16*)A, lda, (const bf16*)W, ldw, M, N, K, epi, bs, Z, causal,
                                               st);
}

// Score-side products of the attention backward (bf16), one per (b, h):
// MODE 0: P = exp2(sc q.k - lse2[m]) (the causal softmax, the row's log-sum-exp
//         in log2 units from the forward pass), from acc = q.k;
// MODE 1: dS = P (acc - Dv[m]) sc, from acc = dO.u, P read from P^T.
// Entries with n > m, or past the Tn rows, are written as zeros, except that
// tiles wholly above the diagonal (n0 > m0 + BM - 1) are skipped and left
// unwritten: out [m][n] (skipped when null) and outT [n][m] are [Tn][ld]
// (ld = Tn rounded up to 64; the tile grid covers every column below ld).
// Their readers never touch the skipped tiles: the dS product reads P^T only
// inside the tiles it computes itself (the same grid and skip), and the
// contractions dU = P^T dO, dK = dS^T Q (over [r0, ld)) and dQ = dS K (over
// [0, r0 + 64)), with r0 the 64-aligned start of their row tile, stay within
// the computed 128 x 128 (or 64 x 64) tiles.  Both copies are gathered in LDS per wave (the transposed one
// in 8-byte chunks XOR-swizzled by row, as for the head's loss gradient; the
// row-major one in column pairs, its 16-byte units XOR-swizzled by row) and
// leave as 16-byte row stores.
template <typename T, int MODE>
struct EpiAttnB {
  static constexpr bool kPreload = false;
  static constexpr bool kCompact = true;
  static constexpr bool kRaw = true;
  typedef int Row;
  typedef int Col;
  typedef int ColX;
  const float* rowv;   // MODE 0: lse2 [Tn]; MODE 1: Dv [Tn] (dO . O of each row)
  const T* PT;         // MODE 1: P^T [Tn][ld]
  T* out;              // may be null (only outT is written)
  T* outT;
  int ld, Tn;
  long long zs;        // elements between consecutive products' [Tn][ld] matrices
  float sc;            // MODE 0: log2(e) / sqrt(D); MODE 1: 1 / sqrt(D)
  __device__ __forceinline__ Row row(int) const { return 0; }
  __device__ __forceinline__ Col col(int, bool) const { return 0; }
  __device__ __forceinline__ ColX colx(int, const Col& c) const { return c; }
  __device__ __forceinline__ float2 preload(int, int, bool) const { return make_float2(0.f, 0.f); }
  __device__ __forceinline__ EpiAttnB at(int b, int h, const BatchStrides& bs) const {
    const long long z = (long long)b * bs.H + h;
    EpiAttnB e = *this;
    e.rowv += z * Tn;
    if (MODE == 1) e.PT += z * zs;
    if (out != nullptr) e.out += z * zs;
    e.outT += z * zs;
    return e;
  }

  // per lane: the row values of its 4 TM rows-quads and, for MODE 1, the
  // P^T quad P^T[n][m0 .. m0 + 3] of each (row quad, column tile)
  template <int TM, int TN>
  struct Pre {
    float r[TM][4][4];
    uint2 p[TM][4][TN];
  };
  template <int TM, int TN>
  __device__ __forceinline__ Pre<TM, TN> raw_preload(int mbase, int nbase) const {
    Pre<TM, TN> R;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m0 = mbase + i * 32 + q * 8 + (lane >> 5) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) R.r[i][q][e] = m0 + e < Tn ? rowv[m0 + e] : 0.f;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = nbase + j * 32 + (lane & 31);
          R.p[i][q][j] = make_uint2(0u, 0u);
          if (MODE == 1 && n < Tn && m0 < ld) R.p[i][q][j] = *reinterpret_cast<const uint2*>(PT + (long long)n * ld + m0);
        }
      }
    return R;
  }

  template <int TM, int TN, int WLB>
  __device__ __forceinline__ void raw(const f32x16 (&acc)[TM][TN], int mbase, int nbase, int, int, lds_char* wl,
                                      const Pre<TM, TN>& R) const {
    static_assert(sizeof(T) == 2, "bf16 only");
    constexpr int WM = TM * 32, WN = TN * 32;
    constexpr int RB = WM * 2, NC = WM / 4, NU = WM / 8;   // staged row bytes, 8-byte chunks, 16-byte units
    static_assert(WLB >= 2 * WN * RB, "the wave's LDS share must hold both copies of its tile");
    constexpr int RBR = WN * 2, NUR = WN / 8;   // row-major staged row bytes, 16-byte units
    lds_char* wr = wl + WN * RB;                // the row-major copy
    const int lane = threadIdx.x & 63;
    const bool odd = lane & 1;
    const bool rowmajor = out != nullptr;   // uniform
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m0 = mbase + i * 32 + q * 8 + (lane >> 5) * 4;   // rows m0 .. m0 + 3
        const float (&r4)[4] = R.r[i][q];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = nbase + j * 32 + (lane & 31);
          float v[4];
          if constexpr (MODE == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = (m0 + e < Tn && n <= m0 + e) ? fast_exp2(fmaf(acc[i][j][4 * q + e], sc, -r4[e])) : 0.f;
          } else {
            // P^T[n][m0 .. m0 + 3] (zero past the diagonal and in the pads)
            const uint2 pw = R.p[i][q][j];
            const float p4[4] = {__uint_as_float(pw.x << 16), __uint_as_float(pw.x & 0xffff0000u),
                                 __uint_as_float(pw.y << 16), __uint_as_float(pw.y & 0xffff0000u)};
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = p4[e] * (acc[i][j][4 * q + e] - r4[e]) * sc;
          }
          // row-major pairs (lanes 2k, 2k + 1 hold columns n, n + 1)
          const int ne = n & ~1;
          if (rowmajor) {
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const float recv = xor1(odd ? v[e] : v[e + 1]);
              const int ml = m0 + e + (odd ? 1 : 0) - mbase, nl = ne - nbase;
              const float a = odd ? recv : v[e], b = odd ? v[e + 1] : recv;
              const int u = (nl >> 3) ^ ((ml >> 2) & (NUR - 1));
              lds_st4(wr + ml * RBR + u * 16 + (nl & 7) * 2, pack_bf16x2(a, b));
            }
          }
          const int r = j * 32 + (lane & 31), c = i * 8 + q * 2 + (lane >> 5);
          lds_st8(wl + r * RB + ((c ^ ((r >> 1) & (NC - 1))) << 3),
                  make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
        }
      }
    __syncthreads();   // every wave has written its tile (each reads back only its own)
#pragma unroll
    for (int it = 0; it < WN * NU / 64; ++it) {
      const int r = it * (64 / NU) + lane / NU, k = lane % NU, f = (r >> 1) & (NC - 1);
      uint4 w = lds_ld16(wl + r * RB + ((k ^ (f >> 1)) << 4));
      if (f & 1) w = make_uint4(w.z, w.w, w.x, w.y);
      const int n = nbase + r, m = mbase + k * 8;
      if (n < Tn && m < ld) *reinterpret_cast<uint4*>(outT + (long long)n * ld + m) = w;   // (m + 8 <= ld)
    }
    if (rowmajor) {
#pragma unroll
      for (int it = 0; it < WM * NUR / 64; ++it) {
        const int r = it * (64 / NUR) + lane / NUR, k = lane % NUR;
        const uint4 w = lds_ld16(wr + r * RBR + ((k ^ ((r >> 2) & (NUR - 1))) << 4));
        const int m = mbase + r, n = nbase + k * 8;
        if (m < Tn && n < ld) *reinterpret_cast<uint4*>(out + (long long)m * ld + n) = w;   // (n + 8 <= ld)
      }
    }
  }
};

// One launch over the Z = B H products of the attention backward's score side
// (q . k for MODE 0, dO . u for MODE 1; K = D), see EpiAttnB.
hipError_t launch_attn_scores_bwd(int mode, const void* A, int lda, const void* W, int ldw, int Tn, int D,
                                  const BatchStrides& bs, int Z, const float* rowv, const void* PT, void* out,
                                  void* outT, int ld, float sc, hipStream_t st) {
  if (ld % 64 != 0 || ld < Tn || Tn <= 0) return hipErrorInvalidValue;
  const long long zs = (long long)Tn * ld;
  // The contractions that read these tiles (launch_gemm_batched with N = D)
  // take 128-row tiles when D >= 128, and a causal row tile of 128 reads the
  // whole 128 x 128 square at its diagonal: the score tiles must then be at
  // least that large, or the skipped (never written) 64 x 64 tile above the
  // diagonal inside that square would be read.
  const bool big = Tn >= 128 || D >= 128;
  if (mode == 0) {
    const EpiAttnB<bf16, 0> e{rowv, nullptr, (bf16*)out, (bf16*)outT, ld, Tn, zs, sc};
    if (big)
      return run_batched<bf16, 128, 128, 64, 64, 64>((const bf16*)A, lda, (const bf16*)W, ldw, Tn, Tn, D, e, bs, Z, 1,
                                                     st);
    return run_batched<bf16, 64, 64, 64, 32, 32>((const bf16*)A, lda, (const bf16*)W, ldw, Tn, Tn, D, e, bs, Z, 1, st);
  }
  const EpiAttnB<bf16, 1> e{rowv, (const bf16*)PT, (bf16*)out, (bf16*)outT, ld, Tn, zs, sc};
  if (big)
    return run_batched<bf16, 128, 128, 64, 64, 64>((const bf16*)A, lda, (const bf16*)W, ldw, Tn, Tn, D, e, bs, Z, 1,
                                                   st);
  return run_batched<bf16, 64, 64, 64, 32, 32>((const bf16*)A, lda, (const bf16*)W, ldw, Tn, Tn, D, e, bs, Z, 1, st);
}

// Loss gradient of the logits A W^T ([M, C] x [V, C]^T) into dz [M, V] (ld).
hipError_t launch_head_dz(int dtype, const void* A, const void* W, int M, int V, int C, const float* lse,
                          const int32_t* y, const float* inv, void* dz, long long ld, void* dzT, long long ldT,
                          hipStream_t st) {
  if (dtype == 0)
    return dispatch_gemm_tiled((const float*)A, C, (const float*)W, C, M, V, C,
                               EpiDz<float>{lse, y, inv, (float*)dz, ld, (float*)dzT, ldT}, st);
  const EpiDz<bf16> e{lse, y, inv, (bf16*)dz, ld, (bf16*)dzT, ldT};
  // at C = 768: 128 x 192 tiles in two stages, two blocks per CU, so one
  // block's store-heavy epilogue overlaps the other's main loop
  if (C == 768 && M >= 1024 && (long long)((M + 127) / 128) * ((V + 191) / 192) >= 512)
    return run_gemm_dma<128, 192, 32, 96, 768, 2, 64>((const bf16*)A, (const bf16*)W, M, V, e, st);
  return dispatch_gemm_tiled((const bf16*)A, C, (const bf16*)W, C, M, V, C, e, st);
}

// The pipelined path at a run-time depth takes bf16 operands whose rows are
// 16-byte aligned, a depth that is a multiple of 32 and at least 256 (the
// 128 x 192 tiles need a multiple of 64; f32out_rt takes 256 x 256 tiles
// otherwise), and row strides small enough that 256 rows stay below 4 GB of
// buffer range.
static bool f32_rt_ok(const void* A, int lda, const void* W, int ldw, int Ks) {
  return Ks % 32 == 0 && Ks >= 256 && lda % 8 == 0 && ldw % 8 == 0 && ((uintptr_t)A & 15) == 0 &&
         ((uintptr_t)W & 15) == 0 && (size_t)256 * lda * 2 < (1ull << 32) && (size_t)256 * ldw * 2 < (1ull << 32);
}

// S slices (S >= 1) of Ks columns; slice z writes out + z zstride, [M, ldo].
// 128 x 192 tiles in two stages when they give at least 512 blocks (two per
// CU); else 256 x 256 tiles (four 32-deep stages; twice the flops per loaded
// byte of 128 x 192) once they fill three quarters of the CUs, else 128 x 192
// in three 64-deep stages (Ks a multiple of 64).
template <bool ACC>
static hipError_t f32out_rt(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int Ks, int S, float* out,
                            int ldo, long long zstride, hipStream_t st) {
  const EpiF32<ACC> epi{out, ldo};
  const long long blocks256 = (long long)((M + 255) / 256) * ((N + 255) / 256) * S;
  const long long blocks192 = (long long)((M + 127) / 128) * ((N + 191) / 192) * S;
  // with at least two blocks per CU: 128 x 192 tiles in two stages (80 KB of
  // LDS), so one block's epilogue and load waits overlap the other's products
  if (N % 192 == 0 && Ks % 64 == 0 && blocks192 >= 512)
    return run_gemm_dma_rt<128, 192, 32, 96, 2, 64>(A, lda, W, ldw, M, N, Ks, S, zstride, epi, st);
  if (blocks256 >= 192 || Ks % 64 != 0)
    return run_gemm_dma_rt<256, 256, 64, 128, 4, 32>(A, lda, W, ldw, M, N, Ks, S, zstride, epi, st);
  return run_gemm_dma_rt<128, 192, 32, 96, 3, 64>(A, lda, W, ldw, M, N, Ks, S, zstride, epi, st);
}

// out [M, N] fp32 (=, or += with accumulate) A [M, K] . W [N, K]^T
hipError_t launch_gemm_f32out(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                              float* out, int ldo, int accumulate, hipStream_t st) {
  if (dtype == 0) {
    if (accumulate)
      return dispatch_gemm_tiled((const float*)A, lda, (const float*)W, ldw, M, N, K, EpiF32<true>{out, ldo}, st);
    return dispatch_gemm_tiled((const float*)A, lda, (const float*)W, ldw, M, N, K, EpiF32<false>{out, ldo}, st);
  }
  // depths without a compile-time main loop (the head's vocabulary and token
  // contractions, 3C) take the run-time one when the product is large
  const long long tiles256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
  const bool templ = (K == 768 || K == 2048 || K == 3072) && lda == K && ldw == K && tiles256 >= 64;
  if (!templ && (long long)M * N >= (long long)256 * 1024 * 16 && ldo % 2 == 0 && f32_rt_ok(A, lda, W, ldw, K)) {
    if (accumulate) return f32out_rt<true>((const bf16*)A, lda, (const bf16*)W, ldw, M, N, K, 1, out, ldo, 0, st);
    return f32out_rt<false>((const bf16*)A, lda, (const bf16*)W, ldw, M, N, K, 1, out, ldo, 0, st);
  }
  if (accumulate)
    return dispatch_gemm_tiled((const bf16*)A, lda, (const bf16*)W, ldw, M, N, K, EpiF32<true>{out, ldo}, st);
  return dispatch_gemm_tiled((const bf16*)A, lda, (const bf16*)W, ldw, M, N, K, EpiF32<false>{out, ldo}, st);
}

// Split-K partials: out + z zstride [M, N] = A[:, z Ks, +Ks) . W[:, z Ks, +Ks)^T
// for z < S (summed afterwards in a fixed order by launch_add_partials).
hipError_t launch_gemm_f32_splitk(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int Ks,
                                  int S, float* out, long long zstride, hipStream_t st) {
  if (dtype != 0 && N % 2 == 0 && f32_rt_ok(A, lda, W, ldw, Ks))
    return f32out_rt<false>((const bf16*)A, lda, (const bf16*)W, ldw, M, N, Ks, S, out, N, zstride, st);
  return launch_gemm_batched(dtype, A, lda, W, ldw, M, N, Ks, out, N, BatchStrides{Ks, 0, Ks, 0, zstride, 0, 1}, S,
                             st);
}

// bf16 heads for C = 768: 256 (vocab) x 256 (token) blocks of eight 128 x 64
// waves for many tokens (128 flops per byte brought into LDS), 192 x 128
// blocks of four 96 x 64 waves for the rest, except a decode step's argmax
// over at most 64 tokens: there the head is a stream of the token table, and
// 256 x 64 blocks of four 64 x 64 waves in three stages keep 120 KB of it in
// flight per CU with one block per CU (197 blocks for V = 50257: one round).
constexpr int HEAD_BIG_MIN_TOKENS = 2048;
static bool head_big(int dtype, int M, int C, bool argmax) {
  return dtype != 0 && C == 768 && !argmax && M >= HEAD_BIG_MIN_TOKENS;
}
static bool head_stream(int dtype, int M, int C, bool argmax) { return dtype != 0 && C == 768 && argmax && M <= 64; }

int head_ntiles(int dtype, int M, int V, int C, bool argmax) {
  const int bn = dtype == 0 ? 64
                            : (C == 768 ? (head_big(dtype, M, C, argmax) || head_stream(dtype, M, C, argmax) ? 256 : 192)
                                        : 256);
  return (V + bn - 1) / bn;
}

template <int BM, int BN, int WM, int WN, int NST, int BK>
static hipError_t run_head_dma(const bf16* wte, const bf16* A, int V, int M, HeadArgs ha, hipStream_t st) {
  typedef DmaCfg<BM, BN, WM, WN, NST, BK> HD;
  ha.ntiles = (V + BM - 1) / BM;
  const int blocks = ((M + BN - 1) / BN) * ha.ntiles;
  hipLaunchKernelGGL((head_ce_dma_kernel<768, BM, BN, WM, WN, NST, BK>), dim3(blocks), dim3(HD::NT), 0, st, wte, A,
                     V, M, ha);
  return hipGetLastError();
}

hipError_t launch_head_ce(int dtype, const void* A, const void* wte, int M, int V, int C, void* logits,
                          long long ld_logits, float* part_max, float* part_sum, float* tgt, int32_t* part_idx,
                          const int32_t* targets, const int32_t* idx, int T_seq, hipStream_t st) {
  HeadArgs ha{logits, ld_logits, part_max, part_sum, tgt, part_idx, 0, targets, idx, T_seq, 0};
  // rows on 128-byte lines (bf16: a stride of 64 elements, an aligned base):
  // the tiles' row pieces are whole lines, written past L2 so that they do
  // not evict the operand tiles the other CUs' main loops re-read
  ha.nt = dtype != 0 && logits && ld_logits % 64 == 0 && reinterpret_cast<uintptr_t>(logits) % 128 == 0;
  if (dtype == 0) {
    constexpr int BM = 64, BN = 64;
    ha.ntiles = (V + BN - 1) / BN;
    const int blocks = ((M + BM - 1) / BM) * ha.ntiles;
    if (C % 32 == 0)
      hipLaunchKernelGGL((head_ce_kernel<float, BM, BN, 32, 32, 32, false>), dim3(blocks),
                         dim3(GemmCfg<float, BM, BN, 32, 32, 32>::NT), 0, st, (const float*)A, C, (const float*)wte, C,
                         M, V, C, ha);
    else
      hipLaunchKernelGGL((head_ce_kernel<float, BM, BN, 32, 32, 32, true>), dim3(blocks),
                         dim3(GemmCfg<float, BM, BN, 32, 32, 32>::NT), 0, st, (const float*)A, C, (const float*)wte, C,
                         M, V, C, ha);
  } else {
    constexpr int BM = 256, BN = 256;
    ha.ntiles = (V + BN - 1) / BN;
    const int blocks = ((M + BM - 1) / BM) * ha.ntiles;
    if (C == 768) {
      if (head_big(dtype, M, C, part_idx != nullptr))
        return run_head_dma<256, 256, 128, 64, 2, 64>((const bf16*)wte, (const bf16*)A, V, M, ha, st);
      if (head_stream(dtype, M, C, part_idx != nullptr))
        return run_head_dma<256, 64, 64, 64, 3, 64>((const bf16*)wte, (const bf16*)A, V, M, ha, st);
      return run_head_dma<192, 128, 96, 64, 2, 64>((const bf16*)wte, (const bf16*)A, V, M, ha, st);
    }
    if (C % 64 == 0)
      hipLaunchKernelGGL((head_ce_kernel<bf16, BM, BN, 64, 128, 64, false>), dim3(blocks),
                         dim3(GemmCfg<bf16, BM, BN, 64, 128, 64>::NT), 0, st, (const bf16*)A, C, (const bf16*)wte, C,
                         M, V, C, ha);
    else
      hipLaunchKernelGGL((head_ce_kernel<bf16, BM, BN, 64, 128, 64, true>), dim3(blocks),
                         dim3(GemmCfg<bf16, BM, BN, 64, 128, 64>::NT), 0, st, (const bf16*)A, C, (const bf16*)wte, C,
                         M, V, C, ha);
  }
  return hipGetLastError();
}

}  // namespace gptmi
