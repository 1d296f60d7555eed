// Cross-entropy reduction over the head's per-tile partials.
//
// For each token row m:  loss = logsumexp(z[m,:]) - z[m, y[m]]  ("预训练一个
// Mini GPT" 第6步 cross_entropy_loss: log-softmax with the maximum removed,
// gather the target), where logsumexp is recombined from the per-N-tile
// (max, sum exp) pairs:  M = max_t m_t,  S = sum_t s_t exp(m_t - M).  The
// mean runs over the positions that have a target ("第 25 章 从小 GPT 到
// GPT-2" §25.7: average over the B*T predicted positions).  Both levels of
// the mean use a fixed summation order, so results are bit-reproducible.
#include "common.h"
#include "kernels.h"

namespace gptmi {

constexpr int CE_ROWS = 4;   // rows per block, one per wave

__device__ __forceinline__ int target_of(const int32_t* targets, const int32_t* idx, int m, int T_seq) {
  if (targets) return targets[m];
  return ((m % T_seq) < T_seq - 1) ? idx[m + 1] : -1;
}

// One wave per token row.  With NPL > 0 the row's (max, sum) pairs sit in
// registers (NPL per lane, ntiles <= 64 NPL), all loaded at once; NPL = 0
// walks any number of tiles in two passes.
template <int NPL>
__global__ void __launch_bounds__(256) ce_rows_kernel(int M, int ntiles, const float* __restrict__ part_max,
                                                      const float* __restrict__ part_sum, const float* __restrict__ tgt,
                                                      const int32_t* targets, const int32_t* idx, int T_seq, int V,
                                                      float* __restrict__ token_loss, double* __restrict__ block_sums) {
  __shared__ double wsum[CE_ROWS][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = blockIdx.x * CE_ROWS + wave;
  double s_loss = 0.0, s_cnt = 0.0;
  if (m < M) {
    const float* pm = part_max + (long long)m * ntiles;
    const float* ps = part_sum + (long long)m * ntiles;
    const int y = target_of(targets, idx, m, T_seq);
    const float zt = tgt[m];
    float mx = -INFINITY, s = 0.f;
    if constexpr (NPL > 0) {
      float vm[NPL], vs[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int t = lane + 64 * i;
        vm[i] = t < ntiles ? pm[t] : -INFINITY;
        vs[i] = t < ntiles ? ps[t] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < NPL; ++i) mx = fmaxf(mx, vm[i]);
      mx = wave_max(mx);
#pragma unroll
      for (int i = 0; i < NPL; ++i) s += vs[i] * fast_exp2((vm[i] - mx) * 1.4426950408889634f);
    } else {
      for (int t = lane; t < ntiles; t += 64) mx = fmaxf(mx, pm[t]);
      mx = wave_max(mx);
      for (int t = lane; t < ntiles; t += 64) s += ps[t] * fast_exp2((pm[t] - mx) * 1.4426950408889634f);
    }
    s = wave_sum(s);
    const bool valid = y >= 0 && y < V;
    const float loss = valid ? (mx + __logf(s)) - zt : 0.f;
    if (lane == 0 && token_loss) token_loss[m] = loss;
    s_loss = (double)loss;
    s_cnt = valid ? 1.0 : 0.0;
  }
  if (lane == 0) { wsum[wave][0] = s_loss; wsum[wave][1] = s_cnt; }
  __syncthreads();
  if (threadIdx.x == 0) {
    block_sums[2 * blockIdx.x] = ((wsum[0][0] + wsum[1][0]) + (wsum[2][0] + wsum[3][0]));
    block_sums[2 * blockIdx.x + 1] = ((wsum[0][1] + wsum[1][1]) + (wsum[2][1] + wsum[3][1]));
  }
}

__global__ void __launch_bounds__(256) ce_mean_kernel(int nblocks, const double* __restrict__ block_sums,
                                                      float* __restrict__ mean_loss) {
  __shared__ double sl[256], sc[256];
  double l = 0.0, c = 0.0;
  for (int i = threadIdx.x; i < nblocks; i += 256) { l += block_sums[2 * i]; c += block_sums[2 * i + 1]; }
  sl[threadIdx.x] = l;
  sc[threadIdx.x] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) { sl[threadIdx.x] += sl[threadIdx.x + o]; sc[threadIdx.x] += sc[threadIdx.x + o]; }
    __syncthreads();
  }
  if (threadIdx.x == 0) mean_loss[0] = sc[0] > 0.0 ? (float)(sl[0] / sc[0]) : __builtin_nanf("");
}

int ce_reduce_blocks(int M) { return (M + CE_ROWS - 1) / CE_ROWS; }

// Greedy next token per row: the largest logit over all vocab tiles, the
// lowest index among equal values ("GPT-1学习笔记" §6.1: greedy generation
// takes the argmax of the last position's logits).  One wave per row.
__global__ void __launch_bounds__(256) argmax_rows_kernel(int M, int ntiles, const float* __restrict__ part_max,
                                                          const int32_t* __restrict__ part_idx,
                                                          int32_t* __restrict__ next_tok, int32_t* pos, int set_pos) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m < M) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int t = lane; t < ntiles; t += 64) {
      const float v = part_max[(long long)m * ntiles + t];
      const int i = part_idx[(long long)m * ntiles + t];
      if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      if (v2 > bv || (v2 == bv && i2 < bi)) { bv = v2; bi = i2; }
    }
    if (lane == 0) next_tok[m] = bi;
  }
  if (pos && blockIdx.x == 0 && threadIdx.x == 0) *pos = set_pos >= 0 ? set_pos : *pos + 1;
}

hipError_t launch_argmax_reduce(int M, int ntiles, const float* part_max, const int32_t* part_idx, int32_t* next_tok,
                                int32_t* pos, int set_pos, hipStream_t st) {
  hipLaunchKernelGGL(argmax_rows_kernel, dim3((M + 3) / 4), dim3(256), 0, st, M, ntiles, part_max, part_idx, next_tok,
                     pos, set_pos);
  return hipGetLastError();
}

hipError_t launch_ce_reduce(int M, int ntiles, const float* part_max, const float* part_sum, const float* tgt,
                            const int32_t* targets, const int32_t* idx, int T_seq, int V, float* token_loss,
                            double* block_sums, float* mean_loss, hipStream_t st) {
  const int nb = ce_reduce_blocks(M);
  if (ntiles <= 256)
    hipLaunchKernelGGL(ce_rows_kernel<4>, dim3(nb), dim3(256), 0, st, M, ntiles, part_max, part_sum, tgt, targets, idx,
                       T_seq, V, token_loss, block_sums);
  else if (ntiles <= 512)
    hipLaunchKernelGGL(ce_rows_kernel<8>, dim3(nb), dim3(256), 0, st, M, ntiles, part_max, part_sum, tgt, targets, idx,
                       T_seq, V, token_loss, block_sums);
  else
    hipLaunchKernelGGL(ce_rows_kernel<0>, dim3(nb), dim3(256), 0, st, M, ntiles, part_max, part_sum, tgt, targets, idx,
                       T_seq, V, token_loss, block_sums);
  if (mean_loss) hipLaunchKernelGGL(ce_mean_kernel, dim3(1), dim3(256), 0, st, nb, block_sums, mean_loss);
  return hipGetLastError();
}

}  // namespace gptmi
