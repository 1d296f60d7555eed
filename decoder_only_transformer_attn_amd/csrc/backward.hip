// Backward of the next-token loss through the head, the final LayerNorm and
// the embeddings: the element-wise and reduction kernels around the two
// gradient products (which run on the GEMM kernels).
//
//   "预训练一个 Mini GPT（1.24 亿参数）" 训练循环: a training step
//   back-propagates the cross-entropy of the logits to every parameter;
//   "第 25 章 从小 GPT 到 GPT-2" §25.4: the tied token table's gradient sums
//   its two uses (output head and input lookup).
//
// Loss gradient of a row with a target y: (softmax(z) - onehot(y)) / n_valid,
// n_valid = number of rows with a target (the loss is their mean).  LayerNorm
// y = g * xh + b:  dx = (gd - mean(gd) - xh * mean(gd * xh)) / sqrt(var + eps)
// with gd = dy * g;  dg = sum_rows dy * xh;  db = sum_rows dy.
// Every sum runs in a fixed order, so results are bit-reproducible.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gptmi {

constexpr int BR_ROWS = 16;   // rows per block of the row kernel (4 per wave)

__device__ __forceinline__ int bwd_target(const int32_t* targets, const int32_t* idx, int m, int T_seq, int V) {
  const int y = targets ? targets[m] : (((m % T_seq) < T_seq - 1) ? idx[m + 1] : -1);
  return (y >= 0 && y < V) ? y : -1;
}

// Per row: log-sum-exp of the logits from the head's per-tile (max, sum exp)
// partials, and the target (-1: none).
__global__ void __launch_bounds__(256) bwd_rows_kernel(int M, int ntiles, const float* __restrict__ part_max,
                                                       const float* __restrict__ part_sum, const int32_t* targets,
                                                       const int32_t* idx, int T_seq, int V, float* __restrict__ lse,
                                                       int32_t* __restrict__ yv) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int rr = wave; rr < BR_ROWS; rr += 4) {
    const int m = blockIdx.x * BR_ROWS + rr;
    if (m >= M) break;
    const float* pm = part_max + (long long)m * ntiles;
    const float* ps = part_sum + (long long)m * ntiles;
    float mx = -INFINITY;
    for (int t = lane; t < ntiles; t += 64) mx = fmaxf(mx, pm[t]);
    mx = wave_max(mx);
    float s = 0.f;
    for (int t = lane; t < ntiles; t += 64) s += ps[t] * fast_exp2((pm[t] - mx) * 1.4426950408889634f);
    s = wave_sum(s);
    if (lane == 0) {
      lse[m] = mx + __logf(s);
      yv[m] = bwd_target(targets, idx, m, T_seq, V);
    }
  }
}

// inv[0] = 1 / (number of rows with a target), 0 when there is none.
__global__ void __launch_bounds__(1024) bwd_count_kernel(int M, const int32_t* __restrict__ yv, float* __restrict__ inv) {
  __shared__ int part[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int c = 0;
  for (int m = threadIdx.x; m < M; m += 1024) c += yv[m] >= 0 ? 1 : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if (lane == 0) part[wave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += part[w];
    inv[0] = t > 0 ? 1.0f / (float)t : 0.f;
  }
}

// out[c, r] = in[r, c] for r < R and 0 for R <= r < Rp (c < Cc), through a
// 64 x 64 LDS tile: both the reads and the writes are row-contiguous.
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(const T* __restrict__ in, long long ld_in, int R, int Cc,
                                                        T* __restrict__ out, long long ld_out, int Rp) {
  __shared__ float tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < Cc) ? to_f32(in[(long long)r * ld_in + c]) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < Cc && r < Rp) out[(long long)c * ld_out + r] = from_f32<T>(tile[tx][i]);
  }
}

// p[r, c] = 0 for r < R, c0 <= c < c1
template <typename T>
__global__ void __launch_bounds__(256) zero_cols_kernel(T* __restrict__ p, long long ld, int R, int c0, int c1) {
  const int w = c1 - c0;
  const long long total = (long long)R * w;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
    const long long r = e / w;
    p[r * ld + c0 + (int)(e - r * w)] = from_f32<T>(0.f);
  }
}

// fp32 rows -> the compute dtype (post-LN models: the head reads the final
// hidden rows themselves)
template <typename T>
__global__ void __launch_bounds__(256) cast_rows_kernel(const float* __restrict__ x, long long n, T* __restrict__ out) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256)
    out[e] = from_f32<T>(x[e]);
}

// LayerNorm backward, one wave per row: dx (overwritten) and the row's mean
// and 1 / sqrt(var + eps) for the column sums.  Statistics as in the forward:
// mean, then the biased variance of the centred row.
template <typename T>
__global__ void __launch_bounds__(256) ln_bwd_rows_kernel(int M, int C, const float* __restrict__ x,
                                                          const T* __restrict__ g, const float* __restrict__ dy,
                                                          float eps, float* __restrict__ dx, float* __restrict__ mu,
                                                          float* __restrict__ rs) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;   // (no block-wide barrier below)
  const float* xr = x + (long long)m * C;
  const float* dr = dy + (long long)m * C;
  float s = 0.f;
  for (int c = lane; c < C; c += 64) s += xr[c];
  const float mean = wave_sum(s) / (float)C;
  float s2 = 0.f;
  for (int c = lane; c < C; c += 64) {
    const float d = xr[c] - mean;
    s2 += d * d;
  }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) / (float)C + eps);
  float sg = 0.f, sgx = 0.f;
  for (int c = lane; c < C; c += 64) {
    const float xh = (xr[c] - mean) * rstd;
    const float gd = dr[c] * to_f32(g[c]);
    sg += gd;
    sgx += gd * xh;
  }
  const float m1 = wave_sum(sg) / (float)C, m2 = wave_sum(sgx) / (float)C;
  float* o = dx + (long long)m * C;
  for (int c = lane; c < C; c += 64) {
    const float xh = (xr[c] - mean) * rstd;
    const float gd = dr[c] * to_f32(g[c]);
    o[c] = rstd * (gd - m1 - xh * m2);
  }
  if (lane == 0) {
    mu[m] = mean;
    rs[m] = rstd;
  }
}

// Column sums of dy * xh and dy over a chunk of LNB_CHUNK rows: block = 64
// columns x 4 row lanes; part[chunk][0 / 1][C].
constexpr int LNB_CHUNK = 256;

__global__ void __launch_bounds__(256) ln_bwd_cols_kernel(int M, int C, const float* __restrict__ x,
                                                          const float* __restrict__ dy, const float* __restrict__ mu,
                                                          const float* __restrict__ rs, float* __restrict__ part) {
  __shared__ float red[2][4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + tx;
  const int r0 = blockIdx.y * LNB_CHUNK, r1 = min(M, r0 + LNB_CHUNK);
  float sg = 0.f, sb = 0.f;
  if (c < C)
    for (int r = r0 + ty; r < r1; r += 4) {
      const float d = dy[(long long)r * C + c];
      sg += d * ((x[(long long)r * C + c] - mu[r]) * rs[r]);
      sb += d;
    }
  red[0][ty][tx] = sg;
  red[1][ty][tx] = sb;
  __syncthreads();
  if (ty == 0 && c < C) {
    float* p = part + (long long)blockIdx.y * 2 * C;
    p[c] = (red[0][0][tx] + red[0][1][tx]) + (red[0][2][tx] + red[0][3][tx]);
    p[C + c] = (red[1][0][tx] + red[1][1][tx]) + (red[1][2][tx] + red[1][3][tx]);
  }
}

// dg[c] += sum of the chunks' partials (chunk order), db likewise
__global__ void __launch_bounds__(256) ln_bwd_final_kernel(int C, int nchunks, const float* __restrict__ part,
                                                           float* __restrict__ dg, float* __restrict__ db) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float a = 0.f, b = 0.f;
  for (int k = 0; k < nchunks; ++k) {
    a += part[(long long)k * 2 * C + c];
    b += part[(long long)k * 2 * C + C + c];
  }
  dg[c] += a;
  db[c] += b;
}

// Token-table rows of the embedding backward.  Block n handles position n if
// no earlier position holds the same token; it then sums, in position order,
// the rows of dx0 of every position holding that token and adds the sum to
// the token's row.  Positions holding an id outside [0, V) contribute nothing.
constexpr int EMB_CHUNK = 4096;   // positions per mask pass
constexpr int EMB_MAXC = 8;       // columns per thread: C <= 2048

__global__ void __launch_bounds__(256) embed_bwd_tok_kernel(const int32_t* __restrict__ idx, int N, int C, int V,
                                                            const float* __restrict__ dx0, float* __restrict__ dwte) {
  __shared__ unsigned long long mask[EMB_CHUNK / 64];
  const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = idx[n];
  if (v < 0 || v >= V) return;   // uniform over the block
  int seen = 0;
  for (int m = tid; m < n; m += 256) seen |= idx[m] == v ? 1 : 0;
  if (__syncthreads_or(seen)) return;
  float acc[EMB_MAXC];
#pragma unroll
  for (int k = 0; k < EMB_MAXC; ++k) acc[k] = 0.f;
  for (int base = n; base < N; base += EMB_CHUNK) {
    for (int gi = wave; gi < EMB_CHUNK / 64; gi += 4) {
      const int m = base + gi * 64 + lane;
      const unsigned long long b = __ballot(m < N && idx[m] == v);
      if (lane == 0) mask[gi] = b;
    }
    __syncthreads();
    for (int gi = 0; gi < EMB_CHUNK / 64; ++gi) {
      unsigned long long b = mask[gi];
      while (b) {
        const int bit = __builtin_ctzll(b);
        b &= b - 1;
        const float* row = dx0 + (long long)(base + gi * 64 + bit) * C;
#pragma unroll
        for (int k = 0; k < EMB_MAXC; ++k) {
          const int c = tid + 256 * k;
          if (c < C) acc[k] += row[c];
        }
      }
    }
    __syncthreads();   // masks are rewritten by the next chunk
  }
  float* out = dwte + (long long)v * C;
#pragma unroll
  for (int k = 0; k < EMB_MAXC; ++k) {
    const int c = tid + 256 * k;
    if (c < C) out[c] += acc[k];
  }
}

// Position-table rows: dwpe[t] += sum over the batch (in order) of dx0[b, t]
__global__ void __launch_bounds__(256) embed_bwd_pos_kernel(int B, int T, int C, const float* __restrict__ dx0,
                                                            float* __restrict__ dwpe) {
  const int t = blockIdx.x, c = blockIdx.y * 256 + threadIdx.x;
  if (c >= C) return;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += dx0[((long long)b * T + t) * C + c];
  dwpe[(long long)t * C + c] += s;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static int grid_for(long long n) { return (int)std::min<long long>((n + 255) / 256, 8192); }

hipError_t launch_bwd_rows(int M, int ntiles, const float* part_max, const float* part_sum, const int32_t* targets,
                           const int32_t* idx, int T_seq, int V, float* lse, int32_t* yv, float* inv,
                           hipStream_t st) {
  hipLaunchKernelGGL(bwd_rows_kernel, dim3((M + BR_ROWS - 1) / BR_ROWS), dim3(256), 0, st, M, ntiles, part_max,
                     part_sum, targets, idx, T_seq, V, lse, yv);
  hipLaunchKernelGGL(bwd_count_kernel, dim3(1), dim3(1024), 0, st, M, (const int32_t*)yv, inv);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const void* in, long long ld_in, int R, int Cc, void* out, int Rp,
                            hipStream_t st) {
  const dim3 grid((Rp + 63) / 64, (Cc + 63) / 64);
  if (dtype == 0)
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, st, (const float*)in, ld_in, R, Cc, (float*)out,
                       (long long)Rp, Rp);
  else
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)in, ld_in, R, Cc, (bf16*)out,
                       (long long)Rp, Rp);
  return hipGetLastError();
}

hipError_t launch_zero_cols(int dtype, void* p, long long ld, int R, int c0, int c1, hipStream_t st) {
  if (c1 <= c0 || R <= 0) return hipSuccess;
  const int grid = grid_for((long long)R * (c1 - c0));
  if (dtype == 0)
    hipLaunchKernelGGL(zero_cols_kernel<float>, dim3(grid), dim3(256), 0, st, (float*)p, ld, R, c0, c1);
  else
    hipLaunchKernelGGL(zero_cols_kernel<bf16>, dim3(grid), dim3(256), 0, st, (bf16*)p, ld, R, c0, c1);
  return hipGetLastError();
}

hipError_t launch_cast_rows(int dtype, const float* x, long long n, void* out, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL(cast_rows_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, x, n, (float*)out);
  else
    hipLaunchKernelGGL(cast_rows_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, st, x, n, (bf16*)out);
  return hipGetLastError();
}

int ln_bwd_chunks(int M) { return (M + LNB_CHUNK - 1) / LNB_CHUNK; }

hipError_t launch_ln_backward(int dtype, int M, int C, const float* x, const void* g, const float* dy, float eps,
                              float* dx, float* mu, float* rs, float* part, float* dg, float* db, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL(ln_bwd_rows_kernel<float>, dim3((M + 3) / 4), dim3(256), 0, st, M, C, x, (const float*)g, dy,
                       eps, dx, mu, rs);
  else
    hipLaunchKernelGGL(ln_bwd_rows_kernel<bf16>, dim3((M + 3) / 4), dim3(256), 0, st, M, C, x, (const bf16*)g, dy,
                       eps, dx, mu, rs);
  const int nch = ln_bwd_chunks(M);
  hipLaunchKernelGGL(ln_bwd_cols_kernel, dim3((C + 63) / 64, nch), dim3(256), 0, st, M, C, x, dy, (const float*)mu,
                     (const float*)rs, part);
  hipLaunchKernelGGL(ln_bwd_final_kernel, dim3((C + 255) / 256), dim3(256), 0, st, C, nch, (const float*)part, dg, db);
  return hipGetLastError();
}

hipError_t launch_embed_backward(const int32_t* idx, int B, int T, int C, int V, const float* dx0, float* dwte,
                                 float* dwpe, hipStream_t st) {
  const int N = B * T;
  hipLaunchKernelGGL(embed_bwd_tok_kernel, dim3(N), dim3(256), 0, st, idx, N, C, V, dx0, dwte);
  if (dwpe) hipLaunchKernelGGL(embed_bwd_pos_kernel, dim3(T, (C + 255) / 256), dim3(256), 0, st, B, T, C, dx0, dwpe);
  return hipGetLastError();
}

}  // namespace gptmi
