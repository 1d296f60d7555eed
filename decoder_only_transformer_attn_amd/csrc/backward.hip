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
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace gptmi {

#define GPT_BWD_TRY(expr)                   \
  do {                                      \
    const hipError_t _e = (expr);           \
    if (_e != hipSuccess) return _e;        \
  } while (0)

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

// bf16 form of the same with 16-byte accesses (Cc, ld_in and Rp multiples of
// 8, 16-byte aligned rows): each thread loads 8 consecutive columns of one
// input row and stores 8 consecutive rows of one output row; the tile sits in
// LDS row-major with a 2-element pad, so the column gathers of the store phase
// (8 halfwords, 66 elements apart) spread over the banks.  Batched over
// blockIdx.z = b H + h: input at b in_b + h in_h, output at z out_z.
__global__ void __launch_bounds__(256) transpose16_kernel(const bf16* __restrict__ in, long long ld_in, long long in_b,
                                                          long long in_h, int H, int R, int Cc,
                                                          bf16* __restrict__ out, long long ld_out, long long out_z,
                                                          int Rp) {
  constexpr int LDT = 66;
  __shared__ __align__(16) uint16_t tile[64 * LDT];
  {
    const int z = blockIdx.z, b = z / H, h = z - b * H;
    in += b * in_b + h * in_h;
    out += (long long)z * out_z;
  }
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x, sub = tid >> 3, k = tid & 7;   // 32 rows x 8 chunks per pass
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int i = p * 32 + sub, r = r0 + i, c = c0 + k * 8;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (r < R && c < Cc) w = *reinterpret_cast<const uint4*>(in + (long long)r * ld_in + c);
    const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)   // 4-byte LDS stores (LDT is even)
      *reinterpret_cast<uint32_t*>(&tile[i * LDT + k * 8 + 2 * e]) = h[e];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int oi = p * 32 + sub, c = c0 + oi, r = r0 + k * 8;   // output row c, columns r .. r + 7
    if (c >= Cc || r >= Rp) continue;
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      h[e] = (uint32_t)tile[(k * 8 + 2 * e) * LDT + oi] | ((uint32_t)tile[(k * 8 + 2 * e + 1) * LDT + oi] << 16);
    *reinterpret_cast<uint4*>(out + (long long)c * ld_out + r) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

// fp32 rows in, both bf16 layouts out: out_rm [R, ld_rm] = in and out_t =
// its transpose [Cc, Rp] (zeros for R <= r < Rp), one pass over the input
// (Cc, ld_in, ld_rm and Rp multiples of 8, 16-byte aligned rows).
__global__ void __launch_bounds__(256) cast_transpose16_kernel(const float* __restrict__ in, long long ld_in, int R,
                                                               int Cc, bf16* __restrict__ out_rm, long long ld_rm,
                                                               bf16* __restrict__ out_t, int Rp) {
  constexpr int LDT = 66;
  __shared__ __align__(16) uint16_t tile[64 * LDT];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x, sub = tid >> 3, k = tid & 7;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int i = p * 32 + sub, r = r0 + i, c = c0 + k * 8;
    uint32_t h[4] = {0u, 0u, 0u, 0u};
    if (r < R && c < Cc) {
      const float4 a = *reinterpret_cast<const float4*>(in + (long long)r * ld_in + c);
      const float4 b = *reinterpret_cast<const float4*>(in + (long long)r * ld_in + c + 4);
      h[0] = pack_bf16x2(a.x, a.y); h[1] = pack_bf16x2(a.z, a.w);
      h[2] = pack_bf16x2(b.x, b.y); h[3] = pack_bf16x2(b.z, b.w);
      *reinterpret_cast<uint4*>(out_rm + (long long)r * ld_rm + c) = make_uint4(h[0], h[1], h[2], h[3]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(&tile[i * LDT + k * 8 + 2 * e]) = h[e];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int oi = p * 32 + sub, c = c0 + oi, r = r0 + k * 8;
    if (c >= Cc || r >= Rp) continue;
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      h[e] = (uint32_t)tile[(k * 8 + 2 * e) * LDT + oi] | ((uint32_t)tile[(k * 8 + 2 * e + 1) * LDT + oi] << 16);
    *reinterpret_cast<uint4*>(out_t + (long long)c * Rp + r) = make_uint4(h[0], h[1], h[2], h[3]);
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

// bf16 form, four elements per thread (n a multiple of 4, 16-byte aligned x)
__global__ void __launch_bounds__(256) cast_rows4_kernel(const float4* __restrict__ x, long long n4,
                                                         uint2* __restrict__ out) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n4; e += (long long)gridDim.x * 256) {
    const float4 v = x[e];
    out[e] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

// LayerNorm backward, one wave per row: dx (overwritten) and the row's mean
// and 1 / sqrt(var + eps) for the column sums.  Statistics as in the forward:
// mean, then the biased variance of the centred row.
template <typename T>
__global__ void __launch_bounds__(256) ln_bwd_rows_kernel(int M, int C, const float* __restrict__ x,
                                                          const T* __restrict__ g, const float* __restrict__ dy,
                                                          float eps, float* __restrict__ dx, float* __restrict__ mu,
                                                          float* __restrict__ rs, int accumulate) {
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
    o[c] = (accumulate ? o[c] : 0.f) + rstd * (gd - m1 - xh * m2);
  }
  if (lane == 0) {
    mu[m] = mean;
    rs[m] = rstd;
  }
}

// The same with the row in registers (C = 256 NV, 16-byte aligned rows):
// lane l holds columns 4 (64 i + l) .. + 3 of x, dy and g for i < NV, so x and
// dy are read once; the sums run over the same terms in another order.
template <typename T, int NV>
__global__ void __launch_bounds__(256) ln_bwd_rows4_kernel(int M, int C, const float* __restrict__ x,
                                                           const T* __restrict__ g, const float* __restrict__ dy,
                                                           float eps, float* __restrict__ dx, float* __restrict__ mu,
                                                           float* __restrict__ rs, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;   // (no block-wide barrier below)
  const float4* xr = reinterpret_cast<const float4*>(x + (long long)m * C);
  const float4* dr = reinterpret_cast<const float4*>(dy + (long long)m * C);
  float xv[NV][4], gd[NV][4];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c4 = i * 64 + lane;
    const float4 a = xr[c4], d = dr[c4];
    float gg[4];
    if constexpr (sizeof(T) == 2) {
      const uint2 w = *reinterpret_cast<const uint2*>(g + 4 * c4);
      gg[0] = __uint_as_float(w.x << 16); gg[1] = __uint_as_float(w.x & 0xffff0000u);
      gg[2] = __uint_as_float(w.y << 16); gg[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
      const float4 w = *reinterpret_cast<const float4*>(g + 4 * c4);
      gg[0] = w.x; gg[1] = w.y; gg[2] = w.z; gg[3] = w.w;
    }
    xv[i][0] = a.x; xv[i][1] = a.y; xv[i][2] = a.z; xv[i][3] = a.w;
    gd[i][0] = d.x * gg[0]; gd[i][1] = d.y * gg[1]; gd[i][2] = d.z * gg[2]; gd[i][3] = d.w * gg[3];
    s += (a.x + a.y) + (a.z + a.w);
  }
  const float mean = wave_sum(s) / (float)C;
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = xv[i][e] - mean;
      s2 += d * d;
    }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) / (float)C + eps);
  float sg = 0.f, sgx = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[i][e] = (xv[i][e] - mean) * rstd;   // now x-hat
      sg += gd[i][e];
      sgx += gd[i][e] * xv[i][e];
    }
  const float m1 = wave_sum(sg) / (float)C, m2 = wave_sum(sgx) / (float)C;
  float4* o = reinterpret_cast<float4*>(dx + (long long)m * C);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c4 = i * 64 + lane;
    float4 r = make_float4(rstd * (gd[i][0] - m1 - xv[i][0] * m2), rstd * (gd[i][1] - m1 - xv[i][1] * m2),
                           rstd * (gd[i][2] - m1 - xv[i][2] * m2), rstd * (gd[i][3] - m1 - xv[i][3] * m2));
    if (accumulate) {
      const float4 p = o[c4];
      r.x = p.x + r.x; r.y = p.y + r.y; r.z = p.z + r.z; r.w = p.w + r.w;
    }
    o[c4] = r;
  }
  if (lane == 0) {
    mu[m] = mean;
    rs[m] = rstd;
  }
}

// Column sums of dy * xh and dy over a chunk of LNB_CHUNK rows: block = 64
// columns x 4 row lanes; part[chunk][0 / 1][C].
constexpr int LNB_CHUNK = 64;

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

// 16-byte form (C a multiple of 4, 16-byte aligned rows): block = 256
// columns x 4 waves taking every 4th row of the chunk; the waves' sums are
// added in wave order.
__global__ void __launch_bounds__(256) ln_bwd_cols4_kernel(int M, int C, const float* __restrict__ x,
                                                           const float* __restrict__ dy, const float* __restrict__ mu,
                                                           const float* __restrict__ rs, float* __restrict__ part) {
  __shared__ __align__(16) float red[2][4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 256 + lane * 4;
  const int r0 = blockIdx.y * LNB_CHUNK;
  float4 sg = make_float4(0.f, 0.f, 0.f, 0.f), sb = sg;
  if (c < C) {
#pragma unroll
    for (int i = 0; i < LNB_CHUNK / 4; ++i) {
      const int r = r0 + w + 4 * i;
      if (r < M) {
        const float4 d = *reinterpret_cast<const float4*>(dy + (long long)r * C + c);
        const float4 a = *reinterpret_cast<const float4*>(x + (long long)r * C + c);
        const float u = mu[r], q = rs[r];
        sg.x += d.x * ((a.x - u) * q); sg.y += d.y * ((a.y - u) * q);
        sg.z += d.z * ((a.z - u) * q); sg.w += d.w * ((a.w - u) * q);
        sb.x += d.x; sb.y += d.y; sb.z += d.z; sb.w += d.w;
      }
    }
  }
  *reinterpret_cast<float4*>(&red[0][w][lane * 4]) = sg;
  *reinterpret_cast<float4*>(&red[1][w][lane * 4]) = sb;
  __syncthreads();
  const int t = threadIdx.x, col = blockIdx.x * 256 + t;
  if (col < C) {
    float* p = part + (long long)blockIdx.y * 2 * C;
    p[col] = ((red[0][0][t] + red[0][1][t]) + red[0][2][t]) + red[0][3][t];
    p[C + col] = ((red[1][0][t] + red[1][1][t]) + red[1][2][t]) + red[1][3][t];
  }
}

// dg[c] += the chunks' partials, db likewise: a block per 64 columns, its 4
// waves taking every 4th chunk, then the waves' sums in wave order.
__global__ void __launch_bounds__(256) ln_bwd_final4_kernel(int C, int nchunks, const float* __restrict__ part,
                                                            float* __restrict__ dg, float* __restrict__ db) {
  __shared__ float red[2][4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float a = 0.f, b = 0.f;
  if (c < C) {
#pragma unroll 8
    for (int k = w; k < nchunks; k += 4) {
      a += part[(long long)k * 2 * C + c];
      b += part[(long long)k * 2 * C + C + c];
    }
  }
  red[0][w][lane] = a;
  red[1][w][lane] = b;
  __syncthreads();
  if (w == 0 && c < C) {
    dg[c] += ((red[0][0][lane] + red[0][1][lane]) + red[0][2][lane]) + red[0][3][lane];
    db[c] += ((red[1][0][lane] + red[1][1][lane]) + red[1][2][lane]) + red[1][3][lane];
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
  else if (Cc % 8 == 0 && ld_in % 8 == 0 && Rp % 8 == 0 && ((uintptr_t)in & 15) == 0 && ((uintptr_t)out & 15) == 0)
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, st, (const bf16*)in, ld_in, 0LL, 0LL, 1, R, Cc,
                       (bf16*)out, (long long)Rp, 0LL, Rp);
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

hipError_t launch_cast_transpose(int dtype, const float* in, int R, int Cc, void* out_rm, void* out_t, int Rp,
                                 hipStream_t st) {
  if (R <= 0 || Cc <= 0) return hipSuccess;
  if (dtype != 0 && Cc % 8 == 0 && Rp % 8 == 0 && ((uintptr_t)in & 15) == 0 && ((uintptr_t)out_rm & 15) == 0 &&
      ((uintptr_t)out_t & 15) == 0) {
    const dim3 grid((Rp + 63) / 64, (Cc + 63) / 64);
    hipLaunchKernelGGL(cast_transpose16_kernel, grid, dim3(256), 0, st, in, (long long)Cc, R, Cc, (bf16*)out_rm,
                       (long long)Cc, (bf16*)out_t, Rp);
    return hipGetLastError();
  }
  const hipError_t e = launch_cast_rows(dtype, in, (long long)R * Cc, out_rm, st);
  if (e != hipSuccess) return e;
  return launch_transpose(dtype, out_rm, Cc, R, Cc, out_t, Rp, st);
}

hipError_t launch_cast_rows(int dtype, const float* x, long long n, void* out, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL(cast_rows_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, x, n, (float*)out);
  else if (n % 4 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)out & 7) == 0)
    hipLaunchKernelGGL(cast_rows4_kernel, dim3(grid_for(n / 4)), dim3(256), 0, st, (const float4*)x, n / 4,
                       (uint2*)out);
  else
    hipLaunchKernelGGL(cast_rows_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, st, x, n, (bf16*)out);
  return hipGetLastError();
}

int ln_bwd_chunks(int M) { return (M + LNB_CHUNK - 1) / LNB_CHUNK; }

hipError_t launch_ln_backward(int dtype, int M, int C, const float* x, const void* g, const float* dy, float eps,
                              float* dx, float* mu, float* rs, float* part, float* dg, float* db, hipStream_t st,
                              int accumulate) {
  if (M <= 0) return hipSuccess;
  const bool v4 = C % 4 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)dy & 15) == 0 && ((uintptr_t)dx & 15) == 0 &&
                  ((uintptr_t)g & (dtype == 0 ? 15 : 7)) == 0;
  const int nv = C % 256 == 0 ? C / 256 : 0;
  const dim3 rg((M + 3) / 4);
#define GPT_LNB_ROWS4(TT, NVV)                                                                                  \
  hipLaunchKernelGGL((ln_bwd_rows4_kernel<TT, NVV>), rg, dim3(256), 0, st, M, C, x, (const TT*)g, dy, eps, dx, \
                     mu, rs, accumulate)
  if (v4 && nv >= 1 && nv <= 4) {
    if (dtype == 0) {
      if (nv == 1) GPT_LNB_ROWS4(float, 1); else if (nv == 2) GPT_LNB_ROWS4(float, 2);
      else if (nv == 3) GPT_LNB_ROWS4(float, 3); else GPT_LNB_ROWS4(float, 4);
    } else {
      if (nv == 1) GPT_LNB_ROWS4(bf16, 1); else if (nv == 2) GPT_LNB_ROWS4(bf16, 2);
      else if (nv == 3) GPT_LNB_ROWS4(bf16, 3); else GPT_LNB_ROWS4(bf16, 4);
    }
  } else if (dtype == 0) {
    hipLaunchKernelGGL(ln_bwd_rows_kernel<float>, rg, dim3(256), 0, st, M, C, x, (const float*)g, dy, eps, dx, mu, rs,
                       accumulate);
  } else {
    hipLaunchKernelGGL(ln_bwd_rows_kernel<bf16>, rg, dim3(256), 0, st, M, C, x, (const bf16*)g, dy, eps, dx, mu, rs,
                       accumulate);
  }
#undef GPT_LNB_ROWS4
  const int nch = ln_bwd_chunks(M);
  if (v4) {
    hipLaunchKernelGGL(ln_bwd_cols4_kernel, dim3((C + 255) / 256, nch), dim3(256), 0, st, M, C, x, dy,
                       (const float*)mu, (const float*)rs, part);
    hipLaunchKernelGGL(ln_bwd_final4_kernel, dim3((C + 63) / 64), dim3(256), 0, st, C, nch, (const float*)part, dg,
                       db);
  } else {
    hipLaunchKernelGGL(ln_bwd_cols_kernel, dim3((C + 63) / 64, nch), dim3(256), 0, st, M, C, x, dy, (const float*)mu,
                       (const float*)rs, part);
    hipLaunchKernelGGL(ln_bwd_final_kernel, dim3((C + 255) / 256), dim3(256), 0, st, C, nch, (const float*)part, dg,
                       db);
  }
  return hipGetLastError();
}

hipError_t launch_embed_backward(const int32_t* idx, int B, int T, int C, int V, const float* dx0, float* dwte,
                                 float* dwpe, hipStream_t st) {
  const int N = B * T;
  hipLaunchKernelGGL(embed_bwd_tok_kernel, dim3(N), dim3(256), 0, st, idx, N, C, V, dx0, dwte);
  if (dwpe) hipLaunchKernelGGL(embed_bwd_pos_kernel, dim3(T, (C + 255) / 256), dim3(256), 0, st, B, T, C, dx0, dwpe);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block backward: element-wise parts and the attention backward
// ---------------------------------------------------------------------------
__device__ __forceinline__ float gelu_tanh_f(float z) {
  const float u = 0.7978845608028654f * (z + 0.044715f * z * z * z);
  return 0.5f * z * (1.0f + tanhf(u));
}
__device__ __forceinline__ float gelu_tanh_d(float z) {   // d/dz 0.5 z (1 + tanh u)
  const float u = 0.7978845608028654f * (z + 0.044715f * z * z * z);
  const float t = tanhf(u);
  return 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * 0.7978845608028654f * (1.0f + 0.134145f * z * z);
}
__device__ __forceinline__ float gelu_erf_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.7071067811865476f)); }
__device__ __forceinline__ float gelu_erf_d(float z) {    // Phi(z) + z phi(z)
  return 0.5f * (1.0f + erff(z * 0.7071067811865476f)) + z * 0.3989422804014327f * __expf(-0.5f * z * z);
}

// h = GELU(u) (act 0: tanh form, 1: exact)
template <typename T>
__global__ void __launch_bounds__(256) act_fwd_kernel(const T* __restrict__ u, long long n, int act, T* __restrict__ h) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const float z = to_f32(u[e]);
    h[e] = from_f32<T>(act ? gelu_erf_f(z) : gelu_tanh_f(z));
  }
}

// d (fp32, in place) *= GELU'(u); dc = d in the compute dtype
template <typename T>
__global__ void __launch_bounds__(256) act_bwd_kernel(float* __restrict__ d, const T* __restrict__ u, long long n,
                                                      int act, T* __restrict__ dc) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const float z = to_f32(u[e]);
    const float v = d[e] * (act ? gelu_erf_d(z) : gelu_tanh_d(z));
    d[e] = v;
    dc[e] = from_f32<T>(v);
  }
}

// bf16 forms, four elements per thread (n a multiple of 4, 8-byte aligned
// bf16 and 16-byte aligned fp32 arrays)
__device__ __forceinline__ void unpack4(uint2 w, float (&z)[4]) {
  z[0] = __uint_as_float(w.x << 16); z[1] = __uint_as_float(w.x & 0xffff0000u);
  z[2] = __uint_as_float(w.y << 16); z[3] = __uint_as_float(w.y & 0xffff0000u);
}

__global__ void __launch_bounds__(256) act_fwd4_kernel(const uint2* __restrict__ u, long long n4, int act,
                                                       uint2* __restrict__ h) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n4; e += (long long)gridDim.x * 256) {
    float z[4];
    unpack4(u[e], z);
#pragma unroll
    for (int k = 0; k < 4; ++k) z[k] = act ? gelu_erf_f(z[k]) : gelu_tanh_f(z[k]);
    h[e] = make_uint2(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]));
  }
}

__global__ void __launch_bounds__(256) act_bwd4_kernel(float4* __restrict__ d, const uint2* __restrict__ u,
                                                       long long n4, int act, uint2* __restrict__ dc) {
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n4; e += (long long)gridDim.x * 256) {
    float z[4];
    unpack4(u[e], z);
    float4 v = d[e];
    v.x *= act ? gelu_erf_d(z[0]) : gelu_tanh_d(z[0]);
    v.y *= act ? gelu_erf_d(z[1]) : gelu_tanh_d(z[1]);
    v.z *= act ? gelu_erf_d(z[2]) : gelu_tanh_d(z[2]);
    v.w *= act ? gelu_erf_d(z[3]) : gelu_tanh_d(z[3]);
    d[e] = v;
    dc[e] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  }
}

// Column sums of an fp32 [M, N] matrix into per-chunk partials (fixed order),
// then out[n] += sum of the partials in chunk order.
__global__ void __launch_bounds__(256) colsum_part_kernel(int M, int N, const float* __restrict__ a,
                                                          float* __restrict__ part) {
  __shared__ float red[4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + tx;
  const int r0 = blockIdx.y * LNB_CHUNK, r1 = min(M, r0 + LNB_CHUNK);
  float s = 0.f;
  if (c < N)
    for (int r = r0 + ty; r < r1; r += 4) s += a[(long long)r * N + c];
  red[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && c < N) part[(long long)blockIdx.y * N + c] = (red[0][tx] + red[1][tx]) + (red[2][tx] + red[3][tx]);
}

// Column sums with 16-byte loads (N a multiple of 4, a 16-byte aligned): a
// block sums CS_ROWS rows of 256 columns, its 4 waves taking every 4th row
// (16 independent loads in flight per thread), then adds the waves' sums in
// wave order; partials [chunk][N].  The final pass: a block per 64 columns,
// its 4 waves taking every 4th chunk, then the waves' sums in wave order.
constexpr int CS_ROWS = 64;
int colsum_chunks(int M) { return (M + CS_ROWS - 1) / CS_ROWS; }

__global__ void __launch_bounds__(256) colsum_part4_kernel(int M, int N, const float* __restrict__ a,
                                                           float* __restrict__ part) {
  __shared__ __align__(16) float red[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 256 + lane * 4;
  const int r0 = blockIdx.y * CS_ROWS;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < N) {
#pragma unroll
    for (int i = 0; i < CS_ROWS / 4; ++i) {
      const int r = r0 + w + 4 * i;
      if (r < M) {
        const float4 v = *reinterpret_cast<const float4*>(a + (long long)r * N + c);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
      }
    }
  }
  *reinterpret_cast<float4*>(&red[w][lane * 4]) = s;
  __syncthreads();
  const int t = threadIdx.x, col = blockIdx.x * 256 + t;
  if (col < N) part[(long long)blockIdx.y * N + col] = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
}

__global__ void __launch_bounds__(256) colsum_final4_kernel(int N, int nchunks, const float* __restrict__ part,
                                                            float* __restrict__ out) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (c < N) {
#pragma unroll 8
    for (int k = w; k < nchunks; k += 4) s += part[(long long)k * N + c];
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && c < N) out[c] += ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

__global__ void __launch_bounds__(256) colsum_final_kernel(int N, int nchunks, const float* __restrict__ part,
                                                           float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= N) return;
  float s = 0.f;
  for (int k = 0; k < nchunks; ++k) s += part[(long long)k * N + c];
  out[c] += s;
}

// Attention backward for causal heads on the matrix cores, with the score
// matrices materialised per head (T x Tp, Tp = T rounded up to 64):
//   S = Q K^T;  P = softmax(S / sqrt(D)) over keys j <= t (0 elsewhere);
//   dP = dO U^T;  dS = P (dP - rowsum(P dP)) / sqrt(D);
//   dU = P^T dO,  dQ = dS K,  dK = dS^T Q.
// The five products are batched launches of the tiled GEMM (grid.y = B*H) on
// zero-padded per-head transposes, so every contraction runs over Tp with
// exact zeros in the pads; the row kernels use one wave per row and
// fixed-order reductions.

// out_z[c, r] = in_z[r, c] (r < R, c < Cc), 0 for R <= r < Rp; in_z starts at
// b * in_b + h * in_h (z = b * H + h), out_z at z * out_z.
template <typename TI, typename TO>
__global__ void __launch_bounds__(256) transpose_batched_kernel(const TI* __restrict__ in, long long ld_in,
                                                                long long in_b, long long in_h, int H, int R, int Cc,
                                                                TO* __restrict__ out, long long ld_out,
                                                                long long out_z, int Rp) {
  __shared__ float tile[64][65];
  const int z = blockIdx.z, b = z / H, h = z - b * H;
  in += b * in_b + h * in_h;
  out += (long long)z * out_z;
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < Cc) ? to_f32(in[(long long)r * ld_in + c]) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < Cc && r < Rp) out[(long long)c * ld_out + r] = from_f32<TO>(tile[tx][i]);
  }
}

template <typename TI, typename TO>
static void transpose_batched(const TI* in, long long ld_in, long long in_b, long long in_h, int H, int R, int Cc,
                              TO* out, long long ld_out, long long out_z, int Rp, int Z, hipStream_t st) {
  const dim3 grid((Rp + 63) / 64, (Cc + 63) / 64, Z);
  if constexpr (std::is_same<TI, bf16>::value && std::is_same<TO, bf16>::value) {
    if (Cc % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0 && Rp % 8 == 0 && in_b % 8 == 0 && in_h % 8 == 0 &&
        out_z % 8 == 0 && ((uintptr_t)in & 15) == 0 && ((uintptr_t)out & 15) == 0) {
      hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, st, in, ld_in, in_b, in_h, H, R, Cc, out, ld_out,
                         out_z, Rp);
      return;
    }
  }
  hipLaunchKernelGGL((transpose_batched_kernel<TI, TO>), grid, dim3(256), 0, st, in, ld_in, in_b, in_h, H, R, Cc, out,
                     ld_out, out_z, Rp);
}

// P row (z, t) from the S row: causal softmax of S / sqrt(D), zeros past t and
// in the pads.  Only S[t, j <= t] is read (the tiles above the diagonal are not
// computed).  NV > 0: the row (Tp <= 256 NV) is held in registers, four
// consecutive columns per lane and step (16-byte loads); NV = 0: strided.
template <typename T, int NV>
__global__ void __launch_bounds__(256) attn_bwd_softmax_kernel(const float* __restrict__ S, T* __restrict__ P,
                                                               int Z, int Tn, int Tp, float scale) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)Z * Tn) return;   // (no block-wide barrier)
  const int t = (int)(row % Tn);
  const float* sr = S + row * Tp;
  T* pr = P + row * Tp;
  if constexpr (NV > 0) {
    float v[NV][4];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = i * 256 + lane * 4;
      if (j <= t) {   // (j < Tp: t < Tn <= Tp)
        const float4 x = *reinterpret_cast<const float4*>(sr + j);
        v[i][0] = x.x * scale; v[i][1] = x.y * scale; v[i][2] = x.z * scale; v[i][3] = x.w * scale;
      } else {
        v[i][0] = v[i][1] = v[i][2] = v[i][3] = -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e > t) v[i][e] = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, v[i][e]);
    }
    m = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[i][e] = __expf(v[i][e] - m);   // exp(-inf) = 0 past t
        l += v[i][e];
      }
    const float inv = 1.0f / wave_sum(l);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = i * 256 + lane * 4;
      if (j < Tp) {
        if constexpr (sizeof(T) == 4) {
          *reinterpret_cast<float4*>(pr + j) = make_float4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
        } else {
          *reinterpret_cast<uint2*>(pr + j) =
              make_uint2(pack_bf16x2(v[i][0] * inv, v[i][1] * inv), pack_bf16x2(v[i][2] * inv, v[i][3] * inv));
        }
      }
    }
  } else {
    float m = -INFINITY;
    for (int j = lane; j <= t; j += 64) m = fmaxf(m, sr[j] * scale);
    m = wave_max(m);
    float l = 0.f;
    for (int j = lane; j <= t; j += 64) l += __expf(sr[j] * scale - m);
    const float inv = 1.0f / wave_sum(l);
    for (int j = lane; j < Tp; j += 64) pr[j] = from_f32<T>(j <= t ? __expf(sr[j] * scale - m) * inv : 0.f);
  }
}

// dS row (z, t) = P (dP - sum_{j <= t} P dP) * scale for j <= t, 0 elsewhere
// (dP is read only at j <= t: the tiles above the diagonal are not computed)
template <typename T, int NV>
__global__ void __launch_bounds__(256) attn_bwd_ds_kernel(const T* __restrict__ P, const float* __restrict__ dP,
                                                          T* __restrict__ dS, int Z, int Tn, int Tp, float scale) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)Z * Tn) return;
  const int t = (int)(row % Tn);
  const T* pr = P + row * Tp;
  const float* gr = dP + row * Tp;
  T* out = dS + row * Tp;
  if constexpr (NV > 0) {
    float p[NV][4], g[NV][4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = i * 256 + lane * 4;
      if (j <= t) {
        const float4 x = *reinterpret_cast<const float4*>(gr + j);
        g[i][0] = x.x; g[i][1] = x.y; g[i][2] = x.z; g[i][3] = x.w;
        if constexpr (sizeof(T) == 4) {
          const float4 y = *reinterpret_cast<const float4*>(pr + j);
          p[i][0] = y.x; p[i][1] = y.y; p[i][2] = y.z; p[i][3] = y.w;
        } else {
          const uint2 y = *reinterpret_cast<const uint2*>(pr + j);
          p[i][0] = __uint_as_float(y.x << 16); p[i][1] = __uint_as_float(y.x & 0xffff0000u);
          p[i][2] = __uint_as_float(y.y << 16); p[i][3] = __uint_as_float(y.y & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) { p[i][e] = 0.f; g[i][e] = 0.f; }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (j + e > t) { p[i][e] = 0.f; g[i][e] = 0.f; }
        s = fmaf(p[i][e], g[i][e], s);
      }
    }
    const float dd = wave_sum(s);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = i * 256 + lane * 4;
      if (j < Tp) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = p[i][e] * (g[i][e] - dd) * scale;   // 0 past t (p = 0)
        if constexpr (sizeof(T) == 4) *reinterpret_cast<float4*>(out + j) = make_float4(o[0], o[1], o[2], o[3]);
        else *reinterpret_cast<uint2*>(out + j) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
      }
    }
  } else {
    float s = 0.f;
    for (int j = lane; j <= t; j += 64) s = fmaf(to_f32(pr[j]), gr[j], s);
    const float dd = wave_sum(s);
    for (int j = lane; j < Tp; j += 64)
      out[j] = from_f32<T>(j <= t ? to_f32(pr[j]) * (gr[j] - dd) * scale : 0.f);
  }
}

// Dv[(b H + h) T + t] = sum_d dO[b, t, h D + d] O[b, t, h D + d]: one wave per
// (b, t, h), whose D-element slices of dO and O are contiguous.  This is
// sum_j P[t, j] dP[t, j] (O = P U, dP = dO U^T), the term the softmax's
// backward subtracts.
template <typename T>
__global__ void __launch_bounds__(256) attn_bwd_rowdot_kernel(const float* __restrict__ dout, const T* __restrict__ o,
                                                              float* __restrict__ Dv, int B, int H, int Tn, int D) {
  const int lane = threadIdx.x & 63;
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, t, h), h fastest
  if (r >= (long long)B * Tn * H) return;
  const long long bt = r / H;
  const int h = (int)(r - bt * H);
  const int b = (int)(bt / Tn), t = (int)(bt - (long long)b * Tn);
  const long long base = bt * H * D + (long long)h * D;
  float s = 0.f;
  for (int d = lane; d < D; d += 64) s = fmaf(dout[base + d], to_f32(o[base + d]), s);
  s = wave_sum(s);
  if (lane == 0) Dv[((long long)b * H + h) * Tn + t] = s;
}

// bf16 form for D = 64: 16 lanes per (b, t, h) row, four elements each
// (16-byte dO and 8-byte O loads), four rows per wave, sums over the 16-lane
// group by butterfly exchanges.
__global__ void __launch_bounds__(256) attn_bwd_rowdot64_kernel(const float* __restrict__ dout,
                                                                const bf16* __restrict__ o, float* __restrict__ Dv,
                                                                int B, int H, int Tn) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const long long r = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);   // (b, t, h)
  const bool ok = r < (long long)B * Tn * H;
  float s = 0.f;
  long long bt = 0;
  int h = 0;
  if (ok) {
    bt = r / H;
    h = (int)(r - bt * H);
    const long long base = bt * H * 64 + (long long)h * 64 + sub * 4;
    const float4 d = *reinterpret_cast<const float4*>(dout + base);
    const uint2 w = *reinterpret_cast<const uint2*>(o + base);
    s = d.x * __uint_as_float(w.x << 16) + d.y * __uint_as_float(w.x & 0xffff0000u) +
        d.z * __uint_as_float(w.y << 16) + d.w * __uint_as_float(w.y & 0xffff0000u);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (ok && sub == 0) {
    const int b = (int)(bt / Tn), t = (int)(bt - (long long)b * Tn);
    Dv[((long long)b * H + h) * Tn + t] = s;
  }
}

template <typename T>
static hipError_t attn_bwd_t(const T* q, const T* k, const T* u, const float* dout, float* dqkv, int B, int H,
                             int Tn, int D, const AttnBwdWs& w, hipStream_t st) {
  const int Z = B * H, C = H * D, Tp = w.Tp;
  const float scale = (float)(1.0 / std::sqrt((double)D));
  const int dt = sizeof(T) == 2 ? 1 : 0;
  const long long hT = (long long)Tn * D, hTT = (long long)Tn * Tp, hDT = (long long)D * Tp;
  T* P = static_cast<T*>(w.P);
  T* PT = static_cast<T*>(w.PT);
  T* dS = static_cast<T*>(w.dS);
  T* dST = static_cast<T*>(w.dST);
  T* doc = static_cast<T*>(w.doc);
  T* dOT = static_cast<T*>(w.dOT);
  T* KT = static_cast<T*>(w.KT);
  T* QT = static_cast<T*>(w.QT);
  const int rows_blocks = (int)(((long long)Z * Tn + 3) / 4);
  GPT_BWD_TRY(launch_cast_rows(dt, dout, (long long)B * Tn * C, doc, st));
  if (sizeof(T) == 2 && w.lse2 != nullptr && w.o != nullptr && w.Dv != nullptr) {
    // fused: P^T straight from the score product with the forward's
    // log-sum-exp (P itself is not needed); dS and dS^T straight from the dP
    // product
    const int rows = B * Tn * H;
    if (D == 64 && ((uintptr_t)dout & 15) == 0 && ((uintptr_t)w.o & 7) == 0)
      hipLaunchKernelGGL(attn_bwd_rowdot64_kernel, dim3((rows + 15) / 16), dim3(256), 0, st, dout,
                         static_cast<const bf16*>(w.o), w.Dv, B, H, Tn);
    else
      hipLaunchKernelGGL(attn_bwd_rowdot_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, st, dout,
                         static_cast<const T*>(w.o), w.Dv, B, H, Tn, D);
    GPT_BWD_TRY(launch_attn_scores_bwd(0, q, D, k, D, Tn, D, BatchStrides{H * hT, hT, H * hT, hT, 0, 0, H}, Z,
                                       w.lse2, nullptr, nullptr, PT, Tp, scale * 1.4426950408889634f, st));
    // dU = P^T dO
    transpose_batched<T, T>(doc, C, (long long)Tn * C, D, H, Tn, D, dOT, Tp, hDT, Tp, Z, st);
    GPT_BWD_TRY(launch_gemm_batched(dt, PT, Tp, dOT, Tp, Tn, D, Tp, dqkv + 2 * C, 3 * C,
                                    BatchStrides{H * hTT, hTT, H * hDT, hDT, (long long)Tn * 3 * C, D, H}, Z, st, 2));
    GPT_BWD_TRY(launch_attn_scores_bwd(1, doc, C, u, D, Tn, D, BatchStrides{(long long)Tn * C, D, H * hT, hT, 0, 0, H},
                                       Z, w.Dv, PT, dS, dST, Tp, scale, st));
    // dQ = dS K, dK = dS^T Q
    transpose_batched<T, T>(k, D, H * hT, hT, H, Tn, D, KT, Tp, hDT, Tp, Z, st);
    GPT_BWD_TRY(launch_gemm_batched(dt, dS, Tp, KT, Tp, Tn, D, Tp, dqkv, 3 * C,
                                    BatchStrides{H * hTT, hTT, H * hDT, hDT, (long long)Tn * 3 * C, D, H}, Z, st, 3));
    transpose_batched<T, T>(q, D, H * hT, hT, H, Tn, D, QT, Tp, hDT, Tp, Z, st);
    GPT_BWD_TRY(launch_gemm_batched(dt, dST, Tp, QT, Tp, Tn, D, Tp, dqkv + C, 3 * C,
                                    BatchStrides{H * hTT, hTT, H * hDT, hDT, (long long)Tn * 3 * C, D, H}, Z, st, 2));
    return hipGetLastError();
  }
  // S = Q K^T
  GPT_BWD_TRY(launch_gemm_batched(dt, q, D, k, D, Tn, Tn, D, w.S, Tp,
                                  BatchStrides{H * hT, hT, H * hT, hT, H * hTT, hTT, H}, Z, st, 1));
  if (Tp <= 1024)
    hipLaunchKernelGGL((attn_bwd_softmax_kernel<T, 4>), dim3(rows_blocks), dim3(256), 0, st, (const float*)w.S, P, Z,
                       Tn, Tp, scale);
  else
    hipLaunchKernelGGL((attn_bwd_softmax_kernel<T, 0>), dim3(rows_blocks), dim3(256), 0, st, (const float*)w.S, P, Z,
                       Tn, Tp, scale);
  // dU = P^T dO
  transpose_batched<T, T>(P, Tp, H * hTT, hTT, H, Tn, Tn, PT, Tp, hTT, Tp, Z, st);
  transpose_batched<T, T>(doc, C, (long long)Tn * C, D, H, Tn, D, dOT, Tp, hDT, Tp, Z, st);
  GPT_BWD_TRY(launch_gemm_batched(dt, PT, Tp, dOT, Tp, Tn, D, Tp, dqkv + 2 * C, 3 * C,
                                  BatchStrides{H * hTT, hTT, H * hDT, hDT, (long long)Tn * 3 * C, D, H}, Z, st, 2));
  // dP = dO U^T (into the S buffer), dS
  GPT_BWD_TRY(launch_gemm_batched(dt, doc, C, u, D, Tn, Tn, D, w.S, Tp,
                                  BatchStrides{(long long)Tn * C, D, H * hT, hT, H * hTT, hTT, H}, Z, st, 1));
  if (Tp <= 1024)
    hipLaunchKernelGGL((attn_bwd_ds_kernel<T, 4>), dim3(rows_blocks), dim3(256), 0, st, (const T*)P,
                       (const float*)w.S, dS, Z, Tn, Tp, scale);
  else
    hipLaunchKernelGGL((attn_bwd_ds_kernel<T, 0>), dim3(rows_blocks), dim3(256), 0, st, (const T*)P,
                       (const float*)w.S, dS, Z, Tn, Tp, scale);
  // dQ = dS K, dK = dS^T Q
  transpose_batched<T, T>(k, D, H * hT, hT, H, Tn, D, KT, Tp, hDT, Tp, Z, st);
  GPT_BWD_TRY(launch_gemm_batched(dt, dS, Tp, KT, Tp, Tn, D, Tp, dqkv, 3 * C,
                                  BatchStrides{H * hTT, hTT, H * hDT, hDT, (long long)Tn * 3 * C, D, H}, Z, st, 3));
  transpose_batched<T, T>(dS, Tp, H * hTT, hTT, H, Tn, Tn, dST, Tp, hTT, Tp, Z, st);
  transpose_batched<T, T>(q, D, H * hT, hT, H, Tn, D, QT, Tp, hDT, Tp, Z, st);
  GPT_BWD_TRY(launch_gemm_batched(dt, dST, Tp, QT, Tp, Tn, D, Tp, dqkv + C, 3 * C,
                                  BatchStrides{H * hTT, hTT, H * hDT, hDT, (long long)Tn * 3 * C, D, H}, Z, st, 2));
  return hipGetLastError();
}

hipError_t launch_attention_backward(int dtype, const void* q, const void* k, const void* u, const float* dout,
                                     float* dqkv, int B, int H, int T, int D, const AttnBwdWs& w, hipStream_t st) {
  if (dtype == 0)
    return attn_bwd_t<float>((const float*)q, (const float*)k, (const float*)u, dout, dqkv, B, H, T, D, w, st);
  return attn_bwd_t<bf16>((const bf16*)q, (const bf16*)k, (const bf16*)u, dout, dqkv, B, H, T, D, w, st);
}

// out (+)= part[0] + part[1] + ... + part[S-1] (slice order), four elements
// per thread when n is a multiple of 4 (the slices then stay 16-byte aligned)
template <bool ACC, int W>
__global__ void __launch_bounds__(256) add_partials_kernel(float* __restrict__ out, const float* __restrict__ part,
                                                           long long n, int S) {
  typedef typename std::conditional<W == 4, float4, float>::type V;
  const long long nv = n / W;
  V* o = reinterpret_cast<V*>(out);
  const V* p = reinterpret_cast<const V*>(part);
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < nv; i += (long long)gridDim.x * 256) {
    V s = p[i];
    for (int z = 1; z < S; ++z) {
      const V t = p[z * nv + i];
      if constexpr (W == 4) {
        s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
      } else {
        s += t;
      }
    }
    if constexpr (ACC) {
      const V a = o[i];
      if constexpr (W == 4) {
        s.x = a.x + s.x; s.y = a.y + s.y; s.z = a.z + s.z; s.w = a.w + s.w;
      } else {
        s = a + s;
      }
    }
    o[i] = s;
  }
}

hipError_t launch_add_partials(float* out, const float* part, long long n, int S, hipStream_t st, int accumulate) {
  if (n <= 0) return hipSuccess;
  const bool v4 = n % 4 == 0 && ((uintptr_t)out & 15) == 0 && ((uintptr_t)part & 15) == 0;
  const long long nv = v4 ? n / 4 : n;
  if (v4 && accumulate)
    hipLaunchKernelGGL((add_partials_kernel<true, 4>), dim3(grid_for(nv)), dim3(256), 0, st, out, part, n, S);
  else if (v4)
    hipLaunchKernelGGL((add_partials_kernel<false, 4>), dim3(grid_for(nv)), dim3(256), 0, st, out, part, n, S);
  else if (accumulate)
    hipLaunchKernelGGL((add_partials_kernel<true, 1>), dim3(grid_for(nv)), dim3(256), 0, st, out, part, n, S);
  else
    hipLaunchKernelGGL((add_partials_kernel<false, 1>), dim3(grid_for(nv)), dim3(256), 0, st, out, part, n, S);
  return hipGetLastError();
}

hipError_t launch_act_fwd(int dtype, const void* u, long long n, int act, void* h, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL(act_fwd_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, (const float*)u, n, act, (float*)h);
  else if (n % 4 == 0 && ((uintptr_t)u & 7) == 0 && ((uintptr_t)h & 7) == 0)
    hipLaunchKernelGGL(act_fwd4_kernel, dim3(grid_for(n / 4)), dim3(256), 0, st, (const uint2*)u, n / 4, act,
                       (uint2*)h);
  else
    hipLaunchKernelGGL(act_fwd_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, st, (const bf16*)u, n, act, (bf16*)h);
  return hipGetLastError();
}

hipError_t launch_act_bwd(int dtype, float* d, const void* u, long long n, int act, void* dc, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL(act_bwd_kernel<float>, dim3(grid_for(n)), dim3(256), 0, st, d, (const float*)u, n, act,
                       (float*)dc);
  else if (n % 4 == 0 && ((uintptr_t)d & 15) == 0 && ((uintptr_t)u & 7) == 0 && ((uintptr_t)dc & 7) == 0)
    hipLaunchKernelGGL(act_bwd4_kernel, dim3(grid_for(n / 4)), dim3(256), 0, st, (float4*)d, (const uint2*)u, n / 4,
                       act, (uint2*)dc);
  else
    hipLaunchKernelGGL(act_bwd_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, st, d, (const bf16*)u, n, act,
                       (bf16*)dc);
  return hipGetLastError();
}

hipError_t launch_colsum(int M, int N, const float* a, float* part, float* out, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (N % 4 == 0 && ((uintptr_t)a & 15) == 0) {
    const int nch = colsum_chunks(M);
    hipLaunchKernelGGL(colsum_part4_kernel, dim3((N + 255) / 256, nch), dim3(256), 0, st, M, N, a, part);
    hipLaunchKernelGGL(colsum_final4_kernel, dim3((N + 63) / 64), dim3(256), 0, st, N, nch, (const float*)part, out);
    return hipGetLastError();
  }
  const int nch = ln_bwd_chunks(M);
  hipLaunchKernelGGL(colsum_part_kernel, dim3((N + 63) / 64, nch), dim3(256), 0, st, M, N, a, part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((N + 255) / 256), dim3(256), 0, st, N, nch, (const float*)part, out);
  return hipGetLastError();
}

}  // namespace gptmi
