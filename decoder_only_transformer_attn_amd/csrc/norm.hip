// Embedding gather and LayerNorm kernels.
//
// Token + position embedding: x[b,t,:] = E[idx[b,t],:] + P[t,:]  ("第 25 章 从小
// GPT 到 GPT-2" §25.1; "预训练一个 Mini GPT" 第1步).  LayerNorm over the C
// channels with biased variance and eps inside the square root ("预训练一个
// Mini GPT" 第4步; "GPT-1学习笔记" §3.2).
//
// One wavefront per row: the row lives in registers (C / 64 values per lane),
// mean and variance are two passes over registers with wavefront reductions,
// so x is read from HBM once and the normalised row written once.  HBM-bound:
// per row the kernel moves C*4 bytes in (fp32 residual) and C*sizeof(T) out.
#include "common.h"
#include "kernels.h"

namespace gptmi {

// NCH = number of 4-float chunks per lane; C <= 256 * NCH.
template <typename T, int NCH, bool EMBED>
__global__ void __launch_bounds__(256) ln_rows_kernel(
    int M, int C, int T_seq, float eps,
    const int32_t* __restrict__ idx, const T* __restrict__ wte, const T* __restrict__ wpe, int vocab,
    float* __restrict__ x,                 // [M, C] fp32 residual (written when EMBED, else read)
    const T* __restrict__ g, const T* __restrict__ b,
    T* __restrict__ out)                   // [M, C] normalised, compute dtype
{
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float v[NCH][4];
  float* xr = x + (size_t)row * C;
  if (EMBED) {
    int tok = idx[row];
    tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);  // ids outside [0,V) violate the contract; never read out of bounds
    const int t = row % T_seq;
    const T* er = wte + (size_t)tok * C;
    const T* pr = wpe + (size_t)t * C;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = (j * 64 + lane) * 4;
      if (c < C) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][e] = to_f32(er[c + e]) + to_f32(pr[c + e]);
        *reinterpret_cast<float4*>(xr + c) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = (j * 64 + lane) * 4;
      if (c < C) {
        float4 q = *reinterpret_cast<const float4*>(xr + c);
        v[j][0] = q.x; v[j][1] = q.y; v[j][2] = q.z; v[j][3] = q.w;
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
    if ((j * 64 + lane) * 4 < C) s += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  const float mean = wave_sum(s) / (float)C;
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
    if ((j * 64 + lane) * 4 < C)
#pragma unroll
      for (int e = 0; e < 4; ++e) { float d = v[j][e] - mean; s2 += d * d; }
  const float var = wave_sum(s2) / (float)C;
  const float rstd = 1.0f / sqrtf(var + eps);
  T* orow = out + (size_t)row * C;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c < C) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        orow[c + e] = from_f32<T>((v[j][e] - mean) * rstd * to_f32(g[c + e]) + to_f32(b[c + e]));
    }
  }
}

template <typename T, bool EMBED>
static hipError_t launch_ln_t(int M, int C, int T_seq, float eps, const int32_t* idx, const T* wte, const T* wpe,
                              int vocab, float* x, const T* g, const T* b, T* out, hipStream_t st) {
  dim3 grid((M + 3) / 4), block(256);
  if (C <= 256)
    hipLaunchKernelGGL((ln_rows_kernel<T, 1, EMBED>), grid, block, 0, st, M, C, T_seq, eps, idx, wte, wpe, vocab, x, g, b, out);
  else if (C <= 512)
    hipLaunchKernelGGL((ln_rows_kernel<T, 2, EMBED>), grid, block, 0, st, M, C, T_seq, eps, idx, wte, wpe, vocab, x, g, b, out);
  else if (C <= 1024)
    hipLaunchKernelGGL((ln_rows_kernel<T, 4, EMBED>), grid, block, 0, st, M, C, T_seq, eps, idx, wte, wpe, vocab, x, g, b, out);
  else if (C <= 2048)
    hipLaunchKernelGGL((ln_rows_kernel<T, 8, EMBED>), grid, block, 0, st, M, C, T_seq, eps, idx, wte, wpe, vocab, x, g, b, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_embed_ln(int dtype, int M, int C, int T_seq, float eps, const int32_t* idx, const void* wte,
                           const void* wpe, int vocab, float* x, const void* g, const void* b, void* out,
                           hipStream_t st) {
  if (dtype == 0)
    return launch_ln_t<float, true>(M, C, T_seq, eps, idx, (const float*)wte, (const float*)wpe, vocab, x,
                                    (const float*)g, (const float*)b, (float*)out, st);
  return launch_ln_t<bf16, true>(M, C, T_seq, eps, idx, (const bf16*)wte, (const bf16*)wpe, vocab, x,
                                 (const bf16*)g, (const bf16*)b, (bf16*)out, st);
}

hipError_t launch_layernorm(int dtype, int M, int C, float eps, const float* x, const void* g, const void* b,
                            void* out, hipStream_t st) {
  if (dtype == 0)
    return launch_ln_t<float, false>(M, C, 1, eps, nullptr, nullptr, nullptr, 0, const_cast<float*>(x),
                                     (const float*)g, (const float*)b, (float*)out, st);
  return launch_ln_t<bf16, false>(M, C, 1, eps, nullptr, nullptr, nullptr, 0, const_cast<float*>(x),
                                  (const bf16*)g, (const bf16*)b, (bf16*)out, st);
}

}  // namespace gptmi
