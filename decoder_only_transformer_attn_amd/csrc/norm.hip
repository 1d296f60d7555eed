// Embedding gather and LayerNorm kernels.
//
// Token + position embedding: x[b,t,:] = E[idx[b,t],:] + P[t,:]  ("第 25 章 从小
// GPT 到 GPT-2" §25.1; "预训练一个 Mini GPT" 第1步).  LayerNorm over the C
// channels with biased variance and eps inside the square root ("预训练一个
// Mini GPT" 第4步; "GPT-1学习笔记" §3.2).  RMSNorm (LLaMA-style models,
// "02 GPT 架构" §6.1; "GPT-1学习笔记" §10.2): no mean centring and no bias,
// g * x / sqrt(mean(x^2) + eps); those models also have no position table.
//
// One wavefront per row: the row lives in registers (C / 64 values per lane),
// mean and variance are two passes over registers with wavefront reductions,
// so x is read from HBM once and the normalised row written once.  HBM-bound:
// per row the kernel moves C*4 bytes in (fp32 residual) and C*sizeof(T) out.
#include "common.h"
#include "kernels.h"

namespace gptmi {

// Four consecutive elements as one 16-byte (fp32) or 8-byte (bf16) access.
__device__ __forceinline__ void load4(const float* p, float (&o)[4]) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w;
}
__device__ __forceinline__ void load4(const bf16* p, float (&o)[4]) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(q.x << 16); o[1] = __uint_as_float(q.x & 0xffff0000u);
  o[2] = __uint_as_float(q.y << 16); o[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16* p, const float (&v)[4]) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// NCH = number of 4-float chunks per lane; C <= 256 * NCH.
template <typename T, int NCH, bool EMBED>
__global__ void __launch_bounds__(256) ln_rows_kernel(LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (EMBED && a.zero)   // the pass's first kernel clears the split-K counters of the products after it
    for (int i = blockIdx.x * 256 + threadIdx.x; i < a.zero_n; i += gridDim.x * 256) a.zero[i] = 0;
  if (row >= a.M) return;
  const int C = a.C;
  const T* __restrict__ g = reinterpret_cast<const T*>(a.g);
  const T* __restrict__ bta = reinterpret_cast<const T*>(a.b);
  float v[NCH][4];
  if (EMBED) {
    float* __restrict__ xr = a.x + (size_t)row * C;
    int tok = a.idx[row];
    tok = tok < 0 ? 0 : (tok >= a.vocab ? a.vocab - 1 : tok);  // ids outside [0,V) violate the contract; never read out of bounds
    int t = row % a.T_seq + (a.pos ? *a.pos : 0);
    t = t < 0 ? 0 : (t < a.ctx ? t : a.ctx - 1);                // positions outside the table violate the contract
    const T* __restrict__ er = reinterpret_cast<const T*>(a.wte) + (size_t)tok * C;
    const T* __restrict__ pr = a.wpe ? reinterpret_cast<const T*>(a.wpe) + (size_t)t * C : nullptr;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = (j * 64 + lane) * 4;
      if (c < C) {
        float e4[4], p4[4] = {0.f, 0.f, 0.f, 0.f};
        load4(er + c, e4);
        if (pr) load4(pr + c, p4);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][e] = e4[e] + p4[e];
        store4(xr + c, v[j]);
      }
    }
  } else {
    const float* __restrict__ xr = a.x + (size_t)(row * a.in_mul + a.in_add) * C;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = (j * 64 + lane) * 4;
      if (c < C) load4(xr + c, v[j]);
    }
  }
  T* __restrict__ orow = reinterpret_cast<T*>(a.out) + (size_t)row * C;
  if (EMBED && a.ident) {   // post-LN model: the first block reads the embedding itself
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = (j * 64 + lane) * 4;
      if (c < C) store4(orow + c, v[j]);
    }
    return;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
    if ((j * 64 + lane) * 4 < C) s += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
  const float mean = a.rms ? 0.f : wave_sum(s) / (float)C;   // (uniform branch)
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
    if ((j * 64 + lane) * 4 < C)
#pragma unroll
      for (int e = 0; e < 4; ++e) { float d = v[j][e] - mean; s2 += d * d; }
  const float var = wave_sum(s2) / (float)C;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  float* __restrict__ xw = (!EMBED && a.write_x) ? a.x + (size_t)(row * a.in_mul + a.in_add) * C : nullptr;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c < C) {
      float g4[4], b4[4] = {0.f, 0.f, 0.f, 0.f}, o4[4];
      load4(g + c, g4);
      if (bta) load4(bta + c, b4);
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (v[j][e] - mean) * rstd * g4[e] + b4[e];
      store4(orow + c, o4);
      if (xw) store4(xw + c, o4);   // post-LN: the normalised row is the new residual stream
    }
  }
}

template <typename T, bool EMBED>
static hipError_t launch_ln_t(const LnArgs& a, hipStream_t st) {
  dim3 grid((a.M + 3) / 4), block(256);
  if (a.C <= 256)
    hipLaunchKernelGGL((ln_rows_kernel<T, 1, EMBED>), grid, block, 0, st, a);
  else if (a.C <= 512)
    hipLaunchKernelGGL((ln_rows_kernel<T, 2, EMBED>), grid, block, 0, st, a);
  else if (a.C <= 1024)
    hipLaunchKernelGGL((ln_rows_kernel<T, 4, EMBED>), grid, block, 0, st, a);
  else if (a.C <= 2048)
    hipLaunchKernelGGL((ln_rows_kernel<T, 8, EMBED>), grid, block, 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_embed_ln(int dtype, const LnArgs& a, hipStream_t st) {
  if (dtype == 0) return launch_ln_t<float, true>(a, st);
  return launch_ln_t<bf16, true>(a, st);
}

hipError_t launch_layernorm(int dtype, const LnArgs& a, hipStream_t st) {
  if (dtype == 0) return launch_ln_t<float, false>(a, st);
  return launch_ln_t<bf16, false>(a, st);
}

}  // namespace gptmi
