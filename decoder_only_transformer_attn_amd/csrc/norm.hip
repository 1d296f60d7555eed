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

// Four raw elements (8 bytes of bf16 or 16 of fp32), converted at use.
template <typename T> struct Raw4 { typedef uint2 type; };
template <> struct Raw4<float> { typedef float4 type; };
__device__ __forceinline__ void unpack4(const uint2& q, float (&o)[4]) {
  o[0] = __uint_as_float(q.x << 16); o[1] = __uint_as_float(q.x & 0xffff0000u);
  o[2] = __uint_as_float(q.y << 16); o[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ __forceinline__ void unpack4(const float4& q, float (&o)[4]) { o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w; }

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
  // gain and bias requested with the row, not after the reductions
  typedef typename Raw4<T>::type R;
  R graw[NCH], braw[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (j * 64 + lane) * 4;
    graw[j] = R{}; braw[j] = R{};
    if (c < C && !(EMBED && a.ident)) {
      graw[j] = *reinterpret_cast<const R*>(g + c);
      if (bta) braw[j] = *reinterpret_cast<const R*>(bta + c);
    }
  }
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
      float g4[4], b4[4], o4[4];
      unpack4(graw[j], g4);
      unpack4(braw[j], b4);   // zero without a bias
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (v[j][e] - mean) * rstd * g4[e] + b4[e];
      store4(orow + c, o4);
      if (xw) store4(xw + c, o4);   // post-LN: the normalised row is the new residual stream
    }
  }
}

// Residual update of a K-split product and the LayerNorm after it, one row
// per 64-thread block: x[row] += (sum over s in order of part[s][row]) +
// bias, in fp32 (the same x + (v + b) form as the products' own residual
// epilogue), the new row written back, then normalised exactly as
// ln_rows_kernel does.  NS = the number of slices (all their loads are issued
// before the first add).
// Block j >= M of the residual LayerNorm: share j of the prefetch ranges
// (range 0's blocks first), 16 bytes per lane and instruction, every load
// issued before the first use.
constexpr int PF_LOADS = 48;   // 48 KB per block
__device__ __forceinline__ void prefetch_share(const LnArgs& a, int j) {
  const int r = j < a.pf_blocks[0] ? 0 : 1;
  const int share = r == 0 ? j : j - a.pf_blocks[0];
  const char* base = static_cast<const char*>(a.pf[r]);
  const size_t nb = a.pf_bytes[r] & ~(size_t)15;
  const size_t off = (size_t)share * PF_LOADS * 1024 + (size_t)threadIdx.x * 16;
  uint4 v[PF_LOADS];
#pragma unroll
  for (int i = 0; i < PF_LOADS; ++i) {
    const size_t o = off + (size_t)i * 1024;
    v[i] = o < nb ? *reinterpret_cast<const uint4*>(base + o) : make_uint4(0, 0, 0, 0);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < PF_LOADS; ++i) acc ^= v[i].x ^ v[i].w;
  if (a.pf_sink) a.pf_sink[threadIdx.x] = acc;
}

template <int NCH, int NS>
__global__ void __launch_bounds__(64) resid_ln_kernel(LnArgs a) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  if (row >= a.M) {
    prefetch_share(a, row - a.M);
    return;
  }
  const int C = a.C;
  const bf16* __restrict__ g = reinterpret_cast<const bf16*>(a.g);
  const bf16* __restrict__ bta = reinterpret_cast<const bf16*>(a.b);
  const bf16* __restrict__ rb = reinterpret_cast<const bf16*>(a.rbias);
  float* __restrict__ xr = a.x + (size_t)row * C;
  float v[NCH][4], g4[NCH][4], gb4[NCH][4];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {   // gain and bias with the first loads, not after the reductions
    const int c = (j * 64 + lane) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) { g4[j][e] = 0.f; gb4[j][e] = 0.f; }
    if (c < C) {
      load4(g + c, g4[j]);
      if (bta) load4(bta + c, gb4[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c < C) {
      float x4[4], b4[4] = {0.f, 0.f, 0.f, 0.f}, p4[NS][4];
      load4(xr + c, x4);
      if (rb) load4(rb + c, b4);
#pragma unroll
      for (int s = 0; s < NS; ++s) load4(a.part + ((size_t)s * a.M + row) * C + c, p4[s]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t = p4[0][e];
#pragma unroll
        for (int s = 1; s < NS; ++s) t += p4[s][e];
        v[j][e] = x4[e] + (t + b4[e]);
      }
      store4(xr + c, v[j]);
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
  const float rstd = 1.0f / sqrtf(var + a.eps);
  bf16* __restrict__ orow = reinterpret_cast<bf16*>(a.out) + (size_t)row * C;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = (j * 64 + lane) * 4;
    if (c < C) {
      float o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (v[j][e] - mean) * rstd * g4[j][e] + gb4[j][e];
      store4(orow + c, o4);
    }
  }
}

template <int NCH>
static hipError_t launch_resid_ln_c(const LnArgs& a, hipStream_t st) {
  const dim3 grid(a.M + a.pf_blocks[0] + a.pf_blocks[1]), block(64);
  switch (a.nsplit) {
    case 1: hipLaunchKernelGGL((resid_ln_kernel<NCH, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((resid_ln_kernel<NCH, 2>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((resid_ln_kernel<NCH, 3>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((resid_ln_kernel<NCH, 4>), grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL((resid_ln_kernel<NCH, 6>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((resid_ln_kernel<NCH, 8>), grid, block, 0, st, a); break;
    case 12: hipLaunchKernelGGL((resid_ln_kernel<NCH, 12>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Prefetch blocks for nbytes of weights (48 KB each).
int resid_ln_prefetch_blocks(size_t nbytes) { return (int)((nbytes + PF_LOADS * 1024 - 1) / (PF_LOADS * 1024)); }

hipError_t launch_resid_layernorm(const LnArgs& a, hipStream_t st) {
  if (!a.part || !a.x || !a.out || !a.g || a.M <= 0 || a.C <= 0 || a.C % 4) return hipErrorInvalidValue;
  for (int r = 0; r < 2; ++r)   // each range: no blocks, or just enough to cover it
    if (a.pf_blocks[r] != (a.pf[r] ? resid_ln_prefetch_blocks(a.pf_bytes[r]) : 0)) return hipErrorInvalidValue;
  if (a.C <= 256) return launch_resid_ln_c<1>(a, st);
  if (a.C <= 512) return launch_resid_ln_c<2>(a, st);
  if (a.C <= 1024) return launch_resid_ln_c<4>(a, st);
  return hipErrorInvalidValue;
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
