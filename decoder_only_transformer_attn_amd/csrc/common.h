// Shared device helpers for the gfx950 kernels: storage types, bf16 rounding,
// MFMA traits and wavefront reductions.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptmi {

typedef uint16_t bf16;  // storage of a bfloat16 value (upper half of an fp32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ bf16 f32_to_bf16(float f) { return __builtin_bit_cast(bf16, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the hardware v_exp_f32 alone (results below 2^-126 flush to zero,
// which no softmax or GELU term here can notice).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return f32_to_bf16(v); }

// 32x32 MFMA traits.  One instruction multiplies a 32 x KPI slice of A (rows
// m) by a KPI x 32 slice of B (columns n).  Lane l holds KPL consecutive k
// values of row (l % 32) of A and of column (l % 32) of B, at k offset
// (l / 32) * KPL; the 32x32 fp32 result is spread over 16 registers per lane:
// register r of lane l holds row (r/4)*8 + (l/32)*4 + (r%4), column l % 32.
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;    // k values per lane per instruction
  static constexpr int KPI = 16;   // k extent of one instruction
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // KPL consecutive values starting at p (16-byte aligned).
  static __device__ __forceinline__ frag load(const bf16* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KPI = 2;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
};

typedef __attribute__((address_space(3))) void lds_void;
// LDS byte and 16-byte types: stage pointers carry the LDS address space in
// their type, so fragment reads are ds_read instructions by construction and
// never depend on the compiler inferring where a generic pointer points.
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) int lds_int;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// The LDS view of a __shared__ array.
template <typename T> __device__ __forceinline__ lds_char* as_lds(T* p) { return (lds_char*)p; }

// 16-, 8- and 4-byte LDS accesses through LDS-typed pointers.
__device__ __forceinline__ uint4 lds_ld16(const lds_char* p) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p));
}
__device__ __forceinline__ bf16x8 lds_frag(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}
__device__ __forceinline__ uint2 lds_ld8(const lds_char* p) {
  return __builtin_bit_cast(uint2, *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(p));
}
__device__ __forceinline__ void lds_st8(lds_char* p, uint2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2_t*>(p) = __builtin_bit_cast(u32x2_t, v);
}
__device__ __forceinline__ void lds_st4(lds_char* p, uint32_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(p) = v;
}

// Row index (within a 32x32 tile) of accumulator register r for lane l.
// Buffer resource over [base, base + bytes): loads beyond `bytes` return zero,
// which handles the tails of a tile without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// An offset past every resource this code builds (at most 2^31 bytes): reads zero.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// The value of the neighbouring lane l ^ 1, by a DPP quad permutation
// [1, 0, 3, 2] inside the VALU instruction (no LDS round trip, unlike a
// general lane shuffle).
__device__ __forceinline__ float xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Reductions over the 32 lanes of one half-wave (lanes sharing l / 32).
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace gptmi
