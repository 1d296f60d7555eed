// Causal multi-head attention, flash style.
//
// Per (sequence b, head h):  O = softmax(Q K^T / sqrt(D) + M) U  with M[t,s] =
// -inf for s > t ("第 25 章 从小 GPT 到 GPT-2" §25.2; "预训练一个 Mini GPT"
// 注意力).  The T x T score matrix is never stored: K/U tiles are staged in
// LDS and the softmax is accumulated online with a running row maximum and
// row sum, the tiling + online-softmax reordering of the same sums that the
// GPT-1 notes (§10.2) describe for FlashAttention.
//
// MI355X mapping.  The kernel computes S^T = K Q^T with 32x32 MFMA tiles, so
// that each lane owns one query column: the row statistics need a single
// cross-lane exchange (lanes l and l^32), and the probabilities P^T sit in
// registers already in the B-operand layout of the second product
// O^T = U^T P^T.  U is stored [B,H,T,D] like K and written transposed,
// U^T [D, keys], when its tile is staged into LDS, so the A operand of that
// product is a contiguous LDS read.  Scores are scaled
// by log2(e)/sqrt(D) and exponentiated with exp2.  Key tiles entirely above
// the diagonal are skipped; only diagonal tiles evaluate the mask.
#include "common.h"
#include "kernels.h"

namespace gptmi {

template <typename T> struct VtFrag;

// bf16: instruction hh of a 32-key sub-tile consumes accumulator registers
// r = 8hh .. 8hh+7 of the S^T tile, i.e. keys 16hh + 4g + {0..3} and
// 16hh + 8 + 4g + {0..3} for lane group g = lane / 32.
template <> struct VtFrag<bf16> {
  static constexpr int NI = 2;  // instructions per 32 keys
  static __device__ __forceinline__ bf16x8 load(const bf16* row, int hh, int g) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + 16 * hh + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + 16 * hh + 8 + 4 * g);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
  static __device__ __forceinline__ bf16x8 pack(const f32x16& p, int hh) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = uint32_t(f32_to_bf16(p[8 * hh + 2 * e])) | (uint32_t(f32_to_bf16(p[8 * hh + 2 * e + 1])) << 16);
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
};

// fp32: instruction hh (0..15) consumes register r = hh: key (hh/4)*8 + 4g + hh%4.
template <> struct VtFrag<float> {
  static constexpr int NI = 16;
  static __device__ __forceinline__ float load(const float* row, int hh, int g) {
    return row[(hh >> 2) * 8 + 4 * g + (hh & 3)];
  }
  static __device__ __forceinline__ float pack(const f32x16& p, int hh) { return p[hh]; }
};

// Block: 4 waves, 32 queries each (BQ = 128); key/value tiles of BKV keys.
template <typename T, int DP, int BKV>
__global__ void __launch_bounds__(256) attn_fwd_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  constexpr int BQ = 128;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LDKS = DP + VEC;    // padded LDS row of K (elements)
  constexpr int LDVS = BKV + VEC;   // padded LDS row of U^T
  constexpr int NDI = DP / MF::KPI; // MFMA k steps over the head dim
  constexpr int NDT = DP / 32;      // 32-row d tiles of O^T
  constexpr int NST = BKV / 32;     // 32-key sub-tiles per KV tile
  __shared__ __align__(16) T sK[BKV * LDKS];
  __shared__ __align__(16) T sV[DP * LDVS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int nqt = gridDim.x;
  const int qt = nqt - 1 - blockIdx.x;  // longest query tiles first
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh - b * a.H;
  const int q0 = qt * BQ;
  const int qw0 = q0 + wave * 32;
  const int qcol = qw0 + (lane & 31);
  const int T_seq = a.T_seq, D = a.D;

  const T* Q = reinterpret_cast<const T*>(a.q) + (long long)bh * a.q_bh;
  const T* K = reinterpret_cast<const T*>(a.k) + (long long)bh * a.k_bh;
  const T* U = reinterpret_cast<const T*>(a.v) + (long long)bh * a.v_bh;

  // Q^T fragments (B operand) for this lane's query column.
  typename MF::frag qf[NDI];
#pragma unroll
  for (int i = 0; i < NDI; ++i) {
    const int d0 = i * MF::KPI + g * MF::KPL;
    if (qcol < T_seq && d0 < D) qf[i] = MF::load(Q + (long long)qcol * D + d0);
    else qf[i] = typename MF::frag{};
  }

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = min(T_seq, q0 + BQ);  // keys [0, kv_end) can be visible to this block
  for (int kb = 0; kb < kv_end; kb += BKV) {
    // stage K [BKV][DP] and U^T [DP][BKV]; rows/cols outside the sequence are zero
    for (int ch = tid; ch < BKV * (DP / VEC); ch += 256) {
      const int row = ch / (DP / VEC), dc = (ch % (DP / VEC)) * VEC;
      const int key = kb + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < T_seq && dc < D) v = *reinterpret_cast<const uint4*>(K + (long long)key * D + dc);
      *reinterpret_cast<uint4*>(sK + row * LDKS + dc) = v;
    }
    // U: each item is two consecutive keys x VEC head columns, written
    // transposed as VEC pairs (key, key + 1) of row d of U^T
    for (int ch = tid; ch < (BKV / 2) * (DP / VEC); ch += 256) {
      const int kp = (ch / (DP / VEC)) * 2, dc = (ch % (DP / VEC)) * VEC;
      const int key = kb + kp;
      T u0[VEC], u1[VEC];
      *reinterpret_cast<uint4*>(u0) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(u1) = make_uint4(0, 0, 0, 0);
      if (dc < D) {
        if (key < T_seq) *reinterpret_cast<uint4*>(u0) = *reinterpret_cast<const uint4*>(U + (long long)key * D + dc);
        if (key + 1 < T_seq)
          *reinterpret_cast<uint4*>(u1) = *reinterpret_cast<const uint4*>(U + (long long)(key + 1) * D + dc);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        T* dst = sV + (dc + e) * LDVS + kp;   // kp and LDVS even: pair-aligned
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint32_t*>(dst) = uint32_t(u0[e]) | (uint32_t(u1[e]) << 16);
        else
          *reinterpret_cast<float2*>(dst) = make_float2(u0[e], u1[e]);
      }
    }
    __syncthreads();

    if (kb <= qw0 + 31) {  // otherwise every key of this tile is in this wave's future
      f32x16 s[NST];
#pragma unroll
      for (int st = 0; st < NST; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
        const T* krow = sK + (st * 32 + (lane & 31)) * LDKS + g * MF::KPL;
#pragma unroll
        for (int i = 0; i < NDI; ++i) s[st] = MF::mma(MF::load(krow + i * MF::KPI), qf[i], s[st]);
      }
      const bool diag = kb + BKV - 1 > qw0;
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[st][r] * a.scale_log2;
          if (diag && kb + st * 32 + acc_row(r, lane) > qcol) v = -INFINITY;
          s[st][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[st][r] - m_new);
          s[st][r] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int hh = 0; hh < VtFrag<T>::NI; ++hh) {
          const auto pb = VtFrag<T>::pack(s[st], hh);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const T* vrow = sV + (dt * 32 + (lane & 31)) * LDVS + st * 32;
            acc[dt] = MF::mma(VtFrag<T>::load(vrow, hh, g), pb, acc[dt]);
          }
        }
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qcol < T_seq) {
    T* orow = reinterpret_cast<T*>(a.o) + ((long long)b * T_seq + qcol) * a.o_ld + h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = dt * 32 + acc_row(r, lane);
        if (d < D) orow[d] = from_f32<T>(acc[dt][r] * inv);
      }
  }
}

template <typename T>
static hipError_t attn_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid((a.T_seq + 127) / 128, a.B * a.H), block(256);
  if (a.D <= 32)
    hipLaunchKernelGGL((attn_fwd_kernel<T, 32, 64>), grid, block, 0, st, a);
  else if (a.D <= 64)
    hipLaunchKernelGGL((attn_fwd_kernel<T, 64, 64>), grid, block, 0, st, a);
  else if (a.D <= 128)
    hipLaunchKernelGGL((attn_fwd_kernel<T, 128, 64>), grid, block, 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t st) {
  if (dtype == 0) return attn_t<float>(a, st);
  return attn_t<bf16>(a, st);
}

}  // namespace gptmi
