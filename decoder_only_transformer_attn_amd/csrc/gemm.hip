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
//   EpiQKV   : + bias, scatter Q -> [B,H,T,D], K -> [B,H,Tk,D], V -> V^T [B,H,D,Tk]
//   EpiResid : + bias, x += (fp32 residual stream)
//   EpiAct   : + bias, optional tanh-GELU, store in the output dtype
//   head     : optional logits store + per-(row, N-tile) softmax partials
//              (max, sum exp) and the target logit, all from fp32 accumulators.
#include "common.h"
#include "kernels.h"

namespace gptmi {

template <typename T, int BM, int BN, int BK, int WM, int WN>
struct GemmCfg {
  static constexpr int NWM = BM / WM, NWN = BN / WN;
  static constexpr int NT = NWM * NWN * WAVE;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int LDK = BK + VEC;                 // padded LDS row (elements)
  static constexpr int CPR = BK / VEC;                 // chunks per tile row
  static constexpr int A_PT = (BM * CPR) / NT;         // chunks per thread
  static constexpr int B_PT = (BN * CPR) / NT;
  static constexpr int SMEM_ELEMS = 2 * (BM + BN) * LDK;
  static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile/threads mismatch");
  static_assert(BK % Mfma<T>::KPI == 0, "BK must hold whole MFMA k steps");
};

// Main loop: acc[i][j] += A[m0 + wm*WM + 32i .., :] . W[n0 + wn*WN + 32j .., :]^T
template <typename T, int BM, int BN, int BK, int WM, int WN>
__device__ __forceinline__ void gemm_mainloop(const T* __restrict__ A, int lda, const T* __restrict__ W, int ldw,
                                              int M, int N, int K, int m0, int n0, T* smem,
                                              f32x16 (&acc)[WM / 32][WN / 32]) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  typedef Mfma<T> MF;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  T* sA = smem;                       // [2][BM][LDK]
  T* sB = smem + 2 * BM * G::LDK;     // [2][BN][LDK]

#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[G::A_PT], rb[G::B_PT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int c = 0; c < G::A_PT; ++c) {
      const int ch = tid + c * G::NT, row = ch / G::CPR, kc = (ch % G::CPR) * G::VEC;
      const int gm = m0 + row, gk = k0 + kc;
      ra[c] = (gm < M && gk < K) ? *reinterpret_cast<const uint4*>(A + (size_t)gm * lda + gk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < G::B_PT; ++c) {
      const int ch = tid + c * G::NT, row = ch / G::CPR, kc = (ch % G::CPR) * G::VEC;
      const int gn = n0 + row, gk = k0 + kc;
      rb[c] = (gn < N && gk < K) ? *reinterpret_cast<const uint4*>(W + (size_t)gn * ldw + gk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < G::A_PT; ++c) {
      const int ch = tid + c * G::NT, row = ch / G::CPR, kc = (ch % G::CPR) * G::VEC;
      *reinterpret_cast<uint4*>(sA + (buf * BM + row) * G::LDK + kc) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < G::B_PT; ++c) {
      const int ch = tid + c * G::NT, row = ch / G::CPR, kc = (ch % G::CPR) * G::VEC;
      *reinterpret_cast<uint4*>(sB + (buf * BN + row) * G::LDK + kc) = rb[c];
    }
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * MF::KPL;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const T* a_base = sA + (cur * BM + wm * WM + lrow) * G::LDK + lk;
    const T* b_base = sB + (cur * BN + wn * WN + lrow) * G::LDK + lk;
#pragma unroll
    for (int kk = 0; kk < BK; kk += MF::KPI) {
      typename MF::frag af[G::TM], bfr[G::TN];
#pragma unroll
      for (int i = 0; i < G::TM; ++i) af[i] = MF::load(a_base + i * 32 * G::LDK + kk);
#pragma unroll
      for (int j = 0; j < G::TN; ++j) bfr[j] = MF::load(b_base + j * 32 * G::LDK + kk);
#pragma unroll
      for (int i = 0; i < G::TM; ++i)
#pragma unroll
        for (int j = 0; j < G::TN; ++j) acc[i][j] = MF::mma(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
}

// Block id -> (m tile, n tile), grouped so that GM consecutive blocks share an
// N tile column band and walk M, keeping W tiles hot in L2.
__device__ __forceinline__ void tile_of(int pid, int num_m, int num_n, int& mt, int& nt) {
  constexpr int GM = 8;
  const int group = GM * num_n;
  const int gid = pid / group;
  const int first_m = gid * GM;
  const int gsz = min(num_m - first_m, GM);
  const int in = pid - gid * group;
  mt = first_m + in % gsz;
  nt = in / gsz;
}

// ---------------------------------------------------------------------------
// Element-wise epilogues
// ---------------------------------------------------------------------------
template <typename T>
struct EpiAct {  // out[m, n] = act(v + bias[n])
  const T* bias;
  void* out;
  int ldo;
  int act;       // 0 none, 1 tanh-GELU
  int out_f32;   // store fp32 instead of T
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    if (bias) v += to_f32(bias[n]);
    if (act == 1) {
      // GELU tanh form: 0.5 z (1 + tanh(u)) with u = sqrt(2/pi)(z + 0.044715 z^3),
      // evaluated as z * sigmoid(2u) (the same function).
      const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);
      v = v / (1.0f + __expf(-2.0f * u));
    }
    if (out_f32) reinterpret_cast<float*>(out)[(size_t)m * ldo + n] = v;
    else reinterpret_cast<T*>(out)[(size_t)m * ldo + n] = from_f32<T>(v);
  }
};

template <typename T>
struct EpiResid {  // x[m, n] += v + bias[n]   (fp32 residual stream)
  const T* bias;
  float* x;
  int ldx;
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    float* p = x + (size_t)m * ldx + n;
    *p = *p + (v + to_f32(bias[n]));
  }
};

template <typename T>
struct EpiQKV {  // + bias, split Q|K|V, heads as column blocks of width D
  const T* bias;
  int C, H, D, T_seq;
  T* q;  long long q_bh;            // q[(b*H+h)*q_bh + t*D + d]
  T* k;  long long k_bh;            // k[(b*H+h)*k_bh + tc*D + d]
  T* vt; long long v_bh; int v_ld;  // vt[(b*H+h)*v_bh + d*v_ld + tc]
  const int32_t* pos;               // nullable: tc = t + *pos (cache append)
  __device__ __forceinline__ void operator()(int m, int n, float v) const {
    v += to_f32(bias[n]);
    const int which = n / C;
    const int c = n - which * C;
    const int h = c / D, d = c - h * D;
    const int b = m / T_seq, t = m - b * T_seq;
    const long long bh = (long long)b * H + h;
    const T val = from_f32<T>(v);
    if (which == 0) {
      q[bh * q_bh + (long long)t * D + d] = val;
    } else {
      const int tc = t + (pos ? *pos : 0);
      if (which == 1) k[bh * k_bh + (long long)tc * D + d] = val;
      else vt[bh * v_bh + (long long)d * v_ld + tc] = val;
    }
  }
};

template <typename T, int BM, int BN, int BK, int WM, int WN, typename Epi>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(const T* __restrict__ A, int lda, const T* __restrict__ W, int ldw, int M, int N, int K, Epi epi) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  __shared__ __align__(16) T smem[G::SMEM_ELEMS];
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, num_m, num_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  f32x16 acc[G::TM][G::TN];
  gemm_mainloop<T, BM, BN, BK, WM, WN>(A, lda, W, ldw, M, N, K, m0, n0, smem, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    const int n = n0 + wn * WN + j * 32 + (lane & 31);
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WM + i * 32 + acc_row(r, lane);
        if (m < M) epi(m, n, acc[i][j][r]);
      }
  }
}

// ---------------------------------------------------------------------------
// Tied head + cross-entropy partials.
//   logits (optional)  : z[m, n] in T
//   part_max/part_sum  : [M, ntiles] per-row max and sum exp(z - max) over
//                        this block's N range (n < N only)
//   tgt                : z[m, y[m]] from the block whose range holds y[m]
// y[m] = targets[m] if targets, else idx[m+1] inside a sequence and -1 at
// the last position ("第 25 章 从小 GPT 到 GPT-2" §25.7: predict the next token).
// ---------------------------------------------------------------------------
struct HeadArgs {
  void* logits;
  long long ld_logits;
  float* part_max;
  float* part_sum;
  float* tgt;
  int ntiles;
  const int32_t* targets;
  const int32_t* idx;
  int T_seq;
};

template <typename T, int BM, int BN, int BK, int WM, int WN>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
head_ce_kernel(const T* __restrict__ A, int lda, const T* __restrict__ W, int ldw, int M, int N, int K, HeadArgs ha) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  __shared__ __align__(16) T smem[G::SMEM_ELEMS];
  __shared__ float red[G::NWN][BM];
  __shared__ float rowmax[BM];
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, num_m, num_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  f32x16 acc[G::TM][G::TN];
  gemm_mainloop<T, BM, BN, BK, WM, WN>(A, lda, W, ldw, M, N, K, m0, n0, smem, acc);
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
      int y;
      if (ha.targets) y = ha.targets[m];
      else y = ((m % ha.T_seq) < ha.T_seq - 1) ? ha.idx[m + 1] : -1;
#pragma unroll
      for (int j = 0; j < G::TN; ++j) {
        const int n = ncol0 + j * 32;
        if (n < N) {
          if (ha.logits) reinterpret_cast<T*>(ha.logits)[(long long)m * ha.ld_logits + n] = from_f32<T>(acc[i][j][r]);
          if (n == y) ha.tgt[m] = acc[i][j][r];
        }
      }
    }

  // row max over this block's columns
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
        if (ncol0 + j * 32 < N) mx = fmaxf(mx, acc[i][j][r]);
      mx = half_max(mx);
      if ((lane & 31) == 0) red[wn][wm * WM + i * 32 + acc_row(r, lane)] = mx;
    }
  __syncthreads();
  for (int rr = threadIdx.x; rr < BM; rr += G::NT) {
    float mx = red[0][rr];
#pragma unroll
    for (int w = 1; w < G::NWN; ++w) mx = fmaxf(mx, red[w][rr]);
    rowmax[rr] = mx;
  }
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
        if (ncol0 + j * 32 < N) s += __expf(acc[i][j][r] - mx);
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
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, Epi>), dim3(blocks), dim3(G::NT), 0, st, A, lda, W, ldw,
                     M, N, K, epi);
  return hipGetLastError();
}

// Tile choice per dtype.  fp32 serves the small correctness configurations.
template <typename T, typename Epi>
static hipError_t dispatch_gemm(const T* A, int lda, const T* W, int ldw, int M, int N, int K, const Epi& epi,
                                hipStream_t st);

template <typename Epi>
static hipError_t dispatch_gemm(const bf16* A, int lda, const bf16* W, int ldw, int M, int N, int K, const Epi& epi,
                                hipStream_t st) {
  if ((long long)M * N >= (long long)256 * 1024 * 16)
    return run_gemm<bf16, 128, 128, 64, 64, 64>(A, lda, W, ldw, M, N, K, epi, st);
  return run_gemm<bf16, 64, 64, 64, 32, 32>(A, lda, W, ldw, M, N, K, epi, st);
}

template <typename Epi>
static hipError_t dispatch_gemm(const float* A, int lda, const float* W, int ldw, int M, int N, int K, const Epi& epi,
                                hipStream_t st) {
  return run_gemm<float, 64, 64, 32, 32, 32>(A, lda, W, ldw, M, N, K, epi, st);
}

template <typename T>
static hipError_t linear_t(const void* A, int lda, const void* W, int ldw, const void* bias, int M, int N, int K,
                           void* out, int ldo, int act, int out_f32, hipStream_t st) {
  EpiAct<T> e{(const T*)bias, out, ldo, act, out_f32};
  return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K, e, st);
}

hipError_t launch_linear(int dtype, const void* A, int lda, const void* W, int ldw, const void* bias, int M, int N,
                         int K, void* out, int ldo, int act, int out_f32, hipStream_t st) {
  if (dtype == 0) return linear_t<float>(A, lda, W, ldw, bias, M, N, K, out, ldo, act, out_f32, st);
  return linear_t<bf16>(A, lda, W, ldw, bias, M, N, K, out, ldo, act, out_f32, st);
}

template <typename T>
static hipError_t resid_t(const void* A, int lda, const void* W, int ldw, const void* bias, int M, int N, int K,
                          float* x, int ldx, hipStream_t st) {
  EpiResid<T> e{(const T*)bias, x, ldx};
  return dispatch_gemm((const T*)A, lda, (const T*)W, ldw, M, N, K, e, st);
}

hipError_t launch_linear_resid(int dtype, const void* A, int lda, const void* W, int ldw, const void* bias, int M,
                               int N, int K, float* x, int ldx, hipStream_t st) {
  if (dtype == 0) return resid_t<float>(A, lda, W, ldw, bias, M, N, K, x, ldx, st);
  return resid_t<bf16>(A, lda, W, ldw, bias, M, N, K, x, ldx, st);
}

template <typename T>
static hipError_t qkv_t(const QKVArgs& a, hipStream_t st) {
  EpiQKV<T> e{(const T*)a.bias, a.C, a.H, a.D, a.T_seq, (T*)a.q, a.q_bh, (T*)a.k, a.k_bh,
              (T*)a.vt, a.v_bh, a.v_ld, a.pos};
  return dispatch_gemm((const T*)a.A, a.C, (const T*)a.W, a.C, a.M, 3 * a.C, a.C, e, st);
}

hipError_t launch_qkv(int dtype, const QKVArgs& a, hipStream_t st) {
  if (dtype == 0) return qkv_t<float>(a, st);
  return qkv_t<bf16>(a, st);
}

int head_tile_n(int dtype) { return dtype == 0 ? 64 : 128; }

hipError_t launch_head_ce(int dtype, const void* A, const void* wte, int M, int V, int C, void* logits,
                          long long ld_logits, float* part_max, float* part_sum, float* tgt, const int32_t* targets,
                          const int32_t* idx, int T_seq, hipStream_t st) {
  HeadArgs ha{logits, ld_logits, part_max, part_sum, tgt, 0, targets, idx, T_seq};
  if (dtype == 0) {
    constexpr int BM = 64, BN = 64;
    ha.ntiles = (V + BN - 1) / BN;
    const int blocks = ((M + BM - 1) / BM) * ha.ntiles;
    hipLaunchKernelGGL((head_ce_kernel<float, BM, BN, 32, 32, 32>), dim3(blocks),
                       dim3(GemmCfg<float, BM, BN, 32, 32, 32>::NT), 0, st, (const float*)A, C, (const float*)wte, C,
                       M, V, C, ha);
  } else {
    constexpr int BM = 128, BN = 128;
    ha.ntiles = (V + BN - 1) / BN;
    const int blocks = ((M + BM - 1) / BM) * ha.ntiles;
    hipLaunchKernelGGL((head_ce_kernel<bf16, BM, BN, 64, 64, 64>), dim3(blocks),
                       dim3(GemmCfg<bf16, BM, BN, 64, 64, 64>::NT), 0, st, (const bf16*)A, C, (const bf16*)wte, C, M,
                       V, C, ha);
  }
  return hipGetLastError();
}

}  // namespace gptmi
