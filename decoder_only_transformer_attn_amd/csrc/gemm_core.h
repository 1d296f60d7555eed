// GEMM building blocks shared by the library's product kernels: the
// register-staged and the direct-to-LDS (buffer_load ... lds) main loops,
// the XCD-aware tile order, the element-wise epilogues and the block-tiled
// kernels that combine them.  Internal to the library.
#pragma once
#include <type_traits>

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
// Rows past M (N) read as zero; KTAIL zeroes the chunks past K when K % BK != 0.
template <typename T, int BM, int BN, int BK, int WM, int WN, bool KTAIL>
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

  // Resources cover exactly the rows of this tile that exist.
  const int mrows = min(BM, M - m0), nrows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(A + (size_t)m0 * lda, (uint32_t)((size_t)mrows * lda * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rb_src = make_rsrc(W + (size_t)n0 * ldw, (uint32_t)((size_t)nrows * ldw * sizeof(T)));
  uint32_t a_off[G::A_PT], b_off[G::B_PT];
  int a_kc[G::A_PT], b_kc[G::B_PT];
#pragma unroll
  for (int c = 0; c < G::A_PT; ++c) {
    const int ch = tid + c * G::NT, row = ch / G::CPR;
    a_kc[c] = (ch % G::CPR) * G::VEC;
    a_off[c] = (uint32_t)((row * lda + a_kc[c]) * sizeof(T));
  }
#pragma unroll
  for (int c = 0; c < G::B_PT; ++c) {
    const int ch = tid + c * G::NT, row = ch / G::CPR;
    b_kc[c] = (ch % G::CPR) * G::VEC;
    b_off[c] = (uint32_t)((row * ldw + b_kc[c]) * sizeof(T));
  }

  uint4 ra[G::A_PT], rb[G::B_PT];
  auto gload = [&](int k0) {
    const uint32_t so = (uint32_t)(k0 * sizeof(T));
#pragma unroll
    for (int c = 0; c < G::A_PT; ++c) {
      ra[c] = buf_load16(ra_src, a_off[c], so);
      if (KTAIL && k0 + a_kc[c] >= K) ra[c] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < G::B_PT; ++c) {
      rb[c] = buf_load16(rb_src, b_off[c], so);
      if (KTAIL && k0 + b_kc[c] >= K) rb[c] = make_uint4(0, 0, 0, 0);
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

// Block id -> (m tile, n tile).  The hardware hands consecutive workgroups to
// the 8 XCDs in turn, and each XCD has its own L2; so the block id is first
// remapped to give every XCD one contiguous range of a grouped tile order, in
// which GM m-tiles sweep the n-tiles together (operand tiles of blocks that
// run at the same time on one XCD overlap and stay in that XCD's L2).
__device__ __forceinline__ void tile_of(int pid, int nblocks, int num_m, int num_n, int& mt, int& nt) {
  constexpr int NXCD = 8, GM = 8;
  const int xcd = pid % NXCD, local = pid / NXCD;
  const int per = nblocks / NXCD, rem = nblocks % NXCD;
  const int logical = xcd * per + min(xcd, rem) + local;
  const int group = GM * num_n;
  const int gid = logical / group;
  const int first_m = gid * GM;
  const int gsz = min(num_m - first_m, GM);
  const int in = logical - gid * group;
  mt = first_m + in % gsz;
  nt = in / gsz;
}

// ---------------------------------------------------------------------------
// Pipelined bf16 main loop with direct-to-LDS loads.
//
// Tiles flow through a ring of NST LDS stages, each holding BK (32 or 64)
// K-columns of the BM rows of A and the BN rows of W: gfx950's buffer_load
// ... lds writes each 16-byte chunk straight into LDS (no VGPR staging, no
// ds_write), NST - 1 stages are in flight while one is multiplied, and one
// barrier per stage hands a stage from the loads to the MFMAs.  Each wave
// waits for its own loads of stage t (s_waitcnt vmcnt) before the barrier, so
// after it every wave's loads of stage t are in LDS.  The stages are distinct
// LDS objects so the compiler can tell a read of one stage from the loads
// into another.
//
// A row of a stage is ROWB = 2 BK bytes, CPR = BK / 8 chunks of 16 bytes.
// With BK = 64 a row is one whole 128-byte cache line, so every load
// instruction (8 rows of 128 bytes) reads whole lines; that is what lets the
// per-CU load path run near its streaming rate (half-line rows, BK = 32,
// reach about half of it).  Chunk c of row r is stored at slot
// c ^ ((r / (16 / CPR)) % CPR): a fragment read (ds_read_b128) has 16
// consecutive lanes read one chunk of 16 consecutive rows, LDS serves 64
// banks (256 bytes) per cycle, and row r, slot s lies in 16-byte bank group
// (r CPR + s) % 16, so rows that share r % (16 / CPR) must use different
// slots, which the XOR term gives.  Fragment reads run one k-substep (16) ahead
// of the MFMAs.  K is a template parameter and the K loop is unrolled
// completely.
// ---------------------------------------------------------------------------
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | (((N >> 4) & 3) << 14));
}

// Workgroup barrier that keeps the compiler from moving memory accesses across
// it but, unlike __syncthreads, does not wait for outstanding loads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int CPR> __device__ __forceinline__ int swz(int r, int c) { return c ^ ((r / (16 / CPR)) % CPR); }

// One 1 KB direct-to-LDS load: lane l's 16 bytes land at lds + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, lds_char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 16, voff, soff, 0, 0);
}

template <int BM, int BN, int WM, int WN, int NST_ = 4, int BK_ = 32>
struct DmaCfg {
  static constexpr int BK = BK_, NST = NST_, ROWB = 2 * BK, CPR = BK / 8, RPI = 1024 / ROWB;
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN, NT = NW * WAVE;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int STAGE = (BM + BN) * ROWB;        // bytes per stage
  static constexpr int NI = (BM + BN) / RPI;            // 1 KB load instructions per stage
  static constexpr int DPW = NI / NW;                   // per wave
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(NI % NW == 0 && BM % RPI == 0 && BN % RPI == 0, "loads must split evenly over the waves");
};

// The ring's stages: up to eight distinct LDS arrays (see above).
struct Stages {
  lds_char* p[8];
};

// Wait until at most g of this wave's load groups (DPW loads each) are still
// in flight; g is a constant once the K loop is unrolled.
// (Counts past the counter's range only appear in cases a given stage count
// never reaches, see the static_assert in dma_mainloop; they are clamped.)
template <int DPW> __device__ __forceinline__ void wait_groups(int g) {
  constexpr int C = 63;
  switch (g) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<(DPW < C ? DPW : C)>(); break;
    case 2: wait_vmcnt<(2 * DPW < C ? 2 * DPW : C)>(); break;
    case 3: wait_vmcnt<(3 * DPW < C ? 3 * DPW : C)>(); break;
    case 4: wait_vmcnt<(4 * DPW < C ? 4 * DPW : C)>(); break;
    case 5: wait_vmcnt<(5 * DPW < C ? 5 * DPW : C)>(); break;
    default: wait_vmcnt<(6 * DPW < C ? 6 * DPW : C)>(); break;
  }
}

// Tile (m0, n0)'s load plan: buffer resources over the tile's A and W rows
// (row strides lda, ldw elements; nk stages of BK columns) and each lane's
// offsets; issue(t, s) sends this wave's share of stage t into LDS stage s.
// A resource spans whole rows of the tile that exist, so rows past M (N)
// read as zero; the host keeps rows * ld * 2 bytes below 2^32.
template <int BM, int BN, int WM, int WN, int NST, int BK>
struct DmaLoads {
  typedef DmaCfg<BM, BN, WM, WN, NST, BK> D;
  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t voff[D::DPW];
  int wave, nk;
  __device__ __forceinline__ DmaLoads(const bf16* A, int lda, const bf16* W, int ldw, int K, int M, int N, int m0,
                                      int n0) {
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    nk = K / BK;
    rsA = make_rsrc(A + (size_t)m0 * lda, (uint32_t)((size_t)min(BM, M - m0) * lda * sizeof(bf16)));
    rsB = make_rsrc(W + (size_t)n0 * ldw, (uint32_t)((size_t)min(BN, N - n0) * ldw * sizeof(bf16)));
#pragma unroll
    for (int d = 0; d < D::DPW; ++d) {
      const int ins = wave + d * D::NW;
      constexpr int IA = BM / D::RPI;   // instructions covering A
      const int row = (ins < IA ? ins : ins - IA) * D::RPI + lane / D::CPR, slot = lane % D::CPR;
      voff[d] = (uint32_t)((row * (ins < IA ? lda : ldw) + swz<D::CPR>(row, slot) * 8) * sizeof(bf16));
    }
  }
  __device__ __forceinline__ void issue(int t, lds_char* s) const {
#pragma unroll
    for (int d = 0; d < D::DPW; ++d) {
      const int ins = wave + d * D::NW;
      dma16(ins < BM / D::RPI ? rsA : rsB, s + ins * 1024, voff[d], t * BK * 2);
    }
  }
  // the first NST - 1 stages of the tile
  __device__ __forceinline__ void prologue(const Stages& st) const {
#pragma unroll
    for (int t = 0; t < NST - 1; ++t)
      if (t < nk) issue(t, st.p[t]);
  }
};

// K > 0: a compile-time depth (rows of K elements, the loop fully unrolled);
// K == 0: depth Kr (a multiple of BK) and row strides lda, ldw at run time,
// the loop unrolled by the ring's length so every stage index is constant.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// K > 0 only: hook() is called once, in stage max(NK - 2, 0) right after that
// stage's DMA issue, and issues NPRE vector loads per lane (the epilogue's
// per-element inputs), so they are in flight during the last stages instead
// of ahead of the first one (loads complete in order: issued before the
// prologue they would hold up stage 0).  The last stage's wait leaves those
// NPRE loads outstanding.
template <int BM, int BN, int WM, int WN, int K, int NST, int BK, int NPRE = 0, typename Hook = NoHook>
__device__ __forceinline__ void dma_mainloop(const bf16* __restrict__ A, int lda, const bf16* __restrict__ W, int ldw,
                                             int Kr, int M, int N, int m0, int n0, const Stages& st,
                                             f32x16 (&acc)[WM / 32][WN / 32], const Hook& hook = Hook()) {
  typedef DmaCfg<BM, BN, WM, WN, NST, BK> D;
  constexpr int KS = BK / 16;         // MFMA k-substeps per stage
  constexpr int CPR = D::CPR;
  static_assert(K % BK == 0, "K must be a multiple of the stage depth");
  static_assert(NST >= 2 && NST <= 8 && (NST - 2) * D::DPW < 64, "stage count");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / D::NWN, wn = wave % D::NWN;
#pragma unroll
  for (int i = 0; i < D::TM; ++i)
#pragma unroll
    for (int j = 0; j < D::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Stage layout: A rows [0, BM) then W rows, ROWB bytes each.  Load
  // instruction i (RPI rows) goes to LDS offset 1024 i and is issued by wave
  // i % NW; the wave index is uniform, so the A/W choice stays scalar.
  const DmaLoads<BM, BN, WM, WN, NST, BK> ld(A, K > 0 ? K : lda, W, K > 0 ? K : ldw, K > 0 ? K : Kr, M, N, m0, n0);
  const int lrow = lane & 31, g = lane >> 5;
  auto ldfrag = [&](const lds_char* s, int ks, bf16x8 (&af)[D::TM], bf16x8 (&bfr)[D::TN]) {
    const int c = ks * 2 + g;
#pragma unroll
    for (int i = 0; i < D::TM; ++i) {
      const int r = wm * WM + i * 32 + lrow;
      af[i] = lds_frag(s + r * D::ROWB + swz<CPR>(r, c) * 16);
    }
#pragma unroll
    for (int j = 0; j < D::TN; ++j) {
      const int r = wn * WN + j * 32 + lrow;
      bfr[j] = lds_frag(s + BM * D::ROWB + r * D::ROWB + swz<CPR>(r, c) * 16);
    }
  };
  auto mm = [&](const bf16x8 (&af)[D::TM], const bf16x8 (&bfr)[D::TN]) {
#pragma unroll
    for (int i = 0; i < D::TM; ++i)
#pragma unroll
      for (int j = 0; j < D::TN; ++j) acc[i][j] = Mfma<bf16>::mma(af[i], bfr[j], acc[i][j]);
  };
  auto step = [&](const lds_char* s) {
    bf16x8 af[2][D::TM], bfr[2][D::TN];
    ldfrag(s, 0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) ldfrag(s, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mm(af[ks & 1], bfr[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  ld.prologue(st);
  if constexpr (K > 0) {
    constexpr int NK = K / BK;        // stages along K
    constexpr int TH = NK >= 2 ? NK - 2 : 0;   // the stage that calls hook()
    static_assert(NPRE >= 0 && NPRE < 64, "outstanding loads past the counter's range");
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      if (NPRE > 0 && t > TH) wait_vmcnt<NPRE>();      // (no DMA is issued after stage TH's)
      else wait_groups<D::DPW>(min(NST - 2, NK - 1 - t));   // this wave's loads of stage t have landed
      lds_barrier();                                   // ... and every other wave's
      if (t + NST - 1 < NK) ld.issue(t + NST - 1, st.p[(t + NST - 1) % NST]);   // the stage consumed at t - 1
      if (t == TH) hook();
      step(st.p[t % NST]);
    }
  } else {
    const int NK = ld.nk;
    for (int t0 = 0; t0 < NK; t0 += NST) {
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int t = t0 + u;
        if (t >= NK) break;
        // near the end fewer groups follow stage t: wait for all of them
        if (t + NST - 2 < NK) wait_groups<D::DPW>(NST - 2);
        else wait_vmcnt<0>();
        lds_barrier();
        if (t + NST - 1 < NK) ld.issue(t + NST - 1, st.p[(u + NST - 1) % NST]);
        step(st.p[u]);
      }
    }
  }
  __syncthreads();  // every wave is done with the stages: the epilogue may reuse LDS
}

// ---------------------------------------------------------------------------
// Epilogues.  Each is called for two adjacent output columns (n, n+1) of
// one row; has_b is false only for the last column of an odd N.  All inputs
// an epilogue reads are fetched before the main loop so that their latency
// hides under the MFMA work: col(n) returns the per-column values (the bias
// pair), and epilogues with kPreload also read a per-element input (the
// residual stream) through preload(m, n).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float gelu_tanh(float v) {
  // 0.5 z (1 + tanh(u)), u = sqrt(2/pi)(z + 0.044715 z^3), evaluated as
  // z * sigmoid(2u) = z / (1 + exp(-2u)), with exp(-2u) = exp2(-2 log2(e) u)
  const float u = v * (0.7978845608028654f + 0.035677408136300125f * v * v);
  return v * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-2.8853900817779268f * u));
}

template <typename T>
__device__ __forceinline__ void store_pair(T* p, float a, float b, bool has_b, bool vec_ok) {
  if (has_b && vec_ok) {
    if constexpr (sizeof(T) == 4) *reinterpret_cast<float2*>(p) = make_float2(a, b);
    else *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
  } else {
    p[0] = from_f32<T>(a);
    if (has_b) p[1] = from_f32<T>(b);
  }
}

// Bias values of a column pair, kept in storage form until the epilogue so
// that no instruction before the main loop waits for their loads.
template <typename T>
struct RawPair {
  uint32_t a, b;   // bit patterns: bf16 zero-extended, fp32 as is
  static __device__ __forceinline__ uint32_t bits(T v) {
    if constexpr (sizeof(T) == 2) return (uint32_t)v;
    else return __float_as_uint(v);
  }
  static __device__ __forceinline__ float f32(uint32_t u) {
    if constexpr (sizeof(T) == 2) return __uint_as_float(u << 16);
    else return __uint_as_float(u);
  }
};

// GELU, exact form: 0.5 z (1 + erf(z / sqrt 2)) (HIP's erff)
__device__ __forceinline__ float gelu_erf(float v) { return 0.5f * v * (1.0f + erff(v * 0.7071067811865476f)); }

template <typename T, int ACT = 0, bool F32OUT = false>
struct EpiAct {  // out[m, n] = act(v + bias[n]); ACT 1 = tanh GELU, 2 = exact GELU; F32OUT: store fp32 instead of T
  static constexpr bool kPreload = false;
  static constexpr bool kCompact = true;
  typedef int Row;
  typedef RawPair<T> Col;
  typedef RawPair<T> ColX;
  typedef typename std::conditional<F32OUT, float, T>::type O;
  __device__ __forceinline__ Row row(int) const { return 0; }
  __device__ __forceinline__ ColX colx(int, const Col& c) const { return c; }
  const T* bias;
  void* out;
  int ldo;
  __device__ __forceinline__ Col col(int n, bool has_b) const {
    // branch-free: without a bias the (valid) output row is read instead and ignored
    const T* bp = bias ? bias : reinterpret_cast<const T*>(out);
    return Col{Col::bits(bp[n]), Col::bits(bp[has_b ? n + 1 : n])};
  }
  __device__ __forceinline__ float2 preload(int, int, bool) const { return make_float2(0.f, 0.f); }
  __device__ __forceinline__ float2 value(float a, float b, const Col& bs) const {
    const float w = bias ? 1.f : 0.f;   // uniform
    a = fmaf(w, Col::f32(bs.a), a);
    b = fmaf(w, Col::f32(bs.b), b);
    if constexpr (ACT == 1) { a = gelu_tanh(a); b = gelu_tanh(b); }
    if constexpr (ACT == 2) { a = gelu_erf(a); b = gelu_erf(b); }
    return make_float2(a, b);
  }
  __device__ __forceinline__ void pair(Row, int m, int n, float a, float b, bool has_b, const Col& bs, float2) const {
    const float2 v = value(a, b, bs);
    store_pair(reinterpret_cast<O*>(out) + (size_t)m * ldo + n, v.x, v.y, has_b, (ldo & 1) == 0);
  }
  // interior tiles: both columns exist and pairs are aligned
  __device__ __forceinline__ bool vec_ok() const { return (ldo & 1) == 0; }
  __device__ __forceinline__ void pair_in(Row, int m, int n, float a, float b, const Col& bs, float2) const {
    const float2 v = value(a, b, bs);
    O* p = reinterpret_cast<O*>(out) + (size_t)m * ldo + n;
    if constexpr (sizeof(O) == 4) *reinterpret_cast<float2*>(p) = v;
    else *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v.x, v.y);
  }
};

template <typename T>
struct EpiResid {  // x[m, n] += v + bias[n]   (fp32 residual stream)
  static constexpr bool kPreload = true;
  static constexpr bool kCompact = false;
  typedef int Row;
  typedef RawPair<T> Col;
  typedef RawPair<T> ColX;
  __device__ __forceinline__ Row row(int) const { return 0; }
  __device__ __forceinline__ ColX colx(int, const Col& c) const { return c; }
  const T* bias;
  float* x;
  int ldx;
  __device__ __forceinline__ Col col(int n, bool has_b) const {
    if (!bias) return Col{0u, 0u};   // no bias
    return Col{Col::bits(bias[n]), Col::bits(bias[has_b ? n + 1 : n])};
  }
  __device__ __forceinline__ float2 preload(int m, int n, bool has_b) const {
    const float* p = x + (size_t)m * ldx + n;
    if (has_b && (ldx & 1) == 0) return *reinterpret_cast<const float2*>(p);
    return make_float2(p[0], has_b ? p[1] : 0.f);
  }
  __device__ __forceinline__ void pair(Row, int m, int n, float a, float b, bool has_b, const Col& bs, float2 xo) const {
    a = xo.x + (a + Col::f32(bs.a));
    if (has_b) b = xo.y + (b + Col::f32(bs.b));
    store_pair(x + (size_t)m * ldx + n, a, b, has_b, (ldx & 1) == 0);
  }
  __device__ __forceinline__ bool vec_ok() const { return (ldx & 1) == 0; }
  __device__ __forceinline__ void pair_in(Row, int m, int n, float a, float b, const Col& bs, float2 xo) const {
    *reinterpret_cast<float2*>(x + (size_t)m * ldx + n) =
        make_float2(xo.x + (a + Col::f32(bs.a)), xo.y + (b + Col::f32(bs.b)));
  }
};

// q = m / d for 0 <= m < 2^24 with a float reciprocal and one correction step.
__device__ __forceinline__ int div_small(int m, int d, float inv_d) {
  int q = (int)((float)m * inv_d);
  q -= (q * d > m);
  q += ((q + 1) * d <= m);
  return q;
}

template <typename T>
struct EpiQKV {  // + bias, split Q|K|U, heads as column blocks of width D; Q [B,H,T,D], K/U [B,Hkv,Tk,D]
  static constexpr bool kPreload = false;
  static constexpr bool kCompact = true;
  const T* bias;                    // nullable
  int C, H, D, T_seq;
  float inv_T;
  T* q; long long q_bh;             // q[(b*H+h)*q_bh + t*D + d]
  T* k; long long k_bh;             // k[(b*Hkv+h)*k_bh + tc*D + d]
  T* v; long long v_bh;             // v[(b*Hkv+h)*v_bh + tc*D + d]
  const int32_t* pos;               // nullable: tc = t + *pos (cache append)
  int Tk;                           // K/U rows; cache positions >= Tk are not written
  int Hkv;
  const float2* rope;               // nullable: rotate the (2i, 2i+1) pairs of Q and K by position tc
  struct Row { int b, t, tc; };
  typedef RawPair<T> Col;   // held across the main loop: the bias pair only
  struct ColX { RawPair<T> bias; T* base; int b_stride; bool is_q; bool rot; int pair; };   // b_stride < 2^31
  __device__ __forceinline__ Row row(int m) const {
    const int bb = div_small(m, T_seq, inv_T), t = m - bb * T_seq;
    return Row{bb, t, t + (pos ? *pos : 0)};
  }
  __device__ __forceinline__ Col col(int n, bool) const {
    if (!bias) return Col{0u, 0u};
    return Col{RawPair<T>::bits(bias[n]), RawPair<T>::bits(bias[n + 1])};
  }
  // Column n (even) -> projection, head and head column, worked out once per
  // column tile when the epilogue starts; D is even, so n and n + 1 fall in
  // the same head of the same projection (and form one rotary pair).
  __device__ __forceinline__ ColX colx(int n, const Col& bs) const {
    const int kvd = Hkv * D;
    const int which = n < C ? 0 : (n < C + kvd ? 1 : 2);
    const int c = n - (which == 0 ? 0 : (which == 1 ? C : C + kvd));
    const int h = c / D, d = c - h * D;
    const long long st = which == 0 ? q_bh : (which == 1 ? k_bh : v_bh);
    T* arr = which == 0 ? q : (which == 1 ? k : v);
    return ColX{bs, arr + h * st + d, (int)(st * (which == 0 ? H : Hkv)), which == 0, rope && which < 2, d >> 1};
  }
  __device__ __forceinline__ float2 preload(int, int, bool) const { return make_float2(0.f, 0.f); }
  __device__ __forceinline__ void pair(const Row& r, int, int, float a, float b, bool, const ColX& cl, float2) const {
    if (!cl.is_q && (r.tc < 0 || r.tc >= Tk)) return;   // outside the cache: contract violation, nothing written
    T* dst = cl.base + (long long)r.b * cl.b_stride + (long long)(cl.is_q ? r.t : r.tc) * D;
    a += RawPair<T>::f32(cl.bias.a);
    b += RawPair<T>::f32(cl.bias.b);
    if (cl.rot) {
      // (a query past the cache also violates the contract: its row is clamped
      // into the table, which has at least Tk rows)
      const int p = r.tc < 0 ? 0 : (r.tc < Tk ? r.tc : Tk - 1);
      const float2 cs = rope[(long long)p * (D >> 1) + cl.pair];
      const float ra = cs.x * a - cs.y * b, rb = cs.y * a + cs.x * b;
      a = ra;
      b = rb;
    }
    store_pair(dst, a, b, true, true);
  }
  __device__ __forceinline__ bool vec_ok() const { return true; }
  __device__ __forceinline__ void pair_in(const Row& r, int m, int n, float a, float b, const ColX& cl,
                                          float2 pre) const {
    pair(r, m, n, a, b, true, cl, pre);
  }
};

// SwiGLU: columns (2j, 2j+1) of the product are (gate, up) of hidden unit j;
// out[m, j] = SiLU(gate) * up, SiLU(z) = z / (1 + e^-z)  ("02 GPT 架构" §6.1;
// "GPT-1学习笔记" §10.2).  N (= 2F) is even, so every pair exists.
template <typename T>
struct EpiSwiGLU {
  static constexpr bool kPreload = false;
  static constexpr bool kCompact = true;
  typedef int Row;
  typedef int Col;
  typedef int ColX;
  T* out;
  int ldo;
  __device__ __forceinline__ Row row(int) const { return 0; }
  __device__ __forceinline__ Col col(int, bool) const { return 0; }
  __device__ __forceinline__ ColX colx(int, const Col& c) const { return c; }
  __device__ __forceinline__ float2 preload(int, int, bool) const { return make_float2(0.f, 0.f); }
  __device__ __forceinline__ void pair(Row, int m, int n, float g, float u, bool, ColX, float2) const {
    out[(size_t)m * ldo + (n >> 1)] = from_f32<T>(g / (1.0f + __expf(-g)) * u);
  }
  __device__ __forceinline__ bool vec_ok() const { return true; }
  __device__ __forceinline__ void pair_in(Row r, int m, int n, float g, float u, ColX c, float2 p) const {
    pair(r, m, n, g, u, true, c, p);
  }
};

// An epilogue with kRaw takes the wave's whole accumulator tile (raw<TM, TN,
// WLB>) instead of the paired-column driver below, together with WLB bytes of
// LDS (16-byte aligned) that are the wave's own once the main loop is done.
template <typename E, typename = void>
struct IsRaw { static constexpr bool value = false; };
template <typename E>
struct IsRaw<E, std::void_t<decltype(E::kRaw)>> { static constexpr bool value = E::kRaw; };

// Loss gradient of the head's logits: dz[m, n] = (exp(v - lse[m]) - [n == y[m]])
// * s[m], s = 1 / (number of rows with a target) for a row with one, else 0.
// Written twice: row-major dz [M, ld] and transposed dzT [N, ldT] (tokens
// contiguous), the operands of the two gradient products.  In the MFMA
// accumulator a lane holds four consecutive rows (tokens) of one column, so
// the transposed copy is one 4-element store per register quad; the row-major
// copy pairs adjacent columns with the neighbouring lane.  In bf16 with a
// wave LDS share that holds the wave's whole transposed tile (and ldT a
// multiple of 8), the quads are first gathered in LDS, tile rows of WM tokens
// with their 8-byte chunks XOR-swizzled by row so that a quad store of 32
// consecutive columns meets no bank twice, and then leave as 16-byte stores
// that cover whole rows of dzT.
template <typename T>
struct EpiDz {
  static constexpr bool kPreload = false;
  static constexpr bool kCompact = true;
  static constexpr bool kRaw = true;
  typedef int Row;
  typedef int Col;
  typedef int ColX;
  const float* lse;      // [M]
  const int32_t* y;      // [M] target of each row, -1 for none
  const float* inv;      // [1] 1 / n_valid (0 when no row has a target)
  T* dz;
  long long ld;          // even
  T* dzT;
  long long ldT;         // multiple of 4
  __device__ __forceinline__ Row row(int) const { return 0; }
  __device__ __forceinline__ Col col(int, bool) const { return 0; }
  __device__ __forceinline__ ColX colx(int, const Col& c) const { return c; }
  __device__ __forceinline__ float2 preload(int, int, bool) const { return make_float2(0.f, 0.f); }

  template <int TM, int TN, int WLB>
  __device__ __forceinline__ void raw(const f32x16 (&acc)[TM][TN], int mbase, int nbase, int M, int N,
                                      lds_char* wl) const {
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr int WM = TM * 32, WN = TN * 32;
    constexpr int RB = WM * 2, NC = WM / 4, NU = WM / 8;   // staged row bytes, 8-byte chunks, 16-byte units
    constexpr bool kStage = sizeof(T) == 2 && WLB >= WN * RB;
    const bool staged = kStage && (ldT & 7) == 0;         // uniform
    const int lane = threadIdx.x & 63;
    const bool odd = lane & 1;
    const float iv = *inv;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m0 = mbase + i * 32 + q * 8 + (lane >> 5) * 4;   // rows m0 .. m0 + 3 (acc_row of 4q + e)
        float l4[4], s4[4];
        int y4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + e;
          const int yy = m < M ? y[m] : -1;
          l4[e] = m < M ? lse[m] : 0.f;
          s4[e] = yy >= 0 ? iv : 0.f;
          y4[e] = yy;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = nbase + j * 32 + (lane & 31);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = (fast_exp2((acc[i][j][4 * q + e] - l4[e]) * LOG2E) - (n == y4[e] ? 1.f : 0.f)) * s4[e];
          // row-major: lanes 2k, 2k+1 hold columns n, n+1; after one exchange
          // per row pair the even lane stores row m0+e and the odd lane row
          // m0+e+1, both at columns (n_even, n_even + 1)
          const int ne = n & ~1;
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float recv = xor1(odd ? v[e] : v[e + 1]);
            const int m = m0 + e + (odd ? 1 : 0);
            const float a = odd ? recv : v[e], b = odd ? v[e + 1] : recv;
            if (m < M && ne < N) store_pair(dz + (long long)m * ld + ne, a, b, ne + 1 < N, true);
          }
          if (kStage && staged) {
            const int r = j * 32 + (lane & 31), c = i * 8 + q * 2 + (lane >> 5);
            lds_st8(wl + r * RB + ((c ^ ((r >> 1) & (NC - 1))) << 3),
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
          } else if (n < N) {
            T* p = dzT + (long long)n * ldT + m0;
            if (m0 + 3 < M) {
              if constexpr (sizeof(T) == 4) {
                *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
              } else {
                const uint2 w = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                *reinterpret_cast<uint2*>(p) = w;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (m0 + e < M) p[e] = from_f32<T>(v[e]);
            }
          }
        }
      }
    if constexpr (kStage) {
      if (!staged) return;
      __syncthreads();   // every wave has written its tile (each reads back only its own)
      // NU lanes per tile row, 64 / NU rows per pass; chunks 2k and 2k + 1 of
      // row r sit, swapped when the row's swizzle is odd, in unit k ^ (f >> 1)
#pragma unroll
      for (int it = 0; it < WN * NU / 64; ++it) {
        const int r = it * (64 / NU) + lane / NU, k = lane % NU, f = (r >> 1) & (NC - 1);
        uint4 w = lds_ld16(wl + r * RB + ((k ^ (f >> 1)) << 4));
        if (f & 1) w = make_uint4(w.z, w.w, w.x, w.y);
        const int n = nbase + r, m = mbase + k * 8;
        if (n >= N || m >= M) continue;
        T* p = dzT + (long long)n * ldT + m;
        if (m + 8 <= M) {
          *reinterpret_cast<uint4*>(p) = w;
        } else {
          const uint32_t h[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (m + e < M) reinterpret_cast<uint16_t*>(p)[e] = (uint16_t)(h[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
};

// fp32 output, out[m, n] = v (ACC false) or out[m, n] += v (ACC true; the
// old value is read at the store, so nothing is held across the main loop)
template <bool ACC>
struct EpiF32 {
  static constexpr bool kPreload = false;
  static constexpr bool kCompact = true;
  typedef int Row;
  typedef int Col;
  typedef int ColX;
  float* out;
  int ldo;
  __device__ __forceinline__ void shift(long long off) { out += off; }
  __device__ __forceinline__ EpiF32 at(int b, int h, const BatchStrides& bs) const {
    return EpiF32{out + b * bs.ob + h * bs.oh, ldo};
  }
  __device__ __forceinline__ Row row(int) const { return 0; }
  __device__ __forceinline__ Col col(int, bool) const { return 0; }
  __device__ __forceinline__ ColX colx(int, const Col& c) const { return c; }
  __device__ __forceinline__ float2 preload(int, int, bool) const { return make_float2(0.f, 0.f); }
  __device__ __forceinline__ void pair(Row, int m, int n, float a, float b, bool has_b, ColX, float2) const {
    float* p = out + (size_t)m * ldo + n;
    if constexpr (ACC) {
      a += p[0];
      if (has_b) b += p[1];
    }
    store_pair(p, a, b, has_b, (ldo & 1) == 0);
  }
  __device__ __forceinline__ bool vec_ok() const { return (ldo & 1) == 0; }
  __device__ __forceinline__ void pair_in(Row, int m, int n, float a, float b, ColX, float2) const {
    float2* p = reinterpret_cast<float2*>(out + (size_t)m * ldo + n);
    if constexpr (ACC) {
      const float2 o = *p;
      a += o.x;
      b += o.y;
    }
    *p = make_float2(a, b);
  }
};

// Output driver.  Lanes 2k and 2k+1 hold columns n and n+1 of a 32x32 tile,
// and registers r, r+1 (r even) are rows m, m+1.  One exchange gives the even
// lane (row m; n, n+1) and the odd lane (row m+1; n, n+1), so every lane
// stores two adjacent outputs.  `pre` holds the preloaded inputs in the same
// assignment.
template <int TM, int TN>
__device__ __forceinline__ void pair_coords(int i, int j, int rp, int mbase, int nbase, int& m, int& n) {
  const int lane = threadIdx.x & 63;
  m = mbase + i * 32 + acc_row(2 * rp, lane) + (lane & 1);
  n = nbase + j * 32 + ((lane & 31) & ~1);
}

// Per-column epilogue inputs (the bias pairs).
template <int TM, int TN, typename Epi>
__device__ __forceinline__ void preload_cols(typename Epi::Col (&colv)[TN], int mbase, int nbase, int N,
                                             const Epi& epi) {
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int m, n;
    pair_coords<TM, TN>(0, j, 0, mbase, nbase, m, n);
    // no branch around these loads (columns past N read column N-1, unused),
    // so nothing waits for them before the main loop
    const int nc = min(n, N - 1);
    colv[j] = epi.col(nc, nc + 1 < N);
  }
}

// Per-element epilogue inputs (kPreload: the residual rows), one load per
// pair: TM * TN * 8 loads per lane.
template <int TM, int TN, typename Epi>
__device__ __forceinline__ void preload_elems(float2 (&pre)[TM][TN][8], int mbase, int nbase, int M, int N,
                                              const Epi& epi) {
  if constexpr (Epi::kPreload) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int rp = 0; rp < 8; ++rp) {
          int m, n;
          pair_coords<TM, TN>(i, j, rp, mbase, nbase, m, n);
          pre[i][j][rp] = (m < M && n < N) ? epi.preload(m, n, n + 1 < N) : make_float2(0.f, 0.f);
        }
  }
}

template <int TM, int TN, typename Epi>
__device__ __forceinline__ void preload_pairs(float2 (&pre)[TM][TN][8], typename Epi::Col (&colv)[TN], int mbase,
                                              int nbase, int M, int N, const Epi& epi) {
  preload_cols<TM, TN>(colv, mbase, nbase, N, epi);
  preload_elems<TM, TN>(pre, mbase, nbase, M, N, epi);
}

template <int TM, int TN, typename Epi>
__device__ __forceinline__ void epilogue_pairs(const f32x16 (&acc)[TM][TN], const float2 (&pre)[TM][TN][8],
                                               const typename Epi::Col (&colv)[TN], int mbase, int nbase, int M, int N,
                                               const Epi& epi) {
  const bool odd = threadIdx.x & 1;
  typename Epi::ColX cx[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int m, n;
    pair_coords<TM, TN>(0, j, 0, mbase, nbase, m, n);
    cx[j] = epi.colx(min(n, N - 1), colv[j]);
  }
  // a wave tile that lies wholly inside [0, M) x [0, N) (uniform test) takes
  // the unguarded path: no per-pair bounds checks, always a paired store
  if (mbase + TM * 32 <= M && nbase + TN * 32 <= N && epi.vec_ok()) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int rp = 0; rp < 8; ++rp) {
        int m, n0;
        pair_coords<TM, TN>(i, 0, rp, mbase, nbase, m, n0);
        const typename Epi::Row rc = epi.row(m);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float v0 = acc[i][j][2 * rp], v1 = acc[i][j][2 * rp + 1];
          const float recv = xor1(odd ? v0 : v1);
          epi.pair_in(rc, m, n0 + j * 32, odd ? recv : v0, odd ? v1 : recv, cx[j], pre[i][j][rp]);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int rp = 0; rp < 8; ++rp) {
      int m, n0;
      pair_coords<TM, TN>(i, 0, rp, mbase, nbase, m, n0);
      const typename Epi::Row rc = epi.row(m);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        // every lane takes part in the exchange; only the store is predicated
        const float v0 = acc[i][j][2 * rp], v1 = acc[i][j][2 * rp + 1];
        const float recv = xor1(odd ? v0 : v1);
        const int n = n0 + j * 32;
        const float a = odd ? recv : v0, b = odd ? v1 : recv;
        if (m < M && n < N) epi.pair(rc, m, n, a, b, n + 1 < N, cx[j], pre[i][j][rp]);
      }
    }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool KTAIL, typename Epi>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(const T* __restrict__ A, int lda, const T* __restrict__ W, int ldw, int M, int N, int K, Epi epi) {
  typedef GemmCfg<T, BM, BN, BK, WM, WN> G;
  __shared__ __align__(16) T smem[G::SMEM_ELEMS];
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, gridDim.x, num_m, num_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int mb = m0 + (wave / G::NWN) * WM, nb = n0 + (wave % G::NWN) * WN;
  float2 pre[G::TM][G::TN][8];
  typename Epi::Col colv[G::TN];
  preload_pairs<G::TM, G::TN>(pre, colv, mb, nb, M, N, epi);
  f32x16 acc[G::TM][G::TN];
  gemm_mainloop<T, BM, BN, BK, WM, WN, KTAIL>(A, lda, W, ldw, M, N, K, m0, n0, smem, acc);
  if constexpr (IsRaw<Epi>::value) {
    constexpr int WLB = (int)(G::SMEM_ELEMS * sizeof(T) / (G::NWM * G::NWN)) & ~15;
    __syncthreads();   // the tiles of the last K step are read: the LDS is free
    epi.template raw<G::TM, G::TN, WLB>(acc, mb, nb, M, N, as_lds(smem) + wave * WLB);
  } else {
    epilogue_pairs<G::TM, G::TN>(acc, pre, colv, mb, nb, M, N, epi);
  }
}

// bf16 GEMM through the pipelined main loop, element-wise epilogue.
// Waves per SIMD the register budget must allow so that every block the LDS
// budget admits (160 KB per CU) can be resident at once.
template <int BM, int BN, int WM, int WN, int NST, int BK>
constexpr int dma_waves_per_eu() {
  typedef DmaCfg<BM, BN, WM, WN, NST, BK> D;
  const int blocks = (160 * 1024) / (D::STAGE * NST);
  const int w = blocks * D::NW / 4;
  return w < 1 ? 1 : (w > 8 ? 8 : w);
}

template <int BM, int BN, int WM, int WN, int K, int NST, int BK, typename Epi>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(dma_waves_per_eu<BM, BN, WM, WN, NST, BK>())))
gemm_dma_kernel(const bf16* __restrict__ A, int lda, const bf16* __restrict__ W, int ldw, int M, int N, int Kr,
                long long zstride, Epi epi) {
  typedef DmaCfg<BM, BN, WM, WN, NST, BK> D;
  __shared__ __align__(1024) char s0[D::STAGE];
  __shared__ __align__(1024) char s1[D::STAGE];
  __shared__ __align__(1024) char s2[D::STAGE];
  __shared__ __align__(1024) char s3[NST > 3 ? D::STAGE : 16];
  __shared__ __align__(1024) char s4[NST > 4 ? D::STAGE : 16];
  __shared__ __align__(1024) char s5[NST > 5 ? D::STAGE : 16];
  __shared__ __align__(1024) char s6[NST > 6 ? D::STAGE : 16];
  __shared__ __align__(1024) char s7[NST > 7 ? D::STAGE : 16];
  const Stages stages{{as_lds(s0), as_lds(s1), as_lds(s2), as_lds(s3), as_lds(s4), as_lds(s5), as_lds(s6),
                       as_lds(s7)}};
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  int mt, nt;
  tile_of(blockIdx.x, gridDim.x, num_m, num_n, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int mb = m0 + (wave / D::NWN) * WM, nb = n0 + (wave % D::NWN) * WN;
  float2 pre[D::TM][D::TN][8];
  typename Epi::Col colv[D::TN];
  // per-element inputs are requested during the last stages when the wait
  // counter can hold them, else (and at a run-time depth) before the main loop
  constexpr int NPRE = D::TM * D::TN * 8;
  constexpr bool kLate = Epi::kPreload && K > 0 && NPRE < 64;
  preload_cols<D::TM, D::TN>(colv, mb, nb, N, epi);
  if constexpr (!kLate) preload_elems<D::TM, D::TN>(pre, mb, nb, M, N, epi);
  f32x16 acc[D::TM][D::TN];
  if constexpr (K == 0) {
    // split K: slice blockIdx.y covers columns [y Kr, (y + 1) Kr) and writes
    // its own output, zstride elements after the previous slice's
    const int z = blockIdx.y;
    dma_mainloop<BM, BN, WM, WN, 0, NST, BK>(A + (size_t)z * Kr, lda, W + (size_t)z * Kr, ldw, Kr, M, N, m0, n0,
                                             stages, acc);
    Epi e = epi;
    e.shift((long long)z * zstride);
    epilogue_pairs<D::TM, D::TN>(acc, pre, colv, mb, nb, M, N, e);
    return;
  } else if constexpr (kLate) {
    dma_mainloop<BM, BN, WM, WN, K, NST, BK, NPRE>(A, K, W, K, K, M, N, m0, n0, stages, acc, [&]() {
      preload_elems<D::TM, D::TN>(pre, mb, nb, M, N, epi);
    });
  } else {
    dma_mainloop<BM, BN, WM, WN, K, NST, BK>(A, K, W, K, K, M, N, m0, n0, stages, acc);
  }
  if constexpr (IsRaw<Epi>::value) {
    // each wave's share of the (now idle) stages, never straddling two of them
    constexpr int WPS = (D::NW + NST - 1) / NST, WLB = (D::STAGE / WPS) & ~15;
    const int sw = __builtin_amdgcn_readfirstlane(wave) / WPS;
    // (only the stages that exist are named, so no unused array is kept)
    lds_char* base = as_lds(s0);
    if constexpr (NST > 1) base = sw == 1 ? as_lds(s1) : base;
    if constexpr (NST > 2) base = sw == 2 ? as_lds(s2) : base;
    if constexpr (NST > 3) base = sw == 3 ? as_lds(s3) : base;
    if constexpr (NST > 4) base = sw == 4 ? as_lds(s4) : base;
    if constexpr (NST > 5) base = sw == 5 ? as_lds(s5) : base;
    if constexpr (NST > 6) base = sw == 6 ? as_lds(s6) : base;
    if constexpr (NST > 7) base = sw == 7 ? as_lds(s7) : base;
    epi.template raw<D::TM, D::TN, WLB>(acc, mb, nb, M, N, base + (wave % WPS) * WLB);
  } else {
    epilogue_pairs<D::TM, D::TN>(acc, pre, colv, mb, nb, M, N, epi);
  }
}

// ---------------------------------------------------------------------------
// Tied head + cross-entropy partials (shared by the head kernels).
//   logits (optional)  : z[m, n] in T
//   part_max/part_sum  : [M, ntiles] per-row max and sum exp(z - max) over
//                        one vocabulary range (n < N only)
//   tgt                : z[m, y[m]] from the range that holds y[m]
// y[m] = targets[m] if targets, else idx[m+1] inside a sequence and -1 at
// the last position ("第 25 章 从小 GPT 到 GPT-2" §25.7: predict the next token).
// ---------------------------------------------------------------------------
struct HeadArgs {
  void* logits;
  long long ld_logits;
  float* part_max;
  float* part_sum;
  float* tgt;
  int32_t* part_idx;      // argmax mode when non-null
  int ntiles;
  const int32_t* targets;
  const int32_t* idx;
  int T_seq;
  int nt;   // 1: logits rows start on 128-byte lines; stored non-temporally, whole lines
};

// (value, index) order of the greedy choice: larger value, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

__device__ __forceinline__ int head_target(const HeadArgs& ha, int m) {
  if (ha.part_idx) return -1;
  if (ha.targets) return ha.targets[m];
  return ((m % ha.T_seq) < ha.T_seq - 1) ? ha.idx[m + 1] : -1;
}

}  // namespace gptmi
