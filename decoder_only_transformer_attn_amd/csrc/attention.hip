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
// U^T rows hold 64 keys as 32 key pairs; pair p of row d is stored at pair
// slot p ^ vt_swz(d).  With a row stride of 68 elements (34 banks) the 32
// rows one ds_read_b64 phase touches start on 32 distinct even banks, and the
// transposed stores (8 rows d, d+8, ... by 8 key pairs per instruction) land
// on 64 distinct banks because rows 32 apart are shifted by 8 pairs.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 5) & 1) << 3; }

template <> struct VtFrag<bf16> {
  static constexpr int NI = 2;  // instructions per 32 keys
  // keys k0 .. k0+3 (k0 % 4 == 0) of row d: pairs k0/2, k0/2+1 stay adjacent
  static __device__ __forceinline__ uint2 keys4(const bf16* row, int d, int k0) {
    return *reinterpret_cast<const uint2*>(row + 2 * ((k0 >> 1) ^ vt_swz(d)));
  }
  static __device__ __forceinline__ bf16x8 load(const bf16* row, int d, int kbase, int hh, int g) {
    const uint2 lo = keys4(row, d, kbase + 16 * hh + 4 * g);
    const uint2 hi = keys4(row, d, kbase + 16 * hh + 8 + 4 * g);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
  static __device__ __forceinline__ bf16x8 pack(const f32x16& p, int hh) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[8 * hh + 2 * e], p[8 * hh + 2 * e + 1]);
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
};

// fp32: instruction hh (0..15) consumes register r = hh: key (hh/4)*8 + 4g + hh%4.
template <> struct VtFrag<float> {
  static constexpr int NI = 16;
  static __device__ __forceinline__ float load(const float* row, int d, int kbase, int hh, int g) {
    const int k = kbase + (hh >> 2) * 8 + 4 * g + (hh & 3);
    return row[2 * ((k >> 1) ^ vt_swz(d)) + (k & 1)];
  }
  static __device__ __forceinline__ float pack(const f32x16& p, int hh) { return p[hh]; }
};

// Block: 4 waves, 32 queries each (BQ = 128); key/value tiles of BKV keys,
// double-buffered in LDS: the global loads of tile k+1 are issued into
// registers before tile k is multiplied and written to the other buffer
// after it, so their latency hides under the tile's MFMA and softmax work.
template <typename T, int DP, int BKV>
__global__ void __launch_bounds__(256) attn_fwd_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  constexpr int BQ = 128;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LDKS = DP + VEC;    // padded LDS row of K (elements)
  constexpr int LDVS = BKV + 4;     // LDS row of U^T (see vt_swz)
  static_assert(BKV == 64, "the U^T swizzle assumes 64-key tiles");
  constexpr int NDI = DP / MF::KPI; // MFMA k steps over the head dim
  constexpr int NDT = DP / 32;      // 32-row d tiles of O^T
  constexpr int NST = BKV / 32;     // 32-key sub-tiles per KV tile
  constexpr int KTOT = BKV * (DP / VEC), UTOT = (BKV / 2) * (DP / VEC);   // items per tile
  constexpr int KCH = (KTOT + 255) / 256, UCH = (UTOT + 255) / 256;        // per thread
  __shared__ __align__(16) T sK[2][BKV * LDKS];
  __shared__ __align__(16) T sV[2][DP * LDVS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  // 1-D grid over work items sorted longest first (query tile major: the
  // blocks with the most key tiles first).  Consecutive rounds of 256 blocks
  // (one per CU) take the order alternately forwards and backwards, so a CU
  // that drew one of the longest items in one round draws one of the
  // shortest in the next: at B8 T1024 (three blocks per CU) the busiest CU
  // walks 28 key tiles instead of 34.
  const int nbh = a.B * a.H;
  const int nqt = (a.T_seq + BQ - 1) / BQ;
  const int nitems = nqt * nbh;
  int item = (int)blockIdx.x;
  {
    constexpr int ROUND = 256;
    const int r = item / ROUND, base = r * ROUND;
    if (r & 1) item = base + (min(ROUND, nitems - base) - 1 - (item - base));
  }
  const int qt = nqt - 1 - item / nbh;
  const int bh = item % nbh;
  const int b = bh / a.H, h = bh - b * a.H;
  const int q0 = qt * BQ;
  const int qw0 = q0 + wave * 32;
  const int qcol = qw0 + (lane & 31);
  const int T_seq = a.T_seq, D = a.D;

  // grouped-query attention: query head h reads K/U head h / (H / Hkv)
  const int hk = h / (a.H / a.Hkv);
  const T* Q = reinterpret_cast<const T*>(a.q) + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const T* K = reinterpret_cast<const T*>(a.k) + (long long)b * a.k_sb + (long long)hk * a.k_sh;
  const T* U = reinterpret_cast<const T*>(a.v) + (long long)b * a.v_sb + (long long)hk * a.v_sh;
  const int qst = a.q_st, kst = a.k_st, vst = a.v_st;

  // Q^T fragments (B operand) for this lane's query column.
  typename MF::frag qf[NDI];
#pragma unroll
  for (int i = 0; i < NDI; ++i) {
    const int d0 = i * MF::KPI + g * MF::KPL;
    if (qcol < T_seq && d0 < D) qf[i] = MF::load(Q + (long long)qcol * qst + d0);
    else qf[i] = typename MF::frag{};
  }

  // prefetch registers: K chunks and U key pairs.  Buffer loads: keys past the
  // sequence lie outside the resources and chunks past D (or past the tile)
  // take an offset outside them, so every such read is zero without a branch;
  // the per-thread offsets are fixed and the tile start is added to them (the
  // range check covers the VGPR offset; OOB_OFFSET plus a tile start stays
  // outside every resource).
  struct RegSet { uint4 kr[KCH], ur0[UCH], ur1[UCH]; };
  // a resource covers rows 0 .. T-1 exactly (the last one only up to D)
  const __amdgpu_buffer_rsrc_t rsk = make_rsrc(K, (uint32_t)(((size_t)(T_seq - 1) * kst + D) * sizeof(T)));
  const __amdgpu_buffer_rsrc_t rsu = make_rsrc(U, (uint32_t)(((size_t)(T_seq - 1) * vst + D) * sizeof(T)));
  uint32_t koff[KCH], uoff[UCH];
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int ch = tid + c * 256, row = ch / (DP / VEC), dc = (ch % (DP / VEC)) * VEC;
    koff[c] = (ch < KTOT && dc < D) ? (uint32_t)((row * kst + dc) * sizeof(T)) : OOB_OFFSET;
  }
#pragma unroll
  for (int c = 0; c < UCH; ++c) {
    const int ch = tid + c * 256, kp = (ch / (DP / VEC)) * 2, dc = (ch % (DP / VEC)) * VEC;
    uoff[c] = (ch < UTOT && dc < D) ? (uint32_t)((kp * vst + dc) * sizeof(T)) : OOB_OFFSET;
  }
  auto gload = [&](RegSet& R, int kb) {
    const uint32_t sk = (uint32_t)(kb * kst * sizeof(T)), sv = (uint32_t)(kb * vst * sizeof(T));
#pragma unroll
    for (int c = 0; c < KCH; ++c) R.kr[c] = buf_load16(rsk, koff[c] + sk, 0);
#pragma unroll
    for (int c = 0; c < UCH; ++c) {
      R.ur0[c] = buf_load16(rsu, uoff[c] + sv, 0);
      R.ur1[c] = buf_load16(rsu, (uoff[c] == OOB_OFFSET ? OOB_OFFSET : uoff[c] + (uint32_t)(vst * sizeof(T))) + sv, 0);
    }
  };
  // K as is; U transposed to U^T [d][key], written as (key, key+1) pairs
  auto sstore = [&](const RegSet& R, int buf) {
    const uint4 (&kr)[KCH] = R.kr;
    const uint4 (&ur0)[UCH] = R.ur0;
    const uint4 (&ur1)[UCH] = R.ur1;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int ch = tid + c * 256, row = ch / (DP / VEC), dc = (ch % (DP / VEC)) * VEC;
      if (ch < KTOT) *reinterpret_cast<uint4*>(&sK[buf][row * LDKS + dc]) = kr[c];
    }
#pragma unroll
    for (int c = 0; c < UCH; ++c) {
      const int ch = tid + c * 256, kp = (ch / (DP / VEC)) * 2, dc = (ch % (DP / VEC)) * VEC;
      if (ch >= UTOT) continue;
      T u0[VEC], u1[VEC];
      *reinterpret_cast<uint4*>(u0) = ur0[c];
      *reinterpret_cast<uint4*>(u1) = ur1[c];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        T* dst = &sV[buf][(dc + e) * LDVS + 2 * ((kp >> 1) ^ vt_swz(dc + e))];   // pair-aligned
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint32_t*>(dst) = uint32_t(u0[e]) | (uint32_t(u1[e]) << 16);
        else
          *reinterpret_cast<float2*>(dst) = make_float2(u0[e], u1[e]);
      }
    }
  };

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;   // exponent reference (log2 domain) and lane-partial sum
  const float sc = a.scale_log2;
  // ALiBi slope m_h = 2^(-8 (h+1) / H) divided by the 1/sqrt(D) score scale
  const float alibi_k = a.alibi ? exp2f(-8.0f * (float)(h + 1) / (float)a.H) * sqrtf((float)D) : 0.f;

  const int kv_end = min(T_seq, q0 + BQ);  // keys [0, kv_end) can be visible to this block
  // one key tile: scores, online softmax, O^T update, from LDS buffer `cur`
  auto tile = [&](int kb, int cur) {
    if (kb <= qw0 + 31) {  // otherwise every key of this tile is in this wave's future
      f32x16 s[NST];
#pragma unroll
      for (int st = 0; st < NST; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
        const T* krow = &sK[cur][(st * 32 + (lane & 31)) * LDKS + g * MF::KPL];
#pragma unroll
        for (int i = 0; i < NDI; ++i) s[st] = MF::mma(MF::load(krow + i * MF::KPI), qf[i], s[st]);
      }
      if (alibi_k != 0.f) {   // ALiBi (uniform): + (m_h sqrt D)(j - t), i.e. -m_h (t - j) after the 1/sqrt D scale
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[st][r] = fmaf(alibi_k, (float)(kb + st * 32 + acc_row(r, lane) - qcol), s[st][r]);
      }
      if (kb + BKV - 1 > qw0) {   // diagonal tile: mask keys after the query
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb + st * 32 + acc_row(r, lane) > qcol) s[st][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sc;
      // The exponent reference moves only when the tile's maximum exceeds it
      // by more than 8 (log2 units): probabilities stay below 2^8, which fp32
      // sums and bf16 P tolerate, and the O rescale below is skipped whenever
      // no lane of the wave moved its reference (alpha == 1 exactly).
      const float m_new = mx > m_run + 8.f ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[st][r], sc, -m_new));
          s[st][r] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      }
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int hh = 0; hh < VtFrag<T>::NI; ++hh) {
          const auto pb = VtFrag<T>::pack(s[st], hh);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int d = dt * 32 + (lane & 31);
            const T* vrow = &sV[cur][d * LDVS];
            acc[dt] = MF::mma(VtFrag<T>::load(vrow, d, st * 32, hh, g), pb, acc[dt]);
          }
        }
    }
  };
  // Global loads run two tiles ahead (register sets RA and RB in turn): tile
  // t + 2 is requested while tile t is computed, and tile t + 1, requested
  // one tile earlier, is written to the other LDS buffer after it.  A block
  // walks up to T / 64 tiles one after another, so the load latency has to
  // hide under more than one tile's work.
  RegSet RA, RB;
  gload(RA, 0);
  sstore(RA, 0);
  __syncthreads();
  if (BKV < kv_end) gload(RA, BKV);
  for (int kb = 0, it = 0; kb < kv_end;) {
    if (kb + 2 * BKV < kv_end) gload(RB, kb + 2 * BKV);
    tile(kb, it & 1);
    if (kb + BKV < kv_end) sstore(RA, (it + 1) & 1);
    __syncthreads();
    kb += BKV;
    ++it;
    if (kb >= kv_end) break;
    if (kb + 2 * BKV < kv_end) gload(RA, kb + 2 * BKV);
    tile(kb, it & 1);
    if (kb + BKV < kv_end) sstore(RB, (it + 1) & 1);
    __syncthreads();
    kb += BKV;
    ++it;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  // the row's log-sum-exp of the scaled scores in log2 units (both lane
  // halves hold the same reference m_run and total)
  if (a.lse2 != nullptr && qcol < T_seq && g == 0) a.lse2[(long long)bh * T_seq + qcol] = m_run + __log2f(l_tot);
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

// ---------------------------------------------------------------------------
// bf16, head width 64: key/value tiles of 64 rows reach LDS by direct-to-LDS
// DMA in their natural [key][d] layout (128-byte rows), K tiles and U tiles
// in two rings of NS stages each; the value operand of O^T = U^T P^T (8
// consecutive keys of one column d per lane) is read with gfx950's
// transposing LDS read ds_read_b64_tr_b16, so no register transpose is
// needed.  Within a group of 16 lanes that instruction returns to lane
// 4a + b element b of the 4-element rows addressed by lanes a, a + 4, a + 8
// and a + 12: when lane j addresses row kb + j / 4 at column d0 + 4 (j % 4),
// lane i receives rows kb .. kb + 3 of column d0 + i.  The 16-byte chunks of
// a row are XOR-swizzled by f(r) (bits 1..3 of the row, reordered) so that
// both the key fragments (16 rows, one chunk) and the transposing reads (4
// rows, 4 chunks) hit distinct bank groups.
//
// Software pipeline, per wave and key tile j: the MFMAs of the scores of
// tile j + 1 and of the product P_{j-1} U_{j-1} have no dependence on the
// softmax of tile j, so one basic block issues all three, and scheduling
// groups interleave about eight VALU operations of the softmax into the
// shadow of every MFMA.  Tile t's K is used at step t - 1 and its U at step
// t + 1; one barrier serves two steps: before step j (j even) the block
// loads K(j + 3), K(j + 4), U(j + 1) and U(j + 2) into the stages that
// steps j - 2 and j - 1 left, two steps before each is read.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kv_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource words over [base, base + bytes) (loads beyond read zero).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
// One direct-to-LDS load of 16 bytes per lane: lane l's bytes land at
// dst + 16 l.  Issued from inline assembly so that the compiler does not
// make every later LDS read wait for all loads in flight (it cannot tell
// the stages apart); the kernel's own vmcnt waits and barriers order each
// stage's reads after its loads.
__device__ __forceinline__ void dma16(const __attribute__((address_space(3))) char* dst, i32x4 rsrc,
                                      uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile("buffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "{m0}"(m0), "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int NS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_d64_kernel(AttnArgs a) {
  static_assert(NS == 4, "stage offsets are folded into 16-bit LDS immediates for four stages");
  constexpr int D = 64, BQ = 128, BKV = 64, TILE = BKV * 128;   // bytes of K (or U) per tile
  typedef Mfma<bf16> MF;
  __shared__ __align__(1024) char ring[2 * NS][TILE];            // K stages, then U stages
  typedef __attribute__((address_space(3))) char lch;
  lch* const lring = (lch*)&ring[0][0];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // work items sorted longest first, rounds of 256 alternately reversed (see attn_fwd_kernel)
  const int nbh = a.B * a.H;
  const int nqt = (a.T_seq + BQ - 1) / BQ;
  const int nitems = nqt * nbh;
  int item = (int)blockIdx.x;
  {
    constexpr int ROUND = 256;
    const int r = item / ROUND, base = r * ROUND;
    if (r & 1) item = base + (min(ROUND, nitems - base) - 1 - (item - base));
  }
  const int qt = nqt - 1 - item / nbh, bh = item % nbh;
  const int b = bh / a.H, h = bh - b * a.H, hk = h / (a.H / a.Hkv);
  const int T_seq = a.T_seq;
  const int q0 = qt * BQ, qw0 = q0 + wave * 32, qcol = qw0 + (lane & 31);
  const bf16* Q = reinterpret_cast<const bf16*>(a.q) + (long long)b * a.q_sb + (long long)h * a.q_sh;
  const bf16* K = reinterpret_cast<const bf16*>(a.k) + (long long)b * a.k_sb + (long long)hk * a.k_sh;
  const bf16* U = reinterpret_cast<const bf16*>(a.v) + (long long)b * a.v_sb + (long long)hk * a.v_sh;
  const int kst = a.k_st, vst = a.v_st;

  // Q^T fragments of this lane's query column, read from LDS in the prologue
  MF::frag qf[4];

  // DMA plan: a K (or U) tile is 8 loads of 1 KB (8 rows each); wave w sends
  // loads w and w + 4 of each.  Lane l writes slot l % 8 of row
  // 8 (i % 8) + l / 8, so it fetches chunk slot ^ f(row) of that row.  Rows
  // past the sequence lie outside the resources and arrive as zeros: the
  // whole byte offset goes in the VGPR offset, which the range check covers.
  const i32x4 rsk = rsrc_words(K, (uint32_t)(((size_t)(T_seq - 1) * kst + D) * 2));
  const i32x4 rsu = rsrc_words(U, (uint32_t)(((size_t)(T_seq - 1) * vst + D) * 2));
  const int rA = 8 * wave + (lane >> 3), rB = rA + 32, sl = lane & 7;
  const uint32_t koffA = (uint32_t)((rA * kst + (sl ^ kv_swz(rA)) * 8) * 2);
  const uint32_t koffB = (uint32_t)((rB * kst + (sl ^ kv_swz(rB)) * 8) * 2);
  const uint32_t voffA = (uint32_t)((rA * vst + (sl ^ kv_swz(rA)) * 8) * 2);
  const uint32_t voffB = (uint32_t)((rB * vst + (sl ^ kv_swz(rB)) * 8) * 2);
  // Each wave's 32 query rows reach LDS the same way (4 loads of 8 rows),
  // into a stage that the first loads of step 0 overwrite: K stage 3 for
  // waves 0 and 1, U stage 2 for waves 2 and 3.  Read through LDS, they
  // leave no register loads that a wait for them would order after every
  // tile load in flight.
  const i32x4 rsq = rsrc_words(Q, (uint32_t)(((size_t)(T_seq - 1) * a.q_st + D) * 2));
  lch* const qarea = lring + (wave < 2 ? (NS - 1) * TILE : (NS + 2) * TILE) + (wave & 1) * 4096;

  const int kv_end = min(T_seq, q0 + BQ);
  const int nt = (kv_end + BKV - 1) / BKV;                        // key tiles of this block
  const int lw = qw0 < T_seq ? min(qw0 + 31, T_seq - 1) / BKV : -1;   // this wave's last tile

  // direct-to-LDS loads of K(t) and U(t) into their stages (t % NS), those that exist
  auto issue_k = [&](int t) {
    if (t >= 0 && t < nt) {
      lch* st = lring + (t & (NS - 1)) * TILE;
      const uint32_t sk = (uint32_t)(t * BKV * kst * 2);
      dma16(st + wave * 1024, rsk, koffA + sk, 0);
      dma16(st + (wave + 4) * 1024, rsk, koffB + sk, 0);
    }
  };
  auto issue_u = [&](int t) {
    if (t >= 0 && t < nt) {
      lch* st = lring + (NS + (t & (NS - 1))) * TILE;
      const uint32_t sv = (uint32_t)(t * BKV * vst * 2);
      dma16(st + wave * 1024, rsu, voffA + sv, 0);
      dma16(st + (wave + 4) * 1024, rsu, voffB + sv, 0);
    }
  };
  // wait until at most n of this lane's loads are in flight (n even, <= 8)
  auto wait_loads = [&](int n) {
    if (n >= 8) __builtin_amdgcn_s_waitcnt(0x70 | 0xF00 | 8);
    else if (n >= 6) __builtin_amdgcn_s_waitcnt(0x70 | 0xF00 | 6);
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x70 | 0xF00 | 4);
    else if (n >= 2) __builtin_amdgcn_s_waitcnt(0x70 | 0xF00 | 2);
    else __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
  };

  // Per-lane LDS offsets within a stage; the stage and the row-block parts
  // are compile-time and fold into the instructions' immediates (rows
  // 16 hh + 32 rb leave f(r) unchanged).
  int kofs[4], uofs[2][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int r = lane & 31, c = ks * 2 + g;
    kofs[ks] = r * 128 + ((c ^ kv_swz(r)) << 4);
  }
  {
    const int G = lane >> 4, i = lane & 15, half = G & 1;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) {
      const int c = 4 * ob + 2 * half + ((i & 3) >> 1);
      const int r0 = g * 4 + (i >> 2), r1 = r0 + 8;
      uofs[ob][0] = r0 * 128 + ((c ^ kv_swz(r0)) << 4) + ((i & 1) << 3);
      uofs[ob][1] = r1 * 128 + ((c ^ kv_swz(r1)) << 4) + ((i & 1) << 3);
    }
  }
  // score fragment: K rows 32 rb + lane % 32, k step ks, of K stage st
  auto kfrag = [&](const lch* st, int rb, int ks) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(st + kofs[ks] + rb * 4096);
  };
  // U^T fragment for O^T rows d = 32 ob + lane % 32, keys 32 rb + 16 hh + 4 g + {0..3, 8..11}
  auto vfrag = [&](const lch* st, int ob, int rb, int hh) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(st + uofs[ob][0] + rb * 4096 + hh * 2048));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(st + uofs[ob][1] + rb * 4096 + hh * 2048));
    return __builtin_bit_cast(bf16x8, i16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
  };

  f32x16 o[2], sa[2], sb[2];
  bf16x8 pa[2][2], pb[2][2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { o[0][r] = 0.f; o[1][r] = 0.f; }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) pb[rb][hh] = bf16x8{};
  // exponent reference (log2 domain), lane-partial row sum, and the factor
  // that O still owes for the last move of the reference
  float m_run = -INFINITY, l_run = 0.f, alpha_o = 1.f;
  const float sc = a.scale_log2;

  auto scores = [&](f32x16 (&sx)[2], const lch* st) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sx[rb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sx[rb] = MF::mma(kfrag(st, rb, ks), qf[ks], sx[rb]);
    }
  };
  auto pv = [&](const bf16x8 (&pp)[2][2], const lch* st) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int ob = 0; ob < 2; ++ob) o[ob] = MF::mma(vfrag(st, ob, rb, hh), pp[rb][hh], o[ob]);
  };
  auto rescale_o = [&]() {
    if (__builtin_amdgcn_ballot_w64(alpha_o != 1.f)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[0][r] *= alpha_o;
        o[1][r] *= alpha_o;
      }
    }
    alpha_o = 1.f;
  };
  // causal mask of this wave's diagonal tile kb .. kb + 63, in place
  auto mask = [&](f32x16 (&s)[2], int kb) {
    const int e = qcol - kb - 4 * g;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (rb * 32 + (r >> 2) * 8 + (r & 3) > e) s[rb][r] = -INFINITY;
  };
  // One pipeline step's arithmetic in 16 MFMA slots.  Slot k issues MFMA
  // k (even: score MFMA k / 2 of tile j + 1, odd: product MFMA k / 2 of
  // tile j - 1), the fragment read of MFMA k + 4, and a share of the online
  // softmax of tile j that takes about as long as one MFMA: the row maximum
  // in slots 0-2, then one pair of probabilities per slot (2 FMA, 2 exp2, a
  // bf16 pack and its row-sum dot product).  sched_barrier keeps the slots
  // apart, so every MFMA runs in the shadow of VALU work and each fragment
  // read has four slots to land.  The exponent reference moves only by > 8
  // (log2 units); the probabilities (bf16, B-operand layout) go to pc.
  auto region = [&](auto S_, const f32x16 (&s)[2], f32x16 (&sn)[2], const bf16x8 (&pp)[2][2],
                    bf16x8 (&pc)[2][2]) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value;
    const lch* kst = lring + ((S + 1) & (NS - 1)) * TILE;             // K of tile j + 1
    const lch* ust = lring + (NS + ((S + NS - 1) & (NS - 1))) * TILE;  // U of tile j - 1
    // score MFMA i: row block i % 2, k step i / 2; product MFMA i: ob = i % 2,
    // hh = (i / 2) % 2, rb = i / 4 (consecutive MFMAs of a kind alternate accumulators)
    bf16x8 fr[16];
    auto load = [&](auto K_) __attribute__((always_inline)) {
      constexpr int k = decltype(K_)::value, i = k / 2;
      if constexpr (k % 2 == 0) fr[k] = kfrag(kst, i % 2, i / 2);
      else fr[k] = vfrag(ust, i % 2, i / 4, (i / 2) % 2);
    };
    float mx = -INFINITY, m_new = 0.f, alpha = 1.f, psum = 0.f;
    uint32_t w[16];
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    auto pair = [&](auto P_) __attribute__((always_inline)) {
      constexpr int p = decltype(P_)::value, rb = p / 8, c = (p % 8) * 2;
      const float p0 = fast_exp2(fmaf(s[rb][c], sc, -m_new));
      const float p1 = fast_exp2(fmaf(s[rb][c + 1], sc, -m_new));
      w[p] = pack_bf16x2(p0, p1);
      // the row sum of the probabilities as they enter the product (bf16)
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[p]), ones, psum, false);
    };
    static_for<0, 4>([&](auto K_) __attribute__((always_inline)) { load(K_); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, 16>([&](auto K_) __attribute__((always_inline)) {
      constexpr int k = decltype(K_)::value, i = k / 2;
      if constexpr (k % 2 == 0) {
        if constexpr (i / 2 == 0) sn[i % 2] = MF::mma(fr[k], qf[0], f32x16{});
        else sn[i % 2] = MF::mma(fr[k], qf[i / 2], sn[i % 2]);
      } else {
        o[i % 2] = MF::mma(fr[k], pp[i / 4][(i / 2) % 2], o[i % 2]);
      }
      if constexpr (k + 4 < 16) load(std::integral_constant<int, k + 4>{});
      if constexpr (k < 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[k][r]);
      } else if constexpr (k == 2) {
        // lanes l and l ^ 32 hold the other keys of the same query: both
        // halves of the swap carry the pair, in every lane
        const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1])) * sc;
        m_new = mx > m_run + 8.f ? mx : m_run;
        alpha = fast_exp2(m_run - m_new);
      } else {
        pair(std::integral_constant<int, k - 3>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<13, 16>([&](auto P_) __attribute__((always_inline)) { pair(P_); });
#pragma unroll
    for (int q = 0; q < 4; ++q)
      pc[q / 2][q % 2] = __builtin_bit_cast(bf16x8, make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]));
    l_run = l_run * alpha + psum;
    m_run = m_new;
    alpha_o = alpha;
  };

  // Before every even step j: K(j + 1), K(j + 2), U(j - 1) and U(j), the
  // tiles of steps j and j + 1, were loaded before step j - 2; wait for this
  // wave's loads, then the barrier publishes everyone's.  Every wave is then
  // done with steps j - 2 and j - 1, which read K(j - 1), K(j), U(j - 3) and
  // U(j - 2): their stages take K(j + 3), K(j + 4), U(j + 1) and U(j + 2),
  // which steps j + 2 and j + 3 read.  One barrier per two key tiles.
  auto sync2 = [&](int j) {
    __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
    __syncthreads();
    issue_k(j + 3);
    issue_k(j + 4);
    issue_u(j + 1);
    issue_u(j + 2);
  };
  // one step of the pipeline, stage S = j % NS: tile j's scores are in s and
  // tile j - 1's probabilities in pp (zeros, against a zeroed U stage, at j = 0)
  auto step = [&](auto S_, int j, f32x16 (&s)[2], f32x16 (&sn)[2], const bf16x8 (&pp)[2][2],
                  bf16x8 (&pc)[2][2]) __attribute__((always_inline)) {
    if (j > lw) return;                   // every key of tile j is in this wave's future
    if (j == lw) mask(s, j * BKV);
    rescale_o();
    region(S_, s, sn, pp, pc);
  };

  // prologue: K(0), this wave's Q rows, then K(1), K(2) and U(0) in flight;
  // a zeroed U stage stands in for tile -1; scores of tile 0 once K(0) and
  // Q have landed
  issue_k(0);
  {
    const int r = lane >> 3, sl8 = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = 8 * i + r;
      dma16(qarea + i * 1024, rsq, (uint32_t)(((qw0 + rl) * a.q_st + (sl8 ^ kv_swz(rl)) * 8) * 2), 0);
    }
  }
  issue_k(1);
  issue_k(2);
  issue_u(0);
  {
    lch* z = lring + (2 * NS - 1) * TILE + tid * 32;
    *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(z) = u32x4_t{0, 0, 0, 0};
    *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(z + 16) = u32x4_t{0, 0, 0, 0};
  }
  wait_loads((nt > 1 ? 2 : 0) + (nt > 2 ? 2 : 0) + 2);   // (K(1), K(2), U(0) may still fly)
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(qarea + kofs[ks]);
  scores(sa, lring);
  for (int j = 0; j < nt; j += NS) {
    sync2(j);
    step(std::integral_constant<int, 0>{}, j, sa, sb, pb, pa);
    if (j + 1 >= nt) break;
    step(std::integral_constant<int, 1>{}, j + 1, sb, sa, pa, pb);
    if (j + 2 >= nt) break;
    sync2(j + 2);
    step(std::integral_constant<int, 2>{}, j + 2, sa, sb, pb, pa);
    if (j + 3 >= nt) break;
    step(std::integral_constant<int, 3>{}, j + 3, sb, sa, pa, pb);
  }
  // the last tile's product: its U stage, once every wave's loads landed
  __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
  __syncthreads();
  if (lw >= 0) {
    rescale_o();
    const lch* st = lring + (NS + (lw & (NS - 1))) * TILE;
    if (lw & 1) pv(pb, st);
    else pv(pa, st);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (a.lse2 != nullptr && qcol < T_seq && g == 0) a.lse2[(long long)bh * T_seq + qcol] = m_run + __log2f(l_tot);
  if (qcol < T_seq) {
    bf16* orow = reinterpret_cast<bf16*>(a.o) + ((long long)b * T_seq + qcol) * a.o_ld + h * D;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = ob * 32 + q * 8 + g * 4;
        *reinterpret_cast<uint2*>(orow + d) =
            make_uint2(pack_bf16x2(o[ob][4 * q] * inv, o[ob][4 * q + 1] * inv),
                       pack_bf16x2(o[ob][4 * q + 2] * inv, o[ob][4 * q + 3] * inv));
      }
  }
}

template <typename T>
static hipError_t attn_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid(((a.T_seq + 127) / 128) * a.B * a.H), block(256);
  if constexpr (sizeof(T) == 2) {
    // 16-byte aligned rows (DMA of whole 128-byte rows) and no distance bias
    const bool rows16 = a.k_st % 8 == 0 && a.v_st % 8 == 0 && a.q_st % 8 == 0 && a.o_ld % 4 == 0 &&
                        ((uintptr_t)a.k & 15) == 0 && ((uintptr_t)a.v & 15) == 0 && ((uintptr_t)a.q & 15) == 0;
    if (a.D == 64 && !a.alibi && rows16) {
      hipLaunchKernelGGL((attn_fwd_d64_kernel<4>), grid, block, 0, st, a);
      return hipGetLastError();
    }
  }
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

// Decode step: the one new query of each (b, h) against cache positions
// 0 .. *pos (its own K/U were appended at *pos by the QKV epilogue), the
// KV-cache form of the same causal attention ("预训练一个 Mini GPT", KV
// cache: only the new token's q, k, u are computed; earlier k, u are read
// back).  One block of 256 threads per (b, h), a single pass over the cache:
// a key row of D values is cut into 16-byte chunks held by LPK adjacent lanes
// (8 lanes for D = 64 in bf16), and group g of LPK lanes takes keys g, g + G,
// ... (G = 256 / LPK groups), loading the key's K and U chunks together, UNR
// keys at a time.  Each group keeps an online softmax of its own keys (running
// maximum, sum and U-weighted sum, rescaled once per batch of UNR keys); the
// G partial states meet in LDS at the end.  HBM-bound: every cached K and U row
// of positions 0 .. *pos is read once, with one round trip of latency per UNR
// keys of a group (one in all for up to 256 positions).
constexpr int DEC_MAXT = 4096;
constexpr int DEC_THREADS = 256;

template <typename T>
__device__ __forceinline__ void chunk_f32(const uint4& v, float (&o)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void chunk_f32<bf16>(const uint4& v, float (&o)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void chunk_f32<float>(const uint4& v, float (&o)[4]) {
  o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y); o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}

// One block per (b, h).  The first batch of UNR keys per group (positions
// up to UNR G - 1: the whole cache for up to 256 positions) is requested
// before the query is ready, so the cache round trip overlaps the prologue's
// (the query's, or the slices' of the fused kernel); the prologue then meets
// the other waves at a bare barrier that leaves those loads in flight.
template <typename T, int LPK>
struct DecPass {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int UNR = 8;
  static constexpr int G = DEC_THREADS / LPK;
  const T* K; const T* U;
  int n, g, c, D;
  bool act;
  __device__ __forceinline__ DecPass(const DecAttnArgs& a) {
    const int tid = threadIdx.x, bh = blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    D = a.D;
    g = tid / LPK; c = tid - g * LPK;
    act = c * VEC < D;                        // lanes past the row's chunks hold zeros
    n = *a.pos + 1;
    n = n < 1 ? 1 : (n < a.Tmax ? n : a.Tmax);   // a position outside [0, Tmax) violates the contract
    const int kvbh = b * a.Hkv + h / (a.H / a.Hkv);   // grouped-query attention
    K = reinterpret_cast<const T*>(a.k) + (long long)kvbh * a.kv_bh + c * VEC;
    U = reinterpret_cast<const T*>(a.v) + (long long)kvbh * a.kv_bh + c * VEC;
  }
  __device__ __forceinline__ void load(int k0, uint4 (&kv)[UNR], uint4 (&uv)[UNR]) const {
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int k = k0 + u * G + g;
      const bool in = act && k < n;
      kv[u] = in ? *reinterpret_cast<const uint4*>(K + (long long)k * D) : z;
      uv[u] = in ? *reinterpret_cast<const uint4*>(U + (long long)k * D) : z;
    }
  }
};

// Everything after the prologue: scores, online softmax and U sums of the
// group's keys (batch 0 already in kv / uv), then the combine of the groups.
// qs holds the query times scale_log2 (fp32, LDS).  Key position newpos (when
// knew is given) is taken from knew / unew in LDS instead of the cache.
template <typename T, int LPK>
__device__ __forceinline__ void dec_attend(const DecAttnArgs& a, const DecPass<T, LPK>& P, const float* qs,
                                           uint4 (&kv)[DecPass<T, LPK>::UNR], uint4 (&uv)[DecPass<T, LPK>::UNR],
                                           const T* knew, const T* unew, int newpos) {
  typedef DecPass<T, LPK> PS;
  constexpr int VEC = PS::VEC, UNR = PS::UNR, G = PS::G;
  __shared__ float gacc[G * LPK * VEC];   // per group: U-weighted sums, columns [0, LPK VEC)
  __shared__ float gm[G], gl[G];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H, D = a.D;
  const int g = P.g, c = P.c, n = P.n;
  float qv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) qv[e] = P.act ? qs[c * VEC + e] : 0.f;

  float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  const float alibi_l2 = a.alibi ? exp2f(-8.0f * (float)(h + 1) / (float)a.H) * 1.4426950408889634f : 0.f;
  for (int k0 = 0; k0 < n; k0 += UNR * G) {
    if (k0 > 0) P.load(k0, kv, uv);
    if (knew && P.act && newpos >= k0 && newpos < k0 + UNR * G) {   // uniform range test
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (k0 + u * G + g == newpos) {
          kv[u] = *reinterpret_cast<const uint4*>(knew + c * VEC);
          uv[u] = *reinterpret_cast<const uint4*>(unew + c * VEC);
        }
    }
    float s[UNR];
    float mb = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float kf[VEC];
      chunk_f32<T>(kv[u], kf);
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) t = fmaf(qv[e], kf[e], t);
#pragma unroll
      for (int o = LPK >> 1; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
      if (alibi_l2 != 0.f) t = fmaf(alibi_l2, (float)(k0 + u * G + g - (n - 1)), t);   // -m_h (pos - j), log2 units
      s[u] = k0 + u * G + g < n ? t : -INFINITY;
      mb = fmaxf(mb, s[u]);
    }
    const float m_new = fmaxf(m, mb);
    if (m_new == -INFINITY) continue;       // no key of this group in the batch
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float pw = fast_exp2(s[u] - m_new);   // 0 for keys past n
      l += pw;
      float uf[VEC];
      chunk_f32<T>(uv[u], uf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(pw, uf[e], acc[e]);
    }
    m = m_new;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) gacc[g * LPK * VEC + c * VEC + e] = acc[e];
  if (c == 0) { gm[g] = m; gl[g] = l; }
  __syncthreads();
  // combine the groups: every group with keys has a finite maximum (group 0
  // holds key 0).  All threads take part: thread t sums the VEC groups of
  // quarter t / DP for column t % DP, then the quarters are added in order.
  constexpr int DP = LPK * VEC, QN = DEC_THREADS / DP;   // DP >= D columns, QN * VEC = G groups
  __shared__ float pnum[DEC_THREADS], pden[DEC_THREADS];
  float M = gm[0];
#pragma unroll
  for (int gg = 1; gg < G; ++gg) M = fmaxf(M, gm[gg]);
  {
    const int d = tid % DP, q = tid / DP;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int gg = q * VEC + i;
      const float w = fast_exp2(gm[gg] - M);   // 0 for a group without keys
      num = fmaf(w, gacc[gg * DP + d], num);
      den = fmaf(w, gl[gg], den);
    }
    pnum[tid] = num;
    pden[tid] = den;
  }
  __syncthreads();
  if (tid < D) {
    float num = pnum[tid], den = pden[tid];
#pragma unroll
    for (int q = 1; q < QN; ++q) {
      num += pnum[q * DP + tid];
      den += pden[q * DP + tid];
    }
    T* orow = reinterpret_cast<T*>(a.o) + (long long)b * a.o_ld + h * D;
    orow[tid] = from_f32<T>(num / den);
  }
}

// LDS writes of the prologue done, then a barrier that does not wait for the
// cache loads still in flight.
__device__ __forceinline__ void dec_prologue_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, int LPK>
__global__ void __launch_bounds__(DEC_THREADS) attn_decode_kernel(DecAttnArgs a) {
  typedef DecPass<T, LPK> PS;
  __shared__ float qs[128];
  const PS P(a);
  const int bh = blockIdx.x;
  const T* q = reinterpret_cast<const T*>(a.q) + (long long)bh * a.D;
  float qd = 0.f;
  if (threadIdx.x < a.D) qd = to_f32(q[threadIdx.x]) * a.scale_log2;   // D <= 128 < DEC_THREADS
  uint4 kv[PS::UNR], uv[PS::UNR];
  P.load(0, kv, uv);
  if (threadIdx.x < a.D) qs[threadIdx.x] = qd;
  dec_prologue_barrier();
  dec_attend<T, LPK>(a, P, qs, kv, uv, nullptr, nullptr, -1);
}

// The same attention fed by the K-slices of the Q|K|U product instead of a
// finished q and an appended cache row: part[s][B][3C] (C = H D, head h's q,
// k, u at columns hD, C + hD, 2C + hD).  The block adds its head's slices in
// slice order with the bias in fp32 and rounds to bf16, exactly the values
// the product's own epilogue stores; it appends k and u at *pos of the caches
// (for the later steps) and attends with the new row taken from LDS in place
// of the cache row its loads read (before the append, or not yet visible).
template <int LPK, int NS>
__global__ void __launch_bounds__(DEC_THREADS) attn_decode_slices_kernel(DecAttnArgs a, const float* __restrict__ part,
                                                                        const bf16* __restrict__ bias) {
  typedef DecPass<bf16, LPK> PS;
  __shared__ float qs[128];
  __shared__ __align__(16) bf16 kn[128];
  __shared__ __align__(16) bf16 un[128];
  const PS P(a);
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H, D = a.D, C3 = 3 * a.H * D;
  const int pos = *a.pos;
  const bool keep = pos >= 0 && pos < a.Tmax;   // the cache row the step appends
  // slices of this thread's q / k / u element (threads past 3D take none)
  const int i = threadIdx.x, which = i / D, d = i - which * D;
  const bool mine = i < 3 * D;
  const int col = which * (C3 / 3) + h * D + d;
  float ps[NS];   // every slice's load issued before the first add
  float bv = 0.f;
  if (mine) {
    const float* p = part + (long long)b * C3 + col;
#pragma unroll
    for (int s = 0; s < NS; ++s) ps[s] = p[(long long)s * a.B * C3];
    if (bias) bv = to_f32(bias[col]);
  }
  uint4 kv[PS::UNR], uv[PS::UNR];
  P.load(0, kv, uv);
  if (mine) {
    float t = ps[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) t += ps[s];
    t += bv;
    const bf16 r = from_f32<bf16>(t);
    bf16* row = reinterpret_cast<bf16*>(const_cast<void*>(which == 1 ? a.k : a.v)) + (long long)bh * a.kv_bh +
                (long long)pos * D;
    if (which == 0) {
      qs[d] = to_f32(r) * a.scale_log2;
    } else {
      (which == 1 ? kn : un)[d] = r;
      if (keep) row[d] = r;
    }
  }
  dec_prologue_barrier();
  // the new row from LDS: the cache copy a batch reads may predate the append
  dec_attend<bf16, LPK>(a, P, qs, kv, uv, kn, un, keep ? pos : -1);
}

template <int LPK>
static hipError_t dec_slices_s(const DecAttnArgs& a, const float* part, int S, const bf16* bias, hipStream_t st) {
  const dim3 grid(a.B * a.H), block(DEC_THREADS);
  switch (S) {
    case 1: hipLaunchKernelGGL((attn_decode_slices_kernel<LPK, 1>), grid, block, 0, st, a, part, bias); break;
    case 2: hipLaunchKernelGGL((attn_decode_slices_kernel<LPK, 2>), grid, block, 0, st, a, part, bias); break;
    case 3: hipLaunchKernelGGL((attn_decode_slices_kernel<LPK, 3>), grid, block, 0, st, a, part, bias); break;
    case 4: hipLaunchKernelGGL((attn_decode_slices_kernel<LPK, 4>), grid, block, 0, st, a, part, bias); break;
    case 6: hipLaunchKernelGGL((attn_decode_slices_kernel<LPK, 6>), grid, block, 0, st, a, part, bias); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_decode_slices(const DecAttnArgs& a, const float* part, int S, const void* bias,
                                          hipStream_t st) {
  if (!part || S <= 0 || a.Tmax > DEC_MAXT || a.D > 128 || a.D % 8 || a.Hkv != a.H || a.alibi)
    return hipErrorInvalidValue;
  const int nch = a.D / 8;
  const int lpk = nch <= 2 ? 2 : (nch <= 4 ? 4 : (nch <= 8 ? 8 : 16));
  const bf16* bb = static_cast<const bf16*>(bias);
  switch (lpk) {
    case 2: return dec_slices_s<2>(a, part, S, bb, st);
    case 4: return dec_slices_s<4>(a, part, S, bb, st);
    case 8: return dec_slices_s<8>(a, part, S, bb, st);
    default: return dec_slices_s<16>(a, part, S, bb, st);
  }
}

hipError_t launch_attention_decode(int dtype, const DecAttnArgs& a, hipStream_t st) {
  const int vec = dtype == 0 ? 4 : 8;
  if (a.Tmax > DEC_MAXT || a.D > 128 || a.D % vec) return hipErrorInvalidValue;
  // lanes per key: the row's 16-byte chunks rounded up to a power of two
  const int nch = a.D / vec;
  const int lpk = nch <= 2 ? 2 : (nch <= 4 ? 4 : (nch <= 8 ? 8 : (nch <= 16 ? 16 : 32)));
  const dim3 grid(a.B * a.H), block(DEC_THREADS);
  if (dtype == 0) {
    switch (lpk) {
      case 2: hipLaunchKernelGGL((attn_decode_kernel<float, 2>), grid, block, 0, st, a); break;
      case 4: hipLaunchKernelGGL((attn_decode_kernel<float, 4>), grid, block, 0, st, a); break;
      case 8: hipLaunchKernelGGL((attn_decode_kernel<float, 8>), grid, block, 0, st, a); break;
      case 16: hipLaunchKernelGGL((attn_decode_kernel<float, 16>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((attn_decode_kernel<float, 32>), grid, block, 0, st, a); break;
    }
  } else {
    switch (lpk) {
      case 2: hipLaunchKernelGGL((attn_decode_kernel<bf16, 2>), grid, block, 0, st, a); break;
      case 4: hipLaunchKernelGGL((attn_decode_kernel<bf16, 4>), grid, block, 0, st, a); break;
      case 8: hipLaunchKernelGGL((attn_decode_kernel<bf16, 8>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((attn_decode_kernel<bf16, 16>), grid, block, 0, st, a); break;
    }
  }
  return hipGetLastError();
}

// Rotary angles ("02 GPT 架构" §5.2): tab[p * D/2 + i] = (cos, sin) of
// p * theta^(-2i/D), computed in double and rounded once to float.
__global__ void __launch_bounds__(256) rope_table_kernel(float2* __restrict__ tab, int rows, int half, int D,
                                                         double theta) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * half) return;
  const int p = e / half, i = e - p * half;
  const double ang = (double)p * pow(theta, -2.0 * i / (double)D);
  tab[e] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_table(float2* tab, int rows, int D, double theta, hipStream_t st) {
  const int n = rows * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, tab, rows, D / 2, D, theta);
  return hipGetLastError();
}

}  // namespace gptmi
