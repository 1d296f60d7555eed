// Next-token sampling from rows of logits: repetition penalty, temperature,
// top-k, top-p (nucleus) and one inverse-CDF draw per row.
//
//   penalty      "02 GPT 架构" §8.4: the logit of a token that already
//                appeared is divided by alpha when positive and multiplied by
//                alpha when negative;
//   temperature  "预训练一个 Mini GPT" 第7步, "02 GPT 架构" §8.1: key = z'/T,
//                T <= 0 is the greedy choice (lowest index among equal maxima);
//   top-k        "02 GPT 架构" §8.2, "GPT-1学习笔记" §6.2: the k most probable;
//   top-p        "02 GPT 架构" §8.3, "GPT-1学习笔记" §6.2: of those, the
//                smallest most-probable prefix whose mass reaches p;
//   draw         "预训练一个 Mini GPT" 第7步: inverse CDF of the renormalised
//                candidates for the caller's uniform u in [0, 1).
//
// Candidate weights are w = exp(key - max key) computed in double and rounded
// once to float; candidates are ordered by descending w, equal w by ascending
// index, and the CDF walks that order.  Probability masses and thresholds
// are double sums of the float weights.
//
// One block of 1024 threads per row; thread t holds the contiguous slice
// [t * npt, t * npt + npt) of the vocabulary, in LDS and registers (npt <=
// 52, so V <= 53248).  Nothing is sorted: top-k, top-p and the draw each find a
// threshold on the weight's bit pattern (monotone for w >= 0) by a binary
// search whose every step is one block-wide count or double sum, then resolve
// the weights equal to the threshold in index order with a block-wide
// exclusive scan.  Every reduction and scan runs in a fixed order, so the
// result is deterministic.
#include "common.h"
#include "kernels.h"

namespace gptmi {

constexpr int SMP_THREADS = 1024, SMP_WAVES = SMP_THREADS / WAVE;

// Block-wide reductions and scans in thread order.  Each call uses one of two
// LDS buffers in turn (ph), so a call's writes never race with the previous
// call's reads and one barrier per call suffices.
struct SmpShared {
  double d[2][SMP_WAVES];
  int i[2][SMP_WAVES];
  float f[2][SMP_WAVES];
};

struct Blk {
  SmpShared* sh;
  int ph, lane, wave;

  __device__ __forceinline__ double sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) sh->d[ph][wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < SMP_WAVES; ++w) t += sh->d[ph][w];
    ph ^= 1;
    return t;
  }
  __device__ __forceinline__ int sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) sh->i[ph][wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < SMP_WAVES; ++w) t += sh->i[ph][w];
    ph ^= 1;
    return t;
  }
  __device__ __forceinline__ float max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if (lane == 0) sh->f[ph][wave] = v;
    __syncthreads();
    float t = sh->f[ph][0];
#pragma unroll
    for (int w = 1; w < SMP_WAVES; ++w) t = fmaxf(t, sh->f[ph][w]);
    ph ^= 1;
    return t;
  }
  // smallest value over the block (ints)
  __device__ __forceinline__ int min(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = ::min(v, __shfl_xor(v, o, 64));
    if (lane == 0) sh->i[ph][wave] = v;
    __syncthreads();
    int t = sh->i[ph][0];
#pragma unroll
    for (int w = 1; w < SMP_WAVES; ++w) t = ::min(t, sh->i[ph][w]);
    ph ^= 1;
    return t;
  }
  __device__ __forceinline__ int max(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = ::max(v, __shfl_xor(v, o, 64));
    if (lane == 0) sh->i[ph][wave] = v;
    __syncthreads();
    int t = sh->i[ph][0];
#pragma unroll
    for (int w = 1; w < SMP_WAVES; ++w) t = ::max(t, sh->i[ph][w]);
    ph ^= 1;
    return t;
  }
  // sum of v over the threads before this one
  template <typename X> __device__ __forceinline__ X exscan(X v) {
    X s = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const X y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    X ex = __shfl_up(s, 1, 64);
    if (lane == 0) ex = X(0);
    X* buf = slot(X(0));
    if (lane == 63) buf[wave] = s;
    __syncthreads();
    X base = X(0);
    for (int w = 0; w < wave; ++w) base += buf[w];
    ph ^= 1;
    return base + ex;
  }
  __device__ __forceinline__ double* slot(double) { return sh->d[ph]; }
  __device__ __forceinline__ int* slot(int) { return sh->i[ph]; }
};

// A thread's slice of the row: the first NREG values in registers, the rest
// in LDS at stride SMP_THREADS (bank-conflict free).  Values are visited in
// index order; f(v, i) may change v, which is written back.
constexpr int SMP_LDS_SLOTS = 36;   // 144 KB of LDS (+ 8 KB for the compacted top-k list)
constexpr int SMP_NREG = 16;
constexpr int SMP_MAXPT = SMP_NREG + SMP_LDS_SLOTS;   // V <= 53248

// After a top-k of at most SMP_THREADS candidates the slice is compacted: each
// thread then holds one candidate (r[0], vocabulary index i0; zero if none).
struct Slice {
  float r[SMP_NREG];
  float* lds;
  int nl, i0, tid;
  bool compact;
  template <typename F> __device__ __forceinline__ void for_each(F f) {
    if (compact) { f(r[0], i0); return; }
#pragma unroll
    for (int j = 0; j < SMP_NREG; ++j) f(r[j], i0 + j);
    for (int l = 0; l < nl; ++l) {
      float v = lds[l * SMP_THREADS + tid];
      f(v, i0 + SMP_NREG + l);
      lds[l * SMP_THREADS + tid] = v;
    }
  }
  template <typename F> __device__ __forceinline__ void visit(F f) const {   // read only
    if (compact) { f(r[0], i0); return; }
#pragma unroll
    for (int j = 0; j < SMP_NREG; ++j) f(r[j], i0 + j);
    for (int l = 0; l < nl; ++l) f(lds[l * SMP_THREADS + tid], i0 + SMP_NREG + l);
  }
  // sum of g(v) over the slice (X = int or double), four interleaved partial
  // sums so that the additions do not form one long dependent chain; the
  // order is fixed, so the result is the same on every run
  template <typename X, typename G> __device__ __forceinline__ X sum(G g) const {
    if (compact) return g(r[0]);
    X p0 = X(0), p1 = X(0), p2 = X(0), p3 = X(0);
#pragma unroll
    for (int j = 0; j < SMP_NREG; j += 4) {
      p0 += g(r[j]); p1 += g(r[j + 1]); p2 += g(r[j + 2]); p3 += g(r[j + 3]);
    }
    int l = 0;
    for (; l + 4 <= nl; l += 4) {
      p0 += g(lds[l * SMP_THREADS + tid]);
      p1 += g(lds[(l + 1) * SMP_THREADS + tid]);
      p2 += g(lds[(l + 2) * SMP_THREADS + tid]);
      p3 += g(lds[(l + 3) * SMP_THREADS + tid]);
    }
    for (; l < nl; ++l) p0 += g(lds[l * SMP_THREADS + tid]);
    return (p0 + p1) + (p2 + p3);
  }
};

template <typename T>
__global__ void __launch_bounds__(SMP_THREADS) sample_kernel(SampleArgs a) {
  __shared__ SmpShared sh;
  __shared__ float slots[SMP_LDS_SLOTS * SMP_THREADS];
  __shared__ float cw[SMP_THREADS];   // compacted top-k candidates (weight, vocabulary index), or the weights a search narrowed to
  __shared__ int ci[SMP_THREADS];
  __shared__ uint32_t tshare;         // a threshold found by wave 0 alone
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Blk blk{&sh, 0, lane, wave};
  const int row = blockIdx.x, V = a.V;
  const int npt = (V + SMP_THREADS - 1) / SMP_THREADS;   // <= SMP_MAXPT (checked at launch)
  const int i0 = tid * npt;
  const int iend = min(V, i0 + npt);                       // this thread's slice is [i0, iend)
  const T* z = reinterpret_cast<const T*>(a.logits) + (long long)row * a.ld;
  const uint32_t* seen = a.seen ? a.seen + (long long)row * a.seen_words : nullptr;
  const bool pen = seen != nullptr && a.penalty != 1.f;
  Slice sl;
  sl.lds = slots;
  sl.nl = max(0, npt - SMP_NREG);
  sl.i0 = i0;
  sl.tid = tid;
  sl.compact = false;

  // penalised logits; indices past the slice hold -inf (weight 0 later)
  sl.for_each([&](float& v, int i) {
    v = -INFINITY;
    if (i < iend) {
      v = to_f32(z[i]);
      if (pen && ((seen[i >> 5] >> (i & 31)) & 1u)) v = v > 0.f ? v / a.penalty : (v < 0.f ? v * a.penalty : v);
    }
  });
  int tok;
  if (!(a.temperature > 0.f)) {
    // greedy: largest penalised logit, lowest index among equals
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    sl.visit([&](float v, int i) {
      if (i < iend && (bi == 0x7fffffff || v > bv)) { bv = v; bi = i; }
    });
    const float m = blk.max(bi == 0x7fffffff ? -INFINITY : bv);
    const bool mine = bi != 0x7fffffff && bv == m;
    tok = blk.min(mine ? bi : 0x7fffffff);
    if (tok == 0x7fffffff) tok = 0;   // no token in range: cannot happen for V >= 1
  } else {
    // Keys z'/T, then weights w = exp(key - max) (double, rounded to float).
    // Indices past the slice weigh 0.  A candidate that top-k or top-p
    // removes gets weight 0 as well, so every later mass simply sums all
    // weights: positive weights have bit patterns >= 1 and every threshold
    // below is >= 1 (the whole set's mass is above any target), so zero
    // weights are never counted, kept or drawn.  w <= 1: patterns < 2^30.
    float kmax = -INFINITY;
    sl.for_each([&](float& v, int i) {
      if (i < iend) v = v / a.temperature;
      kmax = fmaxf(kmax, v);
    });
    const double M = (double)blk.max(kmax);
    sl.for_each([&](float& v, int i) { v = i < iend ? (float)exp((double)v - M) : 0.f; });
    auto wd = [](float w) {   // conversion kept at its use (no hoisting of every value's double)
      asm volatile("" : "+v"(w));
      return (double)w;
    };

    // top-k: T = the k-th largest pattern (largest t with count(w >= t) >= k),
    // then the equal ones with the lowest indices
    if (a.top_k > 0 && a.top_k < V) {
      // (narrowed like the mass searches below: once at most SMP_THREADS
      // weights share the leading bits fixed so far, wave 0 finishes on them
      // with the fixed count of the weights above that range)
      uint32_t t = 0;
      int bit = 29, above_n = 0, total = 0;
      bool small = false;
      for (; bit >= 0; --bit) {
        if (bit == 22 || bit == 19 || bit == 16 || bit == 13) {
          const uint32_t lo = t, hi = t + (2u << bit);
          const int n = sl.sum<int>([&](float v) {
            const uint32_t b = __float_as_uint(v);
            return b >= lo && b < hi ? 1 : 0;
          });
          int at = blk.exscan(n);
          total = blk.sum(n);
          if (total <= SMP_THREADS) {
            int ab = 0;
            sl.visit([&](float v, int) {
              const uint32_t b = __float_as_uint(v);
              ab += b >= hi ? 1 : 0;
              if (b >= lo && b < hi) cw[at++] = v;
            });
            above_n = blk.sum(ab);   // (its barrier also publishes cw)
            small = true;
            break;
          }
        }
        const uint32_t c = t | (1u << bit);
        const int n = sl.sum<int>([&](float v) { return __float_as_uint(v) >= c ? 1 : 0; });
        if (blk.sum(n) >= a.top_k) t = c;
      }
      if (small) {
        if (wave == 0) {
          float v[SMP_THREADS / WAVE];
#pragma unroll
          for (int i = 0; i < SMP_THREADS / WAVE; ++i) {
            const int j = lane + i * WAVE;
            v[i] = j < total ? cw[j] : 0.f;
          }
          for (; bit >= 0; --bit) {
            const uint32_t c = t | (1u << bit);
            int n = 0;
#pragma unroll
            for (int i = 0; i < SMP_THREADS / WAVE; ++i) n += __float_as_uint(v[i]) >= c ? 1 : 0;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
            if (above_n + n >= a.top_k) t = c;
          }
          if (lane == 0) tshare = t;
        }
        __syncthreads();
        t = tshare;
      }
      if (t > 0) {   // (t == 0: fewer than k positive weights, all of them stay)
        int above = 0, ties = 0;
        sl.visit([&](float v, int) {
          above += __float_as_uint(v) > t;
          ties += __float_as_uint(v) == t;
        });
        const int need = a.top_k - blk.sum(above);
        int r = blk.exscan(ties);
        sl.for_each([&](float& v, int) {
          const uint32_t b = __float_as_uint(v);
          if (b < t) v = 0.f;
          else if (b == t) { if (r >= need) v = 0.f; ++r; }
        });
      }
      if (a.top_k <= SMP_THREADS) {
        // at most 1024 candidates (weight > 0) remain: gather them, in index
        // order, one per thread, so that the later searches visit one value each
        int cnt = 0;
        sl.visit([&](float v, int) { cnt += v > 0.f; });
        int at = blk.exscan(cnt);
        const int total = blk.sum(cnt);
        sl.visit([&](float v, int i) {
          if (v > 0.f) { cw[at] = v; ci[at] = i; ++at; }
        });
        __syncthreads();
        const bool have = tid < total;
        sl.compact = true;
        sl.r[0] = have ? cw[tid] : 0.f;
        sl.i0 = have ? ci[tid] : 0;
      }
    }
    // Largest pattern t whose mass(w >= t) is above the target (>= when ge,
    // > otherwise); returns in `cum` the mass of the weights above t plus that
    // of the weights equal to t in the threads before this one, for the caller
    // to resolve the equal ones in index order.
    //
    // Once the bits above `bit` are fixed, only the weights whose patterns
    // share them, [t, t + 2^(bit+1)), are still undecided: those above count
    // in every later step, those below in none.  At a few checkpoints the
    // undecided weights are counted; when at most SMP_THREADS remain they are
    // gathered one per thread (cw) and the remaining steps sum that one value
    // plus the fixed mass above the range.
    auto threshold = [&](double target, bool ge, uint32_t& t, double& cum) {
      t = 0;
      int bit = 29;
      double base = 0.0;
      int total = 0;
      bool small = false;   // the undecided weights (<= SMP_THREADS) are gathered in cw[0, total)
      if (sl.compact) {     // one weight per thread already
        cw[tid] = sl.r[0];
        total = SMP_THREADS;
        small = true;
        __syncthreads();
      }
      for (; bit >= 0 && !small; --bit) {
        if (bit == 22 || bit == 19 || bit == 16 || bit == 13) {
          const uint32_t lo = t, hi = t + (2u << bit);
          const int n = sl.sum<int>([&](float v) {
            const uint32_t b = __float_as_uint(v);
            return b >= lo && b < hi ? 1 : 0;
          });
          int at = blk.exscan(n);
          total = blk.sum(n);
          if (total <= SMP_THREADS) {
            double ab = 0.0;
            sl.visit([&](float v, int) {
              const uint32_t b = __float_as_uint(v);
              ab += b >= hi ? wd(v) : 0.0;
              if (b >= lo && b < hi) cw[at++] = v;
            });
            base = blk.sum(ab);   // (its barrier also publishes cw)
            small = true;
            break;                // bit is still undecided
          }
        }
        const uint32_t c = t | (1u << bit);
        const double sm = blk.sum(sl.sum<double>([&](float v) { return __float_as_uint(v) >= c ? wd(v) : 0.0; }));
        if (ge ? sm >= target : sm > target) t = c;
      }
      if (small) {
        // wave 0 finishes the search on the gathered weights, 16 per lane,
        // with butterfly sums (every lane ends with the same double, so t
        // stays uniform) and no block barrier per step
        if (wave == 0) {
          float v[SMP_THREADS / WAVE];
#pragma unroll
          for (int i = 0; i < SMP_THREADS / WAVE; ++i) {
            const int j = lane + i * WAVE;
            v[i] = j < total ? cw[j] : 0.f;
          }
          for (; bit >= 0; --bit) {
            const uint32_t c = t | (1u << bit);
            double p0 = 0.0, p1 = 0.0;
#pragma unroll
            for (int i = 0; i < SMP_THREADS / WAVE; i += 2) {
              p0 += __float_as_uint(v[i]) >= c ? wd(v[i]) : 0.0;
              p1 += __float_as_uint(v[i + 1]) >= c ? wd(v[i + 1]) : 0.0;
            }
            double sm = p0 + p1;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o, 64);
            sm += base;
            if (ge ? sm >= target : sm > target) t = c;
          }
          if (lane == 0) tshare = t;
        }
        __syncthreads();
        t = tshare;
      }
      double above = 0.0, eq = 0.0;
      sl.visit([&](float v, int) {   // both sums updated every time (no address select)
        const double w = wd(v);
        above += __float_as_uint(v) > t ? w : 0.0;
        eq += __float_as_uint(v) == t ? w : 0.0;
      });
      const double ab = blk.sum(above);
      cum = ab + blk.exscan(eq);
    };
    auto total = [&]() { return blk.sum(sl.sum<double>([&](float v) { return wd(v); })); };

    // top-p: every weight above the threshold, then the equal ones in index
    // order while the mass before them is still below p Z
    double Zn = total();
    if (a.top_p < 1.f) {
      const double X = (double)a.top_p * Zn;
      uint32_t t;
      double cum;
      threshold(X, true, t, cum);
      sl.for_each([&](float& v, int) {
        const uint32_t b = __float_as_uint(v);
        if (b < t) v = 0.f;
        else if (b == t) {
          if (cum < X) cum += wd(v);
          else v = 0.f;
        }
      });
      Zn = total();
    }

    // draw: the first candidate whose cumulative mass exceeds u Zn
    const double r = (double)a.u[row] * Zn;
    uint32_t t;
    double cum;
    threshold(r, false, t, cum);
    int pick = 0x7fffffff, last = -1;
    sl.visit([&](float v, int i) {
      if (__float_as_uint(v) == t) {
        cum += wd(v);
        if (pick == 0x7fffffff && cum > r) pick = i;
        last = i;
      }
    });
    tok = blk.min(pick);
    if (tok == 0x7fffffff) tok = blk.max(last);   // rounding left u Zn at the very end
  }
  if (tok < 0 || tok >= V) tok = 0;   // cannot happen (every search ends on a present weight); keeps the write in range
  if (tid == 0) {
    a.out[row] = tok;
    if (a.seen) atomicOr(a.seen + (long long)row * a.seen_words + (tok >> 5), 1u << (tok & 31));
  }
}

// Bits of `tokens` [B, T] (values in [0, V)) set in the rows of `seen`.
__global__ void mark_seen_kernel(const int32_t* __restrict__ tokens, int B, int T, int V, uint32_t* seen,
                                 int words) {
  const long long n = (long long)B * T;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    const int b = (int)(e / T), tk = tokens[e];
    if (tk >= 0 && tk < V) atomicOr(seen + (long long)b * words + (tk >> 5), 1u << (tk & 31));
  }
}

template <typename T>
static hipError_t sample_t(const SampleArgs& a, hipStream_t st) {
  if (a.V < 1 || (a.V + SMP_THREADS - 1) / SMP_THREADS > SMP_MAXPT) return hipErrorInvalidValue;
  hipLaunchKernelGGL((sample_kernel<T>), dim3(a.B), dim3(SMP_THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sample(int dtype, const SampleArgs& a, hipStream_t st) {
  if (dtype == 0) return sample_t<float>(a, st);
  return sample_t<bf16>(a, st);
}

hipError_t launch_mark_seen(const int32_t* tokens, int B, int T, int V, uint32_t* seen, hipStream_t st) {
  const long long n = (long long)B * T;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(mark_seen_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, st, tokens, B, T, V, seen,
                     (V + 31) / 32);
  return hipGetLastError();
}

}  // namespace gptmi
