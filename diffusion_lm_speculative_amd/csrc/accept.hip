// Acceptance walk of the SimSD pipeline: standard rejection sampling in the
// temporal order the draft induced, committing the longest accepted prefix
// (page "SimSD - Simple Speculative Decoding in Diffusion Language Models",
// section 4, acceptance bullet; tau is the stage map of section 2).
//
// Read as the textbook rule: the candidate x drafted from q at stage t is
// kept with probability min(1, p(x)/q(x)); at the first rejection a
// replacement is drawn from max(0, p - q) normalised.
//
// One workgroup per sequence.  Stage decisions are independent given the
// uniforms, so threads 0..gamma-1 decide one stage each and the prefix length
// is the first rejected stage minus one.  The acceptance compare
// u * q(x) < p(x) is exact in fp64 (24-bit u times a float needs <= 48
// bits).  The replacement is an inverse-CDF pick over fp64 prefix sums of the
// residual, found in two passes: per-tile sums, then a scan inside the tile
// that holds the threshold.
//
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11), key (seed, 0); stage t of sequence b
// uses counter (b, t, 0, offset) and the top 24 bits of word 0; the
// replacement draw uses counter (b, n+1, 1, offset) and the top 53 bits.
#include "simsd_common.hpp"

namespace simsd {
namespace {

constexpr int kAccThreads = 256;
constexpr int kAccEpt = 8;  // elements per thread per tile in the residual scan

// Philox-4x64 with 10 rounds: each round multiplies counter words 0 and 2 by
// the 4x64 multipliers, keeps both 64-bit halves of the products and mixes
// the high halves with counter words 1, 3 and the key; the key advances by
// the two Weyl increments between rounds.
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t k0, uint64_t k1) {
  constexpr uint64_t kMul0 = 0xD2E7470EE14C6C93ull;
  constexpr uint64_t kMul1 = 0xCA5A826395121157ull;
  constexpr uint64_t kWeyl0 = 0x9E3779B97F4A7C15ull;
  constexpr uint64_t kWeyl1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd > 0) {
      k0 += kWeyl0;
      k1 += kWeyl1;
    }
    const uint64_t lo0 = kMul0 * c0, hi0 = __umul64hi(kMul0, c0);
    const uint64_t lo1 = kMul1 * c2, hi1 = __umul64hi(kMul1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kAccThreads / 64; ++i) t += red[i];
  return t;
}

// Exclusive prefix of one double per thread, in thread order; the tile total
// is left in *total.  Block-wide.
__device__ __forceinline__ double block_excl_scan(double v, double* buf, double* total) {
  __syncthreads();
  buf[threadIdx.x] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    double run = 0.0;
    for (int i = 0; i < kAccThreads; ++i) {
      const double x = buf[i];
      buf[i] = run;
      run += x;
    }
    *total = run;
  }
  __syncthreads();
  return buf[threadIdx.x];
}

__device__ __forceinline__ double weight(const float* p, const float* q, int64_t v) {
  const double pv = static_cast<double>(p[v]);
  if (!q) return pv;
  const double r = pv - static_cast<double>(q[v]);
  return r > 0.0 ? r : 0.0;
}

struct ScanShared {
  double red[kAccThreads / 64];
  double buf[kAccThreads];
  double tsum[1024];
  double total;
  double base;
  double thr;
  unsigned long long pick;   // candidate index (min over threads)
  unsigned long long last;   // 1 + last index with positive weight (max over threads)
  int sel;
};

// Smallest v whose fp64 prefix sum of weight() exceeds u * total; -1 when the
// total is zero.  Block-wide (all threads call it).  Pass 1 sums tiles of
// kAccThreads*ept elements; pass 2 rescans from the tile holding the
// threshold.  If rounding of the rescan leaves the threshold past every
// prefix, the last index with positive weight is taken (the top of the CDF).
__device__ int64_t inverse_cdf(const float* p, const float* q, int64_t V, double u, int ept, ScanShared& sh) {
  const int tid = threadIdx.x;
  const int64_t tsz = static_cast<int64_t>(kAccThreads) * ept;
  const int ntile = static_cast<int>((V + tsz - 1) / tsz);
  for (int t = 0; t < ntile; ++t) {
    double part = 0.0;
    const int64_t v0 = t * tsz + static_cast<int64_t>(tid) * ept;
    for (int e = 0; e < ept; ++e)
      if (v0 + e < V) part += weight(p, q, v0 + e);
    const double ts = block_sum(part, sh.red);
    if (tid == 0) sh.tsum[t] = ts;
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int t = 0; t < ntile; ++t) tot += sh.tsum[t];
    const double thr = u * tot;
    int sel = -1;
    double acc = 0.0;
    if (tot > 0.0) {
      sel = ntile - 1;
      for (int t = 0; t < ntile; ++t) {
        if (acc + sh.tsum[t] > thr) {
          sel = t;
          break;
        }
        if (t + 1 < ntile) acc += sh.tsum[t];
      }
    }
    sh.sel = sel;
    sh.base = acc;
    sh.thr = thr;
    sh.pick = ~0ull;
    sh.last = 0ull;
  }
  __syncthreads();
  const int sel = sh.sel;
  if (sel < 0) return -1;
  const double thr = sh.thr;
  double base = sh.base;
  unsigned long long last = 0ull;
  for (int t = sel; t < ntile; ++t) {
    const int64_t v0 = t * tsz + static_cast<int64_t>(tid) * ept;
    double part = 0.0;
    for (int e = 0; e < ept; ++e)
      if (v0 + e < V) part += weight(p, q, v0 + e);
    double run = base + block_excl_scan(part, sh.buf, &sh.total);
    for (int e = 0; e < ept; ++e) {
      if (v0 + e >= V) break;
      const double w = weight(p, q, v0 + e);
      run += w;
      if (w > 0.0) {
        last = static_cast<unsigned long long>(v0 + e) + 1ull;
        if (run > thr) {
          atomicMin(&sh.pick, static_cast<unsigned long long>(v0 + e));
          break;
        }
      }
    }
    __syncthreads();
    if (sh.pick != ~0ull) break;
    base += sh.total;
  }
  if (last) atomicMax(&sh.last, last);
  __syncthreads();
  if (sh.pick != ~0ull) return static_cast<int64_t>(sh.pick);
  return static_cast<int64_t>(sh.last) - 1;
}

__global__ __launch_bounds__(kAccThreads) void accept_kernel(const float* __restrict__ p,
                                                             const float* __restrict__ q,
                                                             const int32_t* __restrict__ draft,
                                                             const int32_t* __restrict__ tau, int B, int gamma,
                                                             int64_t V, uint64_t seed, uint64_t offset, int ept,
                                                             int32_t* n_acc, int32_t* next_tok, int32_t* status) {
  __shared__ int kinv[65];
  __shared__ int st_s, nrej;
  __shared__ ScanShared sh;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* tau_b = tau + static_cast<size_t>(b) * B;
  const int32_t* draft_b = draft + static_cast<size_t>(b) * B;

  if (tid == 0) {
    int st = 0;
    uint64_t seen = 0;
    for (int k = 0; k < B; ++k) {
      const int t = tau_b[k];
      if (t < 1 || t > B) {
        st = SIMSD_ST_TAU_RANGE;
      } else {
        if ((seen >> (t - 1)) & 1ull) {
          if (!st) st = SIMSD_ST_TAU_NOT_PERM;
        }
        seen |= 1ull << (t - 1);
        kinv[t] = k;
      }
    }
    if (st == 0) {
      for (int t = 1; t <= gamma; ++t) {
        const int x = draft_b[kinv[t]];
        if (x < 0 || static_cast<int64_t>(x) >= V) st |= SIMSD_ST_TOKEN_RANGE;
      }
    }
    st_s = st;
    nrej = gamma + 1;
  }
  __syncthreads();
  if (st_s) {
    if (tid == 0) {
      n_acc[b] = -1;
      if (next_tok) next_tok[b] = -1;
      if (status) status[b] = st_s;
    }
    return;
  }
  if (tid < gamma) {
    const int t = tid + 1;
    const int k = kinv[t];
    const int x = draft_b[k];
    const uint64_t w = philox_word0(static_cast<uint64_t>(b), static_cast<uint64_t>(t), 0ull, offset, seed, 0ull);
    const double u = static_cast<double>(w >> 40) * 0x1p-24;
    const size_t row = (static_cast<size_t>(b) * B + k) * static_cast<size_t>(V);
    const double pv = static_cast<double>(p[row + x]);
    const double qv = static_cast<double>(q[row + x]);
    if (!(u * qv < pv)) atomicMin(&nrej, t);
  }
  __syncthreads();
  const int n = nrej - 1;
  if (tid == 0) {
    n_acc[b] = n;
    if (status) status[b] = 0;
  }
  if (!next_tok) return;
  if (n >= gamma) {
    if (tid == 0) next_tok[b] = -1;
    return;
  }
  const int ks = kinv[n + 1];
  const size_t row = (static_cast<size_t>(b) * B + ks) * static_cast<size_t>(V);
  const uint64_t w2 = philox_word0(static_cast<uint64_t>(b), static_cast<uint64_t>(n + 1), 1ull, offset, seed, 0ull);
  const double u2 = static_cast<double>(w2 >> 11) * 0x1p-53;
  int64_t pick_v = inverse_cdf(p + row, q + row, V, u2, ept, sh);
  if (pick_v < 0) pick_v = inverse_cdf(p + row, nullptr, V, u2, ept, sh);
  if (tid == 0) next_tok[b] = static_cast<int32_t>(pick_v);
}

}  // namespace

hipError_t launch_accept(const float* p, const float* q, const int32_t* draft, const int32_t* tau,
                         int NB, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset,
                         int32_t* n_acc, int32_t* next_tok, int32_t* status, hipStream_t s) {
  // Elements per thread per tile: at least kAccEpt, and few enough tiles for
  // the shared tile-sum table.
  int64_t ept = kAccEpt;
  const int64_t need = (V + static_cast<int64_t>(kAccThreads) * 1024 - 1) / (static_cast<int64_t>(kAccThreads) * 1024);
  if (need > ept) ept = need;
  hipLaunchKernelGGL(accept_kernel, dim3(NB), dim3(kAccThreads), 0, s, p, q, draft, tau, B, gamma, V, seed,
                     offset, static_cast<int>(ept), n_acc, next_tok, status);
  return hipGetLastError();
}

}  // namespace simsd
