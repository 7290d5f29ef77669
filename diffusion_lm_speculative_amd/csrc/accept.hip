// Acceptance walk of the SimSD pipeline: standard rejection sampling in the
// temporal order the draft induced, committing the longest accepted prefix
// (page "SimSD - Simple Speculative Decoding in Diffusion Language Models",
// section 4, acceptance bullet; tau is the stage map of section 2).
//
// Read as the textbook rule: the candidate x drafted from q at stage t is
// kept with probability min(1, p(x)/q(x)); at the first rejection a
// replacement is drawn from max(0, p - q) normalised.
//
// Two launches.  Both recompute the walk of their sequence (tau inverse,
// validation, one stage decision per thread; gamma <= 64 Philox draws and
// 2*gamma gathered floats), which is cheaper than passing it between them.
//   1. segment sums: the rejected position's row is split into NSEG segments
//      spread over NB*NSEG workgroups; each sums max(0, p - q) and p over
//      its segment in fp64 with coalesced loads (the rows dominate the bytes
//      of this step: 2 * V * 4 bytes per rejecting sequence).
//   2. select: one workgroup per sequence writes n and the status, walks the
//      segment sums in order to the segment that holds u' * S, and scans that
//      segment tile by tile (block-wide fp64 prefix sums) for the first index
//      whose prefix sum exceeds it.
// The acceptance compare u * q(x) < p(x) is exact in fp64 (24-bit u times a
// float needs <= 48 bits).  Prefix sums are fp64 in a blocked order, so an
// index may differ from a strictly sequential sum only where the threshold
// falls within rounding of a CDF boundary.
//
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11), key (seed, 0); stage t of sequence b
// uses counter (b, t, 0, offset) and the top 24 bits of word 0; the
// replacement draw uses counter (b, n+1, 1, offset) and the top 53 bits.
#include "simsd_common.hpp"

namespace simsd {
namespace {

constexpr int kAccThreads = 256;
constexpr int kScanEpt = 8;  // elements per thread per tile of the in-segment scan

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

struct Walk {
  int kinv[65];  // kinv[t] = position of stage t
  int st;        // status flags
  int nrej;      // first rejected stage (gamma + 1 when none)
};

// Validate tau and the walked tokens, then decide every stage in parallel.
// Block-wide; on return w.st and w.nrej are valid for every thread.
__device__ void tau_walk(Walk& w, const float* p, const float* q, const int32_t* tau_b, const int32_t* draft_b,
                         int b, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    int st = 0;
    uint64_t seen = 0;
    for (int k = 0; k < B; ++k) {
      const int t = tau_b[k];
      if (t < 1 || t > B) {
        st = SIMSD_ST_TAU_RANGE;
      } else {
        if (((seen >> (t - 1)) & 1ull) && !st) st = SIMSD_ST_TAU_NOT_PERM;
        seen |= 1ull << (t - 1);
        w.kinv[t] = k;
      }
    }
    if (st == 0) {
      for (int t = 1; t <= gamma; ++t) {
        const int x = draft_b[w.kinv[t]];
        if (x < 0 || static_cast<int64_t>(x) >= V) st |= SIMSD_ST_TOKEN_RANGE;
      }
    }
    w.st = st;
    w.nrej = gamma + 1;
  }
  __syncthreads();
  if (w.st == 0 && tid < gamma) {
    const int t = tid + 1;
    const int k = w.kinv[t];
    const int x = draft_b[k];
    const uint64_t r = philox_word0(static_cast<uint64_t>(b), static_cast<uint64_t>(t), 0ull, offset, seed, 0ull);
    const double u = static_cast<double>(r >> 40) * 0x1p-24;
    const size_t row = (static_cast<size_t>(b) * B + k) * static_cast<size_t>(V);
    const double pv = static_cast<double>(p[row + x]);
    const double qv = static_cast<double>(q[row + x]);
    if (!(u * qv < pv)) atomicMin(&w.nrej, t);
  }
  __syncthreads();
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Segment sums of the residual max(0, p - q) and of p for the rejected
// position of sequence blockIdx.y; segment blockIdx.x.
__global__ __launch_bounds__(kAccThreads) void accept_segsum_kernel(const float* __restrict__ p,
                                                                    const float* __restrict__ q,
                                                                    const int32_t* __restrict__ draft,
                                                                    const int32_t* __restrict__ tau, int B,
                                                                    int gamma, int64_t V, uint64_t seed,
                                                                    uint64_t offset, int nseg, int64_t segsz,
                                                                    double* __restrict__ seg_sums) {
  __shared__ Walk w;
  __shared__ double red[2][kAccThreads / 64];
  const int b = blockIdx.y;
  const int seg = blockIdx.x;
  tau_walk(w, p, q, tau + static_cast<size_t>(b) * B, draft + static_cast<size_t>(b) * B, b, B, gamma, V, seed,
           offset);
  const int n = w.nrej - 1;
  if (w.st || n >= gamma) return;
  const size_t row = (static_cast<size_t>(b) * B + w.kinv[n + 1]) * static_cast<size_t>(V);
  const float* pr = p + row;
  const float* qr = q + row;
  const int64_t v0 = seg * segsz;
  const int64_t v1 = min(V, v0 + segsz);
  double sr = 0.0, sp = 0.0;
  int64_t v = v0 + threadIdx.x;
  for (; v + 3 * kAccThreads < v1; v += 4 * kAccThreads) {
    float pv[4], qv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pv[u] = pr[v + u * kAccThreads];
      qv[u] = qr[v + u * kAccThreads];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double d = static_cast<double>(pv[u]) - static_cast<double>(qv[u]);
      sr += d > 0.0 ? d : 0.0;
      sp += static_cast<double>(pv[u]);
    }
  }
  for (; v < v1; v += kAccThreads) {
    const double d = static_cast<double>(pr[v]) - static_cast<double>(qr[v]);
    sr += d > 0.0 ? d : 0.0;
    sp += static_cast<double>(pr[v]);
  }
  sr = wave_sum(sr);
  sp = wave_sum(sp);
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wv] = sr;
    red[1][wv] = sp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, c = 0.0;
    for (int i = 0; i < kAccThreads / 64; ++i) {
      a += red[0][i];
      c += red[1][i];
    }
    seg_sums[(static_cast<size_t>(b) * nseg + seg) * 2 + 0] = a;
    seg_sums[(static_cast<size_t>(b) * nseg + seg) * 2 + 1] = c;
  }
}

__device__ __forceinline__ double weight(const float* p, const float* q, int64_t v, bool residual) {
  const double pv = static_cast<double>(p[v]);
  if (!residual) return pv;
  const double r = pv - static_cast<double>(q[v]);
  return r > 0.0 ? r : 0.0;
}

struct Select {
  double wtot[kAccThreads / 64];
  double base, thr, total;
  unsigned long long pick;  // candidate index (min over threads)
  unsigned long long last;  // 1 + last index with positive weight (max over threads)
  int sel;
  int residual;
};

// Exclusive prefix over the block in thread order; the block total is left in
// sh.total.  Wave-level shuffle scan, then the wave totals.
__device__ __forceinline__ double block_excl_scan(double v, Select& sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  double inc = v;
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  __syncthreads();
  if (lane == 63) sh.wtot[wv] = inc;
  __syncthreads();
  double before = 0.0, total = 0.0;
  for (int i = 0; i < kAccThreads / 64; ++i) {
    if (i < wv) before += sh.wtot[i];
    total += sh.wtot[i];
  }
  if (threadIdx.x == 0) sh.total = total;
  return before + (inc - v);
}

__global__ __launch_bounds__(kAccThreads) void accept_select_kernel(const float* __restrict__ p,
                                                                    const float* __restrict__ q,
                                                                    const int32_t* __restrict__ draft,
                                                                    const int32_t* __restrict__ tau, int B,
                                                                    int gamma, int64_t V, uint64_t seed,
                                                                    uint64_t offset, int nseg, int64_t segsz,
                                                                    const double* __restrict__ seg_sums,
                                                                    int32_t* n_acc, int32_t* next_tok,
                                                                    int32_t* status) {
  __shared__ Walk w;
  __shared__ Select sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  tau_walk(w, p, q, tau + static_cast<size_t>(b) * B, draft + static_cast<size_t>(b) * B, b, B, gamma, V, seed,
           offset);
  const int n = w.nrej - 1;
  if (w.st) {
    if (tid == 0) {
      n_acc[b] = -1;
      if (next_tok) next_tok[b] = -1;
      if (status) status[b] = w.st;
    }
    return;
  }
  if (tid == 0) {
    n_acc[b] = n;
    if (status) status[b] = 0;
  }
  if (!next_tok) return;
  if (n >= gamma) {
    if (tid == 0) next_tok[b] = -1;
    return;
  }
  const size_t row = (static_cast<size_t>(b) * B + w.kinv[n + 1]) * static_cast<size_t>(V);
  const float* pr = p + row;
  const float* qr = q + row;
  if (tid == 0) {
    const double* ss = seg_sums + static_cast<size_t>(b) * nseg * 2;
    double tot_r = 0.0, tot_p = 0.0;
    for (int s = 0; s < nseg; ++s) {
      tot_r += ss[2 * s];
      tot_p += ss[2 * s + 1];
    }
    const bool residual = tot_r > 0.0;
    const double tot = residual ? tot_r : tot_p;
    const int col = residual ? 0 : 1;
    const uint64_t r2 = philox_word0(static_cast<uint64_t>(b), static_cast<uint64_t>(n + 1), 1ull, offset, seed,
                                     0ull);
    const double thr = static_cast<double>(r2 >> 11) * 0x1p-53 * tot;
    int sel = -1;
    double acc = 0.0;
    if (tot > 0.0) {
      sel = nseg - 1;
      for (int s = 0; s < nseg; ++s) {
        if (acc + ss[2 * s + col] > thr) {
          sel = s;
          break;
        }
        if (s + 1 < nseg) acc += ss[2 * s + col];
      }
    }
    sh.sel = sel;
    sh.base = acc;
    sh.thr = thr;
    sh.residual = residual;
    sh.pick = ~0ull;
    sh.last = 0ull;
  }
  __syncthreads();
  if (sh.sel < 0) {
    if (tid == 0) next_tok[b] = -1;
    return;
  }
  const bool residual = sh.residual;
  const double thr = sh.thr;
  double base = sh.base;
  const int64_t v_end = V;  // a crossing missed by rounding continues into later segments
  const int64_t tsz = static_cast<int64_t>(kAccThreads) * kScanEpt;
  unsigned long long last = 0ull;
  for (int64_t t0 = sh.sel * segsz; t0 < v_end; t0 += tsz) {
    const int64_t v0 = t0 + static_cast<int64_t>(tid) * kScanEpt;
    double wv[kScanEpt];
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < kScanEpt; ++e) {
      wv[e] = (v0 + e < v_end) ? weight(pr, qr, v0 + e, residual) : 0.0;
      part += wv[e];
    }
    double run = base + block_excl_scan(part, sh);
#pragma unroll
    for (int e = 0; e < kScanEpt; ++e) {
      run += wv[e];
      if (wv[e] > 0.0) {
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
  if (tid == 0) next_tok[b] = sh.pick != ~0ull ? static_cast<int32_t>(sh.pick) : static_cast<int32_t>(sh.last) - 1;
}

}  // namespace

// Segments per row: enough workgroups to spread the row reads over the chip
// (about 512 in total), each segment at least 4096 elements.
void accept_plan(int NB, int64_t V, int& nseg, int64_t& segsz) {
  int64_t ns = NB > 0 ? (512 + NB - 1) / NB : 1;
  const int64_t cap = (V + 4095) / 4096;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  if (ns > 256) ns = 256;
  segsz = (V + ns - 1) / ns;
  nseg = static_cast<int>((V + segsz - 1) / segsz);
}

hipError_t launch_accept(const float* p, const float* q, const int32_t* draft, const int32_t* tau,
                         int NB, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset,
                         int32_t* n_acc, int32_t* next_tok, int32_t* status, double* seg_sums, hipStream_t s) {
  int nseg;
  int64_t segsz;
  accept_plan(NB, V, nseg, segsz);
  if (next_tok) {
    hipLaunchKernelGGL(accept_segsum_kernel, dim3(nseg, NB), dim3(kAccThreads), 0, s, p, q, draft, tau, B, gamma,
                       V, seed, offset, nseg, segsz, seg_sums);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(accept_select_kernel, dim3(NB), dim3(kAccThreads), 0, s, p, q, draft, tau, B, gamma, V, seed,
                     offset, nseg, segsz, seg_sums, n_acc, next_tok, status);
  return hipGetLastError();
}

}  // namespace simsd
