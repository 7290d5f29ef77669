// Coupled-noise acceptance: the drafter and the target share one noise table
// per output position, and a draft is kept exactly when it equals the
// target's noised argmax at its position (SPOT page, "how to use it"
// section, Proposition 2 there: given the noise the target's transition is a
// deterministic argmax, marginalised it samples the target distribution).
// The walk follows the drafted temporal order and commits the longest kept
// prefix (SimSD page, section 4; tau is the stage map of its section 2).
//
// The noise comes in exponential form, E_v = exp(-g_v) for Gumbel g_v, so
// the target token of a row is argmax_v p_v / E_v.  Two candidates a, b are
// compared exactly: p_a * E_b against p_b * E_a, products of two fp32 values
// and so exact in fp64; equal scores go to the smaller index; entries with
// p_v <= 0 never win, and a row without one has no target token (-1).
//
// Two launches:
//   1. row argmax, grid (NB * gamma rows, chunks of a row): the workgroup of
//      stage t of sequence b finds the position k with tau[k] = t, streams
//      its chunk of p[b][k] and E[b][k] (16-byte loads; the rows are this
//      call's bytes: 2 * V * 4 per walked stage, read once, so when they add
//      up to at least the last-level cache they are loaded with the
//      non-temporal bit) and reduces its best
//      (p, E, index) over lanes and waves with the exact comparison.
//   2. walk, one workgroup per sequence: the reduction of every walked row's
//      chunk winners (stages spread over the waves), then validation (labels
//      0..B, the nonzero ones exactly 1..m, drafted tokens in range) and the
//      compare of each draft with its stage's target token.
// Label 0 marks a position committed in an earlier round of the block: no
// stage finds it, and the walk covers stages 1..min(gamma, m).
#include "simsd_common.hpp"

namespace simsd {
namespace {

constexpr int kCoThreads = 512;
constexpr int kCoWaves = kCoThreads / 64;
constexpr int kCoPerLane = 16;                           // elements per lane per chunk
constexpr int kCoChunk = kCoThreads * kCoPerLane;        // 8192 elements per workgroup
constexpr int kMaxB = 64;                                // longest section (stages per sequence)

struct Best {
  float p, e;
  int idx;  // -1: no candidate
};

// true when (p, e, i) beats the current best: larger p/E, else equal and a
// smaller index
__device__ __forceinline__ bool better(float p, float e, int i, const Best& b) {
  if (!(p > 0.0f)) return false;
  if (b.idx < 0) return true;
  const double lhs = static_cast<double>(p) * static_cast<double>(b.e);
  const double rhs = static_cast<double>(b.p) * static_cast<double>(e);
  return lhs > rhs || (lhs == rhs && i < b.idx);
}

__device__ __forceinline__ void take(Best& b, float p, float e, int i) {
  if (better(p, e, i, b)) b = Best{p, e, i};
}

__device__ __forceinline__ Best wave_best(Best b) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Best o;
    o.p = __shfl_xor(b.p, off);
    o.e = __shfl_xor(b.e, off);
    o.idx = __shfl_xor(b.idx, off);
    if (o.idx >= 0) take(b, o.p, o.e, o.idx);
  }
  return b;
}

// Position k of stage t in a wave whose lanes 0..B-1 hold tau; -1 when no
// label equals t (the walk launch reports the fault).
__device__ __forceinline__ int stage_position(const int32_t* tau_b, int B, int t) {
  const int lane = threadIdx.x & 63;
  const int lab = lane < B ? tau_b[lane] : 0;
  const uint64_t hit = __ballot(lane < B && lab == t);
  return hit ? __builtin_ctzll(hit) : -1;
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// One 16-byte load, non-temporal when NT.
template <bool NT>
__device__ __forceinline__ float4 load4(const float* ptr) {
  if constexpr (NT) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(ptr));
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const float4*>(ptr);
  }
}

// NT: the row loads carry the non-temporal bit (a template parameter, so the
// issue loop's code is the same for both policies).
template <bool NT>
__global__ __launch_bounds__(kCoThreads) void coupled_argmax_kernel(const float* __restrict__ p,
                                                                     const float* __restrict__ e,
                                                                     const int32_t* __restrict__ tau, int B,
                                                                     int gamma, int64_t V, int nch, float4* part) {
  __shared__ Best sbest[kCoWaves];
  const int row = blockIdx.x;
  const int c = blockIdx.y;  // chunk of the row
  const int b = row / gamma, t = row % gamma + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = stage_position(tau + static_cast<size_t>(b) * B, B, t);
  Best best{0.0f, 1.0f, -1};
  if (k >= 0) {
    const size_t base = (static_cast<size_t>(b) * B + k) * static_cast<size_t>(V);
    const float* pr = p + base;
    const float* er = e + base;
    const int64_t v0 = static_cast<int64_t>(c) * kCoChunk;
    const int64_t v1 = min(v0 + kCoChunk, V);
    if ((V & 3) == 0) {  // rows start 16-byte aligned: 16-byte loads of 4 elements
      // every load of the lane is issued before the first compare, so a wave
      // keeps 8 x 1 KiB in flight.  Lanes past the row's end load the row's
      // last four elements again (no branch around the loads) and drop them:
      // p = 0 never wins
      constexpr int kU = kCoPerLane / 4;
      float4 p4[kU], e4[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t v = v0 + 4 * (tid + u * kCoThreads);
        const int64_t vc = v < v1 ? v : v1 - 4;
        p4[u] = load4<NT>(pr + vc);
        e4[u] = load4<NT>(er + vc);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (v0 + 4 * (tid + u * kCoThreads) >= v1) p4[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = static_cast<int>(v0) + 4 * (tid + u * kCoThreads);
        take(best, p4[u].x, e4[u].x, i);
        take(best, p4[u].y, e4[u].y, i + 1);
        take(best, p4[u].z, e4[u].z, i + 2);
        take(best, p4[u].w, e4[u].w, i + 3);
      }
    } else {
      for (int64_t v = v0 + tid; v < v1; v += kCoThreads) take(best, pr[v], er[v], static_cast<int>(v));
    }
  }
  best = wave_best(best);
  if (lane == 0) sbest[wave] = best;
  __syncthreads();
  if (wave == 0) {
    Best w = lane < kCoWaves ? sbest[lane] : Best{0.0f, 1.0f, -1};
    w = wave_best(w);
    if (lane == 0)
      part[static_cast<size_t>(row) * nch + c] = make_float4(w.p, w.e, __int_as_float(w.idx), 0.0f);
  }
}

// Target tokens of the walked stages, then the walk.  Wave w reduces the
// chunk winners of stages w, w + 16, w + 32, w + 48 (their loads issued
// together), so the rows' reductions take one round of load latency rather
// than one per stage; wave 0 then validates the sequence and walks.
constexpr int kWalkWaves = 16;
constexpr int kWalkRounds = (kMaxB + kWalkWaves - 1) / kWalkWaves;

__global__ __launch_bounds__(kWalkWaves * 64) void coupled_walk_kernel(
    const int32_t* __restrict__ draft, const int32_t* __restrict__ tau, int B, int gamma, int64_t V, int nch,
    const float4* __restrict__ part, int32_t* n_out, int32_t* next_out, int32_t* status) {
  __shared__ int s_target[kMaxB];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* tau_b = tau + static_cast<size_t>(b) * B;
  const int32_t* draft_b = draft + static_cast<size_t>(b) * B;
  const int lab = wave == 0 && lane < B ? tau_b[lane] : 0;
  const int tok = wave == 0 && lane < B ? draft_b[lane] : 0;
  const float4* part_b = part + static_cast<size_t>(b) * gamma * nch;

  Best w[kWalkRounds];
#pragma unroll
  for (int u = 0; u < kWalkRounds; ++u) w[u] = Best{0.0f, 1.0f, -1};
  for (int c = lane; c < nch; c += 64) {
    float4 q[kWalkRounds];
#pragma unroll
    for (int u = 0; u < kWalkRounds; ++u) {
      const int t = wave + kWalkWaves * u;  // 0-based stage
      q[u] = t < gamma ? part_b[static_cast<size_t>(t) * nch + c] : make_float4(0.0f, 1.0f, __int_as_float(-1), 0.0f);
    }
#pragma unroll
    for (int u = 0; u < kWalkRounds; ++u) {
      const int i = __float_as_int(q[u].z);
      if (i >= 0) take(w[u], q[u].x, q[u].y, i);
    }
  }
#pragma unroll
  for (int u = 0; u < kWalkRounds; ++u) {
    const int t = wave + kWalkWaves * u;
    const Best r = wave_best(w[u]);
    if (lane == 0 && t < gamma) s_target[t] = r.idx;
  }
  __syncthreads();
  if (wave != 0) return;

  int st = 0;
  const int m = __popcll(__ballot(lane < B && lab >= 1));  // open positions
  const int g = min(gamma, m);                              // stages walked
  if (__any(lane < B && (lab < 0 || lab > B))) {
    st = SIMSD_ST_TAU_RANGE;
  } else {
    // the m open labels must be exactly 1..m: none of them without a position
    bool missing = false;
    for (int t = 1; t <= m; ++t) missing |= __ballot(lane < B && lab == t) == 0ull;
    if (missing) {
      st = SIMSD_ST_TAU_NOT_PERM;
    } else if (__any(lane < B && lab >= 1 && lab <= g && (tok < 0 || static_cast<int64_t>(tok) >= V))) {
      st = SIMSD_ST_TOKEN_RANGE;
    }
  }
  int n = -1, nxt = -1;
  if (st == 0) {
    // the lane of position k compares its draft with its stage's target
    // token; the first mismatch in stage order ends the walk
    const bool walked = lane < B && lab >= 1 && lab <= g;
    const uint64_t miss = __ballot(walked && s_target[walked ? lab - 1 : 0] != tok);
    n = g;
    if (miss) {
      int first = kMaxB + 1;  // smallest stage label among the mismatching lanes
      for (uint64_t m = miss; m; m &= m - 1) first = min(first, __shfl(lab, __builtin_ctzll(m)));
      n = first - 1;
      nxt = s_target[first - 1];
    }
  }
  if (lane == 0) {
    n_out[b] = n;
    if (next_out) next_out[b] = nxt;
    if (status) status[b] = st;
  }
}

}  // namespace

int coupled_chunks(int64_t V) { return static_cast<int>((V + kCoChunk - 1) / kCoChunk); }

size_t coupled_workspace_bytes(int NB, int B, int64_t V) {
  const size_t n = static_cast<size_t>(NB) * B * coupled_chunks(V) * sizeof(float4);
  return (n + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_accept_coupled(const float* p, const float* e, const int32_t* draft, const int32_t* tau, int NB,
                                 int B, int gamma, int64_t V, int32_t* n_out, int32_t* next_out, int32_t* status,
                                 void* workspace, hipStream_t s) {
  const int nch = coupled_chunks(V);
  float4* part = static_cast<float4*>(workspace);
  if (gamma > 0) {
    // Rows read once per call: at batch 64, gamma 16 (1.24 GB of p and E)
    // the non-temporal bit took the argmax launch from 220 to 200 us (paired
    // runs, identical outputs).  Rows that fit the last-level cache keep the
    // default policy (a producer's writes may still be there).
    const double bytes = static_cast<double>(NB) * gamma * static_cast<double>(V) * 8.0;
    const bool nt = bytes >= static_cast<double>(kLastLevelCache);
    if (nt)
      hipLaunchKernelGGL(coupled_argmax_kernel<true>, dim3(NB * gamma, nch), dim3(kCoThreads), 0, s, p, e, tau, B,
                         gamma, V, nch, part);
    else
      hipLaunchKernelGGL(coupled_argmax_kernel<false>, dim3(NB * gamma, nch), dim3(kCoThreads), 0, s, p, e, tau, B,
                         gamma, V, nch, part);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(coupled_walk_kernel, dim3(NB), dim3(kWalkWaves * 64), 0, s, draft, tau, B, gamma, V, nch, part, n_out,
                     next_out, status);
  return hipGetLastError();
}

}  // namespace simsd
