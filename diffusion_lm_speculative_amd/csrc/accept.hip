// Acceptance walk of the SimSD pipeline: standard rejection sampling in the
// temporal order the draft induced, committing the longest accepted prefix
// (page "SimSD - Simple Speculative Decoding in Diffusion Language Models",
// section 4, acceptance bullet; tau is the stage map of section 2).
//
// Read as the textbook rule: the candidate x drafted from q at stage t is
// kept with probability min(1, p(x)/q(x)); at the first rejection a
// replacement is drawn from max(0, p - q) normalised.  A position labelled
// 0 was committed in an earlier round of the block and is not walked; the
// open labels are 1..m and the walk covers stages 1..min(gamma, m).
//
// Two launches, both starting with the walk of their sequence in wave 0 (tau
// inverse and validation, one stage per lane: gamma <= 64 Philox draws and
// 2*gamma gathered floats).
//   1. chunk sums, grid (row groups, NB): when a stage rejects, the rejected
//      position's row is cut into chunks of kChunk elements and each wave
//      sums max(0, p - q) and p over its chunks in fp64 with coalesced loads
//      (the rows are the bytes of this step: 2 * V * 4 per rejecting
//      sequence).
//      Its first group also stores the walk's outcome (n, status, rejected
//      position and the replacement draw's Philox word) for launch 2.
//   2. select, one wave per sequence: writes n and the status; from the
//      stored walk and the chunk sums (loaded together) it finds the chunk
//      holding u' * S and scans that chunk for the first index whose prefix
//      sum exceeds it.  Without a replacement draw this launch alone decides
//      the walk.
// The acceptance compare u * q(x) < p(x) is exact in fp64 (24-bit u times a
// float needs <= 48 bits).  Prefix sums are fp64 in a blocked order, so an
// index may differ from a strictly sequential sum only where the threshold
// falls within rounding of a CDF boundary.
//
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11), key (seed, 0); stage t of sequence b
// uses counter (b, t, 0, offset) and the top 24 bits of word 0; the
// replacement draw uses counter (b, n+1, 1, offset) and the top 53 bits.
#include <mutex>

#include "simsd_common.hpp"

namespace simsd {

// Scratch of simsd_accept_prefix_noalloc: the chunk sums and walk records
// that simsd_accept_prefix keeps in the caller's workspace, in a fixed device
// array instead (one copy per GPU, held until the process ends).  Host code
// never passes the array's name to a kernel: the name is a host-side
// stand-in, and the device address comes from hipGetSymbolAddress, taken once
// per device.
constexpr size_t kNoAllocScratchBytes = size_t{4} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kAccThreads = 512;
constexpr int kAccWaves = kAccThreads / 64;
constexpr int kChunk = 1024;                  // elements per chunk: one wave pass, 16 per lane

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

// The walk's outcome for a sequence, stored by the chunk-sum launch for the
// select launch.
struct WalkRecord {
  int32_t n, st, krow, g;  // g: stages walked
  unsigned long long draw;  // word 0 of the replacement draw (stage n + 1)
  unsigned long long pad2;
};

static_assert(sizeof(WalkRecord) == 32, "walk record layout");

struct Walk {
  int kinv[65];  // kinv[t] = position of stage t (-1: no position has stage t)
  int tok[64];   // draft token of each position
  unsigned long long draw[64];  // word 0 of the replacement draw's counter (b, t, 1, offset), stage t = index + 1
  int st;        // status flags
  int n;         // accepted prefix length (g when no stage rejects)
  int g;         // stages walked: min(gamma, open positions)
};

// Validate tau and the walked tokens, then decide every stage in parallel
// (wave 0, one stage per lane).  On return w.st and w.n are valid for every
// thread.
__device__ void tau_walk(Walk& w, const float* p, const float* q, const int32_t* tau_b, const int32_t* draft_b,
                         int b, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset, bool draws) {
  const int tid = threadIdx.x;
  for (int i = tid; i <= 64; i += blockDim.x) w.kinv[i] = -1;
  __syncthreads();
  bool range_bad = false, open = false;
  if (tid < B) {  // stage label and draft token of position tid, loaded together
    const int t = tau_b[tid];
    w.tok[tid] = draft_b[tid];
    range_bad = t < 0 || t > B;
    open = !range_bad && t >= 1;  // label 0: committed in an earlier round, not walked
    if (open) w.kinv[t] = tid;
  }
  __syncthreads();
  if (tid < 64) {  // wave 0 (every position's thread is in it)
    // the m open labels must be exactly 1..m: none of them left without a position
    const int m = __popcll(__ballot(open));
    const int g = min(gamma, m);
    const bool missing = tid < m && w.kinv[tid + 1] < 0;
    int st = __any(range_bad) ? SIMSD_ST_TAU_RANGE : (__any(missing) ? SIMSD_ST_TAU_NOT_PERM : 0);
    int k = 0, x = 0;
    if (st == 0 && tid < g) {
      k = w.kinv[tid + 1];
      x = w.tok[k];
    }
    const bool tok_bad = st == 0 && tid < g && (x < 0 || static_cast<int64_t>(x) >= V);
    if (__any(tok_bad)) st = SIMSD_ST_TOKEN_RANGE;
    bool reject = false;
    if (st == 0 && tid < g) {
      const int t = tid + 1;
      const uint64_t r = philox_word0(static_cast<uint64_t>(b), static_cast<uint64_t>(t), 0ull, offset, seed, 0ull);
      const double u = static_cast<double>(r >> 40) * 0x1p-24;
      const size_t row = (static_cast<size_t>(b) * B + k) * static_cast<size_t>(V);
      const double pv = static_cast<double>(p[row + x]);
      const double qv = static_cast<double>(q[row + x]);
      reject = !(u * qv < pv);
    }
    if (draws && tid < g)  // the replacement draw of every stage that could be the first rejected one
      w.draw[tid] = philox_word0(static_cast<uint64_t>(b), static_cast<uint64_t>(tid + 1), 1ull, offset, seed, 0ull);
    const uint64_t rej = __ballot(reject);
    if (tid == 0) {
      w.st = st;
      w.n = rej ? __builtin_ctzll(rej) : g;
      w.g = g;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kAccThreads) void accept_chunks_kernel(
    const float* __restrict__ p, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ tau, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset, int cpw, int nch,
    double* __restrict__ chunk_sums, WalkRecord* __restrict__ records) {
  __shared__ Walk w;
  const int b = blockIdx.y;
  const int grp = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  tau_walk(w, p, q, tau + static_cast<size_t>(b) * B, draft + static_cast<size_t>(b) * B, b, B, gamma, V, seed,
           offset, grp == 0);
  const int n = w.n;
  if (grp == 0 && tid == 0) {
    WalkRecord r{};
    r.n = n;
    r.st = w.st;
    r.g = w.g;
    r.krow = (w.st == 0 && n < w.g) ? w.kinv[n + 1] : 0;
    r.draw = (w.st == 0 && n < w.g) ? w.draw[n] : 0ull;
    records[b] = r;
  }
  if (w.st || n >= w.g) return;
  const size_t row = (static_cast<size_t>(b) * B + w.kinv[n + 1]) * static_cast<size_t>(V);
  const float* pr = p + row;
  const float* qr = q + row;
  double* cs = chunk_sums + static_cast<size_t>(b) * nch * 2;
  const int c_end = min(nch, (grp + 1) * cpw);
  const bool vec = (reinterpret_cast<uintptr_t>(pr) % 16 == 0) && (reinterpret_cast<uintptr_t>(qr) % 16 == 0);
  for (int c = grp * cpw + wave; c < c_end; c += kAccWaves) {
    float pv[16], qv[16];
    if (vec && static_cast<int64_t>(c + 1) * kChunk <= V) {  // whole chunk, 16-byte loads
      const float4* p4 = reinterpret_cast<const float4*>(pr + static_cast<int64_t>(c) * kChunk) + lane;
      const float4* q4 = reinterpret_cast<const float4*>(qr + static_cast<int64_t>(c) * kChunk) + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = p4[64 * i], bq = q4[64 * i];
        pv[4 * i + 0] = a.x; pv[4 * i + 1] = a.y; pv[4 * i + 2] = a.z; pv[4 * i + 3] = a.w;
        qv[4 * i + 0] = bq.x; qv[4 * i + 1] = bq.y; qv[4 * i + 2] = bq.z; qv[4 * i + 3] = bq.w;
      }
    } else {
      const int64_t v0 = static_cast<int64_t>(c) * kChunk + lane;
#pragma unroll
      for (int i = 0; i < 16; ++i) {  // unconditional loads (clamped index) so they all go out at once
        const int64_t v = min(v0 + 64 * i, V - 1);
        pv[i] = pr[v];
        qv[i] = qr[v];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (v0 + 64 * i >= V) pv[i] = qv[i] = 0.0f;
    }
    double sr = 0.0, sp = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double d = static_cast<double>(pv[i]) - static_cast<double>(qv[i]);
      sr += d > 0.0 ? d : 0.0;
      sp += static_cast<double>(pv[i]);
    }
    sr = wave_sum(sr);
    sp = wave_sum(sp);
    if (lane == 0) {
      cs[2 * c + 0] = sr;
      cs[2 * c + 1] = sp;
    }
  }
}

__device__ __forceinline__ double chunk_sum_global(const double* cs, int c, int col) { return cs[2 * c + col]; }

__device__ __forceinline__ double wave_excl_scan(double v) {
  const int lane = threadIdx.x & 63;
  double inc = v;
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  return inc - v;
}

// One wave per sequence: writes n and the status; when a stage rejected,
// walks the chunk sums (loaded while it decides the walk) to the chunk
// holding u' * S and scans that chunk for the first index whose prefix sum
// exceeds it.  Lane l takes chunks l*kPre.. and elements l*16.. of a chunk,
// so a lane's sequential sum followed by a wave scan keeps index order.
constexpr int kPre = 4;  // chunk sums per lane per pass

__global__ __launch_bounds__(64) void accept_select_kernel(
    const float* __restrict__ p, const float* __restrict__ q, const int32_t* __restrict__ draft,
    const int32_t* __restrict__ tau, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset, int nch,
    const double* __restrict__ chunk_sums, const WalkRecord* __restrict__ records, int32_t* n_acc,
    int32_t* next_tok, int32_t* status, int walk_only) {
  __shared__ Walk w;
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  if (walk_only) {  // no replacement draw (none wanted, or no stage to walk): only the walk
    tau_walk(w, p, q, tau + static_cast<size_t>(b) * B, draft + static_cast<size_t>(b) * B, b, B, gamma, V, seed,
             offset, false);
    if (lane == 0) {
      n_acc[b] = w.st ? -1 : w.n;
      if (next_tok) next_tok[b] = -1;  // n == min(gamma, m) or a fault: no draw
      if (status) status[b] = w.st;
    }
    return;
  }
  // the walk's record and the first pass of chunk sums, loaded together
  // (the sums are unused when no stage rejected)
  const WalkRecord rec = records[b];
  const double* cs = chunk_sums + static_cast<size_t>(b) * nch * 2;
  double pre[kPre][2];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int c = lane * kPre + i;
    const bool ok = c < nch;
    pre[i][0] = ok ? cs[2 * c + 0] : 0.0;
    pre[i][1] = ok ? cs[2 * c + 1] : 0.0;
  }
  const int n = rec.n;
  if (rec.st || n >= rec.g) {
    if (lane == 0) {
      n_acc[b] = rec.st ? -1 : n;
      next_tok[b] = -1;
      if (status) status[b] = rec.st;
    }
    return;
  }
  const size_t row = (static_cast<size_t>(b) * B + rec.krow) * static_cast<size_t>(V);
  const float* pr = p + row;
  const float* qr = q + row;
  constexpr int kPass = 64 * kPre;  // chunks per pass
  auto chunk_sum = [&](int pass, int i, int col) {
    const int c = pass * kPass + lane * kPre + i;
    return pass == 0 ? pre[i][col] : (c < nch ? cs[2 * c + col] : 0.0);
  };

  // ---- totals; all-zero residual: draw from p itself
  double tr = 0.0, tp = 0.0;
  for (int pass = 0; pass * kPass < nch; ++pass)
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      tr += chunk_sum(pass, i, 0);
      tp += chunk_sum(pass, i, 1);
    }
  tr = wave_sum(tr);
  tp = wave_sum(tp);
  const bool residual = tr > 0.0;
  const double tot = residual ? tr : tp;
  const int col = residual ? 0 : 1;
  const double thr = static_cast<double>(rec.draw >> 11) * 0x1p-53 * tot;
  if (!(tot > 0.0)) {
    if (lane == 0) {
      n_acc[b] = n;
      next_tok[b] = -1;
      if (status) status[b] = 0;
    }
    return;
  }

  // ---- first chunk whose inclusive prefix exceeds thr (the last chunk when
  //      rounding leaves none), and the prefix before it
  int pick = nch - 1;
  double base = -1.0;
  double carry = 0.0;
  for (int pass = 0; pass * kPass < nch && base < 0.0; ++pass) {
    double v[kPre], sum = 0.0;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      v[i] = chunk_sum(pass, i, col);
      sum += v[i];
    }
    double run = carry + wave_excl_scan(sum);
    int mine = -1;
    double mybase = 0.0;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int c = pass * kPass + lane * kPre + i;
      if (mine < 0 && c < nch && run + v[i] > thr) {
        mine = c;
        mybase = run;
      }
      run += v[i];
    }
    const uint64_t hit = __ballot(mine >= 0);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      pick = __shfl(mine, src);
      base = __shfl(mybase, src);
    }
    carry += wave_sum(sum);
  }
  if (base < 0.0) base = carry - (pick == nch - 1 ? chunk_sum_global(cs, pick, col) : 0.0);

  // ---- scan from that chunk on (a crossing missed by rounding continues
  //      into later chunks; failing that, the last index with positive weight)
  int64_t found = -1, lastpos = -1;
  for (int64_t t0 = static_cast<int64_t>(pick) * kChunk; t0 < V && found < 0; t0 += kChunk) {
    const int64_t v0 = t0 + lane * 16;
    double wv[16], sum = 0.0;
    // a lane's 16 elements: four 16-byte loads each of p and q where the row
    // allows (the scalar loads they replace cost about 2.7 us a call at
    // batch 32), else clamped scalar loads
    float pf[16], qf[16];
    if (v0 + 16 <= V && (reinterpret_cast<uintptr_t>(pr + v0) % 16) == 0 && (reinterpret_cast<uintptr_t>(qr + v0) % 16) == 0) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 a = reinterpret_cast<const float4*>(pr + v0)[i4];
        const float4 c = reinterpret_cast<const float4*>(qr + v0)[i4];
        pf[4 * i4 + 0] = a.x; pf[4 * i4 + 1] = a.y; pf[4 * i4 + 2] = a.z; pf[4 * i4 + 3] = a.w;
        qf[4 * i4 + 0] = c.x; qf[4 * i4 + 1] = c.y; qf[4 * i4 + 2] = c.z; qf[4 * i4 + 3] = c.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t v = min(v0 + e, V - 1);
        pf[e] = pr[v];
        qf[e] = qr[v];
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const double pv = static_cast<double>(pf[e]);
      double x = pv;
      if (residual) {
        const double r = pv - static_cast<double>(qf[e]);
        x = r > 0.0 ? r : 0.0;
      }
      wv[e] = v0 + e < V ? x : 0.0;
      sum += wv[e];
    }
    double run = base + wave_excl_scan(sum);
    int64_t mine = -1, mylast = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      run += wv[e];
      if (wv[e] > 0.0) {
        mylast = v0 + e;
        if (mine < 0 && run > thr) mine = v0 + e;
      }
    }
    const uint64_t hit = __ballot(mine >= 0);
    if (hit) found = __shfl(mine, __builtin_ctzll(hit));
    const uint64_t pos = __ballot(mylast >= 0);
    if (pos) lastpos = __shfl(mylast, 63 - __builtin_clzll(pos));
    base += wave_sum(sum);
  }
  if (lane == 0) {
    n_acc[b] = n;
    next_tok[b] = static_cast<int32_t>(found >= 0 ? found : lastpos);
    if (status) status[b] = 0;
  }
}

}  // namespace

// Chunks per row and row groups: chunks of kChunk elements, spread over about
// 512 workgroups in total, at least 4 chunks (one per wave) per group.
void accept_plan(int NB, int64_t V, int& nch, int& cpw, int& ngrp) {
  nch = static_cast<int>((V + kChunk - 1) / kChunk);
  const int64_t want = NB > 0 ? (static_cast<int64_t>(nch) * NB + 511) / 512 : 1;
  cpw = static_cast<int>(want < kAccWaves ? kAccWaves : want);
  if (cpw > nch) cpw = nch;
  ngrp = (nch + cpw - 1) / cpw;
}

// Workspace of a call that can draw a replacement: fp64 (residual, target)
// sums per row chunk, then a 32-byte walk record per sequence, each region
// 256-byte aligned.  Zero when there is nothing to walk (B == 0).
size_t accept_workspace_bytes(int NB, int B, int64_t V) {
  if (NB == 0 || B == 0) return 0;
  int nch, cpw, ngrp;
  accept_plan(NB, V, nch, cpw, ngrp);
  return (static_cast<size_t>(NB) * nch * 2 * sizeof(double) + 255) / 256 * 256 +
         (static_cast<size_t>(NB) * sizeof(WalkRecord) + 255) / 256 * 256;
}

hipError_t launch_accept(const float* p, const float* q, const int32_t* draft, const int32_t* tau,
                         int NB, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset,
                         int32_t* n_acc, int32_t* next_tok, int32_t* status, void* workspace, hipStream_t s) {
  int nch, cpw, ngrp;
  accept_plan(NB, V, nch, cpw, ngrp);
  // Only a call that can draw a replacement (next_tok wanted, a stage to
  // walk) streams rows and touches the workspace; otherwise the select
  // launch alone walks and writes next_tok = -1.
  const bool draws = next_tok != nullptr && B > 0 && gamma > 0;
  double* chunk_sums = static_cast<double*>(workspace);
  WalkRecord* records = nullptr;
  if (draws) {
    const size_t off = (static_cast<size_t>(NB) * nch * 2 * sizeof(double) + 255) / 256 * 256;
    records = reinterpret_cast<WalkRecord*>(static_cast<char*>(workspace) + off);
    hipLaunchKernelGGL(accept_chunks_kernel, dim3(ngrp, NB), dim3(kAccThreads), 0, s, p, q, draft, tau, B, gamma, V,
                       seed, offset, cpw, nch, chunk_sums, records);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(accept_select_kernel, dim3(NB), dim3(64), 0, s, p, q, draft, tau, B, gamma, V, seed,
                     offset, nch, chunk_sums, records, n_acc, next_tok, status, draws ? 0 : 1);
  return hipGetLastError();
}

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
hipError_t scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace simsd

extern "C" int simsd_accept_prefix_noalloc(const float* p_target, const float* q_draft, const int32_t* draft_tok,
                                           const int32_t* tau, int32_t batch, int32_t B, int32_t gamma,
                                           int64_t vocab, uint64_t seed, uint64_t offset, int32_t* n_accepted,
                                           int32_t* next_token, int32_t* status, void* stream) {
  using namespace simsd;
  size_t need = 0;
  const int rc = accept_prefix_checks(p_target, q_draft, draft_tok, tau, batch, B, gamma, vocab, n_accepted,
                                      next_token, status, &need);
  if (rc != SIMSD_OK) return rc;
  if (need > kNoAllocScratchBytes) return SIMSD_ERR_SCRATCH;
  if (batch == 0) return SIMSD_OK;
  void* ws = nullptr;
  if (need > 0 && scratch_on_current_device(&ws) != hipSuccess) return SIMSD_ERR_HIP;
  const hipError_t e = launch_accept(p_target, q_draft, draft_tok, tau, batch, B, gamma, vocab, seed, offset,
                                     n_accepted, next_token, status, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}
