// Device helpers shared by the verification kernels, the merge and the debug
// exports: the tau-driven mask rows, per-sequence validation, RoPE-copy
// angles, bf16 conversion and the split-KV plan.  Page: "SimSD - Simple
// Speculative Decoding in Diffusion Language Models" (sections 1-3).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "simsd.h"

namespace simsd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN): the language's
// float -> __bf16 conversion, one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }
  __device__ static __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

// ---------------------------------------------------------------- temporal mask
// Visibility of the block columns for block row r (0 <= r < 2B), as two
// B-bit words: dbits bit j = the row sees data token D_j, mbits bit j = the
// row sees mask slot D~_j.  Section 2 of the page gives the mask-slot rows
// (D_j when tau_j < tau_i, D~_j when tau_j >= tau_i); data rows see D_j with
// tau_j <= tau_i and no slot.  Stage 0 marks a position committed in an
// earlier round of the block: every slot row of an open position sees it.  `tau_at(j)` returns the stage of position j
// (from memory, or from another lane's register).
template <class TauAt>
__device__ __forceinline__ void mask_row_bits_at(TauAt tau_at, int B, int r, int mode, uint64_t& dbits,
                                                 uint64_t& mbits) {
  const uint64_t all = (B >= 64) ? ~0ull : ((1ull << B) - 1ull);
  if (mode == SIMSD_MASK_FULL) {
    dbits = all;
    mbits = all;
    return;
  }
  const bool slot_row = r >= B;
  const int ti = tau_at(slot_row ? r - B : r);
  // D_j is visible when tau_j <= lim (a slot row needs tau_j < tau_i); a slot
  // row sees exactly the slots D~_j whose data token it does not see.
  const int lim = slot_row ? ti - 1 : ti;
  uint32_t lo = 0, hi = 0;
  for (int j = 0; j < B && j < 32; ++j) lo |= static_cast<uint32_t>(tau_at(j) <= lim) << j;
  for (int j = 32; j < B; ++j) hi |= static_cast<uint32_t>(tau_at(j) <= lim) << (j - 32);
  dbits = (static_cast<uint64_t>(hi) << 32) | lo;
  mbits = slot_row ? (all & ~dbits) : 0ull;
}

// The same bits from a wave's view of the stage labels: lanes 0..B-1 hold
// tau_j in `tau_lane` (0..B; 1 <= B <= 64), and every lane of the wave calls this
// (wave ballots).  The D_j row r sees are those with a stage of at most lim,
// the ballot of tau_j <= lim for the lim of the row; a slot row sees the
// slots D~_j whose D_j it does not see.
__device__ __forceinline__ void mask_row_bits_wave(int tau_lane, int lane, int B, int r, int mode, uint64_t& dbits,
                                                   uint64_t& mbits) {
  const uint64_t all = (B >= 64) ? ~0ull : ((1ull << B) - 1ull);
  const int ti = __shfl(tau_lane, r % B);
  const bool slot_row = r >= B;
  const int lim = slot_row ? ti - 1 : ti;
  uint64_t d = 0;
  for (int k = 0; k <= B; ++k) {  // lim = 0: the positions committed in earlier rounds
    const uint64_t pk = __ballot(lane < B && tau_lane <= k);
    d = (lim == k) ? pk : d;
  }
  dbits = d;
  mbits = slot_row ? (all & ~d) : 0ull;
  if (mode == SIMSD_MASK_FULL) {
    dbits = all;
    mbits = all;
  }
}

__device__ __forceinline__ void mask_row_bits(const int32_t* tau, int B, int r, int mode, uint64_t& dbits,
                                              uint64_t& mbits) {
  mask_row_bits_at([tau](int j) { return tau[j]; }, B, r, mode, dbits, mbits);
}

// Per-sequence validation of a verification call (flags of simsd.h).
__device__ __forceinline__ int verify_seq_status(const int32_t* tau_b, int B, int plen, int p_max,
                                                 const int32_t* pos_b) {
  int st = 0;
  for (int j = 0; j < B; ++j) {
    const int t = tau_b[j];
    if (t < 0 || t > B) st |= SIMSD_ST_TAU_RANGE;
    if (pos_b && pos_b[j] < 0) st |= SIMSD_ST_POS_NEG;
  }
  if (plen < 0 || plen > p_max) st |= SIMSD_ST_PROMPT_LEN;
  return st;
}

// ---------------------------------------------------------------- RoPE copy
// Rotate-half RoPE: pair (x_f, x_{f+d/2}) turns by pos * base^(-2f/d).  The
// frequency is exp2(-(2f/d) * log2(base)) in fp64 (log2(base) from the host;
// within a few ulp of base^(-2f/d), i.e. ~1e-10 rad at position 1e5).  The
// angle is formed and reduced to [-pi, pi] in fp64 (positions
// reach 1e4..1e5, where an fp32 angle is off by ~1e-3 rad): a two-constant
// Cody-Waite reduction by 2*pi, exact to ~1e-16 rad for positions below
// ~1e6, keeps the fp64 sine and cosine on their short path.  The results are
// rounded to fp32.
constexpr double kTwoPiHi = 6.28318530717958623200e+00;  // 2*pi rounded to double
constexpr double kTwoPiLo = 2.44929359829470635445e-16;  // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 1.59154943091895335769e-01;

__device__ __forceinline__ double rope_inv_freq(int f, int d, double log2_base) {
  return exp2(-(2.0 * f / d) * log2_base);
}

__device__ __forceinline__ float2 rope_cos_sin(int64_t pos, double inv_freq) {
  const double theta = static_cast<double>(pos) * inv_freq;
  const double k = rint(theta * kInvTwoPi);
  const double red = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, theta));
  double s, c;
  sincos(red, &s, &c);
  return make_float2(static_cast<float>(c), static_cast<float>(s));
}

// Rotate one pair with a (cos, sin) from rope_cos_sin.  Written with explicit
// fmas so every kernel and the debug export round identically.
__device__ __forceinline__ void rope_apply(float x, float y, float2 cs, float& xo, float& yo) {
  xo = fmaf(x, cs.x, -(y * cs.y));
  yo = fmaf(y, cs.x, x * cs.y);
}

// RoPE index of block row r (0..B-1: D_r, B..2B-1: D~_{r-B}) of a sequence:
// D_k at pos_d[k] (default P_b + k); D~_k at the same index (the RoPE copy)
// or B past it (the ablation without the copy, `seq`).
__device__ __forceinline__ int64_t block_row_pos(const int32_t* pos_b, int plen, int r, int B, bool seq) {
  const int k = r < B ? r : r - B;
  const int64_t p = pos_b ? static_cast<int64_t>(pos_b[k]) : static_cast<int64_t>(plen) + k;
  return seq && r >= B ? p + B : p;
}

// ---------------------------------------------------------------- split-KV plan
// Work of one launch: grid = nsplit * nrg * NB * Hkv workgroups.  Split s of
// (b, kvh) covers prompt keys [s*chunk, min((s+1)*chunk, P_b)); split 0 also
// owns the 2B block keys, so every row has at least one visible key in it.
// With nsplit == 1 the kernel writes the final output; otherwise it writes
// unnormalised partials (o, m, l) that the merge combines.
struct Plan {
  int NB, Hq, Hkv, G, d, B, twoB, M;  // M = G * 2B rows per KV head
  int p_max, chunk, nsplit;
  int rows_wg, nrg;                   // rows per workgroup, row groups per KV head
  int threads;                        // threads per workgroup
  int rowt;                           // 16-row tiles per wave
  int ksplit;                         // MFMA: waves sharing the keys of a tile
  int nstage;                         // MFMA: LDS ring stages
  int impl;                           // SIMSD_IMPL_VALU or SIMSD_IMPL_MFMA
  int dtype, mask_mode;
  double rope_base;
  double log2_base;                   // log2(rope_base)
  int qsep;                           // MFMA: query rows staged in their own LDS region
  int blk_rows;                       // MFMA: block K/V rows in their own LDS region (0: through the ring)
  int kv_stream;                      // MFMA: K/V tiles loaded non-temporally (the call streams >= the last-level cache)
  int lpt;                            // MFMA: workgroups take their items longest first
  int rope_seq;                       // D~_k at pos(D_k) + B instead of pos(D_k)
  int tab_rows;                       // distinct block positions: B, or 2B with rope_seq
  float scale_log2;                   // softmax scale * log2(e)
  size_t part_o_floats, part_ml_floats;
};

struct VerifyArgs {
  const void* q_blk;
  const void* k_blk;
  const void* v_blk;
  const void* k_cache;
  const void* v_cache;
  const int32_t* prompt_len;
  const int32_t* tau;
  const int32_t* pos_d;
  void* out;
  float* lse;
  int32_t* status;
  float* part_o;   // [NB*Hkv*nsplit][M][d]
  float* part_ml;  // [NB*Hkv*nsplit][M][2]  (running max in log2 units, sum)
};

// Number of splits of (b) that hold a partial: split 0 always, split s >= 1
// when it starts inside the prompt.
__device__ __forceinline__ int valid_splits(int plen, int chunk, int nsplit) {
  int n = (plen + chunk - 1) / chunk;
  if (n < 1) n = 1;
  return n < nsplit ? n : nsplit;
}

// Let kernel `Kern` use up to `bytes` of dynamic LDS on the current device.
// The attribute is set once per (kernel, device), under std::call_once, so
// first launches from several host threads at once do not race; `bytes` must
// be the same on every call for one kernel (each caller passes its largest).
template <auto Kern>
hipError_t allow_dynamic_lds(int bytes) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices)
    return hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  std::call_once(once[dev], [&] {
    err[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                   bytes);
  });
  return err[dev];
}

// Events a caller binds to a pass: `start` takes the start time of its first
// kernel and `stop` the end time of its last, from the dispatches themselves.
struct PassEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launch `kern` on `s`; when an event is given, through hipExtLaunchKernelGGL,
// which records `start` / `stop` at the kernel's own start and end.
template <typename... KArgs, typename... Args>
hipError_t launch_with_events(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                              hipEvent_t start, hipEvent_t stop, Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kern, grid, block, static_cast<uint32_t>(lds), s, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, s, args...);
  return hipGetLastError();
}

// Host-side launchers (one per translation unit).
hipError_t launch_verify_valu(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev);
hipError_t launch_verify_mfma(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev);
size_t mfma_lds_bytes(int hd, int nstage, int tab_rows, int rows_wg, bool qsep, int blk_rows);

// y = x W^T (bf16, fp32 accumulation); output channels [0, cut1) go to
// out0, [cut1, cut2) to out1, [cut2, N) to out2, row-major with row lengths
// ld0..ld2.
int linear_tile(int64_t M, int N);

hipError_t launch_commit(const int32_t* tau, const int32_t* draft, const int32_t* n_acc, const int32_t* next_tok,
                         int NB, int B, uint64_t* committed, int32_t* block_tok, hipStream_t s);
hipError_t launch_next_round(const uint64_t* committed, const int32_t* block_tok, const int32_t* rank,
                             const int32_t* draft, int NB, int B, int32_t* tau_out, int32_t* tok_out, hipStream_t s);
hipError_t launch_append_kv(const Plan& pl, const void* k_blk, const void* v_blk, const int32_t* pos_d,
                            const uint64_t* committed, int32_t* prompt_len, void* k_cache, void* v_cache,
                            int32_t* status, hipStream_t s);
hipError_t launch_linear(const uint16_t* x, const uint16_t* w, int64_t M, int N, int K, int cut1, int cut2,
                         uint16_t* out0, int ld0, uint16_t* out1, int ld1, uint16_t* out2, int ld2, hipStream_t s);
hipError_t launch_merge(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev);
void accept_plan(int NB, int64_t V, int& nch, int& cpw, int& ngrp);
// MI355X last-level (Infinity) cache: a call that reads at least this many
// bytes once streams them with the non-temporal bit.
constexpr int64_t kLastLevelCache = int64_t{256} << 20;
size_t accept_workspace_bytes(int NB, int B, int64_t V);
int accept_prefix_checks(const float* p_target, const float* q_draft, const int32_t* draft_tok, const int32_t* tau,
                         int32_t batch, int32_t B, int32_t gamma, int64_t vocab, const int32_t* n_accepted,
                         const int32_t* next_token, const int32_t* status, size_t* need);
int coupled_chunks(int64_t V);
size_t coupled_workspace_bytes(int NB, int B, int64_t V);
hipError_t launch_accept_coupled(const float* p, const float* e, const int32_t* draft, const int32_t* tau, int NB,
                                 int B, int gamma, int64_t V, int32_t* n_out, int32_t* next_out, int32_t* status,
                                 void* workspace, hipStream_t s);
hipError_t launch_accept(const float* p, const float* q, const int32_t* draft, const int32_t* tau,
                         int NB, int B, int gamma, int64_t V, uint64_t seed, uint64_t offset,
                         int32_t* n_acc, int32_t* next_tok, int32_t* status, void* workspace, hipStream_t s);
hipError_t launch_debug_mask(const int32_t* tau, int NB, int B, int mode, uint64_t* bits, hipStream_t s);
hipError_t launch_debug_rope(const Plan& pl, const void* q_blk, const void* k_blk,
                             const int32_t* prompt_len, const int32_t* pos_d,
                             void* q_rot, void* k_rot, hipStream_t s);

}  // namespace simsd
