// The commit step between verification rounds (page "SimSD - Simple
// Speculative Decoding in Diffusion Language Models", section 4: the longest
// accepted prefix is committed and the process repeats; "Key contributions"
// item 3: the method runs with a KV cache and blockwise decoding).
//
// The next round of a block labels the committed positions 0 (context for
// every stage, walked by no one) and the open ones 1..m in the drafter's
// order.
//
// commit: one wave per sequence, lane k = response position k.  The
// positions of stages 1..n take their drafted tokens, the position of stage
// n+1 the replacement token when the walk drew one; a ballot over the lanes
// gives the new committed bits.
//
// append: one workgroup per (KV head, sequence) whose block is finished (all
// B positions committed).  The data rows' keys are rotated at their RoPE
// positions with the same angle reduction and rounding as the attention
// kernels (so the cached keys equal the ones the verification pass used for
// D_0..D_{B-1}) and the values copied, both to cache rows P_b .. P_b+B-1.  A
// second launch on the same stream then grows P_b by B and writes the status,
// so no row workgroup can see the new length.
#include "simsd_common.hpp"

namespace simsd {
namespace {

__global__ __launch_bounds__(64) void commit_kernel(const int32_t* __restrict__ tau, const int32_t* __restrict__ draft,
                                                    const int32_t* __restrict__ n_acc,
                                                    const int32_t* __restrict__ next_tok, int B,
                                                    uint64_t* committed, int32_t* block_tok) {
  const int b = blockIdx.x;
  const int k = threadIdx.x;
  const int n = n_acc[b];
  if (n < 0) return;  // a faulted round commits nothing
  const int nx = next_tok ? next_tok[b] : -1;
  int t = 0, tok = -1;
  if (k < B) {
    t = tau[static_cast<size_t>(b) * B + k];
    tok = draft[static_cast<size_t>(b) * B + k];
  }
  const bool accepted = k < B && t >= 1 && t <= n;
  const bool replaced = k < B && nx >= 0 && t == n + 1;
  if (accepted || replaced) block_tok[static_cast<size_t>(b) * B + k] = accepted ? tok : nx;
  const uint64_t bits = __ballot(accepted || replaced);
  if (k == 0) committed[b] |= bits;
}

// next round: one wave per sequence, lane k = response position k.  A
// committed position takes stage 0 and its committed token; an open one
// takes 1 + the number of open positions ahead of it in the drafter's order
// (rank, then position), and the drafter's token.
__global__ __launch_bounds__(64) void next_round_kernel(const uint64_t* __restrict__ committed,
                                                        const int32_t* __restrict__ block_tok,
                                                        const int32_t* __restrict__ rank,
                                                        const int32_t* __restrict__ draft, int B, int32_t* tau_out,
                                                        int32_t* tok_out) {
  const int b = blockIdx.x;
  const int k = threadIdx.x;
  const size_t i = static_cast<size_t>(b) * B + k;
  const uint64_t c = committed[b];
  const bool done = k < B && ((c >> k) & 1ull);
  const bool open = k < B && !done;
  const int r = (k < B && rank) ? rank[i] : k;
  int ahead = 0;
  for (int j = 0; j < B; ++j) {
    const int rj = __shfl(r, j);
    const bool oj = !((c >> j) & 1ull);
    ahead += (oj && (rj < r || (rj == r && j < k))) ? 1 : 0;
  }
  if (k < B) {
    tau_out[i] = open ? ahead + 1 : 0;
    tok_out[i] = open ? draft[i] : block_tok[i];
  }
}

// Whether sequence b's block is finished (every block counts as finished
// without a mask).
__device__ __forceinline__ bool block_finished(const Plan& pl, const uint64_t* committed, int b) {
  const uint64_t full = pl.B >= 64 ? ~0ull : ((1ull << pl.B) - 1ull);
  return !committed || committed[b] == full;
}

// Four consecutive elements of a row (8 bytes of bf16 or 16 of fp32), held
// as fp32 for the rotation and rounded like Elem<T>::store.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  float v[4];
  __device__ static Vec4 load(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    return Vec4{{a.x, a.y, a.z, a.w}};
  }
  __device__ float get(int j) const { return v[j]; }
  __device__ void set(int j, float x) { v[j] = x; }
  __device__ void store(float* p) const { *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]); }
};
template <> struct Vec4<uint16_t> {
  uint16_t v[4];
  __device__ static Vec4 load(const uint16_t* p) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    return Vec4{{static_cast<uint16_t>(a.x & 0xffffu), static_cast<uint16_t>(a.x >> 16),
                 static_cast<uint16_t>(a.y & 0xffffu), static_cast<uint16_t>(a.y >> 16)}};
  }
  __device__ float get(int j) const { return bf16_bits_to_f32(v[j]); }
  __device__ void set(int j, float x) { v[j] = f32_to_bf16_bits(x); }
  __device__ void store(uint16_t* p) const {
    *reinterpret_cast<uint2*>(p) = make_uint2(v[0] | (static_cast<uint32_t>(v[1]) << 16),
                                              v[2] | (static_cast<uint32_t>(v[3]) << 16));
  }
};

// Fault flags of a finished block's append: no room for B more rows, or a
// negative given position (the attention's flag for it).  `neg_pos` says
// whether pos_d holds a negative entry for this sequence.
__device__ __forceinline__ int append_flags(const Plan& pl, int P, bool neg_pos) {
  const bool room = P >= 0 && static_cast<int64_t>(P) + pl.B <= pl.p_max;
  return (room ? 0 : SIMSD_ST_PROMPT_LEN) | (neg_pos ? SIMSD_ST_POS_NEG : 0);
}

// Rows of one (KV head, sequence): B keys rotated and B values copied.
template <typename T>
__global__ __launch_bounds__(128) void append_rows_kernel(Plan pl, const T* __restrict__ k_blk,
                                                          const T* __restrict__ v_blk,
                                                          const int32_t* __restrict__ pos_d,
                                                          const uint64_t* __restrict__ committed,
                                                          const int32_t* __restrict__ prompt_len, T* k_cache,
                                                          T* v_cache) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int B = pl.B, Hkv = pl.Hkv, d = pl.d, half = d / 2;
  const int P = prompt_len[b];
  if (!block_finished(pl, committed, b)) return;
  const int32_t* pos_b = pos_d ? pos_d + static_cast<size_t>(b) * B : nullptr;
  const int lane = threadIdx.x & 63;  // each wave checks the B <= 64 positions itself
  const bool neg_pos = pos_b && __any(lane < B && pos_b[lane] < 0);
  if (append_flags(pl, P, neg_pos)) return;
  const size_t cache0 = (static_cast<size_t>(b) * Hkv + h) * pl.p_max + P;
  // keys: four rotation pairs (f..f+3, f+d/2..f+d/2+3) per item, each half
  // one 8- or 16-byte access (d/2 is a multiple of 4)
  const int q4 = half / 4;
  for (int i = threadIdx.x; i < B * q4; i += blockDim.x) {
    const int f = (i % q4) * 4, k = i / q4;
    const T* src = k_blk + ((static_cast<size_t>(b) * pl.twoB + k) * Hkv + h) * d;
    T* dst = k_cache + (cache0 + k) * d;
    const int64_t pos = pos_b ? static_cast<int64_t>(pos_b[k]) : static_cast<int64_t>(P) + k;
    Vec4<T> x = Vec4<T>::load(src + f), y = Vec4<T>::load(src + f + half), xo, yo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a, c;
      rope_apply(x.get(j), y.get(j), rope_cos_sin(pos, rope_inv_freq(f + j, d, pl.log2_base)), a, c);
      xo.set(j, a);
      yo.set(j, c);
    }
    xo.store(dst + f);
    yo.store(dst + f + half);
  }
  // values: 16-byte copies
  constexpr int kPer = 16 / sizeof(T);
  const int dv = d / kPer;
  for (int i = threadIdx.x; i < B * dv; i += blockDim.x) {
    const int e = (i % dv) * kPer, k = i / dv;
    *reinterpret_cast<uint4*>(v_cache + (cache0 + k) * d + e) =
        *reinterpret_cast<const uint4*>(v_blk + ((static_cast<size_t>(b) * pl.twoB + k) * Hkv + h) * d + e);
  }
}

// Length and status of each sequence; launched after the rows so that every
// row workgroup has read the old length.
__global__ __launch_bounds__(64) void append_len_kernel(Plan pl, const int32_t* __restrict__ pos_d,
                                                        const uint64_t* __restrict__ committed,
                                                        int32_t* prompt_len, int32_t* status) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= pl.NB) return;
  if (!block_finished(pl, committed, b)) {  // open block: nothing to do
    if (status) status[b] = 0;
    return;
  }
  const int P = prompt_len[b];
  bool neg_pos = false;
  if (pos_d)
    for (int k = 0; k < pl.B; ++k) neg_pos |= pos_d[static_cast<size_t>(b) * pl.B + k] < 0;
  const int st = append_flags(pl, P, neg_pos);
  if (st == 0) prompt_len[b] = P + pl.B;
  if (status) status[b] = st;
}

}  // namespace

hipError_t launch_commit(const int32_t* tau, const int32_t* draft, const int32_t* n_acc, const int32_t* next_tok,
                         int NB, int B, uint64_t* committed, int32_t* block_tok, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(NB), dim3(64), 0, s, tau, draft, n_acc, next_tok, B, committed, block_tok);
  return hipGetLastError();
}

hipError_t launch_next_round(const uint64_t* committed, const int32_t* block_tok, const int32_t* rank,
                             const int32_t* draft, int NB, int B, int32_t* tau_out, int32_t* tok_out, hipStream_t s) {
  hipLaunchKernelGGL(next_round_kernel, dim3(NB), dim3(64), 0, s, committed, block_tok, rank, draft, B, tau_out,
                     tok_out);
  return hipGetLastError();
}

hipError_t launch_append_kv(const Plan& pl, const void* k_blk, const void* v_blk, const int32_t* pos_d,
                            const uint64_t* committed, int32_t* prompt_len, void* k_cache, void* v_cache,
                            int32_t* status, hipStream_t s) {
  const dim3 grid(pl.Hkv, pl.NB);
  if (pl.dtype == SIMSD_BF16) {
    hipLaunchKernelGGL(append_rows_kernel<uint16_t>, grid, dim3(128), 0, s, pl, static_cast<const uint16_t*>(k_blk),
                       static_cast<const uint16_t*>(v_blk), pos_d, committed, prompt_len,
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache));
  } else {
    hipLaunchKernelGGL(append_rows_kernel<float>, grid, dim3(128), 0, s, pl, static_cast<const float*>(k_blk),
                       static_cast<const float*>(v_blk), pos_d, committed, prompt_len, static_cast<float*>(k_cache),
                       static_cast<float*>(v_cache));
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(append_len_kernel, dim3((pl.NB + 63) / 64), dim3(64), 0, s, pl, pos_d, committed, prompt_len,
                     status);
  return hipGetLastError();
}

}  // namespace simsd
