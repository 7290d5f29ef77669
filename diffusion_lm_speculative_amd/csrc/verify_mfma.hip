// Split-KV verification attention on the matrix cores (bf16 in, fp32
// accumulate), the hot path of the SimSD verification pass.
//
// Page "SimSD - Simple Speculative Decoding in Diffusion Language Models":
// every block row (D then D~, section 1) attends to the cached prompt and to
// the block under the tau mask of section 2; D~_k is rotated at D_k's RoPE
// position (section 3).  The result is the plain masked softmax; splitting
// the prompt and the online softmax only reorder the sums.
//
// Work decomposition.  One workgroup = (sequence b, KV head, prompt split,
// row group).  All G query heads of the KV head and all 2B block rows share
// every K/V byte, so the G*2B rows are packed into the M dimension and each
// K/V tile is read from HBM once per split.  Each wave owns ROWT tiles of 16
// rows.
//
// MFMA formulation (v_mfma_f32_16x16x32_bf16, wave64).  Scores are computed
// transposed, S^T = K * Q^T, and the output as O^T += V^T * P^T.  In the
// 16x16 accumulator layout lane l holds column l%16, rows 4*(l/16)..+3, so
// with query rows on the N side a lane always holds 4 keys (or 4 head dims)
// of ONE query row: the running max and sum of a row stay in the 4 lanes
// l%16 + 16*g, and the probabilities leave the score accumulator already in
// the B-operand layout of the PV product (keys 4g..4g+3 of two adjacent
// 16-key subtiles form the 8-element k slice of lane group g).  V is stored
// transposed in LDS so its A operand is two 8-byte reads.
//
// Pipeline.  K/V tiles of 64 keys are loaded from HBM with 16-byte
// coalesced loads into registers one tile ahead and stored to a
// double-buffered LDS stage (K row-major, V transposed), one barrier per tile.
#include "simsd_common.hpp"

namespace simsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int KT = 64;  // keys per tile

template <int HD>
struct Layout {
  static constexpr int KSTR = HD * 2 + 16;  // bytes per K row (16-byte pad)
  static constexpr int VSTR = KT * 2 + 8;   // bytes per V^T row (one head dim)
  static constexpr int KBYTES = KT * KSTR;
  static constexpr int VBYTES = HD * VSTR;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int TOTAL = 2 * STAGE;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(const uint16_t (&v)[8]) {
  u16x8 u = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return __builtin_bit_cast(bf16x8, u);
}

template <int HD, int NW, int ROWT>
__global__ __launch_bounds__(NW * 64) void verify_mfma_kernel(Plan pl, VerifyArgs a) {
  using L = Layout<HD>;
  constexpr int NT = NW * 64;
  constexpr int HALF = HD / 2;
  constexpr int KSTEPS = HD / 32;   // k-steps of S^T = K Q^T
  constexpr int DTILES = HD / 16;   // 16-dim tiles of O^T
  constexpr int CPR = HD / 8;       // 16-byte chunks per K/V row
  constexpr int NCH = KT * CPR / NT;  // chunks per thread per tensor per tile
  static_assert(NCH >= 1 && NCH * NT == KT * CPR, "tile must split evenly over threads");

  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int32_t tau_s[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  int idx = blockIdx.x;
  const int s = idx % pl.nsplit;
  idx /= pl.nsplit;
  const int rg = idx % pl.nrg;
  idx /= pl.nrg;
  const int kvh = idx % pl.Hkv;
  const int b = idx / pl.Hkv;

  const int B = pl.B, twoB = pl.twoB;
  const int32_t* tau_b = a.tau + static_cast<size_t>(b) * B;
  const int32_t* pos_b = a.pos_d ? a.pos_d + static_cast<size_t>(b) * B : nullptr;
  const int plen = a.prompt_len ? a.prompt_len[b] : pl.p_max;
  const int st = verify_seq_status(tau_b, B, plen, pl.p_max, pos_b);
  if (a.status && kvh == 0 && s == 0 && rg == 0 && tid == 0) a.status[b] = st;

  // Rows of this wave: m = rg*rows_wg + (wave*ROWT + rt)*16 + n.
  int rm[ROWT];
  bool rok[ROWT];
  size_t rout[ROWT];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    const int m = rg * pl.rows_wg + (wave * ROWT + rt) * 16 + n;
    rm[rt] = m;
    rok[rt] = m < pl.M;
    const int hh = m / twoB, r = m % twoB;
    rout[rt] = (static_cast<size_t>(b) * twoB + r) * pl.Hq + kvh * pl.G + hh;
  }

  if (st) {
    if (pl.nsplit == 1) {
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        if (!rok[rt]) continue;
        uint16_t* op = static_cast<uint16_t*>(a.out) + rout[rt] * HD;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt)
          *reinterpret_cast<uint2*>(op + 16 * dt + 4 * g) = make_uint2(0u, 0u);
        if (a.lse && g == 0) a.lse[rout[rt]] = -INFINITY;
      }
    }
    return;
  }

  const int c0 = s * pl.chunk;
  const int c1 = min(c0 + pl.chunk, plen);
  const int ntiles = c1 > c0 ? (c1 - c0 + KT - 1) / KT : 0;
  const bool has_block = (s == 0);
  if (ntiles == 0 && !has_block) return;

  const size_t cache_base = (static_cast<size_t>(b) * pl.Hkv + kvh) * static_cast<size_t>(pl.p_max) * HD;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + cache_base;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + cache_base;

  // ---- global -> register loads of one prompt tile (keys kb .. kb+63, < c1)
  uint4 kreg[NCH], vreg[NCH];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * NT;
      const int key = c / CPR, col = c % CPR;
      const int kk = kb + key;
      if (kk < c1) {
        const size_t off = static_cast<size_t>(kk) * HD + col * 8;
        kreg[i] = *reinterpret_cast<const uint4*>(kc + off);
        vreg[i] = *reinterpret_cast<const uint4*>(vc + off);
      } else {
        kreg[i] = make_uint4(0u, 0u, 0u, 0u);
        vreg[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  // ---- registers -> LDS stage (K row-major, V transposed)
  auto lstore = [&](int stage) {
    unsigned char* Kb = smem + stage * L::STAGE;
    unsigned char* Vb = Kb + L::KBYTES;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * NT;
      const int key = c / CPR, col = c % CPR;
      *reinterpret_cast<uint4*>(Kb + key * L::KSTR + col * 16) = kreg[i];
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t v = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
        *reinterpret_cast<uint16_t*>(Vb + (col * 8 + e) * L::VSTR + key * 2) = v;
      }
    }
  };

  if (ntiles > 0) gload(c0);

  // ---- RoPE table for the B block positions (aliases stage 0 until the
  //      first prompt tile is stored there)
  float2* cs_tab = reinterpret_cast<float2*>(smem);
  if (tid < B) tau_s[tid] = tau_b[tid];
  for (int i = tid; i < B * HALF; i += NT) {
    const int k = i / HALF, f = i % HALF;
    cs_tab[i] = rope_cos_sin(block_pos(pos_b, plen, k), f, HD, pl.rope_base);
  }
  __syncthreads();

  // ---- rotated Q operands and block visibility per row tile
  bf16x8 qop[ROWT][KSTEPS];
  uint64_t vis_lo[ROWT], vis_hi[ROWT];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    uint16_t qb[KSTEPS][8];
    vis_lo[rt] = 0;
    vis_hi[rt] = 0;
    if (rok[rt]) {
      const int r = rm[rt] % twoB;
      const uint16_t* qp = static_cast<const uint16_t*>(a.q_blk) + rout[rt] * HD;
      float qv[KSTEPS][8];
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i) {
        const uint4 raw = *reinterpret_cast<const uint4*>(qp + 32 * i + 8 * g);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[i][e] = bf16_bits_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))));
      }
      const float2* csr = cs_tab + (r % B) * HALF;
#pragma unroll
      for (int i = 0; i < KSTEPS / 2; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float xo, yo;
          rope_apply(qv[i][e], qv[i + KSTEPS / 2][e], csr[32 * i + 8 * g + e], xo, yo);
          qb[i][e] = f32_to_bf16_bits(xo);
          qb[i + KSTEPS / 2][e] = f32_to_bf16_bits(yo);
        }
      }
      uint64_t dbits, mbits;
      mask_row_bits(tau_s, B, r, pl.mask_mode, dbits, mbits);
      if (B >= 64) {
        vis_lo[rt] = dbits;
        vis_hi[rt] = mbits;
      } else {
        vis_lo[rt] = dbits | (mbits << B);
        vis_hi[rt] = mbits >> (64 - B);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[i][e] = 0;
    }
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) qop[rt][i] = bits_to_bf16x8(qb[i]);
  }

  // ---- online-softmax state
  float mrun[ROWT], lpart[ROWT];
  f32x4 acc[ROWT][DTILES];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    mrun[rt] = -INFINITY;
    lpart[rt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) acc[rt][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // One 64-key tile from LDS stage `stage`.  Prompt mode: key kbase+k is
  // visible iff < klimit.  Block mode: block column kbase+k is visible per
  // the row's tau bits.
  auto compute = [&](int stage, bool block, int kbase, int klimit) {
    const unsigned char* Kb = smem + stage * L::STAGE;
    const unsigned char* Vb = Kb + L::KBYTES;
    f32x4 sacc[ROWT][4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x8 kop[KSTEPS];
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i)
        kop[i] = *reinterpret_cast<const bf16x8*>(Kb + (16 * t4 + n) * L::KSTR + (32 * i + 8 * g) * 2);
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        f32x4 sa = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < KSTEPS; ++i) sa = mfma(kop[i], qop[rt][i], sa);
        sacc[rt][t4] = sa;
      }
    }
    bf16x8 pop[ROWT][2];
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt) {
      float sv[4][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = 16 * t4 + 4 * g + j;
          bool vis;
          if (block) {
            const int c = kbase + k;
            vis = c < 64 ? ((vis_lo[rt] >> c) & 1ull) : ((vis_hi[rt] >> (c - 64)) & 1ull);
          } else {
            vis = kbase + k < klimit;
          }
          const float x = vis ? sacc[rt][t4][j] * pl.scale_log2 : -INFINITY;
          sv[t4][j] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrun[rt], tmax);
      const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
      const float alpha = exp2f(mrun[rt] - muse);
      mrun[rt] = mnew;
      float lsum = 0.0f;
      __bf16 pb[2][8];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = exp2f(sv[t4][j] - muse);
          lsum += p;
          pb[t4 >> 1][(t4 & 1) * 4 + j] = static_cast<__bf16>(p);
        }
      }
      lpart[rt] = lpart[rt] * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) acc[rt][dt] *= alpha;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        pop[rt][u] = bf16x8{pb[u][0], pb[u][1], pb[u][2], pb[u][3], pb[u][4], pb[u][5], pb[u][6], pb[u][7]};
    }
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const unsigned char* vrow = Vb + (16 * dt + n) * L::VSTR;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (32 * u + 4 * g) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (32 * u + 16 + 4 * g) * 2);
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
        for (int rt = 0; rt < ROWT; ++rt) acc[rt][dt] = mfma(vop, pop[rt][u], acc[rt][dt]);
      }
    }
  };

  // ---- block keys (split 0): rotated K and V of this KV head in stage 1
  if (has_block) {
    unsigned char* Kb = smem + L::STAGE;
    unsigned char* Vb = Kb + L::KBYTES;
    const uint16_t* kblk = static_cast<const uint16_t*>(a.k_blk);
    const uint16_t* vblk = static_cast<const uint16_t*>(a.v_blk);
    for (int bt = 0; bt * KT < twoB; ++bt) {
      for (int i = tid; i < KT * HALF; i += NT) {
        const int key = i / HALF, f = i % HALF, c = bt * KT + key;
        float xo = 0.0f, yo = 0.0f;
        if (c < twoB) {
          const uint16_t* kp = kblk + ((static_cast<size_t>(b) * twoB + c) * pl.Hkv + kvh) * HD;
          rope_apply(bf16_bits_to_f32(kp[f]), bf16_bits_to_f32(kp[f + HALF]), cs_tab[(c % B) * HALF + f], xo, yo);
        }
        *reinterpret_cast<uint16_t*>(Kb + key * L::KSTR + f * 2) = f32_to_bf16_bits(xo);
        *reinterpret_cast<uint16_t*>(Kb + key * L::KSTR + (f + HALF) * 2) = f32_to_bf16_bits(yo);
      }
      for (int i = tid; i < KT * HD; i += NT) {
        const int key = i / HD, dd = i % HD, c = bt * KT + key;
        uint16_t v = 0;
        if (c < twoB) v = vblk[((static_cast<size_t>(b) * twoB + c) * pl.Hkv + kvh) * HD + dd];
        *reinterpret_cast<uint16_t*>(Vb + dd * L::VSTR + key * 2) = v;
      }
      __syncthreads();
      compute(1, true, bt * KT, 0);
      __syncthreads();
    }
  } else {
    __syncthreads();  // every wave is done with the RoPE table in stage 0
  }

  // ---- prompt keys [c0, c1)
  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    lstore(stage);
    __syncthreads();
    if (t + 1 < ntiles) gload(c0 + (t + 1) * KT);
    compute(stage, false, c0 + t * KT, c1);
  }

  // ---- epilogue
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    float l = lpart[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!rok[rt]) continue;
    if (pl.nsplit == 1) {
      const float inv = 1.0f / l;
      uint16_t* op = static_cast<uint16_t*>(a.out) + rout[rt] * HD;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const f32x4 v = acc[rt][dt];
        const uint32_t w0 = f32_to_bf16_bits(v[0] * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1] * inv)) << 16);
        const uint32_t w1 = f32_to_bf16_bits(v[2] * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3] * inv)) << 16);
        *reinterpret_cast<uint2*>(op + 16 * dt + 4 * g) = make_uint2(w0, w1);
      }
      if (a.lse && g == 0) a.lse[rout[rt]] = (mrun[rt] + log2f(l)) * kLn2;
    } else {
      const size_t slot = (static_cast<size_t>(b) * pl.Hkv + kvh) * pl.nsplit + s;
      float* po = a.part_o + (slot * pl.M + rm[rt]) * HD;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const f32x4 v = acc[rt][dt];
        *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0) {
        a.part_ml[(slot * pl.M + rm[rt]) * 2 + 0] = mrun[rt];
        a.part_ml[(slot * pl.M + rm[rt]) * 2 + 1] = l;
      }
    }
  }
}

template <int HD, int NW, int ROWT>
hipError_t launch_cfg(const Plan& pl, const VerifyArgs& a, hipStream_t s) {
  auto kern = verify_mfma_kernel<HD, NW, ROWT>;
  const size_t lds = Layout<HD>::TOTAL;
  static bool attr_set = false;  // benign race: setting the same attribute twice is harmless
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = static_cast<unsigned>(pl.nsplit) * pl.nrg * pl.NB * pl.Hkv;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, s, pl, a);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_hd(const Plan& pl, const VerifyArgs& a, hipStream_t s) {
  const int nw = pl.threads / 64;
  if (pl.rowt == 1) {
    switch (nw) {
      case 1: return launch_cfg<HD, 1, 1>(pl, a, s);
      case 2: return launch_cfg<HD, 2, 1>(pl, a, s);
      case 4: return launch_cfg<HD, 4, 1>(pl, a, s);
      default: return launch_cfg<HD, 8, 1>(pl, a, s);
    }
  }
  switch (nw) {
    case 4: return launch_cfg<HD, 4, 2>(pl, a, s);
    default: return launch_cfg<HD, 8, 2>(pl, a, s);
  }
}

}  // namespace

hipError_t launch_verify_mfma(const Plan& pl, const VerifyArgs& a, hipStream_t s) {
  return pl.d == 64 ? launch_hd<64>(pl, a, s) : launch_hd<128>(pl, a, s);
}

}  // namespace simsd
