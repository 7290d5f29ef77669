// Split-KV verification attention on the vector ALUs (fp32 path; also runs
// bf16 as a cross-check of the MFMA kernel).
//
// Page "SimSD - Simple Speculative Decoding in Diffusion Language Models":
// the 2B block rows (D then D~, section 1) attend to the prompt prefix and to
// the block under the tau mask of section 2, with D~_k rotated at D_k's
// position (section 3).
//
// One workgroup = (sequence b, KV head, prompt split, group of 16 rows).
// 256 threads = 16 rows x 16 lanes; lane l16 of a row owns head dims
// l16 + 16e, so a RoPE pair (f, f + d/2) stays in one lane.  Keys are staged
// through LDS 32 at a time as fp32; scores are reduced across the 16 lanes of
// a row with shuffles; the softmax is online in log2 units.
#include "simsd_common.hpp"

namespace simsd {
namespace {

constexpr int kValuKT = 32;    // keys per LDS tile
constexpr int kValuRows = 16;  // rows per workgroup

template <typename T, int HD>
__global__ __launch_bounds__(256) void verify_valu_kernel(Plan pl, VerifyArgs a) {
  constexpr int NE = HD / 16;
  constexpr int HALF = HD / 2;
  __shared__ float Ks[kValuKT][HD];
  __shared__ float Vs[kValuKT][HD];

  const int tid = threadIdx.x;
  const int row = tid >> 4;
  const int l16 = tid & 15;

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

  const int m = rg * kValuRows + row;
  const bool row_ok = m < pl.M;
  const int hh = m / twoB, r = m % twoB;
  const int h = kvh * pl.G + hh;
  const size_t orow = (static_cast<size_t>(b) * twoB + r) * pl.Hq + h;

  if (st) {
    if (pl.nsplit == 1 && row_ok) {
      T* o = static_cast<T*>(a.out) + orow * HD;
      for (int e = 0; e < NE; ++e) Elem<T>::store(o, l16 + 16 * e, 0.0f);
      if (a.lse && l16 == 0) a.lse[orow] = -INFINITY;
    }
    return;
  }
  const int c0 = s * pl.chunk;
  const int c1 = min(c0 + pl.chunk, plen);
  const bool has_block = (s == 0);
  if (c0 >= c1 && !has_block) return;

  // Rotated query row and its block visibility.
  float q[NE];
  uint64_t dbits = 0, mbits = 0;
  if (row_ok) {
    const T* qp = static_cast<const T*>(a.q_blk) + orow * HD;
    const int64_t pos = block_row_pos(pos_b, plen, r, B, pl.rope_seq != 0);
#pragma unroll
    for (int e = 0; e < NE / 2; ++e) {
      const int f = l16 + 16 * e;
      rope_apply(Elem<T>::load(qp, f), Elem<T>::load(qp, f + HALF), rope_cos_sin(pos, rope_inv_freq(f, HD, pl.log2_base)),
                 q[e], q[e + NE / 2]);
    }
    mask_row_bits(tau_b, B, r, pl.mask_mode, dbits, mbits);
  } else {
#pragma unroll
    for (int e = 0; e < NE; ++e) q[e] = 0.0f;
  }

  float mrun = -INFINITY, lrun = 0.0f;
  float o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e] = 0.0f;

  // Softmax update over the keys currently in LDS.  `nkeys` keys are real;
  // in block mode key k is block column kbase + k.
  auto tile = [&](int nkeys, bool block, int kbase) {
    float sc[kValuKT];
    float tmax = -INFINITY;
#pragma unroll
    for (int k = 0; k < kValuKT; ++k) {
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < NE; ++e) part = fmaf(q[e], Ks[k][l16 + 16 * e], part);
      part += __shfl_xor(part, 8, 16);
      part += __shfl_xor(part, 4, 16);
      part += __shfl_xor(part, 2, 16);
      part += __shfl_xor(part, 1, 16);
      bool vis = k < nkeys;
      if (block) {
        const int c = kbase + k;
        vis = vis && (c < B ? ((dbits >> c) & 1ull) : ((mbits >> (c - B)) & 1ull));
      }
      sc[k] = vis ? part * pl.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sc[k]);
    }
    const float mnew = fmaxf(mrun, tmax);
    const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
    const float alpha = exp2f(mrun - muse);
    mrun = mnew;
    lrun *= alpha;
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] *= alpha;
#pragma unroll
    for (int k = 0; k < kValuKT; ++k) {
      const float p = exp2f(sc[k] - muse);
      lrun += p;
#pragma unroll
      for (int e = 0; e < NE; ++e) o[e] = fmaf(p, Vs[k][l16 + 16 * e], o[e]);
    }
  };

  // Block keys (split 0 only): rotated K and V of this KV head, tau-masked.
  if (has_block) {
    for (int bt = 0; bt * kValuKT < twoB; ++bt) {
      for (int i = tid; i < kValuKT * HALF; i += 256) {
        const int key = i / HALF, f = i % HALF, c = bt * kValuKT + key;
        float xo = 0.0f, yo = 0.0f;
        if (c < twoB) {
          const T* kp = static_cast<const T*>(a.k_blk) +
                        ((static_cast<size_t>(b) * twoB + c) * pl.Hkv + kvh) * HD;
          rope_apply(Elem<T>::load(kp, f), Elem<T>::load(kp, f + HALF),
                     rope_cos_sin(block_row_pos(pos_b, plen, c, B, pl.rope_seq != 0),
                                  rope_inv_freq(f, HD, pl.log2_base)),
                     xo, yo);
        }
        Ks[key][f] = xo;
        Ks[key][f + HALF] = yo;
      }
      for (int i = tid; i < kValuKT * HD; i += 256) {
        const int key = i / HD, dd = i % HD, c = bt * kValuKT + key;
        float v = 0.0f;
        if (c < twoB) {
          const T* vp = static_cast<const T*>(a.v_blk) +
                        ((static_cast<size_t>(b) * twoB + c) * pl.Hkv + kvh) * HD;
          v = Elem<T>::load(vp, dd);
        }
        Vs[key][dd] = v;
      }
      __syncthreads();
      tile(min(kValuKT, twoB - bt * kValuKT), true, bt * kValuKT);
      __syncthreads();
    }
  }

  // Prompt keys [c0, c1) of this split.
  const size_t cache_base = (static_cast<size_t>(b) * pl.Hkv + kvh) * static_cast<size_t>(pl.p_max) * HD;
  const T* kc = static_cast<const T*>(a.k_cache) + cache_base;
  const T* vc = static_cast<const T*>(a.v_cache) + cache_base;
  for (int kb = c0; kb < c1; kb += kValuKT) {
    for (int i = tid; i < kValuKT * HD; i += 256) {
      const int key = i / HD, dd = i % HD;
      const int kk = kb + key;
      float kv = 0.0f, vv = 0.0f;
      if (kk < c1) {
        kv = Elem<T>::load(kc, static_cast<size_t>(kk) * HD + dd);
        vv = Elem<T>::load(vc, static_cast<size_t>(kk) * HD + dd);
      }
      Ks[key][dd] = kv;
      Vs[key][dd] = vv;
    }
    __syncthreads();
    tile(min(kValuKT, c1 - kb), false, 0);
    __syncthreads();
  }

  if (!row_ok) return;
  if (pl.nsplit == 1) {
    const float inv = 1.0f / lrun;
    T* op = static_cast<T*>(a.out) + orow * HD;
#pragma unroll
    for (int e = 0; e < NE; ++e) Elem<T>::store(op, l16 + 16 * e, o[e] * inv);
    if (a.lse && l16 == 0) a.lse[orow] = (mrun + log2f(lrun)) * kLn2;
  } else {
    const size_t slot = (static_cast<size_t>(b) * pl.Hkv + kvh) * pl.nsplit + s;
    float* po = a.part_o + (slot * pl.M + m) * HD;
#pragma unroll
    for (int e = 0; e < NE; ++e) po[l16 + 16 * e] = o[e];
    if (l16 == 0) {
      a.part_ml[(slot * pl.M + m) * 2 + 0] = mrun;
      a.part_ml[(slot * pl.M + m) * 2 + 1] = lrun;
    }
  }
}

template <typename T, int HD>
hipError_t launch_typed(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  const unsigned grid = static_cast<unsigned>(pl.nsplit) * pl.nrg * pl.NB * pl.Hkv;
  return launch_with_events(verify_valu_kernel<T, HD>, dim3(grid), dim3(256), 0, s, ev.start, ev.stop, pl, a);
}

}  // namespace

hipError_t launch_verify_valu(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  if (pl.dtype == SIMSD_F32) {
    return pl.d == 64 ? launch_typed<float, 64>(pl, a, s, ev) : launch_typed<float, 128>(pl, a, s, ev);
  }
  return pl.d == 64 ? launch_typed<uint16_t, 64>(pl, a, s, ev) : launch_typed<uint16_t, 128>(pl, a, s, ev);
}

}  // namespace simsd
