// Combine the split-KV partials of the verification attention into the
// final rows.  Each split s of a row holds an unnormalised sum o_s, its
// running max m_s (log2 units) and sum l_s; the softmax over the union of
// the splits' keys is
//   m* = max_s m_s,  l* = sum_s 2^(m_s - m*) l_s,
//   out = (sum_s 2^(m_s - m*) o_s) / l*,  lse = (m* + log2 l*) * ln 2.
// A faulted sequence gets zero rows and lse = -inf.
//
// The kernel is a pure stream (fp32 partials in, one row out per row), so
// what bounds it is how many bytes each wave keeps in flight.  A workgroup
// owns RWG consecutive rows of one (sequence, kv head): a row is HD/4 lanes
// wide (one float4 each), a wave covers 64/(HD/4) rows per pass and U
// passes, and the partials of up to SG splits are loaded in one round, with
// no load waiting on another.  The sequence's prompt length (which splits
// are valid) is one scalar load ahead of them; its fault flags are loaded
// alongside and only decide what is stored.  Splits are summed in index
// order, so the result does not depend on SG.
#include "simsd_common.hpp"

namespace simsd {
namespace {

template <int HD, int SG_, int U_>
struct MergeShape {
  static constexpr int LPR = HD / 4;    // lanes per row
  static constexpr int RPP = 64 / LPR;  // rows per wave and pass
  static constexpr int U = U_;          // passes per wave
  static constexpr int RW = RPP * U;    // rows per wave
  static constexpr int RWG = RW * 4;    // rows per workgroup (4 waves)
  static constexpr int SG = SG_;        // splits loaded per round
};

__device__ __forceinline__ float4 fma4(float w, const float4& x, const float4& y) {
  return make_float4(fmaf(w, x.x, y.x), fmaf(w, x.y, y.y), fmaf(w, x.z, y.z), fmaf(w, x.w, y.w));
}

template <typename T>
__device__ __forceinline__ void store4(T* p, const float4& v);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float4& v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const float4& v) {
  const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_bits(v.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(v.y)) << 16);
  const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_bits(v.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(v.w)) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

// FITS: the launcher has checked nsplit <= SG, so one round loads every split
template <typename T, int HD, int SG, int U, bool FITS>
__global__ __launch_bounds__(256) void merge_kernel(Plan pl, VerifyArgs a) {
  using S = MergeShape<HD, SG, U>;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nchunk = (pl.M + S::RWG - 1) / S::RWG;
  const int bh = static_cast<int>(blockIdx.x) / nchunk;  // b * Hkv + kvh
  const int chunk = static_cast<int>(blockIdx.x) - bh * nchunk;
  const int b = bh / pl.Hkv;
  const int kvh = bh - b * pl.Hkv;
  const int col = (lane % S::LPR) * 4;
  const int m0 = chunk * S::RWG + wave * S::RW + lane / S::LPR;  // row of pass u: m0 + u * RPP
  // rows past M load row M-1 (in bounds) and store nothing; offsets are
  // within one split's [M][HD] block, added to a base that is uniform per split
  uint32_t off_o[S::U], off_ml[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const uint32_t mr = static_cast<uint32_t>(min(m0 + u * S::RPP, pl.M - 1));
    off_o[u] = (mr * HD + col) * 4u;
    off_ml[u] = mr * 8u;
  }

  const int plen = a.prompt_len ? a.prompt_len[b] : pl.p_max;
  // the sequence's fault flags, lane j checking position min(j, B-1) (1 <= B
  // <= 64); loaded with no branch so that nothing waits on them before the
  // partials are in flight
  const size_t jb = static_cast<size_t>(b) * pl.B + min(lane, pl.B - 1);
  // (with no positions the tau word stands in: a negative one faults anyway)
  const int tau_j = a.tau[jb];
  const int pos_j = (a.pos_d ? a.pos_d : a.tau)[jb];
  const int nv = valid_splits(min(max(plen, 0), pl.p_max), pl.chunk, pl.nsplit);
  const size_t slot0 = static_cast<size_t>(bh) * pl.nsplit;
  auto base_o = [&](int s) {
    return reinterpret_cast<const char*>(a.part_o + (slot0 + s) * pl.M * HD);
  };
  auto base_ml = [&](int s) {
    return reinterpret_cast<const char*>(a.part_ml + (slot0 + s) * pl.M * 2);
  };

  float2 ml[S::SG][S::U];
  float4 po[S::SG][S::U];
  auto load_group = [&](int s0) {
#pragma unroll
    for (int g = 0; g < S::SG; ++g) {
      if (s0 + g < nv) {
        const char* bo = base_o(s0 + g);
        const char* bm = base_ml(s0 + g);
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
          ml[g][u] = *reinterpret_cast<const float2*>(bm + off_ml[u]);
          po[g][u] = *reinterpret_cast<const float4*>(bo + off_o[u]);
        }
      }
    }
  };
  load_group(0);

  float mstar[S::U], lstar[S::U];
  float4 o[S::U];
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    mstar[u] = -INFINITY;
    lstar[u] = 0.0f;
    o[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
#pragma unroll
  for (int g = 0; g < S::SG; ++g)
    if (g < nv) {
#pragma unroll
      for (int u = 0; u < S::U; ++u) mstar[u] = fmaxf(mstar[u], ml[g][u].x);
    }
  if constexpr (!FITS) {
    for (int s = S::SG; s < nv; ++s) {
#pragma unroll
      for (int u = 0; u < S::U; ++u) mstar[u] = fmaxf(mstar[u], *reinterpret_cast<const float*>(base_ml(s) + off_ml[u]));
    }
  }
  auto add_group = [&](int s0) {
#pragma unroll
    for (int g = 0; g < S::SG; ++g) {
      if (s0 + g < nv) {
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
          const float ms = ml[g][u].x;
          const float w = (ms == -INFINITY) ? 0.0f : exp2f(ms - mstar[u]);
          lstar[u] = fmaf(w, ml[g][u].y, lstar[u]);
          o[u] = fma4(w, po[g][u], o[u]);
        }
      }
    }
  };
  add_group(0);
  if constexpr (!FITS) {
    for (int s0 = S::SG; s0 < nv; s0 += S::SG) {
      load_group(s0);
      add_group(s0);
    }
  }

  const bool faulted = __any(tau_j < 0 || tau_j > pl.B || pos_j < 0) || plen < 0 || plen > pl.p_max;
#pragma unroll
  for (int u = 0; u < S::U; ++u) {
    const int m = m0 + u * S::RPP;
    if (m >= pl.M) continue;
    const int hh = m / pl.twoB, r = m - hh * pl.twoB;
    const size_t orow = (static_cast<size_t>(b) * pl.twoB + r) * pl.Hq + kvh * pl.G + hh;
    const float inv = 1.0f / lstar[u];
    float4 v = make_float4(o[u].x * inv, o[u].y * inv, o[u].z * inv, o[u].w * inv);
    if (faulted) v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    store4<T>(static_cast<T*>(a.out) + orow * HD + col, v);
    if (a.lse && col == 0) a.lse[orow] = faulted ? -INFINITY : (mstar[u] + log2f(lstar[u])) * kLn2;
  }
}

template <typename T, int HD, int SG, int U, bool FITS>
hipError_t launch_shape(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  using S = MergeShape<HD, SG, U>;
  const size_t nchunk = (static_cast<size_t>(pl.M) + S::RWG - 1) / S::RWG;
  const size_t nwg = static_cast<size_t>(pl.NB) * pl.Hkv * nchunk;
  if (nwg > 0x7fffffffu) return hipErrorInvalidValue;
  return launch_with_events(merge_kernel<T, HD, SG, U, FITS>, dim3(static_cast<unsigned>(nwg)), dim3(256), 0, s, ev.start,
                            ev.stop, pl, a);
}

// two splits (the usual case) keep twice the rows in flight per wave in the
// registers that four splits need
template <typename T, int HD>
hipError_t launch_typed(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  if (pl.nsplit <= 2) return launch_shape<T, HD, 2, 4, true>(pl, a, s, ev);
  if (pl.nsplit <= 4) return launch_shape<T, HD, 4, 2, true>(pl, a, s, ev);
  return launch_shape<T, HD, 4, 2, false>(pl, a, s, ev);
}

}  // namespace

hipError_t launch_merge(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  if (pl.dtype == SIMSD_F32) {
    return pl.d == 64 ? launch_typed<float, 64>(pl, a, s, ev) : launch_typed<float, 128>(pl, a, s, ev);
  }
  return pl.d == 64 ? launch_typed<uint16_t, 64>(pl, a, s, ev) : launch_typed<uint16_t, 128>(pl, a, s, ev);
}

}  // namespace simsd
