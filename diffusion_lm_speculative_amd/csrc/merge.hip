// Combine the split-KV partials of the verification attention into the
// final rows.  Each split s of a row holds an unnormalised sum o_s, its
// running max m_s (log2 units) and sum l_s; the softmax over the union of
// the splits' keys is
//   m* = max_s m_s,  l* = sum_s 2^(m_s - m*) l_s,
//   out = (sum_s 2^(m_s - m*) o_s) / l*,  lse = (m* + log2 l*) * ln 2.
// One wave per row; a faulted sequence gets zero rows and lse = -inf.
#include "simsd_common.hpp"

namespace simsd {
namespace {

template <typename T, int HD>
__global__ __launch_bounds__(256) void merge_kernel(Plan pl, VerifyArgs a) {
  constexpr int PER = HD / 64;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const size_t row = static_cast<size_t>(blockIdx.x) * 4 + wave;  // over NB * Hkv * M
  const size_t nrows = static_cast<size_t>(pl.NB) * pl.Hkv * pl.M;
  if (row >= nrows) return;
  const int m = static_cast<int>(row % pl.M);
  const int kvh = static_cast<int>((row / pl.M) % pl.Hkv);
  const int b = static_cast<int>(row / (static_cast<size_t>(pl.M) * pl.Hkv));
  const int hh = m / pl.twoB, r = m % pl.twoB;
  const size_t orow = (static_cast<size_t>(b) * pl.twoB + r) * pl.Hq + kvh * pl.G + hh;
  T* op = static_cast<T*>(a.out) + orow * HD;

  const int32_t* tau_b = a.tau + static_cast<size_t>(b) * pl.B;
  const int32_t* pos_b = a.pos_d ? a.pos_d + static_cast<size_t>(b) * pl.B : nullptr;
  const int plen = a.prompt_len ? a.prompt_len[b] : pl.p_max;
  // the sequence's fault flags, with lane j checking position j (B <= 64):
  // one round of loads instead of B dependent ones
  bool bad = false;
  if (lane < pl.B) {
    const int t = tau_b[lane];
    bad = t < 0 || t > pl.B || (pos_b && pos_b[lane] < 0);
  }
  if (__any(bad) || plen < 0 || plen > pl.p_max) {
#pragma unroll
    for (int e = 0; e < PER; ++e) Elem<T>::store(op, lane + 64 * e, 0.0f);
    if (a.lse && lane == 0) a.lse[orow] = -INFINITY;
    return;
  }
  const int nv = valid_splits(plen, pl.chunk, pl.nsplit);
  const size_t slot0 = (static_cast<size_t>(b) * pl.Hkv + kvh) * pl.nsplit;
  float mstar = -INFINITY;
  for (int s = 0; s < nv; ++s) mstar = fmaxf(mstar, a.part_ml[((slot0 + s) * pl.M + m) * 2]);
  float lstar = 0.0f;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.0f;
  for (int s = 0; s < nv; ++s) {
    const size_t pr = (slot0 + s) * pl.M + m;
    const float ms = a.part_ml[pr * 2];
    const float w = (ms == -INFINITY) ? 0.0f : exp2f(ms - mstar);
    lstar = fmaf(w, a.part_ml[pr * 2 + 1], lstar);
    const float* po = a.part_o + pr * HD;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = fmaf(w, po[lane + 64 * e], o[e]);
  }
  const float inv = 1.0f / lstar;
#pragma unroll
  for (int e = 0; e < PER; ++e) Elem<T>::store(op, lane + 64 * e, o[e] * inv);
  if (a.lse && lane == 0) a.lse[orow] = (mstar + log2f(lstar)) * kLn2;
}

template <typename T, int HD>
hipError_t launch_typed(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  const size_t nrows = static_cast<size_t>(pl.NB) * pl.Hkv * pl.M;
  const unsigned grid = static_cast<unsigned>((nrows + 3) / 4);
  return launch_with_events(merge_kernel<T, HD>, dim3(grid), dim3(256), 0, s, ev.start, ev.stop, pl, a);
}

}  // namespace

hipError_t launch_merge(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  if (pl.dtype == SIMSD_F32) {
    return pl.d == 64 ? launch_typed<float, 64>(pl, a, s, ev) : launch_typed<float, 128>(pl, a, s, ev);
  }
  return pl.d == 64 ? launch_typed<uint16_t, 64>(pl, a, s, ev) : launch_typed<uint16_t, 128>(pl, a, s, ev);
}

}  // namespace simsd
