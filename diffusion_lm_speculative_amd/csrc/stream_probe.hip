// Measurement kernel: the streaming ceiling of the attention kernel's load
// path, with the attention taken out.  It reads a K and a V region laid out
// like the prompt cache ([stream][len][head_dim] bf16 each, one stream per
// (sequence, KV head)) through the same machinery as verify_mfma_kernel: one
// workgroup of 8 waves per stream on a (KV head, sequence) grid (so
// consecutive workgroups land on consecutive XCDs the same way), 64-key tiles
// through a 4-stage LDS ring filled by direct-to-LDS loads of 1 KiB per wave
// instruction, the same split of K and V rows over the waves, one barrier per
// tile, the same staggered tile order (stream i starts at tile i mod T and
// wraps around), the same cache policy (non-temporal loads once K and V
// together reach the last-level cache's size).  Each step only touches one
// LDS word of the tile.  The time of a
// launch over the bench's cache is the most that workload's bytes can stream
// at through this path, which the attention kernel's time is compared with.
#include "mfma_common.hpp"

namespace simsd {
namespace {

constexpr int kProbeKeys = 64;  // keys per tile
constexpr int kProbeStages = 4;
constexpr int kProbeWaves = 8;
constexpr long long kProbeLastLevelCache = 256ll << 20;  // MI355X Infinity Cache bytes

template <int HD, bool NTL>
__global__ __launch_bounds__(kProbeWaves * 64) void stream_probe_kernel(const uint16_t* __restrict__ kc,
                                                                         const uint16_t* __restrict__ vc, int len,
                                                                         uint32_t* __restrict__ sink) {
  constexpr int ROWB = HD * 2;                      // bytes per row
  constexpr int TILEB = kProbeKeys * ROWB;          // one K or V tile
  constexpr int RPI = 1024 / ROWB;                  // rows per 1 KiB load instruction
  constexpr int IPT = kProbeKeys / RPI;             // load instructions per tensor per tile
  constexpr int LPW = 2 * IPT / kProbeWaves;        // loads per wave per tile
  constexpr int VREG = kProbeStages * TILEB;
  static_assert(LPW * kProbeWaves == 2 * IPT, "tile loads split evenly over the waves");
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t stream = static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x;
  const uint16_t* kt0 = kc + stream * static_cast<size_t>(len) * HD;
  const uint16_t* vt0 = vc + stream * static_cast<size_t>(len) * HD;
  const uint32_t sbase = lds_addr(smem);
  const int T = len / kProbeKeys;
  uint32_t goff[LPW];
#pragma unroll
  for (int mm = 0; mm < LPW; ++mm) {
    const int ii = (wave * LPW + mm) % IPT;
    goff[mm] = (ii * RPI + lane / (ROWB / 16)) * ROWB + (lane % (ROWB / 16)) * 16;
  }
  const int rot = T > 0 ? static_cast<int>(stream % static_cast<size_t>(T)) : 0;
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int st = t % kProbeStages;
    const int tr = t + rot < T ? t + rot : t + rot - T;
#pragma unroll
    for (int mm = 0; mm < LPW; ++mm) {
      const int ins = wave * LPW + mm;
      const bool isv = ins >= IPT;
      const int ii = isv ? ins - IPT : ins;
      const uint16_t* base = (isv ? vt0 : kt0) + static_cast<size_t>(tr) * kProbeKeys * HD;
      if constexpr (NTL)
        dma16s_nt(base, goff[mm], sbase + (isv ? VREG : 0) + st * TILEB + ii * 1024);
      else
        dma16s(base, goff[mm], sbase + (isv ? VREG : 0) + st * TILEB + ii * 1024);
    }
  };
  for (int t = 0; t < kProbeStages && t < T; ++t) issue(t);
  uint32_t acc = 0;
  for (int t = 0; t < T; ++t) {
    // tile t landed; the tiles issued after it may still be in flight
    const int later = min(t == 0 ? kProbeStages - 1 : kProbeStages - 2, T - 1 - t);
    if (later >= 3)
      lds_barrier<3 * LPW>();
    else if (later == 2)
      lds_barrier<2 * LPW>();
    else if (later == 1)
      lds_barrier<LPW>();
    else
      lds_barrier<0>();
    if (t > 0 && t + kProbeStages - 1 < T) issue(t + kProbeStages - 1);  // into the stage tile t-1 left
    acc ^= *reinterpret_cast<const uint32_t*>(smem + (t % kProbeStages) * TILEB + (tid * 64) % TILEB);
  }
  wait_counts<0, 15>();
  if (acc == 0x5eed5eedu && tid == 0) sink[0] = acc;  // keeps the reads; not expected to happen
}

template <int HD, bool NTL>
hipError_t launch_probe(const void* k, const void* v, int sx, int sy, int len, void* sink, hipStream_t s,
                        PassEvents ev) {
  auto kern = stream_probe_kernel<HD, NTL>;
  const int lds = 2 * kProbeStages * kProbeKeys * HD * 2;
  const hipError_t e = allow_dynamic_lds<stream_probe_kernel<HD, NTL>>(lds);
  if (e != hipSuccess) return e;
  return launch_with_events(kern, dim3(sx, sy), dim3(kProbeWaves * 64), lds, s, ev.start, ev.stop,
                            static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), len,
                            static_cast<uint32_t*>(sink));
}

// Plain read of the same K and V regions, for comparison: vector loads of 16
// bytes into registers (no LDS), four in flight per thread, a grid-stride
// loop over each region with one 512-thread workgroup per CU, non-temporal
// by the same rule as the attention kernel's tiles.  Its time is how fast
// this memory streams these bytes without the direct-to-LDS path.
constexpr int kReadThreads = 512;
constexpr int kReadGroups = 256;
constexpr int kReadUnroll = 4;

template <bool NTL>
__global__ __launch_bounds__(kReadThreads) void read_probe_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                                  size_t n16, uint32_t* __restrict__ sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  auto ld = [](const uint4* p) -> uint4 {
    if constexpr (NTL) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      return make_uint4(w.x, w.y, w.z, w.w);
    } else {
      return *p;
    }
  };
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  for (int region = 0; region < 2; ++region) {
    const uint4* src = region == 0 ? k : v;
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
      uint4 w[kReadUnroll];
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) w[u] = ld(src + i + u * stride);
#pragma unroll
      for (int u = 0; u < kReadUnroll; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
    }
    for (; i < n16; i += stride) {
      const uint4 w = ld(src + i);
      acc ^= w.x ^ w.y ^ w.z ^ w.w;
    }
  }
  if (acc == 0x5eed5eedu && threadIdx.x == 0) sink[0] = acc;  // keeps the reads; not expected to happen
}

// Measurement kernel: the sustained rate of the bf16 matrix cores.  Every
// wave runs `iters` rounds of four independent 32x32x16 bf16 MFMAs on
// register operands (no memory traffic in the loop), then each lane stores
// one float of its accumulators.  4 waves per workgroup, one per SIMD.
constexpr int kMfmaProbeThreads = 256;
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kMfmaProbeThreads) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x + i) & 15));
    b[i] = static_cast<__bf16>(1e-3f * static_cast<float>(i + 1));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const f32x16 c = c0 + c1 + c2 + c3;
  float t = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) t += c[e];
  sink[static_cast<size_t>(blockIdx.x) * kMfmaProbeThreads + threadIdx.x] = t;
}

}  // namespace
}  // namespace simsd

extern "C" int simsd_mfma_probe(int32_t workgroups, int32_t iters, float* sink, void* stream, void* start_event,
                                void* stop_event) {
  using namespace simsd;
  if (workgroups < 1 || workgroups > 65536 || iters < 1) return SIMSD_ERR_SHAPE;
  if (!sink) return SIMSD_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(sink) % 4) return SIMSD_ERR_ALIGN;
  const hipError_t e = launch_with_events(mfma_probe_kernel, dim3(static_cast<unsigned>(workgroups)),
                                          dim3(kMfmaProbeThreads), 0, static_cast<hipStream_t>(stream),
                                          static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event),
                                          static_cast<int>(iters), sink);
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}

extern "C" int simsd_read_probe(const void* k, const void* v, int64_t bytes, void* sink, void* stream,
                                void* start_event, void* stop_event) {
  using namespace simsd;
  if (bytes < 0 || bytes % 16 != 0) return SIMSD_ERR_SHAPE;
  if (bytes == 0) return SIMSD_OK;
  if (!k || !v || !sink) return SIMSD_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(k) % 16 || reinterpret_cast<uintptr_t>(v) % 16 ||
      reinterpret_cast<uintptr_t>(sink) % 4)
    return SIMSD_ERR_ALIGN;
  // non-temporal loads by the attention kernel's rule (K and V together at least the last-level cache)
  const hipError_t e = launch_with_events(2 * bytes >= kProbeLastLevelCache ? read_probe_kernel<true> : read_probe_kernel<false>,
                                          dim3(kReadGroups), dim3(kReadThreads), 0,
                                          static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
                                          static_cast<hipEvent_t>(stop_event), static_cast<const uint4*>(k),
                                          static_cast<const uint4*>(v), static_cast<size_t>(bytes / 16),
                                          static_cast<uint32_t*>(sink));
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}

extern "C" int simsd_stream_probe(const void* k, const void* v, int32_t streams_x, int32_t streams_y, int32_t len,
                                  int32_t head_dim, void* sink, void* stream, void* start_event, void* stop_event) {
  using namespace simsd;
  if (streams_x < 1 || streams_y < 1 || streams_y > 65535 || len < 0 || len % kProbeKeys != 0 ||
      (head_dim != 64 && head_dim != 128))
    return SIMSD_ERR_SHAPE;
  if (len == 0) return SIMSD_OK;
  if (!k || !v || !sink) return SIMSD_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(k) % 16 || reinterpret_cast<uintptr_t>(v) % 16 ||
      reinterpret_cast<uintptr_t>(sink) % 4)
    return SIMSD_ERR_ALIGN;
  const PassEvents ev{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the attention kernel's rule: non-temporal tile loads when K and V reach the last-level cache's size
  const bool nt = 4ll * streams_x * streams_y * len * head_dim >= kProbeLastLevelCache;
  hipError_t e;
  if (head_dim == 128)
    e = nt ? launch_probe<128, true>(k, v, streams_x, streams_y, len, sink, s, ev)
           : launch_probe<128, false>(k, v, streams_x, streams_y, len, sink, s, ev);
  else
    e = nt ? launch_probe<64, true>(k, v, streams_x, streams_y, len, sink, s, ev)
           : launch_probe<64, false>(k, v, streams_x, streams_y, len, sink, s, ev);
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}
