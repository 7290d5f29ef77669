// Debug exports: the tau mask rows and the RoPE-copy rotation of the block
// rows, produced by the same device functions the attention kernels use
// (mask_row_bits_wave / mask_row_bits, rope_cos_sin, rope_apply), so tests can compare them with
// the oracle bit for bit.
#include "simsd_common.hpp"

namespace simsd {
namespace {

// One workgroup of 128 threads per sequence, thread r = block row r.  The
// rows come from the wave-ballot form the MFMA kernel uses; the per-thread
// form (the VALU kernel's) must agree, else the row reads all ones in both
// words, which no valid mask has.
__global__ void debug_mask_kernel(const int32_t* tau, int B, int mode, uint64_t* bits) {
  const int b = blockIdx.x;
  const int r = threadIdx.x;
  const int lane = r & 63;
  if (B < 1 || B > 64) return;  // uniform over the workgroup
  const int32_t* tau_b = tau + static_cast<size_t>(b) * B;
  const int tau_lane = lane < B ? tau_b[lane] : 0;
  uint64_t d, m, d1, m1;
  mask_row_bits_wave(tau_lane, lane, B, r % (2 * B), mode, d, m);
  if (r >= 2 * B) return;
  mask_row_bits(tau_b, B, r, mode, d1, m1);
  if (d != d1 || m != m1) d = m = ~0ull;
  uint64_t* o = bits + (static_cast<size_t>(b) * 2 * B + r) * 2;
  o[0] = d;
  o[1] = m;
}

// One workgroup per (b, block row c).  Q rows are rotated for every query
// head, K rows for every KV head; values are rounded to the storage dtype the
// way the kernels round their operands (bf16 round-to-nearest-even).
template <typename T>
__global__ void debug_rope_kernel(Plan pl, const T* q_blk, const T* k_blk, const int32_t* prompt_len,
                                  const int32_t* pos_d, T* q_rot, T* k_rot) {
  const int b = blockIdx.x / pl.twoB;
  const int c = blockIdx.x % pl.twoB;
  const int half = pl.d / 2;
  const int plen = prompt_len ? prompt_len[b] : pl.p_max;
  const int32_t* pos_b = pos_d ? pos_d + static_cast<size_t>(b) * pl.B : nullptr;
  const int64_t pos = block_row_pos(pos_b, plen, c, pl.B, pl.rope_seq != 0);
  const size_t qrow = (static_cast<size_t>(b) * pl.twoB + c) * pl.Hq;
  const size_t krow = (static_cast<size_t>(b) * pl.twoB + c) * pl.Hkv;
  for (int i = threadIdx.x; i < (pl.Hq + pl.Hkv) * half; i += blockDim.x) {
    const int h = i / half, f = i % half;
    const float2 cs = rope_cos_sin(pos, rope_inv_freq(f, pl.d, pl.log2_base));
    const T* src;
    T* dst;
    if (h < pl.Hq) {
      src = q_blk + (qrow + h) * pl.d;
      dst = q_rot + (qrow + h) * pl.d;
    } else {
      src = k_blk + (krow + h - pl.Hq) * pl.d;
      dst = k_rot + (krow + h - pl.Hq) * pl.d;
    }
    float xo, yo;
    rope_apply(Elem<T>::load(src, f), Elem<T>::load(src, f + half), cs, xo, yo);
    Elem<T>::store(dst, f, xo);
    Elem<T>::store(dst, f + half, yo);
  }
}

}  // namespace

hipError_t launch_debug_mask(const int32_t* tau, int NB, int B, int mode, uint64_t* bits, hipStream_t s) {
  hipLaunchKernelGGL(debug_mask_kernel, dim3(NB), dim3(128), 0, s, tau, B, mode, bits);
  return hipGetLastError();
}

hipError_t launch_debug_rope(const Plan& pl, const void* q_blk, const void* k_blk, const int32_t* prompt_len,
                             const int32_t* pos_d, void* q_rot, void* k_rot, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(pl.NB) * pl.twoB;
  if (pl.dtype == SIMSD_F32) {
    hipLaunchKernelGGL(debug_rope_kernel<float>, dim3(grid), dim3(256), 0, s, pl,
                       static_cast<const float*>(q_blk), static_cast<const float*>(k_blk), prompt_len, pos_d,
                       static_cast<float*>(q_rot), static_cast<float*>(k_rot));
  } else {
    hipLaunchKernelGGL(debug_rope_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, pl,
                       static_cast<const uint16_t*>(q_blk), static_cast<const uint16_t*>(k_blk), prompt_len,
                       pos_d, static_cast<uint16_t*>(q_rot), static_cast<uint16_t*>(k_rot));
  }
  return hipGetLastError();
}

}  // namespace simsd
