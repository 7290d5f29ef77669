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
// K/V tile crosses HBM once per split.  The waves form RW row tiles of 16
// rows times KSPLIT key splits of every tile.
//
// MFMA formulation (v_mfma_f32_16x16x32_bf16, wave64).  Scores are computed
// transposed, S^T = K * Q^T, and the output as O^T += V^T * P^T.  In the
// 16x16 accumulator layout lane l holds column l%16, rows 4*(l/16)..+3, so
// with query rows on the N side a lane always holds 4 keys (or 4 head dims)
// of ONE query row: the running max and sum of a row stay in the 4 lanes
// l%16 + 16*g, and the probabilities leave the score accumulator already in
// the B-operand layout of the PV product (keys 4g..4g+3 of two adjacent
// 16-key subtiles form the 8-element k slice of lane group g).
//
// Memory pipeline.  K and V tiles of 64 keys stream from HBM straight into a
// ring of NSTAGE LDS stages with global_load_lds_dwordx4 (no register
// staging): every wave instruction moves 1 KiB of contiguous cache rows.
// Rows are stored as 16-byte granules XOR-swizzled by row, which makes both
// operand reads bank-conflict free: K (A operand of S^T) as ds_read_b128 and
// V^T (A operand of O^T) as two ds_read_b64_tr_b16 transposed reads from the
// row-major tile.  All K stages come first in LDS, then all V stages, so the
// loop (unrolled by NSTAGE) addresses every operand as a loop-invariant
// per-lane register plus an immediate stage offset.
//
// Software pipeline.  Step t waits for tile t+1, refills the stage tile t-1
// left, reads V of tile t, computes the scores of tile t+1 (MFMA) and, while
// those run, the softmax of tile t (VALU), then accumulates P V of tile t.
// One barrier per tile; each wave waits only for its own loads.
#include "simsd_common.hpp"

namespace simsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

#define SIMSD_LDS __attribute__((address_space(3)))
#define SIMSD_GLOBAL __attribute__((address_space(1)))

constexpr int KT = 64;  // keys per tile

template <int HD>
struct Layout {
  static constexpr int ROWB = HD * 2;                // bytes per cache row
  static constexpr int GR = HD / 8;                  // 16-byte granules per row
  static constexpr int TILEB = KT * ROWB;            // one K or V tile
  static constexpr int STAGEB = 2 * TILEB;           // K tile plus V tile
  static constexpr int RPI = 1024 / ROWB;            // rows per 1 KiB load instruction
  static constexpr int IPT = KT / RPI;               // load instructions per tensor per tile
};

template <int V>
struct IC {
  static constexpr int value = V;
};

// Byte offset of granule j of row `row` inside a swizzled tile.
template <int HD>
__device__ __forceinline__ int swz(int row, int j) {
  return row * Layout<HD>::ROWB + ((j ^ (row & (Layout<HD>::GR - 1))) << 4);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(const uint16_t (&v)[8]) {
  u16x8 u = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return __builtin_bit_cast(bf16x8, u);
}

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4 (left at its maximum), lgkmcnt 11:8.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
  static_assert(VM >= 0 && VM <= 63 && LGKM >= 0 && LGKM <= 15, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Workgroup barrier for LDS written by this kernel.  Each wave first waits
// until its own LDS writes (lgkmcnt 0) and all but its VM newest direct-to-LDS
// loads (vmcnt VM) are done; the empty asm keeps the compiler from moving
// memory accesses across the barrier.
template <int VM>
__device__ __forceinline__ void lds_barrier() {
  wait_counts<VM, 0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Two transposed LDS reads (ds_read_b64_tr_b16) at byte addresses a0, a1.
// Written as inline asm: the compiler treats the builtin as possibly aliasing
// the in-flight direct-to-LDS loads and would drain them all (vmcnt 0) before
// it.  The results must not be used before lds_read_wait().
template <int OFF>
__device__ __forceinline__ void tr_read_pair(uint32_t a0, uint32_t a1, bf16x4& lo, bf16x4& hi) {
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%4\n\tds_read_b64_tr_b16 %1, %3 offset:%4"
               : "=&v"(lo), "=&v"(hi)
               : "v"(a0), "v"(a1), "i"(OFF)
               : "memory");
}

// Wait for every outstanding LDS read of this wave; tying the registers makes
// the compiler keep their uses after the wait.
__device__ __forceinline__ void lds_read_wait(bf16x4& a, bf16x4& b, bf16x4& c, bf16x4& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void lds_read_wait(bf16x4& a, bf16x4& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const SIMSD_LDS void*)p));
}

// One direct-to-LDS load: 16 bytes from `src` per lane into LDS at
// m0 + 16*lane (m0 = `lds`, wave-uniform).  Inline asm keeps the load out of
// the compiler's view: otherwise it makes every later LDS access of the wave
// wait for all such loads in flight.  Completion is tracked by hand with
// s_waitcnt vmcnt, and every path drains the loads before the workgroup ends.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

template <int HD, int RW, int KSPLIT, int NSTAGE>
__global__ __launch_bounds__(RW * KSPLIT * 64) void verify_mfma_kernel(Plan pl, VerifyArgs a) {
  using L = Layout<HD>;
  constexpr int NW = RW * KSPLIT;                // waves: RW row waves x KSPLIT key splits
  constexpr int NT = NW * 64;
  constexpr int HALF = HD / 2;
  constexpr int KSTEPS = HD / 32;                // k-steps of S^T = K Q^T
  constexpr int DTILES = HD / 16;                // 16-dim tiles of O^T
  constexpr int NSUB = 4 / KSPLIT;               // 16-key subtiles of a tile per wave
  constexpr int NU = (NSUB + 1) / 2;             // 32-key k-steps of O^T per wave
  constexpr int LPW = 2 * L::IPT / NW;           // direct-to-LDS loads per wave per tile
  constexpr int KREG = 0;                        // K tiles of all stages
  constexpr int VREG = NSTAGE * L::TILEB;        // then V tiles of all stages
  constexpr int XSTR = HD + 4;                   // floats per row of the key-split exchange buffer
  static_assert(KSPLIT == 1 || KSPLIT == 2 || KSPLIT == 4, "key split");
  static_assert(NSTAGE >= 3, "the pipeline keeps two tiles resident");
  static_assert(LPW * NW == 2 * L::IPT, "tile loads must split evenly over waves");
  static_assert((NSTAGE - 2) * LPW <= 63, "too many loads in flight for vmcnt");
  static_assert((NSTAGE - 1) * L::TILEB < 65536, "stage offsets must fit the LDS immediate");
  static_assert((KSPLIT - 1) * RW * 16 * XSTR * 4 <= 2 * NSTAGE * L::TILEB, "exchange buffer fits the ring");
  // The running max moves only when a score exceeds it by more than this
  // (log2 units): probabilities stay below 2^8 and the rescale of the
  // accumulators is skipped for most tiles.
  constexpr float kRescale = 8.0f;

  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int rw = wave % RW;  // row wave: rows rw*16 .. +15 of the row group
  const int ks = wave / RW;  // key split: keys [ks*64/KSPLIT, (ks+1)*64/KSPLIT) of every tile

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

  const int m = rg * pl.rows_wg + rw * 16 + n;
  const bool rok = m < pl.M;
  const int hh = m / twoB, r = m % twoB;
  const size_t rout = (static_cast<size_t>(b) * twoB + r) * pl.Hq + kvh * pl.G + hh;
  const int c0 = s * pl.chunk;
  const bool has_block = (s == 0);

  // ---- the prologue's own loads, issued before the ring loads (a wave's
  //      loads complete in issue order).
  const int plen = a.prompt_len ? a.prompt_len[b] : pl.p_max;
  // every wave keeps tau and the block positions in lanes 0..B-1
  int tau_v = 1, pos_v = 0;
  if (lane < B) {
    tau_v = tau_b[lane];
    if (pos_b) pos_v = pos_b[lane];
  }
  // the table loop below gives this lane frequency tid % HALF on every pass
  const double lane_inv_freq = pl.inv_freq[tid % HALF];
  uint4 qraw[KSTEPS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q_blk) + rout * HD;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i)
      qraw[i] = rok ? *reinterpret_cast<const uint4*>(qp + 32 * i + 8 * g) : make_uint4(0u, 0u, 0u, 0u);
  }
  // raw block rows of the first block tile: K as (first half, second half)
  // granule pairs, V as granules
  constexpr int KITEMS = (KT * (L::GR / 2) + NT - 1) / NT;
  constexpr int VITEMS = (KT * L::GR + NT - 1) / NT;
  const uint16_t* kblk = static_cast<const uint16_t*>(a.k_blk);
  const uint16_t* vblk = static_cast<const uint16_t*>(a.v_blk);
  auto load_block = [&](int bt, uint4 (&kx)[KITEMS], uint4 (&ky)[KITEMS], uint4 (&vv)[VITEMS]) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int i = tid + it * NT;
      const int row = i / (L::GR / 2), j = i % (L::GR / 2), c = bt * KT + row;
      kx[it] = ky[it] = make_uint4(0u, 0u, 0u, 0u);
      if (i < KT * (L::GR / 2) && c < twoB) {
        const uint16_t* kp = kblk + ((static_cast<size_t>(b) * twoB + c) * pl.Hkv + kvh) * HD;
        kx[it] = *reinterpret_cast<const uint4*>(kp + 8 * j);
        ky[it] = *reinterpret_cast<const uint4*>(kp + HALF + 8 * j);
      }
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int i = tid + it * NT;
      const int row = i / L::GR, j = i % L::GR, c = bt * KT + row;
      vv[it] = make_uint4(0u, 0u, 0u, 0u);
      if (i < KT * L::GR && c < twoB)
        vv[it] = *reinterpret_cast<const uint4*>(vblk + ((static_cast<size_t>(b) * twoB + c) * pl.Hkv + kvh) * HD + 8 * j);
    }
  };
  uint4 bkx[KITEMS], bky[KITEMS], bvv[VITEMS];
  if (has_block) load_block(0, bkx, bky, bvv);

  const size_t cache_base = (static_cast<size_t>(b) * pl.Hkv + kvh) * static_cast<size_t>(pl.p_max) * HD;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + cache_base;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + cache_base;

  // ---- direct-to-LDS loads.  Lane `lane` of load instruction `ins` fills
  //      LDS granule position lane%GR of tile row ins*RPI + lane/GR, i.e.
  //      global granule (pos ^ row) of that cache row.  In a tile that ends
  //      past `lim`, rows beyond it re-read key lim-1 (finite values; their
  //      scores are masked).  The last stage is the block's until the first
  //      refill, which follows a barrier.
  int grow[LPW], gcol[LPW];
#pragma unroll
  for (int mm = 0; mm < LPW; ++mm) {
    const int ins = wave * LPW + mm;
    const int ii = ins >= L::IPT ? ins - L::IPT : ins;
    grow[mm] = ii * L::RPI + lane / L::GR;
    gcol[mm] = ((lane % L::GR) ^ (grow[mm] & (L::GR - 1))) * 8;
  }
  auto issue = [&](auto st_c, int t, int lim) {
    constexpr int ST = decltype(st_c)::value;
    const int kb = c0 + t * KT;
    const bool full = kb + KT <= lim;
#pragma unroll
    for (int mm = 0; mm < LPW; ++mm) {
      const int ins = wave * LPW + mm;
      const bool isv = ins >= L::IPT;
      const int ii = isv ? ins - L::IPT : ins;
      const uint16_t* tile = (isv ? vc : kc) + static_cast<size_t>(kb) * HD;
      const uint16_t* src = full ? tile + (grow[mm] * HD + gcol[mm])
                                 : tile + ((min(kb + grow[mm], lim - 1) - kb) * HD + gcol[mm]);
      dma16(src, lds_addr(smem) + (isv ? VREG : KREG) + ST * L::TILEB + ii * 1024);
    }
  };

  // The prologue's loads must be complete before the ring loads go out: the
  // compiler counts only its own loads, so a wait it placed for them later
  // would also wait for every ring load issued in between.  Then the first
  // ring tiles go in flight, before prompt_len is known, assuming the whole
  // cache capacity (always in bounds); the real length masks them.  Every
  // exit below drains them first.
  wait_counts<0, 15>();
  {
    const int c1s = min(c0 + pl.chunk, pl.p_max);
    const int nts = c1s > c0 ? (c1s - c0 + KT - 1) / KT : 0;
    if (nts > 0) issue(IC<0>{}, 0, c1s);
    if (nts > 1) issue(IC<1>{}, 1, c1s);
    if (NSTAGE > 3 && nts > 2) issue(IC<(NSTAGE > 3 ? 2 : 0)>{}, 2, c1s);
  }

  // ---- validation from the lanes' copies of tau and the positions
  if (!pos_b) pos_v = plen + lane;
  const bool bad_tau = lane < B && (tau_v < 1 || tau_v > B);
  const bool bad_pos = lane < B && pos_v < 0;
  int st = (__any(bad_tau) ? SIMSD_ST_TAU_RANGE : 0) | (__any(bad_pos) ? SIMSD_ST_POS_NEG : 0);
  if (plen < 0 || plen > pl.p_max) st |= SIMSD_ST_PROMPT_LEN;
  const bool status_writer = a.status && kvh == 0 && s == 0 && rg == 0 && tid == 0;
  const int c1 = min(c0 + pl.chunk, plen);
  const int ntiles = c1 > c0 ? (c1 - c0 + KT - 1) / KT : 0;
  if (st || (ntiles == 0 && !has_block)) {
    wait_counts<0, 15>();  // drain the ring loads before the workgroup's LDS is released
    if (status_writer) a.status[b] = st;
    if (st && pl.nsplit == 1 && rok && ks == 0) {
      uint16_t* op = static_cast<uint16_t*>(a.out) + rout * HD;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) *reinterpret_cast<uint2*>(op + 16 * dt + 4 * g) = make_uint2(0u, 0u);
      if (a.lse && g == 0) a.lse[rout] = -INFINITY;
    }
    return;
  }

  // ---- RoPE table of the B block positions (after the ring in LDS)
  float2* cs_tab = reinterpret_cast<float2*>(smem + 2 * NSTAGE * L::TILEB);
  static_assert(NT % HALF == 0, "each lane keeps one frequency");
  for (int i0 = 0; i0 < B * HALF; i0 += NT) {  // uniform trip count: the shuffle needs every lane
    const int i = i0 + tid;
    const int k = min(i / HALF, B - 1);
    const int pk = __shfl(pos_v, k);
    if (i < B * HALF) cs_tab[i] = rope_cos_sin(pk, lane_inv_freq);
  }
  lds_barrier<63>();

  // ---- rotated Q operand and block visibility of this lane's row
  bf16x8 qop[KSTEPS];
  uint64_t vis_lo = 0, vis_hi = 0;
  const int tau_row = __shfl(tau_v, r % B);  // stage of this lane's response position
  {
    uint16_t qb[KSTEPS][8];
    if (rok) {
      float qv[KSTEPS][8];
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i) {
        const uint32_t w[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[i][e] = bf16_bits_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))));
      }
      const float4* csr = reinterpret_cast<const float4*>(cs_tab + (r % B) * HALF);
#pragma unroll
      for (int i = 0; i < KSTEPS / 2; ++i) {
        float4 c4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) c4[q4] = csr[(32 * i + 8 * g) / 2 + q4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = (e & 1) ? make_float2(c4[e >> 1].z, c4[e >> 1].w) : make_float2(c4[e >> 1].x, c4[e >> 1].y);
          float xo, yo;
          rope_apply(qv[i][e], qv[i + KSTEPS / 2][e], cs, xo, yo);
          qb[i][e] = f32_to_bf16_bits(xo);
          qb[i + KSTEPS / 2][e] = f32_to_bf16_bits(yo);
        }
      }
      uint64_t dbits, mbits;
      mask_row_bits_at([&](int j) { return j == r % B ? tau_row : __builtin_amdgcn_readlane(tau_v, j); }, B, r,
                       pl.mask_mode, dbits, mbits);
      if (B >= 64) {
        vis_lo = dbits;
        vis_hi = mbits;
      } else {
        vis_lo = dbits | (mbits << B);
        vis_hi = mbits >> (64 - B);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KSTEPS; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[i][e] = 0;
    }
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) qop[i] = bits_to_bf16x8(qb[i]);
  }

  // ---- loop-invariant LDS offsets of this lane's operand reads
  int kofs[NSUB][KSTEPS];  // K: row 16*t4 + n, granule 4*kk + g
#pragma unroll
  for (int i = 0; i < NSUB; ++i)
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) kofs[i][kk] = KREG + swz<HD>(16 * (ks * NSUB + i) + n, 4 * kk + g);
  // V^T: lane (g, r, c) = (lane/16, (lane%16)/4, lane%4) reads the 8 bytes at
  // row 32u + 4g + r (then + 16), columns 16dt + 4c.., and the transposed read
  // hands lane n the column 16dt + n of those 4 rows.
  uint32_t vadr[DTILES][NU][2];
  {
    const uint32_t vbase = lds_addr(smem) + VREG;
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int vc4 = lane & 3;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        const int r0 = 32 * ((ks * NSUB) / 2 + uu) + vr;
        const int gran = 2 * dt + (vc4 >> 1);
        vadr[dt][uu][0] = vbase + swz<HD>(r0, gran) + (vc4 & 1) * 8;
        vadr[dt][uu][1] = vbase + swz<HD>(r0 + 16, gran) + (vc4 & 1) * 8;
      }
  }

  // ---- online-softmax state of this wave's share of the keys
  float mrun = -INFINITY, lpart = 0.0f;
  f32x4 acc[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // S^T of this wave's keys of the tile in stage ST.
  auto scores = [&](auto st_c, f32x4 (&sacc)[NSUB]) {
    constexpr int ST = decltype(st_c)::value;
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      bf16x8 kop[KSTEPS];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        kop[kk] = *reinterpret_cast<const bf16x8*>(smem + ST * L::TILEB + kofs[i][kk]);
      f32x4 sa = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) sa = mfma(kop[kk], qop[kk], sa);
      sacc[i] = sa;
    }
  };

  // V^T reads of the tile in stage ST (they complete during the softmax).
  auto vread = [&](auto st_c, bf16x4 (&vlo)[DTILES][NU], bf16x4 (&vhi)[DTILES][NU]) {
    constexpr int ST = decltype(st_c)::value;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) tr_read_pair<ST * L::TILEB>(vadr[dt][uu][0], vadr[dt][uu][1], vlo[dt][uu], vhi[dt][uu]);
  };

  // Softmax of the scores and O^T += V^T P^T.  MODE 0: every key visible;
  // 1: keys kbase+k < klimit; 2: block column kbase+k per the tau bits.
  auto finish = [&](auto mode_c, const f32x4 (&sacc)[NSUB], bf16x4 (&vlo)[DTILES][NU],
                    bf16x4 (&vhi)[DTILES][NU], int kbase, int klimit) {
    constexpr int MODE = decltype(mode_c)::value;
    float sv[NSUB][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = 16 * (ks * NSUB + i) + 4 * g + j;
        bool vis = true;
        if (MODE == 1) vis = kbase + k < klimit;
        if (MODE == 2) {
          const int c = kbase + k;
          vis = c < 64 ? ((vis_lo >> c) & 1ull) : ((vis_hi >> (c - 64)) & 1ull);
        }
        const float x = vis ? sacc[i][j] * pl.scale_log2 : -INFINITY;
        sv[i][j] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (__any(tmax > mrun + kRescale)) {
      const float mnew = fmaxf(mrun, tmax);
      const float alpha = (mnew == mrun) ? 1.0f : __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      lpart *= alpha;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) acc[dt] *= alpha;
    }
    const float muse = (mrun == -INFINITY) ? 0.0f : mrun;
    float pv[NSUB][4];
    float lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < NSUB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pv[i][j] = __builtin_amdgcn_exp2f(sv[i][j] - muse);
        lsum += pv[i][j];
      }
    lpart += lsum;
    // P^T operand of k-step u: keys 4g..4g+3 of subtile 2u, then of 2u+1;
    // subtiles of other waves contribute zeros.
    bf16x8 pop[NU];
#pragma unroll
    for (int uu = 0; uu < NU; ++uu) {
      const int u = (ks * NSUB) / 2 + uu;
      __bf16 pb[8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int i = 2 * u + h2 - ks * NSUB;
        const int ic = i < 0 ? 0 : (i >= NSUB ? NSUB - 1 : i);
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[4 * h2 + j] = static_cast<__bf16>((i >= 0 && i < NSUB) ? pv[ic][j] : 0.0f);
      }
      pop[uu] = bf16x8{pb[0], pb[1], pb[2], pb[3], pb[4], pb[5], pb[6], pb[7]};
    }
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      if (NU == 2)
        lds_read_wait(vlo[dt][0], vhi[dt][0], vlo[dt][NU - 1], vhi[dt][NU - 1]);
      else
        lds_read_wait(vlo[dt][0], vhi[dt][0]);
    }
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        const bf16x4 lo = vlo[dt][uu], hi = vhi[dt][uu];
        const bf16x8 vop = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[dt] = mfma(vop, pop[uu], acc[dt]);
      }
    }
  };

  // ---- block keys (split 0): rotated K and V of this KV head in the last
  //      stage, one 64-row tile at a time (a second tile only when B > 32)
  auto block_tile = [&](int bt) {
    unsigned char* Kb = smem + KREG + (NSTAGE - 1) * L::TILEB;
    unsigned char* Vb = smem + VREG + (NSTAGE - 1) * L::TILEB;
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int i = tid + it * NT;
      if (i >= KT * (L::GR / 2)) continue;
      const int row = i / (L::GR / 2), j = i % (L::GR / 2), c = bt * KT + row;
      const uint32_t wx[4] = {bkx[it].x, bkx[it].y, bkx[it].z, bkx[it].w};
      const uint32_t wy[4] = {bky[it].x, bky[it].y, bky[it].z, bky[it].w};
      uint16_t lo8[8], hi8[8];
      const float4* csr = reinterpret_cast<const float4*>(cs_tab + (c % B) * HALF + 8 * j);
      float4 c4[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) c4[q4] = csr[q4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = (e & 1) ? make_float2(c4[e >> 1].z, c4[e >> 1].w) : make_float2(c4[e >> 1].x, c4[e >> 1].y);
        float xo, yo;
        rope_apply(bf16_bits_to_f32(static_cast<uint16_t>(wx[e >> 1] >> (16 * (e & 1)))),
                   bf16_bits_to_f32(static_cast<uint16_t>(wy[e >> 1] >> (16 * (e & 1)))), cs, xo, yo);
        lo8[e] = f32_to_bf16_bits(xo);
        hi8[e] = f32_to_bf16_bits(yo);
      }
      *reinterpret_cast<u16x8*>(Kb + swz<HD>(row, j)) = u16x8{lo8[0], lo8[1], lo8[2], lo8[3], lo8[4], lo8[5], lo8[6], lo8[7]};
      *reinterpret_cast<u16x8*>(Kb + swz<HD>(row, j + L::GR / 2)) =
          u16x8{hi8[0], hi8[1], hi8[2], hi8[3], hi8[4], hi8[5], hi8[6], hi8[7]};
    }
#pragma unroll
    for (int it = 0; it < VITEMS; ++it) {
      const int i = tid + it * NT;
      if (i >= KT * L::GR) continue;
      const int row = i / L::GR, j = i % L::GR;
      *reinterpret_cast<uint4*>(Vb + swz<HD>(row, j)) = bvv[it];
    }
    lds_barrier<63>();
    f32x4 sb[NSUB];
    bf16x4 vlo[DTILES][NU], vhi[DTILES][NU];
    vread(IC<NSTAGE - 1>{}, vlo, vhi);
    scores(IC<NSTAGE - 1>{}, sb);
    finish(IC<2>{}, sb, vlo, vhi, bt * KT, 0);
    lds_barrier<63>();
  };
  if (has_block) {
    block_tile(0);
    if (twoB > KT) {  // B > 32: the loads of the second tile wait for the ring loads too (rare shape)
      load_block(1, bkx, bky, bvv);
      block_tile(1);
    }
  }

  // ---- prompt keys [c0, c1): software-pipelined over the ring
  f32x4 scur[NSUB];
  if (ntiles > 0) {
    // tile 0 landed; the loads of tiles 1..NSTAGE-2 may still be in flight
    if (ntiles - 1 >= NSTAGE - 2)
      lds_barrier<(NSTAGE - 2) * LPW>();
    else
      lds_barrier<0>();
    scores(IC<0>{}, scur);
  }
  auto step = [&](auto k_c, int t) {
    constexpr int K = decltype(k_c)::value;  // stage of tile t (t % NSTAGE)
    if (t + 1 < ntiles) {
      // tile t+1 must have landed: only the loads of tiles t+2..t+NSTAGE-2 may
      // still be in flight; the barrier also frees the stage of tile t-1
      if (t + NSTAGE - 2 < ntiles)
        lds_barrier<(NSTAGE - 3) * LPW>();
      else
        lds_barrier<0>();
      if (t + NSTAGE - 1 < ntiles) issue(IC<(K + NSTAGE - 1) % NSTAGE>{}, t + NSTAGE - 1, c1);
    }
    bf16x4 vlo[DTILES][NU], vhi[DTILES][NU];
    vread(IC<K>{}, vlo, vhi);
    f32x4 snext[NSUB];
    if (t + 1 < ntiles) scores(IC<(K + 1) % NSTAGE>{}, snext);
    const int kbase = c0 + t * KT;
    if (kbase + KT <= c1)
      finish(IC<0>{}, scur, vlo, vhi, kbase, c1);
    else
      finish(IC<1>{}, scur, vlo, vhi, kbase, c1);
#pragma unroll
    for (int i = 0; i < NSUB; ++i) scur[i] = snext[i];
  };
  for (int t0 = 0; t0 < ntiles; t0 += NSTAGE) {
    step(IC<0>{}, t0);
    if (t0 + 1 < ntiles) step(IC<1>{}, t0 + 1);
    if (t0 + 2 < ntiles) step(IC<2>{}, t0 + 2);
    if (NSTAGE > 3 && t0 + 3 < ntiles) step(IC<(NSTAGE > 3 ? 3 : 0)>{}, t0 + 3);
  }

  // ---- combine the key splits of each row (through the drained ring)
  wait_counts<0, 15>();  // no ring load may land after the workgroup ends
  if (status_writer) a.status[b] = 0;
  float l = lpart;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (KSPLIT > 1) {
    float* xb = reinterpret_cast<float*>(smem);
    lds_barrier<0>();  // every wave is done reading the ring
    if (ks > 0) {
      float* xr = xb + (((ks - 1) * RW + rw) * 16 + n) * XSTR;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt)
        *reinterpret_cast<float4*>(xr + 16 * dt + 4 * g) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
      if (g == 0) {
        xr[HD] = mrun;
        xr[HD + 1] = l;
      }
    }
    lds_barrier<0>();
    if (ks > 0) return;
#pragma unroll
    for (int k2 = 1; k2 < KSPLIT; ++k2) {
      const float* xr = xb + (((k2 - 1) * RW + rw) * 16 + n) * XSTR;
      const float m2 = xr[HD], l2 = xr[HD + 1];
      const float mnew = fmaxf(mrun, m2);
      const float a1 = (mrun == mnew) ? 1.0f : exp2f(mrun - mnew);
      const float a2 = (m2 == mnew) ? 1.0f : exp2f(m2 - mnew);
      l = l * a1 + l2 * a2;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const float4 o2 = *reinterpret_cast<const float4*>(xr + 16 * dt + 4 * g);
        acc[dt] = acc[dt] * a1 + f32x4{o2.x, o2.y, o2.z, o2.w} * a2;
      }
      mrun = mnew;
    }
  }

  // ---- epilogue (key-split 0 waves)
  if (!rok) return;
  if (pl.nsplit == 1) {
    const float inv = 1.0f / l;
    uint16_t* op = static_cast<uint16_t*>(a.out) + rout * HD;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const f32x4 v = acc[dt];
      const uint32_t w0 = f32_to_bf16_bits(v[0] * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1] * inv)) << 16);
      const uint32_t w1 = f32_to_bf16_bits(v[2] * inv) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3] * inv)) << 16);
      *reinterpret_cast<uint2*>(op + 16 * dt + 4 * g) = make_uint2(w0, w1);
    }
    if (a.lse && g == 0) a.lse[rout] = (mrun + log2f(l)) * kLn2;
  } else {
    const size_t slot = (static_cast<size_t>(b) * pl.Hkv + kvh) * pl.nsplit + s;
    float* po = a.part_o + (slot * pl.M + m) * HD;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const f32x4 v = acc[dt];
      *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g == 0) {
      a.part_ml[(slot * pl.M + m) * 2 + 0] = mrun;
      a.part_ml[(slot * pl.M + m) * 2 + 1] = l;
    }
  }
}

template <int HD, int RW, int KSPLIT, int NSTAGE>
hipError_t launch_cfg(const Plan& pl, const VerifyArgs& a, hipStream_t s) {
  auto kern = verify_mfma_kernel<HD, RW, KSPLIT, NSTAGE>;
  const size_t lds = mfma_lds_bytes(HD, NSTAGE, pl.B);
  static int attr_set = 0;  // largest dynamic LDS size already allowed for this instantiation
  if (static_cast<int>(lds) > attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set = static_cast<int>(lds);
  }
  const unsigned grid = static_cast<unsigned>(pl.nsplit) * pl.nrg * pl.NB * pl.Hkv;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(RW * KSPLIT * 64), lds, s, pl, a);
  return hipGetLastError();
}

template <int HD, int NSTAGE>
hipError_t launch_stages(const Plan& pl, const VerifyArgs& a, hipStream_t s) {
  switch (pl.rows_wg / 16) {
    case 1: return launch_cfg<HD, 1, 4, NSTAGE>(pl, a, s);
    case 2: return launch_cfg<HD, 2, 4, NSTAGE>(pl, a, s);
    case 4: return launch_cfg<HD, 4, 2, NSTAGE>(pl, a, s);
    default: return launch_cfg<HD, 8, 1, NSTAGE>(pl, a, s);
  }
}

}  // namespace

// Dynamic LDS of one workgroup: the tile ring plus the RoPE table.
size_t mfma_lds_bytes(int hd, int nstage, int B) {
  const size_t ring = static_cast<size_t>(nstage) * 2 * KT * hd * 2;
  return ring + static_cast<size_t>(B) * (hd / 2) * sizeof(float2);
}

hipError_t launch_verify_mfma(const Plan& pl, const VerifyArgs& a, hipStream_t s) {
  if (pl.d == 64) return launch_stages<64, 4>(pl, a, s);
  return pl.nstage == 4 ? launch_stages<128, 4>(pl, a, s) : launch_stages<128, 3>(pl, a, s);
}

}  // namespace simsd
