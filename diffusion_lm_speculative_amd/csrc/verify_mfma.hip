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
// Rows are stored as 16-byte granules XOR-swizzled by row (a different
// swizzle for K and V tiles, each matched to its read), which keeps both
// operand reads free of bank conflicts: K (A operand of S^T) as ds_read_b128
// and V^T (A operand of O^T) as two ds_read_b64_tr_b16 transposed reads from
// the row-major tile.  All K stages come first in LDS, then all V stages, so the
// loop (unrolled by NSTAGE) addresses every operand as a loop-invariant
// per-lane register plus an immediate stage offset.
//
// Pipeline.  Step t waits for tile t, refills the stage tile t-1 left (so
// three tiles are in flight behind the one in use), reads K and V of tile t,
// computes its scores (MFMA), softmax (VALU) and P V (MFMA).  One barrier per
// tile; each wave waits only for its own loads.
#include "mfma_common.hpp"

namespace simsd {
namespace {

constexpr int KT = 64;  // keys per tile
constexpr int kLdsMax = 163840;  // LDS bytes of one CU, the most a workgroup may use

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

// V tiles: the transposed reads take both granules 2p, 2p+1 of a row in one
// go, so with the K tiles' swizzle (j ^ row) rows r and r^1 would meet in
// the same banks.  V rows swizzle by an even rotation of the granule pairs
// instead: row r XORs j with ((r & 7) << 1) | ((r >> 3) & 1), so the pairs of
// 8 consecutive rows sit in 8 distinct pair slots.  (Head dim 64 keeps the K
// swizzle: its 128-byte rows put two rows side by side in the banks.)
template <int HD>
__device__ __forceinline__ int vsw(int row) {
  if constexpr (HD == 128) return ((row & 7) << 1) | ((row >> 3) & 1);
  return row & (Layout<HD>::GR - 1);
}
template <int HD>
__device__ __forceinline__ int swz_v(int row, int j) {
  return row * Layout<HD>::ROWB + ((j ^ vsw<HD>(row)) << 4);
}

// Two wave-uniform 4-byte loads through the scalar cache, waited for here.
// (The compiler cannot prove such loads scalar once the direct-to-LDS loads,
// which it sees as arbitrary memory writes, have been issued; a vector load
// would make it wait for every load in flight.)
__device__ __forceinline__ void sload2(const int32_t* p0, const int32_t* p1, int& v0, int& v1) {
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v0), "=&s"(v1)
               : "s"(p0), "s"(p1)
               : "memory");
}

// One direct-to-LDS load of 4 bytes per lane into LDS at m0 + 4*lane.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) | (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Rotate the 8 pairs (x[e], y[e]) held as bf16 in wx / wy with the table
// entries c4 (entry e: cos, sin at c4[e/2].xy or .zw) and round back to bf16.
__device__ __forceinline__ void rotate8(const uint32_t (&wx)[4], const uint32_t (&wy)[4], const float4 (&c4)[4],
                                        uint32_t (&ox)[4], uint32_t (&oy)[4]) {
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float x0, y0, x1, y1;
    rope_apply(bf16_lo(wx[e2]), bf16_lo(wy[e2]), make_float2(c4[e2].x, c4[e2].y), x0, y0);
    rope_apply(bf16_hi(wx[e2]), bf16_hi(wy[e2]), make_float2(c4[e2].z, c4[e2].w), x1, y1);
    ox[e2] = pack_bf16x2(x0, x1);
    oy[e2] = pack_bf16x2(y0, y1);
  }
}

// LDS layout of one workgroup (bytes): NSTAGE K tiles, NSTAGE V tiles, the
// stage labels and positions (2 x 256), the query rows when they have their
// own region, the block K and V rows when they have their own region
// (Plan::blk_rows each, a run-time size), then the RoPE table of the block
// positions.
template <int HD, int NSTAGE, bool QSEP>
struct Smem {
  static constexpr int KREG = 0;
  static constexpr int VREG = NSTAGE * Layout<HD>::TILEB;
  static constexpr int TPREG = 2 * NSTAGE * Layout<HD>::TILEB;
  static constexpr int QREG = TPREG + 512;
  // start of the block rows' region (the table follows it)
  static constexpr int blk(int rows_wg) { return QREG + (QSEP ? rows_wg * Layout<HD>::ROWB : 0); }
  // Byte offset of query row lr (0 <= lr < rows per workgroup) of the staging area.
  // Without a region of their own the rows borrow ring stages from the last
  // one down, 2*KT rows per stage: its K tile, then its V tile.
  static constexpr int qrow(int lr) {
    return QSEP ? QREG + lr * Layout<HD>::ROWB
                : ((lr % (2 * KT)) < KT ? KREG : VREG - KT * Layout<HD>::ROWB) +
                      (NSTAGE - 1 - lr / (2 * KT)) * Layout<HD>::TILEB + (lr % (2 * KT)) * Layout<HD>::ROWB;
  }
};

template <int HD, int RW, int KSPLIT, int NSTAGE, bool QSEP, int ROWT, bool BSEP, bool KVNT>
__global__ __launch_bounds__(RW * KSPLIT * 64) void verify_mfma_kernel(Plan pl, VerifyArgs a) {
  using L = Layout<HD>;
  using S = Smem<HD, NSTAGE, QSEP>;
  constexpr int NW = RW * KSPLIT;                // waves: RW row waves x KSPLIT key splits
  constexpr int ROWS = RW * ROWT * 16;           // rows of a workgroup: ROWT 16-row tiles per row wave
  constexpr int NT = NW * 64;
  constexpr int HALF = HD / 2;
  constexpr int KSTEPS = HD / 32;                // k-steps of S^T = K Q^T
  constexpr int DTILES = HD / 16;                // 16-dim tiles of O^T
  constexpr int NSUB = 4 / KSPLIT;               // 16-key subtiles of a tile per wave
  constexpr int NU = (NSUB + 1) / 2;             // 32-key k-steps of O^T per wave
  constexpr int LPW = 2 * L::IPT / NW;           // direct-to-LDS loads per wave per tile
  constexpr int KREG = S::KREG;
  constexpr int VREG = S::VREG;
  constexpr int BKREG = S::blk(ROWS);
  constexpr int QST = (ROWS + 2 * KT - 1) / (2 * KT);  // ring stages the query rows borrow (without QSEP)
  constexpr int NPRO = QSEP ? NSTAGE : NSTAGE - QST;  // ring tiles issued before the query rows are read
  constexpr int QI = ROWS / L::RPI;              // 1 KiB loads of the workgroup's query rows
  constexpr int XSTR = HD + 4;                   // floats per row of the key-split exchange buffer
  static_assert(KSPLIT == 1 || KSPLIT == 2 || KSPLIT == 4, "key split");
  static_assert(NSTAGE == 3 || NSTAGE == 4, "the pipeline keeps two tiles resident; at most 4 stages");
  static_assert(LPW * NW == 2 * L::IPT, "tile loads must split evenly over waves");
  static_assert(NSTAGE * LPW <= 63, "too many loads in flight for vmcnt");
  static_assert((NSTAGE - 1) * L::TILEB < 65536, "stage offsets must fit the LDS immediate");
  static_assert(QSEP || QST < NSTAGE, "query rows must leave a ring stage to the prologue");
  static_assert(ROWT == 1 || ROWT == 2, "row tiles per wave");
  static_assert(KSPLIT > 1 || (!BSEP && ROWT == 2 && NSUB == 4), "one key split: 32 rows a wave, block keys in the ring");
  static_assert((KSPLIT - 1) * ROWS * XSTR * 4 <= 2 * NSTAGE * L::TILEB, "exchange buffer fits the ring");
  static_assert(NT % HALF == 0, "each lane keeps one RoPE frequency");
  // Probabilities are taken relative to a per-row reference set at the
  // row's first tile with a visible key.  It is raised (and the
  // accumulators rescaled) only when a later score passes it by more than
  // this many log2 units, so probabilities stay below 2^kRaise and the
  // rescale is rare.
  constexpr float kRaise = 16.0f;

  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int rw = wave % RW;  // row wave: rows (rw*ROWT + rt)*16 .. +15 of the row group, rt < ROWT
  const int ks = wave / RW;  // key split: keys [ks*64/KSPLIT, (ks+1)*64/KSPLIT) of every tile

  // Workgroup -> (KV head, sequence and row group, split) straight from the
  // 3-D grid.  The hardware hands consecutive workgroups (x fastest) to
  // consecutive XCDs, so with Hkv a multiple of 8 XCD j streams KV head j of
  // every sequence and every split: the same work on every XCD whatever the
  // prompt lengths.  The row groups of one K/V stream share an XCD and run
  // side by side, the later ones finding its tiles in that XCD's L2, and
  // the splits go out in order, so the ragged last splits come last.
  const int kvh = blockIdx.x;
  int b = blockIdx.y, rg = 0;
  int s = blockIdx.z;
  if (pl.nrg > 1) {
    rg = b % pl.nrg;
    b /= pl.nrg;
  }
  // Longest work first (pl.lpt: more workgroups than the CUs hold at once).
  // The workgroups of one KV head go out in (split, sequence) order; each
  // takes the (sequence, split) item whose rank by key count (longest first,
  // ties in dispatch order) is its own position in that order, so the long
  // items start first and the short ones fill in behind them.  Every
  // workgroup computes the same ranking from the prompt lengths, in the LDS
  // of the tile ring before any tile is issued.  The row groups of an item
  // keep their adjacent positions.
  if (pl.lpt) {
    const int items = pl.NB * pl.nsplit;
    int* lk = reinterpret_cast<int*>(smem);  // keys of each item, then the pick
    for (int t = tid; t < items; t += NT) {
      const int bt = t % pl.NB, st = t / pl.NB;
      const int plen_t = a.prompt_len ? a.prompt_len[bt] : pl.p_max;
      lk[t] = min(max(plen_t - st * pl.chunk, 0), pl.chunk);
    }
    __syncthreads();
    const int mine = s * pl.NB + b;
    for (int t = tid; t < items; t += NT) {
      const int kt = lk[t];
      int r = 0;
      for (int u = 0; u < items; ++u) {
        const int ku = lk[u];
        r += (ku > kt || (ku == kt && u < t)) ? 1 : 0;
      }
      if (r == mine) lk[items] = t;
    }
    __syncthreads();
    const int item = lk[items];
    __syncthreads();  // every wave holds its item before the ring is filled
    b = item % pl.NB;
    s = item / pl.NB;
  }

  const int B = pl.B, twoB = pl.twoB;
  const int32_t* tau_b = a.tau + static_cast<size_t>(b) * B;
  const int32_t* pos_b = a.pos_d ? a.pos_d + static_cast<size_t>(b) * B : nullptr;

  // this lane's query row in row tile rt of the wave (m < M: a real row;
  // r: its block row; its output row index), recomputed where needed rather
  // than held in registers through the loop
  auto row_m = [&](int rt) { return rg * pl.rows_wg + (rw * ROWT + rt) * 16 + n; };
  auto row_out = [&](int mm) {
    return (static_cast<size_t>(b) * twoB + mm % twoB) * pl.Hq + kvh * pl.G + mm / twoB;
  };
  const int c0 = s * pl.chunk;
  const bool has_block = (s == 0);
  // The block keys either sit in their own LDS region (BSEP: R = blk_rows
  // rows of K, then of V; rows past 2B re-read row 2B-1), loaded with the
  // query rows and processed before the first prompt tile lands, or stream
  // through the ring as its first nbt tiles.  (One kernel holding both paths
  // needs about 35 more VGPRs.)
  const int R = BSEP ? pl.blk_rows : 0;
  const bool blk = BSEP && has_block;
  const int nbt = !BSEP && has_block ? (twoB + KT - 1) / KT : 0;
  const int BVREG = BKREG + R * L::ROWB;
  const int plen = a.prompt_len ? a.prompt_len[b] : pl.p_max;  // scalar load
  const uint32_t sbase = lds_addr(smem);

  // ---- prologue loads, all direct to LDS and issued first (a wave's loads
  //      complete in issue order, so waiting for all but the ring loads
  //      waits for exactly these): stage labels and positions, then this
  //      workgroup's query rows (granules swizzled like the ring tiles;
  //      rows past M re-read row M-1), then the block rows if they have
  //      their own region.
  if (wave == 0) {
    const int lc = min(lane, B - 1);
    dma4(tau_b + lc, sbase + S::TPREG);
    if (pos_b) dma4(pos_b + lc, sbase + S::TPREG + 256);
  }
  {
    const uint16_t* qg = static_cast<const uint16_t*>(a.q_blk);
    for (int ins = wave; ins < QI; ins += NW) {
      const int lr = ins * L::RPI + lane / L::GR;
      int mq = rg * pl.rows_wg + lr;
      if (mq >= pl.M) mq = pl.M - 1;
      const size_t ro = (static_cast<size_t>(b) * twoB + mq % twoB) * pl.Hq + kvh * pl.G + mq / twoB;
      const int gsrc = (lane % L::GR) ^ (lr & (L::GR - 1));
      dma16(qg + ro * HD + gsrc * 8, sbase + S::qrow(ins * L::RPI));
    }
  }

  // ---- ring loads.  Lane `lane` of load instruction `ins` fills LDS
  //      granule position lane%GR of tile row ins*RPI + lane/GR, i.e. global
  //      granule (pos ^ row) of that row.  Tile t < nbt is block tile t:
  //      block rows 64t.. of this KV head's K and V (rows past 2B re-read
  //      row 2B-1), rotated in LDS once landed.  Tile nbt + u is prompt tile
  //      u, keys c0 + 64u ..; in a tile that ends past `lim` the rows beyond
  //      it re-read key lim-1 (finite values; their scores are masked).
  const size_t cache_base = (static_cast<size_t>(b) * pl.Hkv + kvh) * static_cast<size_t>(pl.p_max) * HD;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache) + cache_base;
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache) + cache_base;
  const uint16_t* kblk = static_cast<const uint16_t*>(a.k_blk);
  const uint16_t* vblk = static_cast<const uint16_t*>(a.v_blk);
  // per-lane byte offset of load mm inside a full tile: row grow, granule (pos ^ row)
  uint32_t goff[LPW];
#pragma unroll
  for (int mm = 0; mm < LPW; ++mm) {
    const int ins = wave * LPW + mm;
    const bool isv = ins >= L::IPT;
    const int ii = isv ? ins - L::IPT : ins;
    const int grow = ii * L::RPI + lane / L::GR;
    const int sw = isv ? vsw<HD>(grow) : (grow & (L::GR - 1));
    goff[mm] = grow * L::ROWB + (((lane % L::GR) ^ sw) << 4);
  }
  const size_t blk_row = static_cast<size_t>(pl.Hkv) * HD;  // elements between block rows
  const uint16_t* kblk_b = kblk + (static_cast<size_t>(b) * twoB * pl.Hkv + kvh) * HD;
  const uint16_t* vblk_b = vblk + (static_cast<size_t>(b) * twoB * pl.Hkv + kvh) * HD;
  // Staggered tile order: the whole prompt tiles of stream (b, kvh) start at
  // tile (b * Hkv + kvh) mod nfull and wrap around, the ragged last tile
  // stays last.  Streams that all started at tile 0 would read addresses a
  // power of two apart at every step; staggered, they spread over the memory
  // channels (a streaming probe of this ring: 3.5% faster).  The row groups
  // of one stream keep the same order, so they still share each tile in L2.
  // map_nfull / map_rot hold the order the loads are issued in: first for a
  // prompt filling the cache, then for the real prompt length.
  const int rot_key = b * pl.Hkv + kvh;
  int map_nfull = 0, map_rot = 0;
  auto issue = [&](int ST, int t, int lim) __attribute__((always_inline)) {
    if (t >= nbt) {
      int u = t - nbt;
      if (u < map_nfull) {
        u += map_rot;
        if (u >= map_nfull) u -= map_nfull;
      }
      const int kb = c0 + u * KT;
      const uint16_t* ktile = kc + static_cast<size_t>(kb) * HD;
      const uint16_t* vtile = vc + static_cast<size_t>(kb) * HD;
      // A whole tile (the wave-uniform common case) takes the per-lane
      // offsets as they are; kept apart from the clamped form so the
      // compiler branches instead of computing both and selecting.
      // (KVNT: the non-temporal form, for a call whose K/V region is at
      // least the size of the last-level cache)
      if (__builtin_expect(kb + KT <= lim, 1)) {
#pragma unroll
        for (int mm = 0; mm < LPW; ++mm) {
          const int ins = wave * LPW + mm;
          const bool isv = ins >= L::IPT;
          const int ii = isv ? ins - L::IPT : ins;
          const uint32_t dst = sbase + (isv ? VREG : KREG) + ST * L::TILEB + ii * 1024;
          if constexpr (KVNT)
            dma16s_nt(isv ? vtile : ktile, goff[mm], dst);
          else
            dma16s(isv ? vtile : ktile, goff[mm], dst);
        }
      } else {
#pragma unroll
        for (int mm = 0; mm < LPW; ++mm) {
          const int ins = wave * LPW + mm;
          const bool isv = ins >= L::IPT;
          const int ii = isv ? ins - L::IPT : ins;
          const int row = static_cast<int>(goff[mm] / L::ROWB);
          const uint32_t off = (min(kb + row, lim - 1) - kb) * L::ROWB + goff[mm] % L::ROWB;
          const uint32_t dst = sbase + (isv ? VREG : KREG) + ST * L::TILEB + ii * 1024;
          if constexpr (KVNT)
            dma16s_nt(isv ? vtile : ktile, off, dst);
          else
            dma16s(isv ? vtile : ktile, off, dst);
        }
      }
    } else {
#pragma unroll
      for (int mm = 0; mm < LPW; ++mm) {
        const int ins = wave * LPW + mm;
        const bool isv = ins >= L::IPT;
        const int ii = isv ? ins - L::IPT : ins;
        const int c = min(t * KT + static_cast<int>(goff[mm] / L::ROWB), twoB - 1);
        const uint32_t off = static_cast<uint32_t>(c * blk_row * 2) + goff[mm] % L::ROWB;
        dma16s(isv ? vblk_b : kblk_b, off, sbase + (isv ? VREG : KREG) + ST * L::TILEB + ii * 1024);
      }
    }
  };
  // tiles [from, to) of the ring, to <= NSTAGE
  auto issue_range = [&](int from, int to, int lim) __attribute__((always_inline)) {
    for (int t = from; t < to; ++t) issue(t, t, lim);
  };

  // Tile order: the block tiles (split 0 only), then the prompt tiles.  The
  // first tiles go in flight before prompt_len is known, the prompt ones
  // assuming the whole cache capacity (always in bounds).
  const int c1s = min(c0 + pl.chunk, pl.p_max);
  const int nts = c1s > c0 ? (c1s - c0 + KT - 1) / KT : 0;
  map_nfull = c1s > c0 ? (c1s - c0) / KT : 0;
  map_rot = map_nfull > 0 ? rot_key % map_nfull : 0;
  // Only the first two go out before the query rows and stage labels have
  // landed: behind a whole ring of tile loads from every workgroup those small
  // scattered loads land about with its last tile, and the work that needs
  // them would then leave the memory idle once the rings are full.  The rest
  // of the ring is issued once they are in.
  constexpr int kSpecTiles = NPRO < 2 ? NPRO : 2;
  const int nspec = min(kSpecTiles, nbt + nts);
  if (blk) {
    // R K rows then R V rows, RPI rows per 1 KiB load, swizzled like ring rows
    for (int ins = wave; ins < 2 * R / L::RPI; ins += NW) {
      const int row = ins * L::RPI + lane / L::GR;
      const bool isv = row >= R;
      const int lr = isv ? row - R : row;
      const int sw = isv ? vsw<HD>(lr) : (lr & (L::GR - 1));
      const size_t c = static_cast<size_t>(min(lr, twoB - 1));
      dma16((isv ? vblk_b : kblk_b) + c * blk_row + ((lane % L::GR) ^ sw) * 8, sbase + BKREG + ins * 1024);
    }
  }
  issue_range(0, nspec, c1s);

  // ---- RoPE table of the distinct block positions (B with the RoPE copy,
  //      2B without it), while the loads are in flight: positions come by
  //      scalar loads (a wave's 64 entries need at most two)
  float2* cs_tab = reinterpret_cast<float2*>(smem + BKREG + 2 * R * L::ROWB);
  const int nent = pl.tab_rows;  // block row r uses entry r % nent
  {
    const double lane_inv_freq = rope_inv_freq(tid % HALF, HD, pl.log2_base);
    for (int i0 = 0; i0 < nent * HALF; i0 += NT) {
      const int kw = __builtin_amdgcn_readfirstlane((i0 + wave * 64) / HALF);
      const int r0 = min(kw, nent - 1), r1 = min(kw + 1, nent - 1);
      const int k0 = r0 >= B ? r0 - B : r0, k1 = r1 >= B ? r1 - B : r1;  // r < 2B
      int p0 = plen + k0, p1 = plen + k1;
      if (pos_b) sload2(pos_b + k0, pos_b + k1, p0, p1);
      const int64_t q0 = static_cast<int64_t>(p0) + (r0 >= B ? B : 0);
      const int64_t q1 = static_cast<int64_t>(p1) + (r1 >= B ? B : 0);
      const int i = i0 + tid;
      if (i < nent * HALF) cs_tab[i] = rope_cos_sin(i / HALF == kw ? q0 : q1, lane_inv_freq);
    }
  }

  // ---- wait for the prologue loads only (all but the ring's), then share them
  if (NSTAGE > 3 && nspec >= 4)
    wait_counts<(NSTAGE > 3 ? 4 : 0) * LPW, 0>();
  else if (nspec >= 3)
    wait_counts<3 * LPW, 0>();
  else if (nspec == 2)
    wait_counts<2 * LPW, 0>();
  else if (nspec == 1)
    wait_counts<LPW, 0>();
  else
    wait_counts<0, 0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  const int32_t* tp = reinterpret_cast<const int32_t*>(smem + S::TPREG);
  int tau_v = 1, pos_v = 0;  // lanes 0..B-1 of every wave hold tau and the block positions
  if (lane < B) {
    tau_v = tp[lane];
    pos_v = pos_b ? tp[64 + lane] : plen + lane;
  }
  const bool bad_tau = lane < B && (tau_v < 0 || tau_v > B);
  const bool bad_pos = lane < B && pos_v < 0;
  int st = (__any(bad_tau) ? SIMSD_ST_TAU_RANGE : 0) | (__any(bad_pos) ? SIMSD_ST_POS_NEG : 0);
  if (plen < 0 || plen > pl.p_max) st |= SIMSD_ST_PROMPT_LEN;
  const bool status_writer = a.status && kvh == 0 && s == 0 && rg == 0 && tid == 0;
  const int c1 = min(c0 + pl.chunk, plen);
  const int ntiles = c1 > c0 ? (c1 - c0 + KT - 1) / KT : 0;
  const int T = nbt + ntiles;
  if (st || (T == 0 && !blk)) {
    wait_counts<0, 15>();  // drain the ring loads before the workgroup's LDS is released
    if (status_writer) a.status[b] = st;
    if (st && pl.nsplit == 1 && ks == 0) {
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        const int mm = row_m(rt);
        if (mm >= pl.M) continue;
        uint16_t* op = static_cast<uint16_t*>(a.out) + row_out(mm) * HD;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) *reinterpret_cast<uint2*>(op + 16 * dt + 4 * g) = make_uint2(0u, 0u);
        if (a.lse && g == 0) a.lse[row_out(mm)] = -INFINITY;
      }
    }
    return;
  }
  // A speculative prompt tile that reaches past the prompt may hold cache
  // rows beyond P_b (any bits, NaN included, which a zero probability would
  // not cancel in P V), and a prompt shorter than the cache changes the
  // staggered order: then drop the speculative tiles and issue again.  Then
  // fill the remaining prologue stages.
  int issued = nspec;
  const int nfull_p = c1 > c0 ? (c1 - c0) / KT : 0;
  if (nspec > nbt && (c0 + (nspec - nbt) * KT > c1 || nfull_p != map_nfull)) {
    wait_counts<0, 15>();
    issued = nbt;
  }
  map_nfull = nfull_p;
  map_rot = nfull_p > 0 ? rot_key % nfull_p : 0;
  issue_range(issued, min(NPRO, T), c1);

  // ---- Q operands of this lane's rows, rotated in registers: k-steps i and
  //      i + KSTEPS/2 of a lane hold the two halves of the same RoPE pairs
  //      (granules 4i + g and 4i + g + GR/2), so no LDS pass is needed.
  bf16x8 qop[ROWT][KSTEPS];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    const int lr = (rw * ROWT + rt) * 16 + n;
    const int mq = row_m(rt);
    const bool rok = mq < pl.M;
    const unsigned char* qrow = smem + S::qrow(lr);
    uint4 wq[KSTEPS];
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i)
      wq[i] = rok ? *reinterpret_cast<const uint4*>(qrow + (((4 * i + g) ^ (lr & (L::GR - 1))) << 4))
                  : make_uint4(0u, 0u, 0u, 0u);
    if (rok) {
      const float2* csr_row = cs_tab + ((mq % twoB) % nent) * HALF;
#pragma unroll
      for (int i = 0; i < KSTEPS / 2; ++i) {
        const float4* csr = reinterpret_cast<const float4*>(csr_row + 8 * (4 * i + g));
        float4 c4[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) c4[q4] = csr[q4];
        const uint4 x4 = wq[i], y4 = wq[i + KSTEPS / 2];
        const uint32_t wx[4] = {x4.x, x4.y, x4.z, x4.w};
        const uint32_t wy[4] = {y4.x, y4.y, y4.z, y4.w};
        uint32_t ox[4], oy[4];
        rotate8(wx, wy, c4, ox, oy);
        wq[i] = make_uint4(ox[0], ox[1], ox[2], ox[3]);
        wq[i + KSTEPS / 2] = make_uint4(oy[0], oy[1], oy[2], oy[3]);
      }
    }
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) qop[rt][i] = __builtin_bit_cast(bf16x8, wq[i]);
  }
  // Block visibility of row tile rt's row in block tile bt (bit k: key k of
  // the tile), from the stage labels held in lanes 0..B-1 (wave ballots).
  auto block_vis = [&](int rt, int bt) -> uint64_t {
    const int mm = row_m(rt);
    uint64_t dbits, mbits;
    mask_row_bits_wave(tau_v, lane, B, mm % twoB, pl.mask_mode, dbits, mbits);
    if (mm >= pl.M) return 0ull;
    if (B >= 64) return bt == 0 ? dbits : mbits;
    return bt == 0 ? (dbits | (mbits << B)) : (mbits >> (64 - B));
  };
  if (!QSEP) {
    lds_barrier<63>();  // every wave holds its query rows: the stages they borrowed are free
#pragma unroll
    for (int t2 = NPRO; t2 < NSTAGE; ++t2)
      if (t2 < T) issue(t2, t2, c1);
  }

  // ---- loop-invariant LDS offsets of this lane's operand reads
  // K: row 16*(ks*NSUB + i) + n, granule 4*kk + g.  The swizzle depends on
  // the row only through n, so subtile i is a constant offset.
  int kofs[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) kofs[kk] = KREG + swz<HD>(16 * ks * NSUB + n, 4 * kk + g);
  // V^T: lane (g, r, c) = (lane/16, (lane%16)/4, lane%4) reads the 8 bytes at
  // row 32u + 4g + r (then + 16), columns 16dt + 4c.., and the transposed read
  // hands lane n the column 16dt + n of those 4 rows.
  // Rows +16 and +32u keep the swizzle (it depends on the row mod 16), so
  // they are immediate offsets of one address per 16-dim tile.
  uint32_t vadr[DTILES];
  {
    const uint32_t vbase = sbase + VREG;
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int vc4 = lane & 3;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
      vadr[dt] = vbase + swz_v<HD>(32 * ((ks * NSUB) / 2) + vr, 2 * dt + (vc4 >> 1)) + (vc4 & 1) * 8;
  }

  // ---- online-softmax state of this wave's share of the keys, per row tile
  float mref[ROWT], lpart[ROWT];  // reference (log2 units, -inf until set), partial sum
  const float scale = pl.scale_log2;
  f32x4 acc[ROWT][DTILES];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    mref[rt] = -INFINITY;
    lpart[rt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) acc[rt][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // K operands of this wave's keys of the tile in stage ST, all read at once
  // (their latency is then paid once, behind the softmax of the previous tile).
  // With the stage known at compile time (SC >= 0) its offset is part of the
  // instructions' immediate offset; otherwise it is added at run time.
  auto kread = [&](auto stage_c, int st, bf16x8 (&kop)[NSUB][KSTEPS]) __attribute__((always_inline)) {
    constexpr int SC = decltype(stage_c)::value;
#pragma unroll
    for (int i = 0; i < NSUB; ++i)
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        if constexpr (SC >= 0)
          kop[i][kk] = *reinterpret_cast<const bf16x8*>(smem + kofs[kk] + (SC * L::TILEB + i * 16 * L::ROWB));
        else
          kop[i][kk] = *reinterpret_cast<const bf16x8*>(smem + (kofs[kk] + st * L::TILEB) + i * 16 * L::ROWB);
      }
  };
  // S^T of those keys for every row tile (each K operand feeds ROWT MFMAs).
  auto kmma = [&](const bf16x8 (&kop)[NSUB][KSTEPS], f32x4 (&sacc)[ROWT][NSUB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      f32x4 sa[ROWT];
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) sa[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
        for (int rt = 0; rt < ROWT; ++rt) sa[rt] = mfma(kop[i][kk], qop[rt][kk], sa[rt]);
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) sacc[rt][i] = sa[rt];
    }
  };

  // V^T operands of the tile in stage ST (the reads complete during the softmax).
  auto vread = [&](auto stage_c, int st, bf16x8 (&vop)[DTILES][NU]) __attribute__((always_inline)) {
    constexpr int SC = decltype(stage_c)::value;
    constexpr int SO = SC >= 0 ? SC * L::TILEB : 0;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        const uint32_t va = SC >= 0 ? vadr[dt] : vadr[dt] + st * L::TILEB;
        bf16x4 lo, hi;
        if (uu == 0) {
          lo = tr_read<SO>(va);
          hi = tr_read<SO + 16 * L::ROWB>(va);
        } else {
          lo = tr_read<SO + 32 * L::ROWB>(va);
          hi = tr_read<SO + 48 * L::ROWB>(va);
        }
        vop[dt][uu] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };

  // One key split (all 64 keys of a tile per wave, 32 rows): the K operands
  // of 16-key subtile i, and the V^T operands of 32-key half uu, of the tile
  // in stage ST.  Read a subtile or a half at a time: the whole tile's
  // operands at once would not fit beside the accumulators of 32 rows.
  auto ksub = [&](auto stage_c, int st, int i, bf16x8 (&ko)[KSTEPS]) __attribute__((always_inline)) {
    constexpr int SC = decltype(stage_c)::value;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if constexpr (SC >= 0)
        ko[kk] = *reinterpret_cast<const bf16x8*>(smem + kofs[kk] + (SC * L::TILEB + i * 16 * L::ROWB));
      else
        ko[kk] = *reinterpret_cast<const bf16x8*>(smem + (kofs[kk] + st * L::TILEB) + i * 16 * L::ROWB);
    }
  };
  auto vhalf = [&](auto stage_c, int st, int uu, bf16x8 (&vo)[DTILES]) __attribute__((always_inline)) {
    constexpr int SC = decltype(stage_c)::value;
    constexpr int SO = SC >= 0 ? SC * L::TILEB : 0;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const uint32_t va = SC >= 0 ? vadr[dt] : vadr[dt] + st * L::TILEB;
      bf16x4 lo, hi;
      if (uu == 0) {
        lo = tr_read<SO>(va);
        hi = tr_read<SO + 16 * L::ROWB>(va);
      } else {
        lo = tr_read<SO + 32 * L::ROWB>(va);
        hi = tr_read<SO + 48 * L::ROWB>(va);
      }
      vo[dt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // Rotate block K rows row0 .. row0 + nvalid - 1, held from Kb on (K
  // swizzle), in place.
  auto rotate_rows = [&](unsigned char* Kb, int nvalid, int row0) __attribute__((always_inline)) {
    for (int i = tid; i < nvalid * (L::GR / 2); i += NT) {
      const int row = i / (L::GR / 2), j = i % (L::GR / 2);
      uint4* px = reinterpret_cast<uint4*>(Kb + swz<HD>(row, j));
      uint4* py = reinterpret_cast<uint4*>(Kb + swz<HD>(row, j + L::GR / 2));
      const uint4 x4 = *px, y4 = *py;
      const float4* csr = reinterpret_cast<const float4*>(cs_tab + ((row0 + row) % nent) * HALF + 8 * j);
      float4 c4[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) c4[q4] = csr[q4];
      const uint32_t wx[4] = {x4.x, x4.y, x4.z, x4.w};
      const uint32_t wy[4] = {y4.x, y4.y, y4.z, y4.w};
      uint32_t ox[4], oy[4];
      rotate8(wx, wy, c4, ox, oy);
      *px = make_uint4(ox[0], ox[1], ox[2], ox[3]);
      *py = make_uint4(oy[0], oy[1], oy[2], oy[3]);
    }
  };
  // Rotate block tile bt (its K rows in stage st) in place.
  auto rotate_block = [&](int st, int bt) __attribute__((always_inline)) {
    rotate_rows(smem + KREG + st * L::TILEB, min(KT, twoB - bt * KT), bt * KT);
    lds_barrier<63>();
  };

  // Softmax of the scores into the P^T operands, for every row tile.  MODE 0:
  // every key visible; MODE 1: key k of the tile visible for row tile rt when
  // bit k of cmask[rt] is set.
  auto softmax = [&](auto mode_c, const f32x4 (&sacc)[ROWT][NSUB], const uint64_t (&cmask)[ROWT],
                     bf16x8 (&pop)[ROWT][NU]) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    // The probabilities are taken against the current reference right away,
    // alongside the maximum, for every row tile: the exponentials then do not
    // wait for the vote.  A row's first visible key sets its reference and a
    // score more than kRaise above it raises it; in that (rare) case the
    // accumulators are rescaled and the tile's probabilities taken again
    // against the new reference, so the result is the same as deciding
    // first.  One vote covers the wave's row tiles.  The four lanes of a row
    // reduce the same maximum, so they take the same decision.
    float sv[ROWT][NSUB][4], pv[ROWT][NSUB][4], tmax[ROWT], lsum[ROWT];
    bool need_any = false;
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt) {
      tmax[rt] = -INFINITY;
      // this lane's keys are 16*(ks*NSUB + i) + 4g + j: one variable shift, then constant bit tests
      const uint64_t cm = MODE == 0 ? 0ull : cmask[rt] >> (16 * ks * NSUB + 4 * g);
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool vis = MODE == 0 || ((cm >> (16 * i + j)) & 1ull);
          const float x = vis ? sacc[rt][i][j] : -INFINITY;  // raw score; the scale is applied below
          sv[rt][i][j] = x;
          tmax[rt] = fmaxf(tmax[rt], x);
        }
      }
      const float muse = (mref[rt] == -INFINITY) ? 0.0f : mref[rt];
      lsum[rt] = 0.0f;
#pragma unroll
      for (int i = 0; i < NSUB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[rt][i][j] = __builtin_amdgcn_exp2f(fmaf(sv[rt][i][j], scale, -muse));
          lsum[rt] += pv[rt][i][j];
        }
      need_any |= mref[rt] == -INFINITY ? tmax[rt] != -INFINITY : tmax[rt] * scale > mref[rt] + kRaise;
    }
    if (__any(need_any)) {
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        float rmax = fmaxf(tmax[rt], __shfl_xor(tmax[rt], 16));
        rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
        const float nref = rmax * scale;
        if (mref[rt] == -INFINITY ? nref != -INFINITY : nref > mref[rt] + kRaise) {
          const float f = mref[rt] == -INFINITY ? 0.0f : exp2f(mref[rt] - nref);
          lpart[rt] *= f;
#pragma unroll
          for (int dt = 0; dt < DTILES; ++dt) acc[rt][dt] = acc[rt][dt] * f;
          mref[rt] = nref;
          lsum[rt] = 0.0f;
#pragma unroll
          for (int i = 0; i < NSUB; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              pv[rt][i][j] = __builtin_amdgcn_exp2f(fmaf(sv[rt][i][j], scale, -nref));
              lsum[rt] += pv[rt][i][j];
            }
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt) {
      lpart[rt] += lsum[rt];
      // P^T operand of k-step u: keys 4g..4g+3 of subtile 2u, then of 2u+1;
      // subtiles of other waves contribute zeros.
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        const int u = (ks * NSUB) / 2 + uu;
        __bf16 pb[8];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int i = 2 * u + h2 - ks * NSUB;
          const int ic = i < 0 ? 0 : (i >= NSUB ? NSUB - 1 : i);
#pragma unroll
          for (int j = 0; j < 4; ++j) pb[4 * h2 + j] = static_cast<__bf16>((i >= 0 && i < NSUB) ? pv[rt][ic][j] : 0.0f);
        }
        pop[rt][uu] = bf16x8{pb[0], pb[1], pb[2], pb[3], pb[4], pb[5], pb[6], pb[7]};
      }
    }
  };
  // Softmax and O^T += V^T P^T, for every row tile (each V^T operand feeds
  // ROWT MFMAs).
  auto finish = [&](auto mode_c, const f32x4 (&sacc)[ROWT][NSUB], const bf16x8 (&vop)[DTILES][NU],
                    const uint64_t (&cmask)[ROWT]) __attribute__((always_inline)) {
    bf16x8 pop[ROWT][NU];
    softmax(mode_c, sacc, cmask, pop);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int uu = 0; uu < NU; ++uu)
#pragma unroll
        for (int rt = 0; rt < ROWT; ++rt) acc[rt][dt] = mfma(vop[dt][uu], pop[rt][uu], acc[rt][dt]);
  };

  // ---- the T = ntiles + nbt tiles over the ring.  Before step t: tiles
  //      0 .. min(t + NSTAGE - 2, T - 1) are issued (0 .. min(NSTAGE, T) - 1
  //      for t = 0), in tile order.
  f32x4 sb[ROWT][NSUB];
  // ---- the block keys from their own region, before the first prompt tile
  //      (the block work costs about the same at any step: done first, the
  //      result matches the ring path's bit for bit).  Only waves whose key
  //      range starts below 2B take part.  Their operand reads of key row k
  //      use block row k mod R, so the keys past 2B hold finite values; the
  //      mask drops them.
  if (blk) {
    rotate_rows(smem + BKREG, twoB, 0);
    lds_barrier<63>();
  }
  if (blk && 16 * ks * NSUB < twoB) {
    bf16x8 kop[NSUB][KSTEPS];
#pragma unroll
    for (int i = 0; i < NSUB; ++i) {
      const int ro = BKREG + ((16 * (ks * NSUB + i)) % R) * L::ROWB;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        kop[i][kk] = *reinterpret_cast<const bf16x8*>(smem + ro + swz<HD>(n, 4 * kk + g));
    }
    bf16x8 vop[DTILES][NU];
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int vc4 = lane & 3;
#pragma unroll
    for (int uu = 0; uu < NU; ++uu) {
      const int u = (ks * NSUB) / 2 + uu;
      const uint32_t rlo = sbase + BVREG + ((32 * u) % R) * L::ROWB;
      const uint32_t rhi = sbase + BVREG + ((32 * u + 16) % R) * L::ROWB;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const uint32_t co = swz_v<HD>(vr, 2 * dt + (vc4 >> 1)) + (vc4 & 1) * 8;
        vop[dt][uu] = __builtin_shufflevector(tr_read<0>(rlo + co), tr_read<0>(rhi + co), 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
    kmma(kop, sb);
    uint64_t cm[ROWT];
#pragma unroll
    for (int rt = 0; rt < ROWT; ++rt) cm[rt] = block_vis(rt, 0);
    finish(IC<1>{}, sb, vop, cm);
  }
  const int nfull = (c1 - c0) / KT;  // whole prompt tiles: nbt .. nbt + nfull - 1
  // Wide blocks (two row tiles a wave: the step is bound by the work inside
  // the CU, not by memory) take one barrier per pair of tiles: tiles t and
  // t+1 are waited for together at even steps, so two are in flight while
  // two are in use.
  constexpr bool kPairs = ROWT == 2 && NSTAGE == 4;
  if constexpr (kPairs) {
    const int ahead = min(T, NSTAGE) - 2;  // tiles issued beyond tiles 0 and 1
    if (ahead >= 2)
      lds_barrier<2 * LPW>();
    else if (ahead == 1)
      lds_barrier<LPW>();
    else
      lds_barrier<0>();  // tiles 0 and 1 landed
    if (nbt > 0) rotate_block(0, 0);
    if (nbt > 1) rotate_block(1, 1);
  } else {
    if (T >= NSTAGE)
      lds_barrier<(NSTAGE - 1) * LPW>();  // tile 0 landed
    else
      lds_barrier<0>();
    if (nbt > 0) rotate_block(0, 0);
  }
  // Step t waits for tile t only (the barrier also frees the stage of tile
  // t-1, refilled at once), then reads K and V of tile t and runs its score
  // MFMAs, softmax and PV MFMAs, so three tiles stay in flight behind the one
  // in use.  (Keeping tile t+1 resident too, to run its score MFMAs under the
  // softmax of tile t, leaves two in flight and measured 0.3-2% slower on
  // every workload.)
  // Step t.  stage_c: the ring stage of tile t when the caller knows it at
  // compile time (IC<-1>: taken from t at run time).
  auto step = [&](auto mode_c, auto stage_c, int t) __attribute__((always_inline)) {
    constexpr int SC = decltype(stage_c)::value;
    const int K = SC >= 0 ? SC : t % NSTAGE;
    if constexpr (kPairs) {
      // even steps wait for tiles t and t+1 (nothing else is in flight) and
      // refill the stages of t-2 and t-1; odd steps pass straight on
      if (t > 0 && (t & 1) == 0) {
        lds_barrier<0>();
        if (t + 2 < T) issue((K + NSTAGE - 2) % NSTAGE, t + 2, c1);
        if (t + 3 < T) issue((K + NSTAGE - 1) % NSTAGE, t + 3, c1);
      }
    } else if (t > 0) {
      const int later = T - 1 - t;  // tiles after t that may still be in flight (at most NSTAGE - 2)
      if (later >= NSTAGE - 2)
        lds_barrier<(NSTAGE - 2) * LPW>();
      else if (later == 1)
        lds_barrier<LPW>();
      else
        lds_barrier<0>();
      if (t + NSTAGE - 1 < T) issue(K == 0 ? NSTAGE - 1 : K - 1, t + NSTAGE - 1, c1);
      if (t < nbt) rotate_block(K, t);
    }
    if constexpr (KSPLIT == 1) {
      // scores subtile by subtile, the softmax, then P V half by half
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
        bf16x8 ko[KSTEPS];
        ksub(stage_c, K, i, ko);
        f32x4 sa[ROWT];
#pragma unroll
        for (int rt = 0; rt < ROWT; ++rt) sa[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
          for (int rt = 0; rt < ROWT; ++rt) sa[rt] = mfma(ko[kk], qop[rt][kk], sa[rt]);
#pragma unroll
        for (int rt = 0; rt < ROWT; ++rt) sb[rt][i] = sa[rt];
      }
      uint64_t cm[ROWT] = {};
      if (decltype(mode_c)::value != 0) {
        const int nk = c1 - (c0 + (t - nbt) * KT);  // keys of a prompt tile below c1
        const uint64_t tail = nk >= KT ? ~0ull : (1ull << nk) - 1ull;
#pragma unroll
        for (int rt = 0; rt < ROWT; ++rt) cm[rt] = t < nbt ? block_vis(rt, t) : tail;
      }
      bf16x8 pop[ROWT][NU];
      softmax(mode_c, sb, cm, pop);
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        bf16x8 vo[DTILES];
        vhalf(stage_c, K, uu, vo);
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
          for (int rt = 0; rt < ROWT; ++rt) acc[rt][dt] = mfma(vo[dt], pop[rt][uu], acc[rt][dt]);
      }
      return;
    }
    bf16x8 kop[NSUB][KSTEPS];
    kread(stage_c, K, kop);
    bf16x8 vop[DTILES][NU];
    vread(stage_c, K, vop);
    kmma(kop, sb);
    if (decltype(mode_c)::value == 0) {
      const uint64_t cm[ROWT] = {};
      finish(IC<0>{}, sb, vop, cm);
    } else {
      const int nk = c1 - (c0 + (t - nbt) * KT);  // keys of a prompt tile below c1
      const uint64_t tail = nk >= KT ? ~0ull : (1ull << nk) - 1ull;
      uint64_t cm[ROWT];
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) cm[rt] = t < nbt ? block_vis(rt, t) : tail;
      finish(IC<1>{}, sb, vop, cm);
    }
  };
  // block tiles, then whole prompt tiles, then the rest through the masked
  // path
  if (nbt == 1) {
    step(IC<1>{}, IC<-1>{}, 0);
  } else if (nbt == 2) {
    step(IC<1>{}, IC<-1>{}, 0);
    step(IC<1>{}, IC<-1>{}, 1);
  }
  // whole prompt tiles in groups of NSTAGE whose ring stages are known at
  // compile time (the stage of tile t is t mod NSTAGE), then the rest of them
  // and the ragged last tile with the stage taken at run time
  int t0 = nbt;
  const int tw = nbt + nfull;
  if (t0 % NSTAGE == 0) {
    for (; t0 + NSTAGE <= tw; t0 += NSTAGE) {
      step(IC<0>{}, IC<0>{}, t0);
      step(IC<0>{}, IC<1>{}, t0 + 1);
      step(IC<0>{}, IC<2>{}, t0 + 2);
      if constexpr (NSTAGE > 3) step(IC<0>{}, IC<NSTAGE - 1>{}, t0 + 3);
    }
  }
  for (; t0 < tw; ++t0) step(IC<0>{}, IC<-1>{}, t0);
  for (; t0 < T; ++t0) step(IC<1>{}, IC<-1>{}, t0);

  // ---- combine the key splits of each row (through the drained ring)
  wait_counts<0, 15>();  // no ring load may land after the workgroup ends
  if (status_writer) a.status[b] = 0;
  float l[ROWT];
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    l[rt] = lpart[rt];
    l[rt] += __shfl_xor(l[rt], 16);
    l[rt] += __shfl_xor(l[rt], 32);
  }
  if constexpr (KSPLIT > 1) {
    float* xb = reinterpret_cast<float*>(smem);
    lds_barrier<0>();  // every wave is done reading the ring
    if (ks > 0) {
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        float* xr = xb + ((((ks - 1) * RW + rw) * ROWT + rt) * 16 + n) * XSTR;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt)
          *reinterpret_cast<float4*>(xr + 16 * dt + 4 * g) =
              make_float4(acc[rt][dt][0], acc[rt][dt][1], acc[rt][dt][2], acc[rt][dt][3]);
        if (g == 0) {
          xr[HD] = mref[rt];
          xr[HD + 1] = l[rt];
        }
      }
    }
    lds_barrier<0>();
    if (ks > 0) return;
#pragma unroll
    for (int k2 = 1; k2 < KSPLIT; ++k2)
#pragma unroll
      for (int rt = 0; rt < ROWT; ++rt) {
        const float* xr = xb + ((((k2 - 1) * RW + rw) * ROWT + rt) * 16 + n) * XSTR;
        const float m2 = xr[HD], l2 = xr[HD + 1];
        const float mnew = fmaxf(mref[rt], m2);
        const float a1 = (mref[rt] == mnew) ? 1.0f : exp2f(mref[rt] - mnew);
        const float a2 = (m2 == mnew) ? 1.0f : exp2f(m2 - mnew);
        l[rt] = l[rt] * a1 + l2 * a2;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) {
          const float4 o2 = *reinterpret_cast<const float4*>(xr + 16 * dt + 4 * g);
          acc[rt][dt] = acc[rt][dt] * a1 + f32x4{o2.x, o2.y, o2.z, o2.w} * a2;
        }
        mref[rt] = mnew;
      }
  }

  // ---- epilogue (key-split 0 waves)
#pragma unroll
  for (int rt = 0; rt < ROWT; ++rt) {
    const int mm = row_m(rt);
    if (mm >= pl.M) continue;
    if (pl.nsplit == 1) {
      const float inv = 1.0f / l[rt];
      uint16_t* op = static_cast<uint16_t*>(a.out) + row_out(mm) * HD;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const f32x4 v = acc[rt][dt];
        *reinterpret_cast<uint2*>(op + 16 * dt + 4 * g) =
            make_uint2(pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv));
      }
      if (a.lse && g == 0) a.lse[row_out(mm)] = (mref[rt] + log2f(l[rt])) * kLn2;
    } else {
      const size_t slot = (static_cast<size_t>(b) * pl.Hkv + kvh) * pl.nsplit + s;
      float* po = a.part_o + (slot * pl.M + mm) * HD;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const f32x4 v = acc[rt][dt];
        *reinterpret_cast<float4*>(po + 16 * dt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0) {
        a.part_ml[(slot * pl.M + mm) * 2 + 0] = mref[rt];
        a.part_ml[(slot * pl.M + mm) * 2 + 1] = l[rt];
      }
    }
  }
}

template <int HD, int RW, int KSPLIT, int NSTAGE, bool QSEP, int ROWT, bool BSEP, bool KVNT>
hipError_t launch_cfg(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  auto kern = verify_mfma_kernel<HD, RW, KSPLIT, NSTAGE, QSEP, ROWT, BSEP, KVNT>;
  const size_t lds = mfma_lds_bytes(HD, NSTAGE, pl.tab_rows, RW * ROWT * 16, QSEP, pl.blk_rows);
  // the table and staged-row sizes vary per call: allow the whole LDS once
  const hipError_t e = allow_dynamic_lds<verify_mfma_kernel<HD, RW, KSPLIT, NSTAGE, QSEP, ROWT, BSEP, KVNT>>(kLdsMax);
  if (e != hipSuccess) return e;
  if (lds > static_cast<size_t>(kLdsMax)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(pl.Hkv), static_cast<unsigned>(pl.NB) * static_cast<unsigned>(pl.nrg),
                  static_cast<unsigned>(pl.nsplit));
  return launch_with_events(kern, grid, dim3(RW * KSPLIT * 64), lds, s, ev.start, ev.stop, pl, a);
}

// Rows per workgroup -> (row waves, key splits, row tiles per wave): up to 64
// rows one 16-row tile per wave with the keys split over 4 or 2 waves; 128
// rows four row waves of two row tiles each, keys split over 2 waves, so
// every K and V operand read from LDS feeds two MFMAs; 256 rows (head dim
// 128) eight row waves of two row tiles, each over all keys of a tile, so
// that one workgroup, not two, streams each K/V split.
template <int HD, int NSTAGE, bool QSEP, bool BSEP, bool KVNT>
hipError_t launch_rows(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  switch (pl.rows_wg / 16) {
    case 1: return launch_cfg<HD, 1, 4, NSTAGE, QSEP, 1, BSEP, KVNT>(pl, a, s, ev);
    case 2: return launch_cfg<HD, 2, 4, NSTAGE, QSEP, 1, BSEP, KVNT>(pl, a, s, ev);
    case 4: return launch_cfg<HD, 4, 2, NSTAGE, QSEP, 1, BSEP, KVNT>(pl, a, s, ev);
    case 8: return launch_cfg<HD, 4, 2, NSTAGE, QSEP, 2, BSEP, KVNT>(pl, a, s, ev);
    case 16:
      // the query rows borrow two of four ring stages; the block keys stream
      // through the ring
      if constexpr (HD == 128 && NSTAGE == 4 && !QSEP && !BSEP)
        return launch_cfg<HD, 8, 1, NSTAGE, false, 2, false, KVNT>(pl, a, s, ev);
      return hipErrorInvalidConfiguration;
    default: return hipErrorInvalidConfiguration;
  }
}

template <int HD, int NSTAGE, bool QSEP, bool KVNT>
hipError_t launch_stages(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  return pl.blk_rows > 0 ? launch_rows<HD, NSTAGE, QSEP, true, KVNT>(pl, a, s, ev)
                         : launch_rows<HD, NSTAGE, QSEP, false, KVNT>(pl, a, s, ev);
}

}  // namespace

// Dynamic LDS of one workgroup: the tile ring, stage labels and positions,
// the staged query rows when they have their own region, blk_rows block K
// rows and as many V rows, the RoPE table.
size_t mfma_lds_bytes(int hd, int nstage, int tab_rows, int rows_wg, bool qsep, int blk_rows) {
  const size_t ring = static_cast<size_t>(nstage) * 2 * KT * hd * 2;
  return ring + 512 + (qsep ? static_cast<size_t>(rows_wg) * hd * 2 : 0) +
         2 * static_cast<size_t>(blk_rows) * hd * 2 + static_cast<size_t>(tab_rows) * (hd / 2) * sizeof(float2);
}

namespace {

template <bool KVNT>
hipError_t launch_policy(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  if (pl.d == 64) return launch_stages<64, 4, true, KVNT>(pl, a, s, ev);
  if (pl.qsep) return launch_stages<128, 4, true, KVNT>(pl, a, s, ev);
  if (pl.nstage == 4) return launch_stages<128, 4, false, KVNT>(pl, a, s, ev);
  // the planner gives the block rows a region of their own only beside a 4-stage ring
  if (pl.blk_rows > 0) return hipErrorInvalidConfiguration;
  return launch_rows<128, 3, false, false, KVNT>(pl, a, s, ev);
}

}  // namespace

hipError_t launch_verify_mfma(const Plan& pl, const VerifyArgs& a, hipStream_t s, PassEvents ev) {
  // the tiles' cache policy is a template parameter: a run-time choice
  // inside the issue loop changed the code of the whole ring schedule
  return pl.kv_stream ? launch_policy<true>(pl, a, s, ev) : launch_policy<false>(pl, a, s, ev);
}

}  // namespace simsd
