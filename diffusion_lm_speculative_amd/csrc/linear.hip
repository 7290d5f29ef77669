// Projections around the verification attention on the matrix cores: the
// fused QKV projection of the block rows' hidden states and the output
// projection (page "SimSD - Simple Speculative Decoding in Diffusion Language
// Models", section 4: one target forward pass over the paired layout; its
// attention sits between these two linear maps).  y = x W^T in the nn.Linear
// convention, bf16 in, fp32 accumulate, bf16 out (round to nearest even).
//
// Formulation.  The product is computed transposed, Y^T = W X^T, with
// v_mfma_f32_16x16x32_bf16: W rows (output channels) on the MFMA M side, x
// rows on its N side.  Both operands are then "row of k values" reads, one
// 16-byte ds_read_b128 per lane, and in the accumulator layout (lane l holds
// column l%16, rows 4*(l/16)..+3) a lane owns four consecutive output
// channels of one x row: one 8-byte store per lane and tile.
//
// Tiling.  A workgroup computes BM = 128 x rows (64 when M fits) by BN
// output channels (BN = 64, 96 or 128, chosen so the grid covers the 256 CUs
// in as few rounds as possible) with 8 waves: two groups of four, one per
// 32-k half of every 64-k slice, each group 2 x 2 waves of BN/2 channels by
// BM/2 rows.  Two waves share a SIMD, so one wave's operand reads overlap
// the other's MFMAs, while each wave keeps the large tile (few LDS reads per
// MFMA); the second group's partial sums join the first's through LDS at the
// end.  A stage's 1 KiB loads are spread over the waves; where they do not
// divide evenly the last waves issue fewer (their vmcnt waits then pass at
// once).  K advances in slices of 64 through a ring of NSTAGE LDS stages
// filled by direct-to-LDS loads (global_load_lds_dwordx4, 1 KiB per wave
// instruction, no register staging); one barrier per slice.  Rows are 128
// bytes (8 granules of 16 bytes) stored XOR-swizzled so that the operand
// reads are free of bank conflicts.
//
// Grid.  x = channel block (fastest), y = row block: the hardware hands
// consecutive workgroups to consecutive XCDs, so with a multiple of 8
// channel blocks the row blocks of one channel block (which read the same W
// tiles) share an XCD and its L2.
#include "mfma_common.hpp"

namespace simsd {
namespace {

constexpr int kLinBK = 64;      // k per stage
constexpr int kLinRowB = 128;   // bytes per staged row (64 bf16)
constexpr int kLinThreads = 512;
constexpr int kLinStages = 4;
constexpr size_t kLinLdsPerCu = 163840;

// Byte offset of granule g (0..7) of row r in a staged tile: slot g ^ (r & 7).
// The 16 rows a 16-lane group reads then take ds_read_b128 at the full 256
// bytes a cycle (an LDS counter probe on gfx950: 4 cycles per instruction;
// slot g ^ ((r & 7) ^ ((r >> 3) & 1)) took 8, half of them bank conflicts).
__device__ __forceinline__ int lin_swz(int r, int g) {
  return r * kLinRowB + ((g ^ (r & 7)) << 4);
}

struct LinearArgs {
  const uint16_t* x;  // [M][K]
  const uint16_t* w;  // [N][K]
  int64_t M;
  int N, K;
  // output channels [0, cut1) -> out0, [cut1, cut2) -> out1, [cut2, N) ->
  // out2, each row-major with its own row length
  int cut1, cut2;
  uint16_t* out[3];
  int ld[3];
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return f32_to_bf16_bits(f); }

template <int BM, int BN>
__global__ __launch_bounds__(kLinThreads) void linear_kernel(LinearArgs a) {
  static_assert(BM == 64 || BM == 128, "x rows per workgroup");
  constexpr int ATILE = BM * kLinRowB;               // x rows of one stage
  constexpr int WTILE = BN * kLinRowB;               // W rows per stage
  constexpr int STAGEB = ATILE + WTILE;
  constexpr int NW = kLinThreads / 64;
  constexpr int IA = BM / 8;                         // 1 KiB load instructions for the x tile
  constexpr int IW = BN / 8;                         // ... for the W tile
  constexpr int LPW = (IA + IW + NW - 1) / NW;       // loads per wave per stage (the last waves may have fewer)
  static_assert((kLinStages - 1) * LPW <= 63, "vmcnt range");
  constexpr int TN = BN / 32;                        // 16-channel tiles per wave
  constexpr int TM = BM / 32;                        // 16-row tiles per wave (BM/2 rows)
  static_assert(NW == 8, "two groups of four waves, one per 32-k half of every slice");

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = (wave >> 1) & 1, kh = wave >> 2;
  const int n0 = blockIdx.x * BN;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int K = a.K;
  const int nks = K / kLinBK;
  const uint32_t sbase = lds_addr(smem);

  // Per-lane global byte offsets of this wave's stage loads (relative to the
  // tile's first row at k slice 0) and the LDS byte offsets they fill.
  // Instruction i covers rows 8*i .. 8*i+7 of the x tile (i < IA) or of the
  // W tile; lane l fills slot l%8 of row l/8 and so fetches granule
  // (l%8) ^ f(row).
  uint32_t goff[LPW];
  bool isw[LPW];
  uint32_t loff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int ins = min(wave * LPW + j, IA + IW - 1);  // past the last: reloads it (harmless, see issue)
    const bool w = ins >= IA;
    const int r = (w ? ins - IA : ins) * 8 + (lane >> 3);
    const int slot = lane & 7;
    const int g = slot ^ (r & 7);
    int64_t row;
    if (w) {
      row = min(n0 + r, a.N - 1) - n0;  // channels past N reload the last one (never stored)
    } else {
      const int64_t mr = m0 + r;
      row = (mr < a.M ? mr : a.M - 1) - m0;  // rows past M likewise
    }
    goff[j] = static_cast<uint32_t>((row * K + 8 * g) * 2);
    isw[j] = w;
    loff[j] = (w ? ATILE : 0) + (w ? ins - IA : ins) * 1024;
  }
  const uint16_t* xb = a.x + m0 * K;
  const uint16_t* wb = a.w + static_cast<int64_t>(n0) * K;
  auto issue = [&](int ks) __attribute__((always_inline)) {
    const int st = ks % kLinStages;
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      if (wave * LPW + j < IA + IW) dma16s((isw[j] ? wb : xb) + ks * kLinBK, goff[j], sbase + st * STAGEB + loff[j]);
  };

  // Operand read offsets: W rows (MFMA A operand) n = wn*BN/2 + 16*i + l%16,
  // x rows (MFMA B operand) m = wm*BM/2 + 16*i + l%16; k granule 4*kk + l/16.
  int aoff[TN], boff[TM];
#pragma unroll
  for (int i = 0; i < TN; ++i) aoff[i] = ATILE + lin_swz(wn * (BN / 2) + 16 * i + (lane & 15), 4 * kh + (lane >> 4));
#pragma unroll
  for (int i = 0; i < TM; ++i) boff[i] = lin_swz(wm * (BM / 2) + 16 * i + (lane & 15), 4 * kh + (lane >> 4));

  f32x4 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int ks = 0; ks < kLinStages - 1 && ks < nks; ++ks) issue(ks);
  for (int ks = 0; ks < nks; ++ks) {
    // slice ks has landed once at most min(NSTAGE - 2, nks - 1 - ks) later
    // slices are still in flight; the barrier also frees the stage of ks - 1
    const int later = min(kLinStages - 2, nks - 1 - ks);
    if (later >= 2)
      lds_barrier<2 * LPW>();
    else if (later == 1)
      lds_barrier<LPW>();
    else
      lds_barrier<0>();
    if (ks + kLinStages - 1 < nks) issue(ks + kLinStages - 1);
    const unsigned char* sb = smem + (ks % kLinStages) * STAGEB;
    {
      bf16x8 av[TN], bv[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i) av[i] = *reinterpret_cast<const bf16x8*>(sb + aoff[i]);
#pragma unroll
      for (int j = 0; j < TM; ++j) bv[j] = *reinterpret_cast<const bf16x8*>(sb + boff[j]);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma(av[i], bv[j], acc[i][j]);
    }
  }
  // the second k half's partial sums join the first's through LDS
  lds_barrier<0>();  // every wave is done with the ring; nothing lands after this
  float4* xb4 = reinterpret_cast<float4*>(smem) + ((wn * 2 + wm) * TN * TM) * 64 + lane;
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) xb4[(i * TM + j) * 64] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
  }
  lds_barrier<0>();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const float4 o = xb4[(i * TM + j) * 64];
      acc[i][j] += f32x4{o.x, o.y, o.z, o.w};
    }

  // lane: channels n .. n+3 of x row m for every (i, j) tile
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * j + (lane & 15);
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int n = n0 + wn * (BN / 2) + 16 * i + 4 * (lane >> 4);
      if (n >= a.N) continue;
      const int seg = n < a.cut1 ? 0 : (n < a.cut2 ? 1 : 2);
      const int c = n - (seg == 0 ? 0 : (seg == 1 ? a.cut1 : a.cut2));
      uint16_t* dst = a.out[seg] + m * a.ld[seg] + c;
      const f32x4 v = acc[i][j];
      const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
      const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    }
  }
}

constexpr size_t lin_lds_bytes(int bm, int bn) { return static_cast<size_t>(kLinStages) * (bm + bn) * kLinRowB; }

template <int BM, int BN>
hipError_t launch_tile(const LinearArgs& a, hipStream_t s) {
  constexpr size_t lds = lin_lds_bytes(BM, BN);
  static_assert(lds <= kLinLdsPerCu, "LDS");
  const hipError_t e = allow_dynamic_lds<linear_kernel<BM, BN>>(static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>((a.N + BN - 1) / BN), static_cast<unsigned>((a.M + BM - 1) / BM));
  hipLaunchKernelGGL((linear_kernel<BM, BN>), grid, dim3(kLinThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// Tile (rows x channels) for an M x N product: 128-row tiles (each W slice
// feeds 128 rows; 64-row tiles two to a CU measured 12% slower on the
// 512-row projections) unless M fits 64 rows.  Channel width: the fewest
// rounds of workgroups over the 256 CUs times the width (a round of wider
// tiles takes longer); ties go to the wider tile.
int linear_tile(int64_t M, int N) {
  const int bm = M <= 64 ? 64 : 128;
  const int64_t mb = (M + bm - 1) / bm;
  int best = 128;
  int64_t best_cost = -1;
  for (int bn : {128, 96, 64}) {
    const int64_t wgs = ((N + bn - 1) / bn) * mb;
    const int64_t cost = ((wgs + 255) / 256) * bn;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = bn;
    }
  }
  return bm * 1000 + best;
}

hipError_t launch_linear(const uint16_t* x, const uint16_t* w, int64_t M, int N, int K, int cut1, int cut2,
                         uint16_t* out0, int ld0, uint16_t* out1, int ld1, uint16_t* out2, int ld2,
                         hipStream_t s) {
  LinearArgs a{};
  a.x = x;
  a.w = w;
  a.M = M;
  a.N = N;
  a.K = K;
  a.cut1 = cut1;
  a.cut2 = cut2;
  a.out[0] = out0;
  a.out[1] = out1;
  a.out[2] = out2;
  a.ld[0] = ld0;
  a.ld[1] = ld1;
  a.ld[2] = ld2;
  switch (linear_tile(M, N)) {
    case 128128: return launch_tile<128, 128>(a, s);
    case 128096: return launch_tile<128, 96>(a, s);
    case 128064: return launch_tile<128, 64>(a, s);
    case 64128: return launch_tile<64, 128>(a, s);
    case 64096: return launch_tile<64, 96>(a, s);
    default: return launch_tile<64, 64>(a, s);
  }
}

}  // namespace simsd
