// Host side of the C ABI declared in include/simsd.h: argument validation
// (before any HIP call), the split-KV plan, workspace carving and launches.
#include <cmath>
#include <cstring>

#include "simsd_common.hpp"

namespace simsd {
namespace {

constexpr int kKeyTile = 64;        // prompt keys per tile (both kernels iterate in multiples of it)
constexpr int kNumCUs = 256;        // MI355X compute units
constexpr size_t kLdsPerCu = 163840;  // bytes of LDS per CU (and per workgroup at most)
constexpr int kMaxChunk = 8192;     // default split length cap (tail of ragged prompts)
constexpr int kMinSplitTiles = 16;  // default splits of fewer tiles cost more in the merge than they save
constexpr int kMaxQHeads = 65536;   // query heads per layer accepted by the planner
constexpr int kLptMaxItems = 256;   // (sequence, split) items per KV head ranked longest first

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int make_plan(const simsd_verify_desc& d, Plan& pl) {
  if (d.batch < 0 || d.n_q_heads < 1 || d.n_kv_heads < 1 || d.n_q_heads % d.n_kv_heads != 0 ||
      (d.head_dim != 64 && d.head_dim != 128) || d.B < 0 || d.B > 64 || d.p_max < 0)
    return SIMSD_ERR_SHAPE;
  // bounds under which every count and size below fits its type: rows per KV
  // head G*2B <= 2^23, batch x KV heads <= 2^31
  if (d.n_q_heads > kMaxQHeads || static_cast<int64_t>(d.batch) * d.n_kv_heads > (int64_t{1} << 31))
    return SIMSD_ERR_SHAPE;
  if (!(d.rope_base > 0.0) || !std::isfinite(d.rope_base) || !(d.softmax_scale >= 0.0f) ||
      !std::isfinite(d.softmax_scale))
    return SIMSD_ERR_SHAPE;
  if ((d.dtype != SIMSD_F32 && d.dtype != SIMSD_BF16) ||
      (d.mask_mode != SIMSD_MASK_TEMPORAL && d.mask_mode != SIMSD_MASK_FULL) ||
      (d.impl != SIMSD_IMPL_AUTO && d.impl != SIMSD_IMPL_VALU && d.impl != SIMSD_IMPL_MFMA) ||
      (d.rope_mode != SIMSD_ROPE_COPY && d.rope_mode != SIMSD_ROPE_SEQUENTIAL))
    return SIMSD_ERR_DTYPE;
  if (d.impl == SIMSD_IMPL_MFMA && d.dtype != SIMSD_BF16) return SIMSD_ERR_DTYPE;
  if (d.kv_chunk < 0 || d.kv_chunk % kKeyTile != 0) return SIMSD_ERR_KV_CHUNK;

  std::memset(&pl, 0, sizeof(pl));
  pl.NB = d.batch;
  pl.Hq = d.n_q_heads;
  pl.Hkv = d.n_kv_heads;
  pl.G = d.n_q_heads / d.n_kv_heads;
  pl.d = d.head_dim;
  pl.B = d.B;
  pl.twoB = 2 * d.B;
  pl.M = pl.G * pl.twoB;
  pl.p_max = d.p_max;
  pl.dtype = d.dtype;
  pl.mask_mode = d.mask_mode;
  pl.rope_base = d.rope_base;
  pl.log2_base = std::log2(d.rope_base);
  const float scale = d.softmax_scale > 0.0f ? d.softmax_scale : 1.0f / std::sqrt(static_cast<float>(d.head_dim));
  pl.scale_log2 = scale * kLog2e;
  pl.impl = d.impl == SIMSD_IMPL_AUTO ? (d.dtype == SIMSD_BF16 ? SIMSD_IMPL_MFMA : SIMSD_IMPL_VALU) : d.impl;
  pl.rope_seq = d.rope_mode == SIMSD_ROPE_SEQUENTIAL;
  pl.tab_rows = pl.rope_seq ? 2 * d.B : d.B;  // distinct block positions
  if (pl.impl == SIMSD_IMPL_MFMA && d.head_dim == 128 &&
      mfma_lds_bytes(128, 3, pl.tab_rows, 128, false, 0) + 1024 > kLdsPerCu) {
    // the RoPE table does not fit beside a 3-stage ring
    if (d.impl == SIMSD_IMPL_MFMA) return SIMSD_ERR_SHAPE;
    pl.impl = SIMSD_IMPL_VALU;
  }

  if (pl.impl == SIMSD_IMPL_MFMA) {
    // 16-row tiles per workgroup: 1, 2 or 4 (one per row wave), 8 (four row
    // waves of two tiles each, each tile's keys split over two waves) or, at
    // head dim 128, 16 (eight row waves of two tiles, each over all keys of
    // a tile); a workgroup runs 4 to 8 waves.  More rows take more row
    // groups, which read the same K/V split on one XCD at about the same
    // time.  Two groups of 128 rows pull every tile into two CUs' LDS, one
    // group of 256 into one (the grid then takes twice the splits): batch 8 x
    // 8192 keys, B = 32, 115-118 against 121-125 us per call.
    const int tiles = (pl.M + 15) / 16;
    const int max16 = pl.d == 128 ? 16 : 8;
    int nt16 = 1;
    while (nt16 < tiles && nt16 < max16) nt16 *= 2;
    // 256 rows only beside a 4-stage ring (their query rows borrow two
    // stages in the prologue; with three the step's registers spill), and
    // only where they pad no more rows than groups of 128 would: up to 256
    // rows, or a multiple of 256.
    if (nt16 == 16 && (mfma_lds_bytes(pl.d, 4, pl.tab_rows, 256, false, 0) + 1024 > kLdsPerCu ||
                       (tiles > 16 && tiles % 16 != 0)))
      nt16 = 8;
    const int rw = nt16 >= 16 ? 8 : (nt16 >= 8 ? 4 : nt16);
    pl.rowt = nt16 >= 8 ? 2 : 1;
    pl.ksplit = nt16 >= 16 ? 1 : (rw >= 4 ? 2 : 4);
    pl.threads = rw * pl.ksplit * 64;
    pl.rows_wg = nt16 * 16;
    // Four ring stages with the query rows staged in their own LDS region
    // when that fits; else the query rows borrow the last stage during the
    // prologue; else three stages.
    if (mfma_lds_bytes(pl.d, 4, pl.tab_rows, pl.rows_wg, true, 0) + 1024 <= kLdsPerCu) {
      pl.nstage = 4;
      pl.qsep = 1;
    } else {
      pl.nstage = mfma_lds_bytes(pl.d, 4, pl.tab_rows, pl.rows_wg, false, 0) + 1024 <= kLdsPerCu ? 4 : 3;
      pl.qsep = 0;
    }
    // The 2B block K/V rows take a region of their own (16-row multiples)
    // when it fits beside the ring without costing a workgroup per CU; the
    // ring then streams prompt tiles only, and the block keys are done while
    // the first of those are in flight.  Only beside a 4-stage ring: where
    // three stages are all that fit, such a region does not fit either.  Not
    // for 256 rows, whose waves take the block keys through the ring.
    if (pl.nstage == 4 && pl.twoB > 0 && pl.twoB <= kKeyTile && pl.rows_wg <= 128) {
      const int rows = (pl.twoB + 15) / 16 * 16;
      const size_t base = mfma_lds_bytes(pl.d, pl.nstage, pl.tab_rows, pl.rows_wg, pl.qsep != 0, 0) + 1024;
      const size_t with = mfma_lds_bytes(pl.d, pl.nstage, pl.tab_rows, pl.rows_wg, pl.qsep != 0, rows) + 1024;
      if (with <= kLdsPerCu && kLdsPerCu / with == kLdsPerCu / base) pl.blk_rows = rows;
    }
    // K/V tiles are read once per call.  When the cache region the call may
    // stream is at least the size of the last-level cache, none of it can
    // stay cached for the next call either, and the tiles are loaded with
    // the non-temporal bit: batch 32 x 4096 keys measured 95.2 -> 84.2 us
    // with identical outputs.  A region that fits keeps the default policy,
    // under which the next call over the same cache still finds it there
    // (batch 16 x 1024 keys: 20.2 us against 21.4 us non-temporal).
    // (in double: the product of the descriptor's extremes overflows int64)
    const double kv_bytes = static_cast<double>(pl.NB) * pl.Hkv * pl.p_max * pl.d * 2.0 * 2.0;
    pl.kv_stream = kv_bytes >= static_cast<double>(kLastLevelCache) ? 1 : 0;
  } else {
    pl.rowt = 1;
    pl.threads = 256;
    pl.rows_wg = 16;
  }
  pl.nrg = pl.M > 0 ? (pl.M + pl.rows_wg - 1) / pl.rows_wg : 1;

  // Split the prompt so that the grid fills every CU about once: one MFMA
  // workgroup per CU for head dim 128 (its LDS ring takes most of the CU),
  // two for 64; the VALU kernel aims at two per CU.  Splits are capped at
  // kMaxChunk keys: the grid gives every XCD the same share of every
  // sequence, so longer splits (fewer partials to merge) cost little tail.
  int64_t target = 2 * kNumCUs;
  if (pl.impl == SIMSD_IMPL_MFMA) {
    const size_t per_wg = mfma_lds_bytes(pl.d, pl.nstage, pl.tab_rows, pl.rows_wg, pl.qsep != 0, pl.blk_rows) + 1024;
    target = kNumCUs * static_cast<int64_t>(kLdsPerCu / per_wg);
  }
  const int64_t tiles_max = (static_cast<int64_t>(pl.p_max) + kKeyTile - 1) / kKeyTile;
  int64_t chunk;
  if (d.kv_chunk > 0) {
    chunk = d.kv_chunk;
  } else if (tiles_max == 0) {
    chunk = kKeyTile;
  } else {
    const int64_t per_split = static_cast<int64_t>(pl.NB) * pl.Hkv * pl.nrg;
    int64_t ns = per_split > 0 ? (target + per_split - 1) / per_split : 1;
    // Splits shorter than kMinSplitTiles tiles lose more to the merge launch
    // and the partial results than they gain in parallel streaming (batch
    // 16 x 1024 keys: 22.1 us in two splits of 8 tiles, 20.4 us in one).
    const int64_t ns_max = tiles_max / kMinSplitTiles > 1 ? tiles_max / kMinSplitTiles : 1;
    if (ns > ns_max) ns = ns_max;
    if (ns < 1) ns = 1;
    if (ns > tiles_max) ns = tiles_max;
    chunk = ((tiles_max + ns - 1) / ns) * kKeyTile;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
  }
  int64_t nsplit = pl.p_max > 0 ? (pl.p_max + chunk - 1) / chunk : 1;
  if (nsplit < 1) nsplit = 1;
  if (chunk > (1 << 30) || nsplit > (1 << 20)) return SIMSD_ERR_SHAPE;
  pl.chunk = static_cast<int>(chunk);
  pl.nsplit = static_cast<int>(nsplit);
  const int64_t grid = nsplit * pl.nrg * static_cast<int64_t>(pl.NB) * pl.Hkv;
  if (grid > 0x7fffffffLL) return SIMSD_ERR_SHAPE;
  // Longest work first when the grid takes more than one round of
  // workgroups: with ragged prompts the (sequence, split) items differ in
  // length, and in dispatch order long ones would start late (batch 64,
  // prompts 2048..16384, two splits: 1024 workgroups over 256 CUs took 487.5
  // us from the first start to the last end, tiles per CU 151..378 against
  // 280 on average).  Each workgroup ranks the items of its KV head itself,
  // so the ranking stays cheap only for a modest count of them.
  pl.lpt = 0;
  if (pl.impl == SIMSD_IMPL_MFMA) {
    const size_t per_wg = mfma_lds_bytes(pl.d, pl.nstage, pl.tab_rows, pl.rows_wg, pl.qsep != 0, pl.blk_rows) + 1024;
    const int64_t slots = kNumCUs * static_cast<int64_t>(kLdsPerCu / per_wg);
    const int64_t items = static_cast<int64_t>(pl.NB) * nsplit;
    if (grid > slots && items <= kLptMaxItems) pl.lpt = 1;
  }
  // the MFMA kernel's grid is (Hkv, NB * nrg, nsplit): y and z stay below 2^16
  if (pl.impl == SIMSD_IMPL_MFMA && (pl.nsplit > 65535 || static_cast<int64_t>(pl.NB) * pl.nrg > 65535))
    return SIMSD_ERR_SHAPE;
  // a bound the merge grid (at least 16 rows per workgroup) stays well within
  if (pl.nsplit > 1 && static_cast<int64_t>(pl.NB) * pl.twoB * pl.Hq > 4 * 0x7fffffffLL) return SIMSD_ERR_SHAPE;
  if (pl.nsplit > 1) {
    pl.part_o_floats = static_cast<size_t>(pl.NB) * pl.Hkv * pl.nsplit * pl.M * pl.d;
    pl.part_ml_floats = static_cast<size_t>(pl.NB) * pl.Hkv * pl.nsplit * pl.M * 2;
  }
  return SIMSD_OK;
}

}  // namespace

// Host validation of an accept_prefix call (no HIP call).  On success `need`
// is the scratch it streams through: nonzero only when a replacement can be
// drawn (next_token wanted, B and gamma > 0).
int accept_prefix_checks(const float* p_target, const float* q_draft, const int32_t* draft_tok, const int32_t* tau,
                         int32_t batch, int32_t B, int32_t gamma, int64_t vocab, const int32_t* n_accepted,
                         const int32_t* next_token, const int32_t* status, size_t* need) {
  *need = 0;
  // one grid row per sequence
  if (batch < 0 || batch > 65535 || B < 0 || B > 64 || vocab < 1 || vocab >= (int64_t{1} << 31))
    return SIMSD_ERR_SHAPE;
  if (gamma < 0 || gamma > B) return SIMSD_ERR_GAMMA;
  if (batch == 0) return SIMSD_OK;
  if (!n_accepted || (B > 0 && (!p_target || !q_draft || !draft_tok || !tau))) return SIMSD_ERR_NULL;
  if (!aligned(n_accepted, 4) || (next_token && !aligned(next_token, 4)) || (status && !aligned(status, 4)) ||
      (p_target && !aligned(p_target, 4)) || (q_draft && !aligned(q_draft, 4)) ||
      (draft_tok && !aligned(draft_tok, 4)) || (tau && !aligned(tau, 4)))
    return SIMSD_ERR_ALIGN;
  if (next_token && B > 0 && gamma > 0) *need = accept_workspace_bytes(batch, B, vocab);
  return SIMSD_OK;
}

namespace {

size_t workspace_bytes(const Plan& pl) {
  if (pl.nsplit <= 1 || pl.NB == 0 || pl.B == 0) return 0;
  return round_up(pl.part_o_floats * sizeof(float), 256) + round_up(pl.part_ml_floats * sizeof(float), 256);
}

}  // namespace
}  // namespace simsd

using namespace simsd;

namespace {
constexpr int kLinMaxK = 1 << 24;  // per-lane 32-bit byte offsets inside a 128-row tile

int linear_checks(const void* x, const void* w, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 16 || N % 16 != 0 || N > 0x7fffffff || K < 64 || K % 64 != 0 || K > kLinMaxK)
    return SIMSD_ERR_SHAPE;
  if ((M + 127) / 128 > 65535) return SIMSD_ERR_SHAPE;
  if (M > 0 && (!x || !w)) return SIMSD_ERR_NULL;
  if ((x && !aligned(x, 16)) || (w && !aligned(w, 16))) return SIMSD_ERR_ALIGN;
  return SIMSD_OK;
}
}  // namespace

extern "C" {

int simsd_abi_version(void) { return 9; }

const char* simsd_strerror(int code) {
  switch (code) {
    case SIMSD_OK: return "ok";
    case SIMSD_ERR_NULL: return "a required pointer is NULL";
    case SIMSD_ERR_SHAPE: return "invalid shape or size";
    case SIMSD_ERR_DTYPE: return "invalid dtype, mask mode or implementation";
    case SIMSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SIMSD_ERR_GAMMA: return "gamma outside [0, B]";
    case SIMSD_ERR_ALIGN: return "misaligned pointer";
    case SIMSD_ERR_HIP: return "HIP error at launch";
    case SIMSD_ERR_KV_CHUNK: return "kv_chunk must be a non-negative multiple of 64";
    case SIMSD_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point's fixed buffer";
    default: return "unknown error code";
  }
}

int simsd_verify_attn_workspace(const simsd_verify_desc* desc, size_t* bytes) {
  if (!desc || !bytes) return SIMSD_ERR_NULL;
  Plan pl;
  const int rc = make_plan(*desc, pl);
  if (rc) return rc;
  *bytes = workspace_bytes(pl);
  return SIMSD_OK;
}

int simsd_verify_plan_info(const simsd_verify_desc* desc, simsd_verify_plan* plan) {
  if (!desc || !plan) return SIMSD_ERR_NULL;
  Plan pl;
  const int rc = make_plan(*desc, pl);
  if (rc) return rc;
  const bool mfma = pl.impl == SIMSD_IMPL_MFMA;
  simsd_verify_plan o{};
  o.impl = pl.impl;
  o.threads = pl.threads;
  o.rows_wg = pl.rows_wg;
  o.row_groups = pl.nrg;
  o.ksplit = mfma ? pl.ksplit : 0;
  o.row_tiles = pl.rowt;
  o.nstage = mfma ? pl.nstage : 0;
  o.qsep = mfma ? pl.qsep : 0;
  o.blk_rows = mfma ? pl.blk_rows : 0;
  o.nsplit = pl.nsplit;
  o.chunk = pl.chunk;
  o.kv_stream = mfma ? pl.kv_stream : 0;
  o.lpt = mfma ? pl.lpt : 0;
  o.lds_bytes =
      mfma ? static_cast<int32_t>(mfma_lds_bytes(pl.d, pl.nstage, pl.tab_rows, pl.rows_wg, pl.qsep != 0, pl.blk_rows))
           : 0;
  *plan = o;
  return SIMSD_OK;
}

namespace {
int verify_attn_impl(const simsd_verify_desc* desc, const void* q_blk, const void* k_blk, const void* v_blk,
                     const void* k_cache, const void* v_cache, const int32_t* prompt_len, const int32_t* tau,
                     const int32_t* pos_d, void* out, float* lse, int32_t* status, void* workspace,
                     size_t workspace_bytes_in, void* stream, PassEvents ev) {
  if (!desc) return SIMSD_ERR_NULL;
  Plan pl;
  const int rc = make_plan(*desc, pl);
  if (rc) return rc;
  if (pl.NB == 0 || pl.B == 0) return SIMSD_OK;  // nothing to compute
  if (!q_blk || !k_blk || !v_blk || !tau || !out) return SIMSD_ERR_NULL;
  if (pl.p_max > 0 && (!k_cache || !v_cache)) return SIMSD_ERR_NULL;
  if (!aligned(q_blk, 16) || !aligned(k_blk, 16) || !aligned(v_blk, 16) || !aligned(out, 16) ||
      (k_cache && !aligned(k_cache, 16)) || (v_cache && !aligned(v_cache, 16)) || !aligned(tau, 4) ||
      (prompt_len && !aligned(prompt_len, 4)) || (pos_d && !aligned(pos_d, 4)) || (lse && !aligned(lse, 4)) ||
      (status && !aligned(status, 4)))
    return SIMSD_ERR_ALIGN;
  const size_t need = workspace_bytes(pl);
  if (need > 0) {
    if (!workspace || workspace_bytes_in < need) return SIMSD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SIMSD_ERR_ALIGN;
  }
  VerifyArgs a;
  a.q_blk = q_blk;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.prompt_len = prompt_len;
  a.tau = tau;
  a.pos_d = pos_d;
  a.out = out;
  a.lse = lse;
  a.status = status;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (need > 0) {
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         round_up(pl.part_o_floats * sizeof(float), 256));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the start event goes with the attention kernel, the stop event with the
  // last kernel of the pass (the merge when the prompt is split)
  const PassEvents first{ev.start, pl.nsplit > 1 ? nullptr : ev.stop};
  hipError_t e = pl.impl == SIMSD_IMPL_MFMA ? launch_verify_mfma(pl, a, s, first) : launch_verify_valu(pl, a, s, first);
  if (e != hipSuccess) return SIMSD_ERR_HIP;
  if (pl.nsplit > 1) {
    e = launch_merge(pl, a, s, PassEvents{nullptr, ev.stop});
    if (e != hipSuccess) return SIMSD_ERR_HIP;
  }
  return SIMSD_OK;
}
}  // namespace

int simsd_verify_attn(const simsd_verify_desc* desc, const void* q_blk, const void* k_blk, const void* v_blk,
                      const void* k_cache, const void* v_cache, const int32_t* prompt_len, const int32_t* tau,
                      const int32_t* pos_d, void* out, float* lse, int32_t* status, void* workspace,
                      size_t workspace_bytes_in, void* stream) {
  return verify_attn_impl(desc, q_blk, k_blk, v_blk, k_cache, v_cache, prompt_len, tau, pos_d, out, lse, status,
                          workspace, workspace_bytes_in, stream, PassEvents{});
}

int simsd_verify_attn_timed(const simsd_verify_desc* desc, const void* q_blk, const void* k_blk, const void* v_blk,
                            const void* k_cache, const void* v_cache, const int32_t* prompt_len, const int32_t* tau,
                            const int32_t* pos_d, void* out, float* lse, int32_t* status, void* workspace,
                            size_t workspace_bytes_in, void* stream, void* start_event, void* stop_event) {
  return verify_attn_impl(desc, q_blk, k_blk, v_blk, k_cache, v_cache, prompt_len, tau, pos_d, out, lse, status,
                          workspace, workspace_bytes_in, stream,
                          PassEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)});
}

int simsd_accept_prefix_workspace(int32_t batch, int32_t B, int64_t vocab, size_t* bytes) {
  if (!bytes) return SIMSD_ERR_NULL;
  if (batch < 0 || batch > 65535 || B < 0 || B > 64 || vocab < 1 || vocab >= (int64_t{1} << 31))
    return SIMSD_ERR_SHAPE;
  *bytes = accept_workspace_bytes(batch, B, vocab);
  return SIMSD_OK;
}

int simsd_accept_prefix(const float* p_target, const float* q_draft, const int32_t* draft_tok, const int32_t* tau,
                        int32_t batch, int32_t B, int32_t gamma, int64_t vocab, uint64_t seed, uint64_t offset,
                        int32_t* n_accepted, int32_t* next_token, int32_t* status, void* workspace,
                        size_t workspace_bytes_in, void* stream) {
  size_t need = 0;
  const int rc = accept_prefix_checks(p_target, q_draft, draft_tok, tau, batch, B, gamma, vocab, n_accepted,
                                      next_token, status, &need);
  if (rc != SIMSD_OK) return rc;
  if (batch == 0) return SIMSD_OK;
  if (need > 0) {
    if (!workspace || workspace_bytes_in < need) return SIMSD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SIMSD_ERR_ALIGN;
  }
  const hipError_t e = launch_accept(p_target, q_draft, draft_tok, tau, batch, B, gamma, vocab, seed, offset,
                                     n_accepted, next_token, status, workspace,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}

int simsd_accept_coupled_workspace(int32_t batch, int32_t B, int64_t vocab, size_t* bytes) {
  if (!bytes) return SIMSD_ERR_NULL;
  if (batch < 0 || B < 0 || B > 64 || vocab < 1 || vocab >= (int64_t{1} << 31)) return SIMSD_ERR_SHAPE;
  *bytes = coupled_workspace_bytes(batch, B, vocab);
  return SIMSD_OK;
}

int simsd_accept_coupled(const float* p_target, const float* noise_exp, const int32_t* draft_tok,
                         const int32_t* tau, int32_t batch, int32_t B, int32_t gamma, int64_t vocab,
                         int32_t* n_accepted, int32_t* next_token, int32_t* status, void* workspace,
                         size_t workspace_bytes_in, void* stream) {
  if (batch < 0 || B < 0 || B > 64 || vocab < 1 || vocab >= (int64_t{1} << 31)) return SIMSD_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * gamma > 0x7fffffff || coupled_chunks(vocab) > 65535) return SIMSD_ERR_SHAPE;
  if (gamma < 0 || gamma > B) return SIMSD_ERR_GAMMA;
  if (batch == 0) return SIMSD_OK;
  if (!n_accepted || (B > 0 && (!p_target || !noise_exp || !draft_tok || !tau))) return SIMSD_ERR_NULL;
  if (!aligned(n_accepted, 4) || (next_token && !aligned(next_token, 4)) || (status && !aligned(status, 4)) ||
      (p_target && !aligned(p_target, 16)) || (noise_exp && !aligned(noise_exp, 16)) ||
      (draft_tok && !aligned(draft_tok, 4)) || (tau && !aligned(tau, 4)))
    return SIMSD_ERR_ALIGN;
  const size_t need = coupled_workspace_bytes(batch, B, vocab);
  if (!workspace || workspace_bytes_in < need) return SIMSD_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return SIMSD_ERR_ALIGN;
  const hipError_t e = launch_accept_coupled(p_target, noise_exp, draft_tok, tau, batch, B, gamma, vocab, n_accepted,
                                             next_token, status, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}

int simsd_linear(const void* x, const void* w, int64_t M, int32_t N, int32_t K, void* y, void* stream) {
  const int rc = linear_checks(x, w, M, N, K);
  if (rc != SIMSD_OK) return rc;
  if (M == 0) return SIMSD_OK;
  if (!y) return SIMSD_ERR_NULL;
  if (!aligned(y, 16)) return SIMSD_ERR_ALIGN;
  uint16_t* out = static_cast<uint16_t*>(y);
  const hipError_t e = launch_linear(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), M, N, K, N, N,
                                     out, N, out, N, out, N, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}

int simsd_qkv_proj(const void* x, const void* w_qkv, int64_t M, int32_t H, int32_t Hq, int32_t Hkv, int32_t d,
                   void* q, void* k, void* v, void* stream) {
  if (Hq < 1 || Hkv < 1 || d < 16 || d % 16 != 0) return SIMSD_ERR_SHAPE;
  const int64_t nq = static_cast<int64_t>(Hq) * d, nk = static_cast<int64_t>(Hkv) * d;
  const int64_t N = nq + 2 * nk;
  const int rc = linear_checks(x, w_qkv, M, N, H);
  if (rc != SIMSD_OK) return rc;
  if (M == 0) return SIMSD_OK;
  if (!q || !k || !v) return SIMSD_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return SIMSD_ERR_ALIGN;
  const hipError_t e = launch_linear(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_qkv), M,
                                     static_cast<int>(N), H, static_cast<int>(nq), static_cast<int>(nq + nk),
                                     static_cast<uint16_t*>(q), static_cast<int>(nq), static_cast<uint16_t*>(k),
                                     static_cast<int>(nk), static_cast<uint16_t*>(v), static_cast<int>(nk),
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SIMSD_OK : SIMSD_ERR_HIP;
}

int simsd_commit(const int32_t* tau, const int32_t* draft_tok, const int32_t* n_accepted, const int32_t* next_token,
                 int32_t batch, int32_t B, uint64_t* committed, int32_t* block_tok, void* stream) {
  if (batch < 0 || B < 0 || B > 64) return SIMSD_ERR_SHAPE;
  if (batch == 0 || B == 0) return SIMSD_OK;
  if (!tau || !draft_tok || !n_accepted || !committed || !block_tok) return SIMSD_ERR_NULL;
  if (!aligned(tau, 4) || !aligned(draft_tok, 4) || !aligned(n_accepted, 4) || (next_token && !aligned(next_token, 4)) ||
      !aligned(committed, 8) || !aligned(block_tok, 4))
    return SIMSD_ERR_ALIGN;
  return launch_commit(tau, draft_tok, n_accepted, next_token, batch, B, committed, block_tok,
                       static_cast<hipStream_t>(stream)) == hipSuccess
             ? SIMSD_OK
             : SIMSD_ERR_HIP;
}

int simsd_next_round(const uint64_t* committed, const int32_t* block_tok, const int32_t* rank,
                     const int32_t* draft_tok, int32_t batch, int32_t B, int32_t* tau_out, int32_t* tok_out,
                     void* stream) {
  if (batch < 0 || B < 0 || B > 64) return SIMSD_ERR_SHAPE;
  if (batch == 0 || B == 0) return SIMSD_OK;
  if (!committed || !block_tok || !draft_tok || !tau_out || !tok_out) return SIMSD_ERR_NULL;
  if (!aligned(committed, 8) || !aligned(block_tok, 4) || (rank && !aligned(rank, 4)) || !aligned(draft_tok, 4) ||
      !aligned(tau_out, 4) || !aligned(tok_out, 4))
    return SIMSD_ERR_ALIGN;
  return launch_next_round(committed, block_tok, rank, draft_tok, batch, B, tau_out, tok_out,
                           static_cast<hipStream_t>(stream)) == hipSuccess
             ? SIMSD_OK
             : SIMSD_ERR_HIP;
}

int simsd_append_kv(const simsd_verify_desc* desc, const void* k_blk, const void* v_blk, const int32_t* pos_d,
                    const uint64_t* committed, int32_t* prompt_len, void* k_cache, void* v_cache, int32_t* status,
                    void* stream) {
  if (!desc) return SIMSD_ERR_NULL;
  Plan pl;
  const int rc = make_plan(*desc, pl);
  if (rc != SIMSD_OK) return rc;
  if (pl.NB == 0 || pl.B == 0) return SIMSD_OK;
  if (pl.NB > 65535) return SIMSD_ERR_SHAPE;  // one grid row per sequence
  if (!k_blk || !v_blk || !prompt_len || !k_cache || !v_cache) return SIMSD_ERR_NULL;
  if (!aligned(k_blk, 16) || !aligned(v_blk, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(prompt_len, 4) || (pos_d && !aligned(pos_d, 4)) || (committed && !aligned(committed, 8)) ||
      (status && !aligned(status, 4)))
    return SIMSD_ERR_ALIGN;
  return launch_append_kv(pl, k_blk, v_blk, pos_d, committed, prompt_len, k_cache, v_cache, status,
                          static_cast<hipStream_t>(stream)) == hipSuccess
             ? SIMSD_OK
             : SIMSD_ERR_HIP;
}

int simsd_debug_mask(const int32_t* tau, int32_t batch, int32_t B, int32_t mask_mode, uint64_t* bits,
                     void* stream) {
  if (batch < 0 || B < 0 || B > 64) return SIMSD_ERR_SHAPE;
  if (mask_mode != SIMSD_MASK_TEMPORAL && mask_mode != SIMSD_MASK_FULL) return SIMSD_ERR_DTYPE;
  if (batch == 0 || B == 0) return SIMSD_OK;
  if (!tau || !bits) return SIMSD_ERR_NULL;
  if (!aligned(tau, 4) || !aligned(bits, 8)) return SIMSD_ERR_ALIGN;
  return launch_debug_mask(tau, batch, B, mask_mode, bits, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SIMSD_OK
             : SIMSD_ERR_HIP;
}

int simsd_debug_rope(const simsd_verify_desc* desc, const void* q_blk, const void* k_blk,
                     const int32_t* prompt_len, const int32_t* pos_d, void* q_rot, void* k_rot, void* stream) {
  if (!desc) return SIMSD_ERR_NULL;
  Plan pl;
  const int rc = make_plan(*desc, pl);
  if (rc) return rc;
  if (pl.NB == 0 || pl.B == 0) return SIMSD_OK;
  if (static_cast<int64_t>(pl.NB) * pl.twoB > 0x7fffffffLL) return SIMSD_ERR_SHAPE;  // one workgroup per block row
  if (!q_blk || !k_blk || !q_rot || !k_rot) return SIMSD_ERR_NULL;
  if (!aligned(q_blk, 16) || !aligned(k_blk, 16) || !aligned(q_rot, 16) || !aligned(k_rot, 16) ||
      (prompt_len && !aligned(prompt_len, 4)) || (pos_d && !aligned(pos_d, 4)))
    return SIMSD_ERR_ALIGN;
  return launch_debug_rope(pl, q_blk, k_blk, prompt_len, pos_d, q_rot, k_rot, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SIMSD_OK
             : SIMSD_ERR_HIP;
}

}  // extern "C"
