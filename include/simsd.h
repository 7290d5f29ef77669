/*
 * simsd.h -- C ABI of the SimSD verification hot path on MI355X (gfx950).
 *
 * The method (page "SimSD - Simple Speculative Decoding in Diffusion
 * Language Models", gist.science summary of arXiv 2606.02544):
 *   - section 1, input layout: after the prompt come a data section D of B
 *     reference tokens and a mask section D~ of B [MASK] slots; D_k and D~_k
 *     stand for the same response position, D_k gives context and D~_k is
 *     where the logit is read;
 *   - section 2, temporal attention mask: a permutation assigns every
 *     response position a stage tau in 1..B; D~_i attends to D_j only when
 *     tau(j) < tau(i) and to D~_j when tau(j) >= tau(i);
 *   - section 3, position encoding alignment: D~_k reuses the RoPE index of
 *     D_k (the "RoPE copy"; "Experimental results" reports the ablation that
 *     drops it, available here as SIMSD_ROPE_SEQUENTIAL);
 *   - section 4, pipeline: one target forward computes the logits of all
 *     candidates under that mask; acceptance is standard rejection sampling
 *     walked in the drafted temporal order, committing the longest accepted
 *     prefix, and the process repeats.
 *
 * Stage label 0 (read here for the repeated rounds of one block) marks a
 * response position committed in an earlier round: its token sits in D as
 * context, every mask slot sees it (0 is below every stage) and no
 * acceptance walk visits it.  The open positions carry stages 1..m.
 *
 * Conventions where the page is silent: every block row sees the whole
 * prompt prefix [0, P_b); a data row D_i sees D_j when tau(j) <= tau(i) and
 * no mask slot; RoPE is rotate-half with frequencies base^(-2f/d); the
 * softmax scale defaults to 1/sqrt(d); query head h reads KV head
 * h / (Hq/Hkv).
 *
 * General rules for every entry point:
 *   - All array arguments are device pointers to contiguous, caller-owned
 *     memory, 16-byte aligned (4-byte for int32 arrays), except the
 *     descriptor and the size outputs of the *_workspace queries, which are
 *     host pointers.  Inputs are never written; the KV cache is read-only
 *     for every call except simsd_append_kv, which appends committed blocks
 *     (buffers documented as in/out are updated in place).
 *   - The library allocates nothing.  Scratch memory is a caller-provided
 *     workspace sized by the matching *_workspace query (except for
 *     simsd_accept_prefix_noalloc, whose scratch is a fixed device array).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the legacy
 *     default stream) and never synchronise.  The library keeps no state
 *     between calls beyond a kernel attribute (the dynamic LDS limit) that
 *     is set once per kernel and device under std::call_once, so concurrent
 *     calls from several host threads, on different streams with disjoint
 *     buffers and workspaces, are safe.
 *   - A negative return code means the host rejected the arguments before
 *     any HIP call: nothing was launched.  SIMSD_ERR_HIP means a launch was
 *     attempted and HIP reported an error.
 *   - Per-sequence faults found on the device are written to status[b]
 *     (0 = valid) when `status` is not NULL; a faulted sequence's outputs
 *     are defined below.
 */
#ifndef SIMSD_H
#define SIMSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------------- */
#define SIMSD_OK               0
#define SIMSD_ERR_NULL        (-1) /* a required pointer is NULL */
#define SIMSD_ERR_SHAPE       (-2) /* negative size, Hq % Hkv != 0, Hq > 65536, head_dim not 64/128,
                                       B > 64, batch x Hkv > 2^31;
                                       bf16: prompt splits or batch x ceil(Hq/Hkv*2B/128)
                                       above 65535 */
#define SIMSD_ERR_DTYPE       (-3) /* unknown dtype, mask mode, RoPE mode or implementation */
#define SIMSD_ERR_WORKSPACE   (-4) /* workspace NULL or smaller than the query says */
#define SIMSD_ERR_GAMMA       (-5) /* gamma outside [0, B] */
#define SIMSD_ERR_ALIGN       (-6) /* pointer not aligned as documented */
#define SIMSD_ERR_HIP         (-7) /* HIP reported an error at launch */
#define SIMSD_ERR_KV_CHUNK    (-8) /* kv_chunk not a non-negative multiple of 64 */
#define SIMSD_ERR_SCRATCH     (-9) /* needs more than the no-allocation entry point's fixed
                                       4 MiB scratch */

/* ---- per-sequence device status flags (OR-ed together) --------------------------- */
#define SIMSD_ST_TAU_RANGE     1   /* a stage label outside 0..B */
#define SIMSD_ST_TAU_NOT_PERM  2   /* the nonzero labels are not 1..m (acceptance only) */
#define SIMSD_ST_PROMPT_LEN    4   /* prompt_len[b] outside [0, p_max] */
#define SIMSD_ST_TOKEN_RANGE   8   /* a walked draft token outside [0, vocab) */
#define SIMSD_ST_POS_NEG      16   /* a negative RoPE position in pos_d */

typedef enum { SIMSD_F32 = 0, SIMSD_BF16 = 1 } simsd_dtype;

/* SIMSD_MASK_FULL makes every prompt and block column visible (plain
 * bidirectional attention over [prompt; D; D~]); it exists to test the
 * temporal mask against that special case. */
typedef enum { SIMSD_MASK_TEMPORAL = 0, SIMSD_MASK_FULL = 1 } simsd_mask_mode;

/* Kernel family.  AUTO picks the MFMA kernel for bf16 and the VALU kernel for
 * fp32.  VALU works for both dtypes (it is the fp32 path and a cross-check). */
typedef enum { SIMSD_IMPL_AUTO = 0, SIMSD_IMPL_VALU = 1, SIMSD_IMPL_MFMA = 2 } simsd_impl;

/* RoPE index of the mask slots.  COPY is the method (section 3): D~_k
 * takes the index of D_k.  SEQUENTIAL is the ablation without the copy
 * ("Experimental results"), read here as the 2B block rows taking
 * consecutive indices in layout order: D~_k at pos(D_k) + B (by default
 * D_k at P_b + k and D~_k at P_b + B + k).  The MFMA kernel keeps a RoPE
 * table of one entry per distinct block position in LDS; at head_dim 128
 * and B = 63 or 64 the SEQUENTIAL table does not fit beside a 3-stage ring,
 * and AUTO then runs the VALU kernel (an explicit MFMA request is
 * SIMSD_ERR_SHAPE). */
typedef enum { SIMSD_ROPE_COPY = 0, SIMSD_ROPE_SEQUENTIAL = 1 } simsd_rope_mode;

typedef struct {
  int32_t batch;        /* NB >= 0, NB * Hkv <= 2^31 */
  int32_t n_q_heads;    /* Hq in 1..65536 */
  int32_t n_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t B;            /* section length 0..64; B == 0 is a valid no-op */
  int32_t p_max;        /* KV-cache capacity per (sequence, KV head), >= 0 */
  int32_t dtype;        /* simsd_dtype of q/k/v, cache and out */
  int32_t mask_mode;    /* simsd_mask_mode */
  int32_t impl;         /* simsd_impl */
  int32_t kv_chunk;     /* prompt keys per split, multiple of 64; 0 = library picks */
  double rope_base;     /* RoPE base, > 0 (1e4, 1e6, ...) */
  float softmax_scale;  /* 0 => 1/sqrt(d) */
  int32_t rope_mode;    /* simsd_rope_mode */
} simsd_verify_desc;

/* Workspace bytes that simsd_verify_attn needs for `desc` (may be 0).
 * Host only; no HIP call.  Returns SIMSD_OK or a negative code. */
int simsd_verify_attn_workspace(const simsd_verify_desc* desc, size_t* bytes);

/* How simsd_verify_attn would run `desc`: the kernel, the workgroup shape,
 * the LDS layout choices and the prompt split.  Host only; no HIP call.
 * Filled on SIMSD_OK; a descriptor that simsd_verify_attn would reject
 * returns the same negative code and leaves *plan unchanged. */
typedef struct {
  int32_t impl;       /* SIMSD_IMPL_VALU or SIMSD_IMPL_MFMA, after AUTO is resolved */
  int32_t threads;    /* threads per workgroup */
  int32_t rows_wg;    /* query rows per workgroup (16-row multiples) */
  int32_t row_groups; /* workgroups sharing one (sequence, KV head, split) */
  int32_t ksplit;     /* MFMA: waves that share the keys of a tile (else 0) */
  int32_t row_tiles;  /* 16-row tiles per wave */
  int32_t nstage;     /* MFMA: LDS ring stages (else 0) */
  int32_t qsep;       /* MFMA: 1 = query rows staged in their own LDS region */
  int32_t blk_rows;   /* MFMA: rows of the LDS region holding the 2B block K
                         rows (and as many V rows), 0 = block keys streamed
                         through the ring */
  int32_t nsplit;     /* prompt splits per (sequence, KV head) */
  int32_t chunk;      /* prompt keys per split */
  int32_t lds_bytes;  /* MFMA: dynamic LDS per workgroup (else 0) */
  int32_t kv_stream;  /* MFMA: 1 = the prompt K/V tiles are loaded non-temporal,
                         chosen when NB * Hkv * p_max * d * 2 * 2 bytes (K and V
                         in bf16) reach 256 MiB, the last-level cache (else 0) */
  int32_t lpt;        /* MFMA: 1 = the workgroups of a KV head take their
                         (sequence, split) items longest first by prompt
                         length, chosen when the grid needs more than one
                         round of workgroups and a KV head has at most 256
                         items (else 0) */
} simsd_verify_plan;

int simsd_verify_plan_info(const simsd_verify_desc* desc, simsd_verify_plan* plan);

/* The verification attention of the SimSD pass (sections 1-3 above).
 *
 *  q_blk   [NB][2B][Hq][d]   rows 0..B-1 are D_0..D_{B-1}, rows B..2B-1 are
 *                            D~_0..D~_{B-1}; not yet rotated.
 *  k_blk   [NB][2B][Hkv][d]  same row order, not yet rotated.
 *  v_blk   [NB][2B][Hkv][d]
 *  k_cache [NB][Hkv][p_max][d] prompt keys at positions 0..P_b-1, already
 *                            rotated (RoPE applied when they were cached).
 *  v_cache [NB][Hkv][p_max][d]
 *          (the caches may be NULL when p_max == 0)
 *  prompt_len [NB] int32 P_b in [0, p_max], or NULL meaning p_max.
 *  tau     [NB][B] int32 stage labels 0..B (a permutation of 1..B, or 0
 *                            for committed positions and 1..m for the
 *                            others; ties are tolerated: the mask rules
 *                            stay well defined).
 *  pos_d   [NB][B] int32 RoPE position of D_k, or NULL meaning P_b + k;
 *                            D~_k takes the same position (COPY) or that
 *                            position + B (SEQUENTIAL).
 *  out     [NB][2B][Hq][d]   softmax-weighted values, in `dtype`.
 *  lse     [NB][2B][Hq] fp32 natural-log sum of exp of the scaled scores over
 *                            the visible set, or NULL.
 *  status  [NB] int32, or NULL: SIMSD_ST_TAU_RANGE, SIMSD_ST_PROMPT_LEN,
 *                            SIMSD_ST_POS_NEG.  A faulted sequence gets zero
 *                            `out` rows and lse = -inf.
 *  workspace / workspace_bytes: scratch of at least the queried size (may be
 *                            NULL when the query returned 0).
 *
 * Errors: SIMSD_ERR_NULL, _SHAPE, _DTYPE, _WORKSPACE, _ALIGN, _KV_CHUNK,
 * _HIP as described above. */
int simsd_verify_attn(const simsd_verify_desc* desc,
                      const void* q_blk, const void* k_blk, const void* v_blk,
                      const void* k_cache, const void* v_cache,
                      const int32_t* prompt_len, const int32_t* tau, const int32_t* pos_d,
                      void* out, float* lse, int32_t* status,
                      void* workspace, size_t workspace_bytes, void* stream);

/* simsd_verify_attn with the caller's HIP events (hipEvent_t, created with
 * timing enabled, or NULL) bound to the pass's own kernels: `start_event`
 * takes the start time of the attention kernel and `stop_event` the end time
 * of the last kernel of the pass (the split merge when the prompt is split),
 * both recorded from the dispatches themselves (hipExtLaunchKernel), so their
 * elapsed time is the pass's kernel time, without the marker packets that
 * hipEventRecord puts on the stream before and after.  For timing only; the
 * arguments, results and errors are those of simsd_verify_attn. */
int simsd_verify_attn_timed(const simsd_verify_desc* desc,
                            const void* q_blk, const void* k_blk, const void* v_blk,
                            const void* k_cache, const void* v_cache,
                            const int32_t* prompt_len, const int32_t* tau, const int32_t* pos_d,
                            void* out, float* lse, int32_t* status,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* start_event, void* stop_event);

/* Workspace bytes that simsd_accept_prefix needs when next_token is not NULL
 * and B, gamma > 0 (host only, no HIP call): fp64 partial sums of the
 * rejected rows and a record of each sequence's walk (0 when B == 0).  The
 * workspace needs no initialisation; two calls that overlap in time must not
 * share one. */
int simsd_accept_prefix_workspace(int32_t batch, int32_t B, int64_t vocab, size_t* bytes);

/* Acceptance walk in tau order (section 4 above, read as textbook rejection
 * sampling with residual resampling).  Two kernel launches when a
 * replacement can be drawn (chunk sums of the rejected rows, then the draw),
 * one otherwise.
 *
 *  p_target [NB][B][V] fp32  target probabilities read at the D~_k slot,
 *                            row k = response position k.
 *  q_draft  [NB][B][V] fp32  draft probabilities for position k.
 *  draft_tok [NB][B] int32   token placed in D_k.
 *  tau      [NB][B] int32    0 for committed positions, a permutation of
 *                            1..m over the m open ones (m = B in a first
 *                            round).
 *  gamma    0..B             stages walked: stage t = 1..min(gamma, m) is
 *                            position k_t with tau[k_t] = t.
 *  seed, offset              Philox4x64-10 (Salmon et al., SC'11) key
 *                            (seed, 0); the acceptance uniform of stage t of
 *                            sequence b is the top 24 bits of word 0 at
 *                            counter (b, t, 0, offset); stage t accepts iff
 *                            u * q[x] < p[x], evaluated exactly in fp64.
 *  n_accepted [NB] int32     accepted prefix length 0..min(gamma, m).
 *  next_token [NB] int32     or NULL: at the first rejected stage n+1, a
 *                            draw from max(0, p - q) (fp64 prefix sums; the
 *                            uniform is the top 53 bits of word 0 at counter
 *                            (b, n+1, 1, offset)); from p itself when that
 *                            residual is all zero; -1 when
 *                            n == min(gamma, m).
 *  status   [NB] int32 or NULL: SIMSD_ST_TAU_RANGE, SIMSD_ST_TAU_NOT_PERM,
 *                            SIMSD_ST_TOKEN_RANGE; a faulted sequence gets
 *                            n_accepted = next_token = -1.
 *  workspace / workspace_bytes: at least simsd_accept_prefix_workspace bytes,
 *                            256-byte aligned, when next_token is not NULL and
 *                            B, gamma > 0 (otherwise it is never touched and
 *                            may be NULL).
 *
 * Errors: SIMSD_ERR_NULL, _SHAPE (negative sizes, batch > 65535, B > 64,
 * vocab < 1 or >= 2^31), _GAMMA, _WORKSPACE, _ALIGN, _HIP. */
int simsd_accept_prefix(const float* p_target, const float* q_draft,
                        const int32_t* draft_tok, const int32_t* tau,
                        int32_t batch, int32_t B, int32_t gamma, int64_t vocab,
                        uint64_t seed, uint64_t offset,
                        int32_t* n_accepted, int32_t* next_token, int32_t* status,
                        void* workspace, size_t workspace_bytes, void* stream);

/* simsd_accept_prefix without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, outputs and errors as
 * simsd_accept_prefix; the scratch that call keeps in the workspace (the
 * chunk sums and walk records, simsd_accept_prefix_workspace bytes) lives in
 * a fixed 4 MiB device array of the library instead, one per GPU, held until
 * the process ends.  Nothing in it needs to start at zero (every entry is
 * written before it is read).  A call that needs more than 4 MiB (about
 * 1700 sequences at vocab 151936) returns SIMSD_ERR_SCRATCH before any HIP
 * call.  The array of the current device is used: `stream` must belong to
 * it.  All calls on one GPU share that array, so two calls that overlap in
 * time on one GPU (different streams, or different host threads) race;
 * calls in order on one stream do not.  The entry point itself allocates
 * nothing: no hipMalloc, hipFree or allocating library routine (the first
 * call on a device looks the array's address up once). */
int simsd_accept_prefix_noalloc(const float* p_target, const float* q_draft,
                                const int32_t* draft_tok, const int32_t* tau,
                                int32_t batch, int32_t B, int32_t gamma, int64_t vocab,
                                uint64_t seed, uint64_t offset,
                                int32_t* n_accepted, int32_t* next_token, int32_t* status,
                                void* stream);

/* Workspace bytes that simsd_accept_coupled needs (host only, no HIP call):
 * one (p, E, index) winner per 8192-element chunk of every walked row.  It
 * needs no initialisation; two calls that overlap in time must not share one. */
int simsd_accept_coupled_workspace(int32_t batch, int32_t B, int64_t vocab, size_t* bytes);

/* Coupled-noise acceptance (SPOT page, "how to use it" section: the drafter
 * and the target share one Gumbel noise table per output position; given the
 * noise the target's next state is a deterministic argmax, and a draft is
 * kept exactly when it equals that argmax), walked in tau order as above.
 *
 *  p_target  [NB][B][V] fp32  target probabilities for response position k.
 *  noise_exp [NB][B][V] fp32  the shared noise in exponential form,
 *                             E = exp(-g) for the Gumbel value g of (k, v):
 *                             finite and > 0 (an Exp(1) draw).  The caller
 *                             keys the table by output position; row k is
 *                             the table of the position drafted into D_k.
 *  draft_tok [NB][B] int32    token placed in D_k (the drafter's noised
 *                             argmax over its own distribution).
 *  tau       [NB][B] int32    0 for committed positions, a permutation of
 *                             1..m over the m open ones.
 *  gamma     0..B             stages walked: t = 1..min(gamma, m), stage t is
 *                             position k_t with tau[k_t] = t.
 *  The target token of a row is argmax_v p_v / E_v (= argmax ln p_v + g_v),
 *  decided exactly (p_a * E_b against p_b * E_a in fp64, exact for fp32
 *  inputs; equal scores to the smaller index; p_v <= 0 never wins, a row
 *  without a positive p_v has none: -1).
 *  n_accepted [NB] int32      longest prefix of stages whose draft equals the
 *                             target token, 0..min(gamma, m).
 *  next_token [NB] int32      or NULL: the target token of stage n+1 (a draw
 *                             from p once the noise is marginalised); -1 when
 *                             n == min(gamma, m).
 *  status    [NB] int32 or NULL: SIMSD_ST_TAU_RANGE, SIMSD_ST_TAU_NOT_PERM,
 *                             SIMSD_ST_TOKEN_RANGE; a faulted sequence gets
 *                             n_accepted = next_token = -1.
 *  workspace / workspace_bytes: at least simsd_accept_coupled_workspace
 *                             bytes, 256-byte aligned.
 * p_target and noise_exp are 16-byte aligned.
 *
 * Errors: SIMSD_ERR_NULL, _SHAPE (negative sizes, B > 64, vocab < 1 or
 * > 65535 * 8192, batch * gamma >= 2^31), _GAMMA, _WORKSPACE, _ALIGN, _HIP. */
int simsd_accept_coupled(const float* p_target, const float* noise_exp, const int32_t* draft_tok,
                         const int32_t* tau, int32_t batch, int32_t B, int32_t gamma, int64_t vocab,
                         int32_t* n_accepted, int32_t* next_token, int32_t* status, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Export the block visibility that the attention kernels compute from tau,
 * through the same device function (section 2 rules plus the data-row
 * convention).  bits [NB][2B][2] uint64: word 0 bit j = row sees D_j, word 1
 * bit j = row sees D~_j.  Errors: SIMSD_ERR_NULL, _SHAPE, _DTYPE, _HIP. */
int simsd_debug_mask(const int32_t* tau, int32_t batch, int32_t B, int32_t mask_mode,
                     uint64_t* bits, void* stream);

/* Export the RoPE-copy rotation of the block rows exactly as the attention
 * kernels feed it to their dot products (section 3): q_rot [NB][2B][Hq][d]
 * and k_rot [NB][2B][Hkv][d] in desc->dtype.  Uses desc's shape, dtype and
 * rope_base.  Errors as for simsd_verify_attn. */
int simsd_debug_rope(const simsd_verify_desc* desc, const void* q_blk, const void* k_blk,
                     const int32_t* prompt_len, const int32_t* pos_d,
                     void* q_rot, void* k_rot, void* stream);

/* ---- projections around the attention ---------------------------------------------
 * Section 4: the target model checks every candidate in ONE forward pass over
 * the paired layout.  Inside each layer of that pass the attention above is
 * fed by a linear projection of the block rows' hidden states to queries,
 * keys and values and followed by the output projection.  Both are
 * y = x W^T (the nn.Linear convention: W is [out][in], row-major, no bias),
 * bf16 operands, fp32 accumulation, bf16 results rounded to nearest even.
 * RoPE is not applied here: simsd_verify_attn rotates q and k (its RoPE copy).
 *
 * Shapes: M >= 0 rows (M == 0 is a valid no-op); K (the input width) a
 * multiple of 64, at most 2^24; N (the output width) a multiple of 16;
 * ceil(M/128) <= 65535.  x, W and the outputs are 16-byte aligned device
 * memory.  Errors: SIMSD_ERR_SHAPE, _NULL, _ALIGN, _HIP.  No workspace. */

/* y [M][N] = x [M][K] * w [N][K]^T.  Used as the output projection: x is
 * the attention output [NB*2B][Hq*d] and w is [H][Hq*d]. */
int simsd_linear(const void* x, const void* w, int64_t M, int32_t N, int32_t K, void* y, void* stream);

/* Fused QKV projection of the block rows straight into the layouts
 * simsd_verify_attn reads.  x [M][H] holds the hidden states of the 2B block
 * rows of every sequence in layout order (D_0..D_{B-1}, D~_0..D~_{B-1}),
 * sequence after sequence, so M = NB*2B.  w_qkv [(Hq + 2*Hkv)*d][H]: the Hq
 * query heads (d rows each), then the Hkv key heads, then the Hkv value
 * heads.  Writes q [M][Hq][d], k [M][Hkv][d], v [M][Hkv][d] (that is
 * q_blk [NB][2B][Hq][d] and k_blk, v_blk [NB][2B][Hkv][d]).  d a multiple
 * of 16, H a multiple of 64. */
int simsd_qkv_proj(const void* x, const void* w_qkv, int64_t M, int32_t H, int32_t Hq, int32_t Hkv, int32_t d,
                   void* q, void* k, void* v, void* stream);

/* ---- the commit step between rounds ---------------------------------------------
 * Section 4: the longest accepted prefix is committed and the process
 * repeats; "Key contributions" item 3: the method runs with a KV cache and
 * blockwise decoding.  The block state of a sequence is a committed mask
 * (bit k: response position k is committed) and the committed token of each
 * position. */

/* Commit one round.  For every sequence b with n_accepted[b] >= 0: the
 * positions of stages 1..n_accepted[b] take their drafted tokens, and when
 * next_token (may be NULL) holds a token >= 0 the position of stage n+1 takes
 * it; block_tok[b][k] receives the token and bit k of committed[b] is set
 * (bits set by earlier rounds stay set).  Sequences with n_accepted[b] < 0
 * (a faulted round) are left unchanged.
 *  tau, draft_tok [NB][B] int32, n_accepted, next_token [NB] int32 (the
 *  outputs of simsd_accept_prefix / simsd_accept_coupled); committed [NB]
 *  uint64 (in/out, 8-byte aligned); block_tok [NB][B] int32 (in/out).
 * Errors: SIMSD_ERR_SHAPE (B outside 0..64), _NULL, _ALIGN, _HIP. */
int simsd_commit(const int32_t* tau, const int32_t* draft_tok, const int32_t* n_accepted, const int32_t* next_token,
                 int32_t batch, int32_t B, uint64_t* committed, int32_t* block_tok, void* stream);

/* Stage labels and data tokens of the block's next round.  Position k of
 * sequence b gets tau 0 and token block_tok[b][k] when bit k of committed[b]
 * is set; the open positions get stages 1..m in the drafter's order (rank,
 * smaller first, equal ranks by position; position order when rank is NULL)
 * and the drafter's tokens draft_tok[b][k].  The drafter itself (its tokens
 * and order) is the caller's.
 *  committed [NB] uint64 (8-byte aligned), block_tok, rank, draft_tok
 *  [NB][B] int32 in; tau_out, tok_out [NB][B] int32 out.
 * Errors: SIMSD_ERR_SHAPE (batch < 0, B outside 0..64), _NULL, _ALIGN,
 * _HIP. */
int simsd_next_round(const uint64_t* committed, const int32_t* block_tok, const int32_t* rank,
                     const int32_t* draft_tok, int32_t batch, int32_t B, int32_t* tau_out, int32_t* tok_out,
                     void* stream);

/* Append finished blocks to the KV cache.  For every sequence whose
 * committed[b] has all B bits set (every sequence when committed is NULL):
 * key rows D_0..D_{B-1} of k_blk, rotated at their RoPE positions (pos_d, or
 * P_b + k when NULL) with the rounding of simsd_verify_attn, are written to
 * k_cache[b][h][P_b + k], the value rows to v_cache, and prompt_len[b] grows
 * by B.  Uses desc's shape, dtype and rope_base (desc->p_max is the cache
 * capacity).  status [NB] (or NULL): 0, or SIMSD_ST_PROMPT_LEN when
 * P_b + B > p_max and/or SIMSD_ST_POS_NEG when pos_d holds a negative entry
 * for the sequence (that sequence is left unchanged).  The caller provides
 * k_blk / v_blk computed for the committed tokens.
 *  k_blk, v_blk [NB][2B][Hkv][d] (rows 0..B-1 are read); prompt_len [NB]
 *  int32 in/out; k_cache, v_cache [NB][Hkv][p_max][d] in/out.
 * Errors: as for simsd_verify_attn, and SIMSD_ERR_SHAPE for batch > 65535. */
int simsd_append_kv(const simsd_verify_desc* desc, const void* k_blk, const void* v_blk, const int32_t* pos_d,
                    const uint64_t* committed, int32_t* prompt_len, void* k_cache, void* v_cache, int32_t* status,
                    void* stream);

/* Measurement only: the streaming ceiling of simsd_verify_attn's load path.
 * Streams k and v ([streams_y][streams_x][len][head_dim] bf16 each, the
 * prompt-cache layout with streams_x = KV heads and streams_y = sequences;
 * len a multiple of 64, head_dim 64 or 128) through the attention kernel's
 * 4-stage ring of direct-to-LDS loads, one 8-wave workgroup per stream, with
 * its cache policy (non-temporal when k and v together reach 256 MiB), and
 * computes nothing.  `sink` (4 bytes, device) is written only on a condition
 * that is not expected to happen.  The events are bound to the kernel as in
 * simsd_verify_attn_timed (NULL for none).  Errors: SIMSD_ERR_SHAPE
 * (streams_y > 65535 included), _NULL, _ALIGN, _HIP. */
int simsd_stream_probe(const void* k, const void* v, int32_t streams_x, int32_t streams_y, int32_t len,
                       int32_t head_dim, void* sink, void* stream, void* start_event, void* stop_event);

/* Measurement only: the plain read rate of the same bytes, to compare with
 * simsd_stream_probe.  Reads `bytes` (a multiple of 16) from k and then from
 * v with 16-byte vector loads into registers (no LDS), 256 workgroups of 512
 * threads in a grid-stride loop, non-temporal by the same rule, and computes
 * nothing.  `sink`, the events
 * and the errors are as for simsd_stream_probe (SIMSD_ERR_SHAPE for a
 * negative or unaligned size; 0 bytes launches nothing). */
int simsd_read_probe(const void* k, const void* v, int64_t bytes, void* sink, void* stream, void* start_event,
                     void* stop_event);

/* Measurement only: the sustained rate of the bf16 matrix cores, the
 * compute-side ceiling the MFMA kernels are compared with.  Launches
 * `workgroups` (1..65536) workgroups of 4 waves; every wave runs `iters`
 * (>= 1) rounds of four independent v_mfma_f32_32x32x16_bf16 on register
 * operands, 4 * 32768 flops a round, with no memory traffic in the loop, and
 * each of its lanes then writes one float to sink[workgroup * 256 + lane of
 * the workgroup] (`sink`: workgroups * 256 floats, device, 4-byte aligned).
 * Events as for simsd_stream_probe.  Errors: SIMSD_ERR_SHAPE, _NULL, _ALIGN,
 * _HIP. */
int simsd_mfma_probe(int32_t workgroups, int32_t iters, float* sink, void* stream, void* start_event,
                     void* stop_event);

/* Human-readable text for a return code (static storage). */
const char* simsd_strerror(int code);

/* ABI version of this header: 9. */
int simsd_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SIMSD_H */
