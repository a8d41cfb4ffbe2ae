/*
 * sd_verify.h -- C ABI of the speculative-sampling verify step on gfx950.
 *
 * One call verifies B independent requests.  Request r carries K_r draft
 * positions: K_r + 1 target logit rows (positions 0..K_r, the target scored
 * [last committed, x_0, .., x_{K_r-1}] in one forward) and K_r draft logit
 * rows with the draft tokens x_0..x_{K_r-1} that were sampled from them.
 * (Adaptive-SpecDecode-Lab README, implementation section: one target
 * forward verifies the whole proposal; longest-prefix acceptance, a target
 * correction at the first mismatch, a bonus after a full match.)
 *
 * Sampling verify (sd_verify_sample) follows "What I Gave Up to Make
 * Speculative Decoding Faster", section "A knob for accepting more draft
 * tokens": p and q are the target and draft distributions after repetition
 * penalty and temperature (and top-p, "Speculative Decoding" note, section
 * "Warum eine Korrektur noetig ist"); d = TV(p, q) = 1/2 sum |p - q|;
 * theta = min(1, D/d) with theta = 1 when d = 0; pi = (1-theta) p + theta q;
 * a draft token x is accepted with probability min(1, pi(x)/q(x)); after a
 * rejection the correction is drawn from the normalized max(p - q, 0).
 * D = 0 is lossless speculative sampling, D >= 1 follows the draft.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers (hipMalloc'd or equivalent),
 *    owned by the caller; the library keeps no pointer after the call
 *    returns and allocates no memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    legacy default stream).  Host-checkable argument errors are reported
 *    synchronously by the return code and nothing is enqueued.
 *  - Data-dependent problems are reported per request in out_status[r]
 *    (SD_ST_* bits).  A request with an SD_ST_INVALID_MASK bit set gets
 *    out_accepted[r] = -1 and every out_tokens[r][*] = -1.  One invalidating
 *    defect is reported per request, the first found in the order K_r, draft
 *    ids, temperature; SD_ST_BAD_PARAM is reported beside it, SD_ST_BAD_PRIOR
 *    always; the logits of an invalid request are not examined, so
 *    SD_ST_NONFINITE only appears on a request that passed the other checks.
 *  - Calls that share a workspace must not overlap in time.
 *
 * Logit layout
 * ------------
 *  target row (r, j), 0 <= j <= K_max: element i at
 *      target_logits + ((int64)r * (K_max + 1) + j) * ld_target + i
 *  draft row (r, j), 0 <= j < K_max: element i (i < V_draft) at
 *      draft_logits + ((int64)r * K_max + j) * ld_draft + i
 *  Element type is fp32 (SD_F32) or bf16 (SD_BF16, raw 16-bit patterns).
 *  Rows must be 16-byte aligned (ld * element size a multiple of 16 and the
 *  base pointers 16-byte aligned).  Rows j > K_r are never read.
 */
#ifndef SD_VERIFY_H
#define SD_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SD_OK            0
#define SD_EINVAL       (-1)  /* an argument fails a host-side check           */
#define SD_EWORKSPACE   (-2)  /* workspace NULL or smaller than required      */
#define SD_EHIP         (-3)  /* a HIP runtime call failed (launch, query)    */
#define SD_EUNSUPPORTED (-4)  /* valid request outside this build's limits    */
#define SD_ESCRATCH     (-5)  /* sd_verify_sample_noalloc: the call needs more
                                 workspace than SD_NOALLOC_MAX_WORKSPACE       */

/* Element types of the logit rows. */
#define SD_F32  0
#define SD_BF16 1

/* Flags. */
#define SD_NO_BONUS            (1u << 0)  /* after a full acceptance emit no
                                             extra target token ("What I Gave
                                             Up...", section "Even full
                                             acceptance did not buy a speedup") */
#define SD_PENALTY_PRIOR_ONLY  (1u << 1)  /* penalty set = prior ids only
                                             (default: prior ids plus the
                                             draft prefix x_0..x_{j-1})       */

/* Per-request status bits (out_status). */
#define SD_ST_BAD_K        (1u << 0)  /* k_per_row[r] outside [0, K_max]   invalid */
#define SD_ST_BAD_TEMP     (1u << 1)  /* temperature not finite or <= 0    invalid */
#define SD_ST_BAD_DRAFT_ID (1u << 2)  /* x_j outside [0, V) for a j < K_r  invalid */
#define SD_ST_NONFINITE    (1u << 3)  /* NaN or +Inf logit in a used row, or a
                                         used row of only -Inf (greedy: NaN)
                                                                           invalid */
#define SD_ST_BAD_PRIOR    (1u << 4)  /* a prior id outside [0, V) was ignored   */
#define SD_ST_Q_ZERO       (1u << 5)  /* q(x_j) = 0 at some j < K_r (a proposal
                                         the draft could not have drawn)       */
#define SD_ST_RESID_ZERO   (1u << 6)  /* the correction residual had zero mass;
                                         drew from p instead                    */
#define SD_ST_BAD_PARAM    (1u << 7)  /* top_p_per_row[r] outside (0, 1] or
                                         tv_budget_per_row[r] < 0 or NaN invalid */
#define SD_ST_INVALID_MASK 0x8Fu

/* Largest supported K_max (draft positions per request). */
#define SD_MAX_K 32

/* Per-position statistics written when out_stats != NULL:
 * out_stats[(r * (K_max + 1) + j) * SD_NSTAT + s] for s =                  */
#define SD_STAT_D     0   /* TV distance d_j (j < K_r)                          */
#define SD_STAT_THETA 1   /* theta_j                                            */
#define SD_STAT_PX    2   /* p_j(x_j)  processed target prob of the draft token */
#define SD_STAT_QX    3   /* q_j(x_j)                                           */
#define SD_STAT_PIX   4   /* pi_j(x_j)                                          */
#define SD_STAT_U     5   /* acceptance uniform u_j (j <= K_r)                  */
#define SD_STAT_V     6   /* draw uniform v_j (j <= K_r)                        */
#define SD_STAT_S     7   /* at j = n only: mass of the distribution the emitted
                             token was drawn from (residual sum, or ~1 for the
                             bonus)                                             */
#define SD_NSTAT 8

typedef struct sd_verify_args {
  const void    *target_logits;  /* [B][K_max+1] rows, see layout above        */
  const void    *draft_logits;   /* [B][K_max] rows; unused by greedy (NULL ok) */
  int64_t        ld_target;      /* elements between consecutive target rows   */
  int64_t        ld_draft;       /* elements between consecutive draft rows    */
  int32_t        dtype;          /* SD_F32 or SD_BF16                          */
  int32_t        B;              /* requests, >= 1                             */
  int32_t        K_max;          /* draft positions capacity, 0..SD_MAX_K     */
  int32_t        V;              /* vocabulary size, >= 1, < 2^30             */
  const int32_t *draft_ids;      /* [B][K_max] draft tokens x_j                */
  const int32_t *k_per_row;      /* [B] K_r in [0, K_max]; NULL = all K_max    */
  const float   *temperature;    /* [B] T_r > 0; NULL = all 1 (greedy ignores) */
  float          top_p;          /* (0, 1]; 1 = no truncation (greedy ignores) */
  float          rep_penalty;    /* > 0, finite; 1 = no penalty                */
  float          tv_budget;      /* D >= 0 (greedy ignores)                    */
  const int32_t *prior_ids;      /* CSR values of prior-context ids; NULL = none */
  const int32_t *prior_offsets;  /* [B+1] CSR offsets (row r: [off[r], off[r+1]));
                                    any count per row, repeats allowed (the
                                    set is their union)                       */
  uint64_t       seed;           /* Philox4x32-10 key (lo, hi words)           */
  uint64_t       offset;         /* Philox counter words 2-3                   */
  uint32_t       flags;          /* SD_NO_BONUS | SD_PENALTY_PRIOR_ONLY        */
  /* Per-request sampling parameters (device [B] fp32, or NULL for the
   * scalars above, which are then checked on the host).  When given, they
   * replace top_p and tv_budget request by request; a request whose value
   * is out of range gets SD_ST_BAD_PARAM.  Greedy ignores both. */
  const float   *top_p_per_row;
  const float   *tv_budget_per_row;
  /* Draft vocabulary (Adaptive-SpecDecode-Lab README, implementation
   * section: the two tokenizers are fully mapped, but the models' logit rows
   * may differ in length, e.g. 152064 and 151936 for the pages' Qwen2.5
   * 7B / 0.5B pair).  Draft rows hold the logits of ids 0..V_draft-1 only;
   * ids V_draft..V-1 have q = 0 (the draft cannot propose them, a proposal
   * there is a q(x) = 0 proposal).  0 means V; otherwise 1 <= V_draft <= V,
   * and ld_draft >= V_draft.  Greedy ignores it. */
  int32_t        V_draft;
} sd_verify_args_t;

/* Bytes of device workspace sd_verify_sample / sd_verify_greedy need for
 * these arguments (depends on B, K_max, V only).  The workspace holds
 * per-row statistics and counters; its contents need no initialization and
 * are meaningless between calls.  Returns SD_OK or SD_EINVAL. */
int sd_verify_workspace_bytes(const sd_verify_args_t *args, size_t *bytes);

/* Sampling verify.
 * Uniforms: Philox4x32-10 block at counter (j, r, offset_lo, offset_hi),
 * key (seed_lo, seed_hi); word 0 -> u_j (acceptance), word 1 -> v_j (draw),
 * each (w >> 8) * 2^-24.  Position j is accepted iff u_j * q_j(x_j) <
 * pi_j(x_j); n_r = first rejected position, else K_r.  Row r then emits
 * x_0..x_{n-1} and one more token y drawn by inverse CDF (ascending token
 * id, first index whose cumulative mass exceeds v_n * S) from
 * max(p_n - q_n, 0) when n < K_r, or from p_{K_r} when n = K_r (no token
 * when n = K_r and SD_NO_BONUS is set).
 * Outputs (device): out_accepted [B] = n_r; out_tokens [B][K_max+1] (-1
 * padded); out_status [B] (may be NULL); out_stats [B][K_max+1][SD_NSTAT]
 * (may be NULL).  The caller rolls back K_r - n_r positions of its caches. */
int sd_verify_sample(const sd_verify_args_t *args, void *workspace,
                     size_t workspace_bytes, int32_t *out_accepted,
                     int32_t *out_tokens, uint32_t *out_status,
                     float *out_stats, void *stream);

/* Sampling verify that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, outputs,
 * errors and results as sd_verify_sample; the workspace is instead a
 * built-in array of SD_NOALLOC_MAX_WORKSPACE bytes in the library's device
 * code, one per GPU, held until the process ends (its address is looked up
 * on the first call on each device, with that device current).  Calls whose
 * sd_verify_workspace_bytes exceeds that size return SD_ESCRATCH and enqueue
 * nothing (8 MiB covers e.g. B = 2048 requests at K_max = 8 and V = 152064).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, two host threads) race and must be serialized by
 * the caller.  No part of the array needs clearing between calls. */
#define SD_NOALLOC_MAX_WORKSPACE (8u << 20)
int sd_verify_sample_noalloc(const sd_verify_args_t *args, int32_t *out_accepted,
                             int32_t *out_tokens, uint32_t *out_status,
                             float *out_stats, void *stream);

/* Greedy verify (Adaptive-SpecDecode-Lab README, implementation section):
 * g_j = argmax of the penalized target row j (lowest id among equal maxima;
 * temperature and top-p are ignored since they cannot move an argmax);
 * n_r = first j < K_r with x_j != g_j, else K_r; row r emits x_0..x_{n-1}
 * and g_n (no token for n = K_r with SD_NO_BONUS).  Reads target rows only.
 * Outputs as for sd_verify_sample; out_argmax [B][K_max+1] may be NULL and
 * receives g_j for j <= K_r (-1 beyond). */
int sd_verify_greedy(const sd_verify_args_t *args, void *workspace,
                     size_t workspace_bytes, int32_t *out_accepted,
                     int32_t *out_tokens, uint32_t *out_status,
                     int32_t *out_argmax, void *stream);

/* Draft-side confidence ("What I Gave Up to Make Speculative Decoding
 * Faster", section "Confidence-guided early stop": after each draft token
 * the probability of its most likely token is taken from the logits already
 * produced; below a threshold the draft proposes nothing more, and that last
 * token is still verified).
 * draft_logits: device, B x K_max rows of V elements in the draft layout
 *   above (row (r, j) at draft_logits + ((int64)r * K_max + j) * ld_draft),
 *   dtype SD_F32 or SD_BF16, rows 16-byte aligned; read once, not written.
 * temperature: device [B] fp32, or NULL for T = 1.
 * out_top1: device [B][K_max] fp32 (required): max_i softmax(z / T)_i of
 *   each row = 1 / sum_i exp((z_i - max z) / T).  -inf logits count as
 *   masked tokens; a row with a NaN or +inf logit, a row with no finite
 *   logit, or a request with T outside (0, inf) gets NaN.
 * out_k: device [B] int32, or NULL: K_r = j + 1 for the first row j with
 *   top1 < threshold (NaN never stops), else K_max.  It can feed the
 *   k_per_row of sd_verify_sample.
 * No workspace; two launches on `stream`.  Returns SD_OK; SD_EINVAL for a
 * NULL or misaligned pointer, B, K_max or V < 1, ld_draft < V or not a
 * 16-byte multiple, or a NaN threshold; SD_EUNSUPPORTED when B * K_max
 * exceeds 2^31 - 1; SD_EHIP when a launch fails. */
int sd_draft_confidence(const void *draft_logits, int32_t dtype, int32_t B,
                        int32_t K_max, int32_t V, int64_t ld_draft,
                        const float *temperature, float threshold,
                        float *out_top1, int32_t *out_k, void *stream);

/* ------------------------------------------------------------------------
 * Verify fed from hidden states through the LM heads ("What I Gave Up to
 * Make Speculative Decoding Faster", section "Finding the break-even point":
 * the engine scores the verify rows with its LM head; Adaptive-SpecDecode-
 * Lab README, implementation section: one target forward keeps the logits of
 * the rows being verified).  The logits z = h . W^T are computed by a bf16
 * MFMA GEMM with fp32 accumulation and consumed tile by tile: no V-wide
 * logit row is written to memory.  The results are those of sd_verify_sample
 * / sd_verify_greedy on these logits with top_p = 1 and rep_penalty = 1
 * (neither is supported here).
 *
 * target_hidden: device bf16 [B][K_max+1][H_target] (position j of request r
 *   at ((int64)r * (K_max + 1) + j) * H_target); draft_hidden: device bf16
 *   [B][K_max][H_draft].  target_weight: device bf16 [V][H_target], row i
 *   the output vector of token i; draft_weight: [V_draft][H_draft].
 *   H_target and H_draft are multiples of 64; every pointer is 16-byte
 *   aligned; nothing is written to them.  Each hidden-state array is below
 *   2 GiB (else SD_EUNSUPPORTED).
 * V_draft (0 = V) and the draft ids, K, temperature, budget, seed, offset
 * and SD_NO_BONUS mean what they mean in sd_verify_args_t.  Greedy ignores
 * the draft fields and the temperature.
 * ------------------------------------------------------------------------ */
typedef struct sd_lmhead_args {
  const void    *target_hidden;
  const void    *draft_hidden;
  const void    *target_weight;
  const void    *draft_weight;
  int32_t        H_target;
  int32_t        H_draft;
  int32_t        B;
  int32_t        K_max;
  int32_t        V;
  int32_t        V_draft;
  const int32_t *draft_ids;      /* [B][K_max]                                  */
  const int32_t *k_per_row;      /* [B] or NULL (all K_max)                     */
  const float   *temperature;    /* [B] or NULL (all 1)                         */
  float          tv_budget;      /* D >= 0                                      */
  uint32_t       flags;          /* SD_NO_BONUS                                 */
  uint64_t       seed;
  uint64_t       offset;
} sd_lmhead_args_t;

/* Workspace bytes of the two calls below (depends on B, K_max, V, V_draft):
 * per (row, 128-token tile) partials, about 8 B * (2 K_max + 1) * B * V / 128
 * plus per-row statistics; no V-wide row.  SD_OK or SD_EINVAL. */
int sd_lmhead_workspace_bytes(const sd_lmhead_args_t *args, size_t *bytes);

/* Sampling verify on LM-head logits.  Outputs, statistics, status bits and
 * the return codes as for sd_verify_sample (statistics include d; d is
 * computed, at the cost of a second pass over both heads, when
 * 0 < tv_budget < 1 or out_stats is given).  Asynchronous on `stream`. */
int sd_lmhead_verify_sample(const sd_lmhead_args_t *args, void *workspace,
                            size_t workspace_bytes, int32_t *out_accepted,
                            int32_t *out_tokens, uint32_t *out_status,
                            float *out_stats, void *stream);

/* Greedy verify on LM-head logits (target head only), as sd_verify_greedy. */
int sd_lmhead_verify_greedy(const sd_lmhead_args_t *args, void *workspace,
                            size_t workspace_bytes, int32_t *out_accepted,
                            int32_t *out_tokens, uint32_t *out_status,
                            int32_t *out_argmax, void *stream);

/* Test export: the LM-head logits of the rows the sampling verify (out_draft
 * non-NULL) or the greedy verify (out_draft NULL) uses, as fp32 into
 * out_target [B][K_max+1][V] and out_draft [B][K_max][V_draft] (rows it
 * does not use are left untouched), from the same tile engine. */
int sd_debug_lmhead_logits(const sd_lmhead_args_t *args, void *workspace,
                           size_t workspace_bytes, float *out_target,
                           float *out_draft, void *stream);

/* Human-readable text for a return code (static storage). */
const char *sd_strerror(int code);

/* Test export: the processed, truncated, renormalized distributions of the
 * sampling verify for every used row, written as fp32 into out_p
 * [B][K_max+1][V] (target) and out_q [B][K_max][V] (draft); rows beyond K_r
 * are left untouched.  Same arguments and workspace as sd_verify_sample. */
int sd_debug_process_rows(const sd_verify_args_t *args, void *workspace,
                          size_t workspace_bytes, float *out_p, float *out_q,
                          void *stream);

/* Measurement export: run one phase of sd_verify_sample alone, so a caller
 * can bracket a single kernel with events on `stream`.  Running phases 0, 1,
 * 2 in order on one stream is exactly sd_verify_sample.  Same arguments,
 * workspace and outputs as sd_verify_sample.  Which kernels the phases are
 * depends on the arguments (sd_debug_phase_kernel names them):
 *   single-pass path (bf16, top_p < 1, V <= 155648):
 *     0 = one pass over every (row, position) pair and bonus row: top-p
 *         cut, TV, accept test and draw (a unit the pass cannot settle is
 *         recomputed by the same workgroup's exact multi-pass route);
 *     1 = no launch; 2 = longest accepted prefix, output tokens and
 *         statistics;
 *   general path: 0 = per-row statistics and top-p cut, 1 = per-position
 *     TV distance (no launch when not needed), 2 = decisions and draws. */
int sd_debug_run_phase(const sd_verify_args_t *args, void *workspace,
                       size_t workspace_bytes, int phase, int32_t *out_accepted,
                       int32_t *out_tokens, uint32_t *out_status,
                       float *out_stats, void *stream);

/* Measurement export: the name of the kernel that sd_debug_run_phase
 * launches for `phase` with these arguments (static storage), or NULL when
 * that phase launches nothing or the arguments are invalid. */
const char *sd_debug_phase_kernel(const sd_verify_args_t *args, int phase);

/* Test export: after phase 0 of the single-pass path (sd_debug_run_phase),
 * the number of units (draft positions j < K_r and bonus rows of valid
 * requests) that phase settled by its exact route, written to *out_count
 * (host memory).  out_why (host, nullable): B * (K_max + 1) words, unit u =
 * pair (r, j) at r * K_max + j, bonus row r at B * K_max + r; bit 1 a
 * target-row stream state out of range, 2 a target cut the window did not
 * settle, 4 and 8 the same for the draft row, 16 more nucleus candidates
 * than slots, 32 (with 2) a target cut settled from the row's whole exact
 * key histogram instead of its own passes, 64 (with 8) the same for the
 * draft row; 0 for units the single pass settled.  Synchronizes `stream`.
 * SD_EUNSUPPORTED when the arguments select the general path. */
int sd_debug_fallback_units(const sd_verify_args_t *args, const void *workspace,
                            size_t workspace_bytes, int32_t *out_count, uint32_t *out_why,
                            void *stream);

/* Test export: the Philox uniforms u, v for rows 0..B-1 and positions
 * 0..npos-1, written to out_u / out_v [B][npos] (fp32, exact). */
int sd_debug_uniforms(uint64_t seed, uint64_t offset, int32_t B, int32_t npos,
                      float *out_u, float *out_v, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SD_VERIFY_H */
